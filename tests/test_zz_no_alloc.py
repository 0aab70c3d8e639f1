"""The allocation-free one-launch pipeline (kara_compress_fused_noalloc, for
callers that cannot allocate device memory) against kara_compress_fused on the
same seeded inputs, through the C ABI: calls in a row whose second one covers
a smaller batch, every output, pool byte and table bit for bit."""
import numpy as np
import pytest
import torch

from decode_kv_cache_amd import kara as K
from decode_kv_cache_amd.workloads import KaraShape, make_workload
from tests.kara_harness import Outputs, bits, config_of

pytestmark = pytest.mark.gpu

BIG = KaraShape("noalloc_big", 961, num_seqs=5, num_layers=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
                window=300, budget=60, seeds=3, radius=4, prior=("uniform", 5, 80))
SMALL = KaraShape("noalloc_small", 962, num_seqs=2, num_layers=1, num_q_heads=4, num_kv_heads=1, head_dim=128,
                  window=160, budget=40, seeds=2, radius=3, prior=("uniform", 3, 40), block_size=8)


def _run(shape, noalloc, stream=None):
    wl = make_workload(shape, "cuda")
    cfg = config_of(wl)
    out = Outputs(cfg, "cuda")
    torch.cuda.synchronize()
    args = (cfg, wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.prior_lens, out["scores"], out["kept"],
            out["seq_lens"], out["freed"], out["num_freed"])
    if noalloc:
        K.kara_compress_fused_noalloc(*args, mask=out["mask"], stream=stream)
    else:
        done = torch.zeros(shape.num_seqs, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        K.kara_compress_fused(*args, done, mask=out["mask"], stream=stream)
    torch.cuda.synchronize()
    assert out.guards_intact()
    res = {k: bits(out[k]) for k in ("scores", "kept", "mask", "seq_lens", "freed", "num_freed")}
    res.update(k=bits(wl.k_pool), v=bits(wl.v_pool), tables=wl.block_tables.cpu().numpy())
    return res


def _same(a, b, what):
    for k in a:
        assert np.array_equal(a[k], b[k]), (what, k)


def test_noalloc_matches_fused_on_calls_in_a_row():
    print("[noalloc] big, then smaller, then big again", flush=True)
    ref_big, ref_small = _run(BIG, False), _run(SMALL, False)
    _same(ref_big, _run(BIG, True), "first call")
    _same(ref_small, _run(SMALL, True), "second call, smaller batch")
    _same(ref_big, _run(BIG, True), "third call")


def test_noalloc_on_a_side_stream():
    print("[noalloc] side stream", flush=True)
    st = torch.cuda.Stream()
    _same(_run(SMALL, False), _run(SMALL, True, stream=st), "side stream")


STAGED_BIG = KaraShape("noalloc_f32_d64", 963, num_seqs=4, num_layers=2, num_q_heads=6, num_kv_heads=2, head_dim=64,
                       window=256, budget=64, seeds=2, radius=4, dtype="f32", prior=("uniform", 0, 70))
STAGED_SMALL = KaraShape("noalloc_bf16_d64", 964, num_seqs=1, num_layers=1, num_q_heads=4, num_kv_heads=4,
                         head_dim=64, window=40, budget=12, seeds=1, radius=2, prior=("fixed", 9), block_size=4)


def test_noalloc_with_the_staged_key_scorer():
    print("[noalloc] staged-key scorer shapes, big then smaller", flush=True)
    _same(_run(STAGED_BIG, False), _run(STAGED_BIG, True), "first call")
    _same(_run(STAGED_SMALL, False), _run(STAGED_SMALL, True), "second call, smaller batch")


def test_noalloc_replayed_from_a_captured_graph():
    """Code under graph capture is one of the callers the entry point is for:
    the call is captured once on a side stream and the graph is replayed three
    times, with eager copies restoring the inputs and refilling the outputs
    between replays; every replay gives the eager call's results bit for bit.
    The counters are cleared by a kernel, so the graph holds no memset node."""
    print("[noalloc] graph capture and three replays", flush=True)
    ref = _run(SMALL, True)            # eager result; also looks up the per-device counter array
    wl = make_workload(SMALL, "cuda")
    cfg = config_of(wl)
    out = Outputs(cfg, "cuda")
    k0, v0, t0 = wl.k_pool.clone(), wl.v_pool.clone(), wl.block_tables.clone()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(graph, stream=side):
        K.kara_compress_fused_noalloc(cfg, wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.prior_lens,
                                      out["scores"], out["kept"], out["seq_lens"], out["freed"], out["num_freed"],
                                      mask=out["mask"])
    torch.cuda.synchronize()
    for i in range(3):
        wl.k_pool.copy_(k0)
        wl.v_pool.copy_(v0)
        wl.block_tables.copy_(t0)
        for k, buf in out.raw.items():
            buf.fill_(out.fill[k])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert out.guards_intact()
        res = {k: bits(out[k]) for k in ("scores", "kept", "mask", "seq_lens", "freed", "num_freed")}
        res.update(k=bits(wl.k_pool), v=bits(wl.v_pool), tables=wl.block_tables.cpu().numpy())
        _same(ref, res, f"replay {i}")



def _flat_run(S, noalloc, seed=4242, W=32, B=8, bs=16, d=64):
    """S one-layer, one-head bf16 sequences with prior length 0, random
    queries and pools, block tables a seeded permutation of the pool; one
    call of either entry point."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    per = -(-W // bs)
    nb = S * per
    q = torch.randn((S, 1, W, 1, d), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((1, nb, 1, bs, d), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((1, nb, 1, bs, d), generator=g, device="cuda").to(torch.bfloat16)
    tables = torch.randperm(nb, generator=g, device="cuda").to(torch.int32).view(S, per).contiguous()
    prior = torch.zeros(S, dtype=torch.int32, device="cuda")
    cfg = K.kara_config(S, 1, 1, 1, d, W, B, 1, 1, bs, K.KARA_BF16, per, nb)
    assert K.kara_check_config(cfg) == 0 and K.kara_compress_fused_supported(cfg)
    out = Outputs(cfg, "cuda")
    args = (cfg, q, k, v, tables, prior, out["scores"], out["kept"], out["seq_lens"], out["freed"], out["num_freed"])
    torch.cuda.synchronize()
    if noalloc:
        K.kara_compress_fused_noalloc(*args, mask=out["mask"])
    else:
        done = torch.zeros(S, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        K.kara_compress_fused(*args, done, mask=out["mask"])
    torch.cuda.synchronize()
    assert out.guards_intact()
    res = {key: bits(out[key]) for key in ("scores", "kept", "mask", "seq_lens", "freed", "num_freed")}
    res.update(k=bits(k), v=bits(v), tables=tables.cpu().numpy())
    if not noalloc:
        assert bool((done == 0).all())
    return res


def test_noalloc_at_the_scratch_limit():
    """Exactly KARA_NOALLOC_MAX_SEQS = 65536 sequences, then 3, then 65536
    again: each allocation-free call equals kara_compress_fused bit for bit,
    so every counter of the fixed array was used and returned to zero."""
    print("[noalloc] 65536 sequences, then 3, then 65536", flush=True)
    S = 65536
    ref = _flat_run(S, False)
    assert (ref["seq_lens"] == 8).all() and (ref["num_freed"] == 1).all()
    _same(ref, _flat_run(S, True), "65536 sequences")
    _same(_flat_run(3, False, seed=7), _flat_run(3, True, seed=7), "3 sequences")
    _same(ref, _flat_run(S, True), "65536 sequences again")
