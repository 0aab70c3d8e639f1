"""Randomised parity sweep on the GPU: many small seeded configurations
(window, budget, seeds, radius, block size, GQA group, head_dim, dtype,
ragged priors, bridging gap), each against the fp64 oracle with the rules of
the parity tests: scores within the score tolerance, selection exact given the
GPU's scores, pools / tables / lengths / freed lists bit-exact."""
import numpy as np
import pytest

import oracle
from decode_kv_cache_amd.workloads import KaraShape, make_workload
from tests.kara_harness import SCORE_RTOL, bits, run_step, score_errors, unit_inputs

pytestmark = pytest.mark.gpu


def _random_shape(i):
    rng = np.random.default_rng(5000 + i)
    Hkv = int(rng.integers(1, 4))
    G = int(rng.choice([1, 2, 3, 4, 5, 7, 8]))
    d = int(rng.choice([64, 128]))
    dtype = "f32" if rng.random() < 0.2 else "bf16"
    W = int(rng.choice([1, 2, 7, 16, 33, 100, 255, 256, 300, 640, 1024, 1100]))
    r = int(rng.integers(0, min(6, W + 1)))
    s = int(rng.integers(0, max(1, W // (2 * r + 1)) + 1))
    s = min(s, W // (2 * r + 1))
    B = int(rng.integers(max(1, s * (2 * r + 1)), W + 1))
    bs = int(rng.choice([1, 2, 4, 8, 16, 32, 64]))
    lo = int(rng.integers(0, 200))
    gap = 0
    if s > 1 and rng.random() < 0.4:
        for cand in range(W, -1, -1):
            if oracle.chunk_bound(s, r, cand) <= B:
                gap = int(rng.integers(0, cand + 1))
                break
    shape = KaraShape(f"rand{i}", 6000 + i, num_seqs=int(rng.integers(1, 4)), num_layers=int(rng.integers(1, 3)),
                      num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=d, window=W, budget=B, seeds=s, radius=r,
                      block_size=bs, dtype=dtype, prior=("uniform", lo, lo + int(rng.integers(0, 100))),
                      key_model=str(rng.choice(["normal", "outliers", "student_t3"])), plants=bool(rng.random() < 0.5))
    return shape, gap


@pytest.mark.parametrize("i", range(24))
def test_random_configuration(i):
    s, gap = _random_shape(i)
    wl = make_workload(s, "cuda")
    qh = wl.q.float().double().cpu().numpy()
    kh = wl.k_pool.float().double().cpu().numpy()
    k0, v0 = bits(wl.k_pool), bits(wl.v_pool)
    cfg, out = run_step(wl, gap=gap if gap else None)
    assert out.guards_intact()
    c = out["scores"].cpu().numpy()
    for n in range(s.num_seqs):
        for layer in range(s.num_layers):
            for g in range(s.num_kv_heads):
                qg, kw = unit_inputs(qh, kh, wl, n, layer, g)
                assert score_errors(c[n, layer, g], oracle.window_scores(qg, kw)).max() <= SCORE_RTOL, (s, n, layer, g)
    ref = oracle.compress_step(np.zeros((s.num_seqs, s.num_layers, s.window, s.num_q_heads, 1)), k0, v0,
                               wl.host_tables, wl.host_prior_lens, window=s.window, budget=s.budget, seeds=s.seeds,
                               radius=s.radius, block_size=s.block_size, scores_override=c, gap=gap)
    assert np.array_equal(ref["kept"], out["kept"].cpu().numpy())
    assert np.array_equal(bits(wl.k_pool), ref["k_pool"])
    assert np.array_equal(bits(wl.v_pool), ref["v_pool"])
    assert np.array_equal(wl.block_tables.cpu().numpy(), ref["block_tables"])
    assert np.array_equal(out["seq_lens"].cpu().numpy(), ref["seq_lens"])
    assert np.array_equal(out["num_freed"].cpu().numpy(), ref["num_freed"])
    freed = out["freed"].cpu().numpy()
    for n in range(s.num_seqs):
        assert freed[n, :int(ref["num_freed"][n])].tolist() == ref["freed"][n].tolist()


def _one_launch_cases():
    """Indices of the configurations where kara_compress_fused is offered (a
    single-pass scorer runs); the library answers on the host."""
    from decode_kv_cache_amd import kara as K
    return [i for i in range(24)
            if K.kara_compress_fused_supported(K.make_config(_random_shape(i)[0], max_blocks_per_seq=4096,
                                                             num_blocks=100000))]


@pytest.mark.parametrize("i", _one_launch_cases())
def test_random_configuration_one_launch(i):
    """The same configurations through kara_compress_fused, where it is
    offered: every output, pool byte and table equal to the three calls' bit
    for bit (reading R29)."""
    import torch

    from decode_kv_cache_amd import kara as K
    from tests.kara_harness import Outputs, config_of
    s, _ = _random_shape(i)
    wa = make_workload(s, "cuda")
    cfg = config_of(wa)
    assert K.kara_compress_fused_supported(cfg)
    wb = make_workload(s, "cuda")
    _, ref = run_step(wa, cfg)
    out = Outputs(cfg, "cuda")
    done = torch.zeros(s.num_seqs, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    K.kara_compress_fused(cfg, wb.q, wb.k_pool, wb.v_pool, wb.block_tables, wb.prior_lens, out["scores"],
                          out["kept"], out["seq_lens"], out["freed"], out["num_freed"], done, mask=out["mask"])
    torch.cuda.synchronize()
    assert out.guards_intact() and bool((done == 0).all())
    for k in ("scores", "kept", "mask", "seq_lens", "num_freed", "freed"):
        assert np.array_equal(bits(out[k]), bits(ref[k])), (s.name, k)
    assert np.array_equal(bits(wb.k_pool), bits(wa.k_pool))
    assert np.array_equal(bits(wb.v_pool), bits(wa.v_pool))
    assert torch.equal(wb.block_tables, wa.block_tables)
