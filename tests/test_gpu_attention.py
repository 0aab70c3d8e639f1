"""GPU parity of paged decode attention (the consumer of the compacted cache)
against the fp64 oracle, through the C ABI.

Tolerance: |o_gpu - o_ref| <= ATTN_ATOL + ATTN_RTOL * |o_ref| elementwise.  The
kernel forms logits from exact bf16 (or fp32) products summed in fp32, uses
the hardware base-2 exponential (about 1 ulp) and sums up to ~10^5 weighted
rows per output in fp32 across lanes, waves and splits; with N(0, 1) values
the accumulated rounding stays near 1e-6 absolute, and the bound below leaves
a wide margin while still catching a wrong row, head or scale.
"""
import numpy as np
import pytest
import torch

import oracle
from decode_kv_cache_amd import kara as K
from decode_kv_cache_amd.workloads import KaraShape, decode_queries, fill_prior_context, make_workload, \
    shape_by_name
from tests.kara_harness import bits, config_of, oracle_unit_attention, run_step

pytestmark = pytest.mark.gpu

ATTN_ATOL = 5e-5
ATTN_RTOL = 1e-3

SHAPES = [
    shape_by_name("tiny"),                                             # f32, head_dim 64
    KaraShape("attn_g4", 201, num_seqs=3, num_layers=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
              window=200, budget=40, seeds=3, radius=2, prior=("uniform", 0, 700)),
    KaraShape("attn_g7", 202, num_seqs=2, num_layers=1, num_q_heads=14, num_kv_heads=2, head_dim=128,
              window=96, budget=30, seeds=2, radius=3, prior=("uniform", 31, 333), block_size=32),
    KaraShape("attn_mha_d64", 203, num_seqs=2, num_layers=2, num_q_heads=4, num_kv_heads=4, head_dim=64,
              window=64, budget=17, seeds=1, radius=2, prior=("uniform", 1, 150), block_size=8),
    KaraShape("attn_g2_bs1", 204, num_seqs=2, num_layers=1, num_q_heads=4, num_kv_heads=2, head_dim=128,
              window=40, budget=9, seeds=1, radius=4, prior=("fixed", 70), block_size=1),
    KaraShape("attn_g16_f32", 205, num_seqs=1, num_layers=1, num_q_heads=16, num_kv_heads=1, head_dim=128,
              window=50, budget=10, seeds=0, radius=0, prior=("fixed", 300), block_size=16, dtype="f32"),
    KaraShape("attn_long", 206, num_seqs=1, num_layers=1, num_q_heads=8, num_kv_heads=1, head_dim=128,
              window=1024, budget=204, seeds=8, radius=5, prior=("fixed", 20000), block_size=16),
]


def _attend(cfg, wl, q_dec, seq_lens):
    out = torch.full((cfg.num_seqs, cfg.num_layers, cfg.num_q_heads, cfg.head_dim), float("nan"),
                     dtype=torch.float32, device="cuda")
    wsb = K.kara_decode_attention_workspace_bytes(cfg)
    ws = torch.empty(max(wsb // 4, 1) + 64, dtype=torch.float32, device="cuda") if wsb else None
    K.kara_decode_attention(cfg, q_dec, wl.k_pool, wl.v_pool, wl.block_tables, seq_lens, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _check(got, ref, what):
    err = np.abs(got - ref) - ATTN_RTOL * np.abs(ref)
    assert np.all(np.isfinite(got)), what
    assert err.max() <= ATTN_ATOL, (what, float(np.abs(got - ref).max()))
    return float(np.abs(got - ref).max())


def _host(t):
    return t.float().double().cpu().numpy()


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: s.name)
def test_attention_before_and_after_compaction(shape):
    s = shape
    wl = make_workload(s, "cuda")
    fill_prior_context(wl)
    q_dec = decode_queries(s, "cuda")
    cfg = config_of(wl)
    qh = _host(q_dec)
    # full cache: L + W slots
    full_lens = torch.from_numpy((wl.host_prior_lens + s.window).astype(np.int32)).cuda()
    got = _attend(cfg, wl, q_dec, full_lens)
    ref = oracle.paged_decode_attention(qh, _host(wl.k_pool), _host(wl.v_pool), wl.host_tables,
                                        wl.host_prior_lens + s.window, s.block_size)
    e1 = _check(got, ref, "full cache")
    # compress, then attend over the L + B slots of the compacted pages
    k0, v0 = _host(wl.k_pool), _host(wl.v_pool)
    cfg, out = run_step(wl, cfg)
    kept = out["kept"].cpu().numpy()
    seq_lens = out["seq_lens"]
    assert np.array_equal(seq_lens.cpu().numpy(), wl.host_prior_lens + s.budget)
    got = _attend(cfg, wl, q_dec, seq_lens)
    ref = oracle.paged_decode_attention(qh, _host(wl.k_pool), _host(wl.v_pool), wl.block_tables.cpu().numpy(),
                                        wl.host_prior_lens + s.budget, s.block_size)
    e2 = _check(got, ref, "compacted cache")
    # and the same numbers from the prior rows plus the kept rows of the cache
    # as it was before compaction, gathered by hand
    G = s.group
    for n in range(s.num_seqs):
        L = int(wl.host_prior_lens[n])
        for layer in range(s.num_layers):
            for g in range(s.num_kv_heads):
                rows = list(range(L)) + [L + int(j) for j in kept[n, layer, g]]
                Kd = oracle.gather_window_rows(k0, wl.host_tables[n], layer, g, 0, L + s.window, s.block_size)[rows]
                Vd = oracle.gather_window_rows(v0, wl.host_tables[n], layer, g, 0, L + s.window, s.block_size)[rows]
                o = oracle_unit_attention(qh[n, layer, g * G:(g + 1) * G], Kd, Vd)
                sub = got[n, layer, g * G:(g + 1) * G]
                assert np.all(np.abs(sub - o) <= ATTN_ATOL + ATTN_RTOL * np.abs(o)), (n, layer, g)
    print(f"{s.name}: splits {K.kara_decode_attention_splits(cfg)}, max err full {e1:.2e} compacted {e2:.2e}",
          flush=True)


def test_empty_short_and_split_lengths():
    # one long head group, so the slot range is split across workgroups; the
    # lengths cover 0, 1, a ragged step and ranges that leave splits empty
    s = KaraShape("attn_lens", 207, num_seqs=6, num_layers=1, num_q_heads=4, num_kv_heads=1, head_dim=128,
                  window=64, budget=16, seeds=1, radius=1, prior=("fixed", 6000))
    wl = make_workload(s, "cuda")
    fill_prior_context(wl)
    q_dec = decode_queries(s, "cuda")
    cfg = config_of(wl)
    assert K.kara_decode_attention_splits(cfg) > 1
    lens = np.array([0, 1, 33, 1000, 6064, 4097], dtype=np.int32)
    got = _attend(cfg, wl, q_dec, torch.from_numpy(lens).cuda())
    ref = oracle.paged_decode_attention(_host(q_dec), _host(wl.k_pool), _host(wl.v_pool), wl.host_tables, lens,
                                        s.block_size)
    assert np.all(got[0] == 0)
    _check(got, ref, "lengths")


def test_block_table_cap_splits():
    # 2048 units at block size 1 with about 10^4 slots each: one split per
    # unit would stage more block ids than the kernel's LDS table holds, so
    # the slot range is split because of that cap, not for occupancy.
    # Sampled units are checked against the oracle.
    s = KaraShape("attn_tblcap", 208, num_seqs=16, num_layers=16, num_q_heads=8, num_kv_heads=8, head_dim=64,
                  window=64, budget=16, seeds=1, radius=1, prior=("fixed", 10000), block_size=1)
    wl = make_workload(s, "cuda")
    fill_prior_context(wl)
    q_dec = decode_queries(s, "cuda")
    cfg = config_of(wl)
    assert s.units >= 2048 and K.kara_decode_attention_splits(cfg) >= 3
    lens = (wl.host_prior_lens + s.window).astype(np.int32)
    got = _attend(cfg, wl, q_dec, torch.from_numpy(lens).cuda())
    assert np.all(np.isfinite(got))
    rng = np.random.default_rng(208)
    units = {(0, 0, 0), (s.num_seqs - 1, s.num_layers - 1, s.num_kv_heads - 1)}
    while len(units) < 6:
        units.add((int(rng.integers(s.num_seqs)), int(rng.integers(s.num_layers)), int(rng.integers(s.num_kv_heads))))
    for (n, layer, g) in sorted(units):
        T = int(lens[n])
        blk = torch.from_numpy(wl.host_tables[n, :T].astype(np.int64)).cuda()
        Kd = wl.k_pool[layer][blk, g, 0, :].float().double().cpu().numpy()
        Vd = wl.v_pool[layer][blk, g, 0, :].float().double().cpu().numpy()
        qh = q_dec[n, layer, g * s.group:(g + 1) * s.group].float().double().cpu().numpy()
        _check(got[n, layer, g * s.group:(g + 1) * s.group], oracle_unit_attention(qh, Kd, Vd), (n, layer, g))
    del wl
    torch.cuda.empty_cache()


def test_decode_attention_rejects_bad_arguments():
    s = SHAPES[1]
    wl = make_workload(s, "cuda")
    cfg = config_of(wl)
    q_dec = decode_queries(s, "cuda")
    out = torch.zeros((s.num_seqs, s.num_layers, s.num_q_heads, s.head_dim), dtype=torch.float32, device="cuda")
    lens = wl.prior_lens.clone()
    L = K.lib()
    import ctypes
    assert L.kara_decode_attention(ctypes.byref(cfg), None, wl.k_pool.data_ptr(), wl.v_pool.data_ptr(),
                                   wl.block_tables.data_ptr(), lens.data_ptr(), out.data_ptr(), None, 0,
                                   None) == -2
    if K.kara_decode_attention_workspace_bytes(cfg):
        assert L.kara_decode_attention(ctypes.byref(cfg), q_dec.data_ptr(), wl.k_pool.data_ptr(),
                                       wl.v_pool.data_ptr(), wl.block_tables.data_ptr(), lens.data_ptr(),
                                       out.data_ptr(), None, 0, None) == -3
    torch.cuda.synchronize()
    assert torch.all(out == 0)
