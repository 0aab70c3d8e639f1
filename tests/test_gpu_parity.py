"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Scores: relative error <= 2e-3 (floor 1e-30) for every window key.
Selection: kept == oracle.token2chunk_select(scores_gpu) bit for bit, and any
difference from oracle.token2chunk_select(scores_oracle) is a near-tie.
Compaction, block tables, freed lists, lengths: bit-exact against the oracle
applied to the GPU's kept lists; every other pool byte unchanged.
"""
import numpy as np
import pytest
import torch

import oracle
from decode_kv_cache_amd.workloads import KaraShape, make_workload, shape_by_name
from tests.kara_harness import (SCORE_RTOL, Outputs, bits, config_of, near_cutoff_ok, run_step, score_errors,
                                unit_inputs)

pytestmark = pytest.mark.gpu

SMALL = [
    shape_by_name("tiny"),
    KaraShape("ragged_bf16", 101, num_seqs=2, num_layers=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
              window=200, budget=40, seeds=3, radius=2, prior=("uniform", 5, 60)),
    KaraShape("gqa7_plants", 102, num_seqs=1, num_layers=1, num_q_heads=7, num_kv_heads=1, head_dim=128,
              window=300, budget=60, seeds=2, radius=4, prior=("fixed", 17), plants=True),
    KaraShape("d64_keep_all", 103, num_seqs=1, num_layers=2, num_q_heads=4, num_kv_heads=4, head_dim=64,
              window=64, budget=64, seeds=1, radius=0, prior=("fixed", 0)),
    KaraShape("f32_d128_bs8", 104, num_seqs=1, num_layers=1, num_q_heads=2, num_kv_heads=1, head_dim=128,
              window=50, budget=10, seeds=0, radius=0, prior=("fixed", 3), block_size=8, dtype="f32"),
    KaraShape("bs1", 105, num_seqs=2, num_layers=1, num_q_heads=2, num_kv_heads=1, head_dim=64,
              window=40, budget=9, seeds=1, radius=4, prior=("fixed", 7), block_size=1),
    KaraShape("bs32_outliers", 106, num_seqs=3, num_layers=1, num_q_heads=4, num_kv_heads=2, head_dim=128,
              window=256, budget=51, seeds=3, radius=3, prior=("uniform", 100, 300), block_size=32,
              key_model="outliers"),
    KaraShape("w1", 107, num_seqs=1, num_layers=1, num_q_heads=2, num_kv_heads=1, head_dim=64,
              window=1, budget=1, seeds=1, radius=0, prior=("fixed", 5)),
    KaraShape("t3_plants", 108, num_seqs=1, num_layers=1, num_q_heads=8, num_kv_heads=1, head_dim=128,
              window=512, budget=103, seeds=4, radius=6, prior=("fixed", 33), key_model="student_t3", plants=True),
    KaraShape("w2048_g7", 109, num_seqs=1, num_layers=1, num_q_heads=14, num_kv_heads=2, head_dim=128,
              window=2048, budget=410, seeds=12, radius=7, prior=("fixed", 16384), plants=True),
    KaraShape("w4096_t3", 110, num_seqs=1, num_layers=1, num_q_heads=8, num_kv_heads=1, head_dim=128,
              window=4096, budget=820, seeds=24, radius=8, prior=("fixed", 32768), key_model="student_t3",
              plants=True),
    # logits spanning about +-100 exponent units: sharply peaked rows, scores down to the fp32 range
    KaraShape("spiky_fused", 113, num_seqs=2, num_layers=1, num_q_heads=8, num_kv_heads=2, head_dim=128,
              window=512, budget=100, seeds=4, radius=3, prior=("fixed", 40), key_model="spiky"),
    KaraShape("spiky_two_pass", 114, num_seqs=1, num_layers=1, num_q_heads=4, num_kv_heads=1, head_dim=64,
              window=1500, budget=300, seeds=6, radius=4, prior=("fixed", 7), key_model="spiky"),
    # the largest window, the largest block size, and a budget of many seeded chunks
    KaraShape("w8192_bs256", 115, num_seqs=1, num_layers=1, num_q_heads=2, num_kv_heads=1, head_dim=64,
              window=8192, budget=1024, seeds=32, radius=15, prior=("fixed", 300), block_size=256,
              key_model="student_t3", plants=True),
    # the largest window kept whole: compaction moves nothing and frees nothing
    KaraShape("w8192_keep_all", 116, num_seqs=1, num_layers=1, num_q_heads=1, num_kv_heads=1, head_dim=64,
              window=8192, budget=8192, seeds=1, radius=0, prior=("fixed", 21), block_size=128, dtype="f32"),
    # sixteen query heads per KV head
    KaraShape("g16", 117, num_seqs=2, num_layers=1, num_q_heads=16, num_kv_heads=1, head_dim=128,
              window=128, budget=30, seeds=3, radius=2, prior=("uniform", 10, 90), block_size=4),
    # either side of the staged-key scorer's limits (256 keys; 128 for fp32 rows of head_dim 128)
    KaraShape("f32_d128_w128_staged", 118, num_seqs=2, num_layers=1, num_q_heads=6, num_kv_heads=2, head_dim=128,
              window=128, budget=32, seeds=2, radius=3, prior=("uniform", 0, 50), dtype="f32", plants=True),
    KaraShape("f32_d128_w129_two_pass", 119, num_seqs=1, num_layers=1, num_q_heads=6, num_kv_heads=2, head_dim=128,
              window=129, budget=32, seeds=2, radius=3, prior=("fixed", 11), dtype="f32", plants=True),
    KaraShape("d64_g7_w255_staged", 120, num_seqs=2, num_layers=2, num_q_heads=14, num_kv_heads=2, head_dim=64,
              window=255, budget=51, seeds=3, radius=3, prior=("uniform", 1, 99), key_model="outliers"),
    KaraShape("f32_d64_w300_two_pass", 121, num_seqs=2, num_layers=1, num_q_heads=4, num_kv_heads=2, head_dim=64,
              window=300, budget=60, seeds=3, radius=4, prior=("uniform", 0, 64), dtype="f32", block_size=8),
    # the largest query-row counts of the single-pass scorers: G = 16 over their longest windows
    KaraShape("f32_d64_w256_g16", 122, num_seqs=1, num_layers=1, num_q_heads=16, num_kv_heads=1, head_dim=64,
              window=256, budget=64, seeds=4, radius=3, prior=("fixed", 5), dtype="f32", plants=True),
    KaraShape("bf16_w1024_g16", 123, num_seqs=1, num_layers=1, num_q_heads=32, num_kv_heads=2, head_dim=128,
              window=1024, budget=204, seeds=8, radius=5, prior=("fixed", 77), key_model="outliers"),
    # the resident-key scorer's block loop with one, two and three 16-row blocks (its loop is unrolled
    # by two, with the first block and the last one or two outside it), and over a full window of
    # 1024 keys with G = 3, whose blocks straddle window positions
    KaraShape("fused_one_block", 124, num_seqs=2, num_layers=1, num_q_heads=1, num_kv_heads=1, head_dim=128,
              window=16, budget=4, seeds=1, radius=1, prior=("fixed", 9)),
    KaraShape("fused_two_blocks_g3", 125, num_seqs=1, num_layers=2, num_q_heads=3, num_kv_heads=1, head_dim=128,
              window=7, budget=3, seeds=1, radius=1, prior=("uniform", 0, 20)),
    KaraShape("fused_three_blocks", 126, num_seqs=1, num_layers=1, num_q_heads=2, num_kv_heads=2, head_dim=128,
              window=48, budget=10, seeds=2, radius=2, prior=("fixed", 30), plants=True),
    KaraShape("fused_w1024_g3", 127, num_seqs=1, num_layers=1, num_q_heads=6, num_kv_heads=2, head_dim=128,
              window=1024, budget=204, seeds=8, radius=5, prior=("fixed", 5), key_model="student_t3", plants=True),
]


def _host_f64(t):
    return t.float().double().cpu().numpy()


def _full_parity(shape):
    wl = make_workload(shape, "cuda")
    q_h = _host_f64(wl.q)
    k_f = _host_f64(wl.k_pool)
    k0, v0 = bits(wl.k_pool), bits(wl.v_pool)
    cfg, out = run_step(wl)
    s = shape
    c_gpu = out["scores"].cpu().numpy()
    kept = out["kept"].cpu().numpy()
    assert out.guards_intact()
    worst = 0.0
    for n in range(s.num_seqs):
        for layer in range(s.num_layers):
            for g in range(s.num_kv_heads):
                qg, kw = unit_inputs(q_h, k_f, wl, n, layer, g)
                c_orc = oracle.window_scores(qg, kw)
                err = score_errors(c_gpu[n, layer, g], c_orc)
                worst = max(worst, float(err.max()))
                assert err.max() <= SCORE_RTOL, (shape.name, n, layer, g, float(err.max()))
                sel = oracle.token2chunk_select(c_gpu[n, layer, g].astype(np.float64), s.budget, s.seeds, s.radius)
                assert kept[n, layer, g].tolist() == sel.kept.tolist(), (shape.name, n, layer, g)
                ok, nd = near_cutoff_ok(c_orc, kept[n, layer, g], s.budget, s.seeds, s.radius)
                assert ok, (shape.name, n, layer, g, nd)
    mask = out["mask"].cpu().numpy()
    assert np.array_equal(mask.sum(-1), np.full(mask.shape[:-1], s.budget))
    # compaction and tables, bit-exact, on the bit patterns of the pools
    ref = oracle.compress_step(np.zeros((s.num_seqs, s.num_layers, s.window, s.num_q_heads, 1)), k0, v0,
                               wl.host_tables, wl.host_prior_lens, window=s.window, budget=s.budget, seeds=s.seeds,
                               radius=s.radius, block_size=s.block_size, scores_override=c_gpu)
    assert np.array_equal(ref["kept"], kept)
    assert np.array_equal(bits(wl.k_pool), ref["k_pool"])
    assert np.array_equal(bits(wl.v_pool), ref["v_pool"])
    assert np.array_equal(wl.block_tables.cpu().numpy(), ref["block_tables"])
    assert np.array_equal(out["seq_lens"].cpu().numpy(), ref["seq_lens"])
    assert np.array_equal(out["num_freed"].cpu().numpy(), ref["num_freed"])
    freed = out["freed"].cpu().numpy()
    for n in range(s.num_seqs):
        nf = int(ref["num_freed"][n])
        assert freed[n, :nf].tolist() == ref["freed"][n].tolist()
        assert np.all(freed[n, nf:] == -1)
    return worst


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: s.name)
def test_small_shapes_full_parity(shape):
    worst = _full_parity(shape)
    print(f"{shape.name}: worst relative score error {worst:.2e}", flush=True)


def test_empty_batch_is_a_no_op():
    s = shape_by_name("tiny").with_(num_seqs=0)
    wl = make_workload(s, "cuda")
    cfg = config_of(wl)
    out = Outputs(cfg, "cuda")
    run_step(wl, cfg, out)
    assert out.guards_intact()


@pytest.mark.parametrize("idx", [1, 0, 12], ids=["resident_keys", "staged_keys", "two_pass"])
def test_repeat_runs_are_bit_identical_and_stream_ordered(idx):
    """Every scorer reduces in a fixed order: two runs give the same bits."""
    s = SMALL[idx]
    res = []
    for _ in range(2):
        wl = make_workload(s, "cuda")
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())    # the workload was written on the default stream
        with torch.cuda.stream(st):
            cfg, out = run_step(wl, stream=st)
        res.append((out["scores"].cpu(), out["kept"].cpu(), bits(wl.k_pool), bits(wl.v_pool),
                    wl.block_tables.cpu()))
    for a, b in zip(res[0], res[1]):
        assert np.array_equal(np.asarray(a), np.asarray(b))


def test_validate_tables_flags_bad_sequences():
    from decode_kv_cache_amd import kara as K
    s = SMALL[1]
    wl = make_workload(s, "cuda")
    cfg = config_of(wl)
    bad = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    K.kara_validate_tables(cfg, wl.block_tables, wl.prior_lens, bad)
    assert int(bad.item()) == 0
    tb = wl.block_tables.clone()
    L = int(wl.host_prior_lens[1])
    tb[1, (L + 5) // s.block_size] = -1
    pl = wl.prior_lens.clone()
    pl[0] = -3
    K.kara_validate_tables(cfg, tb, pl, bad)
    assert int(bad.item()) == 2


def test_host_rejects_bad_arguments_before_enqueueing():
    from decode_kv_cache_amd import kara as K
    wl = make_workload(SMALL[12], "cuda")     # W = 1500, head_dim 64: two-pass scorer with a workspace
    cfg = config_of(wl)
    out = Outputs(cfg, "cuda")
    small_ws = torch.empty(16, dtype=torch.float32, device="cuda")
    with pytest.raises(K.KaraError) as e:
        K.kara_score_window(cfg, wl.q, wl.k_pool, wl.block_tables, wl.prior_lens, out["scores"], small_ws)
    assert e.value.status == -3
    cfg.seeds = 100
    with pytest.raises(K.KaraError) as e:
        K.kara_select_chunks(cfg, out["scores"], out["kept"])
    assert e.value.status == -1
    torch.cuda.synchronize()
    assert out.guards_intact()
    assert torch.isnan(out["scores"]).all()


BRIDGED = [
    (SMALL[1], 16),                                  # bound 15 + 2 * 12 = 39 <= 40
    (SMALL[2], 40),                                  # its two seeds lie 79 apart: no bridge forms
    (SMALL[5], 40),                                  # one seed: nothing to bridge, gap = window
    (SMALL[8], 29),                                  # bound exactly the budget
    (KaraShape("bridge_wide", 111, num_seqs=2, num_layers=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
               window=256, budget=200, seeds=4, radius=1, prior=("uniform", 0, 40), plants=True), 64),
    (KaraShape("bridge_wide_f32", 112, num_seqs=1, num_layers=1, num_q_heads=4, num_kv_heads=2, head_dim=64,
               window=96, budget=90, seeds=6, radius=0, prior=("fixed", 9), dtype="f32"), 16),
]


@pytest.mark.parametrize("shape,gap", BRIDGED, ids=lambda x: getattr(x, "name", str(x)))
def test_bridged_selection_full_parity(shape, gap):
    from decode_kv_cache_amd import kara as K
    s = shape
    wl = make_workload(s, "cuda")
    k0, v0 = bits(wl.k_pool), bits(wl.v_pool)
    cfg, out = run_step(wl, gap=gap)
    assert out.guards_intact()
    c_gpu = out["scores"].cpu().numpy()
    kept = out["kept"].cpu().numpy()
    mask = out["mask"].cpu().numpy()
    bridged = 0
    for n in range(s.num_seqs):
        for layer in range(s.num_layers):
            for g in range(s.num_kv_heads):
                c = c_gpu[n, layer, g].astype(np.float64)
                sel = oracle.token2chunk_bridge_select(c, s.budget, s.seeds, s.radius, gap)
                assert kept[n, layer, g].tolist() == sel.kept.tolist(), (s.name, n, layer, g)
                assert np.array_equal(np.flatnonzero(mask[n, layer, g]), sel.kept)
                plain = oracle.token2chunk_select(c, s.budget, s.seeds, s.radius)
                bridged += int(sel.span.sum() - plain.span.sum())
    if s.name not in ("gqa7_plants", "bs1"):
        assert bridged > 0, "no unit exercised a bridge"
    ref = oracle.compress_step(np.zeros((s.num_seqs, s.num_layers, s.window, s.num_q_heads, 1)), k0, v0,
                               wl.host_tables, wl.host_prior_lens, window=s.window, budget=s.budget, seeds=s.seeds,
                               radius=s.radius, block_size=s.block_size, scores_override=c_gpu, gap=gap)
    assert np.array_equal(ref["kept"], kept)
    assert np.array_equal(bits(wl.k_pool), ref["k_pool"])
    assert np.array_equal(bits(wl.v_pool), ref["v_pool"])
    assert np.array_equal(wl.block_tables.cpu().numpy(), ref["block_tables"])
    assert np.array_equal(out["seq_lens"].cpu().numpy(), ref["seq_lens"])
    # gap 0 of the bridged call is the main rule, bit for bit
    kept0 = torch.empty_like(out["kept"])
    kept1 = torch.empty_like(out["kept"])
    K.kara_select_chunks_bridged(cfg, 0, out["scores"], kept0)
    K.kara_select_chunks(cfg, out["scores"], kept1)
    torch.cuda.synchronize()
    assert torch.equal(kept0, kept1)
    print(f"{s.name}: gap {gap}, {bridged} bridged positions", flush=True)
