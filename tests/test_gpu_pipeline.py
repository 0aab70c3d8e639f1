"""Single-launch pipeline (kara_compress_fused), with the resident-key scorer
(bf16, head_dim 128, W <= 1024) and the staged-key scorer (other shapes, W up
to 256, 128 for fp32 rows of head_dim 128), against the three-call path and
the fp64 oracle: scores within the score tolerance of the oracle and equal to
the three-call path's; kept lists, pools, block tables, lengths and freed
blocks bit for bit; the done counters back to zero after every call."""
import numpy as np
import pytest
import torch

import oracle
from decode_kv_cache_amd import kara as K
from decode_kv_cache_amd.workloads import KaraShape, make_workload, shape_by_name
from tests.kara_harness import SCORE_RTOL, Outputs, bits, config_of, run_step, score_errors, unit_inputs

pytestmark = pytest.mark.gpu

SHAPES = [
    KaraShape("pipe_ragged", 301, num_seqs=3, num_layers=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
              window=200, budget=40, seeds=3, radius=2, prior=("uniform", 5, 60)),
    KaraShape("pipe_g7_plants", 302, num_seqs=2, num_layers=1, num_q_heads=7, num_kv_heads=1, head_dim=128,
              window=300, budget=60, seeds=2, radius=4, prior=("fixed", 17), plants=True),
    KaraShape("pipe_bs32_outliers", 303, num_seqs=3, num_layers=1, num_q_heads=4, num_kv_heads=2, head_dim=128,
              window=256, budget=51, seeds=3, radius=3, prior=("uniform", 100, 300), block_size=32,
              key_model="outliers"),
    KaraShape("pipe_w1024", 304, num_seqs=2, num_layers=3, num_q_heads=16, num_kv_heads=4, head_dim=128,
              window=1024, budget=204, seeds=8, radius=5, prior=("uniform", 0, 3000), plants=True),
    KaraShape("pipe_w1_keepall", 305, num_seqs=2, num_layers=1, num_q_heads=2, num_kv_heads=1, head_dim=128,
              window=33, budget=33, seeds=1, radius=0, prior=("fixed", 3), block_size=8),
    # one and three 16-row blocks per unit (the scorer's block loop runs zero and one times)
    KaraShape("pipe_one_block", 310, num_seqs=3, num_layers=1, num_q_heads=2, num_kv_heads=2, head_dim=128,
              window=16, budget=5, seeds=1, radius=2, prior=("uniform", 0, 40)),
    KaraShape("pipe_three_blocks_g3", 311, num_seqs=2, num_layers=2, num_q_heads=3, num_kv_heads=1, head_dim=128,
              window=16, budget=6, seeds=2, radius=1, prior=("fixed", 16), block_size=8),
    # windows of at most 256 keys outside bf16 / head_dim 128: the staged-key scorer
    shape_by_name("tiny"),
    KaraShape("pipe_f32_d64_g7_w256", 306, num_seqs=3, num_layers=2, num_q_heads=7, num_kv_heads=1, head_dim=64,
              window=256, budget=60, seeds=3, radius=4, dtype="f32", prior=("uniform", 0, 400), block_size=32,
              plants=True),
    KaraShape("pipe_bf16_d64_w200", 307, num_seqs=2, num_layers=2, num_q_heads=8, num_kv_heads=2, head_dim=64,
              window=200, budget=50, seeds=4, radius=3, prior=("uniform", 10, 90), key_model="outliers"),
    KaraShape("pipe_f32_d128_w128", 308, num_seqs=2, num_layers=1, num_q_heads=12, num_kv_heads=4, head_dim=128,
              window=128, budget=40, seeds=2, radius=5, dtype="f32", prior=("fixed", 37), block_size=8),
    KaraShape("pipe_f32_d64_w17", 309, num_seqs=3, num_layers=1, num_q_heads=3, num_kv_heads=1, head_dim=64,
              window=17, budget=9, seeds=1, radius=2, dtype="f32", prior=("uniform", 0, 20), block_size=4),
]


def _fused(wl, cfg, done, with_mask=True):
    out = Outputs(cfg, "cuda")
    K.kara_compress_fused(cfg, wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.prior_lens, out["scores"],
                          out["kept"], out["seq_lens"], out["freed"], out["num_freed"], done,
                          mask=out["mask"] if with_mask else None)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: s.name)
def test_pipeline_matches_three_calls_and_oracle(shape):
    s = shape
    wa = make_workload(s, "cuda")
    wb = make_workload(s, "cuda")
    cfg = config_of(wa)
    assert K.kara_compress_fused_supported(cfg) == 1
    qh = wa.q.float().double().cpu().numpy()
    kh = wa.k_pool.float().double().cpu().numpy()
    k0, v0 = bits(wa.k_pool), bits(wa.v_pool)
    _, ref = run_step(wa, cfg)
    done = torch.zeros(s.num_seqs, dtype=torch.int32, device="cuda")
    got = _fused(wb, cfg, done)
    assert got.guards_intact()
    assert torch.all(done == 0)
    c_gpu = got["scores"].cpu().numpy()
    assert np.array_equal(c_gpu, ref["scores"].cpu().numpy()), "scores differ from kara_score_window"
    for n in range(s.num_seqs):
        for layer in range(s.num_layers):
            for g in range(s.num_kv_heads):
                qg, kw = unit_inputs(qh, kh, wa, n, layer, g)
                assert score_errors(c_gpu[n, layer, g], oracle.window_scores(qg, kw)).max() <= SCORE_RTOL
    for k in ("kept", "mask", "seq_lens", "num_freed", "freed"):
        assert torch.equal(got[k], ref[k]), k
    assert np.array_equal(bits(wb.k_pool), bits(wa.k_pool))
    assert np.array_equal(bits(wb.v_pool), bits(wa.v_pool))
    assert torch.equal(wb.block_tables, wa.block_tables)
    # and against the oracle applied to the GPU's scores
    o = oracle.compress_step(np.zeros((s.num_seqs, s.num_layers, s.window, s.num_q_heads, 1)), k0, v0,
                             wa.host_tables, wa.host_prior_lens, window=s.window, budget=s.budget, seeds=s.seeds,
                             radius=s.radius, block_size=s.block_size, scores_override=c_gpu)
    assert np.array_equal(o["kept"], got["kept"].cpu().numpy())
    assert np.array_equal(o["k_pool"], bits(wb.k_pool))
    assert np.array_equal(o["v_pool"], bits(wb.v_pool))
    assert np.array_equal(o["block_tables"], wb.block_tables.cpu().numpy())


def test_pipeline_twice_in_a_row_reuses_the_counters():
    s = SHAPES[0]
    done = torch.zeros(s.num_seqs, dtype=torch.int32, device="cuda")
    first = None
    for _ in range(2):
        wl = make_workload(s, "cuda")
        cfg = config_of(wl)
        out = _fused(wl, cfg, done, with_mask=False)
        assert torch.all(done == 0)
        cur = (out["kept"].cpu(), bits(wl.k_pool), wl.block_tables.cpu(), out["seq_lens"].cpu())
        if first is not None:
            for a, b in zip(first, cur):
                assert np.array_equal(np.asarray(a), np.asarray(b))
        first = cur


def test_pipeline_not_offered_outside_its_shapes():
    for s in (SHAPES[0].with_(head_dim=64, window=300), SHAPES[0].with_(dtype="f32", window=129),
              SHAPES[0].with_(dtype="f32", head_dim=64, window=257), SHAPES[0].with_(window=2048, budget=410)):
        wl = make_workload(s.with_(num_seqs=1), "cuda")
        cfg = config_of(wl)
        assert K.kara_compress_fused_supported(cfg) == 0
        done = torch.zeros(1, dtype=torch.int32, device="cuda")
        with pytest.raises(K.KaraError) as e:
            _fused(wl, cfg, done)
        assert e.value.status == -5
