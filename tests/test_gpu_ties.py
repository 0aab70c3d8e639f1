"""Selection on the GPU through exact ties.

The Token2Chunk order compares scores as IEEE floats (-0 equals +0) and
breaks ties by the lower position (reading R30 of the Kara abstract's
"select informative KV pairs ... expand a subset into chunks"), so the result
is unique even when many scores are equal.  The radix selection takes the
keys equal to a cutoff by ascending position; these tests put exact ties on
both cutoffs (the s-th seed and the last singleton of the fill), use rows that
are entirely equal and mixes of +0 and -0, and check kara_select_chunks and
kara_select_chunks_bridged bit for bit against the oracle.  A full step over
windows whose keys are identical (or whose queries are zero) produces exactly
tied scores on the GPU itself; its selection and compaction must equal the
oracle's given those scores.
"""
import numpy as np
import pytest
import torch

import oracle
from decode_kv_cache_amd import kara as K
from decode_kv_cache_amd.workloads import KaraShape, make_workload
from tests.kara_harness import SCORE_RTOL, bits, run_step

pytestmark = pytest.mark.gpu


def _cfg(S, Lyr, Hkv, W, B, s, r):
    shape = KaraShape("ties", 900, num_seqs=S, num_layers=Lyr, num_q_heads=Hkv, num_kv_heads=Hkv, head_dim=64,
                      window=W, budget=B, seeds=s, radius=r)
    return K.make_config(shape, max_blocks_per_seq=-(-W // 16), num_blocks=1)


def _quantised(rng, units, W, levels):
    """Scores k/7 with k drawn from `levels` values: ties everywhere."""
    return (rng.integers(0, levels, size=(units, W)) / 7.0).astype(np.float32)


def _select(cfg, sc, gap):
    S, Lyr, Hkv, W, B = cfg.num_seqs, cfg.num_layers, cfg.num_kv_heads, cfg.window, cfg.budget
    scores = torch.from_numpy(sc.reshape(S, Lyr, Hkv, W)).cuda()
    kept = torch.full((S, Lyr, Hkv, B), -7, dtype=torch.int32, device="cuda")
    mask = torch.full((S, Lyr, Hkv, W), 0xA5, dtype=torch.uint8, device="cuda")
    if gap == 0:
        K.kara_select_chunks(cfg, scores, kept, mask)
    else:
        K.kara_select_chunks_bridged(cfg, gap, scores, kept, mask)
    torch.cuda.synchronize()
    return kept.cpu().numpy().reshape(-1, B), mask.cpu().numpy().reshape(-1, W)


def _oracle(c, B, s, r, gap):
    c = c.astype(np.float64)
    return oracle.token2chunk_select(c, B, s, r) if gap == 0 else oracle.token2chunk_bridge_select(c, B, s, r, gap)


def _cutoff_ties(c, sel, s):
    """(seed cutoff tied with a non-seed position, fill cutoff tied with a dropped position)"""
    c = c.astype(np.float64)
    seed_tie = s > 0 and any(c[j] == c[sel.seeds[-1]] for j in range(len(c)) if j not in set(sel.seeds.tolist()))
    kept = set(sel.kept.tolist())
    fill_tie = sel.fill.size > 0 and any(c[j] == c[sel.fill[-1]] for j in range(len(c)) if j not in kept)
    return seed_tie, fill_tie


CASES = [
    # (S, Lyr, Hkv, W, B, s, r, levels, gap)
    (2, 2, 2, 200, 40, 3, 2, 5, 0),
    (1, 4, 2, 1024, 204, 8, 5, 10, 0),
    (1, 4, 2, 1024, 204, 8, 5, 10, 12),
    (2, 1, 2, 300, 90, 4, 3, 3, 9),
    (1, 2, 2, 2048, 410, 12, 7, 12, 0),
    (1, 1, 4, 129, 17, 1, 8, 2, 0),
]


@pytest.mark.parametrize("S,Lyr,Hkv,W,B,s,r,levels,gap", CASES)
def test_quantised_scores_bit_exact(S, Lyr, Hkv, W, B, s, r, levels, gap):
    print(f"[ties] W={W} B={B} s={s} r={r} levels={levels} gap={gap}", flush=True)
    rng = np.random.default_rng(W * 31 + B + gap)
    cfg = _cfg(S, Lyr, Hkv, W, B, s, r)
    sc = _quantised(rng, S * Lyr * Hkv, W, levels)
    kept, mask = _select(cfg, sc, gap)
    seed_ties = fill_ties = 0
    for u in range(sc.shape[0]):
        sel = _oracle(sc[u], B, s, r, gap)
        assert kept[u].tolist() == sel.kept.tolist(), f"unit {u}"
        expect = np.zeros(W, np.uint8)
        expect[sel.kept] = 1
        assert np.array_equal(mask[u], expect)
        a, b = _cutoff_ties(sc[u], sel, s)
        seed_ties += a
        fill_ties += b
    # the cases are built so that the cutoffs really fall inside tied groups
    assert fill_ties == sc.shape[0]
    if s > 0:
        assert seed_ties == sc.shape[0]


@pytest.mark.parametrize("gap", [0, 6])
def test_all_equal_rows_and_signed_zeros(gap):
    S, Lyr, Hkv, W, B, s, r = 1, 1, 4, 160, 32, 2, 3
    cfg = _cfg(S, Lyr, Hkv, W, B, s, r)
    sc = np.zeros((4, W), np.float32)
    sc[0] = 1.0                                         # every score equal
    sc[1] = np.where(np.arange(W) % 3 == 0, -0.0, 0.0)  # +0 and -0 only
    rng = np.random.default_rng(5)
    sc[2] = np.where(rng.random(W) < 0.5, -0.0, 0.0)
    sc[2, rng.choice(W, 10, replace=False)] = 2.0 / 7.0  # a few winners over signed zeros
    sc[3] = np.float32(1e-30)                           # equal tiny scores
    kept, mask = _select(cfg, sc, gap)
    for u in range(4):
        sel = _oracle(sc[u], B, s, r, gap)
        assert kept[u].tolist() == sel.kept.tolist(), f"row {u}"
    # equal scores: pure position order, so the kept list is fixed by the rule
    first = _oracle(np.ones(W), B, s, r, gap).kept.tolist()
    assert kept[0].tolist() == first == kept[1].tolist()


def _tie_workload(name, sid, make_equal, **kw):
    shape = KaraShape(name, sid, **kw)
    wl = make_workload(shape, "cuda")
    bs = shape.block_size
    for n in range(shape.num_seqs):
        blk, off = wl.window_slot_index(n)
        blk_t = torch.from_numpy(blk.astype(np.int64)).cuda()
        off_t = torch.from_numpy(off.astype(np.int64)).cuda()
        for l in range(shape.num_layers):
            if make_equal == "keys":
                row = wl.k_pool[l][blk_t[0], :, off_t[0], :].clone()      # [Hkv][d]
                wl.k_pool[l][blk_t, :, off_t, :] = row[None].expand(len(blk), -1, -1)
            else:
                wl.q[n, l].zero_()
    torch.cuda.synchronize()
    return wl


TIE_SHAPES = [
    # single-pass scorer (bf16, d 128, W <= 1024)
    ("eq_keys_fused", 951, "keys", dict(num_seqs=2, num_layers=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
                                          window=300, budget=60, seeds=3, radius=4, prior=("uniform", 5, 40))),
    # two-pass scorer (d 64, W > 1024)
    ("eq_keys_two_pass", 952, "keys", dict(num_seqs=1, num_layers=2, num_q_heads=4, num_kv_heads=1, head_dim=64,
                                             window=1500, budget=300, seeds=5, radius=6, prior=("fixed", 9))),
    # fp32 tiny-like shape with zero queries
    ("zero_q_f32", 953, "queries", dict(num_seqs=1, num_layers=1, num_q_heads=4, num_kv_heads=2, head_dim=64,
                                          window=128, budget=32, seeds=2, radius=3, dtype="f32",
                                          prior=("fixed", 256))),
]


@pytest.mark.parametrize("name,sid,how,kw", TIE_SHAPES, ids=[t[0] for t in TIE_SHAPES])
def test_full_step_with_exactly_tied_scores(name, sid, how, kw):
    print(f"[ties] full step {name}", flush=True)
    wl = _tie_workload(name, sid, how, **kw)
    s = wl.shape
    k_before, v_before = bits(wl.k_pool), bits(wl.v_pool)
    cfg, out = run_step(wl)
    assert out.guards_intact()
    c = out["scores"].cpu().numpy()
    # identical keys (or zero queries): every row is uniform, so each unit's
    # scores are all equal -- exactly, on the GPU too -- and equal G in exact
    # arithmetic (the fp32 sums of G*W terms land within the score tolerance)
    flat = c.reshape(-1, s.window)
    assert np.all(flat == flat[:, :1]), "scores of a unit are not all equal"
    np.testing.assert_allclose(flat[:, 0], s.group, rtol=SCORE_RTOL)
    ref = oracle.compress_step(np.zeros((s.num_seqs, s.num_layers, s.window, s.num_q_heads, 1)), k_before, v_before,
                               wl.host_tables, wl.host_prior_lens, window=s.window, budget=s.budget, seeds=s.seeds,
                               radius=s.radius, block_size=s.block_size, scores_override=c)
    assert np.array_equal(out["kept"].cpu().numpy(), ref["kept"])
    assert np.array_equal(bits(wl.k_pool), ref["k_pool"])
    assert np.array_equal(bits(wl.v_pool), ref["v_pool"])
    assert np.array_equal(wl.block_tables.cpu().numpy(), ref["block_tables"])
    assert np.array_equal(out["seq_lens"].cpu().numpy(), ref["seq_lens"])
