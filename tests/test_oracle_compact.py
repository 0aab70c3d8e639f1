"""Pins of the oracle's paged compaction and block-table rewrite (a9-a10).

Readings R14-R17 of the Kara abstract's PagedAttention adaptation: in-place
ordered gather of the kept rows into slots L..L+B-1; table entries of the
logical blocks past ceil((L+B)/bs) up to ceil((L+W)/bs) are freed in order.
"""
import json
import os

import numpy as np
import pytest

from oracle import (compact_paged_sequence, compact_window_rows, compress_step,
                    gather_window_rows, rewrite_block_table, token2chunk_select)
from tests.conftest import GOLDEN


def test_hand_worked_case():
    with open(os.path.join(GOLDEN, "compact_hand.json")) as f:
        case = json.load(f)["case"]
    nb, bs = case["num_blocks"], case["block_size"]
    pool = np.zeros((1, nb, 1, bs, 1), dtype=np.int64)
    for b in range(nb):
        for o in range(bs):
            pool[0, b, 0, o, 0] = 100 * b + o
    before = pool.copy()
    other = pool.copy() + 7
    table = np.array(case["table"])
    kept = np.array(case["kept"]).reshape(1, 1, -1)
    compact_paged_sequence(pool, other, table, case["prior_len"], kept, bs)
    expect = before.copy()
    for b, o, v in case["changed"]:
        expect[0, b, 0, o, 0] = v
    np.testing.assert_array_equal(pool, expect)
    row, freed, new_len = rewrite_block_table(table, case["prior_len"], case["window"], case["budget"], bs)
    assert row.tolist() == case["new_table"]
    assert freed.tolist() == case["freed"]
    assert new_len == case["seq_len"]


def _naive_gather(pool, table, L, kept, bs):
    """Slot-by-slot ordered gather through the table, one value at a time."""
    layers, nb, hkv, _, d = pool.shape
    out = pool.copy()
    for l in range(layers):
        for g in range(hkv):
            vals = {}
            for r, j in enumerate(kept[l, g]):
                p = L + int(j)
                for e in range(d):
                    vals[(r, e)] = pool[l, table[p // bs], g, p % bs, e]
            for (r, e), v in vals.items():
                p = L + r
                out[l, table[p // bs], g, p % bs, e] = v
    return out


@pytest.mark.parametrize("seed", range(8))
def test_matches_naive_ordered_gather(seed):
    rng = np.random.default_rng(seed)
    bs = int(rng.choice([1, 2, 4, 16]))
    L = int(rng.integers(0, 40))
    W = int(rng.integers(1, 50))
    B = int(rng.integers(1, W + 1))
    layers, hkv, d = 2, 3, 4
    nb_seq = -(-(L + W) // bs)
    nb = nb_seq + 5
    table = rng.permutation(nb)[:nb_seq]
    pool = rng.integers(0, 1 << 30, size=(layers, nb, hkv, bs, d))
    kept = np.stack([np.sort(rng.choice(W, B, replace=False)) for _ in range(layers * hkv)]).reshape(layers, hkv, B)
    k = pool.copy()
    v = pool.copy() * 3
    compact_paged_sequence(k, v, table, L, kept, bs)
    np.testing.assert_array_equal(k, _naive_gather(pool, table, L, kept, bs))
    np.testing.assert_array_equal(v, _naive_gather(pool * 3, table, L, kept, bs))
    # dense form agrees with the paged form
    for l in range(layers):
        for g in range(hkv):
            rows = gather_window_rows(pool, table, l, g, L, W, bs)
            after = gather_window_rows(k, table, l, g, L, W, bs)
            np.testing.assert_array_equal(after, compact_window_rows(rows, kept[l, g]))


@pytest.mark.parametrize("L,W,B,bs", [(0, 16, 16, 16), (5, 40, 40, 16), (3, 6, 2, 4), (16, 32, 1, 16),
                                      (15, 32, 1, 16), (31, 100, 20, 8), (0, 1, 1, 1)])
def test_freed_count_closed_form(L, W, B, bs):
    table = np.arange(-(-(L + W) // bs)) + 100
    row, freed, new_len = rewrite_block_table(table, L, W, B, bs)
    n = -(-(L + W) // bs) - (-(-(L + B) // bs))
    assert freed.size == n and new_len == L + B
    assert freed.tolist() == table[len(table) - n:].tolist()
    assert np.all(row[len(table) - n:] == -1) and np.all(row[:len(table) - n] == table[:len(table) - n])
    if B == W:
        assert n == 0


def test_keep_all_is_identity():
    rng = np.random.default_rng(3)
    pool = rng.integers(0, 99, size=(1, 6, 2, 4, 3))
    table = np.array([4, 1, 5])
    kept = np.tile(np.arange(7), (1, 2, 1))
    k = pool.copy()
    v = pool.copy()
    compact_paged_sequence(k, v, table, 3, kept, 4)
    np.testing.assert_array_equal(k, pool)


def test_compress_step_end_to_end_small():
    rng = np.random.default_rng(4)
    S, layers, Hq, Hkv, d, W, B, s, r, bs = 2, 2, 4, 2, 8, 20, 7, 1, 2, 4
    prior = np.array([5, 12])
    nbs = [-(-(int(L) + W) // bs) for L in prior]
    nb = sum(nbs)
    perm = rng.permutation(nb)
    tables = np.full((S, max(nbs)), -1)
    tables[0, :nbs[0]] = perm[:nbs[0]]
    tables[1, :nbs[1]] = perm[nbs[0]:]
    q = rng.standard_normal((S, layers, W, Hq, d))
    kp = rng.standard_normal((layers, nb, Hkv, bs, d))
    vp = rng.standard_normal((layers, nb, Hkv, bs, d))
    out = compress_step(q, kp, vp, tables, prior, window=W, budget=B, seeds=s, radius=r, block_size=bs)
    assert out["kept"].shape == (S, layers, Hkv, B)
    np.testing.assert_allclose(out["scores"].sum(-1), np.full((S, layers, Hkv), 2 * W), rtol=1e-12)
    for n in range(S):
        assert out["seq_lens"][n] == prior[n] + B
        for l in range(layers):
            for g in range(Hkv):
                assert out["kept"][n, l, g].tolist() == token2chunk_select(out["scores"][n, l, g], B, s, r).kept.tolist()
                before = gather_window_rows(kp, tables[n], l, g, int(prior[n]), W, bs)
                after = gather_window_rows(out["k_pool"], tables[n], l, g, int(prior[n]), B, bs)
                np.testing.assert_array_equal(after, before[out["kept"][n, l, g]])
