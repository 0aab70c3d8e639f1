"""Pins of the oracle's compaction with a tail of newer tokens (reading R28).

When the compressed window is the oldest part of the context not yet
compressed (the gist.science explainer of Kara, part 3: the schedule cleans
the back end of the current thought), T newer tokens follow it.  They move,
in order, right behind the B kept rows, and the table keeps the blocks of the
first L + B + T slots.  Pinned by a hand-worked case, a slot-by-slot gather
with the extended source list, the closed-form freed count, the reduction to
T = 0, and mutants.
"""
import json
import os

import numpy as np
import pytest

from oracle import compact_paged_sequence, compress_step, gather_window_rows, rewrite_block_table
from tests.conftest import GOLDEN


def _hand():
    with open(os.path.join(GOLDEN, "compact_tail_hand.json")) as f:
        return json.load(f)["case"]


def _hand_pool(case):
    nb, bs = case["num_blocks"], case["block_size"]
    pool = np.zeros((1, nb, 1, bs, 1), dtype=np.int64)
    for b in range(nb):
        for o in range(bs):
            pool[0, b, 0, o, 0] = 100 * b + o
    return pool


def _check_hand(compact, rewrite):
    """Failures of a (compact, rewrite) pair on the hand-worked case."""
    case = _hand()
    pool = _hand_pool(case)
    before = pool.copy()
    other = pool.copy()
    table = np.array(case["table"])
    kept = np.array(case["kept"]).reshape(1, 1, -1)
    compact(pool, other, table, case["prior_len"], kept, case["block_size"], window=case["window"],
            tail=case["tail"])
    expect = before.copy()
    for b, o, v in case["changed"]:
        expect[0, b, 0, o, 0] = v
    fails = int(not np.array_equal(pool, expect))
    row, freed, new_len = rewrite(table, case["prior_len"], case["window"], case["budget"], case["block_size"],
                                  case["tail"])
    fails += int(row.tolist() != case["new_table"]) + int(freed.tolist() != case["freed"])
    fails += int(new_len != case["seq_len"])
    return fails


def test_hand_worked_case():
    assert _check_hand(compact_paged_sequence, rewrite_block_table) == 0
    row, freed, new_len = rewrite_block_table(np.arange(8) + 50, 0, 16, 4, 4, 13)
    assert freed.tolist() == [55, 56, 57] and new_len == 17 and row.tolist() == [50, 51, 52, 53, 54, -1, -1, -1]


def _naive(pool, table, L, W, kept, T, bs):
    """Slot-by-slot ordered gather with the sources kept[0..B) then W..W+T-1."""
    layers, nb, hkv, _, d = pool.shape
    out = pool.copy()
    for l in range(layers):
        for g in range(hkv):
            src = [L + int(j) for j in kept[l, g]] + [L + W + t for t in range(T)]
            vals = {}
            for r, p in enumerate(src):
                for e in range(d):
                    vals[(r, e)] = pool[l, table[p // bs], g, p % bs, e]
            for (r, e), v in vals.items():
                p = L + r
                out[l, table[p // bs], g, p % bs, e] = v
    return out


@pytest.mark.parametrize("seed", range(10))
def test_matches_naive_gather_with_tail(seed):
    rng = np.random.default_rng(100 + seed)
    bs = int(rng.choice([1, 2, 4, 16]))
    L = int(rng.integers(0, 30))
    W = int(rng.integers(1, 40))
    B = int(rng.integers(1, W + 1))
    T = int(rng.integers(0, 35))
    layers, hkv, d = 2, 2, 3
    nb_seq = -(-(L + W + T) // bs)
    nb = nb_seq + 4
    table = rng.permutation(nb)[:nb_seq]
    pool = rng.integers(0, 1 << 30, size=(layers, nb, hkv, bs, d))
    kept = np.stack([np.sort(rng.choice(W, B, replace=False)) for _ in range(layers * hkv)]).reshape(layers, hkv, B)
    k, v = pool.copy(), pool.copy() * 5
    compact_paged_sequence(k, v, table, L, kept, bs, window=W, tail=T)
    np.testing.assert_array_equal(k, _naive(pool, table, L, W, kept, T, bs))
    np.testing.assert_array_equal(v, _naive(pool * 5, table, L, W, kept, T, bs))
    # the first L + B + T slots read in order are the prior rows, the kept rows, then the tail
    for l in range(layers):
        for g in range(hkv):
            got = gather_window_rows(k, table, l, g, 0, L + B + T, bs)
            want = np.concatenate([gather_window_rows(pool, table, l, g, 0, L, bs),
                                   gather_window_rows(pool, table, l, g, L, W, bs)[kept[l, g]],
                                   gather_window_rows(pool, table, l, g, L + W, T, bs)])
            np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("L,W,B,T,bs", [(0, 16, 4, 0, 16), (5, 40, 8, 3, 16), (3, 6, 2, 3, 4), (16, 32, 1, 15, 16),
                                        (15, 32, 1, 17, 16), (31, 100, 20, 200, 8), (0, 1, 1, 1, 1)])
def test_freed_count_closed_form_with_tail(L, W, B, T, bs):
    nb_total = -(-(L + W + T) // bs)
    table = np.arange(nb_total) + 100
    row, freed, new_len = rewrite_block_table(table, L, W, B, bs, T)
    n = nb_total - (-(-(L + B + T) // bs))
    assert freed.size == n and new_len == L + B + T
    assert freed.tolist() == table[nb_total - n:].tolist()
    assert np.all(row[nb_total - n:] == -1) and np.all(row[:nb_total - n] == table[:nb_total - n])


def test_zero_tail_is_the_plain_compaction():
    rng = np.random.default_rng(7)
    pool = rng.integers(0, 1000, size=(2, 9, 2, 4, 3))
    table = rng.permutation(9)[:7]
    kept = np.stack([np.sort(rng.choice(20, 6, replace=False)) for _ in range(4)]).reshape(2, 2, 6)
    a, b = pool.copy(), pool.copy()
    compact_paged_sequence(a, a.copy(), table, 5, kept, 4)
    compact_paged_sequence(b, b.copy(), table, 5, kept, 4, window=20, tail=0)
    np.testing.assert_array_equal(a, b)
    assert [x.tolist() if hasattr(x, "tolist") else x for x in rewrite_block_table(table, 5, 20, 6, 4)] == \
           [x.tolist() if hasattr(x, "tolist") else x for x in rewrite_block_table(table, 5, 20, 6, 4, 0)]


def test_compress_step_passes_tails_per_sequence():
    rng = np.random.default_rng(8)
    S, layers, Hq, Hkv, d, W, B, bs = 2, 1, 2, 1, 4, 12, 4, 4
    prior, tails = np.array([3, 9]), np.array([5, 0])
    nbs = [-(-(int(prior[n]) + W + int(tails[n])) // bs) for n in range(S)]
    perm = rng.permutation(sum(nbs))
    tables = np.full((S, max(nbs)), -1)
    tables[0, :nbs[0]] = perm[:nbs[0]]
    tables[1, :nbs[1]] = perm[nbs[0]:]
    q = rng.standard_normal((S, layers, W, Hq, d))
    kp = rng.integers(0, 1000, size=(layers, sum(nbs), Hkv, bs, d))
    out = compress_step(q, kp, kp * 3, tables, prior, window=W, budget=B, seeds=1, radius=1, block_size=bs,
                        tail_lens=tails, scores_override=rng.random((S, layers, Hkv, W)))
    for n in range(S):
        L, T = int(prior[n]), int(tails[n])
        assert out["seq_lens"][n] == L + B + T
        after = gather_window_rows(out["k_pool"], tables[n], 0, 0, L + B, T, bs)
        np.testing.assert_array_equal(after, gather_window_rows(kp, tables[n], 0, 0, L + W, T, bs))


# ---------------------------------------------------------------- mutants
def _mut_compact(mistake):
    def fn(k_pool, v_pool, table_row, prior_len, kept, block_size, *, window=None, tail=0):
        layers, kv_heads, B = kept.shape
        for pool in (k_pool, v_pool):
            for layer in range(layers):
                for g in range(kv_heads):
                    src = [prior_len + int(j) for j in kept[layer, g]]
                    if mistake == "tail_off_by_one":
                        src += [prior_len + window + t + 1 for t in range(tail)]
                    elif mistake == "tail_from_budget":
                        src += [prior_len + B + t for t in range(tail)]
                    elif mistake != "tail_not_moved":
                        src += [prior_len + window + t for t in range(tail)]
                    old = []
                    for p in src:
                        blk = int(table_row[p // block_size])
                        if blk < 0:
                            raise IndexError
                        old.append(pool[layer, blk, g, p % block_size].copy())
                    for r in range(len(src)):
                        p = prior_len + r
                        pool[layer, int(table_row[p // block_size]), g, p % block_size] = old[r]
    return fn


def _mut_rewrite(mistake):
    def fn(table_row, prior_len, window, budget, block_size, tail=0):
        row = np.array(table_row, copy=True)
        t_old = 0 if mistake == "freed_ignores_tail" else tail
        nb_old = -(-(prior_len + window + t_old) // block_size)
        nb_new = -(-(prior_len + budget + (0 if mistake == "kept_ignores_tail" else tail)) // block_size)
        freed = row[nb_new:nb_old].copy()
        row[nb_new:nb_old] = -1
        return row, freed, prior_len + budget + (0 if mistake == "length_ignores_tail" else tail)
    return fn


@pytest.mark.parametrize("mistake", ["tail_off_by_one", "tail_from_budget", "tail_not_moved"])
def test_compaction_mutants_fail(mistake):
    try:
        bad = _check_hand(_mut_compact(mistake), rewrite_block_table)
    except IndexError:
        return
    assert bad > 0


@pytest.mark.parametrize("mistake", ["freed_ignores_tail", "kept_ignores_tail", "length_ignores_tail"])
def test_rewrite_mutants_fail(mistake):
    fails = _check_hand(compact_paged_sequence, _mut_rewrite(mistake))
    # L = 0, W = 16, B = 4, T = 13, bs = 4: slots 0..28 in 8 blocks; afterwards
    # 17 slots in 5 blocks, so blocks 5, 6, 7 are freed and the length is 17
    row, freed, new_len = _mut_rewrite(mistake)(np.arange(8) + 50, 0, 16, 4, 4, 13)
    fails += int(freed.tolist() != [55, 56, 57]) + int(new_len != 17)
    fails += int(row.tolist() != [50, 51, 52, 53, 54, -1, -1, -1])
    assert fails > 0
