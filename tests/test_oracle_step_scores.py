"""Pin of the oracle's batch scoring branch (compress_step without
scores_override, through batch_unit_scores): which query heads, which layer,
which sequence and which window rows feed each unit's scores.

Kara's English abstract scores the KV pairs of the recent window with
bidirectional attention; readings R3/R4/R7: the unit (n, layer, g) uses the
window queries of query heads g*G .. g*G+G-1 and the K rows of logical slots
[L, L+W) of its own sequence, layer and KV head, read through the block table.

Every unit gets its own closed form.  Keys are (2 ln r_j, 0, 0, 0) and
queries (x, 0, 0, 0) with d = 4, so a logit is x ln r_j and a softmax row is
r_j^x / sum_j' r_j'^x, an exact ratio of integers.  The ratios r and the
exponents x differ from unit to unit and from head to head, and the slots
outside the windows hold other keys, so taking the wrong head slice, layer,
sequence or window start changes the scores.  Mutants of the branch, each
with one such mistake, must fail the same check.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle

S, LYR, HKV, G, D, W, BS = 2, 2, 2, 2, 4, 3, 2
HQ = HKV * G
PRIOR = (1, 4)            # windows [1, 4) and [4, 7): the first starts inside a block
PERMS = ((1, 2, 4), (4, 1, 2), (2, 4, 1), (1, 4, 2), (2, 1, 4), (4, 2, 1), (1, 2, 3), (3, 1, 2))
OUTSIDE_R = 7             # ratio of every key outside the windows


def _unit(n, layer, g):
    return (n * LYR + layer) * HKV + g


def _x(n, layer, h, i):
    """Exponent of query i of query head h (0, 1 or 2), different per unit and head."""
    return (n + 2 * layer + h + i * (h + 1)) % 3


def _case():
    nb_seq = [-(-(L + W) // BS) for L in PRIOR]
    nb = sum(nb_seq) + 2
    perm = np.random.default_rng(11).permutation(nb)
    tables = np.full((S, max(nb_seq)), -1, dtype=np.int64)
    tables[0, :nb_seq[0]] = perm[:nb_seq[0]]
    tables[1, :nb_seq[1]] = perm[nb_seq[0]:nb_seq[0] + nb_seq[1]]
    k_pool = np.zeros((LYR, nb, HKV, BS, D))
    k_pool[..., 0] = 2.0 * math.log(OUTSIDE_R)
    for n in range(S):
        for layer in range(LYR):
            for g in range(HKV):
                r = PERMS[_unit(n, layer, g)]
                for j in range(W):
                    p = PRIOR[n] + j
                    k_pool[layer, tables[n, p // BS], g, p % BS, 0] = 2.0 * math.log(r[j])
    q = np.zeros((S, LYR, W, HQ, D))
    for n in range(S):
        for layer in range(LYR):
            for h in range(HQ):
                for i in range(W):
                    q[n, layer, i, h, 0] = _x(n, layer, h, i)
    return q, k_pool, tables


def _expected(n, layer, g):
    """c_j = sum_h sum_i r_j^x / sum_j' r_j'^x, with exact integer ratios."""
    r = PERMS[_unit(n, layer, g)]
    c = [Fraction(0)] * W
    for h in range(g * G, (g + 1) * G):
        for i in range(W):
            x = _x(n, layer, h, i)
            tot = sum(Fraction(rj) ** x for rj in r)
            for j in range(W):
                c[j] += Fraction(r[j]) ** x / tot
    return np.array([float(v) for v in c])


def _check(scores_of):
    """Number of units whose scores differ from their closed form."""
    q, k_pool, tables = _case()
    bad = 0
    for n in range(S):
        for layer in range(LYR):
            for g in range(HKV):
                got = scores_of(q, k_pool, tables, np.array(PRIOR), n, layer, g)
                bad += not np.allclose(got, _expected(n, layer, g), rtol=1e-12, atol=0)
    return bad


def test_closed_forms_differ_between_units():
    forms = {tuple(np.round(_expected(n, l, g), 12)) for n in range(S) for l in range(LYR) for g in range(HKV)}
    assert len(forms) == S * LYR * HKV


def test_batch_unit_scores_matches_closed_forms():
    assert _check(lambda q, k, t, p, n, l, g: oracle.batch_unit_scores(q, k, t, p, n, l, g, BS)) == 0


def test_compress_step_scores_match_closed_forms():
    q, k_pool, tables = _case()
    out = oracle.compress_step(q, k_pool, k_pool, tables, np.array(PRIOR), window=W, budget=W, seeds=0, radius=0,
                               block_size=BS)
    for n in range(S):
        for layer in range(LYR):
            for g in range(HKV):
                np.testing.assert_allclose(out["scores"][n, layer, g], _expected(n, layer, g), rtol=1e-12, atol=0)


def _mutant(mistake):
    def fn(q, k_pool, tables, prior, n, layer, g):
        Gm = q.shape[3] // k_pool.shape[2]
        heads = np.arange(g * Gm, (g + 1) * Gm)
        if mistake == "interleaved_groups":
            heads = np.arange(g, q.shape[3], k_pool.shape[2])
        elif mistake == "heads_of_next_group":
            heads = (heads + Gm) % q.shape[3]
        lq = 0 if mistake == "layer_0_queries" else layer
        lk = 0 if mistake == "layer_0_keys" else layer
        nq = 0 if mistake == "sequence_0_queries" else n
        start = int(prior[n])
        if mistake == "window_one_early":
            start -= 1
        elif mistake == "window_one_late":
            start += 1
        elif mistake == "window_at_zero":
            start = 0
        table = tables[0] if mistake == "table_of_sequence_0" else tables[n]
        qg = np.transpose(q[nq, lq][:, heads, :], (1, 0, 2))
        kw = oracle.gather_window_rows(k_pool, table, lk, g, start, q.shape[2], BS)
        return oracle.window_scores(qg, kw)
    return fn


@pytest.mark.parametrize("mistake", ["interleaved_groups", "heads_of_next_group", "layer_0_queries", "layer_0_keys",
                                     "sequence_0_queries", "window_one_early", "window_one_late", "window_at_zero",
                                     "table_of_sequence_0"])
def test_mutants_fail(mistake):
    try:
        bad = _check(_mutant(mistake))
    except (IndexError, ValueError):
        return                      # the mistake reads an unassigned slot: caught as well
    assert bad > 0, f"mutant {mistake} passes the closed forms"
