"""Pins of the oracle's window scores (a2-a4) against closed forms and invariants.

Score of window key j = sum over the KV group's query heads and all window
queries of the softmax mass on j (bidirectional in-window attention, Kara
English abstract; reading R1/R2).
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import window_scores
from tests.conftest import GOLDEN

pytestmark = pytest.mark.filterwarnings("ignore")


def _golden():
    with open(os.path.join(GOLDEN, "scores_hand.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["name"])
def test_hand_derived_cases(case):
    q = np.array(case["q"], dtype=np.float64)
    k = np.array(case["k"], dtype=np.float64)
    assert q.shape == (case["G"], case["W"], case["d"])
    c = window_scores(q, k)
    np.testing.assert_allclose(c, case["expected"], rtol=1e-12, atol=0)


def _rand(seed, G, W, d, scale=1.0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((G, W, d)) * scale, rng.standard_normal((W, d)) * scale


@pytest.mark.parametrize("G,W,d,scale", [(1, 1, 4, 1.0), (2, 7, 8, 1.0), (3, 33, 16, 3.0), (4, 128, 64, 1.0)])
def test_each_row_is_a_distribution(G, W, d, scale):
    q, k = _rand(G * 1000 + W, G, W, d, scale)
    c = window_scores(q, k)
    assert np.all(c >= 0)
    assert abs(c.sum() - G * W) <= 1e-10 * G * W


def test_identical_keys_give_uniform_scores():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((3, 10, 8))
    k = np.tile(rng.standard_normal((1, 8)), (10, 1))
    np.testing.assert_allclose(window_scores(q, k), np.full(10, 3.0), rtol=1e-12)


def test_zero_queries_give_uniform_scores():
    rng = np.random.default_rng(2)
    k = rng.standard_normal((9, 4)) * 5
    np.testing.assert_allclose(window_scores(np.zeros((2, 9, 4)), k), np.full(9, 2.0), rtol=1e-12)


def test_single_key_window():
    rng = np.random.default_rng(3)
    np.testing.assert_allclose(window_scores(rng.standard_normal((5, 1, 8)), rng.standard_normal((1, 8))),
                               [5.0], rtol=1e-12)


def test_two_key_window_is_logistic():
    # W = 2: p(row -> key 0) = sigma(q . (k0 - k1) / sqrt(d))
    rng = np.random.default_rng(4)
    G, d = 3, 16
    q = rng.standard_normal((G, 2, d))
    k = rng.standard_normal((2, d))
    z = q @ (k[0] - k[1]) / math.sqrt(d)
    c0 = np.sum(1.0 / (1.0 + np.exp(-z)))
    c = window_scores(q, k)
    np.testing.assert_allclose(c, [c0, 2 * G - c0], rtol=1e-12)


def test_planted_key_ranks_first():
    rng = np.random.default_rng(5)
    G, W, d = 2, 40, 32
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    q = rng.standard_normal((G, W, d)) * 0.1 + u       # every query has q . u >= ~0.5
    k = rng.standard_normal((W, d))
    k[17] = 40.0 * u
    c = window_scores(q, k)
    assert int(np.argmax(c)) == 17
    assert c[17] > 0.5 * G * W                          # more than half of every row's mass


def test_hard_softmax_limit_counts_argmaxes():
    # Logit gaps of ~1e3 make every row one-hot on its argmax key, so c[j] is
    # the number of (head, query) rows whose best key is j; this also pins the
    # reduction axis (a transposed softmax would give all-ones).
    rng = np.random.default_rng(6)
    G, W, d = 2, 12, 12
    k = np.eye(W, d) * 3000.0
    best = rng.integers(0, W, size=(G, W))
    q = np.zeros((G, W, d))
    for h in range(G):
        for i in range(W):
            q[h, i, best[h, i]] = 1.0
            q[h, i, (best[h, i] + 1) % d] = 0.5
    c = window_scores(q, k)
    expect = np.bincount(best.ravel(), minlength=W).astype(float)
    np.testing.assert_allclose(c, expect, atol=1e-9)
    assert np.all(np.isfinite(c))


def test_query_permutation_invariance_and_key_equivariance():
    q, k = _rand(7, 3, 21, 8, 2.0)
    c = window_scores(q, k)
    rng = np.random.default_rng(8)
    pq = rng.permutation(21)
    np.testing.assert_allclose(window_scores(q[:, pq], k), c, rtol=1e-12)
    pk = rng.permutation(21)
    np.testing.assert_allclose(window_scores(q, k[pk]), c[pk], rtol=1e-12)


def test_group_is_sum_of_single_heads():
    q, k = _rand(9, 4, 17, 8, 1.5)
    total = sum(window_scores(q[h:h + 1], k) for h in range(4))
    np.testing.assert_allclose(window_scores(q, k), total, rtol=1e-12)


def test_shift_of_all_logits_in_a_row_changes_nothing():
    # Adding one vector to every key adds a per-row constant to the logits,
    # which the softmax removes.
    q, k = _rand(10, 2, 15, 6, 1.0)
    shift = np.random.default_rng(11).standard_normal(6) * 10
    np.testing.assert_allclose(window_scores(q, k + shift), window_scores(q, k), rtol=1e-9)


def test_huge_logits_stay_finite():
    q, k = _rand(12, 2, 30, 8, 60.0)    # logits of order 1e3
    c = window_scores(q, k)
    assert np.all(np.isfinite(c))
    assert abs(c.sum() - 60) < 1e-9


@pytest.mark.parametrize("seed", range(12))
def test_scalar_loops_on_tiny_inputs(seed):
    """Scalar loops with math.exp on tiny inputs (W <= 16, d <= 8, G <= 3):
    the softmax of every query row over the window keys, summed down each
    column, element by element, with no array arithmetic.  The closed forms
    above are the pins; this cross-checks the array code's indexing."""
    rng = np.random.default_rng(900 + seed)
    G, W, d = int(rng.integers(1, 4)), int(rng.integers(1, 17)), int(rng.integers(1, 9))
    q = rng.normal(size=(G, W, d)) * float(rng.choice([0.3, 1.0, 3.0]))
    k = rng.normal(size=(W, d))
    want = [0.0] * W
    for h in range(G):
        for i in range(W):
            logits = [sum(float(q[h, i, e]) * float(k[j, e]) for e in range(d)) / math.sqrt(d) for j in range(W)]
            top = max(logits)
            ex = [math.exp(x - top) for x in logits]
            tot = sum(ex)
            for j in range(W):
                want[j] += ex[j] / tot
    got = window_scores(q, k)
    assert np.allclose(got, np.array(want), rtol=1e-12, atol=0)
