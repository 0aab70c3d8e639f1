"""The oracle's pins must catch plausible mistakes.

Each mutant below is a copy of one oracle stage with one planted mistake (on
the CPU only).  The same closed-form and hand-derived checks that pin the
real oracle are run against it, and at least one must fail.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import token2chunk_select, window_scores
from tests.conftest import GOLDEN


# ---------------------------------------------------------------- scores
def _scores_suite(fn):
    """Return the number of failed checks of a window_scores-like function."""
    fails = 0
    with open(os.path.join(GOLDEN, "scores_hand.json")) as f:
        for case in json.load(f)["cases"]:
            c = fn(np.array(case["q"], float), np.array(case["k"], float))
            fails += not np.allclose(c, case["expected"], rtol=1e-12, atol=0)
    rng = np.random.default_rng(4)
    q = rng.standard_normal((3, 2, 16))
    k = rng.standard_normal((2, 16))
    z = q @ (k[0] - k[1]) / 4.0
    c0 = np.sum(1 / (1 + np.exp(-z)))
    fails += not np.allclose(fn(q, k), [c0, 6 - c0], rtol=1e-12)
    q = rng.standard_normal((2, 9, 8))
    k = rng.standard_normal((9, 8))
    fails += not abs(fn(q, k).sum() - 18) < 1e-9
    return fails


def _mk(mistake):
    def fn(q, k):
        G, W, d = q.shape
        c = np.zeros(W)
        heads = range(G - 1) if mistake == "drop_head" and G > 1 else range(G)
        for h in heads:
            scale = 1.0 / d if mistake == "scale_1_over_d" else 1.0 / math.sqrt(d)
            s = (q[h] @ k.T) * scale
            if mistake == "causal_mask":
                s = np.where(np.tril(np.ones((W, W), bool)), s, -np.inf)
            if mistake == "wrong_sign":
                s = -s
            axis = 0 if mistake == "softmax_over_queries" else 1
            e = np.exp(s - s.max(axis=axis, keepdims=True))
            p = e / e.sum(axis=axis, keepdims=True)
            if mistake == "row_sums":
                c += p.sum(axis=1)
            elif mistake == "mean_not_sum":
                c += p.mean(axis=0)
            elif mistake == "no_diagonal":
                c += p.sum(axis=0) - np.diag(p)
            else:
                c += p.sum(axis=0)
        return c
    return fn


def test_real_oracle_passes_suite():
    assert _scores_suite(window_scores) == 0


@pytest.mark.parametrize("mistake", ["drop_head", "scale_1_over_d", "causal_mask", "wrong_sign",
                                     "softmax_over_queries", "row_sums", "mean_not_sum", "no_diagonal"])
def test_score_mutants_are_caught(mistake):
    assert _scores_suite(_mk(mistake)) > 0


# ---------------------------------------------------------------- selection
def _select_suite(fn):
    fails = 0
    with open(os.path.join(GOLDEN, "select_hand.json")) as f:
        for case in json.load(f)["cases"]:
            try:
                kept = fn(np.array(case["scores"], float), case["budget"], case["seeds"], case["radius"])
                fails += list(kept) != case["kept"]
            except Exception:
                fails += 1
    return fails


def _sel_mutant(mistake):
    def fn(c, B, s, r):
        W = len(c)
        if mistake == "ties_by_higher_position":
            order = sorted(range(W), key=lambda j: (-c[j], -j))
        elif mistake == "ascending_scores":
            order = sorted(range(W), key=lambda j: (c[j], j))
        else:
            order = sorted(range(W), key=lambda j: (-c[j], j))
        span = np.zeros(W, bool)
        for p in order[:s]:
            lo, hi = p - r, p + r
            if mistake == "span_one_short":
                hi = p + r - 1
            if mistake == "no_clip":
                lo = lo % W
            span[max(lo, 0):min(hi, W - 1) + 1] = True
            if mistake == "no_clip" and p - r < 0:
                span[lo:] = True
        room = B - int(span.sum())
        if mistake == "fill_ignores_span":
            fill = order[:room]
        else:
            fill = [j for j in order if not span[j]][:room]
        keep = span.copy()
        keep[fill] = True
        out = np.flatnonzero(keep)
        if mistake == "unsorted":
            out = np.array(list(order[:s]) + [j for j in out if j not in order[:s]])
        return out
    return fn


def test_real_selection_passes_suite():
    assert _select_suite(lambda c, B, s, r: token2chunk_select(c, B, s, r).kept) == 0


@pytest.mark.parametrize("mistake", ["ties_by_higher_position", "ascending_scores", "span_one_short",
                                     "no_clip", "fill_ignores_span", "unsorted"])
def test_selection_mutants_are_caught(mistake):
    assert _select_suite(_sel_mutant(mistake)) > 0
