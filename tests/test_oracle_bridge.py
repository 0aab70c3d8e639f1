"""Pins of the oracle's Token2Chunk bridging variant (reading R31).

Rule: seeds and their clipped radius spans as in the main Token2Chunk rule;
seeds taken in ascending position; two neighbouring seeds p < p' that leave at
most ``gap`` positions between them (p' - p - 1 <= gap) also keep everything
between them; the rest of the budget is filled by the order (score desc,
position asc); exactly B kept, ascending.
"""
import itertools
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import Selection, chunk_bound, token2chunk_bridge_select, token2chunk_select
from tests.conftest import GOLDEN


def _golden():
    with open(os.path.join(GOLDEN, "select_bridge_hand.json")) as f:
        return json.load(f)["cases"]


def _better(c, a, b):
    return c[a] > c[b] or (c[a] == c[b] and a < b)


def _u_by_definition(W, seeds, r, gap):
    """U written per position: j is in U when a seed lies within r of it, or
    when the nearest seeds on both sides leave at most ``gap`` between them."""
    S = sorted(seeds)
    U = set()
    for j in range(W):
        if any(abs(j - p) <= r for p in S):
            U.add(j)
            continue
        left = [p for p in S if p < j]
        right = [p for p in S if p > j]
        if left and right and right[0] - left[-1] - 1 <= gap:
            U.add(j)
    return U


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["name"])
def test_hand_worked_cases(case):
    sel = token2chunk_bridge_select(np.array(case["scores"], float), case["budget"], case["seeds"],
                                    case["radius"], case["gap"])
    assert sel.kept.tolist() == case["kept"]
    assert sel.seeds.tolist() == case["seed_list"]
    assert sel.fill.tolist() == case["fill"]


@pytest.mark.parametrize("seed", range(25))
def test_brute_force_enumeration(seed):
    # Among all B-subsets containing U (from the per-position definition),
    # exactly one has every non-U member beating every excluded position.
    rng = np.random.default_rng(700 + seed)
    W = int(rng.integers(3, 12))
    c = rng.integers(0, 4, size=W) / 4.0
    r = int(rng.integers(0, 2))
    gap = int(rng.integers(0, 5))
    s = int(rng.integers(0, 4))
    while s > 0 and chunk_bound(s, r, gap) > W:
        s -= 1
    B = int(rng.integers(chunk_bound(s, r, gap), W + 1))
    sel = token2chunk_bridge_select(c, B, s, r, gap)
    order = sorted(range(W), key=lambda j: (-c[j], j))
    U = _u_by_definition(W, order[:s], r, gap)
    assert set(np.flatnonzero(sel.span).tolist()) == U
    winners = []
    for subset in itertools.combinations(range(W), B):
        S = set(subset)
        if not U <= S:
            continue
        extra, out = S - U, set(range(W)) - S
        if all(_better(c, a, b) for a in extra for b in out):
            winners.append(sorted(S))
    assert len(winners) == 1
    assert sel.kept.tolist() == winners[0]


@pytest.mark.parametrize("s,r,gap", [(1, 0, 5), (2, 0, 3), (3, 1, 4), (3, 2, 1), (4, 1, 6), (2, 3, 9)])
def test_chunk_bound_is_the_largest_union(s, r, gap):
    # Over every placement of s seeds in a window wide enough to hold them
    # apart, the largest |U| equals chunk_bound, and no placement exceeds it.
    W = s * (2 * r + 1) + (s - 1) * (gap + 2) + 2
    best = 0
    for seeds in itertools.combinations(range(W), s):
        best = max(best, len(_u_by_definition(W, seeds, r, gap)))
    assert best == chunk_bound(s, r, gap)


@settings(max_examples=200, deadline=None)
@given(st.data())
def test_gap_zero_reduces_to_main_rule_and_union_grows_with_gap(data):
    W = data.draw(st.integers(1, 48))
    vals = data.draw(st.lists(st.integers(0, 5), min_size=W, max_size=W))
    c = np.array(vals, dtype=np.float64) / 5.0
    r = data.draw(st.integers(0, 3))
    s = data.draw(st.integers(0, W // (2 * r + 1)))
    B = data.draw(st.integers(s * (2 * r + 1), W))
    a = token2chunk_bridge_select(c, B, s, r, 0)
    b = token2chunk_select(c, B, s, r)
    assert a.kept.tolist() == b.kept.tolist() and a.fill.tolist() == b.fill.tolist()
    prev = a.span
    for gap in range(1, 6):
        if chunk_bound(s, r, gap) > W:
            break
        cur = token2chunk_bridge_select(c, W, s, r, gap).span
        assert np.all(cur[prev]), "U must not lose positions when gap grows"
        prev = cur
    # every bridged hole between neighbouring seeds is fully kept
    gap = data.draw(st.integers(0, 6))
    if chunk_bound(s, r, gap) <= W:
        sel = token2chunk_bridge_select(c, W if B < chunk_bound(s, r, gap) else B, s, r, gap)
        keep = np.zeros(W, bool)
        keep[sel.kept] = True
        S = sorted(sel.seeds.tolist())
        for p, q in zip(S[:-1], S[1:]):
            if q - p - 1 <= gap:
                assert keep[p:q + 1].all()


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        token2chunk_bridge_select(np.zeros(10), 4, 2, 0, 3)       # bound 2 + 3 = 5 > 4
    with pytest.raises(ValueError):
        token2chunk_bridge_select(np.zeros(10), 5, 1, 0, -1)
    token2chunk_bridge_select(np.zeros(10), 5, 2, 0, 3)           # bound exactly 5 is fine


# ------------------------------------------------------------------ mutants
def _mutant(mistake):
    def fn(c, B, s, r, gap):
        W = len(c)
        order = sorted(range(W), key=lambda j: (-c[j], j))
        seeds = order[:s]
        span = np.zeros(W, bool)
        for p in seeds:
            span[max(0, p - r):min(W - 1, p + r) + 1] = True
        pairs = list(zip(seeds[:-1], seeds[1:])) if mistake == "score_order_pairs" else \
            list(zip(sorted(seeds)[:-1], sorted(seeds)[1:]))
        for a, b in pairs:
            between = b - a - 1
            ok = between < gap if mistake == "strict_gap" else between <= gap
            if mistake == "gap_counts_ends":
                ok = b - a + 1 <= gap
            if ok:
                span[a:b + 1] = True
        room = B - int(span.sum())
        fill = [j for j in order if not span[j]][:room]
        keep = span.copy()
        keep[fill] = True
        return Selection(kept=np.flatnonzero(keep), seeds=np.asarray(seeds), span=span, fill=np.asarray(fill))
    return fn


def _suite(fn):
    fails = 0
    for case in _golden():
        sel = fn(np.array(case["scores"], float), case["budget"], case["seeds"], case["radius"], case["gap"])
        fails += sel.kept.tolist() != case["kept"]
    return fails


def test_real_bridge_passes_suite():
    assert _suite(token2chunk_bridge_select) == 0


@pytest.mark.parametrize("mistake", ["score_order_pairs", "strict_gap", "gap_counts_ends"])
def test_bridge_mutants_are_caught(mistake):
    assert _suite(_mutant(mistake)) > 0
