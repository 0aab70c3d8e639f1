"""Pins of the oracle's Token2Chunk selection (a5-a8).

Rule (reading R9-R13 of the Kara abstract, where part of the selected KV
pairs grows into chunks): seeds = first s of the order (score desc, position asc),
spans [p-r, p+r] clipped and merged, fill = best positions outside the spans,
exactly B kept, ascending.
"""
import itertools
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import token2chunk_select
from tests.conftest import GOLDEN


def _golden():
    with open(os.path.join(GOLDEN, "select_hand.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["name"])
def test_hand_worked_cases(case):
    sel = token2chunk_select(np.array(case["scores"]), case["budget"], case["seeds"], case["radius"])
    assert sel.kept.tolist() == case["kept"]
    assert sel.seeds.tolist() == case["seed_list"]
    assert sel.fill.tolist() == case["fill"]


def _better(c, a, b):
    """a precedes b in the order (score desc, position asc)."""
    return c[a] > c[b] or (c[a] == c[b] and a < b)


def _check_invariants(c, B, s, r, sel):
    W = len(c)
    kept = sel.kept
    assert kept.size == B
    assert np.all(np.diff(kept) > 0) and (B == 0 or (kept[0] >= 0 and kept[-1] < W))
    keep = np.zeros(W, bool)
    keep[kept] = True
    # seeds are the s best positions: nothing outside beats any seed
    seeds = set(sel.seeds.tolist())
    assert len(seeds) == s
    for p in seeds:
        for x in range(W):
            if x not in seeds:
                assert _better(c, p, x)
    # every clipped seed span is inside keep and contiguous
    for p in seeds:
        span = list(range(max(0, p - r), min(W - 1, p + r) + 1))
        assert all(keep[span])
    # fill optimality: every fill position beats every dropped position
    for f in sel.fill:
        assert not sel.span[f]
        for x in np.flatnonzero(~keep):
            assert _better(c, int(f), int(x))


@settings(max_examples=300, deadline=None)
@given(st.data())
def test_invariants_on_random_inputs(data):
    W = data.draw(st.integers(1, 40))
    vals = data.draw(st.lists(st.integers(0, 6), min_size=W, max_size=W))   # many ties
    c = np.array(vals, dtype=np.float64) / 7.0
    r = data.draw(st.integers(0, 4))
    s = data.draw(st.integers(0, W // (2 * r + 1)))
    B = data.draw(st.integers(s * (2 * r + 1), W))
    sel = token2chunk_select(c, B, s, r)
    _check_invariants(c, B, s, r, sel)


@pytest.mark.parametrize("seed", range(20))
def test_brute_force_enumeration(seed):
    # Among all B-subsets containing the span union U, exactly one has every
    # non-U member beating every excluded position; it must be the oracle's.
    rng = np.random.default_rng(seed)
    W = int(rng.integers(3, 11))
    c = rng.integers(0, 4, size=W) / 4.0
    r = int(rng.integers(0, 2))
    s = int(rng.integers(0, W // (2 * r + 1) + 1))
    B = int(rng.integers(s * (2 * r + 1), W + 1))
    sel = token2chunk_select(c, B, s, r)
    U = set(np.flatnonzero(sel.span).tolist())
    winners = []
    for subset in itertools.combinations(range(W), B):
        S = set(subset)
        if not U <= S:
            continue
        extra = S - U
        out = set(range(W)) - S
        if all(_better(c, a, b) for a in extra for b in out):
            winners.append(sorted(S))
    assert len(winners) == 1
    assert sel.kept.tolist() == winners[0]


@pytest.mark.parametrize("seed", range(10))
def test_no_chunks_reduces_to_stable_top_budget(seed):
    rng = np.random.default_rng(100 + seed)
    W = int(rng.integers(1, 200))
    c = rng.integers(0, 20, size=W).astype(np.float64)
    B = int(rng.integers(1, W + 1))
    top = np.sort(np.lexsort((np.arange(W), -c))[:B])
    for s, r in [(0, 3), (min(B, 3), 0)]:
        assert token2chunk_select(c, B, s, r).kept.tolist() == top.tolist()


def test_rejects_bad_budget():
    with pytest.raises(ValueError):
        token2chunk_select(np.zeros(10), 11, 0, 0)
    with pytest.raises(ValueError):
        token2chunk_select(np.zeros(10), 5, 2, 1)      # 2 * 3 > 5
