"""Plain fp64 CPU oracle of Kara's decode-time window-compression step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test suite, the package smoke check and the
benchmark's ``cpu_baseline`` leg use it.  It shares no code, table or constant
with the HIP path and imports nothing from the package.

Sources (cited by page title and section; the pages give no equations):

* [Kara-abs]  "Kara: Efficient Reasoning LLM Serving via Sliding-Window KV
  Cache Compression", the authors' English abstract (shd-paper.top, section
  "摘要（原文）"; repeated on fugumt.com).  It fixes: compression runs at decode
  time on the most recently generated context only; KV pairs in that window
  are scored and selected with *bidirectional* attention; a Token2Chunk module
  grows a subset of the selected pairs into chunks; the result lives in a
  PagedAttention cache whose memory shrinks.
* [Kara-method]  same page, section "方法详解": the window module selects KV
  pairs while decoding, Token2Chunk turns selected pairs into chunks
  dynamically, and the design is adapted to PagedAttention.
* [gist-de]  gist.science/de explainer of the same paper (AI-written, not by
  the authors), sections "1. Die Zwei-Wege-Konversations-Bewertung" and
  "2. Das Token2Chunk-Modul": the score is a two-way attention measure
  inside the sliding window; chunks have no fixed size.

Readings taken where the pages are silent (each is stated where used):

* R1/R2  score of window key j = sum over the G query heads of the KV group
  and over all W window queries of softmax(q k^T / sqrt(d)) mass on column j;
  the softmax spans the W window keys only, unmasked (both directions),
  diagonal included.
* R3/R4  queries are the window's own query vectors as stored; query head h
  belongs to KV head floor(h / G).
* R9-R13 Token2Chunk rule: seeds = the first ``seeds`` positions of the order
  (score desc, position asc); every seed grows to the span
  [p - radius, p + radius] clipped to the window; spans are merged; the rest
  of the budget goes to the best positions outside the spans, by the same
  order; exactly ``budget`` positions are kept, listed in ascending order.
* R31     bridging variant (not the main rule): neighbouring seeds that leave
  at most ``gap`` positions between them are joined by keeping everything in
  between (the lay explainers of KARA, part 2, describe keeping the tokens
  that lie between two important ones).
* R25/R26 the consumer (decode attention) reads every cached slot [0, seq_len)
  of the sequence through its block table, scale 1/sqrt(d), GQA as in R4; an
  empty cache yields a zero output.
* R14-R18 compaction is in place: logical slot L + r receives the row that
  sat in slot L + kept[r]; block-table entries past the new length are freed
  in ascending logical order and set to -1; every other byte is unchanged.
* R28     when the window is the oldest part of the context not yet
  compressed (the lay explainers, part 3, describe cleaning the back end of
  the current thought), the newer tokens behind it move down, in order,
  right after the kept rows.

Parity pins (``tests/test_oracle_*.py``; every function has at least one,
none is parity unpinned):

* window_scores            closed forms (tests/golden/scores_hand.json), the
                           W = 2 logistic, hard-softmax limits, invariants
                           (sum = G*W, identical keys), planted keys, mutants;
* token2chunk_select       hand cases and brute force over tiny windows;
* token2chunk_bridge_select, chunk_bound
                           hand cases (tests/golden/select_bridge_hand.json), a
                           per-position definition, exhaustive placements;
* gather_window_rows, compact_window_rows, compact_paged_sequence,
  rewrite_block_table      a hand-worked case, a naive slot-by-slot gather,
                           the closed-form freed count, with and without a tail
                           (tests/golden/compact_tail_hand.json), mutants;
* paged_decode_attention   closed forms, torch's attention on gathered rows,
                           invariances, mutants;
* batch_unit_scores, compress_step
                           per-unit closed forms that differ by head, layer,
                           sequence and window start, with mutants of each.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

__all__ = [
    "window_scores",
    "Selection",
    "token2chunk_select",
    "gather_window_rows",
    "compact_window_rows",
    "compact_paged_sequence",
    "rewrite_block_table",
    "batch_unit_scores",
    "compress_step",
]


# --------------------------------------------------------------------------
# a2-a4: bidirectional in-window attention scores  [Kara-abs], [gist-de §1]
# --------------------------------------------------------------------------
def window_scores(q_group, k_window):
    """Column mass of bidirectional in-window attention for one unit.

    Parameters
    ----------
    q_group : array [G, W, d]
        The window's query vectors of the G query heads that share one KV head.
    k_window : array [W, d]
        The window's key vectors of that KV head, in logical order.

    Returns
    -------
    c : float64 array [W]
        c[j] = sum_h sum_i softmax_j'(q[h,i] . k[j'] / sqrt(d))[j]   (R1, R2).

    Every value is upcast exactly to fp64; the softmax is taken per query row
    over all W window keys with no causal mask.  The row maximum is subtracted
    before exponentiation (this leaves the value unchanged and keeps exp in
    range).
    """
    q = np.asarray(q_group, dtype=np.float64)
    k = np.asarray(k_window, dtype=np.float64)
    if q.ndim != 3 or k.ndim != 2 or q.shape[1] != k.shape[0] or q.shape[2] != k.shape[1]:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape}")
    G, W, d = q.shape
    c = np.zeros(W, dtype=np.float64)
    if W == 0:
        return c
    inv_sqrt_d = 1.0 / math.sqrt(d)
    for h in range(G):
        logits = (q[h] @ k.T) * inv_sqrt_d          # [W queries, W keys]
        row_max = logits.max(axis=1, keepdims=True)
        weights = np.exp(logits - row_max)
        probs = weights / weights.sum(axis=1, keepdims=True)
        c += probs.sum(axis=0)                      # column mass
    return c


# --------------------------------------------------------------------------
# a5-a8: Token2Chunk selection  [Kara-abs], [Kara-method]; rule R9-R13
# --------------------------------------------------------------------------
@dataclass
class Selection:
    kept: np.ndarray        # int64 [budget], ascending window-relative positions
    seeds: np.ndarray       # int64 [seeds], in selection order (best first)
    span: np.ndarray        # bool [W], union of the clipped seed spans (U)
    fill: np.ndarray        # int64, singletons added outside U, best first (F)


def _order(scores):
    """Positions sorted by the total order (score descending, position ascending)."""
    vals = [float(x) for x in scores]
    return sorted(range(len(vals)), key=lambda j: (-vals[j], j))


def token2chunk_select(scores, budget, seeds, radius):
    """Select exactly ``budget`` window positions (R9-R13).

    1. seeds  = first ``seeds`` positions of the order (score desc, pos asc);
    2. U      = union over seeds p of [max(0, p - radius), min(W - 1, p + radius)];
    3. F      = first (budget - |U|) positions of the same order not in U;
    4. kept   = U and F together, ascending.
    Requires 0 <= seeds, 0 <= radius, seeds * (2 * radius + 1) <= budget <= W.
    """
    W = len(scores)
    if not (0 <= seeds and 0 <= radius and seeds * (2 * radius + 1) <= budget <= W):
        raise ValueError("need seeds*(2*radius+1) <= budget <= W")
    order = _order(scores)
    seed_pos = order[:seeds]
    span = np.zeros(W, dtype=bool)
    for p in seed_pos:
        lo = max(0, p - radius)
        hi = min(W - 1, p + radius)
        span[lo:hi + 1] = True
    room = budget - int(span.sum())
    fill = [j for j in order if not span[j]][:room]
    keep = span.copy()
    keep[fill] = True
    kept = np.flatnonzero(keep).astype(np.int64)
    assert kept.size == budget
    return Selection(kept=kept, seeds=np.asarray(seed_pos, dtype=np.int64),
                     span=span, fill=np.asarray(fill, dtype=np.int64))


def chunk_bound(seeds, radius, gap):
    """Largest possible |U| of the bridged rule: the clipped spans cover at most
    seeds*(2*radius+1) positions, and each of the seeds-1 bridges between
    neighbouring seeds adds at most max(0, gap - 2*radius) positions that no
    span covers."""
    return seeds * (2 * radius + 1) + max(0, seeds - 1) * max(0, gap - 2 * radius)


def token2chunk_bridge_select(scores, budget, seeds, radius, gap):
    """Token2Chunk with bridging (variant; reading R31 of the lay explainers).

    The explainers of the method ([gist-de] section "2. Das Token2Chunk-Modul",
    and its Japanese twin) describe a chunk as everything lying between two
    important positions, with no fixed size.  Reading taken here: take the
    seeds and their clipped radius spans as in ``token2chunk_select``, then
    list the seeds in ascending position; wherever two neighbouring seeds p < p'
    leave at most ``gap`` positions between them (p' - p - 1 <= gap), every
    position strictly between them joins U as well.  The fill and the kept list
    follow as before.  gap = 0 adds nothing, so the rule reduces to
    ``token2chunk_select``.  Requires 0 <= gap and
    chunk_bound(seeds, radius, gap) <= budget <= W.
    """
    W = len(scores)
    if not (0 <= seeds and 0 <= radius and 0 <= gap and chunk_bound(seeds, radius, gap) <= budget <= W):
        raise ValueError("need chunk_bound(seeds, radius, gap) <= budget <= W and gap >= 0")
    order = _order(scores)
    seed_pos = order[:seeds]
    span = np.zeros(W, dtype=bool)
    for p in seed_pos:
        span[max(0, p - radius):min(W - 1, p + radius) + 1] = True
    by_pos = sorted(seed_pos)
    for a, b in zip(by_pos[:-1], by_pos[1:]):
        if b - a - 1 <= gap:
            span[a:b + 1] = True
    room = budget - int(span.sum())
    fill = [j for j in order if not span[j]][:room]
    keep = span.copy()
    keep[fill] = True
    kept = np.flatnonzero(keep).astype(np.int64)
    assert kept.size == budget
    return Selection(kept=kept, seeds=np.asarray(seed_pos, dtype=np.int64),
                     span=span, fill=np.asarray(fill, dtype=np.int64))


# --------------------------------------------------------------------------
# a1: window addressing through a PagedAttention block table  [Kara-abs]
# --------------------------------------------------------------------------
def _slot(table_row, pos, block_size):
    blk = int(table_row[pos // block_size])
    if blk < 0:
        raise IndexError(f"logical position {pos} maps to an unassigned block")
    return blk, pos % block_size


def gather_window_rows(pool, table_row, layer, kv_head, start, count, block_size):
    """Rows of logical slots [start, start+count) of one (layer, kv head).

    ``pool`` is [layers][num_blocks][kv_heads][block_size][d]; a logical slot p
    lives in physical block table_row[p // block_size] at offset p % block_size.
    """
    out = []
    for p in range(start, start + count):
        blk, off = _slot(table_row, p, block_size)
        out.append(np.array(pool[layer, blk, kv_head, off], copy=True))
    if not out:
        return np.zeros((0,) + pool.shape[4:], dtype=pool.dtype)
    return np.stack(out)


# --------------------------------------------------------------------------
# a9: compaction  (R14, R15)
# --------------------------------------------------------------------------
def compact_window_rows(rows, kept):
    """Dense form of the in-place compaction of one unit's window.

    ``rows`` is [W, ...].  Returns a copy in which row r (r < len(kept)) holds
    the old row kept[r]; rows at and past len(kept) keep their old contents.
    """
    out = np.array(rows, copy=True)
    src = np.array(rows, copy=True)
    for r, j in enumerate(kept):
        out[r] = src[int(j)]
    return out


def compact_paged_sequence(k_pool, v_pool, table_row, prior_len, kept, block_size, *, window=None, tail=0):
    """Apply the compaction of every (layer, kv head) of one sequence, in place.

    ``kept`` is [layers][kv_heads][B].  For each (layer, head) and r < B, the
    K and V rows of logical slot prior_len + r become the old rows of slot
    prior_len + kept[r]; all old rows are read before any is written.

    ``tail`` > 0 (reading R28: the window is the oldest part of the context
    not yet compressed, and ``tail`` newer tokens follow it in the slots
    [prior_len + window, prior_len + window + tail)) moves those tokens, in
    order, right behind the kept rows: slot prior_len + B + t takes the old
    row of slot prior_len + window + t.  ``window`` is then required.
    """
    layers, kv_heads, B = kept.shape
    if tail < 0 or (tail > 0 and window is None):
        raise ValueError("a tail needs the window length, and cannot be negative")
    for pool in (k_pool, v_pool):
        for layer in range(layers):
            for g in range(kv_heads):
                src = [prior_len + int(j) for j in kept[layer, g]]
                src += [prior_len + window + t for t in range(tail)]
                old = []
                for p in src:
                    blk, off = _slot(table_row, p, block_size)
                    old.append(pool[layer, blk, g, off].copy())
                for r in range(len(src)):
                    blk, off = _slot(table_row, prior_len + r, block_size)
                    pool[layer, blk, g, off] = old[r]


# --------------------------------------------------------------------------
# a10: block-table rewrite and freed list  (R16, R17)
# --------------------------------------------------------------------------
def rewrite_block_table(table_row, prior_len, window, budget, block_size, tail=0):
    """Truncate one sequence's block table after compaction.

    Blocks holding logical slots < prior_len + budget + tail stay; the
    entries of logical blocks ceil((L+B+T)/bs) .. ceil((L+W+T)/bs)-1 are
    returned in that order as freed and replaced by -1 (T = tail, the newer
    tokens that followed the window and moved down behind the kept rows; 0
    when the window ends the sequence).  Returns (new_row, freed, new_len).
    """
    row = np.array(table_row, copy=True)
    nb_old = -(-(prior_len + window + tail) // block_size)
    nb_new = -(-(prior_len + budget + tail) // block_size)
    freed = row[nb_new:nb_old].copy()
    row[nb_new:nb_old] = -1
    return row, freed, prior_len + budget + tail


# --------------------------------------------------------------------------
# Consumer: one decode step of paged attention over the (compacted) cache
# --------------------------------------------------------------------------
def paged_decode_attention(q_dec, k_pool, v_pool, block_tables, seq_lens, block_size):
    """Attention of one new query per head over a sequence's cached slots.

    The Kara abstract ([Kara-abs]) places the compressed cache inside a
    PagedAttention store and claims lower KV memory and higher output
    throughput; the decode step that reads the cache is ordinary scaled
    dot-product attention over the logical slots [0, seq_len) reached through
    the block table (reading R25: the query attends every cached slot, no
    mask inside the cache; query head h reads KV head h // G as in R4).

    q_dec        [S][layers][Hq][d]
    k_pool/v_pool [layers][num_blocks][Hkv][block_size][d]
    block_tables [S][max_blocks];  seq_lens [S]
    Returns o [S][layers][Hq][d] in fp64:
        o = sum_j softmax_j(q . k_j / sqrt(d)) v_j ;  seq_len 0 gives o = 0
    (reading R26: an empty cache contributes nothing).
    """
    S, layers, Hq, d = q_dec.shape
    Hkv = k_pool.shape[2]
    G = Hq // Hkv
    out = np.zeros((S, layers, Hq, d), dtype=np.float64)
    for n in range(S):
        T = int(seq_lens[n])
        if T == 0:
            continue
        for layer in range(layers):
            for g in range(Hkv):
                K = gather_window_rows(k_pool, block_tables[n], layer, g, 0, T, block_size).astype(np.float64)
                V = gather_window_rows(v_pool, block_tables[n], layer, g, 0, T, block_size).astype(np.float64)
                for h in range(g * G, (g + 1) * G):
                    logits = K @ np.asarray(q_dec[n, layer, h], dtype=np.float64) / np.sqrt(d)
                    logits -= logits.max()
                    p = np.exp(logits)
                    p /= p.sum()
                    out[n, layer, h] = p @ V
    return out


# --------------------------------------------------------------------------
# The whole step over a batch
# --------------------------------------------------------------------------
def batch_unit_scores(q, k_pool, block_tables, prior_lens, n, layer, g, block_size):
    """Window scores of unit (sequence n, layer, KV head g) inside a batch.

    The unit's queries are the window queries of query heads g*G .. g*G+G-1 of
    sequence n and layer ``layer`` (reading R4: contiguous GQA groups), and its
    keys are the K rows of logical slots [L, L+W) of that sequence, layer and
    KV head, L = prior_lens[n], read through the sequence's block table
    (readings R3, R7).  Returns window_scores of the two.
    """
    _, _, W, Hq, _ = q.shape
    G = Hq // k_pool.shape[2]
    qg = np.transpose(q[n, layer, :, g * G:(g + 1) * G, :], (1, 0, 2))
    kw = gather_window_rows(k_pool, block_tables[n], layer, g, int(prior_lens[n]), W, block_size)
    return window_scores(qg, kw)


def compress_step(q, k_pool, v_pool, block_tables, prior_lens, *, window, budget,
                  seeds, radius, block_size, scores_override=None, gap=0, tail_lens=None):
    """Run a1-a10 for every sequence, layer and KV head.

    q            [S][layers][W][Hq][d]
    k_pool/v_pool [layers][num_blocks][Hkv][block_size][d]   (copied, not modified)
    block_tables [S][max_blocks] int
    prior_lens   [S] int
    scores_override  optional [S][layers][Hkv][W]: select from these scores
                 instead of the oracle's own (used to pin the selection and
                 compaction stages to scores computed elsewhere).
    gap          0: the main Token2Chunk rule; > 0: the bridging variant.
    tail_lens    optional [S]: newer tokens that follow each window and move
                 down behind its kept rows (see compact_paged_sequence).
    Returns a dict with scores, kept, k_pool, v_pool, block_tables, seq_lens,
    freed (list of arrays) and num_freed.
    """
    S, layers, W, Hq, d = q.shape
    Hkv = k_pool.shape[2]
    G = Hq // Hkv
    assert W == window
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    tables = np.array(block_tables, copy=True)
    scores = np.zeros((S, layers, Hkv, W), dtype=np.float64)
    kept = np.zeros((S, layers, Hkv, budget), dtype=np.int64)
    seq_lens = np.zeros(S, dtype=np.int64)
    freed, num_freed = [], np.zeros(S, dtype=np.int64)
    for n in range(S):
        L = int(prior_lens[n])
        for layer in range(layers):
            for g in range(Hkv):
                if scores_override is None:
                    scores[n, layer, g] = batch_unit_scores(q, k_pool, block_tables, prior_lens, n, layer, g,
                                                            block_size)
                else:
                    scores[n, layer, g] = np.asarray(scores_override[n, layer, g], dtype=np.float64)
                if gap == 0:
                    sel = token2chunk_select(scores[n, layer, g], budget, seeds, radius)
                else:
                    sel = token2chunk_bridge_select(scores[n, layer, g], budget, seeds, radius, gap)
                kept[n, layer, g] = sel.kept
        T = 0 if tail_lens is None else int(tail_lens[n])
        compact_paged_sequence(k_out, v_out, block_tables[n], L, kept[n], block_size, window=W, tail=T)
        row, fr, new_len = rewrite_block_table(block_tables[n], L, W, budget, block_size, tail=T)
        tables[n] = row
        freed.append(fr)
        num_freed[n] = fr.size
        seq_lens[n] = new_len
    return dict(scores=scores, kept=kept, k_pool=k_out, v_pool=v_out, block_tables=tables,
                seq_lens=seq_lens, freed=freed, num_freed=num_freed)
