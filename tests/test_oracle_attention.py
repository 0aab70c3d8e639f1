"""Pins of the oracle's paged decode attention (the consumer of the compacted
cache): closed forms, a library routine on a dense layout, invariances, the
equality between attention over the compacted pages and attention over the
kept rows gathered by hand, and planted mistakes."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import paged_decode_attention


def _dense_cache(rng, T, Hkv, d, bs, layers=1, perm=True):
    """A paged pool holding one sequence of T slots; returns (K, V, pools, table)."""
    nb = -(-T // bs) + 1
    K = rng.standard_normal((layers, T, Hkv, d))
    V = rng.standard_normal((layers, T, Hkv, d))
    kp = np.full((layers, nb, Hkv, bs, d), 99.0)
    vp = np.full((layers, nb, Hkv, bs, d), -99.0)
    table = rng.permutation(nb)[: -(-T // bs)] if perm else np.arange(-(-T // bs))
    for p in range(T):
        kp[:, table[p // bs], :, p % bs] = K[:, p]
        vp[:, table[p // bs], :, p % bs] = V[:, p]
    row = np.full(nb + 2, -1, dtype=np.int64)
    row[: table.size] = table
    return K, V, kp, vp, row[None]


def test_single_slot_returns_its_value_row():
    rng = np.random.default_rng(1)
    K, V, kp, vp, tb = _dense_cache(rng, 1, 2, 8, 4)
    q = rng.standard_normal((1, 1, 6, 8))
    o = paged_decode_attention(q, kp, vp, tb, [1], 4)
    for h in range(6):
        assert np.array_equal(o[0, 0, h], V[0, 0, h // 3])


def test_equal_keys_average_the_values():
    rng = np.random.default_rng(2)
    K, V, kp, vp, tb = _dense_cache(rng, 37, 1, 16, 8)
    kp[:] = 0.25                     # every key the same
    q = rng.standard_normal((1, 1, 2, 16))
    o = paged_decode_attention(q, kp, vp, tb, [37], 8)
    np.testing.assert_allclose(o[0, 0, 0], V[0, :, 0].mean(0), rtol=1e-13, atol=1e-14)


def test_two_slots_closed_form():
    rng = np.random.default_rng(3)
    K, V, kp, vp, tb = _dense_cache(rng, 2, 1, 32, 16)
    q = rng.standard_normal((1, 1, 1, 32))
    z = q[0, 0, 0] @ (K[0, 0, 0] - K[0, 1, 0]) / math.sqrt(32)
    w = 1 / (1 + math.exp(-z))
    o = paged_decode_attention(q, kp, vp, tb, [2], 16)
    np.testing.assert_allclose(o[0, 0, 0], w * V[0, 0, 0] + (1 - w) * V[0, 1, 0], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("T,Hq,Hkv,d,bs", [(53, 8, 2, 64, 16), (200, 7, 1, 128, 32), (17, 4, 4, 16, 1)])
def test_matches_library_attention_on_the_gathered_rows(T, Hq, Hkv, d, bs):
    rng = np.random.default_rng(T)
    K, V, kp, vp, tb = _dense_cache(rng, T, Hkv, d, bs, layers=2)
    q = rng.standard_normal((1, 2, Hq, d))
    o = paged_decode_attention(q, kp, vp, tb, [T], bs)
    G = Hq // Hkv
    for layer in range(2):
        qt = torch.from_numpy(q[0, layer]).reshape(Hq, 1, d)
        kt = torch.from_numpy(K[layer]).permute(1, 0, 2).repeat_interleave(G, 0).contiguous()
        vt = torch.from_numpy(V[layer]).permute(1, 0, 2).repeat_interleave(G, 0).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt).reshape(Hq, d).numpy()
        np.testing.assert_allclose(o[0, layer], ref, rtol=1e-12, atol=1e-13)


def test_empty_cache_gives_zero_and_lengths_are_per_sequence():
    rng = np.random.default_rng(5)
    K, V, kp, vp, tb = _dense_cache(rng, 20, 1, 8, 4)
    q = rng.standard_normal((3, 1, 1, 8))
    tbs = np.repeat(tb, 3, axis=0)
    o = paged_decode_attention(q, kp, vp, tbs, [0, 1, 20], 4)
    assert np.all(o[0] == 0)
    assert np.array_equal(o[1, 0, 0], V[0, 0, 0])
    o20 = paged_decode_attention(q[2:], kp, vp, tb, [20], 4)
    assert np.array_equal(o[2], o20[0])


def test_physical_block_placement_does_not_matter():
    rng = np.random.default_rng(6)
    T, bs = 45, 8
    K, V, kp, vp, tb = _dense_cache(np.random.default_rng(7), T, 2, 16, bs, perm=False)
    q = rng.standard_normal((1, 1, 4, 16))
    a = paged_decode_attention(q, kp, vp, tb, [T], bs)
    nb = kp.shape[1]
    perm = rng.permutation(nb)
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    kp2[:, perm] = kp
    vp2[:, perm] = vp
    tb2 = tb.copy()
    tb2[tb2 >= 0] = perm[tb2[tb2 >= 0]]
    b = paged_decode_attention(q, kp2, vp2, tb2, [T], bs)
    np.testing.assert_allclose(a, b, rtol=1e-14, atol=0)


@pytest.mark.parametrize("L,W,B,bs", [(0, 40, 10, 8), (13, 64, 20, 16), (37, 33, 33, 4), (5, 50, 7, 1)])
def test_compacted_cache_equals_hand_gathered_kept_rows(L, W, B, bs):
    # Attention over the compacted pages (first L + B slots) equals attention
    # over [prior rows, the kept window rows in ascending order] taken from the
    # cache before compaction.
    rng = np.random.default_rng(L * 131 + W)
    Hkv, Hq, d = 2, 4, 16
    T = L + W
    K, V, kp, vp, tb = _dense_cache(rng, T, Hkv, d, bs)
    kept = np.stack([np.stack([np.sort(rng.choice(W, B, replace=False)) for _ in range(Hkv)])])
    k2, v2 = kp.copy(), vp.copy()
    oracle.compact_paged_sequence(k2, v2, tb[0], L, kept, bs)
    row, freed, new_len = oracle.rewrite_block_table(tb[0], L, W, B, bs)
    assert new_len == L + B
    q = rng.standard_normal((1, 1, Hq, d))
    got = paged_decode_attention(q, k2, v2, row[None], [new_len], bs)
    G = Hq // Hkv
    for h in range(Hq):
        g = h // G
        rows = list(range(L)) + [L + int(j) for j in kept[0, g]]
        Kd, Vd = K[0, rows, g], V[0, rows, g]
        s = Kd @ q[0, 0, h] / math.sqrt(d)
        p = np.exp(s - s.max())
        np.testing.assert_allclose(got[0, 0, h], (p / p.sum()) @ Vd, rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------ mutants
def _mutant(mistake):
    def fn(q_dec, k_pool, v_pool, block_tables, seq_lens, block_size):
        S, layers, Hq, d = q_dec.shape
        Hkv = k_pool.shape[2]
        G = Hq // Hkv
        out = np.zeros((S, layers, Hq, d))
        for n in range(S):
            T = int(seq_lens[n]) - (1 if mistake == "drop_last_slot" else 0)
            if T <= 0:
                continue
            for layer in range(layers):
                for h in range(Hq):
                    g = h % Hkv if mistake == "interleaved_groups" else h // G
                    K = oracle.gather_window_rows(k_pool, block_tables[n], layer, g, 0, T, block_size)
                    V = oracle.gather_window_rows(v_pool, block_tables[n], layer, g, 0, T, block_size)
                    scale = 1 / d if mistake == "scale_1_over_d" else 1 / math.sqrt(d)
                    s = K @ q_dec[n, layer, h] * scale
                    p = np.exp(s - s.max())
                    if mistake == "unnormalised":
                        out[n, layer, h] = p @ V
                    else:
                        out[n, layer, h] = (p / p.sum()) @ V
        return out
    return fn


def _suite(fn):
    fails = 0
    rng = np.random.default_rng(11)
    K, V, kp, vp, tb = _dense_cache(rng, 2, 2, 32, 16)
    q = rng.standard_normal((1, 1, 4, 32))
    o = fn(q, kp, vp, tb, [2], 16)
    for h in range(4):
        g = h // 2
        z = q[0, 0, h] @ (K[0, 0, g] - K[0, 1, g]) / math.sqrt(32)
        w = 1 / (1 + math.exp(-z))
        fails += not np.allclose(o[0, 0, h], w * V[0, 0, g] + (1 - w) * V[0, 1, g], rtol=1e-12)
    return fails


def test_real_attention_passes_suite():
    assert _suite(paged_decode_attention) == 0


@pytest.mark.parametrize("mistake", ["drop_last_slot", "interleaved_groups", "scale_1_over_d", "unnormalised"])
def test_attention_mutants_are_caught(mistake):
    assert _suite(_mutant(mistake)) > 0
