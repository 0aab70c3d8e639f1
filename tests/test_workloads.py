"""The seeded synthetic inputs (decode_kv_cache_amd.workloads): reproducible,
keyed per (shape, sequence, layer, tensor), rounded to bf16 by
round-to-nearest-even, with the planted runs, outlier channels and canaries
the recipe states.  CPU only."""
import math

import numpy as np
import pytest
import torch

from decode_kv_cache_amd import workloads as wlm
from decode_kv_cache_amd.workloads import KaraShape, make_workload

BASE = KaraShape("synth_base", 701, num_seqs=3, num_layers=2, num_q_heads=4, num_kv_heads=2, head_dim=64,
                 window=96, budget=24, seeds=2, radius=2, prior=("fixed", 21), block_size=8)


def _bits(t):
    return t.view(torch.int16).numpy() if t.dtype == torch.bfloat16 else t.view(torch.int32).numpy()


def _window_rows(wl, pool, n, layer):
    blk, off = wl.window_slot_index(n)
    return pool[layer][torch.from_numpy(blk.astype(np.int64)), :, torch.from_numpy(off.astype(np.int64)), :]


def test_reproducible():
    a, b = make_workload(BASE), make_workload(BASE)
    for x, y in ((a.q, b.q), (a.k_pool, b.k_pool), (a.v_pool, b.v_pool), (a.block_tables, b.block_tables),
                 (a.prior_lens, b.prior_lens)):
        assert np.array_equal(_bits(x) if x.is_floating_point() else x.numpy(),
                              _bits(y) if y.is_floating_point() else y.numpy())


def test_values_are_keyed_per_sequence_and_layer():
    """A sequence's window rows and queries depend on (shape id, sequence,
    layer, tensor) only: a batch with one more sequence leaves the others'
    data as it was, while their block ids may move."""
    small, big = make_workload(BASE.with_(num_seqs=2)), make_workload(BASE)
    for n in range(2):
        for layer in range(BASE.num_layers):
            assert np.array_equal(_bits(small.q[n, layer]), _bits(big.q[n, layer]))
            assert np.array_equal(_bits(_window_rows(small, small.k_pool, n, layer)),
                                  _bits(_window_rows(big, big.k_pool, n, layer)))
    # and different (sequence, layer) pairs do not repeat each other's draws
    assert not np.array_equal(_bits(big.q[0, 0]), _bits(big.q[1, 0]))
    assert not np.array_equal(_bits(big.q[0, 0]), _bits(big.q[0, 1]))


def _rne_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 by round-to-nearest-even on the bit pattern (finite values)."""
    b = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return r.astype(np.uint16).view(np.int16)


def test_bf16_values_are_the_fp32_draws_rounded_to_nearest_even():
    wl = make_workload(BASE)
    n, layer = 1, 1
    qn = torch.randn((BASE.window, BASE.num_q_heads, BASE.head_dim),
                     generator=wlm._torch_gen("cpu", BASE.shape_id, n, layer, wlm._TAG_Q), dtype=torch.float32)
    assert np.array_equal(_bits(wl.q[n, layer]), _rne_bf16_bits(qn.numpy()))
    kn = torch.randn((BASE.window, BASE.num_kv_heads, BASE.head_dim),
                     generator=wlm._torch_gen("cpu", BASE.shape_id, n, layer, wlm._TAG_K), dtype=torch.float32)
    assert np.array_equal(_bits(_window_rows(wl, wl.k_pool, n, layer)), _rne_bf16_bits(kn.numpy()))


def test_fp32_shapes_keep_the_draws():
    s = BASE.with_(dtype="f32")
    wl = make_workload(s)
    qn = torch.randn((s.window, s.num_q_heads, s.head_dim),
                     generator=wlm._torch_gen("cpu", s.shape_id, 0, 0, wlm._TAG_Q), dtype=torch.float32)
    assert torch.equal(wl.q[0, 0], qn)


@pytest.mark.parametrize("seed", range(40))
def test_planted_runs_do_not_overlap(seed):
    rng = np.random.default_rng(seed)
    W = int(rng.integers(260, 2048))
    starts, lens = wlm._plant_runs(np.random.default_rng(1000 + seed), W)
    assert len(starts) == 6 and ((lens >= 5) & (lens <= 40)).all()
    assert starts[0] >= 0 and starts[-1] + lens[-1] <= W
    assert (starts[1:] >= starts[:-1] + lens[:-1] + 1).all()      # a gap of at least one key


def test_planted_keys_and_queries_sit_at_cosine_08_with_the_direction():
    s = BASE.with_(plants=True, window=300, budget=60)
    n, layer, g = 2, 1, 1
    gk = wlm._torch_gen("cpu", s.shape_id, n, layer, wlm._TAG_K)
    kn = torch.randn((s.window, s.num_kv_heads, s.head_dim), generator=gk, dtype=torch.float32)
    u = torch.randn((s.num_kv_heads, s.head_dim), generator=wlm._torch_gen("cpu", s.shape_id, n, layer, wlm._TAG_U),
                    dtype=torch.float32)
    u = u / u.norm(dim=-1, keepdim=True)
    starts, lens = wlm._plant_runs(np.random.default_rng(wlm._seed(s.shape_id, n, layer, g, 0x9A)), s.window)
    tilted = wlm._tilt(kn[:, g], u[g].expand(s.window, s.head_dim))
    cos = (tilted @ u[g]) / tilted.norm(dim=-1)
    for a, b in zip(starts, lens):
        assert torch.allclose(cos[a:a + b], torch.full((int(b),), 0.8), atol=1e-6)
        assert torch.allclose(tilted[a:a + b].norm(dim=-1), kn[a:a + b, g].norm(dim=-1), rtol=1e-6)
    # the stored (bf16) keys of the runs keep that direction, the others do not
    wl = make_workload(s)
    kw = _window_rows(wl, wl.k_pool, n, layer)[:, g].float()
    cw = (kw @ u[g]) / kw.norm(dim=-1)
    inside = np.zeros(s.window, bool)
    for a, b in zip(starts, lens):
        inside[a:a + b] = True
    assert torch.allclose(cw[torch.from_numpy(inside)], torch.tensor(0.8), atol=1e-2)
    assert float(cw[torch.from_numpy(~inside)].abs().mean()) < 0.3
    # every window query of the group shares the direction
    qg = wl.q[n, layer, :, g * s.group:(g + 1) * s.group].float()
    cq = (qg @ u[g]) / qg.norm(dim=-1)
    assert torch.allclose(cq, torch.tensor(0.8), atol=1e-2)


def test_outlier_channels_are_fixed_per_layer_and_head():
    s = BASE.with_(key_model="outliers")
    wl = make_workload(s)
    for layer in range(s.num_layers):
        for g in range(s.num_kv_heads):
            ch = np.random.default_rng(wlm._seed(s.shape_id, layer, g, 7)).choice(s.head_dim, 4, replace=False)
            for n in range(s.num_seqs):
                kn = torch.randn((s.window, s.num_kv_heads, s.head_dim),
                                 generator=wlm._torch_gen("cpu", s.shape_id, n, layer, wlm._TAG_K),
                                 dtype=torch.float32)[:, g]
                scale = torch.ones(s.head_dim)
                scale[torch.from_numpy(ch)] = 8.0
                stored = _window_rows(wl, wl.k_pool, n, layer)[:, g]
                assert np.array_equal(_bits(stored), _rne_bf16_bits((kn * scale).numpy()))


def test_slots_outside_the_windows_hold_the_canary():
    wl = make_workload(BASE)
    touched = np.zeros((wl.num_blocks, BASE.block_size), bool)
    for n in range(BASE.num_seqs):
        L = int(wl.host_prior_lens[n])
        for p in range(L - L % BASE.block_size, L + BASE.window):
            touched[wl.host_tables[n, p // BASE.block_size], p % BASE.block_size] = True
    kb = _bits(wl.k_pool)                                  # [layers][blocks][Hkv][bs][d]
    canary = np.int16(wlm.CANARY_BF16_BITS - 0x10000)
    for blk in range(wl.num_blocks):
        for off in range(BASE.block_size):
            rows = kb[:, blk, :, off, :]
            assert (rows == canary).all() != touched[blk, off]


def test_block_tables_are_a_permutation_of_the_pool():
    wl = make_workload(BASE)
    used = np.concatenate([wl.host_tables[n][wl.host_tables[n] >= 0] for n in range(BASE.num_seqs)])
    assert sorted(used.tolist()) == list(range(wl.num_blocks))
    for n in range(BASE.num_seqs):
        need = math.ceil((int(wl.host_prior_lens[n]) + BASE.window) / BASE.block_size)
        assert (wl.host_tables[n, :need] >= 0).all() and (wl.host_tables[n, need:] == -1).all()
