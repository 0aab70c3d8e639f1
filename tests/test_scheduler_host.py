"""Host logic of the periodic scheduler: block allocator and due-set choice."""
import numpy as np
import pytest

from decode_kv_cache_amd.scheduler import TRACES, BlockAllocator, due_sequences


def test_allocator_hands_out_each_block_once_and_takes_back_only_used_ones():
    a = BlockAllocator(10)
    x = a.alloc(4)
    y = a.alloc(6)
    assert sorted(x + y) == list(range(10)) and a.in_use == 10
    with pytest.raises(MemoryError):
        a.alloc(1)
    a.release(x[:2])
    assert a.in_use == 8
    with pytest.raises(ValueError):
        a.release(x[:1])                 # already free
    with pytest.raises(ValueError):
        a.release([y[0], y[0]])          # twice in one call
    z = a.alloc(2)
    assert sorted(z) == sorted(x[:2])


def test_due_sequences_need_a_full_window_and_take_longest_tails_first():
    lengths = np.array([500, 600, 700, 800, 900])
    tails = np.array([95, 96, 200, 96, 150])
    active = np.array([True, True, True, False, True])
    assert due_sequences(lengths, tails, active, 96, 10) == [2, 4, 1]
    assert due_sequences(lengths, tails, active, 96, 2) == [2, 4]
    assert due_sequences(lengths, tails, active, 201, 4) == []


def test_trace_specs_fit_the_library_limits():
    from decode_kv_cache_amd import kara as K
    for spec in TRACES.values():
        c = K.kara_config(1, spec.num_layers, spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.window,
                          spec.budget, spec.seeds, spec.radius, spec.block_size, 0, 4096, 100)
        assert K.kara_check_config(c) == 0, spec.name
        assert spec.period > 0 and spec.max_per_tick > 0
