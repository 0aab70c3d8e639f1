"""The C ABI library loads, exports every declared symbol, and validates its
arguments on the host (no GPU needed: every call here returns before any HIP
call)."""
import ctypes
import os
import re

import pytest

from decode_kv_cache_amd import kara as K
from decode_kv_cache_amd.workloads import SHAPES, shape_by_name
from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "kara.h")


def _declared(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kara_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = K.lib()
    names = _declared()
    assert len(names) >= 10
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(K.EXPORTED_SYMBOLS)


def test_probe_library_exports_its_declared_symbols():
    lib = ctypes.CDLL(os.path.join(ROOT, "decode_kv_cache_amd", "libkara_probes.so"))
    names = _declared(os.path.join(ROOT, "include", "kara_probes.h"))
    assert len(names) == 8
    for name in names:
        assert hasattr(lib, name), name


def _cfg(name="llama8b_b64", **kw):
    s = shape_by_name(name)
    c = K.make_config(s, max_blocks_per_seq=4096, num_blocks=100000)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_all_benchmark_shapes_are_valid():
    for s in SHAPES:
        assert K.kara_check_config(K.make_config(s, max_blocks_per_seq=4096, num_blocks=10)) == 0, s.name


@pytest.mark.parametrize("field,value", [
    ("num_seqs", -1), ("num_layers", 0), ("num_q_heads", 0), ("num_kv_heads", 0), ("num_q_heads", 30),
    ("head_dim", 96), ("head_dim", 256), ("window", 0), ("window", 8193), ("budget", 0), ("budget", 1025),
    ("seeds", -1), ("radius", -1), ("seeds", 20), ("block_size", 12), ("block_size", 512), ("dtype", 7),
    ("max_blocks_per_seq", 0), ("num_blocks", -1), ("max_blocks_per_seq", 63),
    ("max_blocks_per_seq", 2 ** 30 // 16 + 1),      # more than 2^30 logical slots at block size 16
])
def test_invalid_config_fields(field, value):
    assert K.kara_check_config(_cfg(**{field: value})) == -1


def test_logical_positions_fit_int32():
    assert K.kara_check_config(_cfg(max_blocks_per_seq=2 ** 30 // 16)) == 0
    assert K.kara_check_config(_cfg(max_blocks_per_seq=2 ** 30 // 16 + 1)) == -1


def test_query_rows_per_unit_are_bounded():
    # G * W <= 2^24: the kernels count a unit's query rows in int32
    assert K.kara_check_config(_cfg(num_q_heads=2048 * 8, window=8192, budget=100)) == 0      # G = 2048
    assert K.kara_check_config(_cfg(num_q_heads=2049 * 8, window=8192, budget=100)) == -1
    assert K.kara_check_config(_cfg(num_q_heads=2 ** 30, num_kv_heads=8)) == -1


def test_seed_span_constraint_is_exact():
    assert K.kara_check_config(_cfg(seeds=17, radius=5, budget=187)) == 0      # 17 * 11 = 187
    assert K.kara_check_config(_cfg(seeds=17, radius=5, budget=186)) == -1


def test_workspace_bytes_and_max_freed():
    c = _cfg()
    units = 64 * 32 * 8
    # bf16, head_dim 128, W <= 1024: single-pass scorer, no workspace
    assert K.kara_workspace_bytes(c) == 0
    # two-pass scorer: one fp32 log-sum-exp per query row, rows padded to 32
    c1 = _cfg(window=2048)
    assert K.kara_workspace_bytes(c1) == units * 4 * 2048 * 4
    c2 = _cfg(num_q_heads=28, num_kv_heads=4, window=300, budget=20, seeds=1, head_dim=64)  # G*W = 2100 -> 2112
    assert K.kara_workspace_bytes(c2) == 64 * 32 * 4 * 2112 * 4
    c3 = _cfg(dtype=1)
    assert K.kara_workspace_bytes(c3) == units * 4 * 1024 * 4
    # windows of at most 256 slots outside the resident-key scorer's shape: small single-pass scorer
    small = [_cfg(num_q_heads=28, num_kv_heads=4, window=33, budget=20, seeds=1, head_dim=64),
             _cfg(dtype=1, head_dim=64, window=256, budget=128),
             _cfg(dtype=1, head_dim=128, window=128, budget=64, seeds=4, radius=2),
             _cfg(head_dim=64, window=200, budget=100)]
    for cs in small:
        assert K.kara_workspace_bytes(cs) == 0 and K.kara_score_passes(cs) == 1
    # fp32 rows of head_dim 128 stage at most 128 keys; a longer window takes two passes
    assert K.kara_score_passes(_cfg(dtype=1, head_dim=128, window=129, budget=64, seeds=4, radius=2)) == 2
    assert K.kara_score_passes(_cfg(dtype=1, head_dim=64, window=257, budget=64, seeds=4, radius=2)) == 2
    assert K.kara_max_freed(c) == 1024 // 16 + 1
    assert K.kara_max_freed(_cfg(window=100, budget=90, block_size=32)) == 4 + 1
    assert K.kara_workspace_bytes(_cfg(window=0)) == 0
    assert K.kara_score_passes(c) == 1 and K.kara_score_passes(c1) == 2 and K.kara_score_passes(c3) == 2
    assert K.kara_score_passes(_cfg(window=0)) == 0
    assert K.kara_max_freed(_cfg(window=0)) == 0


def test_entry_points_reject_before_any_device_work():
    lib = K.lib()
    bad = _cfg(budget=5000)
    good = _cfg(window=2048)          # a configuration whose scorer needs a workspace
    n = None
    assert lib.kara_score_window(ctypes.byref(bad), n, n, n, n, n, n, 0, n) == -1
    assert lib.kara_select_chunks(ctypes.byref(bad), n, n, n, n) == -1
    assert lib.kara_compact_paged(ctypes.byref(bad), n, n, n, n, n, n, n, n, n) == -1
    assert lib.kara_validate_tables(ctypes.byref(bad), n, n, n, n) == -1
    assert lib.kara_score_window(ctypes.byref(good), n, n, n, n, n, n, 0, n) == -2
    assert lib.kara_select_chunks(ctypes.byref(good), n, n, n, n) == -2
    assert lib.kara_compact_paged(ctypes.byref(good), n, n, n, n, n, n, n, n, n) == -2
    assert lib.kara_validate_tables(ctypes.byref(good), n, n, n, n) == -2
    assert lib.kara_score_window(None, n, n, n, n, n, n, 0, n) == -2
    # workspace: a non-null fake pointer that is too small or misaligned never reaches the device
    p = ctypes.c_void_p(0x1000)
    assert lib.kara_score_window(ctypes.byref(good), p, p, p, p, p, p, 10, n) == -3
    assert lib.kara_score_window(ctypes.byref(good), p, p, p, p, p, ctypes.c_void_p(0x1010),
                                 K.kara_workspace_bytes(good), n) == -3
    # an empty batch is a no-op that touches nothing
    empty = _cfg(num_seqs=0)
    assert lib.kara_score_window(ctypes.byref(empty), n, n, n, n, n, n, 0, n) == 0
    assert lib.kara_select_chunks(ctypes.byref(empty), n, n, n, n) == 0
    assert lib.kara_compact_paged(ctypes.byref(empty), n, n, n, n, n, n, n, n, n) == 0


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5, 99):
        assert isinstance(K.kara_status_str(code), str) and K.kara_status_str(code)
    assert K.kara_last_hip_error() == 0


def test_chunk_bound_matches_the_union_bound():
    import oracle
    for s, r, gap in [(0, 0, 0), (1, 3, 50), (3, 1, 1), (3, 1, 2), (3, 1, 7), (24, 8, 40), (12, 7, 0)]:
        assert K.kara_chunk_bound(_cfg(seeds=s, radius=r), gap) == oracle.chunk_bound(s, r, gap)
    assert K.kara_chunk_bound(_cfg(), -1) == -1


def test_bridged_select_rejects_bad_gap_before_device_work():
    L = K.lib()
    c = _cfg(window=64, budget=20, seeds=3, radius=1)            # spans 9, bridges add <= 2*(gap-2)
    assert L.kara_select_chunks_bridged(ctypes.byref(c), -1, None, None, None, None) == -1
    assert L.kara_select_chunks_bridged(ctypes.byref(c), 65, None, None, None, None) == -1
    assert L.kara_select_chunks_bridged(ctypes.byref(c), 8, None, None, None, None) == -1    # 9 + 12 > 20
    assert L.kara_select_chunks_bridged(ctypes.byref(c), 7, None, None, None, None) == -2    # 9 + 10 <= 20


def test_allocation_free_pipeline_checks_before_device_work():
    """kara_compress_fused_noalloc: configuration, support, NULL pointers and
    the fixed scratch limit are all decided on the host, before any HIP call."""
    L = K.lib()
    n = None
    p = ctypes.c_void_p(0x1000)
    args = [p] * 11 + [n]                                                 # every pointer set, default stream
    assert L.kara_compress_fused_noalloc(ctypes.byref(_cfg(budget=5000)), *args) == -1
    assert L.kara_compress_fused_noalloc(ctypes.byref(_cfg(window=2048)), *args) == -5     # two-pass shape
    assert L.kara_compress_fused_noalloc(ctypes.byref(_cfg()), *([n] * 11 + [n])) == -2
    # one sequence past the fixed scratch; p is never dereferenced
    assert L.kara_compress_fused_noalloc(ctypes.byref(_cfg(num_seqs=65537, num_layers=1)), *args) == -6
    assert L.kara_compress_fused_noalloc(ctypes.byref(_cfg(num_seqs=0)), *args) == 0
    assert "scratch" in K.kara_status_str(-6)


def test_workspace_grows_with_the_shape():
    """The two-pass scorer's workspace never shrinks when the batch, the
    layers, the heads or the window grow (and is 0 wherever a single-pass
    scorer runs)."""
    base = dict(window=1500, budget=300, seeds=6, radius=4, head_dim=64)
    prev = None
    for S in (1, 2, 7, 64):
        w = K.kara_workspace_bytes(_cfg(num_seqs=S, **base))
        assert prev is None or w >= prev
        prev = w
    for field, values in (("num_layers", (1, 2, 32)), ("window", (1500, 2048, 4096, 8192))):
        prev = None
        for v in values:
            w = K.kara_workspace_bytes(_cfg(**dict(base, **{field: v})))
            assert w > 0 and (prev is None or w >= prev), (field, v)
            prev = w
    prev = None
    for G in (1, 2, 4, 8):
        w = K.kara_workspace_bytes(_cfg(num_q_heads=8 * G, num_kv_heads=8, **base))
        assert prev is None or w >= prev
        prev = w
    for W in (16, 128, 256):
        assert K.kara_workspace_bytes(_cfg(head_dim=64, window=W, budget=W // 2, seeds=1, radius=1)) == 0
