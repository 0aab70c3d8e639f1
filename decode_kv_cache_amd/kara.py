"""ctypes binding of libkara.so (C ABI in include/kara.h).

Argument marshalling only: every function checks tensor dtype, shape,
device and contiguity, then passes raw device pointers and the current HIP
stream to the library function of the same name.  All compute runs in the
library's HIP kernels; if the library is missing the import of any entry
point fails loudly (there is no fallback).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "KaraError", "kara_config", "make_config", "lib", "kara_check_config", "kara_workspace_bytes",
    "kara_max_freed", "kara_score_passes", "kara_score_window", "kara_select_chunks", "kara_chunk_bound",
    "kara_select_chunks_bridged", "kara_compact_paged", "kara_compact_paged_tail", "kara_decode_attention",
    "kara_decode_attention_splits",
    "kara_decode_attention_workspace_bytes", "kara_compress_fused", "kara_compress_fused_supported",
    "kara_compress_fused_noalloc",
    "kara_validate_tables", "kara_status_str", "kara_last_hip_error", "KARA_BF16", "KARA_F32",
    "EXPORTED_SYMBOLS",
]

KARA_BF16 = 0
KARA_F32 = 1
_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkara.so")
EXPORTED_SYMBOLS = ("kara_check_config", "kara_workspace_bytes", "kara_max_freed", "kara_score_passes",
                    "kara_score_window",
                    "kara_select_chunks", "kara_chunk_bound", "kara_select_chunks_bridged",
                    "kara_compact_paged", "kara_compact_paged_tail", "kara_decode_attention_workspace_bytes",
                    "kara_decode_attention_splits",
                    "kara_decode_attention", "kara_compress_fused_supported", "kara_compress_fused",
                    "kara_compress_fused_noalloc", "kara_validate_tables", "kara_status_str",
                    "kara_last_hip_error")


class KaraError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = f"{where}: status {status} ({kara_status_str(status)})"
        if status == -4:
            msg += f", hip error {kara_last_hip_error()}"
        super().__init__(msg)
        self.status = status


class kara_config(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_layers", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("window", ctypes.c_int32),
                ("budget", ctypes.c_int32), ("seeds", ctypes.c_int32), ("radius", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("dtype", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("num_blocks", ctypes.c_int64)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libkara.so from the package directory (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with `python -m decode_kv_cache_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.POINTER(kara_config)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        sig = {
            "kara_check_config": (i32, [P]),
            "kara_workspace_bytes": (sz, [P]),
            "kara_max_freed": (ctypes.c_int32, [P]),
            "kara_score_passes": (i32, [P]),
            "kara_score_window": (i32, [P, vp, vp, vp, vp, vp, vp, sz, vp]),
            "kara_select_chunks": (i32, [P, vp, vp, vp, vp]),
            "kara_chunk_bound": (ctypes.c_int64, [P, ctypes.c_int32]),
            "kara_select_chunks_bridged": (i32, [P, ctypes.c_int32, vp, vp, vp, vp]),
            "kara_compact_paged": (i32, [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
            "kara_compact_paged_tail": (i32, [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
            "kara_validate_tables": (i32, [P, vp, vp, vp, vp]),
            "kara_decode_attention_workspace_bytes": (sz, [P]),
            "kara_decode_attention_splits": (i32, [P]),
            "kara_decode_attention": (i32, [P, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
            "kara_compress_fused_supported": (i32, [P]),
            "kara_compress_fused": (i32, [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
            "kara_compress_fused_noalloc": (i32, [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
            "kara_status_str": (ctypes.c_char_p, [i32]),
            "kara_last_hip_error": (i32, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def make_config(shape, *, max_blocks_per_seq: int, num_blocks: int) -> kara_config:
    """kara_config from any object with the KaraShape field names."""
    return kara_config(shape.num_seqs, shape.num_layers, shape.num_q_heads, shape.num_kv_heads, shape.head_dim,
                       shape.window, shape.budget, shape.seeds, shape.radius, shape.block_size,
                       KARA_BF16 if shape.dtype == "bf16" else KARA_F32, max_blocks_per_seq, num_blocks)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _need(t, name, dtype, shape, device=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")


def _elem(cfg):
    return torch.bfloat16 if cfg.dtype == KARA_BF16 else torch.float32


def _check(status, where):
    if status != 0:
        raise KaraError(status, where)


def kara_check_config(cfg: kara_config) -> int:
    return lib().kara_check_config(ctypes.byref(cfg))


def kara_workspace_bytes(cfg: kara_config) -> int:
    return int(lib().kara_workspace_bytes(ctypes.byref(cfg)))


def kara_score_passes(cfg: kara_config) -> int:
    return int(lib().kara_score_passes(ctypes.byref(cfg)))


def kara_max_freed(cfg: kara_config) -> int:
    return int(lib().kara_max_freed(ctypes.byref(cfg)))


def kara_status_str(status: int) -> str:
    return lib().kara_status_str(int(status)).decode()


def kara_last_hip_error() -> int:
    return int(lib().kara_last_hip_error())


def _pool_shape(cfg):
    return (cfg.num_layers, cfg.num_blocks, cfg.num_kv_heads, cfg.block_size, cfg.head_dim)


def kara_score_window(cfg, q, k_cache, block_tables, prior_lens, scores, workspace, stream=None):
    S, Lyr, W, Hq, Hkv, d = cfg.num_seqs, cfg.num_layers, cfg.window, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    _need(q, "q", _elem(cfg), (S, Lyr, W, Hq, d))
    _need(k_cache, "k_cache", _elem(cfg), _pool_shape(cfg))
    _need(block_tables, "block_tables", torch.int32, (S, cfg.max_blocks_per_seq))
    _need(prior_lens, "prior_lens", torch.int32, (S,))
    _need(scores, "scores", torch.float32, (S, Lyr, Hkv, W))
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().kara_score_window(ctypes.byref(cfg), _ptr(q), _ptr(k_cache), _ptr(block_tables), _ptr(prior_lens),
                                   _ptr(scores), _ptr(workspace), nbytes, _stream(stream)), "kara_score_window")


def kara_select_chunks(cfg, scores, kept, mask=None, stream=None):
    S, Lyr, Hkv, W, B = cfg.num_seqs, cfg.num_layers, cfg.num_kv_heads, cfg.window, cfg.budget
    _need(scores, "scores", torch.float32, (S, Lyr, Hkv, W))
    _need(kept, "kept", torch.int32, (S, Lyr, Hkv, B))
    if mask is not None:
        _need(mask, "mask", torch.uint8, (S, Lyr, Hkv, W))
    _check(lib().kara_select_chunks(ctypes.byref(cfg), _ptr(scores), _ptr(kept), _ptr(mask), _stream(stream)),
           "kara_select_chunks")


def kara_chunk_bound(cfg: kara_config, gap: int) -> int:
    return int(lib().kara_chunk_bound(ctypes.byref(cfg), int(gap)))


def kara_select_chunks_bridged(cfg, gap, scores, kept, mask=None, stream=None):
    S, Lyr, Hkv, W, B = cfg.num_seqs, cfg.num_layers, cfg.num_kv_heads, cfg.window, cfg.budget
    _need(scores, "scores", torch.float32, (S, Lyr, Hkv, W))
    _need(kept, "kept", torch.int32, (S, Lyr, Hkv, B))
    if mask is not None:
        _need(mask, "mask", torch.uint8, (S, Lyr, Hkv, W))
    _check(lib().kara_select_chunks_bridged(ctypes.byref(cfg), int(gap), _ptr(scores), _ptr(kept), _ptr(mask),
                                            _stream(stream)), "kara_select_chunks_bridged")


def kara_compact_paged(cfg, k_cache, v_cache, block_tables, prior_lens, seq_lens, kept, freed_blocks, num_freed,
                       stream=None):
    S = cfg.num_seqs
    _need(k_cache, "k_cache", _elem(cfg), _pool_shape(cfg))
    _need(v_cache, "v_cache", _elem(cfg), _pool_shape(cfg))
    _need(block_tables, "block_tables", torch.int32, (S, cfg.max_blocks_per_seq))
    _need(prior_lens, "prior_lens", torch.int32, (S,))
    _need(seq_lens, "seq_lens", torch.int32, (S,))
    _need(kept, "kept", torch.int32, (S, cfg.num_layers, cfg.num_kv_heads, cfg.budget))
    _need(freed_blocks, "freed_blocks", torch.int32, (S, kara_max_freed(cfg)))
    _need(num_freed, "num_freed", torch.int32, (S,))
    _check(lib().kara_compact_paged(ctypes.byref(cfg), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                    _ptr(prior_lens), _ptr(seq_lens), _ptr(kept), _ptr(freed_blocks),
                                    _ptr(num_freed), _stream(stream)), "kara_compact_paged")


def kara_compact_paged_tail(cfg, k_cache, v_cache, block_tables, prior_lens, tail_lens, seq_lens, kept,
                            freed_blocks, num_freed, stream=None):
    S = cfg.num_seqs
    _need(k_cache, "k_cache", _elem(cfg), _pool_shape(cfg))
    _need(v_cache, "v_cache", _elem(cfg), _pool_shape(cfg))
    _need(block_tables, "block_tables", torch.int32, (S, cfg.max_blocks_per_seq))
    _need(prior_lens, "prior_lens", torch.int32, (S,))
    _need(tail_lens, "tail_lens", torch.int32, (S,))
    _need(seq_lens, "seq_lens", torch.int32, (S,))
    _need(kept, "kept", torch.int32, (S, cfg.num_layers, cfg.num_kv_heads, cfg.budget))
    _need(freed_blocks, "freed_blocks", torch.int32, (S, kara_max_freed(cfg)))
    _need(num_freed, "num_freed", torch.int32, (S,))
    _check(lib().kara_compact_paged_tail(ctypes.byref(cfg), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                         _ptr(prior_lens), _ptr(tail_lens), _ptr(seq_lens), _ptr(kept),
                                         _ptr(freed_blocks), _ptr(num_freed), _stream(stream)),
           "kara_compact_paged_tail")


def kara_decode_attention_workspace_bytes(cfg: kara_config) -> int:
    return int(lib().kara_decode_attention_workspace_bytes(ctypes.byref(cfg)))


def kara_decode_attention_splits(cfg: kara_config) -> int:
    return int(lib().kara_decode_attention_splits(ctypes.byref(cfg)))


def kara_decode_attention(cfg, q_dec, k_cache, v_cache, block_tables, seq_lens, out, workspace=None, stream=None):
    S, Lyr, Hq, d = cfg.num_seqs, cfg.num_layers, cfg.num_q_heads, cfg.head_dim
    _need(q_dec, "q_dec", _elem(cfg), (S, Lyr, Hq, d))
    _need(k_cache, "k_cache", _elem(cfg), _pool_shape(cfg))
    _need(v_cache, "v_cache", _elem(cfg), _pool_shape(cfg))
    _need(block_tables, "block_tables", torch.int32, (S, cfg.max_blocks_per_seq))
    _need(seq_lens, "seq_lens", torch.int32, (S,))
    _need(out, "out", torch.float32, (S, Lyr, Hq, d))
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().kara_decode_attention(ctypes.byref(cfg), _ptr(q_dec), _ptr(k_cache), _ptr(v_cache),
                                       _ptr(block_tables), _ptr(seq_lens), _ptr(out), _ptr(workspace), nbytes,
                                       _stream(stream)), "kara_decode_attention")


def kara_compress_fused_supported(cfg: kara_config) -> int:
    return int(lib().kara_compress_fused_supported(ctypes.byref(cfg)))


def kara_compress_fused(cfg, q, k_cache, v_cache, block_tables, prior_lens, scores, kept, seq_lens, freed_blocks,
                        num_freed, done, mask=None, stream=None):
    S, Lyr, W, Hq, Hkv, d, B = (cfg.num_seqs, cfg.num_layers, cfg.window, cfg.num_q_heads, cfg.num_kv_heads,
                                cfg.head_dim, cfg.budget)
    _need(q, "q", _elem(cfg), (S, Lyr, W, Hq, d))
    _need(k_cache, "k_cache", _elem(cfg), _pool_shape(cfg))
    _need(v_cache, "v_cache", _elem(cfg), _pool_shape(cfg))
    _need(block_tables, "block_tables", torch.int32, (S, cfg.max_blocks_per_seq))
    _need(prior_lens, "prior_lens", torch.int32, (S,))
    _need(scores, "scores", torch.float32, (S, Lyr, Hkv, W))
    _need(kept, "kept", torch.int32, (S, Lyr, Hkv, B))
    if mask is not None:
        _need(mask, "mask", torch.uint8, (S, Lyr, Hkv, W))
    _need(seq_lens, "seq_lens", torch.int32, (S,))
    _need(freed_blocks, "freed_blocks", torch.int32, (S, kara_max_freed(cfg)))
    _need(num_freed, "num_freed", torch.int32, (S,))
    _need(done, "done", torch.int32, (S,))
    _check(lib().kara_compress_fused(ctypes.byref(cfg), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                     _ptr(prior_lens), _ptr(scores), _ptr(kept), _ptr(mask), _ptr(seq_lens),
                                     _ptr(freed_blocks), _ptr(num_freed), _ptr(done), _stream(stream)),
           "kara_compress_fused")


def kara_compress_fused_noalloc(cfg, q, k_cache, v_cache, block_tables, prior_lens, scores, kept, seq_lens,
                                freed_blocks, num_freed, mask=None, stream=None):
    S, Lyr, W, Hq, Hkv, d, B = (cfg.num_seqs, cfg.num_layers, cfg.window, cfg.num_q_heads, cfg.num_kv_heads,
                                cfg.head_dim, cfg.budget)
    _need(q, "q", _elem(cfg), (S, Lyr, W, Hq, d))
    _need(k_cache, "k_cache", _elem(cfg), _pool_shape(cfg))
    _need(v_cache, "v_cache", _elem(cfg), _pool_shape(cfg))
    _need(block_tables, "block_tables", torch.int32, (S, cfg.max_blocks_per_seq))
    _need(prior_lens, "prior_lens", torch.int32, (S,))
    _need(scores, "scores", torch.float32, (S, Lyr, Hkv, W))
    _need(kept, "kept", torch.int32, (S, Lyr, Hkv, B))
    if mask is not None:
        _need(mask, "mask", torch.uint8, (S, Lyr, Hkv, W))
    _need(seq_lens, "seq_lens", torch.int32, (S,))
    _need(freed_blocks, "freed_blocks", torch.int32, (S, kara_max_freed(cfg)))
    _need(num_freed, "num_freed", torch.int32, (S,))
    _check(lib().kara_compress_fused_noalloc(ctypes.byref(cfg), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                             _ptr(block_tables), _ptr(prior_lens), _ptr(scores), _ptr(kept),
                                             _ptr(mask), _ptr(seq_lens), _ptr(freed_blocks), _ptr(num_freed),
                                             _stream(stream)), "kara_compress_fused_noalloc")


def kara_validate_tables(cfg, block_tables, prior_lens, bad_seqs, stream=None):
    _need(block_tables, "block_tables", torch.int32, (cfg.num_seqs, cfg.max_blocks_per_seq))
    _need(prior_lens, "prior_lens", torch.int32, (cfg.num_seqs,))
    _need(bad_seqs, "bad_seqs", torch.int32, (1,))
    _check(lib().kara_validate_tables(ctypes.byref(cfg), _ptr(block_tables), _ptr(prior_lens), _ptr(bad_seqs),
                                      _stream(stream)), "kara_validate_tables")
