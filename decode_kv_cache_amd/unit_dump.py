"""One unit's inputs and outputs of a compression step, saved to an .npz file
so the step can be re-checked offline (on another machine, without a GPU).

A unit is (sequence n, layer, KV head g).  Compaction works in place, so the
inputs are taken before the step and the outputs after it:

    before = unit_inputs(cfg, q, k_cache, v_cache, block_tables, prior_lens, n, layer, g)
    ... kara_score_window / kara_select_chunks / kara_compact_paged ...
    after = unit_outputs(cfg, k_cache, v_cache, block_tables, seq_lens, scores, kept, freed, num_freed,
                         n, layer, g, before["prior_len"])
    save_unit(path, cfg, before, after, (n, layer, g))

Tensors may live on any device; they are copied to the host.  Element data is
stored as raw bit patterns (int16 for bf16, int32 for fp32), so a re-check
sees exactly the bytes the kernels read and wrote.  Logical slot p of the
sequence is physical block block_tables[n][p // bs], row p % bs (the pool
layout [layers][blocks][kv_heads][block_size][head_dim]).
"""
from __future__ import annotations

import json

import numpy as np
import torch

FIELDS = ("num_seqs", "num_layers", "num_q_heads", "num_kv_heads", "head_dim", "window", "budget", "seeds",
          "radius", "block_size", "dtype", "max_blocks_per_seq", "num_blocks")


def _bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.detach().view(torch.int16).cpu().numpy()
    if t.dtype == torch.float32:
        return t.detach().view(torch.int32).cpu().numpy()
    return t.detach().cpu().numpy()


def _rows(pool: torch.Tensor, table_row: np.ndarray, layer: int, g: int, start: int, count: int, bs: int):
    """Bit patterns of logical slots [start, start+count) of one (layer, head)."""
    if count <= 0:
        return _bits(pool[layer, :0, g, 0, :])
    pos = np.arange(start, start + count)
    blk = torch.from_numpy(table_row[pos // bs].astype(np.int64)).to(pool.device)
    off = torch.from_numpy((pos % bs).astype(np.int64)).to(pool.device)
    return _bits(pool[layer][blk, g, off, :])


def unit_inputs(cfg, q, k_cache, v_cache, block_tables, prior_lens, n: int, layer: int, g: int) -> dict:
    """The unit's queries, its window's K and V rows, the bytes of the
    window's first block below L, and the sequence's table row and L."""
    G, bs, W = cfg.num_q_heads // cfg.num_kv_heads, cfg.block_size, cfg.window
    table = block_tables[n].detach().cpu().numpy().astype(np.int32)
    L = int(prior_lens[n].item())
    head = L % bs
    return {
        "q": _bits(q[n, layer, :, g * G:(g + 1) * G, :]),                     # [W][G][d]
        "k_window": _rows(k_cache, table, layer, g, L, W, bs),                # [W][d]
        "v_window": _rows(v_cache, table, layer, g, L, W, bs),
        "k_head": _rows(k_cache, table, layer, g, L - head, head, bs),        # slots [L - L % bs, L)
        "v_head": _rows(v_cache, table, layer, g, L - head, head, bs),
        "table_before": table,
        "prior_len": np.int64(L),
    }


def unit_outputs(cfg, k_cache, v_cache, block_tables, seq_lens, scores, kept, freed, num_freed,
                 n: int, layer: int, g: int, prior_len: int) -> dict:
    """The unit's scores and kept list, its compacted K and V rows (logical
    slots [L, L+B) read through the rewritten table, L = prior_len), the head
    bytes below L, and the sequence's rewritten table row, new length and
    freed blocks."""
    bs, B = cfg.block_size, cfg.budget
    table = block_tables[n].detach().cpu().numpy().astype(np.int32)
    new_len = int(seq_lens[n].item())
    L = int(prior_len)
    head = L % bs
    nf = int(num_freed[n].item())
    return {
        "scores": scores[n, layer, g].detach().cpu().numpy().astype(np.float32),
        "kept": kept[n, layer, g].detach().cpu().numpy().astype(np.int32),
        "k_kept": _rows(k_cache, table, layer, g, L, B, bs),
        "v_kept": _rows(v_cache, table, layer, g, L, B, bs),
        "k_head_after": _rows(k_cache, table, layer, g, L - head, head, bs),
        "v_head_after": _rows(v_cache, table, layer, g, L - head, head, bs),
        "table_after": table,
        "seq_len": np.int64(new_len),
        "freed": freed[n, :nf].detach().cpu().numpy().astype(np.int32),
    }


def save_unit(path: str, cfg, before: dict, after: dict, unit: tuple) -> None:
    """Write one unit's record: the configuration (JSON), the unit's index and
    the two dictionaries, in one compressed .npz file."""
    meta = {f: int(getattr(cfg, f)) for f in FIELDS}
    meta["unit"] = [int(x) for x in unit]
    arrays = {"meta": np.frombuffer(json.dumps(meta).encode(), dtype=np.uint8)}
    arrays.update({f"in_{k}": np.asarray(v) for k, v in before.items()})
    arrays.update({f"out_{k}": np.asarray(v) for k, v in after.items()})
    np.savez_compressed(path, **arrays)


def load_unit(path: str):
    """(meta, inputs, outputs) of a record written by save_unit; loads no
    Python objects from the file."""
    with np.load(path, allow_pickle=False) as z:
        meta = json.loads(bytes(z["meta"]).decode())
        ins = {k[3:]: z[k] for k in z.files if k.startswith("in_")}
        outs = {k[4:]: z[k] for k in z.files if k.startswith("out_")}
    return meta, ins, outs
