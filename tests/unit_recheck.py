"""Offline re-check of one unit's record written by
decode_kv_cache_amd.unit_dump.save_unit, against the fp64 oracle: the scores
(reading R21), the exact selection from the recorded scores (R22), the
compacted rows and the untouched bytes below the window (R8, R23), and the
table rewrite (R16, R17).  Returns the list of what failed (empty: the record
is consistent)."""
import numpy as np

import oracle
from decode_kv_cache_amd.unit_dump import load_unit
from tests.kara_harness import SCORE_RTOL, score_errors

KARA_BF16 = 0


def _values(bits: np.ndarray, dtype: int) -> np.ndarray:
    """float64 values of raw bf16 (int16) or fp32 (int32) bit patterns."""
    if dtype == KARA_BF16:
        return (bits.astype(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return bits.astype(np.int32).view(np.float32).astype(np.float64)


def recheck(path: str) -> list:
    meta, ins, outs = load_unit(path)
    fails = []
    W, B, bs = meta["window"], meta["budget"], meta["block_size"]
    L = int(ins["prior_len"])
    qg = np.transpose(_values(ins["q"], meta["dtype"]), (1, 0, 2))            # [G][W][d]
    kw = _values(ins["k_window"], meta["dtype"])
    c_orc = oracle.window_scores(qg, kw)
    c_gpu = outs["scores"].astype(np.float64)
    if c_gpu.shape != (W,) or score_errors(outs["scores"], c_orc).max() > SCORE_RTOL:
        fails.append("scores")
    sel = oracle.token2chunk_select(c_gpu, B, meta["seeds"], meta["radius"])
    kept = outs["kept"]
    if kept.tolist() != sel.kept.tolist():
        fails.append("kept")
    idx = np.clip(kept, 0, W - 1)
    for pool in ("k", "v"):
        if not np.array_equal(outs[f"{pool}_kept"], ins[f"{pool}_window"][idx]):
            fails.append(f"{pool}_kept")
        if not np.array_equal(outs[f"{pool}_head_after"], ins[f"{pool}_head"]):
            fails.append(f"{pool}_head")
    row, fr, new_len = oracle.rewrite_block_table(ins["table_before"], L, W, B, bs)
    if not np.array_equal(outs["table_after"], row):
        fails.append("table")
    if outs["freed"].tolist() != list(fr):
        fails.append("freed")
    if int(outs["seq_len"]) != new_len:
        fails.append("seq_len")
    return fails
