"""Shared helpers for the parity tests: run the step through the C ABI and
compare it with the fp64 oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from decode_kv_cache_amd import kara as K
from decode_kv_cache_amd.workloads import Workload

SCORE_RTOL = 2e-3          # relative score tolerance
SCORE_FLOOR = 1e-30        # absolute floor (fp32 flush of tiny probabilities)
GUARD = 64                 # guard elements after every output buffer


def config_of(wl: Workload):
    return K.make_config(wl.shape, max_blocks_per_seq=wl.max_blocks, num_blocks=wl.num_blocks)


class Outputs:
    """Output buffers with guard bands; `view`s are what the library sees."""

    def __init__(self, cfg, device):
        S, Lyr, Hkv, W, B = cfg.num_seqs, cfg.num_layers, cfg.num_kv_heads, cfg.window, cfg.budget
        mf = K.kara_max_freed(cfg)
        self.shapes = dict(scores=(S, Lyr, Hkv, W), kept=(S, Lyr, Hkv, B), mask=(S, Lyr, Hkv, W),
                           seq_lens=(S,), freed=(S, mf), num_freed=(S,))
        dt = dict(scores=torch.float32, kept=torch.int32, mask=torch.uint8, seq_lens=torch.int32,
                  freed=torch.int32, num_freed=torch.int32)
        fill = dict(scores=float("nan"), kept=-7, mask=0xA5, seq_lens=-7, freed=-7, num_freed=-7)
        self.raw, self.fill = {}, fill
        for k, shp in self.shapes.items():
            n = int(np.prod(shp))
            self.raw[k] = torch.full((n + GUARD,), fill[k], dtype=dt[k], device=device)
        wsb = K.kara_workspace_bytes(cfg)
        self.ws = torch.empty((max(wsb, 1) + 255) // 256 * 256 // 4, dtype=torch.float32, device=device)

    def __getitem__(self, k):
        n = int(np.prod(self.shapes[k]))
        return self.raw[k][:n].view(self.shapes[k])

    def guards_intact(self):
        for k, buf in self.raw.items():
            n = int(np.prod(self.shapes[k]))
            tail = buf[n:].cpu()
            if k == "scores":
                if not torch.isnan(tail).all():
                    return False
            elif not (tail == self.fill[k]).all():
                return False
        return True


def run_step(wl: Workload, cfg=None, out: Outputs | None = None, with_mask=True, stream=None, gap=None):
    """Score, select and compact through the C ABI; gap selects the bridging
    variant of the selection (None: the main rule)."""
    cfg = cfg or config_of(wl)
    out = out or Outputs(cfg, wl.q.device)
    K.kara_score_window(cfg, wl.q, wl.k_pool, wl.block_tables, wl.prior_lens, out["scores"], out.ws, stream)
    mask = out["mask"] if with_mask else None
    if gap is None:
        K.kara_select_chunks(cfg, out["scores"], out["kept"], mask, stream)
    else:
        K.kara_select_chunks_bridged(cfg, gap, out["scores"], out["kept"], mask, stream)
    K.kara_compact_paged(cfg, wl.k_pool, wl.v_pool, wl.block_tables, wl.prior_lens, out["seq_lens"], out["kept"],
                         out["freed"], out["num_freed"], stream)
    torch.cuda.synchronize()
    return cfg, out


def bits(t: torch.Tensor) -> np.ndarray:
    """Bit patterns of a device tensor as a host integer array."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy()
    if t.dtype == torch.float32:
        return t.view(torch.int32).cpu().numpy()
    return t.cpu().numpy()


def unit_inputs(q_host: np.ndarray, k_pool_f64: np.ndarray, wl: Workload, n: int, layer: int, g: int):
    """fp64 (q_group [G, W, d], k_window [W, d]) of one unit from host copies."""
    s = wl.shape
    G = s.group
    qg = np.transpose(q_host[n, layer, :, g * G:(g + 1) * G, :], (1, 0, 2))
    kw = oracle.gather_window_rows(k_pool_f64, wl.host_tables[n], layer, g, int(wl.host_prior_lens[n]), s.window,
                                   s.block_size)
    return qg, kw


def oracle_unit_attention(q_heads: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray) -> np.ndarray:
    """The oracle's paged decode attention for one KV head's query heads over
    the unit's cached rows [0, T), given in logical order: the rows form a
    one-sequence, one-layer pool of block size 1 with an identity table.
    q_heads [G][d], k_rows / v_rows [T][d]; returns [G][d] in fp64."""
    G, d = q_heads.shape
    T = k_rows.shape[0]
    pool_k = np.asarray(k_rows, dtype=np.float64).reshape(1, T, 1, 1, d)
    pool_v = np.asarray(v_rows, dtype=np.float64).reshape(1, T, 1, 1, d)
    table = np.arange(max(T, 1), dtype=np.int64).reshape(1, -1)
    o = oracle.paged_decode_attention(np.asarray(q_heads, dtype=np.float64).reshape(1, 1, G, d), pool_k, pool_v,
                                      table, np.array([T]), 1)
    return o[0, 0]


def score_errors(c_gpu: np.ndarray, c_orc: np.ndarray) -> np.ndarray:
    """|c_gpu - c_orc| / max(c_orc, floor), elementwise."""
    return np.abs(c_gpu.astype(np.float64) - c_orc) / np.maximum(c_orc, SCORE_FLOOR)


def near_cutoff_ok(c_orc, kept_gpu, budget, seeds, radius, rtol=SCORE_RTOL):
    """Positions where the GPU selection differs from oracle.select(c_orc)
    must be explained by a near-tie: they lie within rtol (relative) of the
    seed cutoff or of the fill cutoff, or within `radius` of a position that
    lies within rtol of the seed cutoff.  Returns (ok, n_diff)."""
    sel = oracle.token2chunk_select(c_orc, budget, seeds, radius)
    W = len(c_orc)
    a = np.zeros(W, bool)
    a[sel.kept] = True
    b = np.zeros(W, bool)
    b[kept_gpu] = True
    diff = np.flatnonzero(a != b)
    if diff.size == 0:
        return True, 0
    order = sorted(range(W), key=lambda j: (-c_orc[j], j))
    taus = []
    if seeds > 0:
        taus.append(c_orc[order[seeds - 1]])
    if sel.fill.size:
        taus.append(c_orc[sel.fill[-1]])
        outside = [j for j in order if not sel.span[j] and j not in set(sel.fill.tolist())]
        if outside:
            taus.append(c_orc[outside[0]])

    def close(x, t):
        return abs(x - t) <= rtol * max(abs(t), SCORE_FLOOR)

    seed_near = [j for j in range(W) if seeds > 0 and close(c_orc[j], taus[0])]
    for j in diff:
        if any(close(c_orc[j], t) for t in taus):
            continue
        if any(abs(j - p) <= radius for p in seed_near):
            continue
        return False, diff.size
    return True, diff.size
