"""Seeded synthetic workloads for the Kara window-compression step.

This module is the one place that makes inputs.  It holds the workload
shapes and the recipe that fills a PagedAttention KV pool, the window
queries and the block tables with seeded random data.  It contains none of
the method's arithmetic (no scoring, selection or compaction), so both the
HIP path and the fp64 oracle can consume what it makes.

Recipe (the pages name no dataset; these tensors stand in for the
reasoning-model decode workloads the Kara pages describe):

* values are drawn in fp32 and rounded to the storage dtype (bf16 rounding
  is torch's round-to-nearest-even);
* Q, K, V entries are i.i.d. N(0, 1) unless the shape says otherwise;
* ``key_model="outliers"``: per (layer, kv head) four key channels, drawn
  without replacement and shared by every token and sequence, are scaled x8;
* ``key_model="spiky"``: N(0, 1) keys scaled x16, so logits span about
  +-100 in base-2 exponent units and every softmax row is sharply peaked (a
  numerical-range stress case, not a model of real keys);
* ``key_model="student_t3"``: key entries are Student-t with 3 degrees of
  freedom, unscaled (z / sqrt(chi2_3 / 3));
* ``plants=True``: per (sequence, layer, kv head) a unit direction u and six
  non-overlapping runs (gap >= 1) of 5..40 consecutive window keys at uniform
  positions; each run key becomes |k| (0.8 u + 0.6 w), w the unit part of k
  orthogonal to u, and every window query of the group becomes
  |q| (0.8 u + 0.6 v) the same way (cosine 0.8 with u before rounding);
* block tables map logical blocks to a seeded permutation of physical block
  ids; the pool holds exactly the blocks every sequence needs for L + W
  tokens.  The window slots and the prior-context slots that share the
  window's first block are random data; every other slot holds a canary
  value so that stray writes show up;
* for the decode-attention consumer, ``fill_prior_context`` overwrites the
  remaining prior slots [0, L - L % bs) with i.i.d. N(0, 1) keys and values,
  and ``decode_queries`` draws one N(0, 1) query per (sequence, layer, head).

Seeds are derived from (shape id, sequence, layer, tensor tag) with numpy's
SeedSequence; torch generators on the target device draw the bulk values,
so a workload is reproducible for a given device type.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch

__all__ = ["KaraShape", "SHAPES", "shape_by_name", "Workload", "make_workload", "fill_prior_context",
           "decode_queries", "CANARY_BF16_BITS", "CANARY_F32"]

# Canary for pool slots the step must never touch (a normal bf16 value that
# random data essentially never produces exactly: -0.013916015625).
CANARY_BF16_BITS = 0xBC64
CANARY_F32 = -0.0139160156


@dataclass(frozen=True)
class KaraShape:
    """One workload shape: model geometry, window/budget and data recipe."""
    name: str
    shape_id: int
    num_seqs: int
    num_layers: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    window: int
    budget: int
    seeds: int
    radius: int
    block_size: int = 16
    dtype: str = "bf16"                     # "bf16" or "f32" (Q, K and V share it)
    prior: tuple = ("fixed", 0)             # ("fixed", L) or ("uniform", lo, hi) inclusive
    key_model: str = "normal"               # "normal" | "outliers" | "student_t3" | "spiky"
    plants: bool = False
    description: str = ""

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def units(self) -> int:
        return self.num_seqs * self.num_layers * self.num_kv_heads

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def with_(self, **kw) -> "KaraShape":
        return replace(self, **kw)


SHAPES = [
    KaraShape("tiny", 1, num_seqs=1, num_layers=1, num_q_heads=4, num_kv_heads=2, head_dim=64,
              window=128, budget=32, seeds=2, radius=3, dtype="f32", prior=("fixed", 256),
              description="tiny reference: fp32, GQA 2, L=256, W=128 -> B=32, s=2, r=3"),
    KaraShape("llama8b_b1", 2, num_seqs=1, num_layers=32, num_q_heads=32, num_kv_heads=8,
              head_dim=128, window=1024, budget=204, seeds=8, radius=5, prior=("fixed", 8192),
              description="Llama-3-8B shape, batch 1, L=8192, W=1024 -> B=204, s=8, r=5"),
    KaraShape("llama8b_b64", 3, num_seqs=64, num_layers=32, num_q_heads=32, num_kv_heads=8,
              head_dim=128, window=1024, budget=204, seeds=8, radius=5,
              prior=("uniform", 4096, 32768), key_model="outliers",
              description="Llama-3-8B shape, 64 sequences, L ~ U[4096, 32768], W=1024 -> B=204, "
                          "keys with 4 outlier channels x8"),
    KaraShape("gqa7b", 4, num_seqs=32, num_layers=28, num_q_heads=28, num_kv_heads=4,
              head_dim=128, window=2048, budget=410, seeds=12, radius=7, prior=("fixed", 16384),
              plants=True,
              description="GQA-heavy 7B shape, 32 sequences, L=16384, W=2048 -> B=410, s=12, r=7, "
                          "6 planted correlated runs per window"),
    KaraShape("large", 5, num_seqs=8, num_layers=80, num_q_heads=64, num_kv_heads=8,
              head_dim=128, window=4096, budget=820, seeds=24, radius=8, prior=("fixed", 32768),
              key_model="student_t3", plants=True,
              description="80-layer one-GPU share, 8 sequences, L=32768, W=4096 -> B=820, s=24, "
                          "r=8, Student-t(3) keys plus planted runs"),
]


def shape_by_name(name: str) -> KaraShape:
    for s in SHAPES:
        if s.name == name:
            return s
    raise KeyError(name)


def _seed(*key) -> int:
    ss = np.random.SeedSequence([int(k) & 0xFFFFFFFF for k in key])
    return int(ss.generate_state(1, np.uint64)[0] & 0x7FFF_FFFF_FFFF_FFFF)


def _torch_gen(device, *key) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*key))
    return g


_TAG_Q, _TAG_K, _TAG_V, _TAG_U, _TAG_HEAD_K, _TAG_HEAD_V = 11, 12, 13, 14, 15, 16
_TAG_PRIOR_K, _TAG_PRIOR_V, _TAG_QDEC = 17, 18, 19


@dataclass
class Workload:
    """Device-resident inputs of one compression step."""
    shape: KaraShape
    q: torch.Tensor               # [S][layers][W][Hq][d]
    k_pool: torch.Tensor          # [layers][num_blocks][Hkv][bs][d]
    v_pool: torch.Tensor
    block_tables: torch.Tensor    # int32 [S][max_blocks]
    prior_lens: torch.Tensor      # int32 [S]
    num_blocks: int
    max_blocks: int
    host_prior_lens: np.ndarray
    host_tables: np.ndarray
    extra: dict = field(default_factory=dict)

    def window_slot_index(self, n: int):
        """(physical block, offset) arrays of sequence n's window slots."""
        L = int(self.host_prior_lens[n])
        bs = self.shape.block_size
        pos = np.arange(L, L + self.shape.window)
        return self.host_tables[n, pos // bs], pos % bs


def _prior_lens(shape: KaraShape) -> np.ndarray:
    kind = shape.prior[0]
    if kind == "fixed":
        return np.full(shape.num_seqs, int(shape.prior[1]), dtype=np.int64)
    if kind == "uniform":
        rng = np.random.default_rng(_seed(shape.shape_id, 0xB10C))
        return rng.integers(shape.prior[1], shape.prior[2] + 1, size=shape.num_seqs).astype(np.int64)
    raise ValueError(kind)


def _plant_runs(rng, W, n_runs=6, lo=5, hi=40):
    """Start/length of n_runs non-overlapping runs (gap >= 1), uniform placement."""
    lens = rng.integers(lo, hi + 1, size=n_runs)
    free = W - int(lens.sum()) - (n_runs - 1)
    if free < 0:
        return np.zeros(0, dtype=np.int64), np.zeros(0, dtype=np.int64)
    offs = np.sort(rng.integers(0, free + 1, size=n_runs))
    starts = np.empty(n_runs, dtype=np.int64)
    used = 0
    for k in range(n_runs):
        starts[k] = offs[k] + used
        used += int(lens[k]) + 1
    return starts, lens.astype(np.int64)


def _tilt(x, u, cos=0.8):
    """|x| (cos * u + sin * w), w = unit part of x orthogonal to u (last dim)."""
    sin = math.sqrt(1.0 - cos * cos)
    norm = x.norm(dim=-1, keepdim=True)
    proj = (x * u).sum(-1, keepdim=True)
    w = x - proj * u
    w = w / w.norm(dim=-1, keepdim=True).clamp_min(1e-30)
    return norm * (cos * u + sin * w)


def make_workload(shape: KaraShape, device="cpu", *, canary=True) -> Workload:
    """Allocate and fill a workload on ``device`` (see the module recipe)."""
    S, Lyr, Hq, Hkv, d = shape.num_seqs, shape.num_layers, shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    W, bs, G = shape.window, shape.block_size, shape.group
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    tdtype = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
    prior = _prior_lens(shape)
    nblk = [-(-(int(prior[n]) + W) // bs) for n in range(S)]
    num_blocks = int(sum(nblk))
    max_blocks = max(nblk) if nblk else -(-W // bs)
    perm = np.random.default_rng(_seed(shape.shape_id, 0xB10C, 1)).permutation(num_blocks)
    tables = np.full((max(S, 0), max_blocks), -1, dtype=np.int32)
    pos = 0
    for n in range(S):
        tables[n, :nblk[n]] = perm[pos:pos + nblk[n]]
        pos += nblk[n]

    pool_shape = (Lyr, num_blocks, Hkv, bs, d)
    k_pool = torch.empty(pool_shape, dtype=tdtype, device=device)
    v_pool = torch.empty(pool_shape, dtype=tdtype, device=device)
    if canary:
        if tdtype == torch.bfloat16:
            k_pool.view(torch.int16).fill_(CANARY_BF16_BITS - 0x10000)
            v_pool.view(torch.int16).fill_(CANARY_BF16_BITS - 0x10000)
        else:
            k_pool.fill_(CANARY_F32)
            v_pool.fill_(CANARY_F32)
    q = torch.empty((S, Lyr, W, Hq, d), dtype=tdtype, device=device)

    if shape.key_model == "outliers":
        ch = np.stack([np.random.default_rng(_seed(shape.shape_id, l, g, 7)).choice(d, 4, replace=False)
                       for l in range(Lyr) for g in range(Hkv)]).reshape(Lyr, Hkv, 4)
        out_scale = torch.ones((Lyr, Hkv, d), dtype=torch.float32)
        for l in range(Lyr):
            for g in range(Hkv):
                out_scale[l, g, ch[l, g]] = 8.0
        out_scale = out_scale.to(device)
    for n in range(S):
        L = int(prior[n])
        p = np.arange(L, L + W)
        blk = torch.from_numpy(tables[n, p // bs].astype(np.int64)).to(device)
        off = torch.from_numpy((p % bs).astype(np.int64)).to(device)
        head = L % bs
        if head:
            hp = np.arange(L - head, L)
            hb = torch.from_numpy(tables[n, hp // bs].astype(np.int64)).to(device)
            ho = torch.from_numpy((hp % bs).astype(np.int64)).to(device)
        for l in range(Lyr):
            qn = torch.randn((W, Hq, d), generator=_torch_gen(device, shape.shape_id, n, l, _TAG_Q),
                             device=device, dtype=torch.float32)
            gk = _torch_gen(device, shape.shape_id, n, l, _TAG_K)
            if shape.key_model == "student_t3":
                z = torch.randn((W, Hkv, d), generator=gk, device=device, dtype=torch.float32)
                chi = torch.randn((3, W, Hkv, d), generator=gk, device=device, dtype=torch.float32)
                kn = z / torch.sqrt((chi * chi).sum(0) / 3.0)
            else:
                kn = torch.randn((W, Hkv, d), generator=gk, device=device, dtype=torch.float32)
            if shape.key_model == "outliers":
                kn = kn * out_scale[l][None, :, :]
            if shape.key_model == "spiky":
                kn = kn * 16.0
            vn = torch.randn((W, Hkv, d), generator=_torch_gen(device, shape.shape_id, n, l, _TAG_V),
                             device=device, dtype=torch.float32)
            if shape.plants:
                u = torch.randn((Hkv, d), generator=_torch_gen(device, shape.shape_id, n, l, _TAG_U),
                                device=device, dtype=torch.float32)
                u = u / u.norm(dim=-1, keepdim=True)
                mask = np.zeros((W, Hkv), dtype=bool)
                for g in range(Hkv):
                    rng = np.random.default_rng(_seed(shape.shape_id, n, l, g, 0x9A))
                    st, ln = _plant_runs(rng, W)
                    for a, b in zip(st, ln):
                        mask[a:a + b, g] = True
                mask_t = torch.from_numpy(mask).to(device)
                kn = torch.where(mask_t[..., None], _tilt(kn, u[None].expand(W, Hkv, d)), kn)
                u_q = u.repeat_interleave(G, dim=0)[None].expand(W, Hq, d)
                qn = _tilt(qn, u_q)
            q[n, l] = qn.to(tdtype)
            # scatter the window rows into the paged pool
            k_pool[l][blk, :, off, :] = kn.to(tdtype)
            v_pool[l][blk, :, off, :] = vn.to(tdtype)
            # prior-context slots that share the window's first block
            if head:
                hk = torch.randn((head, Hkv, d), generator=_torch_gen(device, shape.shape_id, n, l, _TAG_HEAD_K),
                                 device=device, dtype=torch.float32)
                hv = torch.randn((head, Hkv, d), generator=_torch_gen(device, shape.shape_id, n, l, _TAG_HEAD_V),
                                 device=device, dtype=torch.float32)
                k_pool[l][hb, :, ho, :] = hk.to(tdtype)
                v_pool[l][hb, :, ho, :] = hv.to(tdtype)

    return Workload(shape=shape, q=q, k_pool=k_pool, v_pool=v_pool,
                    block_tables=torch.from_numpy(tables).to(device),
                    prior_lens=torch.from_numpy(prior.astype(np.int32)).to(device),
                    num_blocks=num_blocks, max_blocks=max_blocks,
                    host_prior_lens=prior, host_tables=tables)


def fill_prior_context(wl: Workload) -> None:
    """Fill the prior slots [0, L - L % bs) of every sequence with seeded
    N(0, 1) keys and values (the head block's prior slots already hold random
    data), so that attention over the whole cache sees no canary rows."""
    s = wl.shape
    bs, Hkv, d = s.block_size, s.num_kv_heads, s.head_dim
    dev = wl.k_pool.device
    for n in range(s.num_seqs):
        L = int(wl.host_prior_lens[n])
        full = L - L % bs
        if full == 0:
            continue
        p = np.arange(full)
        blk = torch.from_numpy(wl.host_tables[n, p // bs].astype(np.int64)).to(dev)
        off = torch.from_numpy((p % bs).astype(np.int64)).to(dev)
        for l in range(s.num_layers):
            pk = torch.randn((full, Hkv, d), generator=_torch_gen(dev, s.shape_id, n, l, _TAG_PRIOR_K),
                             device=dev, dtype=torch.float32)
            pv = torch.randn((full, Hkv, d), generator=_torch_gen(dev, s.shape_id, n, l, _TAG_PRIOR_V),
                             device=dev, dtype=torch.float32)
            wl.k_pool[l][blk, :, off, :] = pk.to(wl.k_pool.dtype)
            wl.v_pool[l][blk, :, off, :] = pv.to(wl.v_pool.dtype)


def decode_queries(shape: KaraShape, device="cpu") -> torch.Tensor:
    """One seeded N(0, 1) decode query per (sequence, layer, query head):
    [S][layers][Hq][d] in the shape's dtype."""
    tdtype = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
    g = _torch_gen(device, shape.shape_id, 0, 0, _TAG_QDEC)
    q = torch.randn((shape.num_seqs, shape.num_layers, shape.num_q_heads, shape.head_dim), generator=g,
                    device=device, dtype=torch.float32)
    return q.to(tdtype)
