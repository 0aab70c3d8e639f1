// Token2Chunk selection for one unit inside one workgroup of NT threads
// (NT a multiple of 64, at least 256).  Used by the standalone selection
// kernel and by the single-launch pipeline.
//
// Kara's English abstract: a subset of the selected KV pairs is expanded into
// chunks.  Recorded rule: seeds are the first `seeds` positions of the order
// (score desc, position asc); each seed p keeps [p-r, p+r] clipped to the
// window (spans merge); with gap > 0 (the bridging variant of the lay
// explainers) neighbouring seeds that leave at most `gap` positions between
// them also keep what lies between; the rest of the budget goes to the best
// positions outside the chunks under the same order; exactly B positions are
// kept and written ascending.
//
// Scores become order-preserving 32-bit keys in LDS; each top-k threshold is
// found by an MSB-first 8-bit radix select (LDS histogram + block scan), and
// ties at the threshold are taken by ascending position with a block prefix
// count.  Thread t owns the contiguous positions [t*E, t*E+E), so thread order
// is position order.
#pragma once

#include "kara_device.h"

namespace kara {

constexpr uint8_t IN_SPAN = 1, KEEP = 2, SEED = 4;

// float -> uint32 whose unsigned order is the float order (-0 == +0).
__device__ inline uint32_t order_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

template <int NT>
struct SelScratch {
  int hist[256];
  int wave_tot[NT / 64];
  int bcast[3];
};

// Exclusive prefix sum of v over the block in thread order; *total gets the sum.
template <int NT>
__device__ inline int block_scan(int v, int* total, SelScratch<NT>& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh.wave_tot[wave] = x;
  __syncthreads();
  int pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    int t = sh.wave_tot[w];
    pre += (w < wave) ? t : 0;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return pre + x - v;
}

// Find the k-th largest key (1-based) among positions whose flag has
// (flag & emask) == 0.  Returns a threshold T and *need such that the top k
// are exactly the eligible keys > T plus the first *need eligible keys equal
// to T (lowest positions first).  When a digit's bucket holds exactly the k
// keys still wanted, every key with that prefix is taken and the search stops
// early: T is then the largest key below the prefix and *need = 0.
template <int NT>
__device__ uint32_t radix_select(const uint32_t* keys, const uint8_t* flags, uint8_t emask, int W, int E, int k,
                                 int* need, SelScratch<NT>& sh) {
  static_assert(NT >= 256, "one thread per digit");
  const int t = threadIdx.x;
  const int j0 = t * E, j1 = min(W, j0 + E);
  uint32_t prefix = 0, pmask = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (t < 256) sh.hist[t] = 0;
    __syncthreads();
    for (int j = j0; j < j1; ++j) {
      if (flags[j] & emask) continue;
      uint32_t key = keys[j];
      if ((key & pmask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 255], 1);
    }
    __syncthreads();
    const int c = t < 256 ? sh.hist[255 - t] : 0;   // thread t looks at digit 255 - t (descending)
    int total;
    const int before = block_scan<NT>(c, &total, sh);
    if (before < k && k <= before + c) {
      sh.bcast[0] = 255 - t;
      sh.bcast[1] = k - before;
      sh.bcast[2] = c;
    }
    __syncthreads();
    prefix |= (uint32_t)sh.bcast[0] << shift;
    pmask |= 0xFFu << shift;
    k = sh.bcast[1];
    const bool whole = k == sh.bcast[2] && prefix != 0u;   // the same in every thread
    __syncthreads();
    if (whole && shift > 0) {
      *need = 0;
      return prefix - 1u;                         // every key >= prefix, nothing below it
    }
  }
  *need = k;
  return prefix;
}

// Mark with `bit` the top-k eligible positions given threshold T / need.
template <int NT>
__device__ inline void mark_top(const uint32_t* keys, uint8_t* flags, uint8_t emask, uint8_t bit, int W, int E,
                                uint32_t T, int need, SelScratch<NT>& sh, int* marked, int* nmarked) {
  const int t = threadIdx.x;
  const int j0 = t * E, j1 = min(W, j0 + E);
  int eq = 0;
  for (int j = j0; j < j1; ++j)
    if (!(flags[j] & emask) && keys[j] == T) ++eq;
  int tot;
  int rank = block_scan<NT>(eq, &tot, sh);
  int cnt = 0;
  for (int j = j0; j < j1; ++j) {
    if (flags[j] & emask) continue;
    const uint32_t key = keys[j];
    bool take = key > T;
    if (key == T) take = (rank++ < need);
    if (take) {
      if (marked) marked[cnt] = j;
      ++cnt;
      flags[j] |= bit;
    }
  }
  *nmarked = cnt;
}

// Selection of one unit.  On entry keys[0..W) hold the order keys of the
// unit's scores (LDS) and every thread has passed a barrier since they were
// written.  Writes the B kept positions ascending to kept_lds (LDS, may be
// NULL) and kept_out (global, may be NULL), and the 0/1 mask to mask_out
// (global, may be NULL).  Requires ceil(W / NT) <= MAXE.
template <int NT, int MAXE>
__device__ void select_unit(const Geo& g, int gap, const uint32_t* keys, uint8_t* flags, SelScratch<NT>& sh,
                            int32_t* kept_lds, int32_t* __restrict__ kept_out, uint8_t* __restrict__ mask_out) {
  const int W = g.W, B = g.B;
  const int E = (W + NT - 1) / NT;
  const int t = threadIdx.x;
  for (int j = t; j < W; j += NT) flags[j] = 0;
  __syncthreads();

  // seeds and their spans
  if (g.seeds > 0) {
    int need;
    const uint32_t T = radix_select<NT>(keys, flags, 0, W, E, g.seeds, &need, sh);
    int seeds_mine[MAXE];   // a thread owns at most E <= MAXE positions
    int ns;
    mark_top<NT>(keys, flags, 0, KEEP, W, E, T, need, sh, seeds_mine, &ns);
    __syncthreads();
    for (int a = 0; a < ns; ++a) {
      const int p = seeds_mine[a];
      const int lo = max(0, p - g.radius), hi = min(W - 1, p + g.radius);
      for (int x = lo; x <= hi; ++x) flags[x] = IN_SPAN;   // concurrent writers store the same value
    }
    __syncthreads();
    if (gap > 0 && g.seeds > 1) {
      for (int a = 0; a < ns; ++a) flags[seeds_mine[a]] = IN_SPAN | SEED;
      __syncthreads();
      // The owner of seed p looks for the next seed p' within gap + 1 positions;
      // the positions strictly between belong to this pair alone, so each is
      // written by exactly one thread.
      for (int a = 0; a < ns; ++a) {
        const int p = seeds_mine[a];
        const int lim = min(W - 1, p + gap + 1);
        int nxt = -1;
        for (int x = p + 1; x <= lim; ++x)
          if (flags[x] & SEED) {
            nxt = x;
            break;
          }
        for (int x = p + 1; x < nxt; ++x) flags[x] |= IN_SPAN;
      }
      __syncthreads();
    }
  }
  // |U|
  const int j0 = t * E, j1 = min(W, j0 + E);
  int u = 0;
  for (int j = j0; j < j1; ++j) u += (flags[j] & IN_SPAN) ? 1 : 0;
  int usize;
  block_scan<NT>(u, &usize, sh);
  const int room = B - usize;
  if (room > 0) {
    int need;
    const uint32_t T = radix_select<NT>(keys, flags, IN_SPAN, W, E, room, &need, sh);
    int nf;
    mark_top<NT>(keys, flags, IN_SPAN, KEEP, W, E, T, need, sh, nullptr, &nf);
  }
  // kept = U or fill, ascending
  int mine = 0;
  for (int j = j0; j < j1; ++j) mine += (flags[j] & (IN_SPAN | KEEP)) ? 1 : 0;
  int total;
  int pos = block_scan<NT>(mine, &total, sh);
  for (int j = j0; j < j1; ++j) {
    const bool k = (flags[j] & (IN_SPAN | KEEP)) != 0;
    if (k && pos < B) {
      if (kept_lds) kept_lds[pos] = j;
      if (kept_out) kept_out[pos] = j;
    }
    pos += k ? 1 : 0;
    if (mask_out) mask_out[j] = k ? 1 : 0;
  }
}

}  // namespace kara
