// In-place compaction of one unit's kept window rows and the per-sequence
// block-table rewrite, as device functions shared by the compaction kernels
// and the single-launch pipeline.
//
// Kara's English abstract: the method is adapted to PagedAttention and lowers
// KV-cache memory.  Recorded reading: for unit (n, l, g) and r < B, logical
// slot L+r takes the old row of slot L+kept[r] (K and V); afterwards, per
// sequence, the table entries of logical blocks ceil((L+B)/bs) ..
// ceil((L+W)/bs)-1 are handed back in order and set to -1.
//
// When the window is the oldest part of the context not yet compressed, T
// newer tokens follow it in slots [L+W, L+W+T); they move in order right
// behind the kept rows: slot L+B+t takes the old row of slot L+W+t, and the
// table keeps the blocks of the first L+B+T slots (the gist.science
// explainer's periodic schedule cleans the back end of the current thought).
//
// In-place safety: the source list (kept, then W .. W+T-1) is strictly
// ascending, so source[r] >= r.  The rows of a unit are walked in ascending
// chunks: a chunk is read into registers, the reads are waited for, the
// workgroup synchronises, then the chunk is written.  A chunk's writes land on
// slots < L + (end of chunk) while every later source is at or past that
// point, and every source a later write could hit was read before the barrier
// of its own chunk.
#pragma once

#include "kara_device.h"

namespace kara {

// rows are streamed once: non-temporal loads and stores keep them out of the caches
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Copy the B kept rows of one unit into place, in the K pool and the V pool
// together: both use the same source and destination slots, so each row's
// two table lookups serve both copies and the loads of both pools are in
// flight at once.  kl = the unit's kept list (global or LDS), followed by T
// tail rows; NT threads, VEC 16-byte vectors per thread and pool per chunk.
template <int NT, int ROWBYTES, int VEC>
__device__ __forceinline__ void compact_unit_rows(const Geo& g, unsigned char* __restrict__ kpool,
                                                  unsigned char* __restrict__ vpool,
                                                  const int32_t* __restrict__ trow, int layer, int kvh, int L,
                                                  const int32_t* kl, int esize, int T = 0) {
  constexpr int TPR = ROWBYTES / 16;                  // threads per row
  constexpr int RPP = NT / TPR;                       // rows per pass
  constexpr int CH = RPP * VEC;                       // rows per chunk
  const int t = threadIdx.x;
  const int part = t % TPR;
  const int rsub = t / TPR;
  const int rows = g.B + T;
  for (int c0 = 0; c0 < rows; c0 += CH) {
    u32x4 bk[VEC], bv[VEC];
    long long dst[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      const int r = c0 + v * RPP + rsub;
      dst[v] = -1;
      if (r < rows) {
        const int j = r < g.B ? kl[r] : g.W + (r - g.B);
        const long long so = (j >= 0 && j < g.W + T) ? slot_offset(g, trow, layer, kvh, L + j) : -1;
        const long long d = slot_offset(g, trow, layer, kvh, L + r);
        if (so >= 0 && d >= 0) {
          const long long o = so * esize + part * 16;
          bk[v] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kpool + o));
          bv[v] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vpool + o));
          dst[v] = d * esize + part * 16;
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);   // every read of this chunk has returned
    __syncthreads();
#pragma unroll
    for (int v = 0; v < VEC; ++v)
      if (dst[v] >= 0) {
        __builtin_nontemporal_store(bk[v], reinterpret_cast<u32x4*>(kpool + dst[v]));
        __builtin_nontemporal_store(bv[v], reinterpret_cast<u32x4*>(vpool + dst[v]));
      }
  }
}

// Tail length of sequence n: tails[n] clamped to [0, slots the table can
// address after the window]; 0 without a tail array.
__device__ inline int tail_of(const Geo& g, const int32_t* __restrict__ tails, int n, int L) {
  if (!tails) return 0;
  const long long room = (long long)g.max_blocks * g.bs - (long long)L - g.W;
  return (int)max(0LL, min((long long)tails[n], room));
}

// Freed list, table truncation and new length of sequence n, by `nthreads`
// threads of one workgroup (thread `tid`); freed entry k is table entry
// nb_new + k, so the list stays in ascending logical order whatever the
// thread count.
__device__ inline void finalize_sequence(const Geo& g, int n, int32_t* __restrict__ tables,
                                         const int32_t* __restrict__ prior, int32_t* __restrict__ seq_lens,
                                         int32_t* __restrict__ freed, int32_t* __restrict__ num_freed,
                                         int max_freed, const int32_t* __restrict__ tails, int tid, int nthreads) {
  const int L = prior[n];
  int32_t* row = tables + (long long)n * g.max_blocks;
  int32_t* fr = freed + (long long)n * max_freed;
  int cnt = 0;
  if (L >= 0) {
    const int T = tail_of(g, tails, n, L);
    const long long nb_old_ll = ((long long)L + g.W + T + g.bs - 1) >> g.bs_shift;
    const int nb_old = (int)min(nb_old_ll, (long long)g.max_blocks);
    const int nb_new = (int)min((((long long)L + g.B + T + g.bs - 1) >> g.bs_shift), (long long)nb_old);
    cnt = min(nb_old - nb_new, max_freed);
    for (int k = tid; k < cnt; k += nthreads) {
      fr[k] = row[nb_new + k];
      row[nb_new + k] = -1;
    }
    if (tid == 0) seq_lens[n] = L + g.B + T;
  } else if (tid == 0) {
    seq_lens[n] = L;
  }
  if (tid == 0) num_freed[n] = cnt;
  for (int k = cnt + tid; k < max_freed; k += nthreads) fr[k] = -1;
}

}  // namespace kara
