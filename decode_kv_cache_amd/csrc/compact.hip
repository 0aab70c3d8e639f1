// In-place compaction of the kept window rows into PagedAttention blocks, and
// the block-table rewrite that frees the tail.
//
// Kara's English abstract: the method is adapted to PagedAttention and lowers
// KV-cache memory.  Recorded reading: for unit (n, l, g) and r < B, logical
// slot L+r takes the old row of slot L+kept[r] (K and V); afterwards, per
// sequence, the table entries of logical blocks ceil((L+B)/bs) ..
// ceil((L+W)/bs)-1 are handed back in order and set to -1.
//
// In-place safety: kept is strictly ascending, so kept[r] >= r.  One
// workgroup owns one (unit, K-or-V) and walks the rows in ascending chunks:
// it reads a whole chunk into registers, waits for the reads, synchronises,
// then writes the chunk.  A chunk's writes land on slots < L + (end of chunk)
// while every later source is at or past that point, and every source a
// later write could hit was read before the barrier of its own chunk.
#include "kara_device.h"

namespace kara {

constexpr int CMP_THREADS = 256;
// rows are streamed once: non-temporal loads and stores keep them out of the caches
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int CMP_VEC = 16;  // 16-byte vectors per thread per chunk (256 rows of 256 B)

template <int ROWBYTES>
__global__ __launch_bounds__(CMP_THREADS) void compact_kernel(Geo g, unsigned char* __restrict__ kc,
                                                              unsigned char* __restrict__ vc,
                                                              const int32_t* __restrict__ tables,
                                                              const int32_t* __restrict__ prior,
                                                              const int32_t* __restrict__ kept, int esize) {
  constexpr int TPR = ROWBYTES / 16;                  // threads per row
  constexpr int RPP = CMP_THREADS / TPR;              // rows per pass
  constexpr int CH = RPP * CMP_VEC;                   // rows per chunk
  const long long unit = blockIdx.x >> 1;
  unsigned char* pool = (blockIdx.x & 1) ? vc : kc;
  const int kvh = (int)(unit % g.Hkv);
  const int layer = (int)((unit / g.Hkv) % g.Lyr);
  const int n = (int)(unit / ((long long)g.Hkv * g.Lyr));
  const int L = prior[n];
  const int32_t* trow = tables + (long long)n * g.max_blocks;
  const int32_t* kl = kept + unit * g.B;
  const int t = threadIdx.x;
  const int part = t % TPR;
  const int rsub = t / TPR;
  for (int c0 = 0; c0 < g.B; c0 += CH) {
    u32x4 buf[CMP_VEC];
    long long dst[CMP_VEC];
#pragma unroll
    for (int v = 0; v < CMP_VEC; ++v) {
      const int r = c0 + v * RPP + rsub;
      dst[v] = -1;
      if (r < g.B) {
        const int j = kl[r];
        const long long so = (j >= 0 && j < g.W) ? slot_offset(g, trow, layer, kvh, L + j) : -1;
        const long long d = slot_offset(g, trow, layer, kvh, L + r);
        if (so >= 0 && d >= 0) {
          buf[v] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(pool + so * esize + part * 16));
          dst[v] = d;
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);   // every read of this chunk has returned
    __syncthreads();
#pragma unroll
    for (int v = 0; v < CMP_VEC; ++v)
      if (dst[v] >= 0) __builtin_nontemporal_store(buf[v], reinterpret_cast<u32x4*>(pool + dst[v] * esize + part * 16));
  }
}

// One thread per sequence: freed list, table truncation, new length.
__global__ void finalize_kernel(Geo g, int32_t* __restrict__ tables, const int32_t* __restrict__ prior,
                                int32_t* __restrict__ seq_lens, int32_t* __restrict__ freed,
                                int32_t* __restrict__ num_freed, int max_freed) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= g.S) return;
  const int L = prior[n];
  int32_t* row = tables + (long long)n * g.max_blocks;
  int32_t* fr = freed + (long long)n * max_freed;
  int cnt = 0;
  if (L >= 0) {
    const long long nb_old_ll = ((long long)L + g.W + g.bs - 1) >> g.bs_shift;
    const int nb_old = (int)min(nb_old_ll, (long long)g.max_blocks);
    const int nb_new = (int)min((((long long)L + g.B + g.bs - 1) >> g.bs_shift), (long long)nb_old);
    for (int b = nb_new; b < nb_old && cnt < max_freed; ++b) {
      fr[cnt++] = row[b];
      row[b] = -1;
    }
    seq_lens[n] = L + g.B;
  } else {
    seq_lens[n] = L;
  }
  num_freed[n] = cnt;
  for (int k = cnt; k < max_freed; ++k) fr[k] = -1;
}

hipError_t launch_compact(const Geo& g, int dtype, void* kc, void* vc, int32_t* tables, const int32_t* prior,
                          int32_t* seq_lens, const int32_t* kept, int32_t* freed, int32_t* num_freed,
                          int max_freed, hipStream_t st) {
  const long long units = (long long)g.S * g.Lyr * g.Hkv;
  if (2 * units > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const int esize = dtype == KARA_BF16 ? 2 : 4;
  const int rowbytes = g.D * esize;
  if (units > 0) {
    const dim3 grid((unsigned)(2 * units));
    if (rowbytes == 128)
      hipLaunchKernelGGL(compact_kernel<128>, grid, dim3(CMP_THREADS), 0, st, g, (unsigned char*)kc,
                         (unsigned char*)vc, tables, prior, kept, esize);
    else if (rowbytes == 256)
      hipLaunchKernelGGL(compact_kernel<256>, grid, dim3(CMP_THREADS), 0, st, g, (unsigned char*)kc,
                         (unsigned char*)vc, tables, prior, kept, esize);
    else
      hipLaunchKernelGGL(compact_kernel<512>, grid, dim3(CMP_THREADS), 0, st, g, (unsigned char*)kc,
                         (unsigned char*)vc, tables, prior, kept, esize);
  }
  hipLaunchKernelGGL(finalize_kernel, dim3((g.S + 255) / 256), dim3(256), 0, st, g, tables, prior, seq_lens,
                     freed, num_freed, max_freed);
  return hipGetLastError();
}

// One workgroup checks every sequence's addressing data.
__global__ void validate_kernel(Geo g, const int32_t* __restrict__ tables, const int32_t* __restrict__ prior,
                                int32_t* __restrict__ bad) {
  __shared__ int cnt;
  if (threadIdx.x == 0) cnt = 0;
  __syncthreads();
  for (int n = threadIdx.x; n < g.S; n += blockDim.x) {
    const int L = prior[n];
    bool ok = L >= 0 && (long long)L + g.W <= (long long)g.max_blocks * g.bs;
    if (ok) {
      const int b0 = L >> g.bs_shift;
      const int b1 = (int)(((long long)L + g.W + g.bs - 1) >> g.bs_shift);
      for (int b = b0; b < b1; ++b) {
        const int blk = tables[(long long)n * g.max_blocks + b];
        if (blk < 0 || (long long)blk >= g.nblocks) ok = false;
      }
    }
    if (!ok) atomicAdd(&cnt, 1);
  }
  __syncthreads();
  if (threadIdx.x == 0) *bad = cnt;
}

hipError_t launch_validate(const Geo& g, const int32_t* tables, const int32_t* prior, int32_t* bad,
                           hipStream_t st) {
  hipLaunchKernelGGL(validate_kernel, dim3(1), dim3(256), 0, st, g, tables, prior, bad);
  return hipGetLastError();
}

}  // namespace kara
