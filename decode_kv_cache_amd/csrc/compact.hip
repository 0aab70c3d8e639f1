// Compaction kernels: one workgroup per unit copies the kept K and V rows
// into place (compact_core.h), then one wave per sequence rewrites its
// block table.  Kara's English abstract: the method is adapted to
// PagedAttention and lowers KV-cache memory.
#include "compact_core.h"

namespace kara {

constexpr int CMP_THREADS = 256;
// 16-byte vectors per thread and pool per chunk: 80 rows of 256 B per chunk,
// 10 loads in flight per thread; a small register footprint keeps many
// workgroups resident, which is what sustains the bandwidth
constexpr int CMP_VEC = 5;

template <int ROWBYTES>
__global__ __launch_bounds__(CMP_THREADS) void compact_kernel(Geo g, unsigned char* __restrict__ kc,
                                                              unsigned char* __restrict__ vc,
                                                              const int32_t* __restrict__ tables,
                                                              const int32_t* __restrict__ prior,
                                                              const int32_t* __restrict__ kept,
                                                              const int32_t* __restrict__ tails, int esize) {
  const long long unit = blockIdx.x;
  const int kvh = (int)(unit % g.Hkv);
  const int layer = (int)((unit / g.Hkv) % g.Lyr);
  const int n = (int)(unit / ((long long)g.Hkv * g.Lyr));
  const int L = prior[n];
  compact_unit_rows<CMP_THREADS, ROWBYTES, CMP_VEC>(g, kc, vc, tables + (long long)n * g.max_blocks, layer, kvh,
                                                   L, kept + unit * g.B, esize, tail_of(g, tails, n, L));
}

// One wave per sequence: freed list, table truncation, new length.
constexpr int FIN_THREADS = 64;
__global__ __launch_bounds__(FIN_THREADS) void finalize_kernel(Geo g, int32_t* __restrict__ tables,
                                                               const int32_t* __restrict__ prior,
                                                               int32_t* __restrict__ seq_lens,
                                                               int32_t* __restrict__ freed,
                                                               int32_t* __restrict__ num_freed, int max_freed,
                                                               const int32_t* __restrict__ tails) {
  finalize_sequence(g, blockIdx.x, tables, prior, seq_lens, freed, num_freed, max_freed, tails, threadIdx.x,
                    FIN_THREADS);
}

hipError_t launch_compact(const Geo& g, int dtype, void* kc, void* vc, int32_t* tables, const int32_t* prior,
                          int32_t* seq_lens, const int32_t* kept, int32_t* freed, int32_t* num_freed,
                          int max_freed, const int32_t* tails, hipStream_t st) {
  const long long units = (long long)g.S * g.Lyr * g.Hkv;
  if (units > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const int esize = dtype == KARA_BF16 ? 2 : 4;
  const int rowbytes = g.D * esize;
  if (units > 0) {
    const dim3 grid((unsigned)units);
    if (rowbytes == 128)
      hipLaunchKernelGGL(compact_kernel<128>, grid, dim3(CMP_THREADS), 0, st, g, (unsigned char*)kc,
                         (unsigned char*)vc, tables, prior, kept, tails, esize);
    else if (rowbytes == 256)
      hipLaunchKernelGGL(compact_kernel<256>, grid, dim3(CMP_THREADS), 0, st, g, (unsigned char*)kc,
                         (unsigned char*)vc, tables, prior, kept, tails, esize);
    else
      hipLaunchKernelGGL(compact_kernel<512>, grid, dim3(CMP_THREADS), 0, st, g, (unsigned char*)kc,
                         (unsigned char*)vc, tables, prior, kept, tails, esize);
  }
  if (g.S > 0)
    hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)g.S), dim3(FIN_THREADS), 0, st, g, tables, prior, seq_lens,
                       freed, num_freed, max_freed, tails);
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
