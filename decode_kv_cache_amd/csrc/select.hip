// Token2Chunk selection kernel: one workgroup of 256 threads per unit runs
// the selection of select_core.h on the unit's scores (Kara's English
// abstract: a subset of the selected KV pairs is expanded into chunks).
#include "select_core.h"

namespace kara {

constexpr int SEL_THREADS = 256;

// gap > 0 selects the bridging variant: neighbouring seeds (by position) that
// leave at most `gap` positions between them also keep everything in between.
__global__ __launch_bounds__(SEL_THREADS) void select_kernel(Geo g, int gap, const float* __restrict__ scores,
                                                             int32_t* __restrict__ kept,
                                                             uint8_t* __restrict__ mask) {
  extern __shared__ __align__(16) unsigned char smem[];
  SelScratch<SEL_THREADS>& sh = *reinterpret_cast<SelScratch<SEL_THREADS>*>(smem);
  uint32_t* keys = reinterpret_cast<uint32_t*>(smem + sizeof(SelScratch<SEL_THREADS>));
  uint8_t* flags = reinterpret_cast<uint8_t*>(keys + g.W);
  const long long unit = blockIdx.x;
  const float* sc = scores + unit * g.W;
  for (int j = threadIdx.x; j < g.W; j += SEL_THREADS) keys[j] = order_key(sc[j]);
  __syncthreads();
  select_unit<SEL_THREADS, 8192 / SEL_THREADS>(g, gap, keys, flags, sh, nullptr, kept + unit * g.B, mask ? mask + unit * g.W : nullptr);
}

hipError_t launch_select(const Geo& g, int gap, const float* scores, int32_t* kept, uint8_t* mask,
                         hipStream_t st) {
  const long long units = (long long)g.S * g.Lyr * g.Hkv;
  if (units > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const size_t lds = sizeof(SelScratch<SEL_THREADS>) + (size_t)g.W * 4 + (size_t)g.W;
  hipLaunchKernelGGL(select_kernel, dim3((unsigned)units), dim3(SEL_THREADS), lds, st, g, gap, scores, kept, mask);
  return hipGetLastError();
}

}  // namespace kara
