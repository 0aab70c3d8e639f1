// Achievable-peak probes for gfx950, built into libkara_probes.so (not part
// of the Kara library).  Each launcher enqueues one kernel on `stream`; the
// caller times it with events and divides the work stated beside it.
//
//   kara_probe_mfma  : blocks x 4 waves, each iters x 4 MFMA 32x32x16 bf16
//                      (32768 FLOP per wave per MFMA), accumulators independent
//   kara_probe_exp   : blocks x 256 lanes, each iters x 8 v_exp_f32
//   kara_probe_fma   : blocks x 256 lanes, each iters x 8 v_fma_f32
//   kara_probe_read  : reads `bytes` once (16-byte non-temporal loads, 16 in
//                      flight per thread) and writes one float per thread
//   kara_probe_coissue: MFMAs alone, fp32 FMAs alone, and both interleaved in
//                      one instruction stream (4 MFMAs and 16 VALU operations
//                      per iteration), to see how far they run concurrently
//   kara_probe_copy  : copies `bytes` (reads and writes each byte once)
//   kara_probe_rewrite: reads `bytes` and writes them back in place, one
//                      workgroup per 16 KiB (the access shape of in-place
//                      row compaction)
// Work sizes must keep every index inside the buffers: bytes a multiple of
// 16, out holding blocks * 256 floats (read: grid * 256 floats, grid given).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kara_probes.h"

namespace kara_probes {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void probe_mfma(float* out, int iters) {
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(threadIdx.x * 1e-3f);
    b[i] = (__bf16)(i * 1e-3f);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

template <bool EXP>
__global__ __launch_bounds__(256) void probe_valu(float* out, int iters, float a) {
  float x[8];
  for (int e = 0; e < 8; ++e) x[e] = threadIdx.x * 1e-3f + 0.1f * e;
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = EXP ? __builtin_amdgcn_exp2f(x[e] * a) : __builtin_fmaf(x[e], a, 0.5f);
  float s = 0.f;
  for (int e = 0; e < 8; ++e) s += x[e];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Each workgroup streams whole 64 KiB chunks (16 loads of 16 bytes in flight
// per thread, a wave covering 1 KiB per load), chunks handed out grid-stride.
__global__ __launch_bounds__(256) void probe_read(const u32x4* __restrict__ src, size_t n, float* out) {
  constexpr int PER = 16;                                  // loads in flight per thread
  const size_t chunk = (size_t)256 * PER;                  // 16-byte elements per chunk
  const size_t nchunks = n / chunk;
  unsigned acc = 0;
  for (size_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
    const u32x4* p = src + c * chunk + threadIdx.x;
    u32x4 v[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) v[k] = __builtin_nontemporal_load(p + k * 256);
#pragma unroll
    for (int k = 0; k < PER; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (size_t i = nchunks * chunk + blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    acc ^= __builtin_nontemporal_load(src + i).x;
  out[blockIdx.x * blockDim.x + threadIdx.x] = (float)(acc & 1u);
}

__global__ __launch_bounds__(256) void probe_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  for (; i + stride < n; i += 2 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    __builtin_nontemporal_store(a, dst + i);
    __builtin_nontemporal_store(b, dst + i + stride);
  }
  for (; i < n; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// In-place rewrite: one short-lived workgroup per 16 KiB chunk, 4 loads of 16
// bytes in flight per thread, then the same 4 vectors stored back where they
// were read (each element is touched by one thread only).  Measured on
// gfx950 over 4 and 16 GiB: 4 vectors per thread sustain the most, 8 fall
// well behind.
constexpr int RW_PER = 4;
__global__ __launch_bounds__(256) void probe_rewrite(u32x4* buf, size_t n) {
  const size_t base = (size_t)blockIdx.x * 256 * RW_PER + threadIdx.x;
  u32x4 v[RW_PER];
#pragma unroll
  for (int k = 0; k < RW_PER; ++k)
    if (base + k * 256 < n) v[k] = __builtin_nontemporal_load(buf + base + k * 256);
#pragma unroll
  for (int k = 0; k < RW_PER; ++k)
    if (base + k * 256 < n) __builtin_nontemporal_store(v[k], buf + base + k * 256);
}

// MFMA / VALU co-issue: per iteration 4 independent 16x16x32 bf16 MFMAs
// (MODE 0), 16 independent fp32 FMAs (MODE 1), both interleaved as MFMA, 4
// FMAs, MFMA, ... (MODE 2), the MFMAs interleaved with 16 v_exp_f32 (MODE 3),
// or the 16 v_exp_f32 alone (MODE 4); modes 3 and 4 scale each exponent
// argument with a multiply first.  MODE 5: 16 bare v_exp_f32 (the argument is
// negated through the input modifier, no multiply); MODE 6: the 16 bare
// v_exp_f32 interleaved with 16 independent fp32 FMAs on other registers,
// which shows whether the exponential and the FMA pipelines overlap.
template <int MODE>
__global__ __launch_bounds__(512) void probe_coissue(float* out, int iters, float a) {
  bf16x8 x, y;
  for (int i = 0; i < 8; ++i) {
    x[i] = (__bf16)(threadIdx.x * 1e-3f);
    y[i] = (__bf16)(i * 1e-3f);
  }
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  f32x4 c[4] = {};
  float v[16], w[16];
  for (int e = 0; e < 16; ++e) {
    v[e] = threadIdx.x * 1e-3f + e * 1e-2f;
    w[e] = threadIdx.x * 1e-3f - e;
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if (MODE == 0 || MODE == 2 || MODE == 3) c[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, c[m], 0, 0, 0);
      if (MODE != 0) {
#pragma unroll
        for (int e = 4 * m; e < 4 * m + 4; ++e) {
          if (MODE >= 5) {
            v[e] = __builtin_amdgcn_exp2f(-v[e]);
            if (MODE == 6) w[e] = __builtin_fmaf(w[e], a, 0.5f);
          } else {
            v[e] = MODE >= 3 ? __builtin_amdgcn_exp2f(v[e] * a) : __builtin_fmaf(v[e], a, 0.5f);
          }
        }
      }
    }
    if (MODE == 6) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        __builtin_amdgcn_sched_group_barrier(0x400, 1, 0);   // one transcendental
        __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);   // then one other VALU instruction
      }
    }
  }
  float s = 0.f;
  for (int m = 0; m < 4; ++m) s += c[m][0] + c[m][1] + c[m][2] + c[m][3];
  for (int e = 0; e < 16; ++e) s += v[e] + (MODE == 6 ? w[e] : 0.f);
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// MFMA / VALU co-issue with a fixed number of waves per SIMD: 96 KiB of LDS
// keep one workgroup per compute unit, so `threads` / 256 waves share each
// SIMD.  Per iteration: NM independent 16x16x32 bf16 MFMAs and NV independent
// fp32 FMAs (VK = 0) or bare v_exp_f32 (VK = 1); with PAT the instruction
// stream is MFMA, NV / NM vector instructions, MFMA, ...
template <int NM, int NV, int VK, int PAT>
__global__ __launch_bounds__(512, 1) void probe_coissue_cu(float* out, int iters, float a) {
  extern __shared__ float lds_keep[];
  bf16x8 x[8], y;
  for (int i = 0; i < 8; ++i) {
    y[i] = (__bf16)(i * 1e-3f);
    for (int m = 0; m < 8; ++m) x[m][i] = (__bf16)(threadIdx.x * 1e-3f + m);
  }
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  f32x4 c[NM > 0 ? NM : 1];
  for (int m = 0; m < (NM > 0 ? NM : 1); ++m) c[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  float v[NV > 0 ? NV : 1];
  for (int e = 0; e < (NV > 0 ? NV : 1); ++e) v[e] = threadIdx.x * 1e-3f + e * 1e-2f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < NM; ++m) c[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x[m & 7], y, c[m], 0, 0, 0);
#pragma unroll
    for (int e = 0; e < NV; ++e) v[e] = VK == 0 ? __builtin_fmaf(v[e], a, 0.5f) : __builtin_amdgcn_exp2f(-v[e]);
    if (PAT && NM > 0 && NV > 0) {
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, NM > 0 ? NV / NM : 1, 0);
      }
    }
  }
  float s = 0.f;
  for (int m = 0; m < NM; ++m) s += c[m][0] + c[m][1] + c[m][2] + c[m][3];
  for (int e = 0; e < NV; ++e) s += v[e];
  if (s == 12345.f) lds_keep[threadIdx.x] = s;   // the LDS allocation stays
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// MFMA work and vector work in different waves of one SIMD: 512 threads with
// 96 KiB of LDS (one workgroup per compute unit, two waves per SIMD); waves
// 0-3 run NM independent MFMAs per iteration, waves 4-7 NV independent FMAs
// (VK = 0) or bare v_exp_f32 (VK = 1).  Lane 0 of each wave writes
// 1000 + 10 * (its SIMD from the HW_ID register) + (1 for a vector wave), so
// the host can check that every SIMD holds one wave of each kind.
template <int NM, int NV, int VK>
__global__ __launch_bounds__(512, 1) void probe_split_cu(float* out, int iters, float a) {
  extern __shared__ float lds_keep[];
  const int wave = threadIdx.x >> 6;
  const bool mfma_wave = wave < 4;
  float s = 0.f;
  if (mfma_wave) {
    bf16x8 x[8], y;
    for (int i = 0; i < 8; ++i) {
      y[i] = (__bf16)(i * 1e-3f);
      for (int m = 0; m < 8; ++m) x[m][i] = (__bf16)(threadIdx.x * 1e-3f + m);
    }
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    f32x4 c[NM];
    for (int m = 0; m < NM; ++m) c[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int m = 0; m < NM; ++m) c[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x[m & 7], y, c[m], 0, 0, 0);
    }
    for (int m = 0; m < NM; ++m) s += c[m][0] + c[m][1] + c[m][2] + c[m][3];
  } else {
    float v[NV];
    for (int e = 0; e < NV; ++e) v[e] = threadIdx.x * 1e-3f + e * 1e-2f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int e = 0; e < NV; ++e) v[e] = VK == 0 ? __builtin_fmaf(v[e], a, 0.5f) : __builtin_amdgcn_exp2f(-v[e]);
    }
    for (int e = 0; e < NV; ++e) s += v[e];
  }
  // HW_ID (hardware register 4), SIMD_ID field: bits 5:4
  const int simd = (int)__builtin_amdgcn_s_getreg((1 << 11) | (4 << 6) | 4);
  if (s == 12345.f) lds_keep[threadIdx.x] = s;   // the LDS allocation stays
  out[blockIdx.x * blockDim.x + threadIdx.x] =
      (threadIdx.x & 63) == 0 ? 1000.f + 10.f * simd + (mfma_wave ? 0.f : 1.f) : s;
}

static int status(hipError_t e) { return e == hipSuccess ? 0 : (int)e; }

}  // namespace kara_probes

using namespace kara_probes;

extern "C" {

int kara_probe_mfma(float* out, int blocks, int iters, void* stream) {
  if (!out || blocks < 1 || iters < 1) return -1;
  hipLaunchKernelGGL(probe_mfma, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
  return status(hipGetLastError());
}

int kara_probe_exp(float* out, int blocks, int iters, void* stream) {
  if (!out || blocks < 1 || iters < 1) return -1;
  hipLaunchKernelGGL(probe_valu<true>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters, 0.999f);
  return status(hipGetLastError());
}

int kara_probe_fma(float* out, int blocks, int iters, void* stream) {
  if (!out || blocks < 1 || iters < 1) return -1;
  hipLaunchKernelGGL(probe_valu<false>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters, 0.999f);
  return status(hipGetLastError());
}

int kara_probe_read(const void* src, size_t bytes, float* out, int grid, void* stream) {
  if (!src || !out || grid < 1 || (bytes & 15)) return -1;
  hipLaunchKernelGGL(probe_read, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src, bytes / 16,
                     out);
  return status(hipGetLastError());
}

int kara_probe_copy(const void* src, void* dst, size_t bytes, int grid, void* stream) {
  if (!src || !dst || grid < 1 || (bytes & 15)) return -1;
  hipLaunchKernelGGL(probe_copy, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src, (u32x4*)dst,
                     bytes / 16);
  return status(hipGetLastError());
}

int kara_probe_coissue(int mode, float* out, int blocks, int threads, int iters, void* stream) {
  if (!out || blocks < 1 || iters < 1 || threads < 64 || threads > 512 || threads % 64) return -1;
  const dim3 g(blocks), b(threads);
  const hipStream_t st = (hipStream_t)stream;
  switch (mode) {
    case 0: hipLaunchKernelGGL(probe_coissue<0>, g, b, 0, st, out, iters, 0.999f); break;
    case 1: hipLaunchKernelGGL(probe_coissue<1>, g, b, 0, st, out, iters, 0.999f); break;
    case 2: hipLaunchKernelGGL(probe_coissue<2>, g, b, 0, st, out, iters, 0.999f); break;
    case 3: hipLaunchKernelGGL(probe_coissue<3>, g, b, 0, st, out, iters, 0.999f); break;
    case 4: hipLaunchKernelGGL(probe_coissue<4>, g, b, 0, st, out, iters, 0.999f); break;
    case 5: hipLaunchKernelGGL(probe_coissue<5>, g, b, 0, st, out, iters, 0.999f); break;
    case 6: hipLaunchKernelGGL(probe_coissue<6>, g, b, 0, st, out, iters, 0.999f); break;
    default: return -1;
  }
  return status(hipGetLastError());
}

int kara_probe_coissue_cu(int mode, float* out, int blocks, int threads, int iters, void* stream) {
  if (!out || blocks < 1 || iters < 1 || (threads != 256 && threads != 512)) return -1;
  const dim3 g(blocks), b(threads);
  const size_t lds = 96 * 1024;
  const hipStream_t st = (hipStream_t)stream;
  switch (mode) {
    case 0: hipLaunchKernelGGL((probe_coissue_cu<16, 0, 0, 0>), g, b, lds, st, out, iters, 0.999f); break;
    case 1: hipLaunchKernelGGL((probe_coissue_cu<0, 64, 0, 0>), g, b, lds, st, out, iters, 0.999f); break;
    case 2: hipLaunchKernelGGL((probe_coissue_cu<16, 16, 0, 1>), g, b, lds, st, out, iters, 0.999f); break;
    case 3: hipLaunchKernelGGL((probe_coissue_cu<16, 32, 0, 1>), g, b, lds, st, out, iters, 0.999f); break;
    case 4: hipLaunchKernelGGL((probe_coissue_cu<16, 64, 0, 1>), g, b, lds, st, out, iters, 0.999f); break;
    case 5: hipLaunchKernelGGL((probe_coissue_cu<0, 32, 1, 0>), g, b, lds, st, out, iters, 0.999f); break;
    case 6: hipLaunchKernelGGL((probe_coissue_cu<16, 32, 1, 1>), g, b, lds, st, out, iters, 0.999f); break;
    case 7:
    case 8:
      if (threads != 512) return -1;
      if (mode == 7) hipLaunchKernelGGL((probe_split_cu<16, 64, 0>), g, b, lds, st, out, iters, 0.999f);
      else hipLaunchKernelGGL((probe_split_cu<16, 32, 1>), g, b, lds, st, out, iters, 0.999f);
      break;
    default: return -1;
  }
  return status(hipGetLastError());
}

int kara_probe_rewrite(void* buf, size_t bytes, void* stream) {
  if (!buf || (bytes & 15)) return -1;
  const size_t chunks = (bytes / 16 + 256 * RW_PER - 1) / (256 * RW_PER);
  if (chunks == 0) return 0;
  if (chunks > 0x7fffffffULL) return -1;
  hipLaunchKernelGGL(probe_rewrite, dim3((unsigned)chunks), dim3(256), 0, (hipStream_t)stream, (u32x4*)buf,
                     bytes / 16);
  return status(hipGetLastError());
}

}  // extern "C"
