// Single-pass window scoring for windows of up to 1024 keys (bf16, head_dim 128).
//
// Same quantity as the two-pass kernels in score.hip (Kara's bidirectional
// in-window attention column mass, English abstract of "Kara: Efficient
// Reasoning LLM Serving via Sliding-Window KV Cache Compression"):
//     c[j] = sum_{h in group g} sum_{i < W} softmax_j'(q[h,i] . k[j'] / sqrt(d))[j].
//
// One workgroup of 8 waves owns one unit.  Each wave keeps 128 window keys in
// registers for the whole unit (the unit's K is read from memory once), and
// the unit's G*W query rows stream through LDS in blocks of 16.  Per block a
// wave computes the 16 x 128 logits of its keys with 16x16x32 MFMAs in the
// transposed orientation S^T = K Q^T, so a lane owns one query row and 32 of
// the wave's keys:
//   - row max and row sum are lane-local, then merged over the 4 lane groups
//     that share a row (two shuffles) and over the 8 waves (LDS, one barrier
//     each);
//   - the softmax weight of every logit is exp2(x - m) / l with one row
//     weight 1/l per lane, and the column sums accumulate lane-locally across
//     all blocks of the unit; they are reduced over the 16 query lanes once,
//     at the end.
// Each logit is computed once and exponentiated once.
#include "kara_device.h"

namespace kara {

typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int FW = 8;            // waves per workgroup
constexpr int FTHREADS = FW * 64;
constexpr int KTW = 8;           // 16-key tiles per wave (128 keys)
constexpr int QB = 16;           // query rows per block
constexpr int FD = 128;          // head_dim of this kernel
constexpr int QROWB = FD * 2;    // bytes per bf16 row
constexpr int QLROW = QROWB + 16;  // padded LDS row

__device__ __forceinline__ f32x4v mfma16(const bf16x8& a, const bf16x8& b, const f32x4v& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16x16x32 operand layout: lane l supplies row (or column) l % 16 and the 8
// reduction elements 8*(l/16) .. +7 of each instruction.  The reduction order
// over head_dim is free, so lane group q = l/16 feeds the contiguous range
// [32q, 32q+32) of head_dim, 8 elements per instruction, for both operands.
// Result: lane l holds column l % 16 and rows 4*(l/16) .. +3.

__global__ __launch_bounds__(FTHREADS, 1) void fused_score_kernel(Geo g, const __bf16* __restrict__ q,
                                                                   const __bf16* __restrict__ kc,
                                                                   const int32_t* __restrict__ tables,
                                                                   const int32_t* __restrict__ prior,
                                                                   float* __restrict__ scores) {
  __shared__ __align__(16) unsigned char qtile[2][QB * QLROW];
  __shared__ float red_max[QB][FW];
  __shared__ float red_sum[QB][FW];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int qlane = lane & 15, grp = lane >> 4;
  const int unit = blockIdx.x;
  const int kvh = unit % g.Hkv;
  const int layer = (unit / g.Hkv) % g.Lyr;
  const int n = unit / (g.Hkv * g.Lyr);
  const int L = prior[n];
  const int32_t* trow = tables + (long long)n * g.max_blocks;

  // ---- resident keys: tile t of this wave covers window keys key0 + 16 t + (0..15)
  const int key0 = wave * KTW * 16;
  const unsigned char* kbytes = reinterpret_cast<const unsigned char*>(kc);
  const PagedRows pr = paged_rows(g, trow, layer, kvh, L, 2);
  bf16x8 kf[KTW][4];
#pragma unroll
  for (int t = 0; t < KTW; ++t) {
    const int j = min(key0 + 16 * t + qlane, g.W - 1);
    const uint4* src = reinterpret_cast<const uint4*>(kbytes + paged_row(pr, L + j) + grp * 64);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 v = src[s];
      __builtin_memcpy(&kf[t][s], &v, 16);
    }
  }
  // keys this lane holds in tile t: key0 + 16 t + 4 grp + r, valid if < W
  const int kbase = key0 + 4 * grp;

  // ---- query rows of block b: rows 16 b .. 16 b + 15 of the unit (row = i*G + h)
  const unsigned char* qbytes = reinterpret_cast<const unsigned char*>(
      q + (((long long)n * g.Lyr + layer) * g.W) * g.Hq * FD + (long long)kvh * g.G * FD);
  const int nblk = (g.GW + QB - 1) / QB;
  // staging: 256 threads move 16 rows x 256 bytes (one 16-byte chunk each)
  const int srow = (tid >> 4) & 15, sch = tid & 15;
  auto q_fetch = [&](int b) -> uint4 {
    const int row = min(b * QB + srow, g.GW - 1);
    const int qi = row / g.G, qh = row - qi * g.G;
    return *reinterpret_cast<const uint4*>(qbytes + ((long long)qi * g.Hq + qh) * QROWB + sch * 16);
  };

  f32x4v colacc[KTW];
#pragma unroll
  for (int t = 0; t < KTW; ++t) colacc[t] = f32x4v{0.f, 0.f, 0.f, 0.f};

  uint4 pre = make_uint4(0, 0, 0, 0);
  if (tid < 256) {
    pre = q_fetch(0);
    *reinterpret_cast<uint4*>(&qtile[0][srow * QLROW + sch * 16]) = pre;
  }
  __syncthreads();
  const float alpha = g.alpha;
  for (int b = 0; b < nblk; ++b) {
    const int buf = b & 1;
    if (tid < 256) pre = q_fetch(min(b + 1, nblk - 1));
    // B operand: query row qlane of this block, head_dim range [32 grp, 32 grp + 32)
    bf16x8 qf[4];
    {
      const uint4* p = reinterpret_cast<const uint4*>(&qtile[buf][qlane * QLROW + grp * 64]);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint4 v = p[s];
        __builtin_memcpy(&qf[s], &v, 16);
      }
    }
    // logits S^T: acc[t][r] = k[key0 + 16t + 4grp + r] . q[row 16b + qlane]
    f32x4v acc[KTW];
#pragma unroll
    for (int t = 0; t < KTW; ++t) {
      f32x4v a = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) a = mfma16(kf[t][s], qf[s], a);
      acc[t] = a;
    }
    // keys past the window (only in the last tiles) do not take part
    if (key0 + KTW * 16 > g.W) {
#pragma unroll
      for (int t = 0; t < KTW; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (kbase + 16 * t + r >= g.W) acc[t][r] = -INFINITY;
    }
    // row max: lane-local, then the 4 lane groups, then the 8 waves
    float mx = fmaxf(acc[0][0], acc[0][1]);
    mx = fmaxf(mx, fmaxf(acc[0][2], acc[0][3]));
#pragma unroll
    for (int t = 1; t < KTW; ++t) {
      mx = fmaxf(mx, fmaxf(acc[t][0], acc[t][1]));
      mx = fmaxf(mx, fmaxf(acc[t][2], acc[t][3]));
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (lane < 16) red_max[qlane][wave] = mx;
    __syncthreads();
    {
      const f32x4v a = *reinterpret_cast<const f32x4v*>(&red_max[qlane][0]);
      const f32x4v c = *reinterpret_cast<const f32x4v*>(&red_max[qlane][4]);
      mx = fmaxf(fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3])), fmaxf(fmaxf(c[0], c[1]), fmaxf(c[2], c[3])));
    }
    // exponentials (in place) and row sum; a wave with no valid key has mx = -inf
    // only if every wave does, which cannot happen (W >= 1)
    const float moff = -mx * alpha;
    float sm = 0.f;
#pragma unroll
    for (int t = 0; t < KTW; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = fast_exp2(__builtin_fmaf(acc[t][r], alpha, moff));
        acc[t][r] = e;
        sm += e;
      }
    sm += __shfl_xor(sm, 16);
    sm += __shfl_xor(sm, 32);
    if (lane < 16) red_sum[qlane][wave] = sm;
    // publish the next query tile before the barrier that ends this block's reads
    if (tid < 256) *reinterpret_cast<uint4*>(&qtile[buf ^ 1][srow * QLROW + sch * 16]) = pre;
    __syncthreads();
    {
      const f32x4v a = *reinterpret_cast<const f32x4v*>(&red_sum[qlane][0]);
      const f32x4v c = *reinterpret_cast<const f32x4v*>(&red_sum[qlane][4]);
      sm = ((a[0] + a[1]) + (a[2] + a[3])) + ((c[0] + c[1]) + (c[2] + c[3]));
    }
    // rows past G*W contribute nothing
    const float w = (b * QB + qlane < g.GW) ? __builtin_amdgcn_rcpf(sm) : 0.f;
#pragma unroll
    for (int t = 0; t < KTW; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) colacc[t][r] = __builtin_fmaf(acc[t][r], w, colacc[t][r]);
  }
  // column sums over the 16 query lanes of each lane group (xor within 16 lanes)
#pragma unroll
  for (int t = 0; t < KTW; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v = colacc[t][r];
      v += __shfl_xor(v, 1);
      v += __shfl_xor(v, 2);
      v += __shfl_xor(v, 4);
      v += __shfl_xor(v, 8);
      colacc[t][r] = v;
    }
  // lane (grp, qlane) writes value (t = qlane / 2, r = 2 (qlane % 2) .. +1)
  float* out = scores + (long long)unit * g.W;
#pragma unroll
  for (int t = 0; t < KTW; ++t)
    if ((qlane >> 1) == t) {
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const int r = 2 * (qlane & 1) + rr;
        const int key = kbase + 16 * t + r;
        if (key < g.W) out[key] = colacc[t][r];
      }
    }
}

hipError_t launch_fused_score(const Geo& g, const void* q, const void* kc, const int32_t* tables,
                              const int32_t* prior, float* scores, hipStream_t st) {
  const long long units = (long long)g.S * g.Lyr * g.Hkv;
  if (units > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(fused_score_kernel, dim3((unsigned)units), dim3(FTHREADS), 0, st, g, (const __bf16*)q,
                     (const __bf16*)kc, tables, prior, scores);
  return hipGetLastError();
}

bool fused_score_supported(const Geo& g, int dtype) {
  return dtype == KARA_BF16 && g.D == FD && g.W <= FW * KTW * 16;
}

}  // namespace kara
