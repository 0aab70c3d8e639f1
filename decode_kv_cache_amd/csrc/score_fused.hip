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
//   - the row max is lane-local, then merged over the 4 lane groups that
//     share a row (two lane swaps); the row sum of the wave's exponentials is
//     a product with an all-ones matrix on the matrix cores (fp16 terms, fp32
//     sum), which also spans the 4 lane groups; both are merged over the 8
//     waves through LDS, one barrier per block;
//   - every logit's softmax weight is a per-lane scalar times its
//     exponential, and the column sums accumulate lane-locally across all
//     blocks of the unit; they are reduced over the 16 query lanes once, at
//     the end.  A block's column updates are issued among the next block's
//     MFMAs, and so is most of the next block's row max.
// Each logit is computed once and exponentiated once.
#include <mutex>
#include <type_traits>

#include "compact_core.h"
#include "kara_device.h"
#include "select_core.h"

namespace kara {

typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

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

// max / sum over the 4 lane groups that hold the same query row (lanes l,
// l^16, l^32, l^48): two lane-swap steps, no LDS traffic
__device__ __forceinline__ float group_max(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group_sum(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// max over the 8 logits of two tiles, starting from m (or from the first
// logit when FIRST): three-input maxima, two new logits per instruction
__device__ __forceinline__ float pair_max(bool first, float m, const f32x4v& a, const f32x4v& b) {
  if (first) {
    m = fmaxf(fmaxf(a[0], a[1]), a[2]);
    m = fmaxf(fmaxf(m, a[3]), b[0]);
    m = fmaxf(fmaxf(m, b[1]), b[2]);
    return fmaxf(m, b[3]);
  }
  m = fmaxf(fmaxf(m, a[0]), a[1]);
  m = fmaxf(fmaxf(m, a[2]), a[3]);
  m = fmaxf(fmaxf(m, b[0]), b[1]);
  return fmaxf(fmaxf(m, b[2]), b[3]);
}

// Per block, each wave exponentiates its logits against its own row maximum
// m_w and publishes (m_w, l_w = sum of its exponentials).  After the one
// barrier of the block every wave combines the 8 pairs,
//     m = max_w m_w,   l = sum_w l_w 2^(alpha (m_w - m)),
// and weights its exponentials by 2^(alpha (m_w - m)) / l, which is the
// softmax over all W keys of the row.
template <bool MASK, bool LIN>
__device__ __forceinline__ void fused_unit(const Geo& g, int unit, const __bf16* __restrict__ q,
                                           const bf16x8 (&kf)[KTW][4], int key0, unsigned char (*qtile)[QB * QLROW],
                                           float2 (*red)[QB][FW], float* __restrict__ scores,
                                           uint32_t* keys_lds) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int qlane = lane & 15, grp = lane >> 4;
  const int kvh = unit % g.Hkv;
  const int layer = (unit / g.Hkv) % g.Lyr;
  const int n = unit / (g.Hkv * g.Lyr);
  const int kbase = key0 + 4 * grp;    // lane holds keys kbase + 16 t + r

  // ---- query rows of block b: rows 16 b .. 16 b + 15 of the unit (row = i*G + h)
  const unsigned char* qbytes = reinterpret_cast<const unsigned char*>(
      q + (((long long)n * g.Lyr + layer) * g.W) * g.Hq * FD + (long long)kvh * g.G * FD);
  const int nblk = (g.GW + QB - 1) / QB;
  // staging: the 512 threads move 16 rows x 256 bytes, 8 bytes each; tiles are
  // fetched two blocks ahead (two register stages) to cover memory latency
  const int srow = tid >> 5, sbyte = (tid & 31) * 8;
  // LIN (G divides the block height and every block is full): a thread's row
  // of block b sits at a fixed offset plus b times the bytes of QB / G window
  // positions, so the block's base address is one scalar step and a lane adds
  // a 32-bit offset: no vector arithmetic per block.  Otherwise the row is
  // split into (position, head) by division.
  const long long lstep = (long long)(QB / g.G) * g.Hq * QROWB;
  const uint32_t qoff = (uint32_t)(((srow / g.G) * g.Hq + srow % g.G) * QROWB + sbyte);   // < 2^22
  auto q_fetch = [&](int b) -> uint2 {
    if (LIN) return *reinterpret_cast<const uint2*>(qbytes + b * lstep + qoff);
    const int row = min(b * QB + srow, g.GW - 1);
    const int qi = row / g.G, qh = row - qi * g.G;
    return *reinterpret_cast<const uint2*>(qbytes + ((long long)qi * g.Hq + qh) * QROWB + sbyte);
  };
  auto q_stash = [&](int buf, uint2 v) { *reinterpret_cast<uint2*>(&qtile[buf][srow * QLROW + sbyte]) = v; };

  f32x4v colacc[KTW];
#pragma unroll
  for (int t = 0; t < KTW; ++t) colacc[t] = f32x4v{0.f, 0.f, 0.f, 0.f};
  f16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (_Float16)1.f;

  q_stash(0, q_fetch(0));
  uint2 stage1 = q_fetch(min(1, nblk - 1));    // tile b+1
  __syncthreads();
  const float alpha = g.alpha;
  // Each block is split in two steps.  logits(b) fetches tile b+2, reads tile
  // b from LDS and computes the block's logits; when the previous block's
  // exponentials are still in `acc` (PREV), each tile's four are folded into
  // the column sums, with that block's weight, before the tile's accumulator
  // takes the new logits, so the column updates of block b-1 issue among the
  // MFMAs of block b.  stats(b) turns the logits into exponentials,
  // publishes the wave's (max, sum) pair and tile b+1, and after the block's
  // barrier combines the pairs into this wave's weight for block b.  Every
  // column sum still takes its terms in block order, as one FMA each.
  f32x4v acc[KTW];
  float wgt = 0.f;
  float pmx = 0.f;   // running row max over the tiles finished so far (no mask)
  auto logits = [&](auto prev, int b, uint2& nxt) {
    constexpr bool PREV = decltype(prev)::value;
    const int buf = b & 1;
    nxt = q_fetch(min(b + 2, nblk - 1));
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
    // logits S^T: acc[t][r] = k[kbase + 16t + r] . q[row 16b + qlane], two
    // tiles at a time (each tile's four MFMAs chain on one accumulator).
    // The previous block's column updates (32 FMAs) and the row max over the
    // tiles already finished (12 three-input maxima) have no dependence on
    // these MFMAs, so they are issued between them: the matrix core runs an
    // MFMA for 16 cycles while the vector unit takes about two instructions.
    // The section is fenced by scheduling barriers; empty asm statements pin
    // its inputs (query fragments, previous exponentials) and outputs (logits,
    // column sums) to it, and group barriers set the order MFMA, vector
    // instruction(s), MFMA, ...  The wave raises its issue priority for the
    // section so that, of the two waves sharing a SIMD, the one with MFMAs
    // ready goes first.
    __builtin_amdgcn_s_setprio(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 4; ++s) asm volatile("" : "+v"(qf[s]));
    if (PREV) {
#pragma unroll
      for (int t = 0; t < KTW; ++t) asm volatile("" : "+v"(acc[t]));
    }
#pragma unroll
    for (int t0 = 0; t0 < KTW; t0 += 2) {
      f32x4v n0 = mfma16(kf[t0][0], qf[0], f32x4v{0.f, 0.f, 0.f, 0.f});
      f32x4v n1 = mfma16(kf[t0 + 1][0], qf[0], f32x4v{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int s = 1; s < 4; ++s) {
        n0 = mfma16(kf[t0][s], qf[s], n0);
        n1 = mfma16(kf[t0 + 1][s], qf[s], n1);
      }
      if (PREV) {
#pragma unroll
        for (int t = t0; t < t0 + 2; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) colacc[t][r] = __builtin_fmaf(acc[t][r], wgt, colacc[t][r]);
      }
      // the previous pair's logits are complete: extend the row max over them
      if (!MASK && t0 > 0) pmx = pair_max(t0 == 2, pmx, acc[t0 - 2], acc[t0 - 1]);
      acc[t0] = n0;
      acc[t0 + 1] = n1;
    }
#pragma unroll
    for (int t = 0; t < KTW; ++t) asm volatile("" : "+v"(acc[t]));
    if (PREV) {
#pragma unroll
      for (int t = 0; t < KTW; ++t) asm volatile("" : "+v"(colacc[t]));
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
      }
#pragma unroll
      for (int i = 0; i < 12; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, MASK ? 1 : 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
  };
  auto stats = [&](int b, uint2& cur) {
    const int buf = b & 1;
    if (MASK) {                                  // keys past the window take no part
#pragma unroll
      for (int t = 0; t < KTW; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (kbase + 16 * t + r >= g.W) acc[t][r] = -INFINITY;
    }
    // wave-local row max (raw logits)
    // (a linear chain of three-input maxima: two new logits per instruction)
    float mx;
    if (MASK) {
      mx = fmaxf(fmaxf(acc[0][0], acc[0][1]), acc[0][2]);
      mx = fmaxf(fmaxf(mx, acc[0][3]), acc[1][0]);
#pragma unroll
      for (int i = 5; i + 1 < 4 * KTW; i += 2) mx = fmaxf(fmaxf(mx, acc[i >> 2][i & 3]), acc[(i + 1) >> 2][(i + 1) & 3]);
      mx = fmaxf(mx, acc[KTW - 1][3]);
    } else {
      mx = pair_max(false, pmx, acc[KTW - 2], acc[KTW - 1]);
    }
    mx = group_max(mx);
    const float ma = mx * alpha;                 // row max in base-2 exponent units
    const float moff = MASK && mx == -INFINITY ? 0.f : -ma;
    // The wave's row sum runs on the matrix cores: the exponentials of two
    // tiles (8 per lane, all of row qlane) are rounded to fp16 and form the B
    // operand of a product with an all-ones A, so every lane receives the sum
    // over the 32 keys of the four lane groups, accumulated in fp32.
    f32x4v rs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < KTW; t += 2) {
      f16x8 h;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = fast_exp2(__builtin_fmaf(acc[t + u][r], alpha, moff));
          acc[t + u][r] = e;
          h[4 * u + r] = (_Float16)e;
        }
      rs = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, h, rs, 0, 0, 0);
    }
    const float sm = rs[0];
    if (lane < 16) red[buf][qlane][wave] = make_float2(ma, sm);
    // publish tile b+1 before the barrier that ends this block's reads
    q_stash(buf ^ 1, cur);
    __syncthreads();
    // lane group grp merges the pairs of waves 2 grp and 2 grp + 1; two lane
    // swaps then combine the four groups (every lane ends with the row's m, l)
    const float4 pp = *reinterpret_cast<const float4*>(&red[buf][qlane][2 * grp]);
    const float m = group_max(fmaxf(pp.x, pp.z));
    const float l = group_sum(pp.y * fast_exp2(pp.x - m) + pp.w * fast_exp2(pp.z - m));   // m_w = -inf -> 0
    // this wave's weight; rows past G*W contribute nothing
    const float own = MASK && mx == -INFINITY ? 0.f : fast_exp2(ma - m);
    wgt = (LIN || b * QB + qlane < g.GW) ? own * __builtin_amdgcn_rcpf(l) : 0.f;
  };
  uint2 stage2;
  // even blocks fetch into stage2 and publish stage1, odd blocks the reverse;
  // on entry to each pass of the loop `acc` holds the logits of block b
  logits(std::false_type{}, 0, stage2);
  int b = 0;
  for (; b + 2 < nblk; b += 2) {
    stats(b, stage1);
    logits(std::true_type{}, b + 1, stage1);
    stats(b + 1, stage2);
    logits(std::true_type{}, b + 2, stage2);
  }
  stats(b, stage1);
  if (b + 1 < nblk) {
    logits(std::true_type{}, b + 1, stage1);
    stats(b + 1, stage2);
  }
  // the last block's exponentials, which no further MFMAs overwrite
#pragma unroll
  for (int t = 0; t < KTW; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) colacc[t][r] = __builtin_fmaf(acc[t][r], wgt, colacc[t][r]);
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
        if (key < g.W) {
          out[key] = colacc[t][r];
          if (keys_lds) keys_lds[key] = order_key(colacc[t][r]);
        }
      }
    }
}

// Every wave of the workgroup takes the same branch: it depends on the
// geometry only.  MASK: the window is shorter than the 8 waves' 1024 keys.
__device__ __forceinline__ void fused_unit_any(const Geo& g, int unit, const __bf16* __restrict__ q,
                                               const bf16x8 (&kf)[KTW][4], int key0,
                                               unsigned char (*qtile)[QB * QLROW], float2 (*red)[QB][FW],
                                               float* __restrict__ scores, uint32_t* keys_lds) {
  const bool mask = g.W < FW * KTW * 16;
  const bool lin = QB % g.G == 0 && g.GW % QB == 0;
  if (mask) {
    if (lin) fused_unit<true, true>(g, unit, q, kf, key0, qtile, red, scores, keys_lds);
    else fused_unit<true, false>(g, unit, q, kf, key0, qtile, red, scores, keys_lds);
  } else {
    if (lin) fused_unit<false, true>(g, unit, q, kf, key0, qtile, red, scores, keys_lds);
    else fused_unit<false, false>(g, unit, q, kf, key0, qtile, red, scores, keys_lds);
  }
}

__global__ __launch_bounds__(FTHREADS, 1) void fused_score_kernel(Geo g, const __bf16* __restrict__ q,
                                                                   const __bf16* __restrict__ kc,
                                                                   const int32_t* __restrict__ tables,
                                                                   const int32_t* __restrict__ prior,
                                                                   float* __restrict__ scores) {
  __shared__ __align__(16) unsigned char qtile[2][QB * QLROW];
  __shared__ __align__(16) float2 red[2][QB][FW];
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
  fused_unit_any(g, unit, q, kf, key0, qtile, red, scores, nullptr);
}

hipError_t launch_fused_score(const Geo& g, const void* q, const void* kc, const int32_t* tables,
                              const int32_t* prior, float* scores, hipStream_t st) {
  const long long units = (long long)g.S * g.Lyr * g.Hkv;
  if (units > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(fused_score_kernel, dim3((unsigned)units), dim3(FTHREADS), 0, st, g, (const __bf16*)q,
                     (const __bf16*)kc, tables, prior, scores);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Single-launch pipeline: the workgroup that scores a unit also selects its
// kept positions (select_core.h, keys straight from the scores it just
// produced) and compacts the unit's K and V rows in place (compact_core.h).
// The block-table rewrite of a sequence must follow every read of that
// sequence's table, so each workgroup counts itself in done[n] once its
// compaction has read the table; the workgroup that brings the count to
// layers * kv_heads rewrites the table and resets the counter to zero.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(FTHREADS, 1) void pipeline_kernel(Geo g, const __bf16* __restrict__ q,
                                                                unsigned char* __restrict__ kc,
                                                                unsigned char* __restrict__ vc,
                                                                int32_t* __restrict__ tables,
                                                                const int32_t* __restrict__ prior,
                                                                float* __restrict__ scores, int32_t* __restrict__ kept,
                                                                uint8_t* __restrict__ mask,
                                                                int32_t* __restrict__ seq_lens,
                                                                int32_t* __restrict__ freed,
                                                                int32_t* __restrict__ num_freed, int max_freed,
                                                                int32_t* __restrict__ done) {
  __shared__ __align__(16) unsigned char qtile[2][QB * QLROW];
  __shared__ __align__(16) float2 red[2][QB][FW];
  __shared__ __align__(16) uint32_t keys[FW * KTW * 16];
  __shared__ __align__(16) int32_t kl[FW * KTW * 16];
  __shared__ uint8_t flags[FW * KTW * 16];
  __shared__ SelScratch<FTHREADS> sh;
  __shared__ int last;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int qlane = lane & 15, grp = lane >> 4;
  const int unit = blockIdx.x;
  const int kvh = unit % g.Hkv;
  const int layer = (unit / g.Hkv) % g.Lyr;
  const int n = unit / (g.Hkv * g.Lyr);
  const int L = prior[n];
  const int32_t* trow = tables + (long long)n * g.max_blocks;

  {
    const int key0 = wave * KTW * 16;
    const PagedRows pr = paged_rows(g, trow, layer, kvh, L, 2);
    bf16x8 kf[KTW][4];
#pragma unroll
    for (int t = 0; t < KTW; ++t) {
      const int j = min(key0 + 16 * t + qlane, g.W - 1);
      const uint4* src = reinterpret_cast<const uint4*>(kc + paged_row(pr, L + j) + grp * 64);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint4 v = src[s];
        __builtin_memcpy(&kf[t][s], &v, 16);
      }
    }
    fused_unit_any(g, unit, q, kf, key0, qtile, red, scores, keys);
  }
  select_unit<FTHREADS, FW * KTW * 16 / FTHREADS>(g, 0, keys, flags, sh, kl, kept + (long long)unit * g.B,
                        mask ? mask + (long long)unit * g.W : nullptr);
  __syncthreads();                                   // kl complete
  compact_unit_rows<FTHREADS, FD * 2, 8>(g, kc, vc, trow, layer, kvh, L, kl, 2);   // B <= 256 in one round
  __syncthreads();                                   // every table read of this workgroup is done
  if (tid == 0) {
    __threadfence();
    last = atomicAdd(&done[n], 1) == g.Lyr * g.Hkv - 1;
  }
  __syncthreads();
  if (last) {                                       // the whole workgroup rewrites the table
    __threadfence();
    finalize_sequence(g, n, tables, prior, seq_lens, freed, num_freed, max_freed, nullptr, tid, FTHREADS);
    if (tid == 0) done[n] = 0;
  }
}

hipError_t launch_pipeline(const Geo& g, const void* q, void* kc, void* vc, int32_t* tables, const int32_t* prior,
                           float* scores, int32_t* kept, uint8_t* mask, int32_t* seq_lens, int32_t* freed,
                           int32_t* num_freed, int max_freed, int32_t* done, hipStream_t st) {
  const long long units = (long long)g.S * g.Lyr * g.Hkv;
  if (units > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(pipeline_kernel, dim3((unsigned)units), dim3(FTHREADS), 0, st, g, (const __bf16*)q,
                     (unsigned char*)kc, (unsigned char*)vc, tables, prior, scores, kept, mask, seq_lens, freed,
                     num_freed, max_freed, done);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Allocation-free form of the single-launch pipeline.  Its per-sequence
// arrival counters live in `scratch`, a fixed array of this module on every
// GPU, instead of a caller buffer.  Host code never passes the array's name to
// a kernel: the device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and kept.  The counters are
// cleared by a fill kernel on the caller's stream before every pipeline
// launch, so a call never depends on what an earlier call left behind; calls
// that overlap on one GPU share the array and race.
// ---------------------------------------------------------------------------
static __device__ __align__(256) int32_t scratch[KARA_NOALLOC_MAX_SEQS];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch[kMaxDevices] = {};
}  // namespace

__global__ void zero_counters_kernel(int32_t* __restrict__ c, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) c[i] = 0;
}

// Device address of `scratch` on the current device (looked up on first use).
hipError_t noalloc_scratch(int32_t** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = static_cast<int32_t*>(p);
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

bool fused_score_supported(const Geo& g, int dtype);
bool small_score_supported(const Geo& g, int dtype);
hipError_t launch_small_pipeline(const Geo& g, int dtype, const void* q, void* kc, void* vc, int32_t* tables,
                                 const int32_t* prior, float* scores, int32_t* kept, uint8_t* mask,
                                 int32_t* seq_lens, int32_t* freed, int32_t* num_freed, int max_freed,
                                 int32_t* done, hipStream_t st);

// The one-launch step on whichever single-pass scorer covers the shape.
hipError_t launch_pipeline_any(const Geo& g, int dtype, const void* q, void* kc, void* vc, int32_t* tables,
                               const int32_t* prior, float* scores, int32_t* kept, uint8_t* mask, int32_t* seq_lens,
                               int32_t* freed, int32_t* num_freed, int max_freed, int32_t* done, hipStream_t st) {
  if (fused_score_supported(g, dtype))
    return launch_pipeline(g, q, kc, vc, tables, prior, scores, kept, mask, seq_lens, freed, num_freed, max_freed,
                           done, st);
  if (small_score_supported(g, dtype))
    return launch_small_pipeline(g, dtype, q, kc, vc, tables, prior, scores, kept, mask, seq_lens, freed, num_freed,
                                 max_freed, done, st);
  return hipErrorInvalidConfiguration;
}

bool pipeline_supported(const Geo& g, int dtype) {
  return fused_score_supported(g, dtype) || small_score_supported(g, dtype);
}

hipError_t launch_pipeline_noalloc(const Geo& g, int dtype, const void* q, void* kc, void* vc, int32_t* tables,
                                   const int32_t* prior, float* scores, int32_t* kept, uint8_t* mask,
                                   int32_t* seq_lens, int32_t* freed, int32_t* num_freed, int max_freed,
                                   hipStream_t st) {
  if (g.S > KARA_NOALLOC_MAX_SEQS) return hipErrorInvalidValue;
  int32_t* done = nullptr;
  hipError_t e = noalloc_scratch(&done);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(zero_counters_kernel, dim3((g.S + 255) / 256), dim3(256), 0, st, done, g.S);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_pipeline_any(g, dtype, q, kc, vc, tables, prior, scores, kept, mask, seq_lens, freed, num_freed,
                             max_freed, done, st);
}

bool fused_score_supported(const Geo& g, int dtype) {
  return dtype == KARA_BF16 && g.D == FD && g.W <= FW * KTW * 16;
}

}  // namespace kara
