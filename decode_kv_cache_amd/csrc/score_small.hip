// Single-pass window scoring for small windows, any element type and
// head_dim, and the one-launch pipeline built on it.
//
// Same quantity as the other scorers (Kara's bidirectional in-window
// attention column mass, English abstract of "Kara: Efficient Reasoning LLM
// Serving via Sliding-Window KV Cache Compression"):
//     c[j] = sum_{h in group g} sum_{i < W} softmax_j'(q[h,i] . k[j'] / sqrt(d))[j].
//
// For windows of at most 256 keys whose K rows fit in 72 KiB of LDS (128
// keys for fp32 rows of head_dim 128), in the shapes the resident-key scorer
// in score_fused.hip does not take: fp32, or head_dim 64.  One workgroup of
// 4 waves owns one unit and stages the window's K rows in LDS once.  Each
// wave takes every fourth block of 16 query rows and computes the block's
// logits against all W keys with 16x16 MFMAs (16x16x32 bf16, 16x16x4 fp32)
// in the transposed orientation S^T = K Q^T (a lane owns one query row and 4
// keys of every 16-key tile), so each row's max and sum are complete in the
// wave: no exchange between waves and no barrier inside the loop.  The
// softmax weights are fp32 exponentials over the row's fp32 sum (no fp16
// rounding anywhere); the column sums accumulate per lane, are reduced over
// the 16 query lanes and then over the 4 waves in a fixed order.  Each logit
// is computed once.
#include "compact_core.h"
#include "kara_device.h"
#include "select_core.h"

namespace kara {

typedef float f32x4s __attribute__((ext_vector_type(4)));

constexpr int SW = 4;                    // waves per workgroup
constexpr int STHREADS = SW * 64;
constexpr int SMAXW = 256;               // keys of the largest window
constexpr int SMAXT = SMAXW / 16;        // 16-key tiles
constexpr int SK_BYTES = 72 * 1024;      // LDS for the window's K rows (padded)

// 16x16 MFMA on 16-byte operand chunks.  Lane l feeds row (or column) l % 16
// and, for the reduction, the elements of the 16-byte chunk its lane group
// l / 16 holds; a chunk is one bf16 step (8 elements) or four fp32 steps (one
// element each).  Both operands use the same chunk order, so the products
// pair up whatever the order of the reduction.
template <typename T>
struct Chunk16;

template <>
struct Chunk16<__bf16> {
  __device__ static inline f32x4s mma(const uint4& a, const uint4& b, f32x4s c) {
    bf16x8 x, y;
    __builtin_memcpy(&x, &a, 16);
    __builtin_memcpy(&y, &b, 16);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, c, 0, 0, 0);
  }
};

template <>
struct Chunk16<float> {
  __device__ static inline f32x4s mma(const uint4& a, const uint4& b, f32x4s c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  }
};

__device__ __forceinline__ float small_group_max(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float small_group_sum(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

struct SmallLds {
  unsigned char k[SK_BYTES];             // window K rows, `pitch` bytes apart
  float part[SW][SMAXW];                 // per-wave column sums
};

// Row pitch of the staged K rows: 16 padding bytes keep the 16 rows a
// half-wave reads at one column offset in distinct banks.
template <typename T, int D>
struct SmallGeo {
  static constexpr int ROWB = D * (int)sizeof(T);
  static constexpr int PITCH = ROWB + 16;
  static constexpr int CH = ROWB / 16;   // 16-byte chunks per row
  static constexpr int KC = CH / 4;      // chunks per lane group
  // the launch rounds the tiles up to 4, 8 or 16 and stages that many rows
  static constexpr int MAXW = 256 * PITCH <= SK_BYTES ? 256 : 128 * PITCH <= SK_BYTES ? 128 : 64;
};

// Scores of one unit into scores[unit][0..W) and, if keys_lds is set, the
// order keys of select_core.h into keys_lds[0..W).  T = number of 16-key
// tiles the window needs.
template <typename T, int D, int NT>
__device__ void small_unit(const Geo& g, int unit, const T* __restrict__ q, const unsigned char* __restrict__ kc,
                           const int32_t* __restrict__ trow, int L, float* __restrict__ scores, uint32_t* keys_lds,
                           SmallLds& sh) {
  using SG = SmallGeo<T, D>;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int qlane = lane & 15, grp = lane >> 4;
  const int kvh = unit % g.Hkv;
  const int layer = (unit / g.Hkv) % g.Lyr;
  const int n = unit / (g.Hkv * g.Lyr);

  // stage the window's K rows, NT * 16 <= MAXW of them (keys past W are zero
  // rows and are masked)
  static_assert(NT * 16 <= SG::MAXW && SG::MAXW * SG::PITCH <= SK_BYTES, "staged rows fit in LDS");
  const PagedRows pr = paged_rows(g, trow, layer, kvh, L, (int)sizeof(T));
  for (int c = tid; c < NT * 16 * SG::CH; c += STHREADS) {
    const int j = c / SG::CH, ch = c - j * SG::CH;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (j < g.W) v = *reinterpret_cast<const uint4*>(kc + paged_row(pr, L + j) + ch * 16);
    *reinterpret_cast<uint4*>(&sh.k[j * SG::PITCH + ch * 16]) = v;
  }
  __syncthreads();

  const unsigned char* qbytes = reinterpret_cast<const unsigned char*>(
      q + (((long long)n * g.Lyr + layer) * g.W) * g.Hq * D + (long long)kvh * g.G * D);
  const float alpha = g.alpha;
  f32x4s colacc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) colacc[t] = f32x4s{0.f, 0.f, 0.f, 0.f};
  const int nblk = (g.GW + 15) / 16;
  for (int b = wave; b < nblk; b += SW) {
    // B operand: this lane's query row, its lane group's chunks
    const int row = b * 16 + qlane;
    const int rq = min(row, g.GW - 1);
    const int qi = rq / g.G, qh = rq - qi * g.G;
    const uint4* qp = reinterpret_cast<const uint4*>(qbytes + ((long long)qi * g.Hq + qh) * SG::ROWB);
    uint4 qc[SG::KC];
#pragma unroll
    for (int k = 0; k < SG::KC; ++k) qc[k] = qp[k * 4 + grp];
    f32x4s acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      acc[t] = f32x4s{0.f, 0.f, 0.f, 0.f};
      const unsigned char* krow = &sh.k[(16 * t + qlane) * SG::PITCH];
#pragma unroll
      for (int k = 0; k < SG::KC; ++k)
        acc[t] = Chunk16<T>::mma(*reinterpret_cast<const uint4*>(krow + (k * 4 + grp) * 16), qc[k], acc[t]);
    }
    // acc[t][r]: key 16 t + 4 grp + r against query row `row`; keys past W take no part
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (16 * t + 4 * grp + r >= g.W) acc[t][r] = -INFINITY;
        mx = fmaxf(mx, acc[t][r]);
      }
    mx = small_group_max(mx);          // finite: every row has at least one key
    const float moff = -mx * alpha;
    float sum = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        acc[t][r] = fast_exp2(__builtin_fmaf(acc[t][r], alpha, moff));
        sum += acc[t][r];
      }
    sum = small_group_sum(sum);
    const float w = row < g.GW ? __builtin_amdgcn_rcpf(sum) : 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) colacc[t][r] = __builtin_fmaf(acc[t][r], w, colacc[t][r]);
  }
  // column sums: over the 16 query lanes of each lane group, then over the waves
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v = colacc[t][r];
      v += __shfl_xor(v, 1);
      v += __shfl_xor(v, 2);
      v += __shfl_xor(v, 4);
      v += __shfl_xor(v, 8);
      colacc[t][r] = v;
    }
#pragma unroll
  for (int t = 0; t < NT; ++t)
    if (qlane == t) {
#pragma unroll
      for (int r = 0; r < 4; ++r) sh.part[wave][16 * t + 4 * grp + r] = colacc[t][r];
    }
  __syncthreads();
  float* out = scores + (long long)unit * g.W;
  for (int j = tid; j < g.W; j += STHREADS) {
    const float c = (sh.part[0][j] + sh.part[1][j]) + (sh.part[2][j] + sh.part[3][j]);
    out[j] = c;
    if (keys_lds) keys_lds[j] = order_key(c);
  }
}

template <typename T, int D, int NT>
__global__ __launch_bounds__(STHREADS) void small_score_kernel(Geo g, const T* __restrict__ q,
                                                               const unsigned char* __restrict__ kc,
                                                               const int32_t* __restrict__ tables,
                                                               const int32_t* __restrict__ prior,
                                                               float* __restrict__ scores) {
  __shared__ __align__(16) SmallLds sh;
  const int unit = blockIdx.x;
  const int n = unit / (g.Hkv * g.Lyr);
  small_unit<T, D, NT>(g, unit, q, kc, tables + (long long)n * g.max_blocks, prior[n], scores, nullptr, sh);
}

// One launch for the whole step (see the pipeline in score_fused.hip): the
// workgroup scores its unit, selects from its own scores, compacts its rows,
// and the last workgroup of a sequence rewrites the table.
template <typename T, int D, int NT>
__global__ __launch_bounds__(STHREADS) void small_pipeline_kernel(Geo g, const T* __restrict__ q,
                                                                  unsigned char* __restrict__ kc,
                                                                  unsigned char* __restrict__ vc,
                                                                  int32_t* __restrict__ tables,
                                                                  const int32_t* __restrict__ prior,
                                                                  float* __restrict__ scores,
                                                                  int32_t* __restrict__ kept,
                                                                  uint8_t* __restrict__ mask,
                                                                  int32_t* __restrict__ seq_lens,
                                                                  int32_t* __restrict__ freed,
                                                                  int32_t* __restrict__ num_freed, int max_freed,
                                                                  int32_t* __restrict__ done) {
  __shared__ __align__(16) SmallLds sh;
  __shared__ __align__(16) uint32_t keys[SMAXW];
  __shared__ __align__(16) int32_t kl[SMAXW];
  __shared__ uint8_t flags[SMAXW];
  __shared__ SelScratch<STHREADS> sc;
  __shared__ int last;
  const int tid = threadIdx.x;
  const int unit = blockIdx.x;
  const int kvh = unit % g.Hkv;
  const int layer = (unit / g.Hkv) % g.Lyr;
  const int n = unit / (g.Hkv * g.Lyr);
  const int L = prior[n];
  const int32_t* trow = tables + (long long)n * g.max_blocks;
  small_unit<T, D, NT>(g, unit, q, kc, trow, L, scores, keys, sh);
  __syncthreads();                                   // every order key is in LDS
  select_unit<STHREADS, 1>(g, 0, keys, flags, sc, kl, kept + (long long)unit * g.B,
                           mask ? mask + (long long)unit * g.W : nullptr);
  __syncthreads();                                   // kl complete
  compact_unit_rows<STHREADS, D * (int)sizeof(T), 4>(g, kc, vc, trow, layer, kvh, L, kl, (int)sizeof(T));
  __syncthreads();                                   // every table read of this workgroup is done
  if (tid == 0) {
    __threadfence();
    last = atomicAdd(&done[n], 1) == g.Lyr * g.Hkv - 1;
  }
  __syncthreads();
  if (last) {                                       // the whole workgroup rewrites the table
    __threadfence();
    finalize_sequence(g, n, tables, prior, seq_lens, freed, num_freed, max_freed, nullptr, tid, STHREADS);
    if (tid == 0) done[n] = 0;
  }
}

template <typename T, int D>
static bool small_fits(const Geo& g) {
  return g.W <= SmallGeo<T, D>::MAXW;
}

bool fused_score_supported(const Geo& g, int dtype);

bool small_score_supported(const Geo& g, int dtype) {
  if (fused_score_supported(g, dtype)) return false;
  if (dtype == KARA_BF16) return g.D == 64 && small_fits<__bf16, 64>(g);
  return g.D == 64 ? small_fits<float, 64>(g) : small_fits<float, 128>(g);
}

// Tiles: the smallest of 4, 8, 16 that covers the window (16 only where 256
// staged rows fit).  bf16 rows of head_dim 128 always take the resident-key
// scorer, so they have no instance here.
template <typename T, int D, int NT>
static void small_score_t(const Geo& g, long long units, const void* q, const void* kc, const int32_t* tables,
                          const int32_t* prior, float* scores, hipStream_t st) {
  hipLaunchKernelGGL((small_score_kernel<T, D, NT>), dim3((unsigned)units), dim3(STHREADS), 0, st, g, (const T*)q,
                     (const unsigned char*)kc, tables, prior, scores);
}

template <typename T, int D>
static void small_score_tiles(const Geo& g, long long units, const void* q, const void* kc, const int32_t* tables,
                              const int32_t* prior, float* scores, hipStream_t st) {
  const int tiles = (g.W + 15) / 16;
  if (tiles <= 4) small_score_t<T, D, 4>(g, units, q, kc, tables, prior, scores, st);
  else if (tiles <= 8) small_score_t<T, D, 8>(g, units, q, kc, tables, prior, scores, st);
  else if constexpr (SmallGeo<T, D>::MAXW >= 256) small_score_t<T, D, 16>(g, units, q, kc, tables, prior, scores, st);
}

template <typename T, int D, int NT>
static void small_pipe_t(const Geo& g, long long units, const void* q, void* kc, void* vc, int32_t* tables,
                         const int32_t* prior, float* scores, int32_t* kept, uint8_t* mask, int32_t* seq_lens,
                         int32_t* freed, int32_t* num_freed, int max_freed, int32_t* done, hipStream_t st) {
  hipLaunchKernelGGL((small_pipeline_kernel<T, D, NT>), dim3((unsigned)units), dim3(STHREADS), 0, st, g, (const T*)q,
                     (unsigned char*)kc, (unsigned char*)vc, tables, prior, scores, kept, mask, seq_lens, freed,
                     num_freed, max_freed, done);
}

template <typename T, int D>
static void small_pipe_tiles(const Geo& g, long long units, const void* q, void* kc, void* vc, int32_t* tables,
                             const int32_t* prior, float* scores, int32_t* kept, uint8_t* mask, int32_t* seq_lens,
                             int32_t* freed, int32_t* num_freed, int max_freed, int32_t* done, hipStream_t st) {
  const int tiles = (g.W + 15) / 16;
  if (tiles <= 4)
    small_pipe_t<T, D, 4>(g, units, q, kc, vc, tables, prior, scores, kept, mask, seq_lens, freed, num_freed,
                          max_freed, done, st);
  else if (tiles <= 8)
    small_pipe_t<T, D, 8>(g, units, q, kc, vc, tables, prior, scores, kept, mask, seq_lens, freed, num_freed,
                          max_freed, done, st);
  else if constexpr (SmallGeo<T, D>::MAXW >= 256)
    small_pipe_t<T, D, 16>(g, units, q, kc, vc, tables, prior, scores, kept, mask, seq_lens, freed, num_freed,
                           max_freed, done, st);
}

hipError_t launch_small_score(const Geo& g, int dtype, const void* q, const void* kc, const int32_t* tables,
                              const int32_t* prior, float* scores, hipStream_t st) {
  const long long units = (long long)g.S * g.Lyr * g.Hkv;
  if (units > 0x7fffffffLL || !small_score_supported(g, dtype)) return hipErrorInvalidConfiguration;
  if (dtype == KARA_BF16) small_score_tiles<__bf16, 64>(g, units, q, kc, tables, prior, scores, st);
  else if (g.D == 64) small_score_tiles<float, 64>(g, units, q, kc, tables, prior, scores, st);
  else small_score_tiles<float, 128>(g, units, q, kc, tables, prior, scores, st);
  return hipGetLastError();
}

hipError_t launch_small_pipeline(const Geo& g, int dtype, const void* q, void* kc, void* vc, int32_t* tables,
                                 const int32_t* prior, float* scores, int32_t* kept, uint8_t* mask,
                                 int32_t* seq_lens, int32_t* freed, int32_t* num_freed, int max_freed,
                                 int32_t* done, hipStream_t st) {
  const long long units = (long long)g.S * g.Lyr * g.Hkv;
  if (units > 0x7fffffffLL || !small_score_supported(g, dtype)) return hipErrorInvalidConfiguration;
  if (dtype == KARA_BF16)
    small_pipe_tiles<__bf16, 64>(g, units, q, kc, vc, tables, prior, scores, kept, mask, seq_lens, freed, num_freed,
                                 max_freed, done, st);
  else if (g.D == 64)
    small_pipe_tiles<float, 64>(g, units, q, kc, vc, tables, prior, scores, kept, mask, seq_lens, freed, num_freed,
                                max_freed, done, st);
  else
    small_pipe_tiles<float, 128>(g, units, q, kc, vc, tables, prior, scores, kept, mask, seq_lens, freed, num_freed,
                                 max_freed, done, st);
  return hipGetLastError();
}

}  // namespace kara
