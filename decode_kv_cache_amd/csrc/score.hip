// Window scoring: bidirectional in-window attention column mass.
//
// Kara ("Kara: Efficient Reasoning LLM Serving via Sliding-Window KV Cache
// Compression", English abstract) scores the window's KV pairs with
// bidirectional attention.  Recorded reading: for unit (n, l, g)
//     c[j] = sum_{h in group g} sum_{i < W} exp(x[h,i,j] - beta[h,i]),
//     x = (q . k) * log2(e) / sqrt(d),   beta[h,i] = log2 sum_j 2^x[h,i,j]
// i.e. the softmax over the W window keys (no causal mask) summed down each
// key column.  Two passes over the logits:
//   pass 1 (row_lse)  : per query row, running max and sum of 2^(x - max)
//                       over key tiles -> beta (base-2 log-sum-exp);
//   pass 2 (col_mass) : per key column, sum over all G*W query rows of
//                       2^(x - beta), accumulated in fp32 registers.
// Both passes recompute the logits with 32x32 MFMA tiles (bf16 inputs with
// fp32 accumulation, or fp32 inputs on the fp32 MFMA).
#include "kara_device.h"

namespace kara {

// ---------------------------------------------------------------------------
// Pass 1.  S^T tiles: A = 32 window keys, B = 32 query rows (resident), so a
// lane owns one query row and 16 keys of every tile; the row statistics stay
// lane-local until the final merge of the two lane halves.
// Grid: units * ceil(GW / 128) blocks of 256 threads (4 waves x 32 rows).
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void row_lse_kernel(Geo g, const T* __restrict__ q,
                                                      const T* __restrict__ kc,
                                                      const int32_t* __restrict__ tables,
                                                      const int32_t* __restrict__ prior,
                                                      float* __restrict__ beta_ws) {
  using M = Mma<T>;
  constexpr int NF = Frags<T, D>::N;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int rowblocks = (g.GW + 127) >> 7;
  const int unit = blockIdx.x / rowblocks;
  const int rb = blockIdx.x - unit * rowblocks;
  const int row0 = rb * 128 + wave * 32;
  if (row0 >= g.GWp) return;
  const int kvh = unit % g.Hkv;
  const int layer = (unit / g.Hkv) % g.Lyr;
  const int n = unit / (g.Hkv * g.Lyr);
  const int L = prior[n];
  const int32_t* trow = tables + (long long)n * g.max_blocks;

  // query row of this lane (B operand column)
  const int row = row0 + col;
  const bool row_ok = row < g.GW;
  const int rq = row_ok ? row : 0;
  const int qi = rq / g.G, qh = rq - qi * g.G;
  const T* qp = q + ((((long long)n * g.Lyr + layer) * g.W + qi) * g.Hq + kvh * g.G + qh) * D + half * (D / 2);
  typename M::frag bq[NF];
  load_half_row<T, D>(qp, row_ok, bq);

  float m = -INFINITY, l = 0.f;
  const int ktiles = (g.W + 31) >> 5;
  for (int kt = 0; kt < ktiles; ++kt) {
    const int j = kt * 32 + col;           // key row this lane loads for the A operand
    long long off = j < g.W ? slot_offset(g, trow, layer, kvh, L + j) : -1;
    typename M::frag ak[NF];
    load_half_row<T, D>(kc + (off < 0 ? 0 : off) + half * (D / 2), off >= 0, ak);
    f32x16 acc = {};
#pragma unroll
    for (int f = 0; f < NF; ++f) acc = M::mma(ak[f], bq[f], acc);
    // acc[r]: key kt*32 + 8*(r/4) + 4*half + (r%4) against this lane's query row
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (key >= g.W) acc[r] = -INFINITY;
      tmax = fmaxf(tmax, acc[r]);
    }
    if (tmax == -INFINITY) continue;
    const float mnew = fmaxf(m, tmax * g.alpha);
    l *= fast_exp2(m - mnew);               // m = -inf -> 0
#pragma unroll
    for (int r = 0; r < 16; ++r) l += fast_exp2(__builtin_fmaf(acc[r], g.alpha, -mnew));
    m = mnew;
  }
  // merge with the other lane half (same query row, the other 16 keys of each tile)
  const float mo = __shfl_xor(m, 32);
  const float lo = __shfl_xor(l, 32);
  const float mt = fmaxf(m, mo);
  const float lt = (m == -INFINITY ? 0.f : l * fast_exp2(m - mt)) + (mo == -INFINITY ? 0.f : lo * fast_exp2(mo - mt));
  if (half == 0) beta_ws[(long long)unit * g.GWp + row] = row_ok ? mt + fast_log2(lt) : INFINITY;
}

// ---------------------------------------------------------------------------
// Pass 2.  S tiles: A = 32 query rows (streamed), B = 32 window keys
// (resident), so a lane owns one key column and 16 query rows of every tile;
// the column sum stays in one register per lane.
// Grid: units * ceil(W / 128) blocks of 256 threads (4 waves x 32 keys).
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void col_mass_kernel(Geo g, const T* __restrict__ q,
                                                       const T* __restrict__ kc,
                                                       const int32_t* __restrict__ tables,
                                                       const int32_t* __restrict__ prior,
                                                       const float* __restrict__ beta_ws,
                                                       float* __restrict__ scores) {
  using M = Mma<T>;
  constexpr int NF = Frags<T, D>::N;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int keyblocks = (g.W + 127) >> 7;
  const int unit = blockIdx.x / keyblocks;
  const int kb = blockIdx.x - unit * keyblocks;
  const int key0 = kb * 128 + wave * 32;
  if (key0 >= g.W) return;
  const int kvh = unit % g.Hkv;
  const int layer = (unit / g.Hkv) % g.Lyr;
  const int n = unit / (g.Hkv * g.Lyr);
  const int L = prior[n];
  const int32_t* trow = tables + (long long)n * g.max_blocks;

  const int j = key0 + col;
  long long off = j < g.W ? slot_offset(g, trow, layer, kvh, L + j) : -1;
  typename M::frag bk[NF];
  load_half_row<T, D>(kc + (off < 0 ? 0 : off) + half * (D / 2), off >= 0, bk);

  const float* bw = beta_ws + (long long)unit * g.GWp;
  const T* qbase = q + (((long long)n * g.Lyr + layer) * g.W) * g.Hq * D + (long long)kvh * g.G * D + half * (D / 2);
  float csum = 0.f;
  const int rtiles = g.GWp >> 5;
  for (int rt = 0; rt < rtiles; ++rt) {
    const int row = rt * 32 + col;
    const bool row_ok = row < g.GW;
    const int rq = row_ok ? row : 0;
    const int qi = rq / g.G, qh = rq - qi * g.G;
    typename M::frag aq[NF];
    load_half_row<T, D>(qbase + ((long long)qi * g.Hq + qh) * D, row_ok, aq);
    f32x16 acc = {};
#pragma unroll
    for (int f = 0; f < NF; ++f) acc = M::mma(aq[f], bk[f], acc);
    // acc[r]: query row rt*32 + 8*(r/4) + 4*half + (r%4) against this lane's key
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x4 b4 = *reinterpret_cast<const f32x4*>(bw + rt * 32 + 8 * r4 + 4 * half);
#pragma unroll
      for (int e = 0; e < 4; ++e) csum += fast_exp2(__builtin_fmaf(acc[4 * r4 + e], g.alpha, -b4[e]));
    }
  }
  csum += __shfl_xor(csum, 32);
  if (half == 0 && j < g.W) scores[(long long)unit * g.W + j] = csum;
}

// ---------------------------------------------------------------------------
template <typename T, int D>
static hipError_t launch_score_t(const Geo& g, const void* q, const void* kc, const int32_t* tables,
                                 const int32_t* prior, float* scores, float* ws, hipStream_t st) {
  const long long units = (long long)g.S * g.Lyr * g.Hkv;
  const long long b1 = units * ((g.GW + 127) / 128);
  const long long b2 = units * ((g.W + 127) / 128);
  if (b1 > 0x7fffffffLL || b2 > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((row_lse_kernel<T, D>), dim3((unsigned)b1), dim3(256), 0, st, g, (const T*)q,
                     (const T*)kc, tables, prior, ws);
  hipLaunchKernelGGL((col_mass_kernel<T, D>), dim3((unsigned)b2), dim3(256), 0, st, g, (const T*)q,
                     (const T*)kc, tables, prior, (const float*)ws, scores);
  return hipGetLastError();
}

hipError_t launch_score(const Geo& g, int dtype, const void* q, const void* kc, const int32_t* tables,
                        const int32_t* prior, float* scores, float* ws, hipStream_t st) {
  if (dtype == KARA_BF16) {
    if (g.D == 128) return launch_score_t<__bf16, 128>(g, q, kc, tables, prior, scores, ws, st);
    return launch_score_t<__bf16, 64>(g, q, kc, tables, prior, scores, ws, st);
  }
  if (g.D == 128) return launch_score_t<float, 128>(g, q, kc, tables, prior, scores, ws, st);
  return launch_score_t<float, 64>(g, q, kc, tables, prior, scores, ws, st);
}

size_t score_workspace_bytes(const Geo& g) {
  return (size_t)g.S * g.Lyr * g.Hkv * (size_t)g.GWp * sizeof(float);
}

}  // namespace kara
