// Window scoring: bidirectional in-window attention column mass.
//
// Kara ("Kara: Efficient Reasoning LLM Serving via Sliding-Window KV Cache
// Compression", English abstract) scores the window's KV pairs with
// bidirectional attention.  Recorded reading: for unit (n, l, g)
//     c[j] = sum_{h in group g} sum_{i < W} 2^(x[h,i,j] - beta[h,i]),
//     x = (q . k) * log2(e) / sqrt(d),   beta[h,i] = log2 sum_j 2^x[h,i,j]
// i.e. the softmax over the W window keys (no causal mask) summed down each
// key column.  Two passes over the logits:
//   pass 1 (row_lse)  : per query row, running max and sum of 2^(x - max)
//                       over key tiles -> beta (base-2 log-sum-exp);
//   pass 2 (col_mass) : per key column, sum over all G*W query rows of
//                       2^(x - beta), accumulated in fp32 registers.
// Both passes recompute the logits on 32x32 MFMA tiles (bf16 inputs with
// fp32 accumulation, or fp32 inputs on the fp32 MFMA).  The operand that is
// streamed (K tiles in pass 1, Q tiles in pass 2) is staged once per
// workgroup in LDS (double-buffered, rows padded by 16 bytes so the 32 rows
// a half-wave reads hit distinct banks); the other operand stays in
// registers.  Blocks are mapped so that all blocks of one unit run on the
// same XCD and share its L2.
#include "kara_device.h"

namespace kara {

constexpr int TILE = 32;       // MFMA tile edge (keys per K tile, rows per Q tile)
constexpr int WAVES = 4;
constexpr int PER_WAVE = 64;   // query rows (pass 1) or keys (pass 2) per wave: two operand sets
constexpr int PER_BLOCK = WAVES * PER_WAVE;

// Block index -> (unit, sub-block).  The hardware hands consecutive block
// indices to the 8 XCDs in turn; giving XCD x the contiguous flat range
// [x * n8, (x+1) * n8) keeps the sub-blocks of a unit on one XCD.
__device__ inline bool xcd_map(int nflat, int per_unit, int& unit, int& sub) {
  const int n8 = (nflat + 7) >> 3;
  const int f = (blockIdx.x & 7) * n8 + (blockIdx.x >> 3);
  if (f >= nflat) return false;
  unit = f / per_unit;
  sub = f - unit * per_unit;
  return true;
}

static inline unsigned padded_grid(long long nflat) { return (unsigned)(((nflat + 7) >> 3) << 3); }

// Tile staging: 32 rows of ROWB bytes, chunks of 16 bytes, CPT chunks per thread.
template <typename T, int D>
struct Stage {
  static constexpr int ROWB = D * (int)sizeof(T);
  static constexpr int LROW = ROWB + 16;
  static constexpr int CPR = ROWB / 16;                 // chunks per row
  static constexpr int CPT = TILE * CPR / (WAVES * 64); // chunks per thread
  static constexpr int BYTES = TILE * LROW;
};

// Read the lane's half row (row `r`, half `h`) of a staged tile as fragments.
template <typename T, int D>
__device__ inline void lds_half_row(const unsigned char* tile, int r, int h,
                                    typename Mma<T>::frag (&f)[Frags<T, D>::N]) {
  constexpr int VEC = Frags<T, D>::VEC;
  const uint4* p = reinterpret_cast<const uint4*>(tile + r * Stage<T, D>::LROW + h * (Stage<T, D>::ROWB / 2));
  uint4 v[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) v[i] = p[i];
  __builtin_memcpy(&f, &v, sizeof(v));
}

// ---------------------------------------------------------------------------
// Pass 1.  S^T tiles: A = 32 window keys (LDS), B = query rows (registers),
// so a lane owns one query row of each of its two query tiles and 16 keys of
// every key tile; the row statistics stay lane-local until the final merge of
// the two lane halves.  Grid: units * ceil(GW / 256) blocks (XCD-mapped).
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void row_lse_kernel(Geo g, const T* __restrict__ q,
                                                      const T* __restrict__ kc,
                                                      const int32_t* __restrict__ tables,
                                                      const int32_t* __restrict__ prior,
                                                      float* __restrict__ beta_ws) {
  using M = Mma<T>;
  using St = Stage<T, D>;
  constexpr int NF = Frags<T, D>::N;
  __shared__ __align__(16) unsigned char lds[2][St::BYTES];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int per_unit = (g.GW + PER_BLOCK - 1) / PER_BLOCK;
  int unit, rb;
  if (!xcd_map(g.S * g.Lyr * g.Hkv * per_unit, per_unit, unit, rb)) return;
  const int kvh = unit % g.Hkv;
  const int layer = (unit / g.Hkv) % g.Lyr;
  const int n = unit / (g.Hkv * g.Lyr);
  const int L = prior[n];
  const int32_t* trow = tables + (long long)n * g.max_blocks;

  // the wave's two query tiles (B operands)
  const int row0 = rb * PER_BLOCK + wave * PER_WAVE;
  typename M::frag bq[2][NF];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int row = row0 + s * TILE + col;
    const bool ok = row < g.GW;
    const int rq = ok ? row : 0;
    const int qi = rq / g.G, qh = rq - qi * g.G;
    const T* qp = q + ((((long long)n * g.Lyr + layer) * g.W + qi) * g.Hq + kvh * g.G + qh) * D + half * (D / 2);
    load_half_row<T, D>(qp, ok, bq[s]);
  }

  // staging of K tile kt: this thread's chunks (keys clamped into the window)
  const unsigned char* kbytes = reinterpret_cast<const unsigned char*>(kc);
  const PagedRows pr = paged_rows(g, trow, layer, kvh, L, (int)sizeof(T));
  // chunk c of this thread: row (c*256 + tid) / CPR of the tile, 16-byte column (c*256 + tid) % CPR
#define KARA_K_FETCH(kt, v)                                                                         \
  _Pragma("unroll") for (int c = 0; c < St::CPT; ++c) {                                             \
    const int j = min((kt) * TILE + (c * 256 + tid) / St::CPR, g.W - 1);                            \
    (v)[c] = *reinterpret_cast<const uint4*>(kbytes + paged_row(pr, L + j) +                        \
                                             ((c * 256 + tid) % St::CPR) * 16);                     \
  }
#define KARA_K_STASH(buf, v)                                                                        \
  _Pragma("unroll") for (int c = 0; c < St::CPT; ++c)                                               \
    *reinterpret_cast<uint4*>(&lds[buf][((c * 256 + tid) / St::CPR) * St::LROW +                    \
                                        ((c * 256 + tid) % St::CPR) * 16]) = (v)[c];

  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
  // fold one tile of logits into the running row statistics; keys past the
  // window are masked only in the last, partial tile
  auto absorb = [&](f32x16 (&acc)[2], int kt, bool partial) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (partial) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kt * TILE + 8 * (r >> 2) + 4 * half + (r & 3) >= g.W) acc[s][r] = -INFINITY;
      }
      // a chain of three-input maxima: two new logits per instruction
      float tmax = fmaxf(fmaxf(acc[s][0], acc[s][1]), acc[s][2]);
#pragma unroll
      for (int r = 3; r + 1 < 16; r += 2) tmax = fmaxf(fmaxf(tmax, acc[s][r]), acc[s][r + 1]);
      tmax = fmaxf(tmax, acc[s][15]);
      const float mnew = fmaxf(m[s], tmax * g.alpha);
      float sum = fast_exp2(__builtin_fmaf(acc[s][0], g.alpha, -mnew));
#pragma unroll
      for (int r = 1; r < 16; ++r) sum += fast_exp2(__builtin_fmaf(acc[s][r], g.alpha, -mnew));
      if (!partial || mnew != -INFINITY) {
        l[s] = l[s] * fast_exp2(m[s] - mnew) + sum;   // m = -inf -> factor 0
        m[s] = mnew;
      }
    }
  };
  const int ktiles = (g.W + TILE - 1) / TILE;
  const int full = g.W / TILE;
  uint4 pre[St::CPT];
  KARA_K_FETCH(0, pre)
  KARA_K_STASH(0, pre)
  __syncthreads();
  auto tile_logits = [&](int buf, f32x16 (&acc)[2]) {
    typename M::frag ak[NF];
    lds_half_row<T, D>(lds[buf], col, half, ak);
    acc[0] = f32x16{};
    acc[1] = f32x16{};
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      acc[0] = M::mma(ak[f], bq[0][f], acc[0]);
      acc[1] = M::mma(ak[f], bq[1][f], acc[1]);
    }
    // acc[s][r]: key kt*32 + 8*(r/4) + 4*half + (r%4) against query row row0 + 32 s + col
  };
  for (int kt = 0; kt < full; ++kt) {
    const int buf = kt & 1;
    KARA_K_FETCH(kt + 1, pre)                   // clamped: always in the window
    f32x16 acc[2];
    tile_logits(buf, acc);
    absorb(acc, kt, false);
    KARA_K_STASH(buf ^ 1, pre)                  // that buffer was last read before the previous barrier
    __syncthreads();
  }
#undef KARA_K_FETCH
#undef KARA_K_STASH
  if (full < ktiles) {                          // the partial last tile is staged in lds[full & 1]
    f32x16 acc[2];
    tile_logits(full & 1, acc);
    absorb(acc, full, true);
  }
  // merge with the other lane half (same query row, the other 16 keys of each tile)
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const float mo = __shfl_xor(m[s], 32);
    const float lo = __shfl_xor(l[s], 32);
    const float mt = fmaxf(m[s], mo);
    const float lt = (m[s] == -INFINITY ? 0.f : l[s] * fast_exp2(m[s] - mt)) +
                     (mo == -INFINITY ? 0.f : lo * fast_exp2(mo - mt));
    const int row = row0 + s * TILE + col;
    if (half == 0 && row < g.GWp)
      beta_ws[(long long)unit * g.GWp + row] = row < g.GW ? mt + fast_log2(lt) : INFINITY;
  }
}

// Per-thread streaming state of pass 2.  Chunk c of this thread is row
// crow[c] of a 32-row Q tile, 16-byte column cch[c].  Row rho of a unit is
// (window position rho / G, head rho % G); its byte offset advances by a
// fixed step per tile plus a correction when the head index wraps.  Rows past
// G*W are read from the last row (their beta is +inf, so they add zero).
template <typename T, int D>
struct QStream {
  using St = Stage<T, D>;
  int crow[St::CPT], cch[St::CPT], rho[St::CPT], qh[St::CPT];
  unsigned long long addr[St::CPT];
  uint4 pre[St::CPT];
  float pb;
  unsigned long long step0, carry_step, last_addr;
  int h0, G, last_row;
  __device__ __forceinline__ void init(int tid, const Geo& g) {
    constexpr unsigned long long RB = (unsigned long long)D * sizeof(T);
    const unsigned long long pos_bytes = (unsigned long long)g.Hq * RB;
    G = g.G;
    h0 = TILE % g.G;
    step0 = (unsigned long long)(TILE / g.G) * pos_bytes + (unsigned long long)h0 * RB;
    carry_step = pos_bytes - (unsigned long long)g.G * RB;
    last_row = g.GW - 1;
    last_addr = (unsigned long long)(last_row / g.G) * pos_bytes + (unsigned long long)(last_row % g.G) * RB;
#pragma unroll
    for (int c = 0; c < St::CPT; ++c) {
      const int idx = c * 256 + tid;
      crow[c] = idx / St::CPR;
      cch[c] = idx - crow[c] * St::CPR;
      rho[c] = crow[c];
      qh[c] = crow[c] % g.G;
      addr[c] = (unsigned long long)(crow[c] / g.G) * pos_bytes + (unsigned long long)qh[c] * RB;
    }
    pb = 0.f;
  }
  __device__ __forceinline__ void fetch(const unsigned char* qbytes, const float* bw, int rt, int rtiles,
                                        int tid) {
#pragma unroll
    for (int c = 0; c < St::CPT; ++c) {
      const unsigned long long a = rho[c] > last_row ? last_addr : addr[c];
      pre[c] = *reinterpret_cast<const uint4*>(qbytes + a + cch[c] * 16);
      rho[c] += TILE;
      qh[c] += h0;
      const bool wrap = qh[c] >= G;
      qh[c] -= wrap ? G : 0;
      addr[c] += step0 + (wrap ? carry_step : 0ull);
    }
    pb = bw[min(rt, rtiles - 1) * TILE + (tid & (TILE - 1))];
  }
  __device__ __forceinline__ void stash(unsigned char* tile, float* beta, int tid) const {
#pragma unroll
    for (int c = 0; c < St::CPT; ++c)
      *reinterpret_cast<uint4*>(&tile[crow[c] * St::LROW + cch[c] * 16]) = pre[c];
    if (tid < TILE) beta[tid] = pb;
  }
};

// ---------------------------------------------------------------------------
// Pass 2.  S tiles: A = 32 query rows (LDS), B = window keys (registers), so a
// lane owns one key of each of its two key tiles and 16 query rows of every
// row tile; each column sum stays in one register per lane.
// Grid: units * ceil(W / 256) blocks (XCD-mapped).
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void col_mass_kernel(Geo g, const T* __restrict__ q,
                                                       const T* __restrict__ kc,
                                                       const int32_t* __restrict__ tables,
                                                       const int32_t* __restrict__ prior,
                                                       const float* __restrict__ beta_ws,
                                                       float* __restrict__ scores) {
  using M = Mma<T>;
  using St = Stage<T, D>;
  constexpr int NF = Frags<T, D>::N;
  __shared__ __align__(16) unsigned char lds[2][St::BYTES];
  __shared__ __align__(16) float lbeta[2][TILE];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int per_unit = (g.W + PER_BLOCK - 1) / PER_BLOCK;
  int unit, kb;
  if (!xcd_map(g.S * g.Lyr * g.Hkv * per_unit, per_unit, unit, kb)) return;
  const int kvh = unit % g.Hkv;
  const int layer = (unit / g.Hkv) % g.Lyr;
  const int n = unit / (g.Hkv * g.Lyr);
  const int L = prior[n];
  const int32_t* trow = tables + (long long)n * g.max_blocks;

  // the wave's two key tiles (B operands); keys past the window are zeros
  // and their columns are never written
  const int key0 = kb * PER_BLOCK + wave * PER_WAVE;
  const unsigned char* kbytes = reinterpret_cast<const unsigned char*>(kc);
  const PagedRows pr = paged_rows(g, trow, layer, kvh, L, (int)sizeof(T));
  typename M::frag bk[2][NF];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int j = key0 + s * TILE + col;
    const T* kp = reinterpret_cast<const T*>(kbytes + paged_row(pr, L + min(j, g.W - 1))) + half * (D / 2);
    load_half_row<T, D>(kp, j < g.W, bk[s]);
  }

  // staging of Q row tile rt: this thread's chunks.  The element offset of
  // each chunk's row advances by one tile (32 rows) per step; rows past G*W
  // are read from the last row (their beta is +inf, so they add zero).
  const unsigned char* qbytes = reinterpret_cast<const unsigned char*>(
      q + (((long long)n * g.Lyr + layer) * g.W) * g.Hq * D + (long long)kvh * g.G * D);
  const float* bw = beta_ws + (long long)unit * g.GWp;
  const int step_i = TILE / g.G, step_h = TILE - step_i * g.G;
  const int last_i = (g.GW - 1) / g.G, last_h = (g.GW - 1) - last_i * g.G;
  const long long last_off = ((long long)last_i * g.Hq + last_h) * D * (long long)sizeof(T);
  QStream<T, D> qs;
  qs.init(tid, g);
  float csum[2] = {0.f, 0.f};
  const int rtiles = g.GWp / TILE;
#define KARA_Q_FETCH(rt) qs.fetch(qbytes, bw, (rt), rtiles, tid)
#define KARA_Q_STASH(buf) qs.stash(lds[buf], lbeta[buf], tid)
  KARA_Q_FETCH(0);
  KARA_Q_STASH(0);
  __syncthreads();
  for (int rt = 0; rt < rtiles; ++rt) {
    const int buf = rt & 1;
    KARA_Q_FETCH(rt + 1);                       // past the end: last row, last betas
    typename M::frag aq[NF];
    lds_half_row<T, D>(lds[buf], col, half, aq);
    f32x16 acc[2] = {{}, {}};
    // raised issue priority while the MFMAs issue: of the waves sharing a
    // SIMD (three workgroups per compute unit), one with MFMAs ready goes
    // first while the others run their exponentials.  (Pass 1 runs slower
    // with it: its per-tile rescaling chain is what its waves wait on.)
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      acc[0] = M::mma(aq[f], bk[0][f], acc[0]);
      acc[1] = M::mma(aq[f], bk[1][f], acc[1]);
    }
    __builtin_amdgcn_s_setprio(0);
    // acc[s][r]: query row rt*32 + 8*(r/4) + 4*half + (r%4) against key key0 + 32 s + col
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x4 b4 = *reinterpret_cast<const f32x4*>(&lbeta[buf][8 * r4 + 4 * half]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        csum[0] += fast_exp2(__builtin_fmaf(acc[0][4 * r4 + e], g.alpha, -b4[e]));
        csum[1] += fast_exp2(__builtin_fmaf(acc[1][4 * r4 + e], g.alpha, -b4[e]));
      }
    }
    KARA_Q_STASH(buf ^ 1);
    __syncthreads();
  }
#undef KARA_Q_FETCH
#undef KARA_Q_STASH
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const float tot = csum[s] + __shfl_xor(csum[s], 32);
    const int j = key0 + s * TILE + col;
    if (half == 0 && j < g.W) scores[(long long)unit * g.W + j] = tot;
  }
}

// ---------------------------------------------------------------------------
template <typename T, int D>
static hipError_t launch_score_t(const Geo& g, const void* q, const void* kc, const int32_t* tables,
                                 const int32_t* prior, float* scores, float* ws, hipStream_t st) {
  const long long units = (long long)g.S * g.Lyr * g.Hkv;
  const long long b1 = units * ((g.GW + PER_BLOCK - 1) / PER_BLOCK);
  const long long b2 = units * ((g.W + PER_BLOCK - 1) / PER_BLOCK);
  if (b1 > 0x7ffffff0LL || b2 > 0x7ffffff0LL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((row_lse_kernel<T, D>), dim3(padded_grid(b1)), dim3(256), 0, st, g, (const T*)q,
                     (const T*)kc, tables, prior, ws);
  hipLaunchKernelGGL((col_mass_kernel<T, D>), dim3(padded_grid(b2)), dim3(256), 0, st, g, (const T*)q,
                     (const T*)kc, tables, prior, (const float*)ws, scores);
  return hipGetLastError();
}

hipError_t launch_fused_score(const Geo& g, const void* q, const void* kc, const int32_t* tables,
                              const int32_t* prior, float* scores, hipStream_t st);
bool fused_score_supported(const Geo& g, int dtype);
bool small_score_supported(const Geo& g, int dtype);
hipError_t launch_small_score(const Geo& g, int dtype, const void* q, const void* kc, const int32_t* tables,
                              const int32_t* prior, float* scores, hipStream_t st);

hipError_t launch_score(const Geo& g, int dtype, const void* q, const void* kc, const int32_t* tables,
                        const int32_t* prior, float* scores, float* ws, hipStream_t st) {
  // windows that fit in one workgroup's registers: single pass (score_fused.hip)
  if (fused_score_supported(g, dtype)) return launch_fused_score(g, q, kc, tables, prior, scores, st);
  // small windows of the other element types and head_dims: single pass with K in LDS (score_small.hip)
  if (small_score_supported(g, dtype)) return launch_small_score(g, dtype, q, kc, tables, prior, scores, st);
  if (dtype == KARA_BF16) {
    if (g.D == 128) return launch_score_t<__bf16, 128>(g, q, kc, tables, prior, scores, ws, st);
    return launch_score_t<__bf16, 64>(g, q, kc, tables, prior, scores, ws, st);
  }
  if (g.D == 128) return launch_score_t<float, 128>(g, q, kc, tables, prior, scores, ws, st);
  return launch_score_t<float, 64>(g, q, kc, tables, prior, scores, ws, st);
}

size_t score_workspace_bytes(const Geo& g, int dtype) {
  if (fused_score_supported(g, dtype) || small_score_supported(g, dtype)) return 0;
  return (size_t)g.S * g.Lyr * g.Hkv * (size_t)g.GWp * sizeof(float);
}

}  // namespace kara
