// Paged decode attention over the cache: the consumer of the compacted pages.
//
// The Kara abstract (shd-paper.top, English abstract) keeps the compressed
// window inside a PagedAttention store and claims lower KV memory and higher
// output throughput.  One decode step reads, for every (sequence, layer,
// query head), the K and V rows of the logical slots [0, seq_len) through the
// block table and computes softmax(q k^T / sqrt(d)) v.  After compaction the
// sequence holds L + budget slots instead of L + window, so this kernel reads
// fewer bytes; it is HBM-bound (one K row and one V row per slot, each used by
// the G query heads of its KV group).
//
// Layout of the work: a workgroup of four waves owns one (sequence, layer, KV
// head, head chunk of up to GM query heads, split of the slot range).  Each
// wave walks its own steps of KT slots (interleaved with the other waves) with
// its own running max / sum, and the four states are merged in LDS at the end.
// Per step the logits of GM heads x KT slots come from 16x16 MFMA tiles
// (S = Q K^T, heads padded to 16 rows) and the value rows are accumulated on
// the VALU: a lane owns DPL dims of one value row and all GM heads.  When the
// slot range is split across workgroups, each split writes (max, sum, output)
// to the workspace and a second kernel merges them.
#include <algorithm>

#include "kara_device.h"

namespace kara {

// (kernels live in namespace kara so that profilers print their names)
constexpr int DA_WAVES = 4;
constexpr int DA_THREADS = 64 * DA_WAVES;
constexpr int DA_TBL = 4096;   // block-table entries one workgroup stages in LDS
constexpr int DA_TARGET_WGS = 2048;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct AttnGeo {
  int S, Lyr, Hq, Hkv, G, D, bs, bs_shift, max_blocks;
  int hchunks, splits, rows_per_split;
  uint32_t nblocks;
  float alpha;   // log2(e) / sqrt(D)
};

template <typename T, int D, int GM>
struct AttnShape {
  static constexpr bool BF = sizeof(T) == 2;
  static constexpr int KS = BF ? D / 32 : D / 4;      // MFMA k-steps per key row
  static constexpr int KVEC = BF ? D / 32 : D / 16;   // 16-byte K loads per lane per 16-key tile
  static constexpr int NT = BF ? 2 : 1;               // 16-key tiles per step
  static constexpr int KT = 16 * NT;                  // slots per step
  static constexpr int DPL = (GM >= 8 || D == 64) ? 8 : 16;   // value dims per lane
  static constexpr int LPK = D / DPL;                 // lanes per value row
  static constexpr int KSUB = 64 / LPK;               // value rows per sub-step
  static constexpr int NV = KT / KSUB;                // value sub-steps per step
  static constexpr int EPV = 16 / (int)sizeof(T);     // elements per 16-byte load
  static constexpr int VVEC = DPL / EPV;              // 16-byte V loads per lane per sub-step
  static_assert(16 % KSUB == 0, "a value sub-step must lie in one MFMA tile");
  static_assert(VVEC >= 1, "value piece");
};

__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const u32x4& b, const f32x4& c, __bf16) {
  bf16x8 x, y;
  __builtin_memcpy(&x, &a, 16);
  __builtin_memcpy(&y, &b, 16);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, c, 0, 0, 0);
}

__device__ __forceinline__ float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, __shfl_xor(v, 1, 16));
  v = fmaxf(v, __shfl_xor(v, 2, 16));
  v = fmaxf(v, __shfl_xor(v, 4, 16));
  v = fmaxf(v, __shfl_xor(v, 8, 16));
  return v;
}

__device__ __forceinline__ float sum16(float v) {
  v += __shfl_xor(v, 1, 16);
  v += __shfl_xor(v, 2, 16);
  v += __shfl_xor(v, 4, 16);
  v += __shfl_xor(v, 8, 16);
  return v;
}

template <typename T, int D, int GM>
__global__ __launch_bounds__(DA_THREADS) void decode_attn_kernel(AttnGeo g, const T* __restrict__ q,
                                                                 const unsigned char* __restrict__ kc,
                                                                 const unsigned char* __restrict__ vc,
                                                                 const int32_t* __restrict__ tables,
                                                                 const int32_t* __restrict__ seq_lens,
                                                                 float* __restrict__ out, float* __restrict__ part) {
  using A = AttnShape<T, D, GM>;
  constexpr int OW = D + 2;                       // floats per head in the merge area
  __shared__ int tbl[DA_TBL];
  __shared__ float red[DA_WAVES][GM][OW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x % g.splits;
  const int rest = blockIdx.x / g.splits;
  const int hc = rest % g.hchunks;
  const int unit = rest / g.hchunks;                // (n, layer, kvh)
  const int kvh = unit % g.Hkv;
  const int layer = (unit / g.Hkv) % g.Lyr;
  const int n = unit / (g.Hkv * g.Lyr);
  const int h0 = kvh * g.G + hc * GM;               // first query head of this chunk
  const int nh = min(GM, g.G - hc * GM);

  const int len = (int)min((long long)max(seq_lens[n], 0), (long long)g.max_blocks << g.bs_shift);
  const int k0 = split * g.rows_per_split;
  const int k1 = min(len, k0 + g.rows_per_split);

  // stage the block ids of [k0, k1) in LDS
  const int32_t* trow = tables + (long long)n * g.max_blocks;
  const int lb0 = k0 >> g.bs_shift;
  const int nlb = k1 > k0 ? ((k1 - 1) >> g.bs_shift) - lb0 + 1 : 0;
  for (int i = tid; i < nlb; i += DA_THREADS) {
    const int32_t b = trow[lb0 + i];
    tbl[i] = (uint32_t)b < g.nblocks ? b : 0;      // an out-of-range entry reads block 0 (in bounds)
  }
  __syncthreads();

  const uint32_t row_bytes = (uint32_t)(D * sizeof(T));
  const uint64_t blk_stride = (uint64_t)g.Hkv * (g.bs * row_bytes);
  const uint64_t base = (uint64_t)layer * g.nblocks * blk_stride + (uint64_t)kvh * g.bs * row_bytes;
  const int bs_mask = (1 << g.bs_shift) - 1;

  // query operand (A of S = Q K^T): lane l holds head row l%16, reduction slice l/16
  const int col = lane & 15, gq = lane >> 4;
  u32x4 qa[A::KVEC];
  {
    const bool hv = col < nh;
    const unsigned char* qrow =
        reinterpret_cast<const unsigned char*>(q + (((long long)n * g.Lyr + layer) * g.Hq + h0 + (hv ? col : 0)) * D);
#pragma unroll
    for (int j = 0; j < A::KVEC; ++j) {
      const uint32_t off = A::BF ? (uint32_t)(64 * j + 16 * gq) : (uint32_t)(gq * D + 16 * j);
      qa[j] = hv ? *reinterpret_cast<const u32x4*>(qrow + off) : u32x4{0u, 0u, 0u, 0u};
    }
  }

  float m_run[4], l_run[4];
  float o[GM][A::DPL];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m_run[r] = -INFINITY;
    l_run[r] = 0.f;
  }
#pragma unroll
  for (int h = 0; h < GM; ++h)
#pragma unroll
    for (int e = 0; e < A::DPL; ++e) o[h][e] = 0.f;

  const int vkey = lane / A::LPK, piece = lane % A::LPK;
  const float alpha = g.alpha;

  for (int sb = k0 + wave * A::KT; sb < k1; sb += DA_WAVES * A::KT) {
    // ---- loads: K tiles (B operand: key col, slice gq) and V sub-steps
    u32x4 kb[A::NT][A::KVEC];
#pragma unroll
    for (int t = 0; t < A::NT; ++t) {
      const int key = min(sb + 16 * t + col, k1 - 1);
      const uint64_t ro = (uint64_t)tbl[(key >> g.bs_shift) - lb0] * blk_stride + base +
                          (uint32_t)((key & bs_mask) * row_bytes);
#pragma unroll
      for (int j = 0; j < A::KVEC; ++j) {
        const uint32_t off = A::BF ? (uint32_t)(64 * j + 16 * gq) : (uint32_t)(gq * D + 16 * j);
        kb[t][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kc + ro + off));
      }
    }
    u32x4 vb[A::NV][A::VVEC];
#pragma unroll
    for (int v = 0; v < A::NV; ++v) {
      const int key = min(sb + v * A::KSUB + vkey, k1 - 1);
      const uint64_t ro = (uint64_t)tbl[(key >> g.bs_shift) - lb0] * blk_stride + base +
                          (uint32_t)((key & bs_mask) * row_bytes);
#pragma unroll
      for (int j = 0; j < A::VVEC; ++j)
        vb[v][j] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(vc + ro + 16 * piece + 16 * A::LPK * j));
    }

    // ---- logits: lane holds slot col of tile t for heads 4*gq + r
    f32x4 s[A::NT];
#pragma unroll
    for (int t = 0; t < A::NT; ++t) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (A::BF) {
#pragma unroll
        for (int ks = 0; ks < A::KS; ++ks) acc = mfma16(qa[ks], kb[t][ks], acc, __bf16{});
      } else {
#pragma unroll
        for (int j = 0; j < A::KVEC; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(qa[j][e]), __uint_as_float(kb[t][j][e]),
                                                      acc, 0, 0, 0);
      }
      const bool valid = sb + 16 * t + col < k1;
#pragma unroll
      for (int r = 0; r < 4; ++r) s[t][r] = valid ? acc[r] * alpha : -INFINITY;
    }

    // ---- online softmax per head (uniform over the 16 lanes of group gq)
    float resc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float mx = s[0][r];
#pragma unroll
      for (int t = 1; t < A::NT; ++t) mx = fmaxf(mx, s[t][r]);
      mx = max16(mx);
      const float mn = fmaxf(m_run[r], mx);         // finite: every step holds a valid slot
      resc[r] = fast_exp2(m_run[r] - mn);
      m_run[r] = mn;
      float ps = 0.f;
#pragma unroll
      for (int t = 0; t < A::NT; ++t) {
        s[t][r] = fast_exp2(s[t][r] - mn);
        ps += s[t][r];
      }
      l_run[r] = l_run[r] * resc[r] + ps;
    }

    // ---- rescale and accumulate the value rows
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      const float a = __shfl(resc[h & 3], 16 * (h >> 2));
#pragma unroll
      for (int e = 0; e < A::DPL; ++e) o[h][e] *= a;
    }
#pragma unroll
    for (int v = 0; v < A::NV; ++v) {
      const int t = (v * A::KSUB) / 16;
      const int c = (v * A::KSUB) % 16 + vkey;
      float p[GM];
#pragma unroll
      for (int h = 0; h < GM; ++h) p[h] = __shfl(s[t][h & 3], c + 16 * (h >> 2));
#pragma unroll
      for (int j = 0; j < A::VVEC; ++j) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t word = vb[v][j][w];
          if constexpr (A::BF) {
            const float x0 = lo_f(word), x1 = hi_f(word);
#pragma unroll
            for (int h = 0; h < GM; ++h) {
              o[h][j * A::EPV + 2 * w] += p[h] * x0;
              o[h][j * A::EPV + 2 * w + 1] += p[h] * x1;
            }
          } else {
            const float x = __uint_as_float(word);
#pragma unroll
            for (int h = 0; h < GM; ++h) o[h][j * A::EPV + w] += p[h] * x;
          }
        }
      }
    }
  }

  // ---- merge inside the wave: sums over the 16 slot lanes, outputs over the value rows
#pragma unroll
  for (int r = 0; r < 4; ++r) l_run[r] = sum16(l_run[r]);
#pragma unroll
  for (int h = 0; h < GM; ++h)
#pragma unroll
    for (int e = 0; e < A::DPL; ++e) {
      float x = o[h][e];
#pragma unroll
      for (int m = A::LPK; m < 64; m <<= 1) x += __shfl_xor(x, m);
      o[h][e] = x;
    }
  if (col == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * gq + r;
      if (h < GM) {
        red[wave][h][0] = m_run[r];
        red[wave][h][1] = l_run[r];
      }
    }
  }
  if (vkey == 0) {
#pragma unroll
    for (int h = 0; h < GM; ++h)
#pragma unroll
      for (int j = 0; j < A::VVEC; ++j)
#pragma unroll
        for (int i = 0; i < A::EPV; ++i)
          red[wave][h][2 + A::EPV * piece + A::EPV * A::LPK * j + i] = o[h][j * A::EPV + i];
  }
  __syncthreads();

  // ---- merge the four waves; write the output or this split's partial
  for (int idx = tid; idx < nh * D; idx += DA_THREADS) {
    const int h = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < DA_WAVES; ++w) M = fmaxf(M, red[w][h][0]);
    float Lt = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < DA_WAVES; ++w) {
        const float f = fast_exp2(red[w][h][0] - M);   // 0 for a wave without slots
        Lt += red[w][h][1] * f;
        O += red[w][h][2 + d] * f;
      }
    }
    const float val = Lt > 0.f ? O / Lt : 0.f;
    const long long head = ((long long)n * g.Lyr + layer) * g.Hq + h0 + h;
    if (g.splits == 1) {
      out[head * D + d] = val;
    } else {
      float* pp = part + ((((long long)unit * g.hchunks + hc) * g.splits + split) * GM + h) * OW;
      if (d == 0) {
        pp[0] = M;
        pp[1] = Lt;
      }
      pp[2 + d] = val;
    }
  }
}

// One thread per output element: merge the splits of one query head.
__global__ __launch_bounds__(128) void decode_attn_merge_kernel(AttnGeo g, int GM, const float* __restrict__ part,
                                                                float* __restrict__ out) {
  const int D = g.D, OW = D + 2;
  const long long head = blockIdx.x;   // (n, layer, h)
  const int h = (int)(head % g.Hq);
  const long long nl = head / g.Hq;    // n * Lyr + layer
  const int kvh = h / g.G, hg = h % g.G, hc = hg / GM, hh = hg % GM;
  const long long unit = nl * g.Hkv + kvh;
  const float* pp = part + ((unit * g.hchunks + hc) * g.splits * GM + hh) * OW;
  const long long sstride = (long long)GM * OW;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float M = -INFINITY;
    for (int s = 0; s < g.splits; ++s) M = fmaxf(M, pp[s * sstride]);
    float Lt = 0.f, O = 0.f;
    if (M != -INFINITY) {
      for (int s = 0; s < g.splits; ++s) {
        const float w = pp[s * sstride + 1] * fast_exp2(pp[s * sstride] - M);
        Lt += w;
        O += w * pp[s * sstride + 2 + d];
      }
    }
    out[head * D + d] = Lt > 0.f ? O / Lt : 0.f;
  }
}

struct AttnPlan {
  int GM, hchunks, splits, rows_per_split;
  long long wgs;
  size_t ws_bytes;
};

static AttnPlan plan_of(const Geo& g) {
  AttnPlan p;
  p.GM = g.G <= 1 ? 1 : g.G <= 2 ? 2 : g.G <= 4 ? 4 : 8;
  p.hchunks = (g.G + p.GM - 1) / p.GM;
  const long long units = (long long)g.S * g.Lyr * g.Hkv * p.hchunks;
  const long long maxlen = (long long)g.max_blocks * g.bs;
  const long long step = 32LL * DA_WAVES;
  long long splits = 1;
  if (units > 0 && units < DA_TARGET_WGS) splits = (DA_TARGET_WGS + units - 1) / units;
  splits = std::min(splits, std::max(1LL, (maxlen + 255) / 256));
  // rows per split whose blocks fit the LDS table, as a multiple of the step
  const long long cap = (long long)(DA_TBL - 2) * g.bs / step * step;
  splits = std::max(splits, (maxlen + cap - 1) / cap);
  long long rps = (maxlen + splits - 1) / splits;
  rps = (rps + step - 1) / step * step;
  splits = std::max(1LL, (maxlen + rps - 1) / rps);
  p.splits = (int)splits;
  p.rows_per_split = (int)rps;
  p.wgs = units * splits;
  p.ws_bytes = p.splits > 1 ? (size_t)units * splits * p.GM * (g.D + 2) * sizeof(float) : 0;
  return p;
}

template <typename T, int D>
hipError_t launch_t(const AttnGeo& a, int GM, long long wgs, const void* q, const void* kc, const void* vc,
                    const int32_t* tables, const int32_t* lens, float* out, float* part, hipStream_t st) {
  const dim3 grid((unsigned)wgs), block(DA_THREADS);
  const T* qq = static_cast<const T*>(q);
  const unsigned char* k = static_cast<const unsigned char*>(kc);
  const unsigned char* v = static_cast<const unsigned char*>(vc);
  switch (GM) {
    case 1: hipLaunchKernelGGL((decode_attn_kernel<T, D, 1>), grid, block, 0, st, a, qq, k, v, tables, lens, out, part); break;
    case 2: hipLaunchKernelGGL((decode_attn_kernel<T, D, 2>), grid, block, 0, st, a, qq, k, v, tables, lens, out, part); break;
    case 4: hipLaunchKernelGGL((decode_attn_kernel<T, D, 4>), grid, block, 0, st, a, qq, k, v, tables, lens, out, part); break;
    default: hipLaunchKernelGGL((decode_attn_kernel<T, D, 8>), grid, block, 0, st, a, qq, k, v, tables, lens, out, part); break;
  }
  return hipGetLastError();
}

size_t decode_attn_workspace_bytes(const Geo& g) { return plan_of(g).ws_bytes; }

int decode_attn_splits(const Geo& g) { return plan_of(g).splits; }

hipError_t launch_decode_attn(const Geo& g, int dtype, const void* q, const void* kc, const void* vc,
                              const int32_t* tables, const int32_t* lens, float* out, float* ws, hipStream_t st) {
  const AttnPlan p = plan_of(g);
  if (p.wgs == 0) return hipSuccess;
  if (p.wgs > 0x7fffffffLL || (long long)g.S * g.Lyr * g.Hq > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  AttnGeo a;
  a.S = g.S;
  a.Lyr = g.Lyr;
  a.Hq = g.Hq;
  a.Hkv = g.Hkv;
  a.G = g.G;
  a.D = g.D;
  a.bs = g.bs;
  a.bs_shift = g.bs_shift;
  a.max_blocks = g.max_blocks;
  a.hchunks = p.hchunks;
  a.splits = p.splits;
  a.rows_per_split = p.rows_per_split;
  a.nblocks = (uint32_t)g.nblocks;
  a.alpha = (float)(1.4426950408889634 / sqrt((double)g.D));
  hipError_t e;
  if (dtype == KARA_BF16)
    e = g.D == 128 ? launch_t<__bf16, 128>(a, p.GM, p.wgs, q, kc, vc, tables, lens, out, ws, st)
                   : launch_t<__bf16, 64>(a, p.GM, p.wgs, q, kc, vc, tables, lens, out, ws, st);
  else
    e = g.D == 128 ? launch_t<float, 128>(a, p.GM, p.wgs, q, kc, vc, tables, lens, out, ws, st)
                   : launch_t<float, 64>(a, p.GM, p.wgs, q, kc, vc, tables, lens, out, ws, st);
  if (e != hipSuccess || p.splits == 1) return e;
  const long long heads = (long long)g.S * g.Lyr * g.Hq;
  hipLaunchKernelGGL(decode_attn_merge_kernel, dim3((unsigned)heads), dim3(128), 0, st, a, p.GM, ws, out);
  return hipGetLastError();
}

}  // namespace kara
