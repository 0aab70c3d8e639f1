// Internal device helpers shared by the Kara kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kara.h"

namespace kara {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Geometry shared by every kernel, derived once on the host.
struct Geo {
  int S, Lyr, Hq, Hkv, G, D, W, B, seeds, radius;
  int bs, bs_shift, max_blocks, GW, GWp;   // GW = G*W query rows per unit, GWp rounded up to 32
  long long nblocks;
  float alpha;                              // log2(e) / sqrt(D): logits in base-2 units
};

// ---------------------------------------------------------------------------
// MFMA 32x32 fragments.  A lane of a wave64 holds, for the A (or B) operand,
// row (or column) lane%32 and KPL consecutive reduction elements; lanes 0-31
// and 32-63 cover the two halves of the reduction slice of one instruction.
// Because the reduction order over head_dim does not change the product, lane
// half h simply owns the contiguous head_dim range [h*D/2, (h+1)*D/2) and
// feeds it KPL elements per instruction.  Output: lane l holds column l%32,
// register r holds row 8*(r/4) + 4*(l/32) + (r%4).
// ---------------------------------------------------------------------------
template <typename T>
struct Mma;

template <>
struct Mma<__bf16> {
  static constexpr int KPL = 8;
  typedef bf16x8 frag;
  __device__ static inline f32x16 mma(const frag& a, const frag& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mma<float> {
  static constexpr int KPL = 1;
  typedef float frag;
  __device__ static inline f32x16 mma(const frag& a, const frag& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// Number of fragments one lane holds for a row of head_dim D.
template <typename T, int D>
struct Frags {
  static constexpr int N = (D / 2) / Mma<T>::KPL;
  static constexpr int BYTES = (D / 2) * (int)sizeof(T);   // per lane: 64..256 bytes
  static constexpr int VEC = BYTES / 16;                   // 16-byte loads per lane
};

// Load the lane's half row (D/2 contiguous elements) as fragments.  `ok`
// false gives zeros and issues no load.
template <typename T, int D>
__device__ inline void load_half_row(const T* __restrict__ p, bool ok,
                                     typename Mma<T>::frag (&f)[Frags<T, D>::N]) {
  constexpr int VEC = Frags<T, D>::VEC;
  uint4 v[VEC];
  if (ok) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int i = 0; i < VEC; ++i) v[i] = q[i];
  } else {
#pragma unroll
    for (int i = 0; i < VEC; ++i) v[i] = make_uint4(0, 0, 0, 0);
  }
  static_assert(sizeof(f) == sizeof(v), "fragment size");
  __builtin_memcpy(&f, &v, sizeof(v));
}

// Element offset of logical slot `pos` of (layer, kv head) in a paged pool, or
// -1 when the table entry is out of range.
__device__ inline long long slot_offset(const Geo& g, const int32_t* __restrict__ table_row, int layer,
                                        int kvh, int pos) {
  int lb = pos >> g.bs_shift;
  if (pos < 0 || lb >= g.max_blocks) return -1;
  int blk = table_row[lb];
  if (blk < 0 || (long long)blk >= g.nblocks) return -1;
  int off = pos & (g.bs - 1);
  return ((((long long)layer * g.nblocks + blk) * g.Hkv + kvh) * g.bs + off) * (long long)g.D;
}

// Paged addressing for hot loops, in bytes.  `blk_stride` is the byte size
// of one physical block (Hkv * bs * D elements) and `base` the byte offset of
// (layer, kv head, slot 0) inside block 0.  The table read is clamped into the
// row and an out-of-range entry is replaced by block 0 (which exists whenever
// there is a sequence), so the address is always inside the pool; the data of
// such a slot is unspecified.
struct PagedRows {
  const int32_t* trow;
  unsigned long long base;
  uint32_t blk_stride, row_bytes;
  int L, bs_shift, bs_mask, max_blocks;
  uint32_t nblocks;
};

// Byte offset of logical slot `pos` (see PagedRows).
__device__ __forceinline__ unsigned long long paged_row(const PagedRows p, int pos) {
  const int lb = min(max(pos >> p.bs_shift, 0), p.max_blocks - 1);
  const int32_t blk = p.trow[lb];
  const uint32_t b = (uint32_t)blk < p.nblocks ? (uint32_t)blk : 0u;
  return (unsigned long long)b * p.blk_stride + p.base + (uint32_t)((pos & p.bs_mask) * p.row_bytes);
}

__device__ inline PagedRows paged_rows(const Geo& g, const int32_t* table_row, int layer, int kvh, int L,
                                       int elem_bytes) {
  PagedRows p;
  p.trow = table_row;
  p.blk_stride = (uint32_t)(g.Hkv * g.bs * g.D * elem_bytes);
  p.row_bytes = (uint32_t)(g.D * elem_bytes);
  p.base = (unsigned long long)layer * (unsigned long long)g.nblocks * p.blk_stride +
           (unsigned long long)kvh * g.bs * p.row_bytes;
  p.L = L;
  p.bs_shift = g.bs_shift;
  p.bs_mask = g.bs - 1;
  p.max_blocks = g.max_blocks;
  p.nblocks = (uint32_t)g.nblocks;
  return p;
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

}  // namespace kara
