// mfma.hpp -- bf16 MFMA building blocks shared by the prefill kernels.
//
// Products that need about fp32 accuracy run as three bf16 MFMAs on a hi/lo split
// of each operand (a*b ~ a_hi b_hi + a_hi b_lo + a_lo b_hi), which keeps about 16
// significant bits with fp32 range.  CDNA4 has no single-precision-class MFMA
// with a higher rate than this.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// An MFMA 16x16x32 operand gives lane l the k indices 8*(l/16) + e, e < 8.  Where
// an operand is built from two 16x16 accumulator tiles (which give lane l the
// rows 4*(l/16) + j, j < 4), its 32 k values are taken in the order
//     pk(g, e) = 4g + e (e < 4, first tile),  16 + 4g + (e - 4) (e >= 4, second tile)
// for g = l/16; both operands of a product use the same order, so the sum over k
// is unchanged.
__device__ __forceinline__ constexpr int pk(int g, int e) { return e < 4 ? 4 * g + e : 12 + 4 * g + e; }

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8 &a, const bf16x8 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Two floats rounded to bf16 (nearest even) by one v_cvt_pk_bf16_f32, a in the low half.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  typedef float f32x2v __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{a, b}, bf16x2v));
}
// hi = bf16(x), lo = bf16(x - hi) for a pair, as packed words (two conversions, two
// exact widenings and two subtractions; converting one value at a time would need
// a third instruction per pair to pack the halves)
struct Split2 {
  uint32_t hi, lo;
};
__device__ __forceinline__ Split2 split2(float a, float b) {
  const uint32_t hi = cvt_pk_bf16(a, b);
  return Split2{hi, cvt_pk_bf16(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u))};
}

struct Split {
  bf16x8 hi, lo;
};
__device__ __forceinline__ Split split8(const float *v) {
  u32x4 h, l;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const Split2 q = split2(v[2 * p], v[2 * p + 1]);
    h[p] = q.hi;
    l[p] = q.lo;
  }
  return Split{__builtin_bit_cast(bf16x8, h), __builtin_bit_cast(bf16x8, l)};
}
__device__ __forceinline__ Split split44(const f32x4 &x, const f32x4 &y) {
  float v[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[j] = x[j];
    v[4 + j] = y[j];
  }
  return split8(v);
}
// a*b ~ a_hi b_hi + a_hi b_lo + a_lo b_hi (the lo*lo term is ~2^-16 relative)
__device__ __forceinline__ f32x4 mfma3(const Split &a, const Split &b, f32x4 c) {
  c = mfma_bf16(a.lo, b.hi, c);
  c = mfma_bf16(a.hi, b.lo, c);
  c = mfma_bf16(a.hi, b.hi, c);
  return c;
}

// k = 16 products: lane l holds k = 4(l/16) + e of row (A) / column (B) l % 16,
// which is exactly how a lane holds four rows of a 16x16 accumulator tile
typedef short s16x4 __attribute__((ext_vector_type(4)));
struct Split4 {
  s16x4 hi, lo;
};
__device__ __forceinline__ Split4 split4s(const f32x4 &v) {
  const Split2 a = split2(v[0], v[1]), b = split2(v[2], v[3]);
  return Split4{__builtin_bit_cast(s16x4, u32x2{a.hi, b.hi}), __builtin_bit_cast(s16x4, u32x2{a.lo, b.lo})};
}
__device__ __forceinline__ f32x4 mfma3k16(const Split4 &a, const Split4 &b, f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.lo, b.hi, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.hi, b.lo, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.hi, b.hi, c, 0, 0, 0);
  return c;
}

// a0 * b0 + a1 * b1 + c for bf16 pairs (the products are exact in fp32)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, a), __builtin_bit_cast(bf16x2v, b), c, false);
}
// half h of word x (low half) and of word y (high half): one v_perm_b32
__device__ __forceinline__ uint32_t halves(uint32_t x, uint32_t y, int h) {
  return __builtin_amdgcn_perm(y, x, h ? 0x07060302u : 0x05040100u);
}
// channel e of two input rows (8 bf16 channels each) as one pair
__device__ __forceinline__ uint32_t tok_pair(const u32x4 &r0, const u32x4 &r1, int e) {
  return halves(r0[e >> 1], r1[e >> 1], e & 1);
}

__device__ __forceinline__ float bf16_elem(const u32x4 &v, int e) {
  const uint32_t w = v[e >> 1];
  return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
}

// 2^x on the hardware unit; a result below 2^-126 comes out as zero, which only
// drops decay products that are negligible next to the unit-scale terms they join
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x4 ld4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
__device__ __forceinline__ void st4(float *p, const f32x4 &v) { *reinterpret_cast<f32x4 *>(p) = v; }

}  // namespace gdn
