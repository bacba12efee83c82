// lanes.hpp -- device helpers shared by the one-token kernels (decode and the
// draft-tree verify): state vectors in the pool dtype, lane-group sums, and
// bf16 conv-row slices.  Internal; not installed.
#pragma once

#include "common.hpp"

namespace gdn {

// One lane's 16-byte piece of a K-contiguous state row: 4 fp32 or 8 bf16 values.
template <typename TS>
struct StateVec;
template <>
struct StateVec<float> {
  static constexpr int N = 4;
  typedef float raw __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ void to_f32(const raw &r, float *f) {
    f[0] = r[0]; f[1] = r[1]; f[2] = r[2]; f[3] = r[3];
  }
  static __device__ __forceinline__ raw from_f32(const float *f) {
    raw r;
    r[0] = f[0]; r[1] = f[1]; r[2] = f[2]; r[3] = f[3];
    return r;
  }
};
template <>
struct StateVec<uint16_t> {  // bf16
  static constexpr int N = 8;
  typedef uint32_t raw __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ void to_f32(const raw &r, float *f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(r[i] << 16);
      f[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ raw from_f32(const float *f) {
    raw r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    return r;
  }
};

// Sum over each aligned group of N lanes, left in every lane of the group.  The
// first four steps are DPP lane permutes inside the VALU (swap neighbours, swap
// pairs, mirror within 8, mirror within 16), each folded into its add as one
// v_add_f32_dpp (every source lane exists for these patterns, so the bound
// control setting that allows the fold changes nothing); wider groups use the
// gfx950 row swaps (lane ^ 16, lane ^ 32).  Each step adds the same two partial
// sums in every lane of a group, so all lanes end with the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "group of 2^k lanes");
  const int lane = threadIdx.x & 63;
  if constexpr (N >= 2) v = dpp_mov<0xB1>(v) + v;   // quad_perm [1,0,3,2]
  if constexpr (N >= 4) v = dpp_mov<0x4E>(v) + v;   // quad_perm [2,3,0,1]
  if constexpr (N >= 8) v = dpp_mov<0x141>(v) + v;  // row_half_mirror
  if constexpr (N >= 16) v = dpp_mov<0x140>(v) + v; // row_mirror
  if constexpr (N >= 32) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v += __uint_as_float((lane & 16) ? r[0] : r[1]);
  }
  if constexpr (N >= 64) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v += __uint_as_float((lane & 32) ? r[0] : r[1]);
  }
  return v;
}
__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// CW consecutive bf16 conv values (a row slice) as one load / store
template <int CW>
struct ConvVec;
template <>
struct ConvVec<2> {
  typedef uint32_t raw;
  static __device__ __forceinline__ uint32_t word(const raw &v, int) { return v; }
};
template <>
struct ConvVec<4> {
  typedef u32x2 raw;
  static __device__ __forceinline__ uint32_t word(const raw &v, int i) { return v[i]; }
};
template <>
struct ConvVec<8> {
  typedef u32x4 raw;
  static __device__ __forceinline__ uint32_t word(const raw &v, int i) { return v[i]; }
};

}  // namespace gdn
