// decode.hip -- one decode token per request, one workgroup per (request, head).
//
// Per token and head (page "企业官网建设流程全解析", Kimi K3 notes, section
// "Speculative decoding" for the recurrence; section "Linear的kv cache大小具体
// 计算逻辑" for the kernel-4 conv over the last three raw q/k/v rows):
//   y = w0 r0 + w1 r1 + w2 r2 + w3 x;  rows <- (r1, r2, x)
//   k <- k / sqrt(|k|^2 + 1e-6)
//   S' = S Diag(alpha);  u = S' k;  d = beta (v - u);  S = S' + d k^T
//   o = scale S q = scale (S' q + d (k.q))
//
// The state stream is the whole cost: every (request, head) reads and writes
// head_v x head_k state values once.  Rows of S are K-contiguous, so each lane
// owns one 16-byte vector of a row (4 fp32 or 8 bf16 values) and a row is
// spread over D/VEC adjacent lanes: every load and store instruction of a wave
// covers whole contiguous rows.  The per-row dot products S'k and S'q reduce
// over those lanes with cross-lane shuffles.  All of a lane's state vectors are
// loaded before the conv prologue runs, so the HBM reads overlap with it.
#include "common.hpp"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

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
    for (int i = 0; i < 4; ++i)
      r[i] = uint32_t(f32_to_bf16(f[2 * i])) | (uint32_t(f32_to_bf16(f[2 * i + 1])) << 16);
    return r;
  }
};

__device__ __forceinline__ float block_sum(float v, float *scratch) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();  // scratch may still be read by a previous call
  if (lane == 0) scratch[w] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) t += scratch[i];
  return t;
}

template <int D, typename TS, int kAlphaMode>
__global__ __launch_bounds__(kThreads) void gdn_decode_kernel(
    TS *__restrict__ ssm, uint16_t *__restrict__ conv, int32_t *err, int slots, int heads,
    DecodeArgs a) {
  using SV = StateVec<TS>;
  constexpr int VEC = SV::N;
  constexpr int LPR = D / VEC;          // lanes per row
  constexpr int RPI = 64 / LPR;         // rows per wave instruction
  constexpr int GROUPS = (D + RPI - 1) / RPI;  // row groups per head
  constexpr int ITERS = (GROUPS + kWaves - 1) / kWaves;
  static_assert(LPR >= 1 && LPR <= 64 && (64 % LPR) == 0, "row layout");

  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = heads;
  const int64_t C = int64_t(H) * 3 * D;
  const int slot = a.slot_table[b];
  uint16_t *out = a.out + (int64_t(b) * H + h) * D;

  if (slot <= 0 || slot >= slots) {
    if (tid < D) out[tid] = 0;
    if (slot >= slots && err && tid == 0) atomicOr(err, GDN_ERRW_BAD_SLOT);
    return;
  }

  // ---- issue the state loads first ------------------------------------
  TS *Sblk = ssm + ((int64_t(a.layer) * slots + slot) * H + h) * int64_t(D) * D;
  const int row_in_group = lane / LPR;
  const int col0 = (lane % LPR) * VEC;
  typename SV::raw sraw[ITERS];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int g = wave + it * kWaves;
    const int r = g * RPI + row_in_group;
    if (g < GROUPS && r < D) {
      sraw[it] = *reinterpret_cast<const typename SV::raw *>(Sblk + int64_t(r) * D + col0);
    }
  }

  // ---- snapshot target --------------------------------------------------
  int track = 0;
  if (a.track_interval > 0 && a.track_slots && a.seq_len_after[b] % a.track_interval == 0) {
    track = a.track_slots[2 * b + (a.next_track_idx[b] & 1)];
    if (track >= slots) {
      if (err && tid == 0) atomicOr(err, GDN_ERRW_BAD_TRACK_SLOT);
      track = 0;
    }
  }

  // ---- conv over the head's q, k, v channels -----------------------------
  __shared__ float sq[D], sk[D], sv[D];
  __shared__ float red[kWaves];
  uint16_t *crow = conv + (int64_t(a.layer) * slots + slot) * kConvRows * C;
  uint16_t *trow = track > 0 ? conv + (int64_t(a.layer) * slots + track) * kConvRows * C : nullptr;
  const uint16_t *xb = a.x + int64_t(b) * C;
  for (int i = tid; i < 3 * D; i += kThreads) {
    const int part = i / D, j = i - part * D;
    const int64_t ch = int64_t(part) * H * D + int64_t(h) * D + j;
    const uint16_t r0 = crow[ch], r1 = crow[C + ch], r2 = crow[2 * C + ch], xv = xb[ch];
    const uint2 wv = *reinterpret_cast<const uint2 *>(a.conv_w + ch * 4);
    float y = __uint_as_float(wv.x << 16) * bf16_to_f32(r0);
    y = fmaf(__uint_as_float(wv.x & 0xffff0000u), bf16_to_f32(r1), y);
    y = fmaf(__uint_as_float(wv.y << 16), bf16_to_f32(r2), y);
    y = fmaf(__uint_as_float(wv.y & 0xffff0000u), bf16_to_f32(xv), y);
    if (a.flags & GDN_F_CONV_SILU) y = y / (1.f + __expf(-y));
    (part == 0 ? sq : part == 1 ? sk : sv)[j] = y;
    crow[ch] = r1;
    crow[C + ch] = r2;
    crow[2 * C + ch] = xv;
    if (trow) {
      trow[ch] = r1;
      trow[C + ch] = r2;
      trow[2 * C + ch] = xv;
    }
  }
  __syncthreads();

  // ---- normalisation and k.q --------------------------------------------
  if (a.flags & GDN_F_L2NORM_K) {
    const float ss = block_sum(tid < D ? sk[tid] * sk[tid] : 0.f, red);
    const float inv = 1.f / sqrtf(ss + 1e-6f);
    if (tid < D) sk[tid] *= inv;
  }
  if (a.flags & GDN_F_L2NORM_Q) {
    const float ss = block_sum(tid < D ? sq[tid] * sq[tid] : 0.f, red);
    const float inv = 1.f / sqrtf(ss + 1e-6f);
    if (tid < D) sq[tid] *= inv;
  }
  __syncthreads();
  const float kq = block_sum(tid < D ? sk[tid] * sq[tid] : 0.f, red);

  float kk[VEC], qq[VEC], al[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    kk[e] = sk[col0 + e];
    qq[e] = sq[col0 + e];
  }
  if (kAlphaMode == GDN_ALPHA_PER_CHANNEL) {
    const float *ap = a.alpha + (int64_t(b) * H + h) * D + col0;
#pragma unroll
    for (int e = 0; e < VEC; ++e) al[e] = ap[e];
  } else {
    const float av = a.alpha[int64_t(b) * H + h];
#pragma unroll
    for (int e = 0; e < VEC; ++e) al[e] = av;
  }
  const float beta = a.beta[int64_t(b) * H + h];
  TS *Tblk = track > 0 ? ssm + ((int64_t(a.layer) * slots + track) * H + h) * int64_t(D) * D : nullptr;

  // ---- the state stream --------------------------------------------------
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int g = wave + it * kWaves;
    const int r = g * RPI + row_in_group;
    if (g < GROUPS && r < D) {  // uniform over the LPR lanes of a row
      float s[VEC];
      SV::to_f32(sraw[it], s);
      float pu = 0.f, pq = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        s[e] *= al[e];
        pu = fmaf(s[e], kk[e], pu);
        pq = fmaf(s[e], qq[e], pq);
      }
#pragma unroll
      for (int off = LPR / 2; off > 0; off >>= 1) {
        pu += __shfl_xor(pu, off, 64);
        pq += __shfl_xor(pq, off, 64);
      }
      const float d = beta * (sv[r] - pu);
#pragma unroll
      for (int e = 0; e < VEC; ++e) s[e] = fmaf(d, kk[e], s[e]);
      const typename SV::raw w = SV::from_f32(s);
      *reinterpret_cast<typename SV::raw *>(Sblk + int64_t(r) * D + col0) = w;
      if (Tblk) *reinterpret_cast<typename SV::raw *>(Tblk + int64_t(r) * D + col0) = w;
      if ((lane % LPR) == 0) out[r] = f32_to_bf16(a.scale * fmaf(d, kq, pq));
    }
  }
}

template <int D, typename TS>
hipError_t launch_d(const gdn_pool *p, const DecodeArgs &a, hipStream_t s) {
  dim3 grid(p->d.heads, a.batch);
  if (a.alpha_mode == GDN_ALPHA_PER_CHANNEL)
    hipLaunchKernelGGL((gdn_decode_kernel<D, TS, GDN_ALPHA_PER_CHANNEL>), grid, dim3(kThreads), 0,
                       s, static_cast<TS *>(p->d.ssm_base),
                       static_cast<uint16_t *>(p->d.conv_base), p->d.err_word, p->d.slots,
                       p->d.heads, a);
  else
    hipLaunchKernelGGL((gdn_decode_kernel<D, TS, GDN_ALPHA_PER_HEAD>), grid, dim3(kThreads), 0, s,
                       static_cast<TS *>(p->d.ssm_base), static_cast<uint16_t *>(p->d.conv_base),
                       p->d.err_word, p->d.slots, p->d.heads, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dt(const gdn_pool *p, const DecodeArgs &a, hipStream_t s) {
  return p->d.ssm_dtype == GDN_F32 ? launch_d<D, float>(p, a, s) : launch_d<D, uint16_t>(p, a, s);
}

}  // namespace

hipError_t launch_decode(const gdn_pool *p, const DecodeArgs &a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  switch (p->d.head_k) {
    case 16: return launch_dt<16>(p, a, s);
    case 32: return launch_dt<32>(p, a, s);
    case 64: return launch_dt<64>(p, a, s);
    case 128: return launch_dt<128>(p, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
