// decode.hip -- one decode token per request; per (request, head) one workgroup
// whose waves each own a few state rows.
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
// loaded before the conv prologue runs, so the HBM reads overlap with it; the
// state is streamed with non-temporal loads and stores (it is not reused).
#include "common.hpp"
#include "lanes.hpp"

namespace gdn {
namespace {

// One workgroup per (request, head); each of its waves owns ROWS state rows.  The head's conv is split across the waves into shared memory;
// after the single barrier every wave has what it needs, writes back its own
// slice of the conv rows (all old rows were read before the barrier) and runs
// its rows to completion on its own (norms are recomputed per wave).
// Rows per wave: 16-byte vectors per lane.  Measured on MI355X for this in-place
// read-modify-write stream: fp32 state, 8 beat 4 (1024-thread workgroups) and 16;
// bf16 state (KDA pool, 12 heads), 4 (8-wave workgroups, 71 VGPRs) beat 8 by 2.5%
// and 16 by 5%.
template <typename TS>
constexpr int kIters = sizeof(TS) == 4 ? 8 : 4;
template <int D, typename TS>
struct DecodeShape {
  static constexpr int VEC = StateVec<TS>::N;
  static constexpr int LPR = D / VEC;                         // lanes per row
  static constexpr int RPI = 64 / LPR;                        // rows per load instruction
  static constexpr int ROWS = RPI * kIters<TS> < D ? RPI * kIters<TS> : D;  // state rows per wave
  static constexpr int THREADS = 64 * (D / ROWS);
  // fp32 state: 8-wave workgroups; capping registers at 6 waves per SIMD (80 VGPRs,
  // no spills) fits a third workgroup per CU, i.e. more state loads in flight
  static constexpr int WAVES_PER_EU = sizeof(TS) == 4 ? 6 : 1;
};

template <int D, typename TS, int kAlphaMode>
__global__ __launch_bounds__((DecodeShape<D, TS>::THREADS))
__attribute__((amdgpu_waves_per_eu(DecodeShape<D, TS>::WAVES_PER_EU))) void gdn_decode_kernel(
    TS *__restrict__ ssm, uint16_t *__restrict__ conv, int32_t *err, int slots, int heads,
    DecodeArgs a) {
  using SV = StateVec<TS>;
  using SH = DecodeShape<D, TS>;
  constexpr int VEC = SV::N;
  constexpr int ROWS = SH::ROWS;          // state rows per wave
  constexpr int LPR = SH::LPR;            // lanes per row
  constexpr int RPI = SH::RPI;            // rows per load instruction
  constexpr int ITERS = (ROWS + RPI - 1) / RPI;
  // conv items of CW channels: the narrowest width that still gives every item its
  // own thread, which keeps the conv's registers (live while the state loads are in
  // flight) few enough for more workgroups per CU
  constexpr int CW = 3 * D / 2 <= SH::THREADS ? 2 : 3 * D / 4 <= SH::THREADS ? 4 : 8;
  static_assert(3 * D / CW <= SH::THREADS, "one conv item per thread");
  constexpr int ITEMS = 3 * D / CW;       // CW-channel conv items of the head
  using CV = ConvVec<CW>;
  static_assert(LPR >= 1 && LPR <= 64 && (64 % LPR) == 0, "row layout");

  // workgroup -> (request, head), with consecutive heads kept on one XCD: the
  // workgroups of a launch are dealt to the 8 XCDs in turn (XCD x runs w = x, x+8,
  // ...), so each XCD is given its own contiguous run of (request, head) pairs,
  // whose state blocks are adjacent in the pool.  Measured on MI355X: 2% faster for
  // the bf16 state (32 KB per head), 0.5% for fp32.
  const int nwg = heads * a.batch;
  int w = blockIdx.x;
  {
    const int q = nwg >> 3, rm = nwg & 7, x = w & 7, i = w >> 3;
    w = (x < rm ? x * (q + 1) : rm * (q + 1) + (x - rm) * q) + i;
  }
  const int h = w % heads, b = w / heads;
  const int lane = threadIdx.x & 63, part = threadIdx.x >> 6;
  const int H = heads;
  const int64_t C = int64_t(H) * 3 * D;
  const int slot = a.slot_table[b];
  const int r0 = part * ROWS;
  uint16_t *out = a.out + (int64_t(b) * H + h) * D + r0;

  if (slot <= 0 || slot >= slots) {
    if (lane < ROWS) out[lane] = 0;
    if (slot >= slots && err && threadIdx.x == 0) atomicOr(err, GDN_ERRW_BAD_SLOT);
    return;
  }

  // ---- issue the state loads first ------------------------------------
  TS *Sblk = ssm + ((int64_t(a.layer) * slots + slot) * H + h) * int64_t(D) * D;
  const int row_in_group = lane / LPR;
  const int col0 = (lane % LPR) * VEC;
  typename SV::raw sraw[ITERS];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int r = r0 + it * RPI + row_in_group;
    if (r < r0 + ROWS)
      sraw[it] = __builtin_nontemporal_load(
          reinterpret_cast<const typename SV::raw *>(Sblk + int64_t(r) * D + col0));
  }

  // ---- conv over the head's q, k, v channels, CW channels per lane -------
  __shared__ __attribute__((aligned(16))) float sy[3 * D];  // q | k | v of this head
  uint16_t *crow = conv + (int64_t(a.layer) * slots + slot) * kConvRows * C;
  const uint16_t *xb = a.x + int64_t(b) * C;
  const int item = threadIdx.x;  // one CW-channel item per thread (ITEMS <= threads)
  const bool conv_lane = item < ITEMS;
  const int pt = item / (D / CW), jc = (item % (D / CW)) * CW;
  const int64_t ch = int64_t(pt) * H * D + int64_t(h) * D + jc;
  typename CV::raw r0v, r1v, r2v, xv;
  u32x4 wv[CW / 2];  // weights [C][4]: the 4 taps of channels 2i and 2i+1 make up wv[i]
  if (conv_lane) {  // issued right behind the state loads, before anything waits
    r0v = *reinterpret_cast<const typename CV::raw *>(crow + ch);
    r1v = *reinterpret_cast<const typename CV::raw *>(crow + C + ch);
    r2v = *reinterpret_cast<const typename CV::raw *>(crow + 2 * C + ch);
    xv = *reinterpret_cast<const typename CV::raw *>(xb + ch);
    const u32x4 *wp = reinterpret_cast<const u32x4 *>(a.conv_w + ch * 4);
#pragma unroll
    for (int i = 0; i < CW / 2; ++i) wv[i] = wp[i];
  }

  // decay of this lane's columns and beta: loaded here, not behind the barrier
  float al[VEC];
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

  // ---- snapshot target --------------------------------------------------
  int track = 0;
  if (a.track_interval > 0 && a.track_slots && a.seq_len_after[b] % a.track_interval == 0) {
    track = a.track_slots[2 * b + (a.next_track_idx[b] & 1)];
    if (track >= slots) {
      if (err && threadIdx.x == 0) atomicOr(err, GDN_ERRW_BAD_TRACK_SLOT);
      track = 0;
    }
  }
  uint16_t *trow = track > 0 ? conv + (int64_t(a.layer) * slots + track) * kConvRows * C : nullptr;

  if (conv_lane) {
#pragma unroll
    for (int e = 0; e < CW; ++e) {
      const int sh = (e & 1) ? 16 : 0;
      auto pick = [&](const typename CV::raw &v) {
        return __uint_as_float(((CV::word(v, e >> 1) >> sh) & 0xffffu) << 16);
      };
      const u32x4 &w2 = wv[e >> 1];
      const int wb = (e & 1) * 2;
      float y = __uint_as_float(w2[wb] << 16) * pick(r0v);
      y = fmaf(__uint_as_float(w2[wb] & 0xffff0000u), pick(r1v), y);
      y = fmaf(__uint_as_float(w2[wb + 1] << 16), pick(r2v), y);
      y = fmaf(__uint_as_float(w2[wb + 1] & 0xffff0000u), pick(xv), y);
      if (a.flags & GDN_F_CONV_SILU) y = y / (1.f + __expf(-y));
      sy[pt * D + jc + e] = y;
    }
  }
  __syncthreads();  // every old conv row has been read; sy is complete
  if (conv_lane) {
    typedef typename CV::raw R;
    *reinterpret_cast<R *>(crow + ch) = r1v;
    *reinterpret_cast<R *>(crow + C + ch) = r2v;
    *reinterpret_cast<R *>(crow + 2 * C + ch) = xv;
    if (trow) {
      *reinterpret_cast<R *>(trow + ch) = r1v;
      *reinterpret_cast<R *>(trow + C + ch) = r2v;
      *reinterpret_cast<R *>(trow + 2 * C + ch) = xv;
    }
  }
  const float *sq = sy, *sk = sy + D, *sv = sy + 2 * D;

  // ---- normalisation and k.q (wave reductions) ---------------------------
  float kinv = 1.f, qinv = 1.f;
  if (a.flags & GDN_F_L2NORM_K) {
    float ss = 0.f;
    for (int i = lane; i < D; i += 64) ss = fmaf(sk[i], sk[i], ss);
    kinv = 1.f / sqrtf(wave_sum(ss) + 1e-6f);
  }
  if (a.flags & GDN_F_L2NORM_Q) {
    float ss = 0.f;
    for (int i = lane; i < D; i += 64) ss = fmaf(sq[i], sq[i], ss);
    qinv = 1.f / sqrtf(wave_sum(ss) + 1e-6f);
  }
  float kq = 0.f;
  for (int i = lane; i < D; i += 64) kq = fmaf(sk[i] * kinv, sq[i] * qinv, kq);
  kq = wave_sum(kq);

  float kk[VEC], qq[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    kk[e] = sk[col0 + e] * kinv;
    qq[e] = sq[col0 + e] * qinv;
  }
  TS *Tblk = track > 0 ? ssm + ((int64_t(a.layer) * slots + track) * H + h) * int64_t(D) * D : nullptr;

  // ---- the state stream --------------------------------------------------
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int r = r0 + it * RPI + row_in_group;
    const bool on = r < r0 + ROWS;  // uniform over the LPR lanes of a row
    float s[VEC];
    SV::to_f32(sraw[it], s);
    float pu = 0.f, pq = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      s[e] *= al[e];
      pu = fmaf(s[e], kk[e], pu);
      pq = fmaf(s[e], qq[e], pq);
    }
    pu = group_sum<LPR>(pu);
    pq = group_sum<LPR>(pq);
    if (on) {
      const float d = beta * (sv[r] - pu);
#pragma unroll
      for (int e = 0; e < VEC; ++e) s[e] = fmaf(d, kk[e], s[e]);
      const typename SV::raw w = SV::from_f32(s);
      __builtin_nontemporal_store(w, reinterpret_cast<typename SV::raw *>(Sblk + int64_t(r) * D + col0));
      if (Tblk)
        __builtin_nontemporal_store(w, reinterpret_cast<typename SV::raw *>(Tblk + int64_t(r) * D + col0));
      if ((lane % LPR) == 0) out[r - r0] = f32_to_bf16(a.scale * fmaf(d, kq, pq));
    }
  }
}

template <int D, typename TS>
hipError_t launch_d(const gdn_pool *p, const DecodeArgs &a, hipStream_t s) {
  constexpr int THREADS = DecodeShape<D, TS>::THREADS;
  dim3 grid(p->d.heads * a.batch);
  if (a.alpha_mode == GDN_ALPHA_PER_CHANNEL)
    hipLaunchKernelGGL((gdn_decode_kernel<D, TS, GDN_ALPHA_PER_CHANNEL>), grid, dim3(THREADS), 0, s,
                       static_cast<TS *>(p->d.ssm_base), static_cast<uint16_t *>(p->d.conv_base),
                       p->d.err_word, p->d.slots, p->d.heads, a);
  else
    hipLaunchKernelGGL((gdn_decode_kernel<D, TS, GDN_ALPHA_PER_HEAD>), grid, dim3(THREADS), 0, s,
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
