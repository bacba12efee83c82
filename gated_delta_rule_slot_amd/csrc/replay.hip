// replay.hip -- ReplaySSM: a draft-chain verify that records a ring of inputs
// instead of per-step states, and the exact-fold commit of the accepted prefix.
//
// Semantics (page "企业官网建设流程全解析", Kimi K3 notes, section "ReplaySSM"):
// the verify computes every draft position's output but keeps no per-position
// [V, K] state; it records what regenerates it (k as it leaves the conv, before
// L2 normalisation, and v, both bf16; the decay g and beta in fp32).  After
// acceptance only the accepted prefix is replayed, in recurrent order, and
// written back to the slot (page "SGLang之MambaRadixCache机制解析", section 9.10:
// with the track-interval check during the replay).  The ring also keeps each
// position's conv input row, so the commit can advance the conv state.
//
// The commit, and the verify of drafts longer than 8 tokens, use the decode
// kernel's lane layout (one workgroup per (request, head), a lane owns 16-byte
// pieces of K-contiguous state rows, row sums with DPP and row swaps) and keep
// the state in fp32 registers across the tokens: the verify reads the live state
// once and stores no state at all; the commit reads it once, folds every
// accepted token, and stores it once (and at a snapshot).  Drafts of up to 8
// tokens are verified in closed form on MFMA (see below).
#include "common.hpp"
#include "lanes.hpp"
#include "mfma.hpp"

namespace gdn {
namespace {

constexpr int kGroup = 8;  // tokens staged in shared memory at a time

template <int D, typename TS>
struct ReplayShape {
  static constexpr int VEC = StateVec<TS>::N;
  static constexpr int LPR = D / VEC;                        // lanes per row
  static constexpr int RPI = 64 / LPR;                       // rows per load instruction
  static constexpr int ROWS = RPI * 8 < D ? RPI * 8 : D;     // state rows per wave
  static constexpr int THREADS = 64 * (D / ROWS);
  static constexpr int ITERS = (ROWS + RPI - 1) / RPI;
  static constexpr bool FULL = ROWS % RPI == 0;              // every piece of every lane is a row
  // conv items of CW channels, one per thread
  static constexpr int CW = 3 * D / 2 <= THREADS ? 2 : 3 * D / 4 <= THREADS ? 4 : 8;
  static_assert(D <= THREADS, "one staging thread per channel");
};

// CW bf16 values packed for one store
template <int CW>
struct PackCW;
template <>
struct PackCW<2> {
  static __device__ __forceinline__ uint32_t pack(const float *v) { return pack_bf16x2(v[0], v[1]); }
};
template <>
struct PackCW<4> {
  static __device__ __forceinline__ u32x2 pack(const float *v) {
    return u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  }
};
template <>
struct PackCW<8> {
  static __device__ __forceinline__ u32x4 pack(const float *v) {
    return u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                 pack_bf16x2(v[6], v[7])};
  }
};

template <int D, typename TS, int kAlphaMode>
__global__ __launch_bounds__((ReplayShape<D, TS>::THREADS)) void replay_verify_kernel(
    const TS *__restrict__ ssm, const uint16_t *__restrict__ conv, int32_t *err, int slots,
    int heads, ReplayArgs a) {
  using SV = StateVec<TS>;
  using SH = ReplayShape<D, TS>;
  constexpr int VEC = SV::N, LPR = SH::LPR, RPI = SH::RPI, ROWS = SH::ROWS, ITERS = SH::ITERS;
  constexpr int CW = SH::CW, ITEMS = 3 * D / CW;
  static_assert(ITEMS <= SH::THREADS, "one conv item per thread");
  using CV = ConvVec<CW>;
  typedef typename CV::raw CR;

  const int h = blockIdx.x, b = blockIdx.y;
  const int T = a.draft, H = heads, P = a.ring.positions;
  const int lane = threadIdx.x & 63, part = threadIdx.x >> 6;
  const int64_t C = int64_t(H) * 3 * D;
  const int slot = a.slot_table[b];
  const int r0 = part * ROWS;
  const int64_t tok0 = int64_t(b) * T;

  if (slot <= 0 || slot >= slots) {
    for (int t = 0; t < T; ++t)
      if (lane < ROWS) a.out[((tok0 + t) * H + h) * D + r0 + lane] = 0;
    if (slot >= slots && err && h == 0 && threadIdx.x == 0) atomicOr(err, GDN_ERRW_BAD_SLOT);
    return;
  }

  // ---- the live state, once, into fp32 registers --------------------------
  const TS *S0 = ssm + ((int64_t(a.layer) * slots + slot) * H + h) * int64_t(D) * D;
  const int row_in_group = lane / LPR;
  const int col0 = (lane % LPR) * VEC;
  float s[ITERS][VEC];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int r = r0 + it * RPI + row_in_group;
#pragma unroll
    for (int e = 0; e < VEC; ++e) s[it][e] = 0.f;
    if (SH::FULL || r < r0 + ROWS)
      SV::to_f32(__builtin_nontemporal_load(reinterpret_cast<const typename SV::raw *>(S0 + int64_t(r) * D + col0)),
                 s[it]);
  }

  // ---- conv items and the ring rows of (layer, slot, head) ------------------
  const bool conv_lane = int(threadIdx.x) < ITEMS;
  const int item = conv_lane ? int(threadIdx.x) : 0;
  const int pt = item / (D / CW), jc = (item % (D / CW)) * CW;
  const int64_t ch = int64_t(pt) * H * D + int64_t(h) * D + jc;
  const uint16_t *crow = conv + (int64_t(a.layer) * slots + slot) * kConvRows * C;
  CR w0 = *reinterpret_cast<const CR *>(crow + ch);
  CR w1 = *reinterpret_cast<const CR *>(crow + C + ch);
  CR w2 = *reinterpret_cast<const CR *>(crow + 2 * C + ch);
  u32x4 wv[CW / 2];
  {
    const u32x4 *wp = reinterpret_cast<const u32x4 *>(a.conv_w + ch * 4);
#pragma unroll
    for (int i = 0; i < CW / 2; ++i) wv[i] = wp[i];
  }
  const int64_t rrow = ((int64_t(a.layer) * slots + slot) * H + h) * P;  // ring row of position 0
  uint16_t *rk = a.ring.rawk + rrow * D;
  uint16_t *rv = a.ring.rawv + rrow * D;
  float *rg = a.ring.g + rrow * (kAlphaMode == GDN_ALPHA_PER_CHANNEL ? D : 1);
  float *rb = a.ring.beta + rrow;
  uint16_t *rx = a.ring.xrow + (int64_t(a.layer) * slots + slot) * P * C;

  // Tokens go in groups of up to kGroup: the conv of every token of a group
  // (which needs no state) runs first and lands in shared memory with the
  // group's decays and betas, then one barrier, then the state updates follow
  // each other with nothing between them but the wave's own reductions.
  constexpr int NA = kAlphaMode == GDN_ALPHA_PER_CHANNEL ? D : 1;
  __shared__ __attribute__((aligned(16))) float sy[kGroup][3 * D];  // q | k | v per token
  __shared__ float sa[kGroup][NA];
  __shared__ float sb[kGroup];

  for (int t0 = 0; t0 < T; t0 += kGroup) {
    const int tn = T - t0 < kGroup ? T - t0 : kGroup;
    // ---- phase 1: conv, ring records, decays and betas of the group ---------
    CR xs[kGroup];
#pragma unroll
    for (int j = 0; j < kGroup; ++j)
      if (j < tn) xs[j] = *reinterpret_cast<const CR *>(a.x + (tok0 + t0 + j) * C + ch);
    for (int i = threadIdx.x; i < tn * NA; i += SH::THREADS) {
      const int j = i / NA, c = i % NA;
      const float v = a.alpha[((tok0 + t0 + j) * H + h) * NA + c];
      sa[j][c] = v;
      rg[(t0 + j) * NA + c] = v;
    }
    if (int(threadIdx.x) < tn) {
      const float v = a.beta[(tok0 + t0 + threadIdx.x) * H + h];
      sb[threadIdx.x] = v;
      rb[t0 + threadIdx.x] = v;
    }
    if (conv_lane) {
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        if (j >= tn) break;
        const int t = t0 + j;
        float yv[CW];
#pragma unroll
        for (int e = 0; e < CW; ++e) {
          const int sh = (e & 1) ? 16 : 0;
          auto pick = [&](const CR &v) {
            return __uint_as_float(((CV::word(v, e >> 1) >> sh) & 0xffffu) << 16);
          };
          const u32x4 &w = wv[e >> 1];
          const int wb = (e & 1) * 2;
          float acc = __uint_as_float(w[wb] << 16) * pick(w0);
          acc = fmaf(__uint_as_float(w[wb] & 0xffff0000u), pick(w1), acc);
          acc = fmaf(__uint_as_float(w[wb + 1] << 16), pick(w2), acc);
          acc = fmaf(__uint_as_float(w[wb + 1] & 0xffff0000u), pick(xs[j]), acc);
          if (a.flags & GDN_F_CONV_SILU) acc = acc / (1.f + __expf(-acc));
          yv[e] = acc;
          sy[j][pt * D + jc + e] = acc;
        }
        // the ring: k and v as they leave the conv (bf16), and the conv input row
        if (pt == 1) *reinterpret_cast<decltype(PackCW<CW>::pack(yv)) *>(rk + t * D + jc) = PackCW<CW>::pack(yv);
        if (pt == 2) *reinterpret_cast<decltype(PackCW<CW>::pack(yv)) *>(rv + t * D + jc) = PackCW<CW>::pack(yv);
        *reinterpret_cast<CR *>(rx + int64_t(t) * C + ch) = xs[j];
        w0 = w1;
        w1 = w2;
        w2 = xs[j];
      }
    }
    __syncthreads();

    // ---- phase 2: the group's state updates, back to back -------------------
    for (int j = 0; j < tn; ++j) {
      const float *sq = sy[j], *sk = sy[j] + D, *sv = sy[j] + 2 * D;
      float kinv = 1.f, qinv = 1.f;
      if (a.flags & GDN_F_L2NORM_K) {
        float ss = 0.f;
        for (int c = lane; c < D; c += 64) ss = fmaf(sk[c], sk[c], ss);
        kinv = 1.f / sqrtf(wave_sum(ss) + 1e-6f);
      }
      if (a.flags & GDN_F_L2NORM_Q) {
        float ss = 0.f;
        for (int c = lane; c < D; c += 64) ss = fmaf(sq[c], sq[c], ss);
        qinv = 1.f / sqrtf(wave_sum(ss) + 1e-6f);
      }
      float kq = 0.f;
      for (int c = lane; c < D; c += 64) kq = fmaf(sk[c] * kinv, sq[c] * qinv, kq);
      kq = wave_sum(kq);
      float kk[VEC], qq[VEC], al[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        kk[e] = sk[col0 + e] * kinv;
        qq[e] = sq[col0 + e] * qinv;
        al[e] = sa[j][NA == 1 ? 0 : col0 + e];
      }
      const float beta = sb[j];
      uint16_t *out = a.out + ((tok0 + t0 + j) * H + h) * D;
#pragma unroll
      for (int it = 0; it < ITERS; ++it) {
        const int r = r0 + it * RPI + row_in_group;
        float pu = 0.f, pq = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          s[it][e] *= al[e];
          pu = fmaf(s[it][e], kk[e], pu);
          pq = fmaf(s[it][e], qq[e], pq);
        }
        pu = group_sum<LPR>(pu);
        pq = group_sum<LPR>(pq);
        if (SH::FULL || r < r0 + ROWS) {
          const float d = beta * (sv[r] - pu);
#pragma unroll
          for (int e = 0; e < VEC; ++e) s[it][e] = fmaf(d, kk[e], s[it][e]);
          if ((lane % LPR) == 0) out[r] = f32_to_bf16(a.scale * fmaf(d, kq, pq));
        }
      }
    }
    __syncthreads();  // the group's shared inputs are read; the next group may overwrite them
  }
}

template <int D, typename TS, int kAlphaMode>
__global__ __launch_bounds__((ReplayShape<D, TS>::THREADS)) void replay_commit_kernel(
    TS *__restrict__ ssm, uint16_t *__restrict__ conv, int32_t *err, int slots, int heads,
    ReplayArgs a) {
  using SV = StateVec<TS>;
  using SH = ReplayShape<D, TS>;
  constexpr int VEC = SV::N, LPR = SH::LPR, RPI = SH::RPI, ROWS = SH::ROWS, ITERS = SH::ITERS;
  constexpr int CW = SH::CW, ITEMS = 3 * D / CW;
  using CV = ConvVec<CW>;
  typedef typename CV::raw CR;
  constexpr bool PERCH = kAlphaMode == GDN_ALPHA_PER_CHANNEL;

  // (request, head) from the launch index with each XCD given a contiguous run of
  // pairs, heads fastest, whose state blocks are adjacent in the pool (as in the
  // decode kernel; measured 2% faster here, and 2% slower for the verify kernels)
  int h, b;
  {
    const int n = int(gridDim.x) * int(gridDim.y), w = int(blockIdx.y * gridDim.x + blockIdx.x);
    const int q = n >> 3, rm = n & 7, x = w & 7, i = w >> 3;
    const int id = (x < rm ? x * (q + 1) : rm * (q + 1) + (x - rm) * q) + i;
    h = id % int(gridDim.x);
    b = id / int(gridDim.x);
  }
  const int H = heads, P = a.ring.positions;
  const int lane = threadIdx.x & 63, part = threadIdx.x >> 6;
  const int64_t C = int64_t(H) * 3 * D;
  const int n = a.accepted[b];
  if (n < 0 || n > P) {
    if (err && h == 0 && threadIdx.x == 0) atomicOr(err, GDN_ERRW_BAD_TREE);
    return;
  }
  const int slot = a.slot_table[b];
  if (slot <= 0 || slot >= slots) {
    if (slot >= slots && err && h == 0 && threadIdx.x == 0) atomicOr(err, GDN_ERRW_BAD_SLOT);
    return;
  }
  if (n == 0) return;

  // ---- the live state, once, into fp32 registers --------------------------
  const int64_t hd = int64_t(D) * D;
  auto state_block = [&](int sl) { return ssm + ((int64_t(a.layer) * slots + sl) * H + h) * hd; };
  const TS *S0 = state_block(slot);
  const int r0 = part * ROWS;
  const int row_in_group = lane / LPR;
  const int col0 = (lane % LPR) * VEC;
  float s[ITERS][VEC];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int r = r0 + it * RPI + row_in_group;
#pragma unroll
    for (int e = 0; e < VEC; ++e) s[it][e] = 0.f;
    if (SH::FULL || r < r0 + ROWS)
      SV::to_f32(__builtin_nontemporal_load(reinterpret_cast<const typename SV::raw *>(S0 + int64_t(r) * D + col0)),
                 s[it]);
  }

  // ---- conv rows of the head's channels -----------------------------------
  const bool conv_lane = int(threadIdx.x) < ITEMS;
  const int item = conv_lane ? int(threadIdx.x) : 0;
  const int pt = item / (D / CW), jc = (item % (D / CW)) * CW;
  const int64_t ch = int64_t(pt) * H * D + int64_t(h) * D + jc;
  auto conv_rows = [&](int sl) { return conv + (int64_t(a.layer) * slots + sl) * kConvRows * C; };
  const uint16_t *crow = conv_rows(slot);
  CR c0 = *reinterpret_cast<const CR *>(crow + ch);
  CR c1 = *reinterpret_cast<const CR *>(crow + C + ch);
  CR c2 = *reinterpret_cast<const CR *>(crow + 2 * C + ch);

  // ---- the ring of (layer, slot, head) --------------------------------------
  const int64_t rrow = ((int64_t(a.layer) * slots + slot) * H + h) * P;
  const uint16_t *rk = a.ring.rawk + rrow * D;
  const uint16_t *rv = a.ring.rawv + rrow * D;
  const float *rg = a.ring.g + rrow * (PERCH ? D : 1);
  const float *rb = a.ring.beta + rrow;
  const uint16_t *rx = a.ring.xrow + (int64_t(a.layer) * slots + slot) * P * C;
  // staging: thread i < D holds channel i of a position's k, v (and g)
  const int ci = int(threadIdx.x) < D ? int(threadIdx.x) : 0;
  struct Pos {
    uint16_t k, v;
    float g;
    CR x;
  };
  auto load_pos = [&](int t) {
    Pos p;
    p.k = rk[t * D + ci];
    p.v = rv[t * D + ci];
    p.g = PERCH ? rg[t * D + ci] : 0.f;
    p.x = *reinterpret_cast<const CR *>(rx + int64_t(t) * C + ch);
    return p;
  };
  __shared__ float sk[2][D], svv[2][D], sg[2][D];
  Pos cur = load_pos(0);

  const bool track = a.track_interval > 0;
  const int64_t before = track ? a.seq_len_before[b] : 0;
  int crossings = 0;
  auto store_to = [&](int sl) {
    TS *dst = state_block(sl);
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int r = r0 + it * RPI + row_in_group;
      if (SH::FULL || r < r0 + ROWS)
        __builtin_nontemporal_store(SV::from_f32(s[it]),
                                    reinterpret_cast<typename SV::raw *>(dst + int64_t(r) * D + col0));
    }
    if (conv_lane) {
      uint16_t *cr = conv_rows(sl);
      *reinterpret_cast<CR *>(cr + ch) = c0;
      *reinterpret_cast<CR *>(cr + C + ch) = c1;
      *reinterpret_cast<CR *>(cr + 2 * C + ch) = c2;
    }
  };

  for (int t = 0; t < n; ++t) {
    const int buf = t & 1;
    if (int(threadIdx.x) < D) {
      sk[buf][ci] = __uint_as_float(uint32_t(cur.k) << 16);
      svv[buf][ci] = __uint_as_float(uint32_t(cur.v) << 16);
      if (PERCH) sg[buf][ci] = cur.g;
    }
    c0 = c1;
    c1 = c2;
    c2 = cur.x;
    const float gh = PERCH ? 0.f : rg[t];
    const float beta = rb[t];
    cur = load_pos(t + 1 < n ? t + 1 : t);  // the next position, ahead of the barrier
    __syncthreads();

    const float *kr = sk[buf], *vr = svv[buf], *gr = sg[buf];
    float kinv = 1.f;
    if (a.flags & GDN_F_L2NORM_K) {
      float ss = 0.f;
      for (int j = lane; j < D; j += 64) ss = fmaf(kr[j], kr[j], ss);
      kinv = 1.f / sqrtf(wave_sum(ss) + 1e-6f);
    }
    float kk[VEC], gg[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      kk[e] = kr[col0 + e] * kinv;
      gg[e] = PERCH ? gr[col0 + e] : gh;
    }
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int r = r0 + it * RPI + row_in_group;
      float pu = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        s[it][e] *= gg[e];
        pu = fmaf(s[it][e], kk[e], pu);
      }
      pu = group_sum<LPR>(pu);
      if (SH::FULL || r < r0 + ROWS) {
        const float d = beta * (vr[r] - pu);
#pragma unroll
        for (int e = 0; e < VEC; ++e) s[it][e] = fmaf(d, kk[e], s[it][e]);
      }
    }
    // a snapshot where the replayed length completes a multiple of the interval
    if (track && (before + t + 1) % a.track_interval == 0) {
      const int dst = a.track_slots[2 * b + ((a.next_track_idx[b] + crossings) & 1)];
      ++crossings;
      if (dst >= slots) {
        if (err && threadIdx.x == 0) atomicOr(err, GDN_ERRW_BAD_TRACK_SLOT);
      } else if (dst > 0) {
        store_to(dst);
      }
    }
  }
  store_to(slot);
}

// ------------------------------------------------------- verify on MFMA ----
// A draft of T <= 8 tokens needs no per-token pass over the state.  With
// Gam_t = prod_{s <= t} a_s and P(i, t) = prod_{i < s <= t} a_s (per channel), the
// state after token t is S0 Diag(Gam_t) + sum_{i <= t} d_i (k_i . P(i, t))^T, so
//     u_t = S0 (Gam_t . k_t) + sum_{i < t} A[t][i] d_i,    A[t][i] = sum_c k_i P(i, t) k_t
//     d_t = b_t (v_t - u_t)
//     o_t = scale (S0 (Gam_t . q_t) + sum_{i <= t} M[t][i] d_i),  M[t][i] = sum_c k_i P(i, t) q_t
// (k and q after their normalisation).  The 2T products with S0 are one
// [D x D] x [D x 2T] contraction per head on bf16 MFMA: the state as stored is
// the A operand (a bf16 state exactly; an fp32 state split hi/lo), the columns
// Gam_t . k_t and Gam_t . q_t are split hi/lo, so every product keeps about 16
// significant bits.  The T x T coefficients A and M come from per-channel sums,
// and each state row then solves its own T-step triangular recurrence for d.
// Measured on MI355X (KDA pool, 12 heads, batch 256): 4 tokens 53.9 -> 33 us,
// 8 tokens 87 -> 48 us, 1 token 28.6 -> 25 us against the token-by-token kernel;
// at 16 tokens the token-by-token kernel was faster, so longer drafts run there.
template <int D>
struct MmaShape {
  static constexpr int RB = D / 16;               // 16-row blocks of the state
  static constexpr int KS = D / 32;               // 32-channel k slabs
  static constexpr int WAVES = RB < 4 ? RB : 4;
  static constexpr int RBW = RB / WAVES;          // row blocks per wave
  static constexpr int ROWS = 16 * RBW;           // state rows per wave
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int CL = D < 64 ? D : 64;      // lanes holding channels in the per-channel steps
  static constexpr int CPL = D / CL;              // channels per such lane
};

template <int D, typename TS, int kAlphaMode, int TMAX>
__global__ __launch_bounds__((MmaShape<D>::THREADS)) void replay_verify_mma_kernel(
    const TS *__restrict__ ssm, const uint16_t *__restrict__ conv, int32_t *err, int slots,
    int heads, ReplayArgs a) {
  using SH = MmaShape<D>;
  constexpr int RBW = SH::RBW, KS = SH::KS, ROWS = SH::ROWS;
  constexpr int NCOL = 2 * TMAX, NT = (NCOL + 15) / 16;  // columns: Gam.k of every token, then Gam.q
  constexpr int HALF = D / 2;                            // two-channel conv items per part (q, k, v)
  constexpr int ITEMS = 3 * HALF;
  constexpr bool PERCH = kAlphaMode == GDN_ALPHA_PER_CHANNEL;
  constexpr int NA = PERCH ? D : 1;
  constexpr int PIECES = sizeof(TS) / 2;                 // 16-byte loads per 8 state values
  static_assert(D % 32 == 0 && ITEMS <= SH::THREADS && SH::WAVES >= 2, "shape");
  static_assert(HALF <= 64 && 64 % HALF == 0, "a part's conv items lie within one wave");

  const int h = blockIdx.x, b = blockIdx.y;
  const int T = a.draft, H = heads, P = a.ring.positions;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t C = int64_t(H) * 3 * D;
  const int slot = a.slot_table[b];
  const int rw0 = wv * ROWS;  // first state row of this wave
  const int64_t tok0 = int64_t(b) * T;

  if (slot <= 0 || slot >= slots) {
    for (int t = 0; t < T; ++t)
      if (lane < ROWS) a.out[((tok0 + t) * H + h) * D + rw0 + lane] = 0;
    if (slot >= slots && err && h == 0 && threadIdx.x == 0) atomicOr(err, GDN_ERRW_BAD_SLOT);
    return;
  }

  // ---- loads: the small inputs of phase 1 first, then the state ------------
  // Loads complete in issue order, so phase 1 (conv, decays, betas) and phase 2
  // run while the state blocks are still streaming in.
  constexpr int AL = (TMAX * NA + SH::THREADS - 1) / SH::THREADS;  // decays per thread
  float av[AL];
#pragma unroll
  for (int k = 0; k < AL; ++k) {
    const int i = int(threadIdx.x) + k * SH::THREADS;
    av[k] = i < T * NA ? a.alpha[((tok0 + i / NA) * H + h) * NA + i % NA] : 0.f;
  }
  const float bv = int(threadIdx.x) < T ? a.beta[(tok0 + threadIdx.x) * H + h] : 0.f;
  const bool conv_lane = int(threadIdx.x) < ITEMS;
  const int item = conv_lane ? int(threadIdx.x) : 0;
  const int pt = item / HALF, jc = (item % HALF) * 2;
  const int64_t ch = int64_t(pt) * H * D + int64_t(h) * D + jc;
  const uint16_t *crow = conv + (int64_t(a.layer) * slots + slot) * kConvRows * C;
  uint32_t w0 = *reinterpret_cast<const uint32_t *>(crow + ch);
  uint32_t w1 = *reinterpret_cast<const uint32_t *>(crow + C + ch);
  uint32_t w2 = *reinterpret_cast<const uint32_t *>(crow + 2 * C + ch);
  const u32x4 wt = *reinterpret_cast<const u32x4 *>(a.conv_w + ch * 4);  // taps of channels jc, jc+1
  uint32_t xs[TMAX];
#pragma unroll
  for (int j = 0; j < TMAX; ++j)
    if (j < T) xs[j] = *reinterpret_cast<const uint32_t *>(a.x + (tok0 + j) * C + ch);

  // the live state as MFMA A operands: row block rb, slab ks: lane l holds row
  // rw0 + 16 rb + l % 16, channels 32 ks + 8 (l / 16) + e, e < 8
  const TS *S0 = ssm + ((int64_t(a.layer) * slots + slot) * H + h) * int64_t(D) * D;
  const int fr = lane & 15, fg = lane >> 4;
  u32x4 st[RBW][KS][PIECES];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 *src = reinterpret_cast<const u32x4 *>(S0 + int64_t(rw0 + 16 * rb + fr) * D + 32 * ks + 8 * fg);
#pragma unroll
      for (int q = 0; q < PIECES; ++q) st[rb][ks][q] = __builtin_nontemporal_load(src + q);
    }

  const int64_t rrow = ((int64_t(a.layer) * slots + slot) * H + h) * P;  // ring row of position 0
  uint16_t *rk = a.ring.rawk + rrow * D;
  uint16_t *rv = a.ring.rawv + rrow * D;
  float *rg = a.ring.g + rrow * NA;
  float *rbt = a.ring.beta + rrow;
  uint16_t *rx = a.ring.xrow + (int64_t(a.layer) * slots + slot) * P * C;

  __shared__ __attribute__((aligned(16))) float sy[TMAX][3 * D];  // q | k | v per token
  __shared__ float sal[TMAX][NA];
  __shared__ float sbe[TMAX];
  __shared__ float sinv[TMAX][2];  // 1 / |q|, 1 / |k| (1 where the norm is off)
  __shared__ __attribute__((aligned(16))) u32x4 sB[NT][KS][2][64]; // B operands, hi | lo
  __shared__ float sC[D][NCOL + 1];
  __shared__ float sA[TMAX][TMAX], sM[TMAX][TMAX];

  // ---- phase 1: conv of every token, ring records, decays and betas ---------
#pragma unroll
  for (int k = 0; k < AL; ++k) {
    const int i = int(threadIdx.x) + k * SH::THREADS;
    if (i < T * NA) sal[i / NA][i % NA] = av[k];
  }
  if (int(threadIdx.x) < T) sbe[threadIdx.x] = bv;
#pragma unroll
  for (int j = 0; j < TMAX; ++j) {
    if (j >= T) break;
    float y[2] = {0.f, 0.f};
    if (conv_lane) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int sh = e ? 16 : 0;
        auto pick = [&](uint32_t v) { return __uint_as_float(((v >> sh) & 0xffffu) << 16); };
        float acc = __uint_as_float(wt[2 * e] << 16) * pick(w0);
        acc = fmaf(__uint_as_float(wt[2 * e] & 0xffff0000u), pick(w1), acc);
        acc = fmaf(__uint_as_float(wt[2 * e + 1] << 16), pick(w2), acc);
        acc = fmaf(__uint_as_float(wt[2 * e + 1] & 0xffff0000u), pick(xs[j]), acc);
        if (a.flags & GDN_F_CONV_SILU) acc = acc / (1.f + __expf(-acc));
        y[e] = acc;
        sy[j][pt * D + jc + e] = acc;
      }
      w0 = w1;
      w1 = w2;
      w2 = xs[j];
    }
    // inverse norms of q and k (a part's items are HALF adjacent lanes of one wave)
    float ss = conv_lane && pt < 2 ? fmaf(y[0], y[0], y[1] * y[1]) : 0.f;
    ss = group_sum<HALF>(ss);
    if (conv_lane && pt < 2 && (item % HALF) == 0) {
      const bool on = (a.flags & (pt == 0 ? GDN_F_L2NORM_Q : GDN_F_L2NORM_K)) != 0;
      sinv[j][pt] = on ? 1.f / sqrtf(ss + 1e-6f) : 1.f;
    }
  }
  __syncthreads();

  // ---- phase 2: B operands and the T x T coefficients ------------------------
  // B operands: thread c < D takes channel c.  Column t is Gam_t . k_t, column
  // TMAX + t is Gam_t . q_t (zero for t >= T); channel c sits in slab c / 32 at lane
  // 16 ((c / 8) % 4) + column % 16, element c % 8.
  if (int(threadIdx.x) < D) {
    const int c = threadIdx.x;
    const int ks = c >> 5, g = (c >> 3) & 3, e = c & 7;
    float gam = 1.f;
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      float xk = 0.f, xq = 0.f;
      if (t < T) {
        gam *= sal[t][PERCH ? c : 0];
        xk = gam * (sy[t][D + c] * sinv[t][1]);
        xq = gam * (sy[t][c] * sinv[t][0]);
      }
      const Split2 sp = split2(xk, xq);
      const int nk = t, nq = TMAX + t;
      reinterpret_cast<uint16_t *>(&sB[nk / 16][ks][0][16 * g + nk % 16])[e] = uint16_t(sp.hi);
      reinterpret_cast<uint16_t *>(&sB[nk / 16][ks][1][16 * g + nk % 16])[e] = uint16_t(sp.lo);
      reinterpret_cast<uint16_t *>(&sB[nq / 16][ks][0][16 * g + nq % 16])[e] = uint16_t(sp.hi >> 16);
      reinterpret_cast<uint16_t *>(&sB[nq / 16][ks][1][16 * g + nq % 16])[e] = uint16_t(sp.lo >> 16);
    }
  }
  // columns 2 TMAX .. 15 of the last tile (TMAX = 4) are zero
  if constexpr (NT * 16 > NCOL) {
    if (wv == SH::WAVES - 1) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        if ((lane & 15) >= NCOL % 16) sB[NT - 1][ks][0][lane] = sB[NT - 1][ks][1][lane] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  // A[t][i] (i < t) and M[t][i] (i <= t): the 32 lanes of group i (thread 32 i + l)
  // take channels l, l + 32, ... (D / 32 of them; adjacent lanes read adjacent
  // words), carry P(i, t) along t and sum each t's products over the group; the
  // norm factors multiply the sums.
  constexpr int CB = D / 32;
  static_assert(TMAX % 2 == 0, "whole waves of coefficient groups (uniform trip counts)");
  for (int u = threadIdx.x; u < 32 * TMAX; u += SH::THREADS) {
    const int i = u >> 5, cl = u & 31;
    const bool row = i < T;
    float ki[CB], pr[CB];
#pragma unroll
    for (int m = 0; m < CB; ++m) {
      ki[m] = row ? sy[i][D + cl + 32 * m] : 0.f;
      pr[m] = 1.f;
    }
    const float kin = row ? sinv[i][1] : 0.f;
    for (int t = 0; t < T; ++t) {  // T is uniform: every lane takes part in the sums
      float pa = 0.f, pm = 0.f;
#pragma unroll
      for (int m = 0; m < CB; ++m) {
        const int c = cl + 32 * m;
        if (t > i) pr[m] *= sal[t][PERCH ? c : 0];
        const float w = t >= i ? ki[m] * pr[m] : 0.f;
        pa = fmaf(w, sy[t][D + c], pa);
        pm = fmaf(w, sy[t][c], pm);
      }
      pa = group_sum<32>(pa);
      pm = group_sum<32>(pm);
      if (row && t >= i && cl == 0) {
        sA[t][i] = pa * kin * sinv[t][1];
        sM[t][i] = pm * kin * sinv[t][0];
      }
    }
  }
  __syncthreads();

  // ---- phase 3: S0 times the 2 TMAX columns on MFMA -------------------------
  f32x4 acc[RBW][NT];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[rb][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    Split bop[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      bop[nt].hi = __builtin_bit_cast(bf16x8, sB[nt][ks][0][lane]);
      bop[nt].lo = __builtin_bit_cast(bf16x8, sB[nt][ks][1][lane]);
    }
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      if constexpr (PIECES == 1) {  // bf16 state: exact as an operand
        const bf16x8 av = __builtin_bit_cast(bf16x8, st[rb][ks][0]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          acc[rb][nt] = mfma_bf16(av, bop[nt].lo, acc[rb][nt]);
          acc[rb][nt] = mfma_bf16(av, bop[nt].hi, acc[rb][nt]);
        }
      } else {  // fp32 state: split hi/lo
        float v[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = __uint_as_float(st[rb][ks][0][e]);
          v[4 + e] = __uint_as_float(st[rb][ks][1][e]);
        }
        const Split av = split8(v);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[rb][nt] = mfma3(av, bop[nt], acc[rb][nt]);
      }
    }
  }
  // accumulator tile (rb, nt): lane l holds column 16 nt + l % 16, rows 4 (l / 16) + j
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = 16 * nt + fr;
      if (n < NCOL) {
#pragma unroll
        for (int j = 0; j < 4; ++j) sC[rw0 + 16 * rb + 4 * fg + j][n] = acc[rb][nt][j];
      }
    }
  __syncthreads();

  // ---- the ring (stored only now: loads and stores retire in one order, so a
  // store ahead of the MFMA phase would make it wait for the whole state) ----
  //   k and v as they leave the conv (bf16), the conv input rows, decays, betas
#pragma unroll
  for (int j = 0; j < TMAX; ++j) {
    if (j >= T) break;
    if (conv_lane) {
      if (pt == 1) *reinterpret_cast<uint32_t *>(rk + j * D + jc) = pack_bf16x2(sy[j][D + jc], sy[j][D + jc + 1]);
      if (pt == 2) *reinterpret_cast<uint32_t *>(rv + j * D + jc) = pack_bf16x2(sy[j][2 * D + jc], sy[j][2 * D + jc + 1]);
      *reinterpret_cast<uint32_t *>(rx + int64_t(j) * C + ch) = xs[j];
    }
  }
#pragma unroll
  for (int k = 0; k < AL; ++k) {
    const int i = int(threadIdx.x) + k * SH::THREADS;
    if (i < T * NA) rg[i] = av[k];
  }
  if (int(threadIdx.x) < T) rbt[threadIdx.x] = bv;

  // ---- phase 4: each state row's T-step recurrence, outputs ----------------
  if (lane < ROWS) {
    const int r = rw0 + lane;
    float d[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      if (t >= T) break;
      float u = sC[r][t];
#pragma unroll
      for (int i = 0; i < t; ++i) u = fmaf(sA[t][i], d[i], u);
      d[t] = sbe[t] * (sy[t][2 * D + r] - u);
      float o = sC[r][TMAX + t];
#pragma unroll
      for (int i = 0; i <= t; ++i) o = fmaf(sM[t][i], d[i], o);
      a.out[((tok0 + t) * H + h) * D + r] = f32_to_bf16(a.scale * o);
    }
  }
}

template <int D, typename TS, int TMAX>
void launch_verify_mma(const gdn_pool *p, const ReplayArgs &a, hipStream_t s) {
  const dim3 grid(p->d.heads, a.batch), block(MmaShape<D>::THREADS);
  const TS *ssm = static_cast<const TS *>(p->d.ssm_base);
  const uint16_t *conv = static_cast<const uint16_t *>(p->d.conv_base);
  if (a.ring.alpha_mode == GDN_ALPHA_PER_CHANNEL)
    hipLaunchKernelGGL((replay_verify_mma_kernel<D, TS, GDN_ALPHA_PER_CHANNEL, TMAX>), grid, block, 0, s, ssm,
                       conv, p->d.err_word, p->d.slots, p->d.heads, a);
  else
    hipLaunchKernelGGL((replay_verify_mma_kernel<D, TS, GDN_ALPHA_PER_HEAD, TMAX>), grid, block, 0, s, ssm, conv,
                       p->d.err_word, p->d.slots, p->d.heads, a);
}

template <int D, typename TS, bool kVerify>
hipError_t launch_r(const gdn_pool *p, const ReplayArgs &a, hipStream_t s) {
  using SH = ReplayShape<D, TS>;
  dim3 grid(p->d.heads, a.batch);
  TS *ssm = static_cast<TS *>(p->d.ssm_base);
  uint16_t *conv = static_cast<uint16_t *>(p->d.conv_base);
  const bool pc = a.ring.alpha_mode == GDN_ALPHA_PER_CHANNEL;
  if (kVerify) {
    if constexpr (D >= 32) {  // drafts of up to 8 tokens: the MFMA form
      if (a.draft <= 8) {
        if (a.draft <= 4) launch_verify_mma<D, TS, 4>(p, a, s);
        else launch_verify_mma<D, TS, 8>(p, a, s);
        return hipGetLastError();
      }
    }
    if (pc)
      hipLaunchKernelGGL((replay_verify_kernel<D, TS, GDN_ALPHA_PER_CHANNEL>), grid, dim3(SH::THREADS), 0, s,
                         ssm, conv, p->d.err_word, p->d.slots, p->d.heads, a);
    else
      hipLaunchKernelGGL((replay_verify_kernel<D, TS, GDN_ALPHA_PER_HEAD>), grid, dim3(SH::THREADS), 0, s,
                         ssm, conv, p->d.err_word, p->d.slots, p->d.heads, a);
  } else {
    if (pc)
      hipLaunchKernelGGL((replay_commit_kernel<D, TS, GDN_ALPHA_PER_CHANNEL>), grid, dim3(SH::THREADS), 0, s,
                         ssm, conv, p->d.err_word, p->d.slots, p->d.heads, a);
    else
      hipLaunchKernelGGL((replay_commit_kernel<D, TS, GDN_ALPHA_PER_HEAD>), grid, dim3(SH::THREADS), 0, s,
                         ssm, conv, p->d.err_word, p->d.slots, p->d.heads, a);
  }
  return hipGetLastError();
}

template <bool kVerify>
hipError_t launch_any(const gdn_pool *p, const ReplayArgs &a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  const bool f32 = p->d.ssm_dtype == GDN_F32;
  switch (p->d.head_k) {
    case 16: return f32 ? launch_r<16, float, kVerify>(p, a, s) : launch_r<16, uint16_t, kVerify>(p, a, s);
    case 32: return f32 ? launch_r<32, float, kVerify>(p, a, s) : launch_r<32, uint16_t, kVerify>(p, a, s);
    case 64: return f32 ? launch_r<64, float, kVerify>(p, a, s) : launch_r<64, uint16_t, kVerify>(p, a, s);
    case 128: return f32 ? launch_r<128, float, kVerify>(p, a, s) : launch_r<128, uint16_t, kVerify>(p, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_replay_verify(const gdn_pool *p, const ReplayArgs &a, hipStream_t s) {
  return launch_any<true>(p, a, s);
}
hipError_t launch_replay_commit(const gdn_pool *p, const ReplayArgs &a, hipStream_t s) {
  return launch_any<false>(p, a, s);
}

}  // namespace gdn
