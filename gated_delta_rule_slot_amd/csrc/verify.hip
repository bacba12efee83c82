// verify.hip -- speculative verify of a draft tree: every node of the tree takes
// one token from its parent's state without touching the live slot.
//
// Semantics (page "SGLang之MambaRadixCache机制解析", section 8.3: the verify
// pass keeps the main state as it is and writes the result of each draft
// position into an intermediate buffer; section 9.6: retrieve_parent_token
// names each node's parent, -1 for the main state, and nodes are processed
// parent first).  Node n of request b:
//   window  = the parent's three conv rows and x_n (for a root: the live slot's
//             rows; deeper: the x rows of its nearest ancestors, topped up with
//             the live rows when the path is shorter than three)
//   S_n     = one step of the recurrence from S_parent (as stored in the pool
//             dtype), o_n = scale S_n q_n
//   stored  : node_ssm[b][n] (pool dtype), node_conv[b][n] = window rows 1..3,
//             out[b][n]
//
// Layout and work split.  A workgroup owns a block of state rows of one
// (request, head) and walks the tree's nodes in index order (a valid tree lists
// parents first).  Every lane owns the same 16-byte row pieces for every node,
// so a node's state is re-read only by the lane that stored it: in-order
// memory access within a lane makes that read see the store, and no barrier is
// needed for the state.  When a node's parent is the node just computed (a
// chain), the state stays in registers and only the stores go out.  The conv
// windows are built from x and the live rows alone, never from another
// workgroup's node buffers, so the row blocks of one head are independent;
// the block with the first rows writes the node conv rows.
#include "common.hpp"
#include "lanes.hpp"

namespace gdn {
namespace {

template <int D, typename TS>
struct VerifyShape {
  static constexpr int VEC = StateVec<TS>::N;
  static constexpr int LPR = D / VEC;                                 // lanes per row
  static constexpr int RPI = 64 / LPR;                                // rows per load instruction
  static constexpr int ROWS = RPI * 8 < D ? RPI * 8 : D;              // state rows per wave
  static constexpr int WAVES = D / ROWS < 4 ? D / ROWS : 4;           // waves per workgroup
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int SPLIT = D / (ROWS * WAVES);                    // workgroups per head
  static constexpr int CW = 3 * D / 2 <= THREADS ? 2 : 3 * D / 4 <= THREADS ? 4 : 8;
};

template <int D, typename TS, int kAlphaMode>
__global__ __launch_bounds__((VerifyShape<D, TS>::THREADS)) void gdn_verify_kernel(
    const TS *__restrict__ ssm, const uint16_t *__restrict__ conv, int32_t *err, int slots,
    int heads, VerifyArgs a) {
  using SV = StateVec<TS>;
  using SH = VerifyShape<D, TS>;
  constexpr int VEC = SV::N;
  constexpr int ROWS = SH::ROWS;
  constexpr int LPR = SH::LPR;
  constexpr int RPI = SH::RPI;
  constexpr int ITERS = (ROWS + RPI - 1) / RPI;
  constexpr int CW = SH::CW;
  constexpr int ITEMS = 3 * D / CW;
  static_assert(ITEMS <= SH::THREADS, "one conv item per thread");
  static_assert(LPR >= 1 && LPR <= 64 && (64 % LPR) == 0, "row layout");
  using CV = ConvVec<CW>;
  typedef typename CV::raw CR;
  typedef typename SV::raw SR;

  const int h = blockIdx.x, b = blockIdx.y, split = blockIdx.z;
  const int T = a.nodes;
  const int H = heads;
  const int64_t C = int64_t(H) * 3 * D;
  const int lane = threadIdx.x & 63, part = threadIdx.x >> 6;
  const int r0 = (split * SH::WAVES + part) * ROWS;
  const int slot = a.slot_table[b];
  const int64_t tok0 = int64_t(b) * T;  // node 0's row in x, alpha, beta and out

  __shared__ int spar[kMaxTreeNodes];
  __shared__ __attribute__((aligned(16))) float sy[2][3 * D];  // q | k | v, double buffered

  const int32_t *par = a.parent + tok0;
  int bad = 0;
  for (int i = threadIdx.x; i < T; i += SH::THREADS) {
    const int p = par[i];
    spar[i] = p;
    bad |= (p < -1 || p >= i);
  }
  bad = __syncthreads_or(bad);

  if (bad || slot <= 0 || slot >= slots) {
    for (int n = 0; n < T; ++n)
      if (lane < ROWS) a.out[((tok0 + n) * H + h) * D + r0 + lane] = 0;
    if (err && h == 0 && split == 0 && threadIdx.x == 0) {
      if (slot >= slots) atomicOr(err, GDN_ERRW_BAD_SLOT);
      if (bad) atomicOr(err, GDN_ERRW_BAD_TREE);
    }
    return;
  }

  // ---- node 0 reads the live state (a valid tree's first node is a root) ----
  const int64_t hd = int64_t(D) * D;
  const TS *live = ssm + ((int64_t(a.layer) * slots + slot) * H + h) * hd;
  TS *nodes = static_cast<TS *>(a.node_ssm) + (tok0 * H + h) * hd;
  const int64_t nstride = int64_t(H) * hd;
  const int row_in_group = lane / LPR;
  const int col0 = (lane % LPR) * VEC;
  SR cur[ITERS];
  auto load_state = [&](const TS *blk) {
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int r = r0 + it * RPI + row_in_group;
      if (r < r0 + ROWS) cur[it] = *reinterpret_cast<const SR *>(blk + int64_t(r) * D + col0);
    }
  };
  load_state(live);

  // ---- conv items: CW channels of the head's q | k | v per thread ------------
  const uint16_t *lconv = conv + (int64_t(a.layer) * slots + slot) * kConvRows * C;
  uint16_t *nconv = a.node_conv + tok0 * kConvRows * C;
  const int item = threadIdx.x;
  const bool conv_lane = item < ITEMS;
  const bool conv_writer = conv_lane && split == 0;
  const int pt = item / (D / CW), jc = (item % (D / CW)) * CW;
  const int64_t ch = int64_t(pt) * H * D + int64_t(h) * D + jc;
  CR w0v, w1v, w2v, xv;  // the window: three rows before the token, then the token
  u32x4 wv[CW / 2];      // taps [C][4]: channels 2i and 2i+1 make up wv[i]
  if (conv_lane) {
    w0v = *reinterpret_cast<const CR *>(lconv + ch);
    w1v = *reinterpret_cast<const CR *>(lconv + C + ch);
    w2v = *reinterpret_cast<const CR *>(lconv + 2 * C + ch);
    const u32x4 *wp = reinterpret_cast<const u32x4 *>(a.conv_w + ch * 4);
#pragma unroll
    for (int i = 0; i < CW / 2; ++i) wv[i] = wp[i];
  }
  // row j (0..2) of a window whose token follows node p: an ancestor's x, or
  // the live row once the path runs out
  auto window_row = [&](int p, int j) -> CR {
    int q = p;
    for (int s = j; s < 2 && q >= 0; ++s) q = spar[q];   // climb 2 - j steps
    if (q >= 0) return *reinterpret_cast<const CR *>(a.x + (tok0 + q) * C + ch);
    // the path reached the live state after `used` of its rows were x rows
    int used = 0;
    for (int qq = p; qq >= 0 && used < 3; qq = spar[qq]) ++used;
    return *reinterpret_cast<const CR *>(lconv + int64_t(j + used) * C + ch);
  };

  for (int n = 0; n < T; ++n) {
    const int64_t tok = tok0 + n;
    float *y = sy[n & 1];
    if (conv_lane) {
      xv = *reinterpret_cast<const CR *>(a.x + tok * C + ch);
#pragma unroll
      for (int e = 0; e < CW; ++e) {
        const int sh = (e & 1) ? 16 : 0;
        auto pick = [&](const CR &v) {
          return __uint_as_float(((CV::word(v, e >> 1) >> sh) & 0xffffu) << 16);
        };
        const u32x4 &w2 = wv[e >> 1];
        const int wb = (e & 1) * 2;
        float acc = __uint_as_float(w2[wb] << 16) * pick(w0v);
        acc = fmaf(__uint_as_float(w2[wb] & 0xffff0000u), pick(w1v), acc);
        acc = fmaf(__uint_as_float(w2[wb + 1] << 16), pick(w2v), acc);
        acc = fmaf(__uint_as_float(w2[wb + 1] & 0xffff0000u), pick(xv), acc);
        if (a.flags & GDN_F_CONV_SILU) acc = acc / (1.f + __expf(-acc));
        y[pt * D + jc + e] = acc;
      }
      if (conv_writer) {
        uint16_t *dst = nconv + int64_t(n) * kConvRows * C;
        *reinterpret_cast<CR *>(dst + ch) = w1v;
        *reinterpret_cast<CR *>(dst + C + ch) = w2v;
        *reinterpret_cast<CR *>(dst + 2 * C + ch) = xv;
      }
    }
    float al[VEC];
    if (kAlphaMode == GDN_ALPHA_PER_CHANNEL) {
      const float *ap = a.alpha + (tok * H + h) * D + col0;
#pragma unroll
      for (int e = 0; e < VEC; ++e) al[e] = ap[e];
    } else {
      const float av = a.alpha[tok * H + h];
#pragma unroll
      for (int e = 0; e < VEC; ++e) al[e] = av;
    }
    const float beta = a.beta[tok * H + h];
    __syncthreads();  // y complete (the other buffer is free again for node n + 1)

    const float *sq = y, *sk = y + D, *sv = y + 2 * D;
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

    TS *dst = nodes + int64_t(n) * nstride;
    uint16_t *out = a.out + (tok * H + h) * D;
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int r = r0 + it * RPI + row_in_group;
      const bool on = r < r0 + ROWS;
      float s[VEC];
      SV::to_f32(cur[it], s);
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
        cur[it] = SV::from_f32(s);  // what the pool dtype holds: a child starts from this
        *reinterpret_cast<SR *>(dst + int64_t(r) * D + col0) = cur[it];
        if ((lane % LPR) == 0) out[r] = f32_to_bf16(a.scale * fmaf(d, kq, pq));
      }
    }

    // ---- the next node's parent: carried, or re-read -----------------------
    if (n + 1 < T) {
      const int p = spar[n + 1];
      if (p != n) {
        load_state(p < 0 ? live : nodes + int64_t(p) * nstride);
        if (conv_lane) {
          w0v = window_row(p, 0);
          w1v = window_row(p, 1);
          w2v = window_row(p, 2);
        }
      } else if (conv_lane) {
        w0v = w1v;
        w1v = w2v;
        w2v = xv;
      }
    }
  }
}

template <int D, typename TS>
hipError_t launch_v(const gdn_pool *p, const VerifyArgs &a, hipStream_t s) {
  using SH = VerifyShape<D, TS>;
  dim3 grid(p->d.heads, a.batch, SH::SPLIT);
  const TS *ssm = static_cast<const TS *>(p->d.ssm_base);
  const uint16_t *conv = static_cast<const uint16_t *>(p->d.conv_base);
  if (a.alpha_mode == GDN_ALPHA_PER_CHANNEL)
    hipLaunchKernelGGL((gdn_verify_kernel<D, TS, GDN_ALPHA_PER_CHANNEL>), grid, dim3(SH::THREADS),
                       0, s, ssm, conv, p->d.err_word, p->d.slots, p->d.heads, a);
  else
    hipLaunchKernelGGL((gdn_verify_kernel<D, TS, GDN_ALPHA_PER_HEAD>), grid, dim3(SH::THREADS), 0,
                       s, ssm, conv, p->d.err_word, p->d.slots, p->d.heads, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_vt(const gdn_pool *p, const VerifyArgs &a, hipStream_t s) {
  return p->d.ssm_dtype == GDN_F32 ? launch_v<D, float>(p, a, s) : launch_v<D, uint16_t>(p, a, s);
}

}  // namespace

hipError_t launch_verify(const gdn_pool *p, const VerifyArgs &a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  switch (p->d.head_k) {
    case 16: return launch_vt<16>(p, a, s);
    case 32: return launch_vt<32>(p, a, s);
    case 64: return launch_vt<64>(p, a, s);
    case 128: return launch_vt<128>(p, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
