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
// (request, head).  It visits the nodes depth first (preorder, children in index
// order), so every node's parent is either the node visited just before or one
// of its ancestors on the current path.  The parent state a node starts from
// comes from registers: the node just computed (carried over), or the kept state
// of the live slot or of the current depth-1 or depth-2 ancestor (a node of
// depth 1 or 2 that has children is kept when it is computed).  The only parents
// read from memory, besides the live state once, are ancestors deeper than 2
// that are not the node just computed.  Every lane owns the same 16-byte
// row pieces for every node, so a node's state is re-read only by the lane that
// stored it: in-order memory access within a lane makes that read see the
// store, and no barrier is needed for the state.  The conv windows are built from x and the
// live rows alone, never from another workgroup's node buffers, so the row
// blocks of one head are independent; the block with the first rows writes the
// node conv rows.
#include "common.hpp"
#include "lanes.hpp"

namespace gdn {
namespace {

template <int D, typename TS>
struct VerifyShape {
  static constexpr int VEC = StateVec<TS>::N;
  static constexpr int LPR = D / VEC;                                 // lanes per row
  static constexpr int RPI = 64 / LPR;                                // rows per load instruction
  // state rows per wave: up to 8 pieces per lane, and at least two waves per
  // head where the rows allow it
  static constexpr int HALF = D / 2 > RPI ? D / 2 : RPI;
  static constexpr int ROWS0 = RPI * 8 < HALF ? RPI * 8 : HALF;
  static constexpr int ROWS = ROWS0 < D ? ROWS0 : D;
  static constexpr int WAVES = D / ROWS < 4 ? D / ROWS : 4;           // waves per workgroup
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int SPLIT = D / (ROWS * WAVES);                    // workgroups per head
  static constexpr int CW = 3 * D / 2 <= THREADS ? 2 : 3 * D / 4 <= THREADS ? 4 : 8;
};

template <int D, typename TS, int kAlphaMode>
__global__ __launch_bounds__((VerifyShape<D, TS>::THREADS))
__attribute__((amdgpu_waves_per_eu(D == 128 ? 2 : 1))) void gdn_verify_kernel(
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

  // (request, head) from the launch index with each XCD given a contiguous run of
  // pairs, heads fastest: the node buffers of a request's heads are adjacent
  // (measured 1.5-2.5% faster on the 32-request, 63-node launch)
  int h, b;
  {
    const int n = int(gridDim.x) * int(gridDim.y), w = int(blockIdx.y * gridDim.x + blockIdx.x);
    const int q = n >> 3, rm = n & 7, x = w & 7, i = w >> 3;
    const int id = (x < rm ? x * (q + 1) : rm * (q + 1) + (x - rm) * q) + i;
    h = id % int(gridDim.x);
    b = id / int(gridDim.x);
  }
  const int split = blockIdx.z;
  const int T = a.nodes;
  const int H = heads;
  const int64_t C = int64_t(H) * 3 * D;
  const int lane = threadIdx.x & 63, part = threadIdx.x >> 6;
  const int r0 = (split * SH::WAVES + part) * ROWS;
  const int slot = a.slot_table[b];
  const int64_t tok0 = int64_t(b) * T;  // node 0's row in x, alpha, beta and out

  __shared__ int spar[kMaxTreeNodes];  // parent of each node
  __shared__ int sord[kMaxTreeNodes];  // nodes in visiting order: depth-first preorder
  __shared__ short sfirst[kMaxTreeNodes + 1], snext[kMaxTreeNodes], sdepth[kMaxTreeNodes];
  // per visiting position: {node, successor, successor's parent, flags}, see below
  __shared__ int4 splan[kMaxTreeNodes];
  __shared__ __attribute__((aligned(16))) float sy[2][3 * D];  // q | k | v, double buffered

  const int32_t *par = a.parent + tok0;
  int bad = 0;
  for (int i = threadIdx.x; i < T; i += SH::THREADS) {
    const int p = par[i];
    spar[i] = p;
    bad |= (p < -1 || p >= i);
  }
  bad = __syncthreads_or(bad);
  if (!bad) {
    // children lists in index order (entry T stands for the live state), then the
    // depth-first preorder by one thread (the tree has at most 1024 nodes)
    if (threadIdx.x == 0) {
      for (int n = 0; n <= T; ++n) sfirst[n] = -1;
      for (int n = T - 1; n >= 0; --n) {
        const int p = spar[n] < 0 ? T : spar[n];
        snext[n] = sfirst[p];
        sfirst[p] = short(n);
      }
      int n = sfirst[T], k = 0;
      while (n >= 0) {
        sord[k++] = n;
        sdepth[n] = short(spar[n] < 0 ? 1 : sdepth[spar[n]] + 1);
        if (sfirst[n] >= 0) {
          n = sfirst[n];
        } else {
          while (n >= 0 && snext[n] < 0) n = spar[n];
          if (n >= 0) n = snext[n];
        }
      }
    }
    __syncthreads();
    // The walk's plan, one entry per position i, so that a step reads its tree
    // facts with one shared-memory load instead of chasing parents:
    //   x: node n,  y: successor nn (n itself after the last node),
    //   z: nn's parent np (the state nn starts from),
    //   w: bits 0-1 used = x rows in nn's window (its nearest ancestors, up to 3),
    //      bits 2-11 np's parent, 12-21 np's grandparent (window rows 1 and 0),
    //      bit 22 carry (np is n), bit 23 load (np's state from np's node buffer),
    //      bits 24/25 take the kept depth-1 / depth-2 state, bits 26/27 keep n's
    //      state as the depth-1 / depth-2 one (n has children), bit 28 take the
    //      kept live state.
    for (int i = threadIdx.x; i < T; i += SH::THREADS) {
      const int n = sord[i];
      const bool last = i + 1 == T;
      const int nn = last ? n : sord[i + 1];
      const int np = last ? spar[n] : spar[nn];
      const int dn = sdepth[n], dp = np >= 0 ? sdepth[np] : 0;
      // a sibling successor starts from the parent state already in place
      const bool carry = !last && np == n, keep = !last && np == spar[n];
      const bool take0 = !last && !carry && !keep && dp == 0;
      const bool take1 = !last && !carry && !keep && dp == 1, take2 = !last && !carry && !keep && dp == 2;
      const bool load = !last && !carry && !keep && dp >= 3;
      const bool kids = sfirst[n] >= 0;
      const int a1 = np >= 0 ? spar[np] : -1;
      const int a2 = a1 >= 0 ? spar[a1] : -1;
      const int used = np < 0 ? 0 : a1 < 0 ? 1 : a2 < 0 ? 2 : 3;
      splan[i] = make_int4(n, nn, np, used | (max(a1, 0) << 2) | (max(a2, 0) << 12) |
                                          (int(carry) << 22) | (int(load) << 23) | (int(take1) << 24) |
                                          (int(take2) << 25) | (int(kids && dn == 1) << 26) |
                                          (int(kids && dn == 2) << 27) | (int(take0) << 28));
    }
    __syncthreads();
  }

  if (bad || slot <= 0 || slot >= slots) {
    for (int n = 0; n < T; ++n)
      if (lane < ROWS) a.out[((tok0 + n) * H + h) * D + r0 + lane] = 0;
    if (err && h == 0 && split == 0 && threadIdx.x == 0) {
      if (slot >= slots) atomicOr(err, GDN_ERRW_BAD_SLOT);
      if (bad) atomicOr(err, GDN_ERRW_BAD_TREE);
    }
    return;
  }

  // ---- the first group's parent is the live state (node 0 is a root) --------
  const int64_t hd = int64_t(D) * D;
  const TS *live = ssm + ((int64_t(a.layer) * slots + slot) * H + h) * hd;
  TS *nodes = static_cast<TS *>(a.node_ssm) + (tok0 * H + h) * hd;
  const int64_t nstride = int64_t(H) * hd;
  const int row_in_group = lane / LPR;
  const int col0 = (lane % LPR) * VEC;
  // State blocks are addressed through buffer resources: one 32-bit lane offset
  // plus a per-piece constant instead of a 64-bit address per piece.
  constexpr int kBlockBytes = D * D * int(sizeof(TS));
  constexpr int kPieceStep = RPI * D * int(sizeof(TS));  // bytes between a lane's pieces
  const int loff = ((r0 + row_in_group) * D + col0) * int(sizeof(TS));
  auto block = [&](const TS *base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<TS *>(base), 0, kBlockBytes, 0x00020000);
  };
  SR cur[ITERS];  // the parent state of the node being computed, in the pool dtype
  // the kept states of the live slot and of the current depth-1 and depth-2 ancestors
  SR keep0[ITERS], keep1[ITERS], keep2[ITERS];
  {
    const __amdgpu_buffer_rsrc_t lr = block(live);
#pragma unroll
    for (int it = 0; it < ITERS; ++it)
      if (ROWS % RPI == 0 || it * RPI + row_in_group < ROWS)
        cur[it] = __builtin_bit_cast(SR, __builtin_amdgcn_raw_buffer_load_b128(lr, loff, it * kPieceStep, 0));
#pragma unroll
    for (int it = 0; it < ITERS; ++it) keep0[it] = cur[it];
  }

  // ---- conv items: CW channels of the head's q | k | v per thread ------------
  const uint16_t *lconv = conv + (int64_t(a.layer) * slots + slot) * kConvRows * C;
  uint16_t *nconv = a.node_conv + tok0 * kConvRows * C;
  const bool conv_lane = int(threadIdx.x) < ITEMS;
  const bool conv_writer = conv_lane && split == 0;
  // lanes past the conv items still load item 0's x slice (unused), so that the
  // number of loads in flight does not depend on the lane
  const int item = conv_lane ? int(threadIdx.x) : 0;
  const int pt = item / (D / CW), jc = (item % (D / CW)) * CW;
  const int64_t ch = int64_t(pt) * H * D + int64_t(h) * D + jc;
  u32x4 wv[CW / 2];  // taps [C][4]: channels 2i and 2i+1 make up wv[i]
  if (conv_lane) {
    const u32x4 *wp = reinterpret_cast<const u32x4 *>(a.conv_w + ch * 4);
#pragma unroll
    for (int i = 0; i < CW / 2; ++i) wv[i] = wp[i];
  }
  // Row j (0..2) of a window whose last `used` rows are x rows of the nodes
  // q2 (row 2), q1 (row 1), q0 (row 0) and whose first rows are live rows:
  // one load from a selected (scalar) address.
  auto window_row = [&](int j, int used, int q0, int q1, int q2) -> CR {
    const int q = j == 0 ? q0 : j == 1 ? q1 : q2;
    const uint16_t *src = j >= 3 - used ? a.x + (tok0 + q) * C : lconv + int64_t(j + used) * C;
    return *reinterpret_cast<const CR *>(src + ch);
  };

  // What one node needs besides the parent state: the window rows (the parent's
  // conv rows), its x slice, the decay of this lane's columns and beta.  Two
  // sets alternate between consecutive nodes, so a successor's loads land in
  // registers of their own and nothing has to be copied (a copy would have to
  // wait for its load).
  constexpr int NAL = kAlphaMode == GDN_ALPHA_PER_CHANNEL ? VEC : 1;
  struct In {
    CR w0, w1, w2, x;
    float al[NAL];
    float beta;
  };
  auto load_inputs = [&](int node, In &o) {
    const int64_t tok = tok0 + node;
    o.x = *reinterpret_cast<const CR *>(a.x + tok * C + ch);
    if (kAlphaMode == GDN_ALPHA_PER_CHANNEL) {
      const float *ap = a.alpha + (tok * H + h) * D + col0;
#pragma unroll
      for (int e = 0; e < NAL; ++e) o.al[e] = ap[e];
    } else {
      o.al[0] = a.alpha[tok * H + h];
    }
    o.beta = a.beta[tok * H + h];
  };
  In in0, in1;
  in0.w0 = *reinterpret_cast<const CR *>(lconv + ch);
  in0.w1 = *reinterpret_cast<const CR *>(lconv + C + ch);
  in0.w2 = *reinterpret_cast<const CR *>(lconv + 2 * C + ch);
  load_inputs(__builtin_amdgcn_readfirstlane(splan[0].x), in0);

  // Software pipeline: the loads a node's successor needs (its inputs, and on a
  // change of group its window rows and parent state) are issued before this
  // node's state stores.  Loads and stores share one in-order completion
  // counter, so a load issued after the stores could only be waited for by
  // waiting for the stores as well.
  auto node_step = [&](int i, In &c, In &nx) {
    // tree facts in scalar registers, so that branches on them stay branches
    // (not selects that would wait for loads)
    const int4 pl = splan[i];
    const int n = __builtin_amdgcn_readfirstlane(pl.x);
    const int nn = __builtin_amdgcn_readfirstlane(pl.y);
    const int np = __builtin_amdgcn_readfirstlane(pl.z);
    const int fl = __builtin_amdgcn_readfirstlane(pl.w);
    const int64_t tok = tok0 + n;
    float *y = sy[i & 1];
    // the next node: a sibling (same parent state), the child of this node
    // (carry this node's state), or the first child of an earlier node (load)
    const bool carry = (fl >> 22) & 1;
    const bool regroup = (fl >> 23) & 1;  // np's state from its node buffer
    const bool take0 = (fl >> 28) & 1, take1 = (fl >> 24) & 1, take2 = (fl >> 25) & 1;
    const bool keepn1 = (fl >> 26) & 1, keepn2 = (fl >> 27) & 1;
    if (conv_lane) {
#pragma unroll
      for (int e = 0; e < CW; ++e) {
        const int sh = (e & 1) ? 16 : 0;
        auto pick = [&](const CR &v) {
          return __uint_as_float(((CV::word(v, e >> 1) >> sh) & 0xffffu) << 16);
        };
        const u32x4 &w2 = wv[e >> 1];
        const int wb = (e & 1) * 2;
        float acc = __uint_as_float(w2[wb] << 16) * pick(c.w0);
        acc = fmaf(__uint_as_float(w2[wb] & 0xffff0000u), pick(c.w1), acc);
        acc = fmaf(__uint_as_float(w2[wb + 1] << 16), pick(c.w2), acc);
        acc = fmaf(__uint_as_float(w2[wb + 1] & 0xffff0000u), pick(c.x), acc);
        if (a.flags & GDN_F_CONV_SILU) acc = acc / (1.f + __expf(-acc));
        y[pt * D + jc + e] = acc;
      }
      if (conv_writer) {
        uint16_t *dst = nconv + int64_t(n) * kConvRows * C;
        *reinterpret_cast<CR *>(dst + ch) = c.w1;
        *reinterpret_cast<CR *>(dst + C + ch) = c.w2;
        *reinterpret_cast<CR *>(dst + 2 * C + ch) = c.x;
      }
    }
    __syncthreads();  // y complete (the other buffer is free again for the next node)

    const float *sq = y, *sk = y + D, *sv = y + 2 * D;
    float kinv = 1.f, qinv = 1.f;
    if (a.flags & GDN_F_L2NORM_K) {
      float ss = 0.f;
      for (int j = lane; j < D; j += 64) ss = fmaf(sk[j], sk[j], ss);
      kinv = 1.f / sqrtf(wave_sum(ss) + 1e-6f);
    }
    if (a.flags & GDN_F_L2NORM_Q) {
      float ss = 0.f;
      for (int j = lane; j < D; j += 64) ss = fmaf(sq[j], sq[j], ss);
      qinv = 1.f / sqrtf(wave_sum(ss) + 1e-6f);
    }
    float kq = 0.f;
    for (int j = lane; j < D; j += 64) kq = fmaf(sk[j] * kinv, sq[j] * qinv, kq);
    kq = wave_sum(kq);
    float kk[VEC], qq[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      kk[e] = sk[col0 + e] * kinv;
      qq[e] = sq[col0 + e] * qinv;
    }

    // ---- the successor's loads, ahead of this node's stores -------------------
    // (issued for every node, the last one re-reading its own, so that the wait
    // counts the compiler derives hold on every path)
    load_inputs(nn, nx);
    // the successor's window rows, always loaded (x rows and live rows are small
    // and cached), so they never wait on a select
    {
      const int used = fl & 3, q1 = (fl >> 2) & 1023, q0 = (fl >> 12) & 1023;
      nx.w0 = window_row(0, used, q0, q1, np);
      nx.w1 = window_row(1, used, q0, q1, np);
      nx.w2 = window_row(2, used, q0, q1, np);
    }
    const __amdgpu_buffer_rsrc_t nsrc = block(nodes + int64_t(regroup ? np : 0) * nstride);
    const __amdgpu_buffer_rsrc_t dst = block(nodes + int64_t(n) * nstride);
    const __amdgpu_buffer_rsrc_t orow =
        __builtin_amdgcn_make_buffer_rsrc(a.out + (tok * H + h) * D, 0, D * 2, 0x00020000);
    const float beta = c.beta;
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int r = r0 + it * RPI + row_in_group;
      // whole row blocks (every supported shape but the smallest) need no test,
      // which keeps the stores unconditional for the wait counts
      const bool on = ROWS % RPI == 0 || r < r0 + ROWS;
      float s[VEC];
      SV::to_f32(cur[it], s);
      float pu = 0.f, pq = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        s[e] *= c.al[NAL == 1 ? 0 : e];
        pu = fmaf(s[e], kk[e], pu);
        pq = fmaf(s[e], qq[e], pq);
      }
      pu = group_sum<LPR>(pu);
      pq = group_sum<LPR>(pq);
      if (on) {
        const float d = beta * (sv[r] - pu);
#pragma unroll
        for (int e = 0; e < VEC; ++e) s[e] = fmaf(d, kk[e], s[e]);
        const SR w = SV::from_f32(s);  // what the pool dtype holds: a child starts from this
        if (keepn1) keep1[it] = w;
        if (keepn2) keep2[it] = w;
        if (carry) cur[it] = w;
        else if (take0) cur[it] = keep0[it];
        else if (take1) cur[it] = keep1[it];
        else if (take2) cur[it] = keep2[it];
        else if (regroup)
          cur[it] = __builtin_bit_cast(SR, __builtin_amdgcn_raw_buffer_load_b128(nsrc, loff, it * kPieceStep, 0));
        // The piece offset goes into the lane offset, not the scalar offset: a
        // 16-byte buffer store reads its data registers over several cycles, and
        // the compiler keeps an overwriting instruction away from them only when
        // the scalar offset is not a register.  With a register scalar offset the
        // next instruction was allowed to overwrite the first data register, and
        // under a full launch some lanes stored that new value.
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, w), dst, loff + it * kPieceStep, 0, 2);
        // every lane of the row stores the same value: no divergent branch
        __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(a.scale * fmaf(d, kq, pq)), orow, r * 2, 0, 0);
      }
    }
  };

  // node 0 runs ahead of the loop, so that every entry into the loop body
  // follows a whole node step and the wait counts are the same on each entry
  node_step(0, in0, in1);
  int i = 1;
  for (; i + 1 < T; i += 2) {
    node_step(i, in1, in0);
    node_step(i + 1, in0, in1);
  }
  if (i < T) node_step(i, in1, in0);
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
