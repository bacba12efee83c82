// prefill.hip -- chunked prefill of the gated delta rule on CDNA4 MFMA.
//
// The recurrence (page "企业官网建设流程全解析", Kimi K3 notes, section
// "Speculative decoding")
//     S_t = S_{t-1} Diag(a_t) + d_t k_t^T,   d_t = b_t (v_t - S_{t-1} Diag(a_t) k_t),
//     o_t = scale * S_t q_t
// is unrolled over chunks of 64 tokens (page "SGLang Mamba Radix Cache 深度解析",
// configuration: chunk size 64).  Inside a chunk with entry state S0, writing
// G(t, i) = prod_{i < tau <= t} a_tau (per channel) and g_t = G(t, -1):
//     A[t][i] = sum_c k_t k_i G(t,i)     (i < t),   M[t][i] = sum_c q_t k_i G(t,i)  (i <= t)
//     T = (I + Diag(b) A)^-1,  T' = T Diag(b)
//     W = T' (g . K),  U = T' V,  Dl = U - W S0^T          (rows d_t)
//     O = (g . Q) S0^T + M Dl,   S_end = S0 Diag(g_63) + Dl^T (G(63, t) . K)
// (a restatement checked against the sequential form by the oracle's tests).
//
// Two kernels per window of chunks:
//   prep  (one 1024-thread workgroup per (request, chunk, head); all chunks in
//         parallel): conv + norms, log2 decays, A and M, T, and the chunk's
//         operands -W, U, g.Q, G(63,.)K, M, g_63 written to a workspace record.
//         Every contraction runs on bf16 MFMA in a three-product hi/lo split,
//         which carries about 16 mantissa bits and fp32 range.
//   scan  (one workgroup per (request, head, 16 rows of V); serial over chunks):
//         state wave w keeps the state columns of channels [32w, 32w+32) in fp32
//         registers and forms Dl for one 16-token block; one LDS exchange per
//         chunk completes Dl, and every state wave updates its own columns.  As
//         many output waves form (g.Q) S0^T + M Dl for their token blocks and
//         store them, off the state's serial chain.  No operand is transposed
//         on the way: the record is stored in MFMA operand order, with the
//         32-wide k steps permuted the way two 16x16 accumulator tiles lie in a
//         wave's registers (see pk below), so accumulators feed the next product
//         directly, and the next chunk's operands are loaded while the current
//         one is computed.
//
// Chunks are aligned to absolute positions: the first chunk of a request starts
// at start_len rounded down to a multiple of 64 and is padded at the front
// (pad tokens have a = 1, b = 0, k = q = v = 0, which leaves the state exactly
// unchanged), so every snapshot boundary is a chunk end.
//
// Decay products are handled in log2 space inside a chunk, on one of two paths
// chosen per chunk by the prep workgroup:
//   chunk reference (no 16-token block decays a channel by more than 2^-24):
//         with L the log2 decay cumulated from the chunk start, the factors split
//         exactly into P = k 2^L, R = k 2^-L, Q = q 2^L (all within 2^+-96), so
//         A = P R^T and M = Q R^T are single products of planes built once, and
//         (I + Diag(b) A) X = Diag(b) [V | P] is solved by block forward
//         substitution on k = 16 MFMA;
//   blockwise (any decay): every factor is exp2 of a difference of partial sums
//         that is <= 0, except on the diagonal 16x16 blocks where the
//         factorisation goes through the block's middle token (factors up to
//         2^60); a block whose channels span more than that uses an exact
//         per-pair evaluation instead.
#include "common.hpp"
#include "lanes.hpp"
#include "mfma.hpp"

namespace gdn {
namespace {

constexpr int kPrepThreads = 1024;

// min(max(v, 0), hi) for a wave-uniform v, kept in a scalar register: the compiler
// otherwise forms a vector med3 for the clamp, and a buffer resource built from a
// vector register costs a readfirstlane loop around every load that uses it.
__device__ __forceinline__ int uniform_clamp(int v, int hi) {
  return __builtin_amdgcn_readfirstlane(max(min(v, hi), 0));
}
// lane s of each quad's value v, in all four lanes (DPP quad_perm [s, s, s, s]; s
// is a constant after unrolling)
__device__ __forceinline__ float quad_bcast(float v, int s) {
  switch (s) {
    case 0: return dpp_mov<0x00>(v);
    case 1: return dpp_mov<0x55>(v);
    case 2: return dpp_mov<0xAA>(v);
    default: return dpp_mov<0xFF>(v);
  }
}
constexpr float kMidRange = 60.f;  // max |log2| of a factor on the diagonal fast path
// A chunk takes the chunk-reference path when no 16-token block decays any channel
// by more than 2^-kBlockSpan, so that e^{+-L} stays within 2^(+-4 kBlockSpan).
constexpr float kBlockSpan = 24.f;

// ------------------------------------------------------------ record layout --
// One record per (request, chunk, head).  A "fragment" is one bf16 plane (hi or
// lo) of one MFMA operand: 64 lanes x 8 values, 1 KiB, lane-major.
template <int D>
struct Rec {
  static constexpr int KD = D < 32 ? 32 : D;  // channels padded to a k step
  static constexpr int NKS = KD / 32;         // 32-channel k steps
  static constexpr int NCB = D / 16;          // 16-wide tiles of channels (and of V)
  static constexpr size_t FRAG = 1024;
  // -W   [tb][ks][plane]: rows 16tb + l%16, channels 32ks + pk(l/16, e)
  static constexpr size_t WF = 0;
  // g.Q  [tb][ks][plane]: same order
  static constexpr size_t QF = WF + size_t(4) * NKS * 2 * FRAG;
  // M    [tb][ks'][plane]: rows 16tb + l%16, tokens 32ks' + pk(l/16, e)
  static constexpr size_t MF = QF + size_t(4) * NKS * 2 * FRAG;
  // G(63,t)k_t transposed [cb][ks'][plane]: channel 16cb + l%16, tokens 32ks' + pk(l/16, e)
  static constexpr size_t KF = MF + size_t(4) * 2 * 2 * FRAG;
  // U    fp32 [tb][vb][lane][4]: rows 16tb + 4(l/16) + j, column 16vb + l%16
  static constexpr size_t UF = KF + size_t(NCB) * 2 * 2 * FRAG;
  // g_63 fp32 [D]
  static constexpr size_t GC = UF + size_t(4) * NCB * 64 * 16;
  static constexpr size_t BYTES = (GC + size_t(D) * 4 + 255) / 256 * 256;
};

struct KArgs {
  PrefillArgs a;
  void *ssm;
  uint16_t *conv;
  int32_t *err;
  int slots, heads;
  int c0, w, vt_count;
  char *ws;            // workspace base: the fp32 state carry, then record windows
  size_t rec_off;      // byte offset of this launch's record window
};

// a fragment pair (hi, lo) of a record
__device__ __forceinline__ void frag_store(char *base, int idx, int lane, const Split &s) {
  *reinterpret_cast<bf16x8 *>(base + size_t(2 * idx) * 1024 + lane * 16) = s.hi;
  *reinterpret_cast<bf16x8 *>(base + size_t(2 * idx + 1) * 1024 + lane * 16) = s.lo;
}

// =============================================================== prep kernel ==
// Two layouts share one LDS array (fp32 words); the log2 decays, block totals, beta
// and block flags sit in a common tail that both use.
template <int D>
struct PrepLds {
  static constexpr int KD = D < 32 ? 32 : D;
  static constexpr int DP = KD + 4;  // fp32 pitch of [t][c] arrays
  static constexpr int TP = 68;      // fp32 pitch of [v][t] and [t][i] arrays
  // blockwise path: q, k, v^T, Diag(b) A, T and scratch in fp32
  static constexpr int RQ = (64 * DP > 64 * TP ? 64 * DP : 64 * TP);  // q, later T
  static constexpr int RK = 64 * DP;                                  // k, later g.k
  static constexpr int RV = D * TP;                                   // v^T
  static constexpr int RA = 64 * TP;                                  // Diag(b) A
  static constexpr int RP = 3 * 16 * 17;                              // 16x16 scratch per level block
  static constexpr int OQ = 0, OK = OQ + RQ, OV = OK + RK, OA = OV + RV, OP = OA + RA,
                       SLOW_END = OP + RP;
  // chunk-reference path: bf16 hi/lo planes [64][KP] of P = k e^L, R = k e^-L and
  // Q = q e^L; Diag(b) A and the diagonal inverses reuse the R planes (or follow
  // the planes when those are too small), W reuses the Q planes, V the decays
  static constexpr int KP = KD + 8;          // bf16 pitch of a plane row (16-byte rows)
  static constexpr int PS = 64 * KP / 2;     // one plane in fp32 words
  static constexpr int DPITCH = 20;          // fp32 pitch of a diagonal inverse row
  static constexpr int RD = 4 * 16 * DPITCH;
  static constexpr int RN = 6 * 64 * 4;      // -N_mk (m > k) as split k = 16 operand fragments
  static constexpr bool A_IN_R = 2 * PS >= 64 * TP + RD + RN;
  static constexpr int FPH = 0, FPL = PS, FRH = 2 * PS, FRL = 3 * PS, FQH = 4 * PS, FQL = 5 * PS;
  static constexpr int FA = A_IN_R ? FRH : 6 * PS, FD = FA + 64 * TP, FN = FD + RD, FW = FQH;
  static constexpr int FAST_END = A_IN_R ? 6 * PS : FN + RN;
  static_assert(64 * DP <= 2 * PS, "W fits the Q planes");
  // common tail
  static constexpr int RL = 64 * DP;                                  // log2 decays, later V (fast path)
  static constexpr int OL = SLOW_END > FAST_END ? SLOW_END : FAST_END;
  static constexpr int OTOT = OL + RL, OB = OTOT + 4 * KD, OF = OB + 64, TOTAL = OF + 4;
};

template <int D, int AMODE>
__global__ __launch_bounds__(kPrepThreads) void prefill_prep_kernel(KArgs ka) {
  using LY = PrepLds<D>;
  using RC = Rec<D>;
  constexpr int KD = LY::KD, DP = LY::DP, TP = LY::TP;
  constexpr int NKS = RC::NKS, NCB = RC::NCB;
  __shared__ __attribute__((aligned(16))) float smem[LY::TOTAL];
  float *sQ = smem + LY::OQ, *sK = smem + LY::OK, *sL = smem + LY::OL, *sV = smem + LY::OV;
  float *sA = smem + LY::OA, *sP = smem + LY::OP, *sTot = smem + LY::OTOT, *sB = smem + LY::OB;
  int *sWF = reinterpret_cast<int *>(smem + LY::OF);
  float *sT = sQ;  // T [64][TP], once q has been consumed

  const PrefillArgs &a = ka.a;
  const int H = ka.heads;
  // (chunk, head) items in dispatch order with the head fastest: the heads of one
  // chunk, which read adjacent pieces of the same input and decay rows and write
  // adjacent records, run at the same time.  (Measured on MI355X against the chunk
  // fastest: 4% faster for a 64-request window, 3% for one long request.  Keeping
  // each XCD on one contiguous range of items as well was 9% slower for the
  // 64-request window.)
  const int id = blockIdx.y * gridDim.x + blockIdx.x;
  const int h = id % H, bc = id / H, b = bc / ka.w, cl = bc % ka.w, c = ka.c0 + cl;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g4 = lane >> 4;

  const ReqGeom rg = req_geom(a, b);
  const int slot = a.slot_table[b];
  if (!rg.ok || slot <= 0 || slot >= ka.slots || c >= rg.nch) return;
  const bool warm = a.has_initial_state[b] != 0;
  const int64_t C = int64_t(H) * 3 * D;
  char *rec = ka.ws + ka.rec_off + (size_t(b * ka.w + cl) * H + h) * RC::BYTES;
  const int p0 = 64 * c - rg.off;  // request position of local token 0

  // ---- phase 1: causal conv + norms (waves 0..11), log2 decays + beta (12..15) ----
  // The conv results stay in registers until the decays decide which path runs.
  constexpr int G = D / 8;                // 8-channel groups per head part
  constexpr int R = G >= 8 ? G / 4 : 1;   // consecutive tokens per conv item
  constexpr int NR = 64 / R;
  constexpr int CONV_ITEMS = 3 * NR * G;  // 768, or 384 when D = 16
  static_assert(CONV_ITEMS <= 768 && CONV_ITEMS % 64 == 0, "conv items must fill waves 0..11");
  const bool conv_thread = tid < CONV_ITEMS;
  const int cg = tid % G, cpart = tid / (G * NR);
  const int ct0 = ((tid / G) % NR) * R;
  float y[R][8];
  if (conv_thread) {
    const int g = cg, part = cpart, t0 = ct0;
    const int64_t ch0 = int64_t(part) * H * D + int64_t(h) * D + 8 * g;
    const uint16_t *crow = ka.conv + (int64_t(a.layer) * ka.slots + slot) * kConvRows * C;
    u32x4 wr[4], xr[R + 3];
#pragma unroll
    for (int i = 0; i < 4; ++i) wr[i] = *reinterpret_cast<const u32x4 *>(a.conv_w + (ch0 + 2 * i) * 4);
    // The chunk's input rows (positions p0 - 3 .. p0 + 63) as a buffer resource based
    // at its first row inside the request: a row before it (negative offset) or past
    // the request's end lies outside the resource and reads zero, so no load is
    // branched around.  A warm start's rows at positions -3..-1 come from the conv
    // rows of the slot, patched in for the first chunk only.
    const int qb = max(p0 - 3, 0);
    const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.x) + (int64_t(rg.bos) + qb) * C, 0, uniform_clamp(rg.len - qb, 67) * int(C) * 2,
        0x00020000);
#pragma unroll
    for (int r = 0; r < R + 3; ++r)  // positions p0 + t0 - 3 + r
      xr[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            xres, ((p0 + t0 - 3 + r - qb) * int(C) + int(ch0)) * 2, 0, 0));
    if (warm && p0 + t0 - 3 < 0) {  // p0 < 0 when the request starts inside the chunk
#pragma unroll
      for (int r = 0; r < R + 3; ++r) {
        const int q = p0 + t0 - 3 + r;
        if (q < 0 && q >= -3) xr[r] = *reinterpret_cast<const u32x4 *>(crow + int64_t(3 + q) * C + ch0);
      }
    }
    const bool silu = (a.flags & GDN_F_CONV_SILU) != 0;
    const bool norm = part == 0 ? (a.flags & GDN_F_L2NORM_Q) != 0 : part == 1 ? (a.flags & GDN_F_L2NORM_K) != 0 : false;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int pos = p0 + t0 + r;
      const bool valid = pos >= 0 && pos < rg.len;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // taps (0, 1) and (2, 3) multiply positions (pos - 3, pos - 2) and (pos - 1, pos)
        float acc = dot2_bf16(wr[e >> 1][2 * (e & 1)], tok_pair(xr[r], xr[r + 1], e), 0.f);
        acc = dot2_bf16(wr[e >> 1][2 * (e & 1) + 1], tok_pair(xr[r + 2], xr[r + 3], e), acc);
        y[r][e] = valid ? acc : 0.f;
      }
    }
    // SiLU in one branch after the loops (silu(0) = 0 keeps the masked values): a
    // flag tested inside the unrolled loops costs a branch per conv output
    if (silu) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) y[r][e] = y[r][e] / (1.f + __expf(-y[r][e]));
    }
    if (norm) {  // wave-uniform: the G lanes of a token set share the sum
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(y[r][e], y[r][e], ss);
        ss = group_sum<G>(ss);
        const float inv = __builtin_amdgcn_rsqf(ss + 1e-6f);
#pragma unroll
        for (int e = 0; e < 8; ++e) y[r][e] *= inv;
      }
    }
  } else if (wave >= 12) {
    // wave 12 + m handles token block m.  Lane l takes channels l and l + 64 (those
    // below KD) and cumulates their log2 decays token by token, so no step crosses
    // lanes.  The block's decay rows are a buffer resource based at its first row
    // inside the request: rows outside it read zero and are masked below.
    const int m = wave - 12;
    if (wave == 12) {
      const int pos = p0 + lane;
      sB[lane] = (pos >= 0 && pos < rg.len) ? a.beta[int64_t(rg.bos + pos) * H + h] : 0.f;
    }
    constexpr int NA = AMODE == GDN_ALPHA_PER_CHANNEL ? D : 1;
    constexpr int CPL = (KD + 63) / 64;
    const int pb = p0 + 16 * m, pbase = max(pb, 0);
    const __amdgpu_buffer_rsrc_t ares = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(a.alpha) + (int64_t(rg.bos + pbase) * H + h) * NA, 0,
        uniform_clamp(rg.len - pbase, 16) * H * NA * 4, 0x00020000);
    // every load is issued before the first use, so the 16 rows are in flight together
    float av[16][CPL];
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
      for (int q = 0; q < CPL; ++q) {
        const int ch = lane + 64 * q;
        av[j][q] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                 ares, ((pb + j - pbase) * H * NA + (NA == 1 || ch >= D ? 0 : ch)) * 4, 0, 0));
      }
    float cum[CPL], l0[CPL], l7[CPL];
#pragma unroll
    for (int q = 0; q < CPL; ++q) cum[q] = l0[q] = l7[q] = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int pos = pb + j;
      const bool vpos = pos >= 0 && pos < rg.len;
#pragma unroll
      for (int q = 0; q < CPL; ++q) {
        const int ch = lane + 64 * q;
        const float la = (vpos && ch < D) ? fmaxf(__log2f(av[j][q]), -512.f) : 0.f;  // a == 0: full decay
        cum[q] += la;
        if (ch < KD) sL[(16 * m + j) * DP + ch] = cum[q];
        if (j == 0) l0[q] = cum[q];
        if (j == 7) l7[q] = cum[q];
      }
    }
    bool big = false, wide = false;
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      const int ch = lane + 64 * q;
      if (ch < KD) {
        big = big || fmaxf(l0[q] - l7[q], l7[q] - cum[q]) > kMidRange;
        wide = wide || -cum[q] > kBlockSpan;
        sTot[m * KD + ch] = cum[q];
      }
    }
    const bool any_big = __ballot(big) != 0, any_wide = __ballot(wide) != 0;
    // bit 0: the blockwise path evaluates this diagonal block exactly;
    // bit 1: the block rules out the chunk-reference path
    if (lane == 0) sWF[m] = (any_big ? 1 : 0) | (any_wide ? 2 : 0);
  }
  __syncthreads();

  if (((sWF[0] | sWF[1] | sWF[2] | sWF[3]) & 2) == 0) {
    // ====== chunk-reference path ================================================
    // With L_t the log2 decay cumulated from the chunk start, G(t,i) = e^{L_t - L_i}
    // factors exactly into P = k e^L and R = k e^-L, so A = P R^T, M = Q R^T with
    // Q = q e^L, and g.K = P, g.Q = Q, G(63,.)K = R e^{L_63}.  The operands are
    // rounded to hi/lo bf16 planes once, here, and every product reads them as is.
    constexpr int KP = LY::KP;
    __bf16 *pPh = reinterpret_cast<__bf16 *>(smem + LY::FPH), *pPl = reinterpret_cast<__bf16 *>(smem + LY::FPL);
    __bf16 *pRh = reinterpret_cast<__bf16 *>(smem + LY::FRH), *pRl = reinterpret_cast<__bf16 *>(smem + LY::FRL);
    __bf16 *pQh = reinterpret_cast<__bf16 *>(smem + LY::FQH), *pQl = reinterpret_cast<__bf16 *>(smem + LY::FQL);
    float *fA = smem + LY::FA, *fD = smem + LY::FD, *fW = smem + LY::FW;
    s16x4 *fN = reinterpret_cast<s16x4 *>(smem + LY::FN);  // [pair][lane][hi, lo]
    float *fV = sL;  // V over the decays once the planes are built
    constexpr int DPT = LY::DPITCH;

    // ---- F1: planes from the conv outputs ----------------------------------
    if constexpr (KD != D) {  // channel padding of P, R, Q
      for (int i = tid; i < 64 * (KD - D); i += kPrepThreads) {
        const int t = i / (KD - D), cc = D + i % (KD - D);
        const __bf16 z = static_cast<__bf16>(0.f);
        pPh[t * KP + cc] = z;
        pPl[t * KP + cc] = z;
        pRh[t * KP + cc] = z;
        pRl[t * KP + cc] = z;
        pQh[t * KP + cc] = z;
        pQl[t * KP + cc] = z;
      }
    }
    if (conv_thread && cpart < 2) {
      const int m = ct0 >> 4;  // the item's tokens share one 16-token block
      f32x4 pre0 = {0.f, 0.f, 0.f, 0.f}, pre1 = pre0;
      for (int kb = 0; kb < m; ++kb) {
        pre0 += ld4(sTot + kb * KD + 8 * cg);
        pre1 += ld4(sTot + kb * KD + 8 * cg + 4);
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int t = ct0 + r;
        const f32x4 l0 = pre0 + ld4(sL + t * DP + 8 * cg), l1 = pre1 + ld4(sL + t * DP + 8 * cg + 4);
        float lam[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          lam[j] = l0[j];
          lam[4 + j] = l1[j];
        }
        float u[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) u[e] = y[r][e] * fexp2(lam[e]);
        const Split su = split8(u);
        const int o = t * KP + 8 * cg;
        if (cpart == 0) {
          *reinterpret_cast<bf16x8 *>(pQh + o) = su.hi;
          *reinterpret_cast<bf16x8 *>(pQl + o) = su.lo;
        } else {
          *reinterpret_cast<bf16x8 *>(pPh + o) = su.hi;
          *reinterpret_cast<bf16x8 *>(pPl + o) = su.lo;
          float w[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) w[e] = y[r][e] * fexp2(-lam[e]);
          const Split sw = split8(w);
          *reinterpret_cast<bf16x8 *>(pRh + o) = sw.hi;
          *reinterpret_cast<bf16x8 *>(pRl + o) = sw.lo;
        }
      }
    }
    __syncthreads();
    if (conv_thread && cpart == 2) {  // V over the decays, which are no longer read
#pragma unroll
      for (int r = 0; r < R; ++r) {
        st4(fV + (ct0 + r) * DP + 8 * cg, f32x4{y[r][0], y[r][1], y[r][2], y[r][3]});
        st4(fV + (ct0 + r) * DP + 8 * cg + 4, f32x4{y[r][4], y[r][5], y[r][6], y[r][7]});
      }
    }

    // ---- F2: A^T, M^T tiles (waves 0..9); g.Q, G(63,.)K, g_63 records (10..15) ----
    f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accM = {0.f, 0.f, 0.f, 0.f};
    const int pi = wave;  // (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) ...
    const int pm = pi < 1 ? 0 : pi < 3 ? 1 : pi < 6 ? 2 : 3;
    const int pn = pi - pm * (pm + 1) / 2;
    if (wave < 10) {
      const int i = 16 * pn + r16, t = 16 * pm + r16;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int c0 = 32 * ks + 8 * g4;
        Split Ra, Pb, Qb;
        Ra.hi = *reinterpret_cast<const bf16x8 *>(pRh + i * KP + c0);
        Ra.lo = *reinterpret_cast<const bf16x8 *>(pRl + i * KP + c0);
        Pb.hi = *reinterpret_cast<const bf16x8 *>(pPh + t * KP + c0);
        Pb.lo = *reinterpret_cast<const bf16x8 *>(pPl + t * KP + c0);
        Qb.hi = *reinterpret_cast<const bf16x8 *>(pQh + t * KP + c0);
        Qb.lo = *reinterpret_cast<const bf16x8 *>(pQl + t * KP + c0);
        accA = mfma3(Ra, Pb, accA);
        accM = mfma3(Ra, Qb, accM);
      }
    } else {
      const int rel = tid - 640;
      for (int it = rel; it < 4 * NKS * 64; it += 384) {  // g.Q: the Q planes in fragment order
        const int ln = it & 63, tb = (it >> 6) & 3, ks = it >> 8;
        const int o = (16 * tb + (ln & 15)) * KP + 32 * ks + 4 * (ln >> 4);  // channels o, o+16
        Split sp;
        sp.hi = __builtin_shufflevector(*reinterpret_cast<const bf16x4 *>(pQh + o),
                                        *reinterpret_cast<const bf16x4 *>(pQh + o + 16), 0, 1, 2, 3, 4, 5, 6, 7);
        sp.lo = __builtin_shufflevector(*reinterpret_cast<const bf16x4 *>(pQl + o),
                                        *reinterpret_cast<const bf16x4 *>(pQl + o + 16), 0, 1, 2, 3, 4, 5, 6, 7);
        frag_store(rec + RC::QF, tb * NKS + ks, ln, sp);
      }
      // M fragments (tb 0 and 1, ks' 1) lie above the diagonal; the scan multiplies
      // them where a wave holds several token blocks (head dims below 128), so store
      // zeros
      for (int it = rel; it < 256; it += 384) {
        const int idx = (it >> 7) ? 3 : 1, plane = (it >> 6) & 1, ln = it & 63;
        *reinterpret_cast<u32x4 *>(rec + RC::MF + size_t(2 * idx + plane) * 1024 + ln * 16) = u32x4{0u, 0u, 0u, 0u};
      }
      float *recGC = reinterpret_cast<float *>(rec + RC::GC);
      for (int cc = rel; cc < D; cc += 384) {
        float tot = 0.f;
        for (int kb = 0; kb < 4; ++kb) tot += sTot[kb * KD + cc];
        recGC[cc] = fexp2(tot);
      }
    }
    // G(63,.)K = R e^{L_63}, tokens along k, on every wave (the tile products of waves
    // 0..9 take less time than the record writes of waves 10..15)
    for (int it = tid; it < NCB * 2 * 64; it += kPrepThreads) {
      const int ln = it & 63, ksp = (it >> 6) & 1, cb = it >> 7;
      const int cc = 16 * cb + (ln & 15), g = ln >> 4;
      float tot = 0.f;
      for (int kb = 0; kb < 4; ++kb) tot += sTot[kb * KD + cc];
      const float g63 = fexp2(tot);
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int o = (32 * ksp + pk(g, e)) * KP + cc;
        v[e] = (static_cast<float>(pRh[o]) + static_cast<float>(pRl[o])) * g63;
      }
      frag_store(rec + RC::KF, cb * 2 + ksp, ln, split8(v));
    }
    __syncthreads();  // the R and Q planes are free from here on
    if (wave < 10) {
      // lane (t, g4) holds A[t][16n + 4g4 + j] and M[t][16n + 4g4 + j]
      const bool diag = pm == pn;
      const int t = 16 * pm + r16;
      const float bt = sB[t];
      f32x4 av;
      float mv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ii = 16 * pn + 4 * g4 + j;
        av[j] = (!diag || ii < t) ? bt * accA[j] : 0.f;  // Diag(b) A
        mv[j] = (!diag || ii <= t) ? accM[j] : 0.f;
      }
      st4(fA + t * TP + 16 * pn + 4 * g4, av);
      bf16x4 mh, ml;
      {
        const Split2 a = split2(mv[0], mv[1]), b = split2(mv[2], mv[3]);
        mh = __builtin_bit_cast(bf16x4, u32x2{a.hi, b.hi});
        ml = __builtin_bit_cast(bf16x4, u32x2{a.lo, b.lo});
      }
      char *mf = rec + RC::MF + size_t(2 * (2 * pm + (pn >> 1))) * 1024 + lane * 16 + (pn & 1) * 8;
      *reinterpret_cast<bf16x4 *>(mf) = mh;
      *reinterpret_cast<bf16x4 *>(mf + 1024) = ml;
      if (diag && !(pm & 1)) {  // tile (m, m+1) above the diagonal is zero
        const bf16x4 z = {static_cast<__bf16>(0.f), static_cast<__bf16>(0.f), static_cast<__bf16>(0.f),
                          static_cast<__bf16>(0.f)};
        *reinterpret_cast<bf16x4 *>(mf + 8) = z;
        *reinterpret_cast<bf16x4 *>(mf + 1024 + 8) = z;
      }
    }
    __syncthreads();

    // ---- F3: inverses D_m of the unit lower-triangular diagonal blocks --------
    if (wave < 4) {
      // Block m = wave, column j of the inverse on the four lanes 4j..4j+3: lane p
      // owns rows 4k + p of the column's right-hand side and subtracts each x_t as
      // soon as it is known (x_t is broadcast from its owner lane), so every row
      // takes the same fused multiply-adds in the same order as a row-by-row
      // substitution, and the chain per row step is one broadcast and one FMA.
      const int m = wave, j = lane >> 2, p = lane & 3;
      f32x4 Lr[4][4];  // rows 4k + p of block m, columns 0..15
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) Lr[k][c4] = ld4(fA + (16 * m + 4 * k + p) * TP + 16 * m + 4 * c4);
      float bc[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) bc[k] = (4 * k + p == j) ? 1.f : 0.f;
#pragma unroll
      for (int t = 0; t < 15; ++t) {
        const float xt = quad_bcast(bc[t >> 2], t & 3);
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (4 * k + p > t) bc[k] = fmaf(-Lr[k][t >> 2][t & 3], xt, bc[k]);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) fD[(16 * m + 4 * k + p) * DPT + j] = bc[k];
    } else if (wave < 10) {
      // -N_mk for the six blocks below the diagonal, split once for every wave
      const int q = wave - 4;
      const int m = q < 1 ? 1 : q < 3 ? 2 : 3, k = q - m * (m - 1) / 2;
      const Split4 nf = split4s(-ld4(fA + (16 * m + r16) * TP + 16 * k + 4 * g4));
      fN[(q * 64 + lane) * 2] = nf.hi;
      fN[(q * 64 + lane) * 2 + 1] = nf.lo;
    } else {
      if constexpr (KD != D) {  // W's channel padding (the solve writes channels < D)
        for (int i = tid - 640; i < 64 * (KD - D); i += kPrepThreads - 640) {
          const int t = i / (KD - D), cc = D + i % (KD - D);
          fW[t * DP + cc] = 0.f;
        }
      }
    }
    __syncthreads();

    // ---- F4: (I + Diag(b) A) X = Diag(b) [V | g.K] by block forward substitution,
    //      X_m = D_m (Y_m - sum_{k<m} N_mk X_k).  Wave w owns one 16-column tile: V
    //      tiles give U, g.K tiles give W.  The 16-row blocks of X stay in the wave's
    //      accumulators and enter the next k = 16 products as operands unchanged.
    if (wave < 2 * NCB) {
      const bool isw = wave >= NCB;
      const int tile = isw ? wave - NCB : wave;
      const int col = 16 * tile + r16;
      Split4 XS[4];
      // every block's right-hand side first: its LDS reads are then in flight together
      // instead of one round trip per block step of the substitution
      f32x4 Yb[4];
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = 16 * m + 4 * g4 + j;
          const float yv = isw ? static_cast<float>(pPh[t * KP + col]) + static_cast<float>(pPl[t * KP + col])
                               : fV[t * DP + col];
          Yb[m][j] = sB[t] * yv;
        }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        f32x4 acc = Yb[m];
#pragma unroll
        for (int k = 0; k < m; ++k) {
          const int q = m * (m - 1) / 2 + k;
          const Split4 nf{fN[(q * 64 + lane) * 2], fN[(q * 64 + lane) * 2 + 1]};
          acc = mfma3k16(nf, XS[k], acc);
        }
        const f32x4 X = mfma3k16(split4s(ld4(fD + (16 * m + r16) * DPT + 4 * g4)), split4s(acc),
                                 f32x4{0.f, 0.f, 0.f, 0.f});
        XS[m] = split4s(X);
        if (!isw) {
          *reinterpret_cast<f32x4 *>(rec + RC::UF + size_t(m * NCB + tile) * 1024 + lane * 16) = X;
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) fW[(16 * m + 4 * g4 + j) * DP + col] = X[j];
        }
      }
    }
    __syncthreads();

    // ---- F5: -W fragments ------------------------------------------------------
    for (int it = tid; it < 4 * NKS * 64; it += kPrepThreads) {
      const int ln = it & 63, tb = (it >> 6) & 3, ks = it >> 8;
      const int o = (16 * tb + (ln & 15)) * DP + 32 * ks + 4 * (ln >> 4);  // channels o, o+16
      const f32x4 w0 = ld4(fW + o), w1 = ld4(fW + o + 16);
      float w[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        w[j] = -w0[j];
        w[4 + j] = -w1[j];
      }
      frag_store(rec + RC::WF, tb * NKS + ks, ln, split8(w));
    }
    return;
  }

  // ====== blockwise path (any decay) ==============================================
  if constexpr (KD != D) {  // channel padding of q and k
    for (int i = tid; i < 64 * (KD - D); i += kPrepThreads) {
      const int t = i / (KD - D), cc = D + i % (KD - D);
      sQ[t * DP + cc] = 0.f;
      sK[t * DP + cc] = 0.f;
    }
  }
  if (conv_thread) {
    if (cpart == 2) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float *dst = sV + (8 * cg + e) * TP + ct0;
        if constexpr (R == 4) {
          st4(dst, f32x4{y[0][e], y[1][e], y[2][e], y[3][e]});
        } else {
#pragma unroll
          for (int r = 0; r < R; ++r) dst[r] = y[r][e];
        }
      }
    } else {
      float *base = cpart == 0 ? sQ : sK;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        st4(base + (ct0 + r) * DP + 8 * cg, f32x4{y[r][0], y[r][1], y[r][2], y[r][3]});
        st4(base + (ct0 + r) * DP + 8 * cg + 4, f32x4{y[r][4], y[r][5], y[r][6], y[r][7]});
      }
    }
  }
  __syncthreads();

  if (wave < 10) {
    // ---- phase 2a: A^T and M^T tiles of pair (m, n), n <= m (waves 0..9) ----------
    const int flags = (sWF[0] & 1) | ((sWF[1] & 1) << 1) | ((sWF[2] & 1) << 2) | ((sWF[3] & 1) << 3);
    const int pi = wave;  // (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) ...
    const int m = pi < 1 ? 0 : pi < 3 ? 1 : pi < 6 ? 2 : 3;
    const int n = pi - m * (m + 1) / 2;
    const bool diag = m == n;
    const int i = 16 * n + r16;  // rows of the first operand (keys k_i)
    const int t = 16 * m + r16;  // rows of the second operand (k_t, q_t)
    f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accM = {0.f, 0.f, 0.f, 0.f};
    if (!(diag && ((flags >> m) & 1))) {
      const int r = 16 * m + 7;
#pragma unroll 1
      for (int ks = 0; ks < NKS; ++ks) {
        const int c0 = ks * 32 + 8 * g4;
        float rv[8], lk[8], lq[8];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int cc = c0 + 4 * hf;
          const f32x4 ki = ld4(sK + i * DP + cc), li = ld4(sL + i * DP + cc);
          const f32x4 kt = ld4(sK + t * DP + cc), qt = ld4(sQ + t * DP + cc), lt = ld4(sL + t * DP + cc);
          f32x4 rexp, lexp;
          if (diag) {
            const f32x4 lr = ld4(sL + r * DP + cc);
            rexp = lr - li;
            lexp = lt - lr;
          } else {
            f32x4 between = {0.f, 0.f, 0.f, 0.f};
            for (int kb = n + 1; kb < m; ++kb) between += ld4(sTot + kb * KD + cc);
            rexp = ld4(sTot + n * KD + cc) - li;
            lexp = lt + between;
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            rv[4 * hf + j] = ki[j] * fexp2(rexp[j]);
            const float f = fexp2(lexp[j]);
            lk[4 * hf + j] = kt[j] * f;
            lq[4 * hf + j] = qt[j] * f;
          }
        }
        const Split Rs = split8(rv), LK = split8(lk), LQ = split8(lq);
        accA = mfma3(Rs, LK, accA);
        accM = mfma3(Rs, LQ, accM);
      }
    } else {
      // exact per-pair evaluation for a diagonal block with extreme decays
#pragma unroll 1
      for (int j = 0; j < 4; ++j) {
        const int ii = 16 * n + 4 * g4 + j;
        float sa = 0.f, sm = 0.f;
        if (ii <= t) {
          for (int cc = 0; cc < KD; ++cc) {
            const float f = fexp2(sL[t * DP + cc] - sL[ii * DP + cc]) * sK[ii * DP + cc];
            sa = fmaf(sK[t * DP + cc], f, sa);
            sm = fmaf(sQ[t * DP + cc], f, sm);
          }
        }
        accA[j] = sa;
        accM[j] = sm;
      }
    }
    // lane (t, g4) holds A[t][16n + 4g4 + j] and M[t][16n + 4g4 + j]
    const float bt = sB[t];
    f32x4 av;
    float mv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ii = 16 * n + 4 * g4 + j;
      av[j] = (!diag || ii < t) ? bt * accA[j] : 0.f;  // Diag(b) A
      mv[j] = (!diag || ii <= t) ? accM[j] : 0.f;
    }
    st4(sA + t * TP + 16 * n + 4 * g4, av);
    bf16x4 mh, ml;
    {
      const Split2 a = split2(mv[0], mv[1]), b = split2(mv[2], mv[3]);
      mh = __builtin_bit_cast(bf16x4, u32x2{a.hi, b.hi});
      ml = __builtin_bit_cast(bf16x4, u32x2{a.lo, b.lo});
    }
    char *mf = rec + RC::MF + size_t(2 * (2 * m + (n >> 1))) * 1024 + lane * 16 + (n & 1) * 8;
    *reinterpret_cast<bf16x4 *>(mf) = mh;
    *reinterpret_cast<bf16x4 *>(mf + 1024) = ml;
    if (diag && !(m & 1)) {  // tile (m, m+1) above the diagonal is zero
      const bf16x4 z = {static_cast<__bf16>(0.f), static_cast<__bf16>(0.f), static_cast<__bf16>(0.f),
                        static_cast<__bf16>(0.f)};
      *reinterpret_cast<bf16x4 *>(mf + 8) = z;
      *reinterpret_cast<bf16x4 *>(mf + 1024 + 8) = z;
    }
  } else {
    // ---- phase 2b: g.Q, G(63,.)K and g_63 to the record (waves 10..15) -----------
    const int rel = tid - 640;
    for (int it = rel; it < 4 * NKS * 64; it += 384) {
      const int ln = it & 63, tb = (it >> 6) & 3, ks = it >> 8;
      const int t = 16 * tb + (ln & 15), g = ln >> 4;
      float v[8];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int cc = 32 * ks + 16 * hf + 4 * g;  // channels 32ks + pk(g, 4hf + j)
        f32x4 pre = {0.f, 0.f, 0.f, 0.f};
        for (int kb = 0; kb < tb; ++kb) pre += ld4(sTot + kb * KD + cc);
        const f32x4 q4 = ld4(sQ + t * DP + cc), l4 = ld4(sL + t * DP + cc);
#pragma unroll
        for (int j = 0; j < 4; ++j) v[4 * hf + j] = q4[j] * fexp2(pre[j] + l4[j]);
      }
      frag_store(rec + RC::QF, tb * NKS + ks, ln, split8(v));
    }
    for (int it = rel; it < NCB * 2 * 64; it += 384) {
      const int ln = it & 63, ksp = (it >> 6) & 1, cb = it >> 7;
      const int cc = 16 * cb + (ln & 15), g = ln >> 4;
      float v[8];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int tbk = 2 * ksp + hf;  // tokens 32ksp + pk(g, 4hf + j) lie in block tbk
        float post = 0.f;
        for (int kb = tbk; kb < 4; ++kb) post += sTot[kb * KD + cc];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int tt = 16 * tbk + 4 * g + j;
          v[4 * hf + j] = sK[tt * DP + cc] * fexp2(post - sL[tt * DP + cc]);
        }
      }
      frag_store(rec + RC::KF, cb * 2 + ksp, ln, split8(v));
    }
    // M fragments (tb 0 and 1, ks' 1) lie above the diagonal; the scan multiplies
    // them where a wave holds several token blocks (head dims below 128), so store
    // zeros
    for (int it = rel; it < 256; it += 384) {
      const int idx = (it >> 7) ? 3 : 1, plane = (it >> 6) & 1, ln = it & 63;
      *reinterpret_cast<u32x4 *>(rec + RC::MF + size_t(2 * idx + plane) * 1024 + ln * 16) = u32x4{0u, 0u, 0u, 0u};
    }
    float *recGC = reinterpret_cast<float *>(rec + RC::GC);
    for (int cc = rel; cc < D; cc += 384) {
      float s = 0.f;
      for (int kb = 0; kb < 4; ++kb) s += sTot[kb * KD + cc];
      recGC[cc] = fexp2(s);
    }
  }
  __syncthreads();

  // ---- phase 3: diagonal blocks of T (wave 0) while the others form g.k in place ---
  if (wave == 0) {
    // lane (m, j): column j of the inverse of the unit lower-triangular block m
    const int m = lane >> 4, j = lane & 15;
    float x[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      float v = (t == j) ? 1.f : 0.f;
#pragma unroll
      for (int i = 0; i < t; ++i) v = fmaf(-sA[(16 * m + t) * TP + 16 * m + i], x[i], v);
      x[t] = v;
      sT[(16 * m + t) * TP + 16 * m + j] = v;
    }
  } else {
    const int rel = tid - 64;
    // upper tiles (0,1) and (2,3) of T are read by the U/W products: zero them
    for (int i = rel; i < 512; i += kPrepThreads - 64) {
      const int mb = 2 * (i >> 8), rr = (i >> 4) & 15, cc = i & 15;
      sT[(16 * mb + rr) * TP + 16 * (mb + 1) + cc] = 0.f;
    }
    for (int i = rel; i < 64 * KD / 4; i += kPrepThreads - 64) {
      const int t = i / (KD / 4), cc = 4 * (i % (KD / 4)), m = t >> 4;
      f32x4 pre = {0.f, 0.f, 0.f, 0.f};
      for (int kb = 0; kb < m; ++kb) pre += ld4(sTot + kb * KD + cc);
      f32x4 k4 = ld4(sK + t * DP + cc);
      const f32x4 l4 = ld4(sL + t * DP + cc);
#pragma unroll
      for (int j = 0; j < 4; ++j) k4[j] *= fexp2(pre[j] + l4[j]);
      st4(sK + t * DP + cc, k4);
    }
  }
  __syncthreads();
  // off-diagonal blocks: T_mn = -T_mm sum_{k=n}^{m-1} (Diag(b)A)_mk T_kn, n = m - d
#pragma unroll
  for (int d = 1; d < 4; ++d) {
    const bool act = wave < 4 - d;
    const int m = wave + d, n = wave;
    const int rr = lane >> 2, cc = 4 * (lane & 3);
    float *P = sP + wave * 16 * 17;
    if (act) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 16
      for (int kk = 0; kk < 16 * d; ++kk) {
        const int k = 16 * n + kk;
        acc += sA[(16 * m + rr) * TP + k] * ld4(sT + k * TP + 16 * n + cc);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) P[rr * 17 + cc + e] = acc[e];
    }
    __syncthreads();
    if (act) {
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const float tv = sT[(16 * m + rr) * TP + 16 * m + q];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = fmaf(tv, P[q * 17 + cc + e], acc[e]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) sT[(16 * m + rr) * TP + 16 * n + cc + e] = -acc[e];
    }
    __syncthreads();
  }

  // ---- phase 4: U = T' V and -W^T = -(g.K)^T T'^T, T' = T Diag(b) ---------------
  {
    const int tb = wave & 3, qq = wave >> 2;
    const int nks = tb < 2 ? 1 : 2;  // T' is lower triangular
    const int t = 16 * tb + r16;
    Split TF[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (ks < nks) {
        float v[8];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int i0 = 32 * ks + 16 * hf + 4 * g4;  // tokens 32ks + pk(g4, 4hf + j)
          const f32x4 tv = ld4(sT + t * TP + i0), bv = ld4(sB + i0);
#pragma unroll
          for (int j = 0; j < 4; ++j) v[4 * hf + j] = tv[j] * bv[j];
        }
        TF[ks] = split8(v);
      }
    }
#pragma unroll 1
    for (int vb = qq; vb < NCB; vb += 4) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (ks < nks) {
          float v[8];
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const f32x4 x4 = ld4(sV + (16 * vb + r16) * TP + 32 * ks + 16 * hf + 4 * g4);
#pragma unroll
            for (int j = 0; j < 4; ++j) v[4 * hf + j] = x4[j];
          }
          acc = mfma3(TF[ks], split8(v), acc);
        }
      }
      *reinterpret_cast<f32x4 *>(rec + RC::UF + size_t(tb * NCB + vb) * 1024 + lane * 16) = acc;
    }
#pragma unroll 1
    for (int ksc = qq; ksc < NKS; ksc += 4) {
      f32x4 acc2[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int cc = 16 * (2 * ksc + hh) + r16;
        acc2[hh] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          if (ks < nks) {
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = sK[(32 * ks + pk(g4, e)) * DP + cc];
            acc2[hh] = mfma3(split8(v), TF[ks], acc2[hh]);
          }
        }
      }
      // lane (t, g4) holds W[16tb + r16][32ksc + pk(g4, e)]; the record keeps -W
      float w[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        w[j] = -acc2[0][j];
        w[4 + j] = -acc2[1][j];
      }
      frag_store(rec + RC::WF, tb * NKS + ksc, lane, split8(w));
    }
  }
}

// =============================================================== scan kernel ==
template <typename TS>
__device__ __forceinline__ f32x4 load_state4(const TS *p);
template <>
__device__ __forceinline__ f32x4 load_state4<float>(const float *p) { return ld4(p); }
template <>
__device__ __forceinline__ f32x4 load_state4<uint16_t>(const uint16_t *p) {
  const u32x2 u = *reinterpret_cast<const u32x2 *>(p);
  return f32x4{__uint_as_float(u[0] << 16), __uint_as_float(u[0] & 0xffff0000u), __uint_as_float(u[1] << 16),
               __uint_as_float(u[1] & 0xffff0000u)};
}
__device__ __forceinline__ void store_state4(float *p, const f32x4 &v) { st4(p, v); }
__device__ __forceinline__ void store_state4(uint16_t *p, const f32x4 &v) {
  u32x2 u;
  u[0] = pack_bf16x2(v[0], v[1]);
  u[1] = pack_bf16x2(v[2], v[3]);
  *reinterpret_cast<u32x2 *>(p) = u;
}
__device__ __forceinline__ void store_state(float *p, float v) { *p = v; }
__device__ __forceinline__ void store_state(uint16_t *p, float v) { *p = f32_to_bf16(v); }

// One fragment pair (hi, lo) of the record held by buffer resource r; byte_off is
// wave-uniform, so the address needs no per-lane arithmetic.
__device__ __forceinline__ Split frag_buf(__amdgpu_buffer_rsrc_t r, int voff, int byte_off) {
  Split s;
  s.hi = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, byte_off, 0));
  s.lo = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, byte_off + 1024, 0));
  return s;
}
__device__ __forceinline__ f32x4 f4_buf(__amdgpu_buffer_rsrc_t r, int voff, int byte_off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, byte_off, 0));
}
__device__ __forceinline__ void split4(const f32x4 &v, bf16x4 &hi, bf16x4 &lo) {
  const Split2 a = split2(v[0], v[1]), b = split2(v[2], v[3]);
  hi = __builtin_bit_cast(bf16x4, u32x2{a.hi, b.hi});
  lo = __builtin_bit_cast(bf16x4, u32x2{a.lo, b.lo});
}

template <int D, typename TS>
__global__ __launch_bounds__((128 * Rec<D>::NKS)) void prefill_scan_kernel(KArgs ka) {
  using RC = Rec<D>;
  constexpr int NW = RC::NKS, NT = 128 * NW, NCB = RC::NCB;
  constexpr int TBW = 4 / NW;  // 16-token blocks per wave
  // every wave's two channel tiles exist unless D = 16 (then tile 1 is padding);
  // keeping the guards compile-time leaves the chunk loop without branches, so
  // the wait counts at its head cover only the operands actually needed
  constexpr bool kAllCb = 2 * NW <= NCB;
  // entry-state operand fragments of each 32-channel slice, and Dl operand
  // fragments of each 32-token step (two 16-token halves of 4 values per lane)
  __shared__ bf16x8 sS[NW][2][64];
  __shared__ bf16x4 sD[2][2][64][2];

  const PrefillArgs &a = ka.a;
  const int H = ka.heads, VT = ka.vt_count;
  // consecutive workgroups go to different XCDs; give each XCD a contiguous range
  // of (request, head, V-tile) ids so that the V-tiles of one head share an L2
  const int nblk = gridDim.x, lin = blockIdx.x;
  const int qn = nblk / 8, rn = nblk % 8, xcd = lin % 8;
  const int id = xcd * qn + min(xcd, rn) + lin / 8;
  const int bh = id / VT, vt = id % VT, b = bh / H, h = bh % H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g4 = lane >> 4;
  const int v0 = 16 * vt;

  const ReqGeom rg = req_geom(a, b);
  if (!rg.ok) {
    if (ka.err && ka.c0 == 0 && vt == 0 && h == 0 && tid == 0) atomicOr(ka.err, GDN_ERRW_BAD_SEQLENS);
    return;
  }
  const int slot = a.slot_table[b];
  const int cend = min(ka.c0 + ka.w, rg.nch);
  if (slot <= 0 || slot >= ka.slots) {
    if (slot >= ka.slots && ka.err && ka.c0 == 0 && vt == 0 && h == 0 && tid == 0)
      atomicOr(ka.err, GDN_ERRW_BAD_SLOT);
    for (int c = ka.c0; c < cend; ++c)
      for (int i = tid; i < 64 * 16; i += NT) {
        const int pos = 64 * c - rg.off + i / 16;
        if (pos >= 0 && pos < rg.len) a.out[(int64_t(rg.bos + pos) * H + h) * D + v0 + i % 16] = 0;
      }
    return;
  }
  const bool warm = a.has_initial_state[b] != 0;
  const int64_t C = int64_t(H) * 3 * D;
  TS *ssm = static_cast<TS *>(ka.ssm);
  TS *Slive = ssm + ((int64_t(a.layer) * ka.slots + slot) * H + h) * int64_t(D) * D;
  float *carry = reinterpret_cast<float *>(ka.ws) + (int64_t(b) * H + h) * D * D;
  uint16_t *conv_live = ka.conv + (int64_t(a.layer) * ka.slots + slot) * kConvRows * C;

  // conv rows of head h at request position q (raw x, or the slot's rows before the call)
  auto conv_row_value = [&](int q, int64_t ch) -> uint16_t {
    if (q >= 0) return a.x[int64_t(rg.bos + q) * C + ch];
    return warm ? conv_live[int64_t(3 + q) * C + ch] : uint16_t(0);
  };

  if (rg.nch == 0) {  // empty request: a cold start still zeroes the slot
    if (ka.c0 == 0 && !warm) {
      for (int i = tid; i < 16 * D; i += NT) store_state(Slive + int64_t(v0) * D + i, 0.f);
      if (vt == 0)
        for (int i = tid; i < 3 * 3 * D; i += NT) {
          const int row = i / (3 * D), k = i % (3 * D);
          const int64_t ch = int64_t(k / D) * H * D + int64_t(h) * D + k % D;
          conv_live[row * C + ch] = 0;
        }
    }
    return;
  }
  if (ka.c0 >= rg.nch) return;

  // ---- roles: waves 0..NW-1 carry the state recurrence (Δ and the state update);
  // waves NW..2NW-1 form the outputs (g.Q S0^T + M Δ) and store them.  Both run the
  // same chunk loop with the same two barriers per chunk: A (the entry state's
  // operand fragments are in LDS) and B (Δ's fragments are in LDS).  Each LDS
  // buffer is read before the barrier that precedes its next write, so one copy of
  // each suffices.
  const bool state_wave = wave < NW;
  const int tw = state_wave ? wave : wave - NW;  // this wave's first 16-token block

  // ---- state: lane (r16, g4) of state wave w holds S[v0 + r16][16cb + 4g4 + j], cb = 2w + hh
  f32x4 S[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int cb = 2 * wave + hh;
    S[hh] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (state_wave && (kAllCb || cb < NCB)) {
      const int64_t o = int64_t(v0 + r16) * D + 16 * cb + 4 * g4;
      if (ka.c0 > 0) S[hh] = ld4(carry + o);
      else if (warm) S[hh] = load_state4<TS>(Slive + o);
    }
  }

  // snapshots: every boundary of the call is stored, or with GDN_F_SNAP_LAST_ONLY
  // only the last boundary of each ping-pong parity (an earlier one is overwritten
  // by a later boundary of the same call, so the pool afterwards is the same);
  // per-request values are read once here so that no load inside the chunk loop
  // waits behind the operand loads
  int sl = 0, nxt = 0, trk0 = 0, trk1 = 0, snap_lo = 0x7fffffff;
  if (a.snap_interval > 0) {
    sl = a.start_len[b];
    nxt = a.next_track_idx[b];
    trk0 = a.track_slots[2 * b];
    trk1 = a.track_slots[2 * b + 1];
    snap_lo = (a.flags & GDN_F_SNAP_LAST_ONLY)
                  ? (sl + rg.len) / a.snap_interval - sl / a.snap_interval - 2
                  : 0;
  }
  // the track slot a chunk ending at request position `done` snapshots into, or 0
  auto snap_dst = [&](int done) {
    const int n_end = sl + done;
    const int j = n_end / a.snap_interval - sl / a.snap_interval - 1;
    if (n_end % a.snap_interval != 0 || j < snap_lo) return 0;
    return ((nxt + j) & 1) ? trk1 : trk0;
  };

  // operands of one chunk for this wave: the state waves' token blocks (W, U) and
  // channel tiles (G(63,.)K, g_63); the output waves' token blocks (g.Q, M)
  auto rec_rsrc = [&](int cc) {
    return __builtin_amdgcn_make_buffer_rsrc(
        ka.ws + ka.rec_off + (size_t(b * ka.w + (cc - ka.c0)) * H + h) * RC::BYTES, 0, int(RC::BYTES),
        0x00020000);
  };
  const int voff = lane * 16;
  Split Wn[TBW][NW], Qn[TBW][NW], Mn[TBW][2], Kn[2][2];
  f32x4 Un[TBW], Gn[2];
  auto load_wu = [&](__amdgpu_buffer_rsrc_t r) {
#pragma unroll
    for (int u = 0; u < TBW; ++u) {
      const int tb = tw + NW * u;
#pragma unroll
      for (int ks = 0; ks < NW; ++ks) Wn[u][ks] = frag_buf(r, voff, int(RC::WF) + (tb * NW + ks) * 2048);
      Un[u] = f4_buf(r, voff, int(RC::UF) + (tb * NCB + vt) * 1024);
    }
  };
  auto load_q = [&](__amdgpu_buffer_rsrc_t r) {
#pragma unroll
    for (int u = 0; u < TBW; ++u) {
      const int tb = tw + NW * u;
#pragma unroll
      for (int ks = 0; ks < NW; ++ks) Qn[u][ks] = frag_buf(r, voff, int(RC::QF) + (tb * NW + ks) * 2048);
    }
  };
  auto load_kg = [&](__amdgpu_buffer_rsrc_t r) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int cb = 2 * wave + hh;
      if (kAllCb || cb < NCB) {
#pragma unroll
        for (int ksp = 0; ksp < 2; ++ksp) Kn[hh][ksp] = frag_buf(r, voff, int(RC::KF) + (cb * 2 + ksp) * 2048);
        Gn[hh] = f4_buf(r, g4 * 16, int(RC::GC) + cb * 64);
      }
    }
  };
  // (KM: the k steps of M that hold nonzero tiles for this wave's token blocks)
  auto load_m = [&](__amdgpu_buffer_rsrc_t r, auto km) {
    constexpr int KM = decltype(km)::value;
#pragma unroll
    for (int u = 0; u < TBW; ++u) {
      const int tb = tw + NW * u;
#pragma unroll
      for (int ksp = 0; ksp < KM; ++ksp) Mn[u][ksp] = frag_buf(r, voff, int(RC::MF) + (tb * 2 + ksp) * 2048);
    }
  };
  // the entry state's operand fragments (all channel slices) and Δ's (all tokens)
  auto read_sf = [&](Split (&Sf)[NW]) {
#pragma unroll
    for (int ks = 0; ks < NW; ++ks) {
      Sf[ks].hi = sS[ks][0][lane];
      Sf[ks].lo = sS[ks][1][lane];
    }
  };
  auto read_db = [&](Split (&Db)[2]) {
#pragma unroll
    for (int ksp = 0; ksp < 2; ++ksp) {
      Db[ksp].hi = *reinterpret_cast<const bf16x8 *>(&sD[ksp][0][lane][0]);
      Db[ksp].lo = *reinterpret_cast<const bf16x8 *>(&sD[ksp][1][lane][0]);
    }
  };

  if (state_wave) {
    {
      // same issue order as inside the loop, so that the wait counts the compiler
      // derives at the loop head do not force later groups to land early
      const __amdgpu_buffer_rsrc_t r0 = rec_rsrc(ka.c0);
      load_wu(r0);
      __builtin_amdgcn_sched_barrier(0);
      load_kg(r0);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll 1
    for (int c = ka.c0; c < cend; ++c) {
      const __amdgpu_buffer_rsrc_t rnext = rec_rsrc(min(c + 1, cend - 1));  // next chunk's operands

      // this wave's channel slice of the entry state, as an operand, to every wave
      {
        const Split sb = split44(S[0], S[1]);
        sS[wave][0][lane] = sb.hi;
        sS[wave][1][lane] = sb.lo;
      }
      __syncthreads();  // A
      Split Sf[NW];
      read_sf(Sf);

      // Dl = U - W S0^T for this wave's token blocks (the record keeps -W)
#pragma unroll
      for (int u = 0; u < TBW; ++u) {
        const int tb = tw + NW * u;
        f32x4 d = Un[u];
#pragma unroll
        for (int ks = 0; ks < NW; ++ks) d = mfma3(Wn[u][ks], Sf[ks], d);
        bf16x4 dh, dl;
        split4(d, dh, dl);
        sD[tb >> 1][0][lane][tb & 1] = dh;
        sD[tb >> 1][1][lane][tb & 1] = dl;
      }
      load_wu(rnext);
      __syncthreads();  // B
      Split Db[2];
      read_db(Db);

      // S = S Diag(g_63) + Dl^T (G(63,.) K) on this wave's channels
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        if (kAllCb || 2 * wave + hh < NCB) {
          S[hh] *= Gn[hh];
#pragma unroll
          for (int ksp = 0; ksp < 2; ++ksp) S[hh] = mfma3(Kn[hh][ksp], Db[ksp], S[hh]);
        }
      }
      load_kg(rnext);

      // snapshot of the state at a boundary that ends this chunk (the output waves
      // copy the conv rows)
      if (a.snap_interval > 0) {
        const int dst = snap_dst(min(64 * (c + 1) - rg.off, rg.len));
        if (dst >= ka.slots) {
          if (ka.err && vt == 0 && tid == 0) atomicOr(ka.err, GDN_ERRW_BAD_TRACK_SLOT);
        } else if (dst > 0) {
          TS *Sdst = ssm + ((int64_t(a.layer) * ka.slots + dst) * H + h) * int64_t(D) * D;
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int cb = 2 * wave + hh;
            if (kAllCb || cb < NCB) store_state4(Sdst + int64_t(v0 + r16) * D + 16 * cb + 4 * g4, S[hh]);
          }
        }
      }
    }
  } else {
    const int otid = tid - 64 * NW;  // thread index among the output waves
    // conv rows of a boundary snapshot of head h: 3 rows x (q, k, v) x D channels,
    // one 16-byte piece per output thread.  The piece of chunk c's boundary is
    // loaded during chunk c - 1, right after that chunk's Q operands, so that its
    // store in chunk c waits on no load issued later (loads and stores retire in
    // issue order through one counter).
    constexpr int kSegPieces = D / 8, kConvPieces = 9 * kSegPieces;
    const bool conv_snap_thread = a.snap_interval > 0 && vt == 0 && otid < kConvPieces;
    const int cp_row = otid / (3 * kSegPieces), cp_seg = (otid / kSegPieces) % 3;
    const int64_t cp_ch = int64_t(cp_seg) * H * D + int64_t(h) * D + (otid % kSegPieces) * 8;
    auto conv_fetch = [&](int cc, int &dst) -> u32x4 {
      dst = 0;
      if (!conv_snap_thread || cc >= cend) return u32x4{0u, 0u, 0u, 0u};
      const int done = min(64 * (cc + 1) - rg.off, rg.len);
      dst = snap_dst(done);
      if (dst <= 0 || dst >= ka.slots) return u32x4{0u, 0u, 0u, 0u};
      const int q = done - 3 + cp_row;
      if (q >= 0) return *reinterpret_cast<const u32x4 *>(a.x + int64_t(rg.bos + q) * C + cp_ch);
      if (warm) return *reinterpret_cast<const u32x4 *>(conv_live + int64_t(3 + q) * C + cp_ch);
      return u32x4{0u, 0u, 0u, 0u};
    };
    // The tiles of M above the diagonal are zero: a wave whose only token block
    // is 0 or 1 reads and multiplies its first k step of M alone.  The choice is made
    // once, outside the chunk loop, so each loop has fixed loads.
    auto run = [&](auto km) {
    int cdst;
    u32x4 cpiece;
    {
      const __amdgpu_buffer_rsrc_t r0 = rec_rsrc(ka.c0);
      load_q(r0);
      __builtin_amdgcn_sched_barrier(0);
      cpiece = conv_fetch(ka.c0, cdst);
      __builtin_amdgcn_sched_barrier(0);
      load_m(r0, km);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll 1
    for (int c = ka.c0; c < cend; ++c) {
      const __amdgpu_buffer_rsrc_t rnext = rec_rsrc(min(c + 1, cend - 1));
      __syncthreads();  // A
      Split Sf[NW];
      read_sf(Sf);
      // (g.Q) S0^T for this wave's token blocks
      f32x4 Oq[TBW];
#pragma unroll
      for (int u = 0; u < TBW; ++u) {
        Oq[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NW; ++ks) Oq[u] = mfma3(Qn[u][ks], Sf[ks], Oq[u]);
      }
      load_q(rnext);
      __builtin_amdgcn_sched_barrier(0);
      int cdst_next;
      const u32x4 cpiece_next = conv_fetch(c + 1, cdst_next);
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();  // B
      Split Db[2];
      read_db(Db);

      // O = (g.Q) S0^T + M Dl; the stores go through a buffer resource spanning this
      // chunk's rows of the request, and a padding token's offset lies outside it,
      // so the hardware drops that store
      const int pbase = max(64 * c - rg.off, 0), pend = min(64 * c - rg.off + 64, rg.len);
      const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
          a.out + (int64_t(rg.bos) + pbase) * H * D, 0, (pend - pbase) * H * D * 2, 0x00020000);
#pragma unroll
      for (int u = 0; u < TBW; ++u) {
        const int tb = tw + NW * u;
        f32x4 o = Oq[u];
#pragma unroll
        for (int ksp = 0; ksp < decltype(km)::value; ++ksp) o = mfma3(Mn[u][ksp], Db[ksp], o);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int pos = 64 * c - rg.off + 16 * tb + 4 * g4 + j;
          const int offs = (pos >= pbase && pos < pend) ? (((pos - pbase) * H + h) * D + v0 + r16) * 2 : 0x7fffffff;
          __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(a.scale * o[j]), orsrc, offs, 0, 0);
        }
      }
      load_m(rnext, km);

      // conv rows of a snapshot at a boundary that ends this chunk
      if (cdst > 0 && cdst < ka.slots) {
        uint16_t *conv_dst = ka.conv + (int64_t(a.layer) * ka.slots + cdst) * kConvRows * C;
        *reinterpret_cast<u32x4 *>(conv_dst + int64_t(cp_row) * C + cp_ch) = cpiece;
      }
      cpiece = cpiece_next;
      cdst = cdst_next;
    }
    };
    if (TBW == 1 && tw < 2) run(std::integral_constant<int, 1>());
    else run(std::integral_constant<int, 2>());
  }

  // ---- end of the window: live slot (request done) or the carry ----------------
  const bool done_all = cend == rg.nch;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int cb = 2 * wave + hh;
    if (state_wave && (kAllCb || cb < NCB)) {
      const int64_t o = int64_t(v0 + r16) * D + 16 * cb + 4 * g4;
      if (done_all) store_state4(Slive + o, S[hh]);
      else st4(carry + o, S[hh]);
    }
  }
  if (done_all && vt == 0) {
    // read every new row before writing any: the old rows may be inputs
    constexpr int NI = (9 * D + NT - 1) / NT;
    uint16_t nv[NI];
#pragma unroll
    for (int u = 0; u < NI; ++u) {
      const int i = tid + u * NT;
      if (i < 9 * D) {
        const int row = i / (3 * D), k = i % (3 * D);
        const int64_t ch = int64_t(k / D) * H * D + int64_t(h) * D + k % D;
        nv[u] = conv_row_value(rg.len - 3 + row, ch);
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < NI; ++u) {
      const int i = tid + u * NT;
      if (i < 9 * D) {
        const int row = i / (3 * D), k = i % (3 * D);
        const int64_t ch = int64_t(k / D) * H * D + int64_t(h) * D + k % D;
        conv_live[row * C + ch] = nv[u];
      }
    }
  }
}

// ================================================================ dispatch ==
template <int D>
hipError_t launch_prep(const KArgs &ka, hipStream_t s) {
  const dim3 grid(ka.a.batch * ka.w, ka.heads);
  if (ka.a.alpha_mode == GDN_ALPHA_PER_CHANNEL)
    hipLaunchKernelGGL((prefill_prep_kernel<D, GDN_ALPHA_PER_CHANNEL>), grid, dim3(kPrepThreads), 0, s, ka);
  else
    hipLaunchKernelGGL((prefill_prep_kernel<D, GDN_ALPHA_PER_HEAD>), grid, dim3(kPrepThreads), 0, s, ka);
  return hipGetLastError();
}

template <int D>
hipError_t launch_scan(const KArgs &ka, bool bf, hipStream_t s) {
  const dim3 grid(unsigned(ka.a.batch) * ka.heads * ka.vt_count), block(128 * Rec<D>::NKS);
  if (bf) hipLaunchKernelGGL((prefill_scan_kernel<D, uint16_t>), grid, block, 0, s, ka);
  else hipLaunchKernelGGL((prefill_scan_kernel<D, float>), grid, block, 0, s, ka);
  return hipGetLastError();
}

#define GDN_TRY(x)                        \
  do {                                    \
    const hipError_t e_ = (x);            \
    if (e_ != hipSuccess) return e_;      \
  } while (0)

template <int D>
hipError_t launch_d(const gdn_pool *p, const PrefillArgs &a, hipStream_t s) {
  const int B = a.batch, H = p->d.heads;
  const size_t rec = Rec<D>::BYTES;
  const size_t carry = (size_t(B) * H * D * D * 4 + 255) / 256 * 256;
  const int nch_max = a.start_len ? (a.max_seqlen + 126) / 64 : (a.max_seqlen + 63) / 64;
  const size_t avail = (a.workspace_bytes - carry) / (size_t(B) * H * rec);  // chunks per window
  constexpr int VT = D / 16;  // one scan workgroup per 16 rows of V
  KArgs ka{a, p->d.ssm_base, static_cast<uint16_t *>(p->d.conv_base), p->d.err_word,
           p->d.slots, H, 0, 1, VT, static_cast<char *>(a.workspace), carry};
  const bool bf = p->d.ssm_dtype == GDN_BF16;

  // Windows on the caller's stream: as many chunks per window as the workspace
  // holds (all of them when it is large enough).
  int w = int(avail < size_t(nch_max) ? avail : size_t(nch_max));
  if (w < 1) w = 1;
  ka.w = w;
  const int rounds = nch_max > 0 ? (nch_max + w - 1) / w : 1;
  for (int rnd = 0; rnd < rounds; ++rnd) {
    ka.c0 = rnd * w;
    if (nch_max > 0) GDN_TRY(launch_prep<D>(ka, s));
    GDN_TRY(launch_scan<D>(ka, bf, s));
  }
  return hipSuccess;
}

#undef GDN_TRY

}  // namespace

size_t prefill_record_bytes(const gdn_pool *p) {
  switch (p->d.head_k) {
    case 16: return Rec<16>::BYTES;
    case 32: return Rec<32>::BYTES;
    case 64: return Rec<64>::BYTES;
    default: return Rec<128>::BYTES;
  }
}

size_t prefill_carry_bytes(const gdn_pool *p, int batch) {
  return (size_t(batch) * p->d.heads * p->d.head_v * p->d.head_k * 4 + 255) / 256 * 256;
}

hipError_t launch_prefill(const gdn_pool *p, const PrefillArgs &a, hipStream_t s) {
  switch (p->d.head_k) {
    case 16: return launch_d<16>(p, a, s);
    case 32: return launch_d<32>(p, a, s);
    case 64: return launch_d<64>(p, a, s);
    case 128: return launch_d<128>(p, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
