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
//   prep  (one workgroup per (request, chunk, head); all chunks in parallel):
//         conv + key norm, log2 decays, A and M, T, and the chunk's operands
//         W, U, g.Q, G(63,.)K, M, g_63 written to a workspace record.  Every
//         contraction here runs on bf16 MFMA in a three-product hi/lo split, so
//         it carries about 16 mantissa bits and fp32 range.
//   scan  (one workgroup per (request, head, V-tile); serial over chunks):
//         Dl = U - W S0^T, O = gQ S0^T + M Dl, S = S Diag(g) + Dl^T K~ with the
//         same hi/lo bf16 split, the state held in fp32 registers across chunks;
//         snapshots at boundaries; the live slot written at the end.  The
//         record stores W, g.Q, K~ and M as pre-split bf16 planes, which the
//         scan loads straight into MFMA operand registers.
//
// Chunks are aligned to absolute positions: the first chunk of a request starts
// at start_len rounded down to a multiple of 64 and is padded at the front
// (pad tokens have a = 1, b = 0, k = q = v = 0, which leaves the state exactly
// unchanged), so every snapshot boundary is a chunk end.
//
// Decay products are handled in log2 space inside a chunk: every factor is
// exp2 of a difference of partial sums that is <= 0, except on the diagonal
// 16x16 blocks where the factorisation goes through the block's middle token
// (factors up to 2^60); a block whose channels span more than that uses an
// exact per-pair evaluation instead.
#include "common.hpp"

namespace gdn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr float kMidRange = 60.f;  // max |log2| of a factor on the diagonal fast path

// ------------------------------------------------------------ record layout --
template <int D>
struct Rec {
  // bf16 hi/lo planes (x ~ hi + lo) of the scan's operands, then fp32 arrays
  static constexpr size_t WH = 0;                          // [64][D]  W
  static constexpr size_t WL = WH + size_t(64) * D * 2;
  static constexpr size_t QH = WL + size_t(64) * D * 2;    // [64][D]  g_t q_t
  static constexpr size_t QL = QH + size_t(64) * D * 2;
  static constexpr size_t KH = QL + size_t(64) * D * 2;    // [D][64]  G(63,t) k_t, transposed
  static constexpr size_t KL = KH + size_t(64) * D * 2;
  static constexpr size_t MH = KL + size_t(64) * D * 2;    // [64][64] M
  static constexpr size_t ML = MH + size_t(64) * 64 * 2;
  static constexpr size_t U = ML + size_t(64) * 64 * 2;    // fp32 [64][D]
  static constexpr size_t GC = U + size_t(64) * D * 4;     // fp32 [D]   g_63
  static constexpr size_t BYTES = (GC + size_t(D) * 4 + 255) / 256 * 256;
};

struct KArgs {
  PrefillArgs a;
  void *ssm;
  uint16_t *conv;
  int32_t *err;
  int slots, heads;
  int c0, w, vt_count;
  char *ws;            // workspace base
  size_t carry_bytes;  // fp32 state carry at the start of the workspace
};

struct ReqGeom {
  int bos, len, off, nch;
  bool ok;
};

__device__ __forceinline__ ReqGeom req_geom(const PrefillArgs &a, int b) {
  ReqGeom g;
  g.bos = a.cu_seqlens[b];
  const int eos = a.cu_seqlens[b + 1];
  g.len = eos - g.bos;
  const int sl = a.start_len ? a.start_len[b] : 0;
  g.ok = g.bos >= 0 && g.len >= 0 && eos <= a.total_tokens && g.len <= a.max_seqlen && sl >= 0;
  g.off = sl & 63;
  g.nch = (g.ok && g.len > 0) ? (g.off + g.len + 63) / 64 : 0;
  return g;
}

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8 &a, const bf16x8 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(const f16x8 &a, const f16x8 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

struct Split {
  bf16x8 hi, lo;
};
__device__ __forceinline__ Split split8(const float *v) {
  Split s;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 h = static_cast<__bf16>(v[e]);
    s.hi[e] = h;
    s.lo[e] = static_cast<__bf16>(v[e] - static_cast<float>(h));
  }
  return s;
}
// a*b ~ a_hi b_hi + a_hi b_lo + a_lo b_hi (the lo*lo term is ~2^-16 relative)
__device__ __forceinline__ f32x4 mfma3(const Split &a, const Split &b, f32x4 c) {
  c = mfma_bf16(a.lo, b.hi, c);
  c = mfma_bf16(a.hi, b.lo, c);
  c = mfma_bf16(a.hi, b.hi, c);
  return c;
}

__device__ __forceinline__ void split1(float v, __bf16 &hi, __bf16 &lo) {
  hi = static_cast<__bf16>(v);
  lo = static_cast<__bf16>(v - static_cast<float>(hi));
}
__device__ __forceinline__ bf16x8 neg8(const bf16x8 &v) {
  u32x4 u = __builtin_bit_cast(u32x4, v);
  u ^= 0x80008000u;
  return __builtin_bit_cast(bf16x8, u);
}
__device__ __forceinline__ Split load_split(const __bf16 *hi, const __bf16 *lo) {
  Split s;
  s.hi = *reinterpret_cast<const bf16x8 *>(hi);
  s.lo = *reinterpret_cast<const bf16x8 *>(lo);
  return s;
}

__device__ __forceinline__ void load_bf16x8(const uint16_t *p, float *f) {
  const u32x4 r = *reinterpret_cast<const u32x4 *>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(r[i] << 16);
    f[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
  }
}

// =============================================================== prep kernel ==
template <int D>
struct PrepLds {
  static constexpr int KD = D < 32 ? 32 : D;  // channel extent padded to an MFMA k-step
  static constexpr int DP = KD + 4;           // fp32 pitch of [t][c] arrays
  static constexpr int TP = 68;               // fp32 pitch of [c][t] and [t][i] arrays
  static constexpr int RQ = (64 * DP > KD * TP ? 64 * DP : KD * TP);  // q, later (g.k)^T
  static constexpr int RK = 64 * DP;                                  // k
  static constexpr int RL = (64 * DP > 64 * TP ? 64 * DP : 64 * TP);  // log2 decays, later T
  static constexpr int RV = KD * TP;                                  // v^T
  static constexpr int RA = 64 * TP;                                  // Diag(b) A
  static constexpr int RP = 4 * 16 * 17;                              // per-wave 16x16 scratch
  static constexpr int RTOT = 4 * KD;                                 // block totals of log2 a
  static constexpr int OQ = 0, OK = OQ + RQ, OL = OK + RK, OV = OL + RL, OA = OV + RV,
                       OP = OA + RA, OTOT = OP + RP, OB = OTOT + RTOT, TOTAL = OB + 64 + 4;
};

template <int D, int AMODE>
__global__ __launch_bounds__(kThreads) void prefill_prep_kernel(KArgs ka) {
  using LY = PrepLds<D>;
  constexpr int KD = LY::KD, DP = LY::DP, TP = LY::TP;
  constexpr int G = D / 8;  // 8-channel groups per head part
  __shared__ __attribute__((aligned(16))) float smem[LY::TOTAL];
  float *sQ = smem + LY::OQ, *sK = smem + LY::OK, *sL = smem + LY::OL, *sV = smem + LY::OV;
  float *sA = smem + LY::OA, *sP = smem + LY::OP, *sTot = smem + LY::OTOT, *sB = smem + LY::OB;
  int *sFlag = reinterpret_cast<int *>(smem + LY::OB + 64);
  float *sKG = sQ;  // (g . k)^T [KD][TP], after q is consumed
  float *sT = sL;   // T [64][TP], after the decays are consumed

  const PrefillArgs &a = ka.a;
  const int H = ka.heads;
  const int b = blockIdx.x / ka.w, cl = blockIdx.x % ka.w, c = ka.c0 + cl, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;

  const ReqGeom rg = req_geom(a, b);
  const int slot = a.slot_table[b];
  if (!rg.ok || slot <= 0 || slot >= ka.slots || c >= rg.nch) return;
  const bool warm = a.has_initial_state[b] != 0;
  const int64_t C = int64_t(H) * 3 * D;
  char *rec = ka.ws + ka.carry_bytes + (size_t(b * ka.w + cl) * H + h) * Rec<D>::BYTES;
  const int p0 = 64 * c - rg.off;  // request position of local token 0

  // ---- phase 1: zero fills, beta, log2 decays ---------------------------------
  for (int i = tid; i < 64 * TP; i += kThreads) sA[i] = 0.f;
  for (int i = tid; i < 64 * DP; i += kThreads) {
    sQ[i] = 0.f;
    sK[i] = 0.f;
  }
  for (int i = tid; i < KD * TP; i += kThreads) sV[i] = 0.f;
  if (tid == 0) *sFlag = 0;
  if (tid >= 192) {
    const int t = tid - 192;
    const int pos = p0 + t;
    sB[t] = (pos >= 0 && pos < rg.len) ? a.beta[int64_t(rg.bos + pos) * H + h] : 0.f;
  }
  __syncthreads();
  if (tid < KD) {
    const int ch = tid;
    float acc = 0.f;
#pragma unroll 4
    for (int t = 0; t < 64; ++t) {
      if ((t & 15) == 0) acc = 0.f;
      const int pos = p0 + t;
      float la = 0.f;
      if (ch < D && pos >= 0 && pos < rg.len) {
        const float av = AMODE == GDN_ALPHA_PER_CHANNEL
                             ? a.alpha[(int64_t(rg.bos + pos) * H + h) * D + ch]
                             : a.alpha[int64_t(rg.bos + pos) * H + h];
        la = fmaxf(__log2f(av), -512.f);  // a == 0 behaves as a full decay
      }
      acc += la;
      sL[t * DP + ch] = acc;  // cumulative inside the 16-token block
      if ((t & 15) == 15) sTot[(t >> 4) * KD + ch] = acc;
    }
    int flags = 0;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const float lr = sL[(16 * m + 7) * DP + ch];
      const float up = sL[(16 * m) * DP + ch] - lr, dn = lr - sL[(16 * m + 15) * DP + ch];
      if (fmaxf(up, dn) > kMidRange) flags |= 1 << m;
    }
    if (flags) atomicOr(sFlag, flags);
  }

  // ---- phase 2: causal conv, key (and query) norm -----------------------------
  {
    const uint16_t *crow = ka.conv + (int64_t(a.layer) * ka.slots + slot) * kConvRows * C;
    constexpr int ITEMS = 64 * G;
    constexpr int ITERS = (ITEMS + kThreads - 1) / kThreads;
#pragma unroll 1
    for (int part = 0; part < 3; ++part) {
#pragma unroll 1
      for (int it = 0; it < ITERS; ++it) {
        const int item = it * kThreads + tid;
        const bool active = item < ITEMS;
        const int t = active ? item / G : 0, g = active ? item % G : 0;
        const int pos = p0 + t;
        const bool valid = active && pos >= 0 && pos < rg.len;
        const int64_t ch0 = int64_t(part) * H * D + int64_t(h) * D + 8 * g;
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = 0.f;
        if (valid) {
          float wv[8][4];
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            float tmp[8];
            load_bf16x8(a.conv_w + (ch0 + e) * 4, tmp);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              wv[e][j] = tmp[j];
              wv[e + 1][j] = tmp[4 + j];
            }
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {  // tap j multiplies position pos - 3 + j
            const int q = pos - 3 + j;
            float xv[8];
            if (q >= 0) {
              load_bf16x8(a.x + int64_t(rg.bos + q) * C + ch0, xv);
            } else if (warm) {
              load_bf16x8(crow + int64_t(3 + q) * C + ch0, xv);
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e) xv[e] = 0.f;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = j == 0 ? wv[e][0] * xv[e] : fmaf(wv[e][j], xv[e], y[e]);
          }
          if (a.flags & GDN_F_CONV_SILU) {
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = y[e] / (1.f + __expf(-y[e]));
          }
        }
        const bool norm = part == 1 ? (a.flags & GDN_F_L2NORM_K) : part == 0 ? (a.flags & GDN_F_L2NORM_Q) : false;
        if (norm) {  // uniform branch: every lane takes part in the shuffles
          float ss = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) ss = fmaf(y[e], y[e], ss);
#pragma unroll
          for (int off = G / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
          const float inv = 1.f / sqrtf(ss + 1e-6f);
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] *= inv;
        }
        if (active) {
          if (part == 2) {
#pragma unroll
            for (int e = 0; e < 8; ++e) sV[(8 * g + e) * TP + t] = y[e];
          } else {
            float *dst = (part == 0 ? sQ : sK) + t * DP + 8 * g;
#pragma unroll
            for (int e = 0; e < 8; ++e) dst[e] = y[e];
          }
        }
      }
    }
  }
  __syncthreads();

  // ---- phase 3: A and M tiles ---------------------------------------------------
  const int flags = *sFlag;
  {
    __bf16 *recMh = reinterpret_cast<__bf16 *>(rec + Rec<D>::MH);
    __bf16 *recMl = reinterpret_cast<__bf16 *>(rec + Rec<D>::ML);
#pragma unroll 1
    for (int pi = wave; pi < 10; pi += 4) {
      // pair index -> (m, n), n <= m, in the order (0,0) (1,0) (1,1) (2,0) ...
      const int m = pi < 1 ? 0 : pi < 3 ? 1 : pi < 6 ? 2 : 3;
      const int n = pi - m * (m + 1) / 2;
      const bool diag = m == n;
      const int t = 16 * m + r16;  // A-operand row
      const int i = 16 * n + r16;  // B-operand column
      f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accM = {0.f, 0.f, 0.f, 0.f};
      if (!(diag && ((flags >> m) & 1))) {
        const int r = 16 * m + 7;
#pragma unroll 1
        for (int ks = 0; ks < KD / 32; ++ks) {
          const int c0 = ks * 32 + 8 * g4;
          float rv[8], lk[8], lq[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int cc = c0 + e;
            float rexp, lexp;
            if (diag) {
              const float lr = sL[r * DP + cc];
              rexp = lr - sL[i * DP + cc];
              lexp = sL[t * DP + cc] - lr;
            } else {
              float between = 0.f;
              for (int kb = n + 1; kb < m; ++kb) between += sTot[kb * KD + cc];
              rexp = sTot[n * KD + cc] - sL[i * DP + cc];
              lexp = sL[t * DP + cc] + between;
            }
            rv[e] = sK[i * DP + cc] * exp2f(rexp);
            const float f = exp2f(lexp);
            lk[e] = sK[t * DP + cc] * f;
            lq[e] = sQ[t * DP + cc] * f;
          }
          const Split R = split8(rv), LK = split8(lk), LQ = split8(lq);
          accA = mfma3(LK, R, accA);
          accM = mfma3(LQ, R, accM);
        }
      } else {
        // exact per-pair evaluation for a diagonal block with extreme decays
        const int ii = 16 * n + r16;
#pragma unroll 1
        for (int j = 0; j < 4; ++j) {
          const int tt = 16 * m + 4 * g4 + j;
          float sa = 0.f, sm = 0.f;
          if (ii <= tt) {
            for (int cc = 0; cc < KD; ++cc) {
              const float f = exp2f(sL[tt * DP + cc] - sL[ii * DP + cc]) * sK[ii * DP + cc];
              sa = fmaf(sK[tt * DP + cc], f, sa);
              sm = fmaf(sQ[tt * DP + cc], f, sm);
            }
          }
          accA[j] = sa;
          accM[j] = sm;
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tt = 16 * m + 4 * g4 + j, ii = 16 * n + r16;
        const float av = (!diag || ii < tt) ? accA[j] : 0.f;
        const float mv = (!diag || ii <= tt) ? accM[j] : 0.f;
        sA[tt * TP + ii] = sB[tt] * av;  // Diag(b) A
        split1(mv, recMh[tt * 64 + ii], recMl[tt * 64 + ii]);
      }
    }
    // upper 16x16 tiles of M are zero
    for (int ui = wave; ui < 6; ui += 4) {
      // (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
      const int um = ui < 3 ? 0 : ui < 5 ? 1 : 2;
      const int un = ui < 3 ? ui + 1 : ui < 5 ? ui - 1 : 3;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int o = (16 * um + 4 * g4 + j) * 64 + 16 * un + r16;
        recMh[o] = static_cast<__bf16>(0.f);
        recMl[o] = static_cast<__bf16>(0.f);
      }
    }
  }

  // ---- phase 4: operands for the scan: g.Q, G(63,.)K (transposed), g_63 -------
  {
    __bf16 *recQh = reinterpret_cast<__bf16 *>(rec + Rec<D>::QH);
    __bf16 *recQl = reinterpret_cast<__bf16 *>(rec + Rec<D>::QL);
    __bf16 *recKh = reinterpret_cast<__bf16 *>(rec + Rec<D>::KH);
    __bf16 *recKl = reinterpret_cast<__bf16 *>(rec + Rec<D>::KL);
    float *recGC = reinterpret_cast<float *>(rec + Rec<D>::GC);
    for (int it = tid; it < 64 * G; it += kThreads) {
      const int t = it / G, cg = (it % G) * 8, m = t >> 4;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float pre = 0.f;
        for (int kb = 0; kb < m; ++kb) pre += sTot[kb * KD + cg + e];
        v[e] = sQ[t * DP + cg + e] * exp2f(pre + sL[t * DP + cg + e]);
      }
      const Split sp = split8(v);
      *reinterpret_cast<bf16x8 *>(recQh + t * D + cg) = sp.hi;
      *reinterpret_cast<bf16x8 *>(recQl + t * D + cg) = sp.lo;
    }
    for (int it = tid; it < D * 8; it += kThreads) {
      const int ch = it / 8, t0 = (it % 8) * 8, m = t0 >> 4;
      float post = sTot[m * KD + ch];
      for (int kb = m + 1; kb < 4; ++kb) post += sTot[kb * KD + ch];
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = sK[(t0 + e) * DP + ch] * exp2f(post - sL[(t0 + e) * DP + ch]);
      const Split sp = split8(v);
      *reinterpret_cast<bf16x8 *>(recKh + ch * 64 + t0) = sp.hi;
      *reinterpret_cast<bf16x8 *>(recKl + ch * 64 + t0) = sp.lo;
    }
    for (int ch = tid; ch < D; ch += kThreads) {
      float s = 0.f;
      for (int kb = 0; kb < 4; ++kb) s += sTot[kb * KD + ch];
      recGC[ch] = exp2f(s);
    }
  }
  __syncthreads();
  // (g . k)^T into the q region
  for (int it = tid; it < KD * 64; it += kThreads) {
    const int ch = it / 64, t = it % 64, m = t >> 4;
    float pre = 0.f;
    for (int kb = 0; kb < m; ++kb) pre += sTot[kb * KD + ch];
    sKG[ch * TP + t] = sK[t * DP + ch] * exp2f(pre + sL[t * DP + ch]);
  }
  __syncthreads();

  // ---- phase 5: T = (I + Diag(b) A)^-1, blockwise -------------------------------
  for (int i = tid; i < 64 * TP; i += kThreads) sT[i] = 0.f;
  __syncthreads();
  if (lane < 16) {  // diagonal blocks: wave m inverts block m, lane j owns column j
    const int m = wave, j = lane;
    float x[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      float v = (t == j) ? 1.f : 0.f;
#pragma unroll
      for (int i = 0; i < t; ++i) v = fmaf(-sA[(16 * m + t) * TP + 16 * m + i], x[i], v);
      x[t] = v;
      sT[(16 * m + t) * TP + 16 * m + j] = v;
    }
  }
  __syncthreads();
#pragma unroll 1
  for (int d = 1; d < 4; ++d) {
    // T_mn = -T_mm sum_{k=n}^{m-1} (Diag(b)A)_mk T_kn,  n = m - d, one wave per block
    const bool act = wave < 4 - d;
    const int m = wave + d, n = wave;
    const int rr = lane >> 2, cc = 4 * (lane & 3);
    float *P = sP + wave * 16 * 17;
    if (act) {
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
      for (int k = 16 * n; k < 16 * m; ++k) {
        const float l = sA[(16 * m + rr) * TP + k];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = fmaf(l, sT[k * TP + 16 * n + cc + e], acc[e]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) P[rr * 17 + cc + e] = acc[e];
    }
    __syncthreads();
    if (act) {
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
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

  // ---- phase 6: U = T' V and W = T' (g.K), T' = T Diag(b) -----------------------
  {
    float *recU = reinterpret_cast<float *>(rec + Rec<D>::U);
    __bf16 *recWh = reinterpret_cast<__bf16 *>(rec + Rec<D>::WH);
    __bf16 *recWl = reinterpret_cast<__bf16 *>(rec + Rec<D>::WL);
    const int tb = wave;                 // 16-row block of tokens
    const int nks = tb < 2 ? 1 : 2;      // T' is lower triangular
    Split Af[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (ks < nks) {
        float v[8];
        const int t = 16 * tb + r16, i0 = 32 * ks + 8 * g4;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = sT[t * TP + i0 + e] * sB[i0 + e];
        Af[ks] = split8(v);
      }
    }
#pragma unroll 1
    for (int which = 0; which < 2; ++which) {
      const float *src = which == 0 ? sV : sKG;
#pragma unroll 1
      for (int vb = 0; vb < D / 16; ++vb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          if (ks < nks) {
            float v[8];
            const int col = 16 * vb + r16, i0 = 32 * ks + 8 * g4;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = src[col * TP + i0 + e];
            acc = mfma3(Af[ks], split8(v), acc);
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = 16 * tb + 4 * g4 + j, col = 16 * vb + r16;
          if (which == 0) recU[t * D + col] = acc[j];
          else split1(acc[j], recWh[t * D + col], recWl[t * D + col]);
        }
      }
    }
  }
}

// =============================================================== scan kernel ==
template <int D, int VTR>
struct ScanLds {
  static constexpr int KD = D < 32 ? 32 : D;
  static constexpr int KP = KD + 8;  // bf16 pitch of [v][c] rows (16-byte rows, +4 banks)
  static constexpr int TP = 72;      // bf16 pitch of [v][t] rows
  static constexpr int OSH = 0, OSL = OSH + VTR * KP, ODH = OSL + VTR * KP, ODL = ODH + VTR * TP,
                       TOTAL = ODL + VTR * TP;
};

template <typename TS>
__device__ __forceinline__ float load_state(const TS *p);
template <>
__device__ __forceinline__ float load_state<float>(const float *p) { return *p; }
template <>
__device__ __forceinline__ float load_state<uint16_t>(const uint16_t *p) { return bf16_to_f32(*p); }
__device__ __forceinline__ void store_state(float *p, float v) { *p = v; }
__device__ __forceinline__ void store_state(uint16_t *p, float v) { *p = f32_to_bf16(v); }

template <int D, int VTR, typename TS>
__global__ __launch_bounds__(kThreads) void prefill_scan_kernel(KArgs ka) {
  using LY = ScanLds<D, VTR>;
  constexpr int KD = LY::KD, KP = LY::KP, TP = LY::TP;
  constexpr int NVB = VTR / 16, NCB = D / 16;
  constexpr int NTS = NVB * NCB;                  // 16x16 state tiles of this V-tile
  constexpr int MAXT = (NTS + 3) / 4;             // per wave
  __shared__ __attribute__((aligned(16))) __bf16 smem[LY::TOTAL];
  __bf16 *sSh = smem + LY::OSH, *sSl = smem + LY::OSL;  // S0 [v][c] hi/lo
  __bf16 *sDh = smem + LY::ODH, *sDl = smem + LY::ODL;  // Dl^T [v][t] hi/lo

  const PrefillArgs &a = ka.a;
  const int H = ka.heads;
  const int VT = ka.vt_count;
  const int b = blockIdx.x / VT, vt = blockIdx.x % VT, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int v0 = vt * VTR;

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
      for (int i = tid; i < 64 * VTR; i += kThreads) {
        const int pos = 64 * c - rg.off + i / VTR;
        if (pos >= 0 && pos < rg.len)
          a.out[(int64_t(rg.bos + pos) * H + h) * D + v0 + i % VTR] = 0;
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
      for (int i = tid; i < VTR * D; i += kThreads) store_state(Slive + int64_t(v0) * D + i, 0.f);
      if (vt == 0)
        for (int i = tid; i < 3 * 3 * D; i += kThreads) {
          const int row = i / (3 * D), k = i % (3 * D);
          const int64_t ch = int64_t(k / D) * H * D + int64_t(h) * D + k % D;
          conv_live[row * C + ch] = 0;
        }
    }
    return;
  }
  if (ka.c0 >= rg.nch) return;

  // zero the channel padding of S0 once (only when D < 32)
  if (KD != D)
    for (int i = tid; i < VTR * KP; i += kThreads) {
      sSh[i] = static_cast<__bf16>(0.f);
      sSl[i] = static_cast<__bf16>(0.f);
    }

  // ---- state in registers: wave owns tiles tt = wave + 4k -----------------------
  f32x4 S[MAXT];
#pragma unroll
  for (int k = 0; k < MAXT; ++k) {
    const int tt = wave + 4 * k;
    const int vb = tt / NCB, cb = tt % NCB;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v = 0.f;
      if (tt < NTS) {
        const int row = v0 + 16 * vb + 4 * g4 + j, col = 16 * cb + r16;
        if (ka.c0 > 0) v = carry[int64_t(row) * D + col];
        else if (warm) v = load_state<TS>(Slive + int64_t(row) * D + col);
      }
      S[k][j] = v;
    }
  }

  const int nks2 = wave < 2 ? 1 : 2;  // M is lower triangular
#pragma unroll 1
  for (int c = ka.c0; c < cend; ++c) {
    const char *rec = ka.ws + ka.carry_bytes + (size_t(b * ka.w + (c - ka.c0)) * H + h) * Rec<D>::BYTES;
    const __bf16 *Wh = reinterpret_cast<const __bf16 *>(rec + Rec<D>::WH);
    const __bf16 *Wl = reinterpret_cast<const __bf16 *>(rec + Rec<D>::WL);
    const __bf16 *Qh = reinterpret_cast<const __bf16 *>(rec + Rec<D>::QH);
    const __bf16 *Ql = reinterpret_cast<const __bf16 *>(rec + Rec<D>::QL);
    const __bf16 *Kh = reinterpret_cast<const __bf16 *>(rec + Rec<D>::KH);
    const __bf16 *Kl = reinterpret_cast<const __bf16 *>(rec + Rec<D>::KL);
    const __bf16 *Mh = reinterpret_cast<const __bf16 *>(rec + Rec<D>::MH);
    const __bf16 *Ml = reinterpret_cast<const __bf16 *>(rec + Rec<D>::ML);
    const float *recU = reinterpret_cast<const float *>(rec + Rec<D>::U);
    const float *recGC = reinterpret_cast<const float *>(rec + Rec<D>::GC);

    // the wave's rows of W (for Dl) and of g.Q and M (for O): direct operand loads
    Split Wf[KD / 32], Qf[KD / 32], Mf[2];
#pragma unroll
    for (int ks = 0; ks < KD / 32; ++ks) {
      if (32 * ks + 8 * g4 < D) {
        const int o = (16 * wave + r16) * D + 32 * ks + 8 * g4;
        Wf[ks] = load_split(Wh + o, Wl + o);
        Wf[ks].hi = neg8(Wf[ks].hi);
        Wf[ks].lo = neg8(Wf[ks].lo);
        Qf[ks] = load_split(Qh + o, Ql + o);
      } else {  // channel padding (D < 32)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          Wf[ks].hi[e] = Wf[ks].lo[e] = Qf[ks].hi[e] = Qf[ks].lo[e] = static_cast<__bf16>(0.f);
        }
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int o = (16 * wave + r16) * 64 + 32 * ks + 8 * g4;
      Mf[ks] = load_split(Mh + o, Ml + o);
    }

    // the entry state as split operands
#pragma unroll
    for (int k = 0; k < MAXT; ++k) {
      const int tt = wave + 4 * k;
      if (tt < NTS) {
        const int vb = tt / NCB, cb = tt % NCB;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int o = (16 * vb + 4 * g4 + j) * KP + 16 * cb + r16;
          split1(S[k][j], sSh[o], sSl[o]);
        }
      }
    }
    __syncthreads();

    // Dl = U - W S0^T   (wave = 16-token block)
#pragma unroll 1
    for (int vb = 0; vb < NVB; ++vb) {
      f32x4 acc;
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = recU[(16 * wave + 4 * g4 + j) * D + v0 + 16 * vb + r16];
#pragma unroll
      for (int ks = 0; ks < KD / 32; ++ks) {
        const int o = (16 * vb + r16) * KP + 32 * ks + 8 * g4;
        acc = mfma3(Wf[ks], load_split(sSh + o, sSl + o), acc);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int o = (16 * vb + r16) * TP + 16 * wave + 4 * g4 + j;
        split1(acc[j], sDh[o], sDl[o]);
      }
    }
    __syncthreads();

    // O = (g.Q) S0^T + M Dl
#pragma unroll 1
    for (int vb = 0; vb < NVB; ++vb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KD / 32; ++ks) {
        const int o = (16 * vb + r16) * KP + 32 * ks + 8 * g4;
        acc = mfma3(Qf[ks], load_split(sSh + o, sSl + o), acc);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (ks < nks2) {
          const int o = (16 * vb + r16) * TP + 32 * ks + 8 * g4;
          acc = mfma3(Mf[ks], load_split(sDh + o, sDl + o), acc);
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int pos = 64 * c - rg.off + 16 * wave + 4 * g4 + j;
        if (pos >= 0 && pos < rg.len)
          a.out[(int64_t(rg.bos + pos) * H + h) * D + v0 + 16 * vb + r16] = f32_to_bf16(a.scale * acc[j]);
      }
    }

    // S = S Diag(g_63) + Dl^T (G(63,.) K)
#pragma unroll
    for (int k = 0; k < MAXT; ++k) {
      const int tt = wave + 4 * k;
      if (tt < NTS) {
        const int vb = tt / NCB, cb = tt % NCB;
        const float gc = recGC[16 * cb + r16];
#pragma unroll
        for (int j = 0; j < 4; ++j) S[k][j] *= gc;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int od = (16 * vb + r16) * TP + 32 * ks + 8 * g4;
          const int ok = (16 * cb + r16) * 64 + 32 * ks + 8 * g4;
          S[k] = mfma3(load_split(sDh + od, sDl + od), load_split(Kh + ok, Kl + ok), S[k]);
        }
      }
    }

    // snapshot at a boundary that ends this chunk
    if (a.snap_interval > 0) {
      const int sl = a.start_len[b];
      const int done = min(64 * (c + 1) - rg.off, rg.len);
      const int n_end = sl + done;
      if (n_end % a.snap_interval == 0) {
        const int j = n_end / a.snap_interval - sl / a.snap_interval - 1;
        const int dst = a.track_slots[2 * b + ((a.next_track_idx[b] + j) & 1)];
        if (dst >= ka.slots) {
          if (ka.err && vt == 0 && tid == 0) atomicOr(ka.err, GDN_ERRW_BAD_TRACK_SLOT);
        } else if (dst > 0) {
          TS *Sdst = ssm + ((int64_t(a.layer) * ka.slots + dst) * H + h) * int64_t(D) * D;
#pragma unroll
          for (int k = 0; k < MAXT; ++k) {
            const int tt = wave + 4 * k;
            if (tt < NTS) {
              const int vb = tt / NCB, cb = tt % NCB;
#pragma unroll
              for (int jj = 0; jj < 4; ++jj)
                store_state(Sdst + int64_t(v0 + 16 * vb + 4 * g4 + jj) * D + 16 * cb + r16, S[k][jj]);
            }
          }
          if (vt == 0) {
            uint16_t *conv_dst = ka.conv + (int64_t(a.layer) * ka.slots + dst) * kConvRows * C;
            for (int i = tid; i < 3 * 3 * D; i += kThreads) {
              const int row = i / (3 * D), k = i % (3 * D);
              const int64_t ch = int64_t(k / D) * H * D + int64_t(h) * D + k % D;
              conv_dst[row * C + ch] = conv_row_value(done - 3 + row, ch);
            }
          }
        }
      }
    }
    __syncthreads();
  }

  // ---- end of the window: live slot (request done) or the carry ----------------
  const bool done_all = cend == rg.nch;
#pragma unroll
  for (int k = 0; k < MAXT; ++k) {
    const int tt = wave + 4 * k;
    if (tt < NTS) {
      const int vb = tt / NCB, cb = tt % NCB;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t o = int64_t(v0 + 16 * vb + 4 * g4 + j) * D + 16 * cb + r16;
        if (done_all) store_state(Slive + o, S[k][j]);
        else carry[o] = S[k][j];
      }
    }
  }
  if (done_all && vt == 0) {
    // read every new row before writing any: the old rows may be inputs
    constexpr int NI = (9 * D + kThreads - 1) / kThreads;
    uint16_t nv[NI];
#pragma unroll
    for (int u = 0; u < NI; ++u) {
      const int i = tid + u * kThreads;
      if (i < 9 * D) {
        const int row = i / (3 * D), k = i % (3 * D);
        const int64_t ch = int64_t(k / D) * H * D + int64_t(h) * D + k % D;
        nv[u] = conv_row_value(rg.len - 3 + row, ch);
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < NI; ++u) {
      const int i = tid + u * kThreads;
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
hipError_t launch_d(const gdn_pool *p, const PrefillArgs &a, hipStream_t s) {
  const int B = a.batch, H = p->d.heads;
  const size_t rec = Rec<D>::BYTES;
  const size_t carry = (size_t(B) * H * D * D * 4 + 255) / 256 * 256;
  const int nch_max = a.start_len ? (a.max_seqlen + 126) / 64 : (a.max_seqlen + 63) / 64;
  size_t avail = (a.workspace_bytes - carry) / (size_t(B) * H * rec);
  int w = int(avail < size_t(nch_max) ? avail : size_t(nch_max));
  if (w < 1) w = 1;
  // V-tiles: enough workgroups to cover the chip when batch x heads is small
  int vtr = D;
  while (vtr > 16 && int64_t(B) * H * (D / vtr) < 512) vtr /= 2;
  KArgs ka{a, p->d.ssm_base, static_cast<uint16_t *>(p->d.conv_base), p->d.err_word,
           p->d.slots, H, 0, w, D / vtr, static_cast<char *>(a.workspace), carry};
  const bool bf = p->d.ssm_dtype == GDN_BF16;
  const int rounds = nch_max > 0 ? (nch_max + w - 1) / w : 1;
  for (int rnd = 0; rnd < rounds; ++rnd) {
    ka.c0 = rnd * w;
    if (nch_max > 0) {
      dim3 grid(B * w, H);
      if (a.alpha_mode == GDN_ALPHA_PER_CHANNEL)
        hipLaunchKernelGGL((prefill_prep_kernel<D, GDN_ALPHA_PER_CHANNEL>), grid, dim3(kThreads), 0, s, ka);
      else
        hipLaunchKernelGGL((prefill_prep_kernel<D, GDN_ALPHA_PER_HEAD>), grid, dim3(kThreads), 0, s, ka);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    dim3 grid(B * ka.vt_count, H);
#define GDN_SCAN(VTR_)                                                                        \
  if (vtr == VTR_) {                                                                          \
    if (bf) hipLaunchKernelGGL((prefill_scan_kernel<D, VTR_, uint16_t>), grid, dim3(kThreads), 0, s, ka); \
    else hipLaunchKernelGGL((prefill_scan_kernel<D, VTR_, float>), grid, dim3(kThreads), 0, s, ka);      \
  }
    if constexpr (D >= 16) { GDN_SCAN(16) }
    if constexpr (D >= 32) { GDN_SCAN(32) }
    if constexpr (D >= 64) { GDN_SCAN(64) }
    if constexpr (D >= 128) { GDN_SCAN(128) }
#undef GDN_SCAN
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

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
