// prefill_fused.hip -- chunked prefill in one kernel per (request, head), head dim
// 128: prefill_fused_kernel for a decay shared by all channels of a head (the GDN
// form, described here), prefill_fused_kda_kernel for a decay per channel (the KDA
// form, described where it starts below).
//
// The recurrence (page "企业官网建设流程全解析", Kimi K3 notes, section
// "Speculative decoding")
//     S_t = a_t S_{t-1} + d_t k_t^T,   d_t = b_t (v_t - a_t S_{t-1} k_t),   o_t = scale S_t q_t
// is unrolled over chunks of 64 tokens (page "SGLang Mamba Radix Cache 深度解析",
// configuration: chunk size 64).  With G(t, i) = prod_{i < tau <= t} a_tau and
// g_t = G(t, -1) inside a chunk whose entry state is S0:
//     A[t][i] = G(t,i) k_t.k_i (i < t),      M[t][i] = G(t,i) q_t.k_i (i <= t)
//     (I + Diag(b) A) Dl = Diag(b) (V - Diag(g) K S0^T)    (rows d_t)
//     O  = Diag(g) Q S0^T + M Dl
//     S_end = g_63 S0 + Dl^T Diag(G(63, .)) K
// (the chunked form the oracle's tests check against the sequential one, with the
// decay taken out of the products: a scalar per token commutes with them).  Every
// factor G is applied outside a product as a number <= 1, so any decay, down to
// a = 0, is handled without a range problem.
//
// One workgroup of 8 waves takes one (request, head) and walks all of the
// request's chunks with the state in registers: wave w owns the rows v in
// [16w, 16w + 16), held transposed (tiles of S^T, 16 channels x 16 rows) in fp32
// accumulators.  Per chunk:
//   P1  conv + norms of q and k (an item is 8 channels x 4 tokens) written as
//       bf16 hi/lo MFMA fragments K and Q (rows = tokens); raw v rows staged;
//       log2 decays (cumulated) and b (wave 0).
//   P2  waves 0-3: the diagonal 16x16 block m = w of N = Diag(b) A and the
//       inverse D_m of I + N_mm by forward substitution; waves 4-7: the M
//       fragments and the blocks of N below the diagonal blocks.  Then every
//       wave: K S0^T and Q S0^T for its rows, its V values from the staged rows,
//       and Y = Diag(b) (V - Diag(g) K S0^T).
//   P3  every wave: Dl for its rows by block forward substitution,
//       Dl_m = D_m (Y_m - sum_{k<m} N_mk Dl_k), then O (staged in LDS and
//       written out as whole rows during the next chunk) and the state update,
//       whose K^T operand is read from the K fragments by transposing LDS reads;
//       a snapshot when the chunk ends on a boundary.
// Every contraction runs on bf16 MFMA in the three-product hi/lo split of
// mfma.hpp.  Accumulators enter the next product without a transpose (the k order
// pk), and fragments in LDS are stored in operand order.
#include <type_traits>

#include "common.hpp"
#include "lanes.hpp"
#include "mfma.hpp"

namespace gdn {
namespace {

constexpr int kFD = 128;      // head dim K = V
constexpr int kFThreads = 512;
constexpr int kOrderedBatch = 1024;  // batches up to this size are taken longest request first

// ---------------------------------------------------------------- LDS layout --
// A fragment is one bf16 plane (hi or lo) of one 16x16x32 operand: 64 lanes x 8
// values, 1 KiB, lane-major.
constexpr int kKN = 0;                    // K  [tb 4][ks 4][plane 2]
constexpr int kQN = kKN + 32 * 1024;      // Q  [tb 4][ks 4][plane 2]
constexpr int kMF = kQN + 32 * 1024;      // M  [pair 6][plane 2], pairs (tb, ks), ks <= tb/2
// k = 16 A-operand fragments, split once where they are made: lane l holds row
// l % 16, columns 4(l/16)..+3 of a 16x16 block as hi[4] | lo[4] bf16 (16 bytes)
constexpr int kNF = kMF + 12 * 1024;      // -N_mk, blocks below the diagonal, [6][64][16 B]
constexpr int kDF = kNF + 6 * 1024;       // D_m = (I + N_mm)^-1, [4][64][16 B]
constexpr int kLD = kDF + 4 * 1024;       // diagonal blocks N_mm, then D_m, fp32 [4][16][kBP]
constexpr int kBP = 20;                   // fp32 pitch of a 16x16 block row
// per token t of the chunk: log2 decay L_t cumulated from the chunk start, b_t,
// g_t = 2^L_t and G(63, t) = 2^(L_63 - L_t)
constexpr int kLB = kLD + 4 * 16 * kBP * 4;
// raw v rows [67][256 B]: row i is request position p0 - 3 + i; its 16-byte
// chunks are XOR-swizzled by 2((i >> 2) & 3), so that the four lane groups of a
// wave, which read rows 4 apart, hit different banks
constexpr int kXV = kLB + 256 * 4;
// a chunk's outputs, bf16 [64][kOP bytes]: written in the last phase of a chunk,
// sent out in the first phase of the next
constexpr int kOS = kXV + 67 * 256;
constexpr int kOP = 264;
constexpr int kLdsBytes = kOS + 64 * kOP;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");

__device__ __forceinline__ int xv_off(int row, int byte) {
  return kXV + row * 256 + ((((byte >> 4) ^ (2 * ((row >> 2) & 3))) << 4) | (byte & 15));
}

__device__ __forceinline__ int pair_idx(int tb, int ks) { return tb < 2 ? tb : 2 * tb - 2 + ks; }

// Operand lane l of a K or Q fragment idx (= tb * 4 + ks) is stored in slot
// l ^ (idx & 3) ^ 8((l >> 5) & 1).  The writers fill several fragments at once with
// lanes that would otherwise share banks, and the XOR by idx spreads them.  The
// XOR of bit 3 by bit 5 serves the transposing reads of the state update: a
// 16-lane group of such a read addresses 4 tokens in each of 4 channel octets,
// slots 16 apart, which without it fall on the same banks (measured on gfx950
// with in-bounds probes: 64 -> 45 cycles per read instruction and wave with 8
// waves reading; the 16-byte operand reads and the writers are no slower).
__device__ __forceinline__ int kn_slot(int idx, int l) { return l ^ (idx & 3) ^ (8 * ((l >> 5) & 1)); }
__device__ __forceinline__ int nf_idx(int m, int k) { return m * (m - 1) / 2 + k; }  // m > k

__device__ __forceinline__ void split4_put(char *lds, int off, int lane, const f32x4 &v) {
  const Split4 sp = split4s(v);
  *reinterpret_cast<s16x4 *>(lds + off + lane * 16) = sp.hi;
  *reinterpret_cast<s16x4 *>(lds + off + lane * 16 + 8) = sp.lo;
}
__device__ __forceinline__ Split4 split4_get(const char *lds, int off, int lane) {
  return Split4{*reinterpret_cast<const s16x4 *>(lds + off + lane * 16),
                *reinterpret_cast<const s16x4 *>(lds + off + lane * 16 + 8)};
}

__device__ __forceinline__ Split frag_lds(const char *lds, int off, int idx, int lane) {
  Split s;
  s.hi = *reinterpret_cast<const bf16x8 *>(lds + off + (2 * idx) * 1024 + lane * 16);
  s.lo = *reinterpret_cast<const bf16x8 *>(lds + off + (2 * idx + 1) * 1024 + lane * 16);
  return s;
}

// A K^T operand fragment (rows = channels 16cb..16cb+15, k = tokens 32ks + pk)
// read from the K fragments with the gfx950 transposing LDS read: within each
// 16-lane group, ds_read_b64_tr_b16 hands lane 4a + b element b of the 4 x 16-bit
// chunk addressed by lane 4k + a, as its element k.  So lane 4k + a of group g
// addresses channels 16cb + 4a..+3 of token 32ks + 4g + k (first read) or
// 32ks + 16 + 4g + k (second read); in a K fragment those four channels are one
// 8-byte half of a lane's slot.
typedef short s16x4t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ s16x4t lds_read_tr16(const char *lds, int off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4t *)(const_cast<char *>(lds) + off));
}
// (base: the fragment region; SLOT: its lane-slot permutation; tb_pad: bytes added to
// the fragments of each later token block)
template <typename SLOT>
__device__ __forceinline__ Split kt_frag_at(const char *lds, int base, SLOT slot, int cb, int ks, int lane,
                                            int tb_pad = 0) {
  const int g = lane >> 4, a = lane & 3, k = (lane >> 2) & 3;
  const int kc = cb >> 1, e0 = 4 * (cb & 1);  // channel group of K, first slot of the half
  s16x4t h[2], l[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int t = 32 * ks + 16 * half + 4 * g + k;
    const int idx = (t >> 4) * 4 + kc;
    const int off = base + 2 * idx * 1024 + tb_pad * (idx >> 2) + slot(idx, (t & 15) + 16 * a) * 16 + 2 * e0;
    h[half] = lds_read_tr16(lds, off);
    l[half] = lds_read_tr16(lds, off + 1024);
  }
  Split s;
  s.hi = __builtin_bit_cast(bf16x8, __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7));
  s.lo = __builtin_bit_cast(bf16x8, __builtin_shufflevector(l[0], l[1], 0, 1, 2, 3, 4, 5, 6, 7));
  return s;
}
__device__ __forceinline__ Split kt_frag(const char *lds, int cb, int ks, int lane) {
  return kt_frag_at(lds, kKN, [](int idx, int l) { return kn_slot(idx, l); }, cb, ks, lane);
}

// 4 consecutive values of one fragment lane, both planes, already split
__device__ __forceinline__ void frag_put4w(char *lds, int off, int idx, int lanep, int e0, const Split2 &a,
                                           const Split2 &b) {
  const u32x2 h = {a.hi, b.hi}, l = {a.lo, b.lo};
  *reinterpret_cast<u32x2 *>(lds + off + (2 * idx) * 1024 + lanep * 16 + 2 * e0) = h;
  *reinterpret_cast<u32x2 *>(lds + off + (2 * idx + 1) * 1024 + lanep * 16 + 2 * e0) = l;
}
__device__ __forceinline__ void frag_put4(char *lds, int off, int idx, int lanep, int e0, const float *v) {
  frag_put4w(lds, off, idx, lanep, e0, split2(v[0], v[1]), split2(v[2], v[3]));
}

// Workgroup barrier that orders LDS accesses only: global loads issued before it
// stay in flight (a full __syncthreads would wait for them), which lets the next
// chunk's inputs load across the barriers of the current one.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename TS>
__device__ __forceinline__ f32x4 load_s4(const TS *p);
template <>
__device__ __forceinline__ f32x4 load_s4<float>(const float *p) { return ld4(p); }
template <>
__device__ __forceinline__ f32x4 load_s4<uint16_t>(const uint16_t *p) {
  const u32x2 u = *reinterpret_cast<const u32x2 *>(p);
  return f32x4{__uint_as_float(u[0] << 16), __uint_as_float(u[0] & 0xffff0000u), __uint_as_float(u[1] << 16),
               __uint_as_float(u[1] & 0xffff0000u)};
}
__device__ __forceinline__ void store_s4(float *p, const f32x4 &v) { st4(p, v); }
__device__ __forceinline__ void store_s4(uint16_t *p, const f32x4 &v) {
  *reinterpret_cast<u32x2 *>(p) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}

struct FArgs {
  PrefillArgs a;
  void *ssm;
  uint16_t *conv;
  int32_t *err;
  int slots, heads;
};

// SILU is a template parameter: a flag tested inside the unrolled conv loops costs a
// branch (and register copies at its merge) per conv output.
template <typename TS, bool SILU>
__global__ __launch_bounds__(kFThreads) void prefill_fused_kernel(FArgs fa) {
  constexpr int D = kFD;
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  float *LB = reinterpret_cast<float *>(lds + kLB);  // L, b, g, G(63, .): 64 each

  const PrefillArgs &a = fa.a;
  const int H = fa.heads;
  const int h = blockIdx.x % H;
  const int tid = threadIdx.x, lane = tid & 63;
  // Requests are taken longest first (most chunks; ties by index): workgroups
  // start in index order, so a long request that came late would keep its CU
  // busy after the others finish.  Every workgroup ranks the batch itself.
  int b = blockIdx.x / H;
  if (a.batch <= kOrderedBatch) {
    __shared__ int s_req;
    for (int i = tid; i < a.batch; i += kFThreads) {
      const int ni = req_geom(a, i).nch;
      int rank = 0;
      for (int j = 0; j < a.batch; ++j) {
        const int nj = req_geom(a, j).nch;
        rank += (nj > ni) | ((nj == ni) & (j < i));
      }
      if (rank == b) s_req = i;
    }
    __syncthreads();
    b = s_req;
  }
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;

  const ReqGeom rg = req_geom(a, b);
  if (!rg.ok) {
    if (fa.err && h == 0 && tid == 0) atomicOr(fa.err, GDN_ERRW_BAD_SEQLENS);
    return;
  }
  const int64_t C = int64_t(H) * 3 * D;
  const int slot = a.slot_table[b];
  if (slot <= 0 || slot >= fa.slots) {
    if (slot >= fa.slots && fa.err && h == 0 && tid == 0) atomicOr(fa.err, GDN_ERRW_BAD_SLOT);
    for (int i = tid; i < rg.len * (D / 8); i += kFThreads) {
      const int pos = i / (D / 8), o = i % (D / 8);
      *reinterpret_cast<u32x4 *>(a.out + (int64_t(rg.bos + pos) * H + h) * D + 8 * o) = u32x4{0u, 0u, 0u, 0u};
    }
    return;
  }
  const bool warm = a.has_initial_state[b] != 0;
  TS *ssm = static_cast<TS *>(fa.ssm);
  TS *Slive = ssm + ((int64_t(a.layer) * fa.slots + slot) * H + h) * int64_t(D) * D;
  uint16_t *conv_live = fa.conv + (int64_t(a.layer) * fa.slots + slot) * kConvRows * C;

  // 8 channels (from channel ch) of the input row at request position q.  The
  // request's rows are a buffer resource, and a load whose offset lies outside
  // its range (q < 0 or q >= len) returns zero, so no load is clamped, masked or
  // branched around.  (The one-kernel path is only taken when len * C * 2 bytes
  // fits a signed int.)
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(a.x) + int64_t(rg.bos) * C, 0, rg.len * int(C) * 2, 0x00020000);
  auto row_x = [&](int q, int ch) -> u32x4 {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xres, (q * int(C) + ch) * 2, 0, 0));
  };
  // the same, with positions -3..-1 taken from the slot's conv rows on a warm start
  auto row_vec = [&](int q, int ch) -> u32x4 {
    if (q < 0 && q >= -3 && warm) return *reinterpret_cast<const u32x4 *>(conv_live + (3 + q) * C + ch);
    return row_x(q, ch);
  };
  // the 3 conv rows of head h after `done` tokens: 144 items of 8 channels
  auto conv_item = [&](int i, int done, int &ch, int &row) -> u32x4 {
    row = i / 48;
    const int oc = i % 48;
    ch = (oc >> 4) * H * D + h * D + 8 * (oc & 15);
    return row_vec(done - 3 + row, ch);
  };

  if (rg.nch == 0) {  // empty request: a cold start still zeroes the slot
    if (!warm) {
      for (int i = tid; i < D * D / 4; i += kFThreads) store_s4(Slive + 4 * i, f32x4{0.f, 0.f, 0.f, 0.f});
      for (int i = tid; i < 144; i += kFThreads) {
        const int row = i / 48, oc = i % 48;
        const int64_t ch = int64_t(oc >> 4) * H * D + int64_t(h) * D + 8 * (oc & 15);
        *reinterpret_cast<u32x4 *>(conv_live + row * C + ch) = u32x4{0u, 0u, 0u, 0u};
      }
    }
    return;
  }

  constexpr bool silu = SILU;

  // ---- constants of the call --------------------------------------------------
  // conv item (P1) of waves 0-3: q, of waves 4-7: k
  const bool inorm = (a.flags & (w < 4 ? GDN_F_L2NORM_Q : GDN_F_L2NORM_K)) != 0;
  // taps of this lane's V column
  const int vcol = 16 * w + r;
  const u32x2 vw = *reinterpret_cast<const u32x2 *>(a.conv_w + (2 * int64_t(H) * D + int64_t(h) * D + vcol) * 4);

  // ---- state: lane (r, g) of wave w holds S[16w + r][16kb + 4g + j] in S[kb][j] ----
  f32x4 S[8];
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) {
    S[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (warm) S[kb] = load_s4<TS>(Slive + int64_t(vcol) * D + 16 * kb + 4 * g);
  }

  // snapshots: every boundary of the call is stored, or with GDN_F_SNAP_LAST_ONLY
  // only the last boundary of each ping-pong parity (an earlier one is overwritten
  // by a later one of the same parity)
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

  f32x4 Y[4], OQ[4];  // per chunk: Diag(b) (V - Diag(g) K S0^T) and Diag(g) Q S0^T

  // The staged outputs of the chunk at position p0 go out as 16-byte rows pieces
  // (rows outside the request fall outside the resource and are dropped), NT
  // threads writing 1024 / NT pieces each.
  const __amdgpu_buffer_rsrc_t ores = __builtin_amdgcn_make_buffer_rsrc(
      a.out + (int64_t(rg.bos) * H + h) * D, 0, rg.len * H * D * 2, 0x00020000);
  auto flush_out = [&](int t, int p0, auto nt) {
    constexpr int NT = decltype(nt)::value;
#pragma unroll
    for (int u = 0; u < 1024 / NT; ++u) {
      const int it = t + u * NT, row = it >> 4, pc = it & 15;
      const u32x4 v = *reinterpret_cast<const u32x4 *>(lds + kOS + row * kOP + 16 * pc);
      __builtin_amdgcn_raw_buffer_store_b128(v, ores, ((p0 + row) * H * D + 8 * pc) * 2, 0, 0);
    }
  };

  // Global inputs of a chunk: 7 rows of the thread's conv item, its 3 staged v
  // chunks, and (one token per lane) the decay and b.  They are loaded one chunk
  // ahead, during the previous chunk's last phase; nothing waits for them before
  // the next chunk uses them.  Rows at positions -3..-1 (a warm start's conv
  // rows) are patched in when the chunk is used.
  u32x4 xr[7], sv[3];
  float av, bv;
  const __amdgpu_buffer_rsrc_t ares = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float *>(a.alpha) + int64_t(rg.bos) * H + h, 0, rg.len * H * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t bres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float *>(a.beta) + int64_t(rg.bos) * H + h, 0, rg.len * H * 4, 0x00020000);
  auto load_chunk = [&](int t, int p0) {
    const int co = t & 15, tq = (t & 255) >> 4;
    const int ch0 = (w >> 2) * H * D + h * D + 8 * co;
    // byte offsets: one multiply per thread, then a uniform step per row
    const int rs = int(C) * 2;
    const int xo = ((p0 + 4 * tq - 3) * int(C) + ch0) * 2;
#pragma unroll
    for (int i = 0; i < 7; ++i)
      xr[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xres, xo + i * rs, 0, 0));
    const int it0 = t, vo = ((p0 - 3 + (it0 >> 4)) * int(C) + 2 * H * D + h * D + 8 * (it0 & 15)) * 2;
    // Every load instruction issued here costs the CU's vector-memory path, which
    // bounds this phase: the third group of staged pieces (pieces 1024..1071) is
    // loaded by wave 0 alone, and the decays and b (one token per lane) only by
    // wave 0, which uses them.
#pragma unroll
    for (int u = 0; u < 3; ++u) {  // 67 staged rows x 16 chunks of 16 bytes
      if (u < 2 || w == 0) {
        const int it = t + u * kFThreads;  // row (it >> 4) = (t >> 4) + 32u
        const int off =
            it < 67 * 16 ? vo + 32 * u * rs : ((p0 - 3 + 66) * int(C) + 2 * H * D + h * D + 8 * 15) * 2;
        sv[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xres, off, 0, 0));
      }
    }
    if (w == 0) {
      const int toff = (p0 + (t & 63)) * H * 4;  // outside [0, len) reads zero
      av = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ares, toff, 0, 0));
      bv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(bres, toff, 0, 0));
    }
  };
  load_chunk(tid, -rg.off);
  u32x4 iw[4];  // taps of the conv item's 8 channels
#pragma unroll
  for (int i = 0; i < 4; ++i)
    iw[i] = *reinterpret_cast<const u32x4 *>(
        a.conv_w + (int64_t(w >> 2) * H * D + int64_t(h) * D + 8 * (tid & 15) + 2 * i) * 4);

#pragma unroll 1
  for (int c = 0; c < rg.nch; ++c) {
    const int p0 = 64 * c - rg.off;  // request position of chunk token 0
    // Lane-dependent values are formed anew in every chunk: hoisted out of the
    // loop they would stay live across all of it and spill.
    int tid_c = tid;
    asm volatile("" : "+v"(tid_c));
    const int lane = tid_c & 63, r = lane & 15, g = lane >> 4, vcol = 16 * w + r;  // (shadow the call's)
    // conv item: channels 8co..8co+7 of part w / 4 (q, k), tokens 4tq..4tq+3
    const int co = tid_c & 15, tq = (tid_c & 255) >> 4;

    // Y = Diag(b) (V - Diag(g) K S0^T) and Diag(g) Q S0^T for this wave's rows;
    // V comes from the staged raw rows
    auto ks0_products = [&]() {
      f32x4 X1[4], XQ[4];
  #pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        X1[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
        XQ[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      // fragments of step i = ks * 4 + tb are read one step ahead of their products
      Split kf[2], qf[2], sop;
      kf[0] = frag_lds(lds, kKN, 0, kn_slot(0, lane));
      qf[0] = frag_lds(lds, kQN, 0, kn_slot(0, lane));
  #pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int ks = i >> 2, tb = i & 3;
        if (i + 1 < 16) {
          const int n = ((i + 1) & 3) * 4 + ((i + 1) >> 2);
          kf[(i + 1) & 1] = frag_lds(lds, kKN, n, kn_slot(n, lane));
          qf[(i + 1) & 1] = frag_lds(lds, kQN, n, kn_slot(n, lane));
        }
        if (tb == 0) sop = split44(S[2 * ks], S[2 * ks + 1]);
        X1[tb] = mfma3(kf[i & 1], sop, X1[tb]);
        XQ[tb] = mfma3(qf[i & 1], sop, XQ[tb]);
      }
      // staged row 16tb + 4g + q of this lane's V column: the row swizzle takes one
      // value for q < 4 and another for q >= 4, the same in every tb
      const int xb0 = kXV + 4 * g * 256 + (((vcol >> 3) ^ (2 * (g & 3))) << 4) + 2 * (vcol & 7);
      const int xb1 = kXV + 4 * g * 256 + (((vcol >> 3) ^ (2 * ((g + 1) & 3))) << 4) + 2 * (vcol & 7);
  #pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        // staged rows t0 .. t0 + 6 of this lane's V column, as pairs of adjacent rows
        const int t0 = 16 * tb + 4 * g;
        uint32_t xc[7], xp[6];
  #pragma unroll
        for (int q = 0; q < 7; ++q)
          xc[q] = *reinterpret_cast<const uint16_t *>(lds + (q < 4 ? xb0 : xb1) + tb * 4096 + q * 256);
  #pragma unroll
        for (int q = 0; q < 6; ++q) xp[q] = halves(xc[q], xc[q + 1], 0);
  #pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = t0 + j;
          float acc = dot2_bf16(vw[0], xp[j], 0.f);
          acc = dot2_bf16(vw[1], xp[j + 2], acc);
          if (silu) acc = acc / (1.f + __expf(-acc));
          // a token outside the request has b = 0, so its row of Y is zero whatever
          // its conv value
          const float gt = LB[128 + t];
          Y[tb][j] = LB[64 + t] * (acc - gt * X1[tb][j]);
          OQ[tb][j] = gt * XQ[tb][j];
        }
      }
    };


    // ================= P1: conv, norms, fragments; staged v rows; decays =========
    if (p0 < 3 && warm) {  // rows at positions -3..-1 come from the slot's conv rows
#pragma unroll
      for (int i = 0; i < 7; ++i) xr[i] = row_vec(p0 + 4 * tq - 3 + i, (w >> 2) * H * D + h * D + 8 * co);
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        const int it = min(tid_c + u * kFThreads, 67 * 16 - 1);
        sv[u] = row_vec(p0 - 3 + (it >> 4), 2 * H * D + h * D + 8 * (it & 15));
      }
    }
    const int dpos = p0 + lane;  // decays and b: wave 0, one token per lane
    if (w == 0) {
      const bool valid = dpos >= 0 && dpos < rg.len;
      float la = valid ? fmaxf(__log2f(av), -512.f) : 0.f;  // a == 0: full decay
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const float u = __shfl_up(la, d, 64);
        if (lane >= d) la += u;
      }
      LB[lane] = la;
      LB[64 + lane] = valid ? bv : 0.f;
      LB[128 + lane] = fexp2(la);
      LB[192 + lane] = fexp2(__shfl(la, 63, 64) - la);
    }
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int it = tid_c + u * kFThreads;
      if (it < 67 * 16)
        *reinterpret_cast<u32x4 *>(lds + xv_off(it >> 4, 16 * (it & 15))) = sv[u];
    }
    {
      float y[4][8];
#pragma unroll
      // Tokens outside the request (padding before a warm start's first position,
      // or past its end) keep their conv values: their b is zero, so their rows of
      // Y, of N = Diag(b) A and of Dl are zero, and every product that reads their
      // k or q multiplies it by a zero of Dl (their outputs are not stored).
      for (int rr = 0; rr < 4; ++rr) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // taps (0, 1) and (2, 3) multiply positions (pos - 3, pos - 2) and (pos - 1, pos)
          float acc = dot2_bf16(iw[e >> 1][2 * (e & 1)], tok_pair(xr[rr], xr[rr + 1], e), 0.f);
          acc = dot2_bf16(iw[e >> 1][2 * (e & 1) + 1], tok_pair(xr[rr + 2], xr[rr + 3], e), acc);
          if (silu) acc = acc / (1.f + __expf(-acc));
          y[rr][e] = acc;
        }
      }
      // (the norm's flag in one branch: tested inside the unrolled loop it costs a
      // branch per token)
      if (inorm) {  // wave-uniform; the 16 lanes of a token quad share the sum
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          float ss = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) ss = fmaf(y[rr][e], y[rr][e], ss);
          ss = group_sum<16>(ss);
          // v_rsq_f32 (about 1 ulp): a full-precision square root and division here
          // held the k waves ~1.2k cycles per chunk behind the q waves at the barrier
          const float inv = __builtin_amdgcn_rsqf(ss + 1e-6f);
#pragma unroll
          for (int e = 0; e < 8; ++e) y[rr][e] *= inv;
        }
      }
      // rows = tokens: element (t, 32ks + p) of fragment (t>>4, ks) sits in lane
      // (t&15) + 16((p&15)>>2), slot (p&3) + 4(p>>4)
      // each value is split once (pairs of adjacent channels)
      const int fo = w < 4 ? kQN : kKN;
      Split2 sp[4][4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int t = 4 * tq + rr;
#pragma unroll
        for (int p = 0; p < 4; ++p) sp[rr][p] = split2(y[rr][2 * p], y[rr][2 * p + 1]);
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
          frag_put4w(lds, fo, (t >> 4) * 4 + (co >> 2), kn_slot(co >> 2, (t & 15) + 16 * (2 * (co & 1) + hf)),
                     4 * ((co >> 1) & 1), sp[rr][2 * hf], sp[rr][2 * hf + 1]);
      }
    }
    lds_barrier();

    // ================= P2 =======================================================
    // The next chunk's inputs are issued in two halves, so that the CU's vector-
    // memory path is shared out: waves 0-3 (their P2 work is the latency-bound
    // diagonal inverse) here, waves 4-7 at the start of P3.
    if (w < 4) load_chunk(tid_c, p0 + 64);
    // a transposed M tile (lane holds M[16m+r][16k+4g+j]): decay mask, then this
    // lane's own slot run of the M fragment
    auto put_m = [&](int m, int k, const f32x4 &cc) {
      const int t = 16 * m + r;
      const float lt = LB[t];
      float mv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 16 * k + 4 * g + j;
        mv[j] = i <= t ? fexp2(lt - LB[i]) * cc[j] : 0.f;
      }
      frag_put4(lds, kMF, pair_idx(m, k >> 1), lane, 4 * (k & 1), mv);
      if (m == k && !(m & 1)) {  // block (m, m+1) above the diagonal is zero
        const float z[4] = {0.f, 0.f, 0.f, 0.f};
        frag_put4(lds, kMF, pair_idx(m, m >> 1), lane, 4, z);
      }
    };
    if (w < 4) {
      // diagonal block m of N = Diag(b) A: lane holds k_{16m+4g+j} . k_{16m+r}
      const int m = w;
      f32x4 c2[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const Split kf = frag_lds(lds, kKN, m * 4 + ks, kn_slot(m * 4 + ks, lane));
        c2[ks & 1] = mfma3(kf, kf, c2[ks & 1]);
      }
      const f32x4 cc = c2[0] + c2[1];
      float *blk = reinterpret_cast<float *>(lds + kLD) + m * 16 * kBP;
      const float li = LB[16 * m + r];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 4 * g + j;  // row (token) in the block; column i = r
        blk[t * kBP + r] = t > r ? LB[64 + 16 * m + t] * fexp2(LB[16 * m + t] - li) * cc[j] : 0.f;
      }
      wave_lds_sync();
      // (I + N_mm) X = I, column r (every lane group computes the same column)
      float x[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        float v = (t == r) ? 1.f : 0.f;
#pragma unroll
        for (int i = 0; i < t; ++i) v = fmaf(-blk[t * kBP + i], x[i], v);
        x[t] = v;
      }
      // D_m over N_mm, then split once into its operand fragment
      wave_lds_sync();
      if (g == 0) {
#pragma unroll
        for (int t = 0; t < 16; ++t) blk[t * kBP + r] = x[t];
      }
      wave_lds_sync();
      split4_put(lds, kDF + m * 1024, lane, ld4(blk + r * kBP + 4 * g));
      // and the diagonal M tile (m, m)
      f32x4 cm[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        cm[ks & 1] = mfma3(frag_lds(lds, kKN, m * 4 + ks, kn_slot(m * 4 + ks, lane)),
                           frag_lds(lds, kQN, m * 4 + ks, kn_slot(m * 4 + ks, lane)), cm[ks & 1]);
      put_m(m, m, cm[0] + cm[1]);
    } else {
      // three tiles per wave: the M blocks below the diagonal and the N blocks.
      // Entry (one byte per tile, wave 4 first): type (0 = M, 1 = N) << 4 | m << 2 | k.
      // Wave 4: M10 M20 N10; 5: M21 M30 N20; 6: M31 N21 N30; 7: M32 N31 N32
      constexpr uint64_t kTilesLo = 0x190d180c09140804ull, kTilesHi = 0x1e1d0e1cull;
      auto tile_entry = [&](int q) {
        const int i = (w - 4) * 3 + q;
        return int(((i < 8 ? kTilesLo >> (8 * i) : kTilesHi >> (8 * (i - 8)))) & 0xff);
      };
      // two tiles, then one: products first (independent accumulators), then stores
#pragma unroll
      for (int q0 = 0; q0 < 3; q0 += 2) {
      f32x4 cc[3];
#pragma unroll
      for (int q = q0; q < min(q0 + 2, 3); ++q) cc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int q = q0; q < min(q0 + 2, 3); ++q) {
          const int e = tile_entry(q);
          const int m = (e >> 2) & 3, k = e & 3;
          // transposed tiles: lane holds (k_{16k+4g+j} . q_{16m+r}) = M[16m+r][16k+4g+j]
          // or (k_{16k+4g+j} . k_{16m+r}) = A[16m+r][16k+4g+j], i.e. row r and columns
          // 4g..4g+3 of the block: this lane's own operand slots
          const int ia = k * 4 + ks, ib = m * 4 + ks;
          cc[q] = mfma3(frag_lds(lds, kKN, ia, kn_slot(ia, lane)),
                        frag_lds(lds, (e >> 4) ? kKN : kQN, ib, kn_slot(ib, lane)), cc[q]);
        }
      }
#pragma unroll
      for (int q = q0; q < min(q0 + 2, 3); ++q) {
        const int e = tile_entry(q);
        const int m = (e >> 2) & 3, k = e & 3;
        if ((e >> 4) == 0) {
          put_m(m, k, cc[q]);
        } else {  // -N_mk = -b_t G(t, i) A[t][i]
          const int t = 16 * m + r;
          const float lt = LB[t], bt = LB[64 + t];
          f32x4 nv;
#pragma unroll
          for (int j = 0; j < 4; ++j) nv[j] = -bt * fexp2(lt - LB[16 * k + 4 * g + j]) * cc[q][j];
          split4_put(lds, kNF + nf_idx(m, k) * 1024, lane, nv);
        }
      }
      }
    }
    // the previous chunk's outputs (the staged rows are rewritten only in phase 3):
    // here the stores meet no load issue on the vector-memory path
    if (c > 0) flush_out(tid_c, p0 - 64, std::integral_constant<int, kFThreads>());
    ks0_products();  // every wave, two per SIMD
    lds_barrier();

    // ================= P3: Dl, O, state update ==================================
    if (w >= 4) load_chunk(tid_c, p0 + 64);  // the next chunk's inputs (clamped on the last)
    // (I + N) Dl = Y by blocks: Dl_m = D_m (Y_m - sum_{k<m} N_mk Dl_k); each block of
    // Dl enters the next products as a k = 16 B operand straight from its accumulator
    f32x4 Dl[4];
    {
      Split4 db[3];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        f32x4 acc = Y[m];
#pragma unroll
        for (int k = 0; k < m; ++k) acc = mfma3k16(split4_get(lds, kNF + nf_idx(m, k) * 1024, lane), db[k], acc);
        Dl[m] = mfma3k16(split4_get(lds, kDF + m * 1024, lane), split4s(acc), f32x4{0.f, 0.f, 0.f, 0.f});
        if (m < 3) db[m] = split4s(Dl[m]);
      }
    }
    Split dop[2], dgop[2];
    dop[0] = split44(Dl[0], Dl[1]);
    dop[1] = split44(Dl[2], Dl[3]);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int j = 0; j < 4; ++j) Dl[tb][j] *= LB[192 + 16 * tb + 4 * g + j];  // G(63, t) Dl
    dgop[0] = split44(Dl[0], Dl[1]);
    dgop[1] = split44(Dl[2], Dl[3]);
    // outputs
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      f32x4 o = OQ[tb];
#pragma unroll
      for (int ks = 0; ks <= (tb >> 1); ++ks) o = mfma3(frag_lds(lds, kMF, pair_idx(tb, ks), lane), dop[ks], o);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<uint16_t *>(lds + kOS + (16 * tb + 4 * g + j) * kOP + 2 * vcol) = f32_to_bf16(a.scale * o[j]);
    }
    // S^T = g_63 S0^T + K^T Diag(G(63, .)) Dl
    const float g63 = LB[128 + 63];
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      S[kb] *= g63;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        S[kb] = mfma3(kt_frag(lds, kb, ks, lane), dgop[ks], S[kb]);
    }

    // snapshot at a boundary that ends this chunk
    if (a.snap_interval > 0) {
      const int done = min(64 * (c + 1) - rg.off, rg.len);
      const int n_end = sl + done;
      const int j = n_end / a.snap_interval - sl / a.snap_interval - 1;
      if (n_end % a.snap_interval == 0 && j >= snap_lo) {
        const int dst = ((nxt + j) & 1) ? trk1 : trk0;
        if (dst >= fa.slots) {
          if (fa.err && tid == 0) atomicOr(fa.err, GDN_ERRW_BAD_TRACK_SLOT);
        } else if (dst > 0) {
          TS *Sd = ssm + ((int64_t(a.layer) * fa.slots + dst) * H + h) * int64_t(D) * D;
#pragma unroll
          for (int kb = 0; kb < 8; ++kb) store_s4(Sd + int64_t(vcol) * D + 16 * kb + 4 * g, S[kb]);
          uint16_t *cd = fa.conv + (int64_t(a.layer) * fa.slots + dst) * kConvRows * C;
          if (tid < 144) {
            int ch, row;
            const u32x4 v = conv_item(tid, done, ch, row);
            *reinterpret_cast<u32x4 *>(cd + row * C + ch) = v;
          }
        }
      }
    }
    lds_barrier();  // the next chunk overwrites every fragment
  }

  // ---- end of the request: live slot -------------------------------------------
  flush_out(tid, 64 * (rg.nch - 1) - rg.off, std::integral_constant<int, kFThreads>());
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) store_s4(Slive + int64_t(vcol) * D + 16 * kb + 4 * g, S[kb]);
  // read every new conv row before writing any: the old rows may be inputs
  int ch = 0, row = 0;
  u32x4 nv = {0u, 0u, 0u, 0u};
  if (tid < 144) nv = conv_item(tid, rg.len, ch, row);
  __syncthreads();
  if (tid < 144) *reinterpret_cast<u32x4 *>(conv_live + row * C + ch) = nv;
}

// =========================================================== decay per channel ==
// The same walk for a decay per channel (the KDA form).  With L_t the log2 decay
// of each channel cumulated from the chunk start, g_t = 2^L_t is a vector, and the
// decay factor of a pair (t, i) splits as 2^L_t 2^-L_i.  In a chunk where every
// channel keeps g_63 >= 2^-96, these factors lie within 2^+-96 and are folded into
// three operand planes built once per chunk (rows = tokens):
//     P = k . g,   R = k . g^-1,   Q' = q . g
//     A = P R^T (i < t),   M = Q' R^T (i <= t)
//     (I + Diag(b) A) Dl = Diag(b) (V - P S0^T)
//     O = Q' S0^T + M Dl,   S_end = (S0 + Dl^T R) Diag(g_63)
// (the derivation: unroll S_t = S_{t-1} Diag(a_t) + d_t k_t^T from the chunk start;
// S_{t-1} Diag(a_t) = S0 Diag(g_t) + sum_{i<t} d_i (k_i . 2^(L_t - L_i))^T).  The
// planes hold the conv outputs before the key and query norms, which are scalars
// per token and are applied outside the products.  A conv item here is 4 channels x
// 4 tokens of both q and k, laid out so that the 16 token groups of a channel are
// the 16 lanes of a row: the decay products are scanned across the row with DPP.
// A chunk in which some channel decays below 2^-96 is run token by token instead,
// which is exact for any decay down to a = 0.
// A plane's fragments [tb 4][ks 4][plane 2] of 1 KB; the fragments of token block tb
// start 16 tb bytes later (kTbPad), so that the phase-1 writers, whose 16 lanes of a
// channel group write into all four token blocks at once, reach different banks.
constexpr int kTbPad = 16;
constexpr int kAPlane = 32 * 1024 + 3 * kTbPad;
constexpr int kAP = 0;                         // P
constexpr int kAQ = kAP + kAPlane;             // Q'
constexpr int kAR = kAQ + kAPlane;             // R (a chunk run token by token: a, fp32 [64][128])
constexpr int kAM = kAR + kAPlane;             // M  [pair 6][plane 2]
constexpr int kANF = kAM + 12 * 1024;          // -N_mk
constexpr int kADF = kANF + 6 * 1024;          // D_m
constexpr int kALD = kADF + 4 * 1024;          // diagonal blocks; in phase 1 the norm partial sums [8][64][2]
constexpr int kALB = kALD + 4 * 16 * kBP * 4;  // b, 1/|q|, 1/|k| per token; g_63 per channel; flags
constexpr int kAXV = kALB + 336 * 4;           // raw v rows, as kXV
constexpr int kAOS = kAXV + 67 * 256;          // outputs, as kOS
constexpr int kAW = kAOS + 64 * kOP;           // conv taps of q and k, bf16 [2][128][4]
constexpr int kALdsBytes = kAW + 2 * 128 * 8;
static_assert(kALdsBytes <= 160 * 1024, "LDS budget");
static_assert(8 * 64 * 2 * 4 <= 4 * 16 * kBP * 4, "norm partial sums fit the diagonal-block region");
constexpr int kLbIq = 64, kLbIk = 128, kLbG = 192, kLbFlag = 320;  // float offsets in the kALB block
constexpr float kPlaneFloor = 0x1p-96f;  // smallest g_63 the planes take

// Lane-slot permutation of the plane fragments: as for the decay per head (the XOR by
// idx & 3 spreads writers; bit 3 XORed by bit 5 serves the transposing reads).  With
// the token-block offset kTbPad, the 16 lanes of a channel group, which write 4 tokens
// into each of the 4 token blocks at once, put two lanes on a bank pair instead of
// eight (measured on gfx950 with in-bounds probes: 512 -> 128 cycles per 8-byte
// write pair and wave with 8 waves writing), and every read still adds a constant
// per token block, which folds into the instruction's offset.
__device__ __forceinline__ int ka_slot(int idx, int l) { return l ^ (idx & 3) ^ (8 * ((l >> 5) & 1)); }
__device__ __forceinline__ int ka_frag(int idx) { return kTbPad * (idx >> 2); }  // token-block offset
__device__ __forceinline__ Split ka_frag_lds(const char *lds, int plane, int idx, int lane) {
  return frag_lds(lds, plane + ka_frag(idx), idx, ka_slot(idx, lane));
}

__device__ __forceinline__ int xv_off_at(int base, int row, int byte) {
  return base + row * 256 + ((((byte >> 4) ^ (2 * ((row >> 2) & 3))) << 4) | (byte & 15));
}

// product of v over the lanes at or below this one in its row of 16 (DPP row shifts;
// a lane with no source multiplies by the 1.0 kept as the old value)
template <int N>
__device__ __forceinline__ float row_shr_or_one(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.f), __float_as_int(v), 0x110 + N, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_prefix_prod(float v) {
  v *= row_shr_or_one<1>(v);
  v *= row_shr_or_one<2>(v);
  v *= row_shr_or_one<4>(v);
  v *= row_shr_or_one<8>(v);
  return v;
}
// the value of the lane one down in its row of 16 (lane 0 takes lane 15's): DPP row_ror:1
__device__ __forceinline__ uint32_t row_ror1(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x121, 0xF, 0xF, false));
}
// sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the gfx950 row swaps)
__device__ __forceinline__ float cross_row_sum(float v) {
  const int lane = threadIdx.x & 63;
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v += __uint_as_float((lane & 16) ? r[0] : r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v += __uint_as_float((lane & 32) ? r[0] : r[1]);
  return v;
}

template <typename TS, bool SILU>
__global__ __launch_bounds__(kFThreads) void prefill_fused_kda_kernel(FArgs fa) {
  constexpr int D = kFD;
  __shared__ __attribute__((aligned(16))) char lds[kALdsBytes];
  float *LB = reinterpret_cast<float *>(lds + kALB);  // b, 1/|q|, 1/|k| (64 each), g_63 (128), flags
  int *LF = reinterpret_cast<int *>(lds + kALB) + kLbFlag;
  const auto slot_fn = [](int idx, int l) { return ka_slot(idx, l); };

  const PrefillArgs &a = fa.a;
  const int H = fa.heads;
  const int h = blockIdx.x % H;
  const int tid = threadIdx.x, lane = tid & 63;
  // requests longest first, as in the kernel above
  int b = blockIdx.x / H;
  if (a.batch <= kOrderedBatch) {
    __shared__ int s_req;
    for (int i = tid; i < a.batch; i += kFThreads) {
      const int ni = req_geom(a, i).nch;
      int rank = 0;
      for (int j = 0; j < a.batch; ++j) {
        const int nj = req_geom(a, j).nch;
        rank += (nj > ni) | ((nj == ni) & (j < i));
      }
      if (rank == b) s_req = i;
    }
    __syncthreads();
    b = s_req;
  }
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;

  const ReqGeom rg = req_geom(a, b);
  if (!rg.ok) {
    if (fa.err && h == 0 && tid == 0) atomicOr(fa.err, GDN_ERRW_BAD_SEQLENS);
    return;
  }
  const int64_t C = int64_t(H) * 3 * D;
  const int slot = a.slot_table[b];
  if (slot <= 0 || slot >= fa.slots) {
    if (slot >= fa.slots && fa.err && h == 0 && tid == 0) atomicOr(fa.err, GDN_ERRW_BAD_SLOT);
    for (int i = tid; i < rg.len * (D / 8); i += kFThreads) {
      const int pos = i / (D / 8), o = i % (D / 8);
      *reinterpret_cast<u32x4 *>(a.out + (int64_t(rg.bos + pos) * H + h) * D + 8 * o) = u32x4{0u, 0u, 0u, 0u};
    }
    return;
  }
  const bool warm = a.has_initial_state[b] != 0;
  TS *ssm = static_cast<TS *>(fa.ssm);
  TS *Slive = ssm + ((int64_t(a.layer) * fa.slots + slot) * H + h) * int64_t(D) * D;
  uint16_t *conv_live = fa.conv + (int64_t(a.layer) * fa.slots + slot) * kConvRows * C;

  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(a.x) + int64_t(rg.bos) * C, 0, rg.len * int(C) * 2, 0x00020000);
  auto row_vec = [&](int q, int ch) -> u32x4 {
    if (q < 0 && q >= -3 && warm) return *reinterpret_cast<const u32x4 *>(conv_live + (3 + q) * C + ch);
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xres, (q * int(C) + ch) * 2, 0, 0));
  };
  auto conv_item = [&](int i, int done, int &ch, int &row) -> u32x4 {
    row = i / 48;
    const int oc = i % 48;
    ch = (oc >> 4) * H * D + h * D + 8 * (oc & 15);
    return row_vec(done - 3 + row, ch);
  };

  if (rg.nch == 0) {  // empty request: a cold start still zeroes the slot
    if (!warm) {
      for (int i = tid; i < D * D / 4; i += kFThreads) store_s4(Slive + 4 * i, f32x4{0.f, 0.f, 0.f, 0.f});
      for (int i = tid; i < 144; i += kFThreads) {
        const int row = i / 48, oc = i % 48;
        const int64_t ch = int64_t(oc >> 4) * H * D + int64_t(h) * D + 8 * (oc & 15);
        *reinterpret_cast<u32x4 *>(conv_live + row * C + ch) = u32x4{0u, 0u, 0u, 0u};
      }
    }
    return;
  }

  constexpr bool silu = SILU;
  const bool nq = (a.flags & GDN_F_L2NORM_Q) != 0, nk = (a.flags & GDN_F_L2NORM_K) != 0;
  const int vcol = 16 * w + r;
  const u32x2 vw = *reinterpret_cast<const u32x2 *>(a.conv_w + (2 * int64_t(H) * D + int64_t(h) * D + vcol) * 4);

  // state: lane (r, g) of wave w holds S[16w + r][16kb + 4g + j] in S[kb][j]
  f32x4 S[8];
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) {
    S[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (warm) S[kb] = load_s4<TS>(Slive + int64_t(vcol) * D + 16 * kb + 4 * g);
  }

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

  f32x4 Y[4], OQ[4];

  const __amdgpu_buffer_rsrc_t ores = __builtin_amdgcn_make_buffer_rsrc(
      a.out + (int64_t(rg.bos) * H + h) * D, 0, rg.len * H * D * 2, 0x00020000);
  auto flush_out = [&](int t, int p0) {
#pragma unroll
    for (int u = 0; u < 1024 / kFThreads; ++u) {
      const int it = t + u * kFThreads, row = it >> 4, pc = it & 15;
      const u32x4 v = *reinterpret_cast<const u32x4 *>(lds + kAOS + row * kOP + 16 * pc);
      __builtin_amdgcn_raw_buffer_store_b128(v, ores, ((p0 + row) * H * D + 8 * pc) * 2, 0, 0);
    }
  };

  // Global inputs of a chunk, loaded one chunk ahead: 3 staged v pieces, the rows of
  // the item's 4 tokens (4 channels of q and of k), the item's decays (4 tokens x 4
  // channels) and b (wave 0, one token per lane), in the order phase 1 uses them.
  // The conv's 3 earlier rows are the rows of the lane one token group down (a DPP
  // row rotate); the first group's lanes load theirs into hq / hk (the other lanes
  // address past the range, which reads zero and moves no data).  Positions
  // outside the request read zero through the resources' ranges.
  u32x2 xq[4], xk[4], hq[3], hk[3];
  f32x4 al[4];
  u32x4 sv[3];
  float bv;
  const __amdgpu_buffer_rsrc_t ares = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float *>(a.alpha) + int64_t(rg.bos) * H * D, 0, rg.len * H * D * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t bres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float *>(a.beta) + int64_t(rg.bos) * H + h, 0, rg.len * H * 4, 0x00020000);
  auto load_chunk = [&](int t, int p0) {
    const int tq = t & 15, c0 = 16 * w + 4 * ((t & 63) >> 4);
    const int rs = int(C) * 2;
    const int vo = ((p0 - 3 + (t >> 4)) * int(C) + 2 * H * D + h * D + 8 * (t & 15)) * 2;
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      if (u < 2 || w == 0) {
        const int it = t + u * kFThreads;
        const int off =
            it < 67 * 16 ? vo + 32 * u * rs : ((p0 - 3 + 66) * int(C) + 2 * H * D + h * D + 8 * 15) * 2;
        sv[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xres, off, 0, 0));
      }
    }
    const int xo = ((p0 + 4 * tq) * int(C) + h * D + c0) * 2, ko = xo + H * D * 2;
    const int ho = tq == 0 ? xo - 3 * rs : 0x7ffffff0, hko = tq == 0 ? ko - 3 * rs : 0x7ffffff0;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      hq[i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(xres, ho + i * rs, 0, 0));
      hk[i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(xres, hko + i * rs, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xq[i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(xres, xo + i * rs, 0, 0));
      xk[i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(xres, ko + i * rs, 0, 0));
    }
    const int ao = ((p0 + 4 * tq) * H + h) * D * 4 + c0 * 4;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      al[rr] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ares, ao + rr * H * D * 4, 0, 0));
    if (w == 0)
      bv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(bres, (p0 + (t & 63)) * H * 4, 0, 0));
  };
  load_chunk(tid, -rg.off);
  // conv taps of the head's q and k channels, kept in LDS (registers are short here)
  if (tid < 128) {
    const int part = tid >> 6, ch = tid & 63;  // 2 channels per thread
    *reinterpret_cast<u32x4 *>(lds + kAW + (part * 128 + 2 * ch) * 8) =
        *reinterpret_cast<const u32x4 *>(a.conv_w + (int64_t(part) * H * D + int64_t(h) * D + 2 * ch) * 4);
  }
  __syncthreads();

#pragma unroll 1
  for (int c = 0; c < rg.nch; ++c) {
    const int p0 = 64 * c - rg.off;
    int tid_c = tid;
    asm volatile("" : "+v"(tid_c));
    const int lane = tid_c & 63, r = lane & 15, g = lane >> 4, vcol = 16 * w + r;
    // conv item: tokens 4tq..4tq+3, channels c0..c0+3 of q and of k
    const int tq = lane & 15, cg = lane >> 4, c0 = 16 * w + 4 * cg;

    // the item's conv outputs (after SiLU, before the norms)
    // (PATCH: the first chunks of a warm start, whose rows at positions -3..-1 are the
    // slot's conv rows: loaded into fresh registers and selected, since reloading the
    // prefetched ones under a branch makes the compiler wait for every load in flight;
    // the other chunks take a copy of this code without the selects)
    auto conv_items = [&](float (&yq)[4][4], float (&yk)[4][4], auto patch_c) {
      constexpr bool PATCH = decltype(patch_c)::value;
      u32x2 pq[7], pkk[7];
      if constexpr (PATCH) {
#pragma unroll
        for (int i = 0; i < 7; ++i) {  // rows 4tq - 3 + i
          const int pos = i < 3 ? p0 - 3 + i : p0 + 4 * tq + i - 3;
          pq[i] = pkk[i] = u32x2{0u, 0u};
          if (pos >= -3 && pos < 0) {
            pq[i] = *reinterpret_cast<const u32x2 *>(conv_live + (3 + pos) * C + h * D + c0);
            pkk[i] = *reinterpret_cast<const u32x2 *>(conv_live + (3 + pos) * C + H * D + h * D + c0);
          }
        }
        // (vmcnt 0 here, where only the first chunks pass: left pending, these loads
        // would make the compiler wait for every load in flight on the common path)
        __builtin_amdgcn_s_waitcnt(0x0f70);
      }
      auto use = [&](int i, int pos, const u32x2 &v, const u32x2 *pv) {
        return (PATCH && pos >= -3 && pos < 0) ? pv[i] : v;
      };
      // rows 4tq-3 .. 4tq+3: three from the lane one token group down (or loaded, in
      // the first group), then its own
      u32x2 rq[7], rk[7];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        rq[3 + i] = use(3 + i, p0 + 4 * tq + i, xq[i], pq);
        rk[3 + i] = use(3 + i, p0 + 4 * tq + i, xk[i], pkk);
      }
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const u32x2 fq = use(i, p0 - 3 + i, hq[i], pq), fk = use(i, p0 - 3 + i, hk[i], pkk);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const uint32_t nq = row_ror1(rq[4 + i][e]), nk = row_ror1(rk[4 + i][e]);
          rq[i][e] = tq == 0 ? fq[e] : nq;
          rk[i][e] = tq == 0 ? fk[e] : nk;
        }
      }
      u32x4 wq[2], wk[2];  // taps of the item's channels, two channels per vector
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        wq[i] = *reinterpret_cast<const u32x4 *>(lds + kAW + (c0 + 2 * i) * 8);
        wk[i] = *reinterpret_cast<const u32x4 *>(lds + kAW + (128 + c0 + 2 * i) * 8);
      }
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float accq = dot2_bf16(wq[e >> 1][2 * (e & 1)], halves(rq[rr][e >> 1], rq[rr + 1][e >> 1], e & 1), 0.f);
          accq = dot2_bf16(wq[e >> 1][2 * (e & 1) + 1], halves(rq[rr + 2][e >> 1], rq[rr + 3][e >> 1], e & 1), accq);
          float acck = dot2_bf16(wk[e >> 1][2 * (e & 1)], halves(rk[rr][e >> 1], rk[rr + 1][e >> 1], e & 1), 0.f);
          acck = dot2_bf16(wk[e >> 1][2 * (e & 1) + 1], halves(rk[rr + 2][e >> 1], rk[rr + 3][e >> 1], e & 1), acck);
          if (silu) {
            accq = accq / (1.f + __expf(-accq));
            acck = acck / (1.f + __expf(-acck));
          }
          yq[rr][e] = accq;
          yk[rr][e] = acck;
        }
      }
    };
    // fragment of token t for this item: rows = tokens, channel c0 + e in lane
    // (t & 15) + 16 cg, slot e + 4 (w & 1) of fragment (t >> 4, w >> 1)
    auto put_item = [&](int off, int rr, const float *v) {
      const int t = 4 * tq + rr, idx = (t >> 4) * 4 + (w >> 1);
      frag_put4(lds, off + ka_frag(idx), idx, ka_slot(idx, (t & 15) + 16 * cg), 4 * (w & 1), v);
    };

    // ================= P1: conv, planes, staged v rows, decays, norm sums =======
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int it = tid_c + u * kFThreads;
      if (it < 67 * 16) *reinterpret_cast<u32x4 *>(lds + xv_off_at(kAXV, it >> 4, 16 * (it & 15))) = sv[u];
    }
    // On a warm start, the staged pieces at positions -3..-1 are the slot's conv rows:
    // each thread overwrites the pieces it has just written (LDS writes of one thread
    // land in order).  Fresh registers, consumed here: reloading the prefetched ones
    // under a branch would make the compiler wait for every load in flight.
    if (p0 < 3 && warm) {
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        const int it = tid_c + u * kFThreads, pos = p0 - 3 + (it >> 4);
        if (it < 67 * 16 && pos >= -3 && pos < 0)
          *reinterpret_cast<u32x4 *>(lds + xv_off_at(kAXV, it >> 4, 16 * (it & 15))) =
              *reinterpret_cast<const u32x4 *>(conv_live + (3 + pos) * C + 2 * H * D + h * D + 8 * (it & 15));
      }
    }
    {
      float yq[4][4], yk[4][4];
      if (p0 < 3 && warm) conv_items(yq, yk, std::true_type());
        else conv_items(yq, yk, std::false_type());
      // squared norms over this wave's 16 channels, per token, to the partial sums
      {
        float s[8];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          float a2 = 0.f, b2 = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            a2 = fmaf(yq[rr][e], yq[rr][e], a2);
            b2 = fmaf(yk[rr][e], yk[rr][e], b2);
          }
          s[2 * rr] = cross_row_sum(a2);
          s[2 * rr + 1] = cross_row_sum(b2);
        }
        if (cg == 0) {
          float *pt = reinterpret_cast<float *>(lds + kALD) + (w * 64 + 4 * tq) * 2;
          *reinterpret_cast<f32x4 *>(pt) = f32x4{s[0], s[1], s[2], s[3]};
          *reinterpret_cast<f32x4 *>(pt + 4) = f32x4{s[4], s[5], s[6], s[7]};
        }
      }
      // decays: g_t per channel as a product (a token outside the request has a = 1)
      f32x4 gf[4];
      {
        f32x4 run = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int pos = p0 + 4 * tq + rr;
          const bool valid = pos >= 0 && pos < rg.len;
#pragma unroll
          for (int e = 0; e < 4; ++e) run[e] *= valid ? al[rr][e] : 1.f;
          gf[rr] = run;
        }
        f32x4 ex;
#pragma unroll
        for (int e = 0; e < 4; ++e) ex[e] = row_shr_or_one<1>(row_prefix_prod(run[e]));  // tokens < 4tq
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) gf[rr] *= ex;
        bool bad = false;
        if (tq == 15) {  // g_63 of the item's channels
          *reinterpret_cast<f32x4 *>(LB + kLbG + c0) = gf[3];
#pragma unroll
          for (int e = 0; e < 4; ++e) bad |= !(gf[3][e] >= kPlaneFloor);
        }
        const bool any_bad = __builtin_amdgcn_ballot_w64(bad) != 0;
        if (lane == 0) LF[w] = any_bad ? 1 : 0;
      }
      // the planes P = k g, R = k / g, Q' = q g
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        float pv[4], rv[4], qv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pv[e] = yk[rr][e] * gf[rr][e];
          rv[e] = yk[rr][e] * __builtin_amdgcn_rcpf(gf[rr][e]);
          qv[e] = yq[rr][e] * gf[rr][e];
        }
        put_item(kAP, rr, pv);
        put_item(kAR, rr, rv);
        put_item(kAQ, rr, qv);
      }
    }
    if (w == 0) {  // b, the last load of the chunk
      const int dpos = p0 + lane;
      LB[lane] = (dpos >= 0 && dpos < rg.len) ? bv : 0.f;
    }
    lds_barrier();
    // the norms (wave 0, one token per lane) and the chunk's path
    if (w == 0) {
      const float *pt = reinterpret_cast<const float *>(lds + kALD) + lane * 2;
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int ww = 0; ww < 8; ++ww) {
        sq += pt[ww * 128];
        sk += pt[ww * 128 + 1];
      }
      LB[kLbIq + lane] = nq ? __builtin_amdgcn_rsqf(sq + 1e-6f) : 1.f;
      LB[kLbIk + lane] = nk ? __builtin_amdgcn_rsqf(sk + 1e-6f) : 1.f;
      if (lane == 0) {
        int f = 0;
#pragma unroll
        for (int ww = 0; ww < 8; ++ww) f |= LF[ww];
        LF[8] = f;
      }
    }
    lds_barrier();
    const int by_token = __builtin_amdgcn_readfirstlane(LF[8]);
    if (by_token) {
      // A chunk run token by token: the planes again without the decay factors (k
      // into P, q into Q'), and the decays themselves, fp32 [t][c], in R's place.
      {
        float yq[4][4], yk[4][4];
        if (p0 < 3 && warm) conv_items(yq, yk, std::true_type());
        else conv_items(yq, yk, std::false_type());
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          put_item(kAP, rr, yk[rr]);
          put_item(kAQ, rr, yq[rr]);
          const int pos = p0 + 4 * tq + rr;
          const bool valid = pos >= 0 && pos < rg.len;
          f32x4 av = al[rr];
#pragma unroll
          for (int e = 0; e < 4; ++e) av[e] = valid ? av[e] : 1.f;
          *reinterpret_cast<f32x4 *>(lds + kAR + ((4 * tq + rr) * D + c0) * 4) = av;
        }
      }
    }

    // ================= P2 =======================================================
    // The next chunk's inputs are issued in two halves (waves 0-3 here, 4-7 at the
    // start of P3), at the same two points on both paths: a third call site would
    // keep the loop's registers from coalescing and cost a wait for every load in
    // flight at the end of each chunk.
    if (w < 4) load_chunk(tid_c, p0 + 64);
    if (!by_token) {
      // a transposed M tile (lane holds M[16m+r][16k+4g+j]): causal mask and norms
      auto put_m = [&](int m, int k, const f32x4 &cc) {
        const int t = 16 * m + r;
        const float qt = LB[kLbIq + t];
        float mv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 16 * k + 4 * g + j;
          mv[j] = i <= t ? qt * LB[kLbIk + i] * cc[j] : 0.f;
        }
        frag_put4(lds, kAM, pair_idx(m, k >> 1), lane, 4 * (k & 1), mv);
        if (m == k && !(m & 1)) {
          const float z[4] = {0.f, 0.f, 0.f, 0.f};
          frag_put4(lds, kAM, pair_idx(m, m >> 1), lane, 4, z);
        }
      };
      if (w < 4) {
        // diagonal block m of N = Diag(b) A: lane holds P_{16m+4g+j} . R_{16m+r}
        const int m = w;
        f32x4 c2[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int idx = m * 4 + ks;
          c2[ks & 1] = mfma3(ka_frag_lds(lds, kAP, idx, lane), ka_frag_lds(lds, kAR, idx, lane),
                             c2[ks & 1]);
        }
        const f32x4 cc = c2[0] + c2[1];
        float *blk = reinterpret_cast<float *>(lds + kALD) + m * 16 * kBP;
        const float ki = LB[kLbIk + 16 * m + r];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = 4 * g + j;
          blk[t * kBP + r] = t > r ? LB[16 * m + t] * LB[kLbIk + 16 * m + t] * ki * cc[j] : 0.f;
        }
        wave_lds_sync();
        float x[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          float v = (t == r) ? 1.f : 0.f;
#pragma unroll
          for (int i = 0; i < t; ++i) v = fmaf(-blk[t * kBP + i], x[i], v);
          x[t] = v;
        }
        wave_lds_sync();
        if (g == 0) {
#pragma unroll
          for (int t = 0; t < 16; ++t) blk[t * kBP + r] = x[t];
        }
        wave_lds_sync();
        split4_put(lds, kADF + m * 1024, lane, ld4(blk + r * kBP + 4 * g));
        // the diagonal M tile (m, m): lane holds R_{16m+4g+j} . Q'_{16m+r}
        f32x4 cm[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int idx = m * 4 + ks;
          cm[ks & 1] = mfma3(ka_frag_lds(lds, kAR, idx, lane), ka_frag_lds(lds, kAQ, idx, lane),
                             cm[ks & 1]);
        }
        put_m(m, m, cm[0] + cm[1]);
      } else {
        // the M blocks below the diagonal and the N blocks, three tiles per wave,
        // in the order of the kernel above; lane holds R_{16k+4g+j} . (Q' or P)_{16m+r}
        constexpr uint64_t kTilesLo = 0x190d180c09140804ull, kTilesHi = 0x1e1d0e1cull;
        auto tile_entry = [&](int q) {
          const int i = (w - 4) * 3 + q;
          return int(((i < 8 ? kTilesLo >> (8 * i) : kTilesHi >> (8 * (i - 8)))) & 0xff);
        };
#pragma unroll
        for (int q0 = 0; q0 < 3; q0 += 2) {
          f32x4 cc[3];
#pragma unroll
          for (int q = q0; q < min(q0 + 2, 3); ++q) cc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int q = q0; q < min(q0 + 2, 3); ++q) {
              const int e = tile_entry(q);
              const int m = (e >> 2) & 3, k = e & 3;
              const int ia = k * 4 + ks, ib = m * 4 + ks;
              cc[q] = mfma3(ka_frag_lds(lds, kAR, ia, lane),
                            ka_frag_lds(lds, (e >> 4) ? kAP : kAQ, ib, lane), cc[q]);
            }
          }
#pragma unroll
          for (int q = q0; q < min(q0 + 2, 3); ++q) {
            const int e = tile_entry(q);
            const int m = (e >> 2) & 3, k = e & 3;
            if ((e >> 4) == 0) {
              put_m(m, k, cc[q]);
            } else {  // -N_mk = -b_t A[t][i] / (|k_t| |k_i|)
              const int t = 16 * m + r;
              const float f = -LB[t] * LB[kLbIk + t];
              f32x4 nv;
#pragma unroll
              for (int j = 0; j < 4; ++j) nv[j] = f * LB[kLbIk + 16 * k + 4 * g + j] * cc[q][j];
              split4_put(lds, kANF + nf_idx(m, k) * 1024, lane, nv);
            }
          }
        }
      }
      if (c > 0) flush_out(tid_c, p0 - 64);
      // Y = Diag(b) (V - P S0^T / |k|) and Q' S0^T / |q| for this wave's rows
      {
        f32x4 X1[4], XQ[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          X1[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
          XQ[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        Split kf[2], qf[2], sop;
        kf[0] = ka_frag_lds(lds, kAP, 0, lane);
        qf[0] = ka_frag_lds(lds, kAQ, 0, lane);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int ks = i >> 2, tb = i & 3;
          if (i + 1 < 16) {
            const int n = ((i + 1) & 3) * 4 + ((i + 1) >> 2);
            kf[(i + 1) & 1] = ka_frag_lds(lds, kAP, n, lane);
            qf[(i + 1) & 1] = ka_frag_lds(lds, kAQ, n, lane);
          }
          if (tb == 0) sop = split44(S[2 * ks], S[2 * ks + 1]);
          X1[tb] = mfma3(kf[i & 1], sop, X1[tb]);
          XQ[tb] = mfma3(qf[i & 1], sop, XQ[tb]);
        }
        const int xb0 = kAXV + 4 * g * 256 + (((vcol >> 3) ^ (2 * (g & 3))) << 4) + 2 * (vcol & 7);
        const int xb1 = kAXV + 4 * g * 256 + (((vcol >> 3) ^ (2 * ((g + 1) & 3))) << 4) + 2 * (vcol & 7);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          const int t0 = 16 * tb + 4 * g;
          uint32_t xc[7], xp[6];
#pragma unroll
          for (int q = 0; q < 7; ++q)
            xc[q] = *reinterpret_cast<const uint16_t *>(lds + (q < 4 ? xb0 : xb1) + tb * 4096 + q * 256);
#pragma unroll
          for (int q = 0; q < 6; ++q) xp[q] = halves(xc[q], xc[q + 1], 0);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int t = t0 + j;
            float acc = dot2_bf16(vw[0], xp[j], 0.f);
            acc = dot2_bf16(vw[1], xp[j + 2], acc);
            if (silu) acc = acc / (1.f + __expf(-acc));
            Y[tb][j] = LB[t] * (acc - LB[kLbIk + t] * X1[tb][j]);
            OQ[tb][j] = LB[kLbIq + t] * XQ[tb][j];
          }
        }
      }
      lds_barrier();

    } else {
      if (c > 0) flush_out(tid_c, p0 - 64);
      lds_barrier();
      const int xv0 = 2 * vcol;
#pragma unroll 1
      for (int t = 0; t < 64; ++t) {
        const float bt = LB[t], qi = LB[kLbIq + t], ki = LB[kLbIk + t];
        const float *arow = reinterpret_cast<const float *>(lds + kAR) + t * D + 4 * g;
        // this lane's 32 channels of k and q: slots 0-3 are channels 32ks + 4g + j,
        // slots 4-7 channels 32ks + 16 + 4g + j, of fragment (t >> 4, ks)
        const int fl = (t & 15) + 16 * g;  // this lane's fragment lane
        float u = 0.f, sq = 0.f, kq = 0.f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int fi = (t >> 4) * 4 + ks, fo = 2 * fi * 1024 + ka_frag(fi) + ka_slot(fi, fl) * 16;
          const u32x4 kh = *reinterpret_cast<const u32x4 *>(lds + kAP + fo);
          const u32x4 kl = *reinterpret_cast<const u32x4 *>(lds + kAP + fo + 1024);
          const u32x4 qh = *reinterpret_cast<const u32x4 *>(lds + kAQ + fo);
          const u32x4 ql = *reinterpret_cast<const u32x4 *>(lds + kAQ + fo + 1024);
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const int kb = 2 * ks + hf;
            const f32x4 a4 = *reinterpret_cast<const f32x4 *>(arow + 16 * kb);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float kv = bf16_elem(kh, 4 * hf + j) + bf16_elem(kl, 4 * hf + j);
              const float qv = bf16_elem(qh, 4 * hf + j) + bf16_elem(ql, 4 * hf + j);
              S[kb][j] *= a4[j];
              u = fmaf(S[kb][j], kv, u);
              sq = fmaf(S[kb][j], qv, sq);
              kq = fmaf(kv, qv, kq);
            }
          }
        }
        u = cross_row_sum(u);
        sq = cross_row_sum(sq);
        kq = cross_row_sum(kq);
        // v of row vcol at token t: conv of staged rows t..t+3
        uint32_t xc[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) xc[q] = *reinterpret_cast<const uint16_t *>(lds + xv_off_at(kAXV, t + q, xv0));
        float vt = dot2_bf16(vw[0], halves(xc[0], xc[1], 0), 0.f);
        vt = dot2_bf16(vw[1], halves(xc[2], xc[3], 0), vt);
        if (silu) vt = vt / (1.f + __expf(-vt));
        const float dk = bt * (vt - ki * u) * ki;  // d_t / |k_t|
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int fi = (t >> 4) * 4 + ks, fo = 2 * fi * 1024 + ka_frag(fi) + ka_slot(fi, fl) * 16;
          const u32x4 kh = *reinterpret_cast<const u32x4 *>(lds + kAP + fo);
          const u32x4 kl = *reinterpret_cast<const u32x4 *>(lds + kAP + fo + 1024);
#pragma unroll
          for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              S[2 * ks + hf][j] = fmaf(dk, bf16_elem(kh, 4 * hf + j) + bf16_elem(kl, 4 * hf + j), S[2 * ks + hf][j]);
        }
        // o_t = scale S_t q_t = scale (S' q + d (k . q))
        if (g == 0)
          *reinterpret_cast<uint16_t *>(lds + kAOS + t * kOP + 2 * vcol) =
              f32_to_bf16(a.scale * qi * (sq + dk * kq));
      }
    }

    // ================= P3: Dl, O, state update ==================================
    if (w >= 4) load_chunk(tid_c, p0 + 64);
    if (!by_token) {
      f32x4 Dl[4];
      {
        Split4 db[3];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          f32x4 acc = Y[m];
#pragma unroll
          for (int k = 0; k < m; ++k) acc = mfma3k16(split4_get(lds, kANF + nf_idx(m, k) * 1024, lane), db[k], acc);
          Dl[m] = mfma3k16(split4_get(lds, kADF + m * 1024, lane), split4s(acc), f32x4{0.f, 0.f, 0.f, 0.f});
          if (m < 3) db[m] = split4s(Dl[m]);
        }
      }
      Split dop[2], dgop[2];
      dop[0] = split44(Dl[0], Dl[1]);
      dop[1] = split44(Dl[2], Dl[3]);
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int j = 0; j < 4; ++j) Dl[tb][j] *= LB[kLbIk + 16 * tb + 4 * g + j];  // Dl / |k|
      dgop[0] = split44(Dl[0], Dl[1]);
      dgop[1] = split44(Dl[2], Dl[3]);
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        f32x4 o = OQ[tb];
#pragma unroll
        for (int ks = 0; ks <= (tb >> 1); ++ks) o = mfma3(frag_lds(lds, kAM, pair_idx(tb, ks), lane), dop[ks], o);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<uint16_t *>(lds + kAOS + (16 * tb + 4 * g + j) * kOP + 2 * vcol) = f32_to_bf16(a.scale * o[j]);
      }
      // S^T = Diag(g_63) (S0^T + R^T Diag(1/|k|) Dl)
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) S[kb] = mfma3(kt_frag_at(lds, kAR, slot_fn, kb, ks, lane, kTbPad), dgop[ks], S[kb]);
        S[kb] *= *reinterpret_cast<const f32x4 *>(LB + kLbG + 16 * kb + 4 * g);
      }
    }

    // snapshot at a boundary that ends this chunk
    if (a.snap_interval > 0) {
      const int done = min(64 * (c + 1) - rg.off, rg.len);
      const int n_end = sl + done;
      const int j = n_end / a.snap_interval - sl / a.snap_interval - 1;
      if (n_end % a.snap_interval == 0 && j >= snap_lo) {
        const int dst = ((nxt + j) & 1) ? trk1 : trk0;
        if (dst >= fa.slots) {
          if (fa.err && tid == 0) atomicOr(fa.err, GDN_ERRW_BAD_TRACK_SLOT);
        } else if (dst > 0) {
          TS *Sd = ssm + ((int64_t(a.layer) * fa.slots + dst) * H + h) * int64_t(D) * D;
#pragma unroll
          for (int kb = 0; kb < 8; ++kb) store_s4(Sd + int64_t(vcol) * D + 16 * kb + 4 * g, S[kb]);
          uint16_t *cd = fa.conv + (int64_t(a.layer) * fa.slots + dst) * kConvRows * C;
          if (tid < 144) {
            int ch, row;
            const u32x4 v = conv_item(tid, done, ch, row);
            *reinterpret_cast<u32x4 *>(cd + row * C + ch) = v;
          }
        }
      }
    }
    lds_barrier();
  }

  // ---- end of the request: live slot -------------------------------------------
  flush_out(tid, 64 * (rg.nch - 1) - rg.off);
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) store_s4(Slive + int64_t(vcol) * D + 16 * kb + 4 * g, S[kb]);
  int ch = 0, row = 0;
  u32x4 nv = {0u, 0u, 0u, 0u};
  if (tid < 144) nv = conv_item(tid, rg.len, ch, row);
  __syncthreads();
  if (tid < 144) *reinterpret_cast<u32x4 *>(conv_live + row * C + ch) = nv;
}

}  // namespace

hipError_t launch_prefill_fused(const gdn_pool *p, const PrefillArgs &a, hipStream_t s) {
  if (p->d.head_k != kFD || p->d.head_v != kFD) return hipErrorInvalidValue;
  FArgs fa{a, p->d.ssm_base, static_cast<uint16_t *>(p->d.conv_base), p->d.err_word, p->d.slots, p->d.heads};
  const dim3 grid(unsigned(a.batch) * p->d.heads), block(kFThreads);
  const bool bf16 = p->d.ssm_dtype == GDN_BF16, silu = (a.flags & GDN_F_CONV_SILU) != 0;
  if (a.alpha_mode == GDN_ALPHA_PER_CHANNEL) {
    if (bf16 && silu) hipLaunchKernelGGL((prefill_fused_kda_kernel<uint16_t, true>), grid, block, 0, s, fa);
    else if (bf16) hipLaunchKernelGGL((prefill_fused_kda_kernel<uint16_t, false>), grid, block, 0, s, fa);
    else if (silu) hipLaunchKernelGGL((prefill_fused_kda_kernel<float, true>), grid, block, 0, s, fa);
    else hipLaunchKernelGGL((prefill_fused_kda_kernel<float, false>), grid, block, 0, s, fa);
  } else {
    if (bf16 && silu) hipLaunchKernelGGL((prefill_fused_kernel<uint16_t, true>), grid, block, 0, s, fa);
    else if (bf16) hipLaunchKernelGGL((prefill_fused_kernel<uint16_t, false>), grid, block, 0, s, fa);
    else if (silu) hipLaunchKernelGGL((prefill_fused_kernel<float, true>), grid, block, 0, s, fa);
    else hipLaunchKernelGGL((prefill_fused_kernel<float, false>), grid, block, 0, s, fa);
  }
  return hipGetLastError();
}

}  // namespace gdn
