// common.hpp -- internal declarations shared by the library's translation units.
// Not installed; the public interface is include/gdn_slot.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gdn_slot.h"

struct gdn_pool {
  gdn_pool_desc d;
  int64_t C;                 // conv channels = heads * (2*head_k + head_v)
  int64_t ssm_block_bytes;   // one (layer, slot) ssm block
  int64_t conv_block_bytes;  // one (layer, slot) conv block (3 rows)
};

namespace gdn {

constexpr int kConvRows = 3;
constexpr int kChunk = 64;

// ------------------------------------------------------------ bf16 helpers --
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
// Round to nearest even with gfx950's conversion instruction (v_cvt_pk_bf16_f32;
// NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
// Two values packed low | high, one instruction.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// ------------------------------------------------------------- launchers --
// Copy layers [layer_begin, layer_end) for n (src, dst) pairs read from device
// arrays (dst <= 0 skipped).
hipError_t launch_copy_device_pairs(const gdn_pool *p, int layer_begin, int layer_end, int n,
                                    const int32_t *src, const int32_t *dst, hipStream_t s);
// Copy all layers for n host-validated pairs (both in [1, slots), src != dst).
hipError_t launch_copy_host_pairs(const gdn_pool *p, int n, const int32_t *src,
                                  const int32_t *dst, hipStream_t s);

struct DecodeArgs {
  int layer, batch;
  const int32_t *slot_table;
  const uint16_t *x;
  const uint16_t *conv_w;
  const float *alpha;
  int alpha_mode;
  const float *beta;
  float scale;
  uint32_t flags;
  uint16_t *out;
  const int32_t *seq_len_after;
  int track_interval;
  const int32_t *track_slots;
  const int32_t *next_track_idx;
};
hipError_t launch_decode(const gdn_pool *p, const DecodeArgs &a, hipStream_t s);

struct PrefillArgs {
  int layer, batch, total_tokens, max_seqlen;
  const int32_t *cu_seqlens;
  const int32_t *slot_table;
  const int32_t *has_initial_state;
  const int32_t *start_len;
  const uint16_t *x;
  const uint16_t *conv_w;
  const float *alpha;
  int alpha_mode;
  const float *beta;
  float scale;
  uint32_t flags;
  uint16_t *out;
  int snap_interval;
  const int32_t *track_slots;
  const int32_t *next_track_idx;
  void *workspace;
  size_t workspace_bytes;
};
hipError_t launch_prefill(const gdn_pool *p, const PrefillArgs &a, hipStream_t s);
hipError_t launch_prefill_fused(const gdn_pool *p, const PrefillArgs &a, hipStream_t s);

// Extent of request b in a prefill call: first token, length, front padding of
// its first 64-token chunk (chunks are aligned to absolute positions) and chunk
// count.  ok is false when cu_seqlens or start_len is inconsistent.
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

// Draft trees: nodes per request are limited so that a workgroup can hold the
// parent list in shared memory.
constexpr int kMaxTreeNodes = GDN_MAX_TREE_NODES;

struct VerifyArgs {
  int layer, batch, nodes;
  const int32_t *slot_table;
  const int32_t *parent;
  const uint16_t *x;
  const uint16_t *conv_w;
  const float *alpha;
  int alpha_mode;
  const float *beta;
  float scale;
  uint32_t flags;
  uint16_t *out;
  void *node_ssm;
  uint16_t *node_conv;
};
hipError_t launch_verify(const gdn_pool *p, const VerifyArgs &a, hipStream_t s);

struct ScatterArgs {
  int layer, batch, nodes;
  const int32_t *slot_table;
  const int32_t *parent;
  const int32_t *accepted;
  const int32_t *seq_len_before;
  int track_interval;
  const int32_t *track_slots;
  const int32_t *next_track_idx;
  const void *node_ssm;
  const uint16_t *node_conv;
};
hipError_t launch_accept_scatter(const gdn_pool *p, const ScatterArgs &a, hipStream_t s);

struct ReplayArgs {
  gdn_replay_ring ring;
  int layer, batch, draft;
  const int32_t *slot_table;
  // verify
  const uint16_t *x;
  const uint16_t *conv_w;
  const float *alpha;
  const float *beta;
  float scale;
  uint32_t flags;
  uint16_t *out;
  // commit
  const int32_t *accepted;
  const int32_t *seq_len_before;
  int track_interval;
  const int32_t *track_slots;
  const int32_t *next_track_idx;
};
hipError_t launch_replay_verify(const gdn_pool *p, const ReplayArgs &a, hipStream_t s);
hipError_t launch_replay_commit(const gdn_pool *p, const ReplayArgs &a, hipStream_t s);
// Workspace of the two-phase prefill: one record per (request, chunk, head) of
// the chunks processed in one window, plus an fp32 state carry per (request, head).
size_t prefill_record_bytes(const gdn_pool *p);
size_t prefill_carry_bytes(const gdn_pool *p, int batch);

}  // namespace gdn
