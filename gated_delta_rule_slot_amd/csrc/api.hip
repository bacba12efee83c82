// api.hip -- the C ABI declared in include/gdn_slot.h: host-side validation,
// error strings, and dispatch to the kernels.  No device memory is allocated
// here; every buffer belongs to the caller.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <new>

#include "common.hpp"
#include "errors.hpp"

#define GDN_API extern "C" __attribute__((visibility("default")))

namespace {
thread_local char g_err[512] = "";
}  // namespace

namespace gdn {
gdn_status set_error(gdn_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}
gdn_status clear_error() {
  g_err[0] = '\0';
  return GDN_OK;
}
}  // namespace gdn

namespace {

#define fail(...) gdn::set_error(__VA_ARGS__)

gdn_status ok() { return gdn::clear_error(); }

// (request, head) units from which the prefill runs in one kernel by default: a
// workgroup per unit then keeps most compute units busy, while fewer units run
// faster on the two-kernel path, which spreads each request over its chunks.
constexpr int64_t kOneKernelMinUnits = 128;

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

gdn_status check_shape(const gdn_pool_desc *d) {
  if (!d) return fail(GDN_ERR_ARG, "descriptor is NULL");
  if (d->layers <= 0 || d->slots < 2 || d->heads <= 0)
    return fail(GDN_ERR_ARG, "need layers >= 1, slots >= 2 (slot 0 is reserved), heads >= 1");
  if (d->conv_kernel != 4) return fail(GDN_ERR_UNSUPPORTED, "conv_kernel must be 4");
  if (d->ssm_dtype != GDN_F32 && d->ssm_dtype != GDN_BF16)
    return fail(GDN_ERR_ARG, "ssm_dtype must be GDN_F32 or GDN_BF16");
  if (d->conv_dtype != GDN_BF16) return fail(GDN_ERR_UNSUPPORTED, "conv_dtype must be GDN_BF16");
  if (d->head_k != d->head_v)
    return fail(GDN_ERR_UNSUPPORTED, "head_k must equal head_v (got %d, %d)", d->head_k, d->head_v);
  if (d->head_k != 16 && d->head_k != 32 && d->head_k != 64 && d->head_k != 128)
    return fail(GDN_ERR_UNSUPPORTED, "head dim %d not in {16, 32, 64, 128}", d->head_k);
  if (d->heads > 65535) return fail(GDN_ERR_UNSUPPORTED, "heads > 65535");
  return GDN_OK;
}

void sizes(const gdn_pool_desc *d, int64_t *C, int64_t *ssm_block, int64_t *conv_block) {
  *C = int64_t(d->heads) * (2 * d->head_k + d->head_v);
  *ssm_block = int64_t(d->heads) * d->head_v * d->head_k * (d->ssm_dtype == GDN_F32 ? 4 : 2);
  *conv_block = int64_t(gdn::kConvRows) * (*C) * 2;
}

gdn_status check_pool(gdn_pool_t p, int layer) {
  if (!p) return fail(GDN_ERR_ARG, "pool handle is NULL");
  if (layer < 0 || layer >= p->d.layers)
    return fail(GDN_ERR_RANGE, "layer %d outside [0, %d)", layer, p->d.layers);
  return GDN_OK;
}

gdn_status launched(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(GDN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

// ---- fixed scratch of the allocation-free prefill entry point ----------------
// The two-kernel prefill's records and state carry, for callers that cannot
// allocate.  Each GPU the library runs on holds one copy of this array until the
// process ends.  Its host-side name is only a stand-in for the symbol: host code
// uses the device address that hipGetSymbolAddress returns for the current
// device, kept per device after the first call on it.  Every call on one GPU
// shares that GPU's copy: calls that overlap on one GPU race.  Nothing needs
// clearing between calls, since every byte the kernels read is written earlier
// in the same call.
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices];  // device address of `scratch`, per device

gdn_status scratch_for_current_device(void **addr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GDN_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(GDN_ERR_UNSUPPORTED, "device %d is beyond the %d the scratch table holds", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(GDN_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return GDN_OK;
}
}  // namespace

GDN_API gdn_status state_pool_bytes(const gdn_pool_desc *desc, size_t *ssm_bytes,
                                    size_t *conv_bytes) {
  gdn_status s = check_shape(desc);
  if (s != GDN_OK) return s;
  int64_t C, sb, cb;
  sizes(desc, &C, &sb, &cb);
  if (ssm_bytes) *ssm_bytes = size_t(sb) * desc->layers * desc->slots;
  if (conv_bytes) *conv_bytes = size_t(cb) * desc->layers * desc->slots;
  return ok();
}

GDN_API gdn_status state_pool_create(const gdn_pool_desc *desc, gdn_pool_t *out) {
  if (!out) return fail(GDN_ERR_ARG, "out is NULL");
  *out = nullptr;
  gdn_status s = check_shape(desc);
  if (s != GDN_OK) return s;
  if (!desc->ssm_base || !desc->conv_base) return fail(GDN_ERR_ARG, "pool base pointer is NULL");
  if (!aligned(desc->ssm_base, 16) || !aligned(desc->conv_base, 16))
    return fail(GDN_ERR_UNSUPPORTED, "pool base pointers must be 16-byte aligned");
  if (desc->err_word && !aligned(desc->err_word, 4))
    return fail(GDN_ERR_ARG, "err_word must be 4-byte aligned");
  gdn_pool *p = new (std::nothrow) gdn_pool;
  if (!p) return fail(GDN_ERR_ARG, "out of host memory");
  p->d = *desc;
  sizes(desc, &p->C, &p->ssm_block_bytes, &p->conv_block_bytes);
  if ((p->ssm_block_bytes % 16) || (p->conv_block_bytes % 16)) {
    delete p;
    return fail(GDN_ERR_UNSUPPORTED, "state blocks must be multiples of 16 bytes");
  }
  *out = p;
  return ok();
}

GDN_API void state_pool_destroy(gdn_pool_t pool) { delete pool; }

GDN_API const char *gdn_last_error(void) { return g_err; }

GDN_API gdn_status gdn_prefill_workspace_bytes(gdn_pool_t pool, int32_t batch,
                                               int32_t max_seqlen, size_t *bytes) {
  if (!pool || !bytes) return fail(GDN_ERR_ARG, "pool or bytes is NULL");
  if (batch < 0 || max_seqlen < 0) return fail(GDN_ERR_RANGE, "batch or max_seqlen < 0");
  // chunks are aligned to absolute positions, so a request may touch one more
  // chunk than ceil(len / 64) when its start is not a multiple of 64
  const size_t chunks = (size_t(max_seqlen) + 2 * gdn::kChunk - 2) / gdn::kChunk;
  *bytes = (chunks ? chunks : 1) * size_t(batch) * pool->d.heads * gdn::prefill_record_bytes(pool) +
           gdn::prefill_carry_bytes(pool, batch);
  return ok();
}

namespace {
// The prefill entry points share this body.  With use_scratch the two-kernel
// path takes the fixed per-device scratch instead of a caller workspace.
gdn_status prefill_entry(
    gdn_pool_t pool, int32_t layer, int32_t batch, int32_t total_tokens, int32_t max_seqlen,
    const int32_t *cu_seqlens, const int32_t *slot_table, const int32_t *has_initial_state,
    const int32_t *start_len, const uint16_t *x, const uint16_t *conv_w, const float *alpha,
    int32_t alpha_mode, const float *beta, float scale, uint32_t flags, uint16_t *out,
    int32_t snap_interval, const int32_t *track_slots, const int32_t *next_track_idx,
    void *workspace, size_t workspace_bytes, bool use_scratch, void *stream) {
  gdn_status s = check_pool(pool, layer);
  if (s != GDN_OK) return s;
  if (batch < 0 || batch > 65535) return fail(GDN_ERR_RANGE, "batch %d outside [0, 65535]", batch);
  if (total_tokens < 0 || max_seqlen < 0) return fail(GDN_ERR_RANGE, "negative token count");
  if (batch == 0) return ok();
  if (!cu_seqlens || !slot_table || !has_initial_state || !conv_w || !alpha || !beta)
    return fail(GDN_ERR_ARG, "a required pointer is NULL");
  if (total_tokens > 0 && (!x || !out)) return fail(GDN_ERR_ARG, "x or out is NULL");
  if (alpha_mode != GDN_ALPHA_PER_HEAD && alpha_mode != GDN_ALPHA_PER_CHANNEL)
    return fail(GDN_ERR_ARG, "alpha_mode %d unknown", alpha_mode);
  if (flags & ~uint32_t(GDN_F_L2NORM_K | GDN_F_L2NORM_Q | GDN_F_CONV_SILU | GDN_F_PREFILL_ONE_KERNEL |
                        GDN_F_PREFILL_TWO_KERNEL | GDN_F_SNAP_LAST_ONLY))
    return fail(GDN_ERR_ARG, "unknown flag bits 0x%x", flags);
  if ((flags & GDN_F_PREFILL_ONE_KERNEL) && (flags & GDN_F_PREFILL_TWO_KERNEL))
    return fail(GDN_ERR_ARG, "GDN_F_PREFILL_ONE_KERNEL and GDN_F_PREFILL_TWO_KERNEL both set");
  // (the one-kernel path addresses a request's rows with 32-bit byte offsets)
  const bool one_ok = pool->d.head_k == 128 && int64_t(max_seqlen) * pool->C * 2 < (int64_t(1) << 31);
  if ((flags & GDN_F_PREFILL_ONE_KERNEL) && !one_ok)
    return fail(GDN_ERR_UNSUPPORTED, "the one-kernel prefill serves head dim 128 (and max_seqlen * channels * 2 < 2^31)");
  const bool one_kernel = (flags & GDN_F_PREFILL_ONE_KERNEL) ||
                          (one_ok && !(flags & GDN_F_PREFILL_TWO_KERNEL) &&
                           int64_t(batch) * pool->d.heads >= kOneKernelMinUnits);
  if (snap_interval < 0 || (snap_interval % gdn::kChunk) != 0)
    return fail(GDN_ERR_ARG, "snap_interval %d must be 0 or a positive multiple of 64",
                snap_interval);
  if (snap_interval > 0 && (!track_slots || !next_track_idx || !start_len))
    return fail(GDN_ERR_ARG, "snapshots need track_slots, next_track_idx and start_len");
  if (!aligned(conv_w, 16)) return fail(GDN_ERR_UNSUPPORTED, "conv_w must be 16-byte aligned");
  if (x && !aligned(x, 16)) return fail(GDN_ERR_UNSUPPORTED, "x must be 16-byte aligned");
  if (out && !aligned(out, 16)) return fail(GDN_ERR_UNSUPPORTED, "out must be 16-byte aligned");
  if (!aligned(alpha, 16)) return fail(GDN_ERR_UNSUPPORTED, "alpha must be 16-byte aligned");
  // the one-kernel path keeps every intermediate on chip and takes no workspace
  if (!one_kernel) {
    const size_t need_min = size_t(batch) * pool->d.heads * gdn::prefill_record_bytes(pool) +
                            gdn::prefill_carry_bytes(pool, batch);
    if (use_scratch) {
      if (need_min > size_t(GDN_NOALLOC_SCRATCH_BYTES))
        return fail(GDN_ERR_RANGE,
                    "the two-kernel prefill of %d requests x %d heads needs %zu bytes of scratch "
                    "at least; the fixed scratch holds %zu (split the batch)",
                    batch, pool->d.heads, need_min, size_t(GDN_NOALLOC_SCRATCH_BYTES));
      gdn_status ss = scratch_for_current_device(&workspace);
      if (ss != GDN_OK) return ss;
      workspace_bytes = size_t(GDN_NOALLOC_SCRATCH_BYTES);
    }
    if (!workspace || workspace_bytes < need_min)
      return fail(GDN_ERR_ARG, "workspace of %zu bytes is below the minimum %zu", workspace_bytes,
                  need_min);
    if (!aligned(workspace, 256))
      return fail(GDN_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  }
  gdn::PrefillArgs a{layer,       batch,          total_tokens,  max_seqlen, cu_seqlens,
                     slot_table,  has_initial_state, start_len, x,          conv_w,
                     alpha,       alpha_mode,     beta,          scale,      flags,
                     out,         snap_interval,  track_slots,   next_track_idx,
                     workspace,   workspace_bytes};
  if (one_kernel)
    return launched(gdn::launch_prefill_fused(pool, a, static_cast<hipStream_t>(stream)),
                    "conv_gdn_prefill_chunked launch (one kernel)");
  return launched(gdn::launch_prefill(pool, a, static_cast<hipStream_t>(stream)),
                  "conv_gdn_prefill_chunked launch");
}
}  // namespace

GDN_API gdn_status conv_gdn_prefill_chunked(
    gdn_pool_t pool, int32_t layer, int32_t batch, int32_t total_tokens, int32_t max_seqlen,
    const int32_t *cu_seqlens, const int32_t *slot_table, const int32_t *has_initial_state,
    const int32_t *start_len, const uint16_t *x, const uint16_t *conv_w, const float *alpha,
    int32_t alpha_mode, const float *beta, float scale, uint32_t flags, uint16_t *out,
    int32_t snap_interval, const int32_t *track_slots, const int32_t *next_track_idx,
    void *workspace, size_t workspace_bytes, void *stream) {
  return prefill_entry(pool, layer, batch, total_tokens, max_seqlen, cu_seqlens, slot_table,
                       has_initial_state, start_len, x, conv_w, alpha, alpha_mode, beta, scale,
                       flags, out, snap_interval, track_slots, next_track_idx, workspace,
                       workspace_bytes, false, stream);
}

GDN_API gdn_status conv_gdn_prefill_chunked_noalloc(
    gdn_pool_t pool, int32_t layer, int32_t batch, int32_t total_tokens, int32_t max_seqlen,
    const int32_t *cu_seqlens, const int32_t *slot_table, const int32_t *has_initial_state,
    const int32_t *start_len, const uint16_t *x, const uint16_t *conv_w, const float *alpha,
    int32_t alpha_mode, const float *beta, float scale, uint32_t flags, uint16_t *out,
    int32_t snap_interval, const int32_t *track_slots, const int32_t *next_track_idx,
    void *stream) {
  return prefill_entry(pool, layer, batch, total_tokens, max_seqlen, cu_seqlens, slot_table,
                       has_initial_state, start_len, x, conv_w, alpha, alpha_mode, beta, scale,
                       flags, out, snap_interval, track_slots, next_track_idx, nullptr, 0, true,
                       stream);
}

GDN_API gdn_status gdn_decode_step(gdn_pool_t pool, int32_t layer, int32_t batch,
                                   const int32_t *slot_table, const uint16_t *x,
                                   const uint16_t *conv_w, const float *alpha, int32_t alpha_mode,
                                   const float *beta, float scale, uint32_t flags, uint16_t *out,
                                   const int32_t *seq_len_after, int32_t track_interval,
                                   const int32_t *track_slots, const int32_t *next_track_idx,
                                   void *stream) {
  gdn_status s = check_pool(pool, layer);
  if (s != GDN_OK) return s;
  if (batch < 0 || batch > 65535) return fail(GDN_ERR_RANGE, "batch %d outside [0, 65535]", batch);
  if (batch == 0) return ok();
  if (!slot_table || !x || !conv_w || !alpha || !beta || !out)
    return fail(GDN_ERR_ARG, "a required pointer is NULL");
  if (alpha_mode != GDN_ALPHA_PER_HEAD && alpha_mode != GDN_ALPHA_PER_CHANNEL)
    return fail(GDN_ERR_ARG, "alpha_mode %d unknown", alpha_mode);
  if (flags & ~uint32_t(GDN_F_L2NORM_K | GDN_F_L2NORM_Q | GDN_F_CONV_SILU))
    return fail(GDN_ERR_ARG, "unknown flag bits 0x%x", flags);
  if (track_interval < 0) return fail(GDN_ERR_ARG, "track_interval < 0");
  if (track_interval > 0 && (!seq_len_after || !track_slots || !next_track_idx))
    return fail(GDN_ERR_ARG, "tracking needs seq_len_after, track_slots and next_track_idx");
  if (!aligned(conv_w, 16)) return fail(GDN_ERR_UNSUPPORTED, "conv_w must be 16-byte aligned");
  if (!aligned(x, 16)) return fail(GDN_ERR_UNSUPPORTED, "x must be 16-byte aligned");
  if (!aligned(alpha, 16)) return fail(GDN_ERR_UNSUPPORTED, "alpha must be 16-byte aligned");
  gdn::DecodeArgs a{layer,       batch,         slot_table,     x,           conv_w,
                    alpha,       alpha_mode,    beta,           scale,       flags,
                    out,         seq_len_after, track_interval, track_slots, next_track_idx};
  return launched(gdn::launch_decode(pool, a, static_cast<hipStream_t>(stream)),
                  "gdn_decode_step launch");
}

GDN_API gdn_status track_snapshot(gdn_pool_t pool, int32_t layer_begin, int32_t layer_end,
                                  int32_t n, const int32_t *src_slots, const int32_t *dst_slots,
                                  void *stream) {
  if (!pool) return fail(GDN_ERR_ARG, "pool handle is NULL");
  if (layer_begin < 0 || layer_end > pool->d.layers || layer_begin > layer_end)
    return fail(GDN_ERR_RANGE, "layer range [%d, %d) outside [0, %d)", layer_begin, layer_end,
                pool->d.layers);
  if (n < 0) return fail(GDN_ERR_RANGE, "n < 0");
  if (n == 0 || layer_begin == layer_end) return ok();
  if (!src_slots || !dst_slots) return fail(GDN_ERR_ARG, "slot arrays are NULL");
  return launched(gdn::launch_copy_device_pairs(pool, layer_begin, layer_end, n, src_slots,
                                                dst_slots, static_cast<hipStream_t>(stream)),
                  "track_snapshot launch");
}

GDN_API gdn_status restore_slots(gdn_pool_t pool, int32_t n_ops, const gdn_restore_op *ops,
                                 int64_t *has_initial_state, void *stream) {
  if (!pool) return fail(GDN_ERR_ARG, "pool handle is NULL");
  if (n_ops < 0) return fail(GDN_ERR_RANGE, "n_ops < 0");
  if (n_ops == 0) return ok();
  if (!ops || !has_initial_state) return fail(GDN_ERR_ARG, "ops or has_initial_state is NULL");
  int32_t *src = new (std::nothrow) int32_t[n_ops];
  int32_t *dst = new (std::nothrow) int32_t[n_ops];
  if (!src || !dst) {
    delete[] src;
    delete[] dst;
    return fail(GDN_ERR_ARG, "out of host memory");
  }
  // the copies of one call run in parallel, so no copy may read a slot that another
  // copy of the call writes, and no two copies may write one slot: such a call is
  // rejected before any outcome is set
  int n = 0;
  const int slots = pool->d.slots;
  for (int i = 0; i < n_ops; ++i) {
    const gdn_restore_op &op = ops[i];
    const int s = op.restore_src_slot_id, d = op.linear_state_id;
    if (op.restore_requested && s >= 1 && s < slots && d >= 1 && d < slots && s != d) {
      src[n] = s;
      dst[n] = d;
      ++n;
    }
  }
  if (n > 1) {
    int32_t *sorted = new (std::nothrow) int32_t[n];
    if (!sorted) {
      delete[] src;
      delete[] dst;
      return fail(GDN_ERR_ARG, "out of host memory");
    }
    std::copy(dst, dst + n, sorted);
    std::sort(sorted, sorted + n);
    int bad = 0, what = 0;
    for (int i = 0; i + 1 < n && !bad; ++i)
      if (sorted[i] == sorted[i + 1]) bad = sorted[i], what = 1;
    for (int i = 0; i < n && !bad; ++i)
      if (std::binary_search(sorted, sorted + n, src[i])) bad = src[i], what = 2;
    delete[] sorted;
    if (bad) {
      delete[] src;
      delete[] dst;
      return fail(GDN_ERR_ARG,
                  what == 1 ? "restore_slots: slot %d is the destination of two copies"
                            : "restore_slots: slot %d is both a copy source and a copy destination",
                  bad);
    }
  }
  for (int i = 0; i < n_ops; ++i) {
    const gdn_restore_op &op = ops[i];
    if (!op.restore_requested) continue;
    const int s = op.restore_src_slot_id, d = op.linear_state_id;
    has_initial_state[i] = (s < 1 || s >= slots || d < 1 || d >= slots) ? 0   // COLD_START
                                                                          : 1;  // RESTORED
  }
  hipError_t e = n ? gdn::launch_copy_host_pairs(pool, n, src, dst,
                                                 static_cast<hipStream_t>(stream))
                   : hipSuccess;
  delete[] src;
  delete[] dst;
  if (e != hipSuccess) {
    for (int i = 0; i < n_ops; ++i)
      if (ops[i].restore_requested) has_initial_state[i] = 0;
    return fail(GDN_ERR_HIP, "restore_slots launch: %s", hipGetErrorString(e));
  }
  return ok();
}

GDN_API gdn_status gdn_verify_tree(gdn_pool_t pool, int32_t layer, int32_t batch,
                                   int32_t tree_nodes, const int32_t *slot_table,
                                   const int32_t *parent, const uint16_t *x,
                                   const uint16_t *conv_w, const float *alpha, int32_t alpha_mode,
                                   const float *beta, float scale, uint32_t flags, uint16_t *out,
                                   void *node_ssm, uint16_t *node_conv, void *stream) {
  gdn_status s = check_pool(pool, layer);
  if (s != GDN_OK) return s;
  if (batch < 0 || batch > 65535) return fail(GDN_ERR_RANGE, "batch %d outside [0, 65535]", batch);
  if (tree_nodes < 1 || tree_nodes > GDN_MAX_TREE_NODES)
    return fail(GDN_ERR_RANGE, "tree_nodes %d outside [1, %d]", tree_nodes, GDN_MAX_TREE_NODES);
  if (batch == 0) return ok();
  if (!slot_table || !parent || !x || !conv_w || !alpha || !beta || !out || !node_ssm ||
      !node_conv)
    return fail(GDN_ERR_ARG, "a required pointer is NULL");
  if (alpha_mode != GDN_ALPHA_PER_HEAD && alpha_mode != GDN_ALPHA_PER_CHANNEL)
    return fail(GDN_ERR_ARG, "alpha_mode %d unknown", alpha_mode);
  if (flags & ~uint32_t(GDN_F_L2NORM_K | GDN_F_L2NORM_Q | GDN_F_CONV_SILU))
    return fail(GDN_ERR_ARG, "unknown flag bits 0x%x", flags);
  if (!aligned(conv_w, 16) || !aligned(x, 16) || !aligned(alpha, 16))
    return fail(GDN_ERR_UNSUPPORTED, "x, conv_w and alpha must be 16-byte aligned");
  if (!aligned(node_ssm, 16) || !aligned(node_conv, 16))
    return fail(GDN_ERR_UNSUPPORTED, "node_ssm and node_conv must be 16-byte aligned");
  gdn::VerifyArgs a{layer, batch,      tree_nodes, slot_table, parent, x,        conv_w,
                    alpha, alpha_mode, beta,       scale,      flags,  out,      node_ssm,
                    node_conv};
  return launched(gdn::launch_verify(pool, a, static_cast<hipStream_t>(stream)),
                  "gdn_verify_tree launch");
}

GDN_API gdn_status gdn_accept_scatter(gdn_pool_t pool, int32_t layer, int32_t batch,
                                      int32_t tree_nodes, const int32_t *slot_table,
                                      const int32_t *parent, const int32_t *accepted,
                                      const int32_t *seq_len_before, int32_t track_interval,
                                      const int32_t *track_slots, const int32_t *next_track_idx,
                                      const void *node_ssm, const uint16_t *node_conv,
                                      void *stream) {
  gdn_status s = check_pool(pool, layer);
  if (s != GDN_OK) return s;
  if (batch < 0 || batch > 65535) return fail(GDN_ERR_RANGE, "batch %d outside [0, 65535]", batch);
  if (tree_nodes < 1 || tree_nodes > GDN_MAX_TREE_NODES)
    return fail(GDN_ERR_RANGE, "tree_nodes %d outside [1, %d]", tree_nodes, GDN_MAX_TREE_NODES);
  if (track_interval < 0) return fail(GDN_ERR_ARG, "track_interval < 0");
  if (batch == 0) return ok();
  if (!slot_table || !parent || !accepted || !node_ssm || !node_conv)
    return fail(GDN_ERR_ARG, "a required pointer is NULL");
  if (track_interval > 0 && (!seq_len_before || !track_slots || !next_track_idx))
    return fail(GDN_ERR_ARG, "tracking needs seq_len_before, track_slots and next_track_idx");
  if (!aligned(node_ssm, 16) || !aligned(node_conv, 16))
    return fail(GDN_ERR_UNSUPPORTED, "node_ssm and node_conv must be 16-byte aligned");
  gdn::ScatterArgs a{layer,          batch,       tree_nodes,     slot_table,
                     parent,         accepted,    seq_len_before, track_interval,
                     track_slots,    next_track_idx, node_ssm,    node_conv};
  return launched(gdn::launch_accept_scatter(pool, a, static_cast<hipStream_t>(stream)),
                  "gdn_accept_scatter launch");
}

namespace {
gdn_status check_ring(gdn_pool_t, const gdn_replay_ring *r) {
  if (!r) return fail(GDN_ERR_ARG, "ring is NULL");
  if (r->positions < 1 || r->positions > GDN_MAX_RING_POSITIONS)
    return fail(GDN_ERR_RANGE, "ring positions %d outside [1, %d]", r->positions, GDN_MAX_RING_POSITIONS);
  if (r->alpha_mode != GDN_ALPHA_PER_HEAD && r->alpha_mode != GDN_ALPHA_PER_CHANNEL)
    return fail(GDN_ERR_ARG, "ring alpha_mode %d unknown", r->alpha_mode);
  if (!r->rawk || !r->rawv || !r->g || !r->beta || !r->xrow)
    return fail(GDN_ERR_ARG, "a ring array is NULL");
  if (!aligned(r->rawk, 16) || !aligned(r->rawv, 16) || !aligned(r->xrow, 16) || !aligned(r->g, 4) ||
      !aligned(r->beta, 4))
    return fail(GDN_ERR_UNSUPPORTED, "rawk, rawv, xrow must be 16-byte aligned, g and beta 4-byte");
  return GDN_OK;
}
}  // namespace

GDN_API gdn_status replayssm_ring_bytes(gdn_pool_t pool, int32_t positions, int32_t alpha_mode,
                                        size_t bytes[5]) {
  if (!pool || !bytes) return fail(GDN_ERR_ARG, "pool or bytes is NULL");
  if (positions < 1 || positions > GDN_MAX_RING_POSITIONS)
    return fail(GDN_ERR_RANGE, "positions %d outside [1, %d]", positions, GDN_MAX_RING_POSITIONS);
  if (alpha_mode != GDN_ALPHA_PER_HEAD && alpha_mode != GDN_ALPHA_PER_CHANNEL)
    return fail(GDN_ERR_ARG, "alpha_mode %d unknown", alpha_mode);
  const size_t rows = size_t(pool->d.layers) * pool->d.slots * pool->d.heads * positions;
  bytes[0] = rows * pool->d.head_k * 2;
  bytes[1] = rows * pool->d.head_v * 2;
  bytes[2] = rows * (alpha_mode == GDN_ALPHA_PER_CHANNEL ? pool->d.head_k : 1) * 4;
  bytes[3] = rows * 4;
  bytes[4] = size_t(pool->d.layers) * pool->d.slots * positions * size_t(pool->C) * 2;
  return ok();
}

GDN_API gdn_status replayssm_verify(gdn_pool_t pool, const gdn_replay_ring *ring, int32_t layer,
                                    int32_t batch, int32_t draft, const int32_t *slot_table,
                                    const uint16_t *x, const uint16_t *conv_w, const float *alpha,
                                    const float *beta, float scale, uint32_t flags, uint16_t *out,
                                    void *stream) {
  gdn_status s = check_pool(pool, layer);
  if (s != GDN_OK) return s;
  if ((s = check_ring(pool, ring)) != GDN_OK) return s;
  if (batch < 0 || batch > 65535) return fail(GDN_ERR_RANGE, "batch %d outside [0, 65535]", batch);
  if (draft < 1 || draft > ring->positions)
    return fail(GDN_ERR_RANGE, "draft %d outside [1, %d]", draft, ring->positions);
  if (batch == 0) return ok();
  if (!slot_table || !x || !conv_w || !alpha || !beta || !out)
    return fail(GDN_ERR_ARG, "a required pointer is NULL");
  if (flags & ~uint32_t(GDN_F_L2NORM_K | GDN_F_L2NORM_Q | GDN_F_CONV_SILU))
    return fail(GDN_ERR_ARG, "unknown flag bits 0x%x", flags);
  if (!aligned(conv_w, 16) || !aligned(x, 16) || !aligned(alpha, 16))
    return fail(GDN_ERR_UNSUPPORTED, "x, conv_w and alpha must be 16-byte aligned");
  gdn::ReplayArgs a{};
  a.ring = *ring;
  a.layer = layer;
  a.batch = batch;
  a.draft = draft;
  a.slot_table = slot_table;
  a.x = x;
  a.conv_w = conv_w;
  a.alpha = alpha;
  a.beta = beta;
  a.scale = scale;
  a.flags = flags;
  a.out = out;
  return launched(gdn::launch_replay_verify(pool, a, static_cast<hipStream_t>(stream)),
                  "replayssm_verify launch");
}

GDN_API gdn_status replayssm_commit(gdn_pool_t pool, const gdn_replay_ring *ring, int32_t layer,
                                    int32_t batch, const int32_t *slot_table,
                                    const int32_t *accepted, uint32_t flags,
                                    const int32_t *seq_len_before, int32_t track_interval,
                                    const int32_t *track_slots, const int32_t *next_track_idx,
                                    void *stream) {
  gdn_status s = check_pool(pool, layer);
  if (s != GDN_OK) return s;
  if ((s = check_ring(pool, ring)) != GDN_OK) return s;
  if (batch < 0 || batch > 65535) return fail(GDN_ERR_RANGE, "batch %d outside [0, 65535]", batch);
  if (track_interval < 0) return fail(GDN_ERR_ARG, "track_interval < 0");
  if (batch == 0) return ok();
  if (!slot_table || !accepted) return fail(GDN_ERR_ARG, "slot_table or accepted is NULL");
  if (flags & ~uint32_t(GDN_F_L2NORM_K | GDN_F_L2NORM_Q | GDN_F_CONV_SILU))
    return fail(GDN_ERR_ARG, "unknown flag bits 0x%x", flags);
  if (track_interval > 0 && (!seq_len_before || !track_slots || !next_track_idx))
    return fail(GDN_ERR_ARG, "tracking needs seq_len_before, track_slots and next_track_idx");
  gdn::ReplayArgs a{};
  a.ring = *ring;
  a.layer = layer;
  a.batch = batch;
  a.slot_table = slot_table;
  a.flags = flags;
  a.accepted = accepted;
  a.seq_len_before = seq_len_before;
  a.track_interval = track_interval;
  a.track_slots = track_slots;
  a.next_track_idx = next_track_idx;
  return launched(gdn::launch_replay_commit(pool, a, static_cast<hipStream_t>(stream)),
                  "replayssm_commit launch");
}
