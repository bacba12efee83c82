/*
 * gdn_slot.h -- C ABI of the MI355X (gfx950) slot-indexed gated delta rule.
 *
 * What it computes.  Hybrid linear-attention models keep, per linear layer and
 * per request, a fixed-size recurrent state in a pooled buffer: a conv window
 * of the last three projected q/k/v rows and a temporal state S of shape
 * [heads, head_v, head_k] (page "企业官网建设流程全解析", Kimi K3 notes,
 * sections "Temporal/SSM state" and "Linear的kv cache大小具体计算逻辑"; page
 * "SGLang之MambaRadixCache机制", section 1.3).  Every token of a request
 * updates the slot that the request's slot-table entry names, in place (page
 * "SGLang之MambaRadixCache机制", section 5.1; page "Qwen3.5 Linear-State Prefix
 * Cache", section 2.1):
 *
 *   y      = causal conv, kernel 4, over [r0, r1, r2, x_t]   (r = conv rows)
 *   q|k|v  = split of y, head-major;  k <- k / sqrt(sum k^2 + 1e-6)
 *   S'     = S Diag(alpha_t)                       (alpha per head or per channel)
 *   d      = beta_t (v - S' k)
 *   S      = S' + d k^T
 *   o_t    = scale * S q                           (bf16)
 *
 * (recurrence: page "企业官网建设流程全解析", section "Speculative decoding").
 * Snapshots copy the live state into ping-pong track slots at chunk and
 * track-interval boundaries (page "SGLang Mamba Radix Cache 深度解析：
 * extra_buffer 模式的 Ping-Pong 缓冲机制", sections "Prefill 阶段" and "Decode
 * 阶段"), and a prefix hit copies the deepest checkpoint slot into the live
 * slot across all layers before a warm prefill (page "Qwen3.5 Linear-State
 * Prefix Cache", sections 5.1, 6.1 and 6.4).  Speculative decoding verifies a
 * draft tree without touching the live slot and then commits the accepted step
 * (page "SGLang之MambaRadixCache机制解析", sections 8.3, 8.4, 8.6 and 9.6).
 *
 * Memory.  The caller owns every buffer (pool bytes, inputs, outputs, tables,
 * the error word, the prefill workspace); the library allocates and frees no
 * device memory.  All
 * pointers marked "device" must be device-accessible on the current device.
 *
 *   ssm  pool  [layers][slots][heads][head_v][head_k]  fp32 or bf16, head_k fastest
 *   conv pool  [layers][slots][3][C]                   bf16, C = heads*(2*head_k+head_v)
 *   x          [tokens][C]     bf16, channel order q | k | v, each head-major
 *   conv_w     [C][4]          bf16, tap 3 multiplies the current token
 *   alpha      [tokens][heads] or [tokens][heads][head_k]   fp32, decay in (0, 1]
 *   beta       [tokens][heads] fp32
 *   out        [tokens][heads][head_v] bf16
 *
 * Slot ids.  Slot 0 is reserved (padding) and never written (page "Qwen3.5
 * Linear-State Prefix Cache", section 2.3).  A slot-table entry <= 0 skips the
 * request: nothing is read or written for it and its output rows are zeroed.
 * An entry >= slots is skipped the same way and sets bit GDN_ERRW_BAD_SLOT in
 * the pool's error word.  Live slots within one call must be distinct, and so
 * must destination slots within one copy call.
 *
 * Streams and errors.  Every call is asynchronous on the given stream
 * (a hipStream_t passed as void*, NULL = the default stream) with no internal
 * synchronisation (page "Qwen3.5 Linear-State Prefix Cache", section 7.1).
 * Arguments that the host can check are checked before any launch; a failure
 * returns a negative gdn_status, launches nothing, and leaves a message for
 * gdn_last_error() on the calling thread.  Calls that write the same slots must
 * be ordered by the caller (same stream, or events).
 */
#ifndef GDN_SLOT_H
#define GDN_SLOT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct gdn_pool *gdn_pool_t;

typedef enum {
  GDN_OK = 0,
  GDN_ERR_ARG = -1,         /* null pointer, bad enum, inconsistent sizes */
  GDN_ERR_RANGE = -2,       /* layer or count out of range */
  GDN_ERR_UNSUPPORTED = -3, /* shape or alignment the kernels do not handle */
  GDN_ERR_HIP = -4          /* a HIP call failed; see gdn_last_error() */
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

enum { GDN_ALPHA_PER_HEAD = 0, GDN_ALPHA_PER_CHANNEL = 1 };

/* flags */
enum { GDN_F_L2NORM_K = 1u, GDN_F_L2NORM_Q = 2u, GDN_F_CONV_SILU = 4u };
/* prefill path (conv_gdn_prefill_chunked only; with neither bit the library
 * chooses): ONE_KERNEL runs each (request, head) start to end in one workgroup with
 * the state on chip and takes no workspace (NULL and 0 are accepted); it serves
 * head dim 128 with max_seqlen * channels * 2 < 2^31, for a decay per head or per
 * channel, and suits batches of many requests.  (With a decay per channel, a chunk
 * of 64 tokens in which some channel decays below 2^-96 in all is run token by
 * token, which is exact but several times slower.)
 * TWO_KERNEL prepares every chunk in parallel and then scans them; it serves every
 * shape, needs the workspace, and suits a few long requests. */
enum { GDN_F_PREFILL_ONE_KERNEL = 8u, GDN_F_PREFILL_TWO_KERNEL = 16u };
/* prefill snapshots (conv_gdn_prefill_chunked only): by default every boundary of
 * the call is written to its track slot.  With SNAP_LAST_ONLY only the last
 * boundary of each ping-pong parity is written: an earlier boundary of the same
 * parity is overwritten within the call, so the pool after the call is the same,
 * but another stream reading a track slot during the call sees fewer states. */
enum { GDN_F_SNAP_LAST_ONLY = 32u };

/* bits a kernel may set in the pool's error word (sticky; the caller clears it) */
enum {
  GDN_ERRW_BAD_SLOT = 1,
  GDN_ERRW_BAD_TRACK_SLOT = 2,
  GDN_ERRW_BAD_SEQLENS = 4,
  GDN_ERRW_BAD_TREE = 8  /* a draft tree or accepted node that is not valid */
};

/* Largest draft tree (nodes per request) the verify and scatter calls accept. */
#define GDN_MAX_TREE_NODES 1024

/* Largest ReplaySSM ring (positions per slot). */
#define GDN_MAX_RING_POSITIONS 64

typedef struct {
  int32_t layers, slots, heads, head_k, head_v;
  int32_t conv_kernel;   /* must be 4 */
  int32_t ssm_dtype;     /* GDN_F32 | GDN_BF16 */
  int32_t conv_dtype;    /* GDN_BF16 */
  void *ssm_base;        /* device, 16-byte aligned, state_pool_bytes() bytes */
  void *conv_base;       /* device, 16-byte aligned */
  int32_t *err_word;     /* device int32 or NULL */
} gdn_pool_desc;

/* ReplaySSM ring (page "企业官网建设流程全解析", Kimi K3 notes, section
 * "ReplaySSM"): per (layer, slot, head, position) the inputs that regenerate a
 * draft step's state, so that a verify keeps no per-step state.  All arrays are
 * device memory owned by the caller, indexed by the pool's layers and slots:
 *   rawk  bf16 [layers][slots][heads][positions][head_k]  k as it leaves the conv
 *         (before L2 normalisation)
 *   rawv  bf16 [layers][slots][heads][positions][head_v]  v as it leaves the conv
 *   g     fp32 [layers][slots][heads][positions] (GDN_ALPHA_PER_HEAD) or
 *         [layers][slots][heads][positions][head_k] (GDN_ALPHA_PER_CHANNEL): the decay
 *   beta  fp32 [layers][slots][heads][positions]
 *   xrow  bf16 [layers][slots][positions][C]: the conv input row of the position
 *         (the conv state must advance with the accepted tokens)
 * Sizes: replayssm_ring_bytes.  rawk, rawv, xrow 16-byte aligned. */
typedef struct {
  int32_t positions;   /* 1 .. GDN_MAX_RING_POSITIONS */
  int32_t alpha_mode;  /* GDN_ALPHA_PER_HEAD | GDN_ALPHA_PER_CHANNEL: layout of g and of alpha */
  uint16_t *rawk;
  uint16_t *rawv;
  float *g;
  float *beta;
  uint16_t *xrow;
} gdn_replay_ring;

/* Restore request, one per sequence (page "Qwen3.5 Linear-State Prefix Cache",
 * section 6.1): copy restore_src_slot_id into linear_state_id. */
typedef struct {
  int32_t linear_state_id;
  int32_t restore_requested;   /* 0 or 1 */
  int32_t restore_src_slot_id; /* < 0: no source was found */
} gdn_restore_op;

/* Byte sizes of the two pool buffers for a descriptor's shape (pointers in the
 * descriptor are ignored).  Pure host arithmetic. */
gdn_status state_pool_bytes(const gdn_pool_desc *desc, size_t *ssm_bytes, size_t *conv_bytes);

/* Validate a descriptor and wrap it in a handle (host memory only).  Supported:
 * head_k == head_v in {16, 32, 64, 128}, conv_kernel 4, bf16 conv state, fp32 or
 * bf16 ssm state, both bases 16-byte aligned.  The handle does not own the
 * buffers.  Thread-safe; the handle is immutable. */
gdn_status state_pool_create(const gdn_pool_desc *desc, gdn_pool_t *out);

/* Free a handle (not the buffers).  NULL is ignored. */
void state_pool_destroy(gdn_pool_t pool);

/* Message of the last failing call on this thread ("" if none). */
const char *gdn_last_error(void);

/* Device workspace that conv_gdn_prefill_chunked needs to process a batch of
 * `batch` requests, none longer than max_seqlen tokens, in a single pass.  Less
 * is accepted (the call then works through the chunks in several windows) down
 * to the minimum reported for max_seqlen = 64.  Pure host arithmetic. */
gdn_status gdn_prefill_workspace_bytes(gdn_pool_t pool, int32_t batch, int32_t max_seqlen,
                                       size_t *bytes);

/* Chunked prefill of one layer for a batch of variable-length requests.
 * cu_seqlens  device int32 [batch+1], non-decreasing, cu_seqlens[batch] <= total_tokens
 * max_seqlen  host int: no request is longer (longer ones set GDN_ERRW_BAD_SEQLENS
 *             and are skipped)
 * slot_table  device int32 [batch]   live slot of each request
 * has_initial_state device int32 [batch]: 1 = continue from the slot, 0 = start
 *             from zero state and zero conv rows (page "Qwen3.5 Linear-State Prefix
 *             Cache", section 6.4, warm/cold)
 * start_len   device int32 [batch]   tokens already folded into the slot before
 *             this call (only used to place snapshots; may be NULL if snap_interval == 0)
 * snap_interval 0 (no snapshots) or a positive multiple of 64: after the token that
 *             makes the request length n = start_len + i + 1 a multiple of it, the
 *             j-th such boundary of the call is written to
 *             track_slots[2b + ((next_track_idx[b] + j) & 1)] (device int32 [batch][2]
 *             and [batch]); an entry <= 0 skips that snapshot.  Chunks are 64 tokens
 *             (page "SGLang Mamba Radix Cache 深度解析", configuration:
 *             mamba_cache_chunk_size defaults to 64).
 * workspace   device scratch of workspace_bytes bytes, 256-byte aligned, owned by the
 *             caller and not read across calls (see gdn_prefill_workspace_bytes).  The
 *             one-kernel path does not use it (NULL and 0 are accepted there); the
 *             two-kernel path returns GDN_ERR_ARG below the minimum.
 * flags       GDN_F_L2NORM_K | GDN_F_L2NORM_Q | GDN_F_CONV_SILU, GDN_F_SNAP_LAST_ONLY,
 *             and at most one of GDN_F_PREFILL_ONE_KERNEL / GDN_F_PREFILL_TWO_KERNEL
 *             (ONE_KERNEL on a shape it does not serve returns GDN_ERR_UNSUPPORTED).
 *             Without either, the one-kernel path runs when it serves the shape and
 *             batch * heads >= 128.  Both paths compute the same thing to the stated
 *             tolerance.
 * The live slot receives the state after the last token.  Requests of length 0
 * leave a warm slot unchanged and zero a cold one. */
gdn_status conv_gdn_prefill_chunked(gdn_pool_t pool, int32_t layer, int32_t batch,
                                    int32_t total_tokens, int32_t max_seqlen,
                                    const int32_t *cu_seqlens, const int32_t *slot_table,
                                    const int32_t *has_initial_state, const int32_t *start_len,
                                    const uint16_t *x, const uint16_t *conv_w, const float *alpha,
                                    int32_t alpha_mode, const float *beta, float scale,
                                    uint32_t flags, uint16_t *out, int32_t snap_interval,
                                    const int32_t *track_slots, const int32_t *next_track_idx,
                                    void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of the fixed device scratch behind conv_gdn_prefill_chunked_noalloc: one
 * copy per GPU the library runs on, held until the process ends. */
#define GDN_NOALLOC_SCRATCH_BYTES (64u << 20)

/* conv_gdn_prefill_chunked for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, meaning and results, without the workspace: the two-kernel
 * path works in the library's fixed per-device scratch of
 * GDN_NOALLOC_SCRATCH_BYTES bytes (in windows of as many chunks as it holds), and
 * the one-kernel path needs none.  The call allocates nothing and frees nothing.
 * A two-kernel batch whose minimum workspace (gdn_prefill_workspace_bytes with
 * max_seqlen = 64) exceeds the scratch returns GDN_ERR_RANGE and launches
 * nothing; split the batch.  The first call on a device looks up the scratch's
 * address there (GDN_ERR_HIP if that fails).  All calls on one GPU share its
 * scratch, and the scratch keeps the last call's contents: calls that overlap on
 * one GPU (different streams, or different host threads without ordering) race
 * and must not be issued. */
gdn_status conv_gdn_prefill_chunked_noalloc(gdn_pool_t pool, int32_t layer, int32_t batch,
                                            int32_t total_tokens, int32_t max_seqlen,
                                            const int32_t *cu_seqlens, const int32_t *slot_table,
                                            const int32_t *has_initial_state,
                                            const int32_t *start_len, const uint16_t *x,
                                            const uint16_t *conv_w, const float *alpha,
                                            int32_t alpha_mode, const float *beta, float scale,
                                            uint32_t flags, uint16_t *out, int32_t snap_interval,
                                            const int32_t *track_slots,
                                            const int32_t *next_track_idx, void *stream);

/* One decode token per request for one layer (x [batch][C], alpha [batch][heads]
 * or [batch][heads][head_k], beta [batch][heads], out [batch][heads][head_v]).
 * The state is always read from the slot.  If track_interval > 0 and
 * seq_len_after[b] % track_interval == 0 (tokens folded after this step), the
 * updated conv + ssm state is also written to track_slots[2b + next_track_idx[b]]
 * (page "企业官网建设流程全解析", section "--mamba-track-interval"; page
 * "SGLang Mamba Radix Cache 深度解析", section "Decode 阶段").  The caller flips
 * next_track_idx once per step, after the last layer. */
gdn_status gdn_decode_step(gdn_pool_t pool, int32_t layer, int32_t batch,
                           const int32_t *slot_table, const uint16_t *x, const uint16_t *conv_w,
                           const float *alpha, int32_t alpha_mode, const float *beta, float scale,
                           uint32_t flags, uint16_t *out, const int32_t *seq_len_after,
                           int32_t track_interval, const int32_t *track_slots,
                           const int32_t *next_track_idx, void *stream);

/* Copy conv + ssm state of layers [layer_begin, layer_end) from src_slots[i] to
 * dst_slots[i] for i < n (device int32 arrays).  dst <= 0 skips the entry; an id
 * >= slots (or src <= 0 with dst > 0) skips it and sets GDN_ERRW_BAD_TRACK_SLOT.
 * This is the masked track copy (page "企业官网建设流程全解析", section
 * "--mamba-track-interval", the scatter into the track slot) and copy_from /
 * fork (page "SGLang之MambaRadixCache机制", section 3.2).  Byte-exact.
 * The pairs are copied in parallel: the destinations must be distinct and no
 * source may be the destination of another pair (a chain a->b, b->c has no
 * defined result).  The arrays live on the device, so this is not checked. */
gdn_status track_snapshot(gdn_pool_t pool, int32_t layer_begin, int32_t layer_end, int32_t n,
                          const int32_t *src_slots, const int32_t *dst_slots, void *stream);

/* restore_linear_state_slots (page "Qwen3.5 Linear-State Prefix Cache", sections
 * 5.1 and 6.4).  ops and has_initial_state are HOST arrays of n_ops entries; the
 * host decides each op's outcome before launching:
 *   restore_requested == 0                       -> has_initial_state[i] unchanged
 *   src < 1 or src >= slots or dst < 1 or dst >= slots -> 0 (COLD_START), no copy
 *   src == dst                                   -> 1 (RESTORED), no copy
 *   otherwise: copy conv + ssm of every layer    -> 1 (RESTORED)
 * The copies run in parallel, so a call in which two copies write one slot, or
 * a copy reads a slot that another copy of the call writes, returns GDN_ERR_ARG
 * with has_initial_state untouched and launches nothing.  If a launch fails,
 * every requested op of the call is set to 0 and GDN_ERR_HIP is returned.  The
 * copies are queued on the stream (no synchronisation). */
gdn_status restore_slots(gdn_pool_t pool, int32_t n_ops, const gdn_restore_op *ops,
                         int64_t *has_initial_state, void *stream);

/* Verify a draft tree for one layer (page "SGLang之MambaRadixCache机制解析",
 * section 8.3: the main state is not updated and every draft position's result
 * goes to an intermediate buffer; section 9.6: parent -> child inheritance
 * through retrieve_parent_token, parents processed first).  Each request has
 * tree_nodes nodes (1 <= tree_nodes <= GDN_MAX_TREE_NODES).
 * parent      device int32 [batch][tree_nodes]: -1 = start from the live slot,
 *             otherwise an earlier node (parent[b][n] < n)
 * x           device bf16 [batch][tree_nodes][C]: the node's projected token
 * alpha, beta device fp32 [batch][tree_nodes][heads](*head_k for per-channel alpha)
 * out         device bf16 [batch][tree_nodes][heads][head_v]
 * node_ssm    device, pool ssm dtype, [batch][tree_nodes][heads][head_v][head_k]
 * node_conv   device bf16 [batch][tree_nodes][3][C]
 * Node n starts from its parent's state as stored (pool dtype) and conv rows,
 * takes its token as gdn_decode_step would, and stores its state, conv rows
 * and output.  The live slot is only read.  A request whose tree is invalid
 * sets GDN_ERRW_BAD_TREE; it and any request with a skipped slot (see "Slot
 * ids") get zero outputs and no node writes.  node_ssm and node_conv are caller
 * scratch (16-byte aligned) that gdn_accept_scatter reads afterwards. */
gdn_status gdn_verify_tree(gdn_pool_t pool, int32_t layer, int32_t batch, int32_t tree_nodes,
                           const int32_t *slot_table, const int32_t *parent, const uint16_t *x,
                           const uint16_t *conv_w, const float *alpha, int32_t alpha_mode,
                           const float *beta, float scale, uint32_t flags, uint16_t *out,
                           void *node_ssm, uint16_t *node_conv, void *stream);

/* Commit the accepted step of each request after a verify (page
 * "SGLang之MambaRadixCache机制解析", section 8.4: main state of the slot =
 * intermediate state of the last accepted step; section 8.6: the ping-pong
 * track slot too when the accepted tokens cross the track interval; section
 * 9.10: the snapshot is the state at the token that completes the multiple).
 * accepted        device int32 [batch]: last accepted node, -1 = none (no writes)
 * seq_len_before  device int32 [batch]: tokens in the slot before the tree
 * track_interval  0 (no tracking) or > 0
 * track_slots     device int32 [batch][2], next_track_idx device int32 [batch]
 * The accepted node (all heads' state and the conv rows) is copied into the
 * live slot.  With d = depth of the accepted node (1 for a root), every i in
 * [1, d] with (seq_len_before + i) % track_interval == 0 is a crossing; the
 * j-th crossing copies the accepted path's node at depth i into
 * track_slots[2b + ((next_track_idx[b] + j) & 1)] (an entry <= 0 skips it, one
 * >= slots sets GDN_ERRW_BAD_TRACK_SLOT).  An invalid tree or accepted index
 * sets GDN_ERRW_BAD_TREE and skips the request.  Track slots must differ from
 * the live slot.  Byte-exact copies. */
gdn_status gdn_accept_scatter(gdn_pool_t pool, int32_t layer, int32_t batch, int32_t tree_nodes,
                              const int32_t *slot_table, const int32_t *parent,
                              const int32_t *accepted, const int32_t *seq_len_before,
                              int32_t track_interval, const int32_t *track_slots,
                              const int32_t *next_track_idx, const void *node_ssm,
                              const uint16_t *node_conv, void *stream);

/* Byte sizes {rawk, rawv, g, beta, xrow} of a ReplaySSM ring for the pool's
 * shape.  Pure host arithmetic. */
gdn_status replayssm_ring_bytes(gdn_pool_t pool, int32_t positions, int32_t alpha_mode,
                                size_t bytes[5]);

/* Verify a chain of `draft` draft tokens per request with a ReplaySSM ring
 * (page "企业官网建设流程全解析", section "ReplaySSM": every position's output is
 * computed, no per-position state is kept, and the lightweight inputs are
 * recorded).  Token t of request b follows token t-1 (t = 0 follows the live
 * slot); the state stays in fp32 between the tokens, as in a prefill call.
 * x [batch][draft][C], alpha [batch][draft][heads] (or ...[head_k], following
 * ring->alpha_mode), beta [batch][draft][heads], out [batch][draft][heads][head_v];
 * 1 <= draft <= ring->positions.  The live slot is only read; ring positions
 * 0 .. draft-1 of the request's slot are overwritten.  Slot rules as for decode. */
gdn_status replayssm_verify(gdn_pool_t pool, const gdn_replay_ring *ring, int32_t layer,
                            int32_t batch, int32_t draft, const int32_t *slot_table,
                            const uint16_t *x, const uint16_t *conv_w, const float *alpha,
                            const float *beta, float scale, uint32_t flags, uint16_t *out,
                            void *stream);

/* Exact-fold commit (page "企业官网建设流程全解析", section "ReplaySSM": only the
 * accepted prefix is replayed, in recurrent order, into the slot; page
 * "SGLang之MambaRadixCache机制解析", section 9.10: the track boundary is checked
 * during the replay).  accepted device int32 [batch]: 0 .. ring->positions
 * tokens from ring positions 0 .. accepted-1 of the request's slot are folded:
 * k = rawk normalised (flags & GDN_F_L2NORM_K), v = rawv, S' = S Diag(g),
 * d = beta (v - S'k), S = S' + d k^T; conv rows shift through the x rows.  The
 * state is rounded to the pool dtype once, at the end (and at a snapshot).
 * Tracking (track_interval > 0; seq_len_before, track_slots [batch][2],
 * next_track_idx [batch] device int32): for every i in [1, accepted] with
 * (seq_len_before + i) % track_interval == 0, the state and conv rows after
 * token i go to track_slots[2b + ((next_track_idx[b] + j) & 1)] for the j-th
 * such i (entry <= 0 skips, >= slots sets GDN_ERRW_BAD_TRACK_SLOT).  accepted
 * outside [0, positions] sets GDN_ERRW_BAD_TREE and skips the request. */
gdn_status replayssm_commit(gdn_pool_t pool, const gdn_replay_ring *ring, int32_t layer,
                            int32_t batch, const int32_t *slot_table, const int32_t *accepted,
                            uint32_t flags, const int32_t *seq_len_before, int32_t track_interval,
                            const int32_t *track_slots, const int32_t *next_track_idx,
                            void *stream);

#ifdef __cplusplus
}
#endif
#endif /* GDN_SLOT_H */
