/*
 * gdn_oracle.h -- CPU oracle for the slot-indexed gated delta rule.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the package
 * smoke check and the benchmark's CPU-baseline leg may load this library.  The
 * HIP path never links it, includes this header, or calls it; the two share no
 * source.  It is built twice from one source file: liboracle_f64.so computes in
 * double, liboracle_f32.so in float (the "plain sequential fp32" oracle).
 *
 * Everything here is a slow, sequential restatement of what the pages define:
 *   - the recurrence S' = S Diag(alpha) + d k^T, d = beta (v - S Diag(alpha) k)
 *     (page "企业官网建设流程全解析", Kimi K3 notes, section "Speculative
 *     decoding"), with o = S q taken from the updated state;
 *   - the kernel-4 causal short convolution whose state keeps the last three raw
 *     projected q/k/v rows, shape [3, Q+K+V] (same page, section
 *     "Linear的kv cache大小具体计算逻辑");
 *   - the in-kernel L2 normalisation of the raw key (same page, "Speculative
 *     decoding": the kernel sees k before L2 normalisation);
 *   - pool slots [layer][slot] holding conv + temporal state, slot 0 reserved
 *     (page "SGLang之MambaRadixCache机制", section 1.3; page "Qwen3.5
 *     Linear-State Prefix Cache", section 2.3);
 *   - snapshot into ping-pong track slots (page "SGLang Mamba Radix Cache
 *     深度解析：extra_buffer 模式的 Ping-Pong 缓冲机制", sections "Prefill 阶段"
 *     and "Decode 阶段"; Kimi K3 notes, section "--mamba-track-interval");
 *   - the copy semantics of copy_from (page "SGLang之MambaRadixCache机制",
 *     section 3.2) and of restore_linear_state_slots (page "Qwen3.5
 *     Linear-State Prefix Cache", sections 6.1 and 6.4);
 *   - the speculative verify over a draft tree and the accepted-step scatter
 *     (page "SGLang之MambaRadixCache机制", sections 8.3, 8.4, 8.6 and 9.6);
 *   - the ReplaySSM ring verify and exact-fold commit (page "企业官网建设流程全解析",
 *     Kimi K3 notes, section "ReplaySSM"; page "SGLang之MambaRadixCache机制",
 *     sections 9.2 and 9.10).
 *
 * Pool byte layout (identical to the product's so that pool images can be
 * compared byte for byte):
 *   ssm  [layers][slots][heads][head_v][head_k]   float32 or bf16, head_k fastest
 *   conv [layers][slots][3][C]                    bf16, C = heads*(2*head_k+head_v)
 * Channel order inside x and conv rows: q | k | v, each head-major.
 *
 * Error returns: bitmask, 0 = clean.  1 = a live slot id >= slots was skipped,
 * 2 = a track/destination slot id >= slots was skipped, 4 = bad argument,
 * 8 = an invalid draft tree or accepted node was skipped.
 */
#ifndef GDN_ORACLE_H
#define GDN_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_SSM_F32 = 0, ORACLE_SSM_BF16 = 1 };
enum { ORACLE_ALPHA_PER_HEAD = 0, ORACLE_ALPHA_PER_CHANNEL = 1 };
enum { ORACLE_L2NORM_K = 1u, ORACLE_L2NORM_Q = 2u, ORACLE_CONV_SILU = 4u };

typedef struct {
  int32_t layers, slots, heads, head_k, head_v;
  int32_t ssm_dtype;   /* ORACLE_SSM_F32 | ORACLE_SSM_BF16 */
  void *ssm;           /* host bytes, layout above */
  uint16_t *conv;      /* host bf16, layout above */
} oracle_pool;

/* ReplaySSM ring: per (layer, slot, head, position) the inputs that regenerate
 * a draft step's state.  rawk/rawv bf16 [L][N][H][P][K|V]; g fp32 [L][N][H][P]
 * (per-head decay) or [L][N][H][P][K] (per channel); beta fp32 [L][N][H][P];
 * xrow bf16 [L][N][P][C] (the conv input row of the position). */
typedef struct {
  int32_t positions;   /* P */
  int32_t alpha_mode;  /* ORACLE_ALPHA_PER_HEAD | ORACLE_ALPHA_PER_CHANNEL */
  uint16_t *rawk;
  uint16_t *rawv;
  float *g;
  float *beta;
  uint16_t *xrow;
} oracle_ring;

typedef struct {
  int32_t linear_state_id;
  int32_t restore_requested;
  int32_t restore_src_slot_id;
} oracle_restore_op;

/* Size of the arithmetic type of this compiled variant of the oracle: 4 or 8. */
int oracle_real_bytes(void);

/* Threads the OpenMP loops use. */
int oracle_num_threads(void);

/* Bytes of the two pool buffers for the given shape. Returns 4 on bad shape. */
int oracle_pool_bytes(int32_t layers, int32_t slots, int32_t heads, int32_t head_k,
                      int32_t head_v, int32_t ssm_dtype, size_t *ssm_bytes,
                      size_t *conv_bytes);

/* Fold the tokens of each request into its live slot (prefill).
 * cu_seqlens[batch+1] token offsets into x/alpha/beta/out.  x bf16 [T][C];
 * conv_w bf16 [C][4] (tap 3 multiplies the current token); alpha float
 * [T][H] or [T][H][K]; beta float [T][H]; out bf16 [T][H][V].
 * has_initial_state[b] == 0 starts from zero state and zero conv rows.
 * Snapshots: for snap_interval > 0, after folding the token that makes the
 * request's length n = start_len[b] + i + 1 a multiple of snap_interval, the
 * j-th such boundary in this call goes to track_slots[2b + ((next_track_idx[b]
 * + j) & 1)].  Optional out_exact [T][H][V] and state_exact [batch][H][V][K]
 * (may be NULL) receive the unrounded outputs and final states (as double). */
int oracle_prefill(const oracle_pool *pool, int32_t layer, int32_t batch,
                   const int32_t *cu_seqlens, const int32_t *slot_table,
                   const int32_t *has_initial_state, const int32_t *start_len,
                   const uint16_t *x, const uint16_t *conv_w, const float *alpha,
                   int32_t alpha_mode, const float *beta, float scale, uint32_t flags,
                   uint16_t *out, int32_t snap_interval, const int32_t *track_slots,
                   const int32_t *next_track_idx, double *out_exact, double *state_exact);

/* One decode token per request: x bf16 [B][C], alpha [B][H] or [B][H][K],
 * beta [B][H], out bf16 [B][H][V].  The state is always loaded from the slot.
 * If track_interval > 0 and seq_len_after[b] % track_interval == 0 the updated
 * state is also written to track_slots[2b + next_track_idx[b]]. */
int oracle_decode_step(const oracle_pool *pool, int32_t layer, int32_t batch,
                       const int32_t *slot_table, const uint16_t *x,
                       const uint16_t *conv_w, const float *alpha, int32_t alpha_mode,
                       const float *beta, float scale, uint32_t flags, uint16_t *out,
                       const int32_t *seq_len_after, int32_t track_interval,
                       const int32_t *track_slots, const int32_t *next_track_idx,
                       double *out_exact, double *state_exact);

/* Copy conv + ssm of layers [layer_begin, layer_end) from src_slots[i] to
 * dst_slots[i]; dst <= 0 skips the entry. */
int oracle_track_snapshot(const oracle_pool *pool, int32_t layer_begin, int32_t layer_end,
                          int32_t n, const int32_t *src_slots, const int32_t *dst_slots);

/* restore_linear_state_slots semantics; has_initial_state updated in place. */
int oracle_restore_slots(const oracle_pool *pool, int32_t n_ops, const oracle_restore_op *ops,
                         int64_t *has_initial_state);

/* Verify a draft tree of `nodes` nodes per request for one layer; the live slots
 * are only read.  parent [B][T]: -1 = start from the live slot, else an earlier
 * node.  x [B][T][C], alpha [B][T][H] or [B][T][H][K], beta [B][T][H], out bf16
 * [B][T][H][V]; node_ssm [B][T][H][V][K] in the pool's ssm dtype and node_conv
 * bf16 [B][T][3][C] receive every node's state and conv rows.  out_exact may be
 * NULL. */
int oracle_verify_tree(const oracle_pool *pool, int32_t layer, int32_t batch, int32_t nodes,
                       const int32_t *slot_table, const int32_t *parent, const uint16_t *x,
                       const uint16_t *conv_w, const float *alpha, int32_t alpha_mode,
                       const float *beta, float scale, uint32_t flags, uint16_t *out,
                       void *node_ssm, uint16_t *node_conv, double *out_exact);

/* Copy node accepted[b] (>= 0) of each request into its live slot, and the node
 * on the accepted path that reaches each multiple of track_interval (counting
 * from seq_len_before[b]) into the ping-pong track slots. */
int oracle_accept_scatter(const oracle_pool *pool, int32_t layer, int32_t batch, int32_t nodes,
                          const int32_t *slot_table, const int32_t *parent, const int32_t *accepted,
                          const int32_t *seq_len_before, int32_t track_interval,
                          const int32_t *track_slots, const int32_t *next_track_idx,
                          const void *node_ssm, const uint16_t *node_conv);

/* Byte sizes of the ring arrays {rawk, rawv, g, beta, xrow} for the pool's shape. */
int oracle_ring_bytes(const oracle_pool *pool, int32_t positions, int32_t alpha_mode,
                      size_t bytes[5]);

/* Verify a chain of `draft` tokens per request from its live slot (only read),
 * out [B][D][H][V]; ring positions 0 .. draft-1 of the slot receive the inputs
 * the commit replays.  x [B][D][C], alpha [B][D][H] or [B][D][H][K], beta
 * [B][D][H].  out_exact may be NULL. */
int oracle_replay_verify(const oracle_pool *pool, const oracle_ring *ring, int32_t layer,
                         int32_t batch, int32_t draft, const int32_t *slot_table,
                         const uint16_t *x, const uint16_t *conv_w, const float *alpha,
                         int32_t alpha_mode, const float *beta, float scale, uint32_t flags,
                         uint16_t *out, double *out_exact);

/* Fold ring positions 0 .. accepted[b]-1 into each live slot (state and conv
 * rows), snapshotting at multiples of track_interval. */
int oracle_replay_commit(const oracle_pool *pool, const oracle_ring *ring, int32_t layer,
                         int32_t batch, const int32_t *slot_table, const int32_t *accepted,
                         int32_t alpha_mode, uint32_t flags, const int32_t *seq_len_before,
                         int32_t track_interval, const int32_t *track_slots,
                         const int32_t *next_track_idx);

/* The bare recurrence for one head over T prepared tokens (no conv, no norm):
 * q, k, v [T][K|V] as given, alpha [T][K], beta [T]; S [V][K] in/out;
 * o [T][V] = scale * S_t q_t. */
void oracle_recurrence_head(int32_t T, int32_t K, int32_t V, const double *q,
                            const double *k, const double *v, const double *alpha,
                            const double *beta, double scale, double *S, double *o);

/* The same map computed chunk by chunk in the WY form, in double, for pinning
 * that algebra against oracle_recurrence_head. */
void oracle_chunked_head_f64(int32_t T, int32_t K, int32_t V, int32_t chunk,
                             const double *q, const double *k, const double *v,
                             const double *alpha, const double *beta, double scale,
                             double *S, double *o);

/* RNE conversion helpers, exported so tests can check them. */
uint16_t oracle_bf16_round(double x);
double oracle_bf16_widen(uint16_t h);

#ifdef __cplusplus
}
#endif
#endif
