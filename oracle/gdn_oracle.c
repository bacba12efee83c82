/*
 * gdn_oracle.c -- CPU oracle for the slot-indexed gated delta rule.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE: see gdn_oracle.h for who may use it
 * and for the passages each function restates.  Plain loops, one token at a
 * time, no blocking or fusion.  Built with -ffp-contract=off and without fast
 * math so every sum is evaluated in the written order.  OpenMP only splits
 * independent (request, head) units or copy entries; results do not depend on
 * the thread count.
 */
#include "gdn_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORACLE_REAL
#define ORACLE_REAL double
#endif
typedef ORACLE_REAL real;

#define CONV_TAPS 4
#define CONV_ROWS (CONV_TAPS - 1)
#define L2_EPS 1e-6

int oracle_real_bytes(void) { return (int)sizeof(real); }

#ifdef _OPENMP
#include <omp.h>
int oracle_num_threads(void) { return omp_get_max_threads(); }
#else
int oracle_num_threads(void) { return 1; }
#endif

/* ---------------------------------------------------------------- bf16 ---- */

double oracle_bf16_widen(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Round to the nearest bf16 (8 significant bits), ties to even, directly from
 * double so that no intermediate float rounding can double-round. */
uint16_t oracle_bf16_round(double x) {
  if (isnan(x)) return 0x7FC0;
  if (isinf(x)) return x > 0 ? 0x7F80 : 0xFF80;
  if (x == 0.0) return signbit(x) ? 0x8000 : 0x0000;
  int e = ilogb(x);
  if (e < -126) e = -126;                  /* subnormal quantum is 2^-133 */
  double quantum = ldexp(1.0, e - 7);
  double r = nearbyint(x / quantum) * quantum; /* default mode: ties to even */
  if (fabs(r) > 3.3895313892515355e38) return signbit(x) ? 0xFF80 : 0x7F80;
  float f = (float)r;                       /* exact: r has <= 8 bits */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

static real widen(uint16_t h) { return (real)oracle_bf16_widen(h); }

/* ---------------------------------------------------------------- pool ---- */

static size_t conv_channels(const oracle_pool *p) {
  return (size_t)p->heads * (size_t)(2 * p->head_k + p->head_v);
}
static size_t ssm_block_elems(const oracle_pool *p) {
  return (size_t)p->heads * p->head_v * p->head_k;
}
static size_t ssm_esize(const oracle_pool *p) { return p->ssm_dtype == ORACLE_SSM_F32 ? 4 : 2; }

/* Byte address of the ssm block of (layer, slot). */
static unsigned char *ssm_block(const oracle_pool *p, int layer, int slot) {
  size_t idx = ((size_t)layer * p->slots + (size_t)slot) * ssm_block_elems(p);
  return (unsigned char *)p->ssm + idx * ssm_esize(p);
}
/* Address of conv row 0 of (layer, slot). */
static uint16_t *conv_block(const oracle_pool *p, int layer, int slot) {
  return p->conv + ((size_t)layer * p->slots + (size_t)slot) * CONV_ROWS * conv_channels(p);
}

static real load_ssm(const oracle_pool *p, const unsigned char *blk, size_t i) {
  if (p->ssm_dtype == ORACLE_SSM_F32) {
    float f;
    memcpy(&f, blk + 4 * i, 4);
    return (real)f;
  }
  uint16_t h;
  memcpy(&h, blk + 2 * i, 2);
  return widen(h);
}
static void store_ssm(const oracle_pool *p, unsigned char *blk, size_t i, real x) {
  if (p->ssm_dtype == ORACLE_SSM_F32) {
    float f = (float)x; /* round to nearest even */
    memcpy(blk + 4 * i, &f, 4);
  } else {
    uint16_t h = oracle_bf16_round((double)x);
    memcpy(blk + 2 * i, &h, 2);
  }
}

int oracle_pool_bytes(int32_t layers, int32_t slots, int32_t heads, int32_t head_k,
                      int32_t head_v, int32_t ssm_dtype, size_t *ssm_bytes,
                      size_t *conv_bytes) {
  if (layers <= 0 || slots <= 0 || heads <= 0 || head_k <= 0 || head_v <= 0) return 4;
  if (ssm_dtype != ORACLE_SSM_F32 && ssm_dtype != ORACLE_SSM_BF16) return 4;
  size_t es = ssm_dtype == ORACLE_SSM_F32 ? 4 : 2;
  size_t C = (size_t)heads * (size_t)(2 * head_k + head_v);
  if (ssm_bytes) *ssm_bytes = (size_t)layers * slots * heads * head_v * head_k * es;
  if (conv_bytes) *conv_bytes = (size_t)layers * slots * CONV_ROWS * C * 2;
  return 0;
}

/* ------------------------------------------------------ the recurrence ---- */

/* One token of the gated delta rule for one head, row by row of S [V][K]:
 *   S' = S Diag(alpha);  u = S' k;  d = beta (v - u);  S = S' + d k^T;
 *   o = scale * S q  (o from the updated state). */
static void token_step(int K, int V, real *S, const real *q, const real *k,
                       const real *v, const real *alpha, real beta, real scale,
                       real *o) {
  for (int r = 0; r < V; ++r) {
    real *row = S + (size_t)r * K;
    for (int c = 0; c < K; ++c) row[c] = row[c] * alpha[c];
    real u = 0;
    for (int c = 0; c < K; ++c) u += row[c] * k[c];
    real d = beta * (v[r] - u);
    for (int c = 0; c < K; ++c) row[c] = row[c] + d * k[c];
    real acc = 0;
    for (int c = 0; c < K; ++c) acc += row[c] * q[c];
    o[r] = scale * acc;
  }
}

void oracle_recurrence_head(int32_t T, int32_t K, int32_t V, const double *q,
                            const double *k, const double *v, const double *alpha,
                            const double *beta, double scale, double *S, double *o) {
  real *s = malloc(sizeof(real) * (size_t)V * K);
  real *qq = malloc(sizeof(real) * K), *kk = malloc(sizeof(real) * K);
  real *aa = malloc(sizeof(real) * K), *vv = malloc(sizeof(real) * V);
  real *oo = malloc(sizeof(real) * V);
  for (size_t i = 0; i < (size_t)V * K; ++i) s[i] = (real)S[i];
  for (int t = 0; t < T; ++t) {
    for (int c = 0; c < K; ++c) {
      qq[c] = (real)q[(size_t)t * K + c];
      kk[c] = (real)k[(size_t)t * K + c];
      aa[c] = (real)alpha[(size_t)t * K + c];
    }
    for (int r = 0; r < V; ++r) vv[r] = (real)v[(size_t)t * V + r];
    token_step(K, V, s, qq, kk, vv, aa, (real)beta[t], (real)scale, oo);
    for (int r = 0; r < V; ++r) o[(size_t)t * V + r] = (double)oo[r];
  }
  for (size_t i = 0; i < (size_t)V * K; ++i) S[i] = (double)s[i];
  free(s); free(qq); free(kk); free(aa); free(vv); free(oo);
}

/* ------------------------------------------------ chunked WY form (f64) ---- */

/* Within a chunk of n tokens with entry state S0 and per-channel decays a_t:
 *   ratio(t,i)[c] = prod_{i<tau<=t} a_tau[c]   (i <= t; ratio(t,t) = 1)
 *   gam(t)[c]     = prod_{tau<=t} a_tau[c]
 *   A[t][i] = sum_c k_t[c] k_i[c] ratio(t,i)[c]          (i < t)
 *   T = (I + Diag(beta) A)^-1            (unit lower triangular)
 *   W = T Diag(beta) Kg,  Kg[t][c] = gam(t)[c] k_t[c]
 *   U = T Diag(beta) V
 *   D = U - W S0^T                        (rows d_t of the token updates)
 *   O[t] = scale (S0 (gam(t) . q_t) + sum_{i<=t} M[t][i] d_i),
 *          M[t][i] = sum_c q_t[c] k_i[c] ratio(t,i)[c]
 *   S_end = S0 Diag(gam(n-1)) + sum_i d_i (k_i . ratio(n-1,i))^T
 * This restates the same recurrence after unrolling it over the chunk; it is
 * checked against oracle_recurrence_head by the tests. */
void oracle_chunked_head_f64(int32_t T, int32_t K, int32_t V, int32_t chunk,
                             const double *q, const double *k, const double *v,
                             const double *alpha, const double *beta, double scale,
                             double *S, double *o) {
  int C = chunk;
  double *ratio = malloc(sizeof(double) * (size_t)C * C * K); /* [t][i][c] */
  double *gam = malloc(sizeof(double) * (size_t)C * K);
  double *A = malloc(sizeof(double) * (size_t)C * C);
  double *Tm = malloc(sizeof(double) * (size_t)C * C);
  double *W = malloc(sizeof(double) * (size_t)C * K);
  double *U = malloc(sizeof(double) * (size_t)C * V);
  double *D = malloc(sizeof(double) * (size_t)C * V);
  double *Snew = malloc(sizeof(double) * (size_t)V * K);
  for (int c0 = 0; c0 < T; c0 += C) {
    int n = T - c0 < C ? T - c0 : C;
    const double *qc = q + (size_t)c0 * K, *kc = k + (size_t)c0 * K;
    const double *vc = v + (size_t)c0 * V, *ac = alpha + (size_t)c0 * K;
    const double *bc = beta + c0;
    /* decay products */
    for (int t = 0; t < n; ++t) {
      for (int c = 0; c < K; ++c) {
        ratio[((size_t)t * C + t) * K + c] = 1.0;
        for (int i = 0; i < t; ++i)
          ratio[((size_t)t * C + i) * K + c] = ratio[((size_t)(t - 1) * C + i) * K + c] * ac[(size_t)t * K + c];
        gam[(size_t)t * K + c] = (t == 0 ? 1.0 : gam[(size_t)(t - 1) * K + c]) * ac[(size_t)t * K + c];
      }
    }
    /* A (strictly lower) */
    for (int t = 0; t < n; ++t)
      for (int i = 0; i < n; ++i) {
        double s = 0;
        if (i < t)
          for (int c = 0; c < K; ++c)
            s += kc[(size_t)t * K + c] * kc[(size_t)i * K + c] * ratio[((size_t)t * C + i) * K + c];
        A[(size_t)t * C + i] = s;
      }
    /* T = (I + Diag(beta) A)^-1 by forward substitution on each column of I */
    for (int col = 0; col < n; ++col)
      for (int t = 0; t < n; ++t) {
        double s = (t == col) ? 1.0 : 0.0;
        for (int i = 0; i < t; ++i) s -= bc[t] * A[(size_t)t * C + i] * Tm[(size_t)i * C + col];
        Tm[(size_t)t * C + col] = s;
      }
    /* W, U */
    for (int t = 0; t < n; ++t) {
      for (int c = 0; c < K; ++c) {
        double s = 0;
        for (int i = 0; i < n; ++i) s += Tm[(size_t)t * C + i] * bc[i] * gam[(size_t)i * K + c] * kc[(size_t)i * K + c];
        W[(size_t)t * K + c] = s;
      }
      for (int r = 0; r < V; ++r) {
        double s = 0;
        for (int i = 0; i < n; ++i) s += Tm[(size_t)t * C + i] * bc[i] * vc[(size_t)i * V + r];
        U[(size_t)t * V + r] = s;
      }
    }
    /* D = U - W S0^T */
    for (int t = 0; t < n; ++t)
      for (int r = 0; r < V; ++r) {
        double s = 0;
        for (int c = 0; c < K; ++c) s += W[(size_t)t * K + c] * S[(size_t)r * K + c];
        D[(size_t)t * V + r] = U[(size_t)t * V + r] - s;
      }
    /* outputs */
    for (int t = 0; t < n; ++t)
      for (int r = 0; r < V; ++r) {
        double inter = 0;
        for (int c = 0; c < K; ++c) inter += S[(size_t)r * K + c] * gam[(size_t)t * K + c] * qc[(size_t)t * K + c];
        double intra = 0;
        for (int i = 0; i <= t; ++i) {
          double m = 0;
          for (int c = 0; c < K; ++c) m += qc[(size_t)t * K + c] * kc[(size_t)i * K + c] * ratio[((size_t)t * C + i) * K + c];
          intra += m * D[(size_t)i * V + r];
        }
        o[(size_t)(c0 + t) * V + r] = scale * (inter + intra);
      }
    /* state at chunk end */
    for (int r = 0; r < V; ++r)
      for (int c = 0; c < K; ++c) {
        double s = S[(size_t)r * K + c] * gam[(size_t)(n - 1) * K + c];
        for (int i = 0; i < n; ++i)
          s += D[(size_t)i * V + r] * kc[(size_t)i * K + c] * ratio[((size_t)(n - 1) * C + i) * K + c];
        Snew[(size_t)r * K + c] = s;
      }
    memcpy(S, Snew, sizeof(double) * (size_t)V * K);
  }
  free(ratio); free(gam); free(A); free(Tm); free(W); free(U); free(D); free(Snew);
}

/* ---------------------------------------------- one (request, head) unit ---- */

/* Where a folded token sends a snapshot. */
typedef struct {
  int mode;                 /* 0 none, 1 prefill boundaries, 2 decode interval */
  int32_t interval;
  int32_t start_len;        /* prefill: tokens already folded before the call */
  int32_t seq_len_after;    /* decode */
  int32_t track[2];
  int32_t next;
} snap_rule;

typedef struct {
  const oracle_pool *pool;
  int layer;
  int K, V, H;
  size_t C;
  const uint16_t *conv_w;
  real scale;
  uint32_t flags;
} unit_ctx;

/* Store the head's state and conv channels into a slot of the pool. */
static void store_head(const unit_ctx *u, int slot, int h, const real *S, real R[][CONV_ROWS],
                       const size_t *chan, int nchan) {
  unsigned char *blk = ssm_block(u->pool, u->layer, slot);
  size_t base = (size_t)h * u->V * u->K;
  for (size_t i = 0; i < (size_t)u->V * u->K; ++i) store_ssm(u->pool, blk, base + i, S[i]);
  uint16_t *cb = conv_block(u->pool, u->layer, slot);
  for (int j = 0; j < CONV_ROWS; ++j)
    for (int i = 0; i < nchan; ++i) cb[(size_t)j * u->C + chan[i]] = oracle_bf16_round((double)R[i][j]);
}

/* One token of head h: causal conv over [R0, R1, R2, x_t] (tap 3 is the current
 * token) with the rows then shifted to [R1, R2, x_t], optional SiLU, key (and
 * query) normalisation, then the recurrence.  y holds the 2K+V conv outputs; raw
 * (K+V values, may be NULL) receives k and v as they leave the conv, before the
 * key is normalised. */
static void step_token(const unit_ctx *u, const size_t *chan, int nchan, real *S,
                       real (*R)[CONV_ROWS], const uint16_t *xt, const float *alpha,
                       int alpha_mode, real beta, real *y, real *a, real *o, real *raw) {
  const int K = u->K, V = u->V;
  for (int i = 0; i < nchan; ++i) {
    const uint16_t *w = u->conv_w + chan[i] * CONV_TAPS;
    real xi = widen(xt[chan[i]]);
    real acc = 0;
    acc += widen(w[0]) * R[i][0];
    acc += widen(w[1]) * R[i][1];
    acc += widen(w[2]) * R[i][2];
    acc += widen(w[3]) * xi;
    if (u->flags & ORACLE_CONV_SILU) acc = acc / (1 + exp(-acc));
    y[i] = acc;
    R[i][0] = R[i][1];
    R[i][1] = R[i][2];
    R[i][2] = xi;
  }
  real *q = y, *k = y + K, *v = y + 2 * K;
  if (raw)
    for (int i = 0; i < K + V; ++i) raw[i] = y[K + i];
  if (u->flags & ORACLE_L2NORM_K) {
    real ss = 0;
    for (int c = 0; c < K; ++c) ss += k[c] * k[c];
    real inv = 1 / sqrt(ss + (real)L2_EPS);
    for (int c = 0; c < K; ++c) k[c] = k[c] * inv;
  }
  if (u->flags & ORACLE_L2NORM_Q) {
    real ss = 0;
    for (int c = 0; c < K; ++c) ss += q[c] * q[c];
    real inv = 1 / sqrt(ss + (real)L2_EPS);
    for (int c = 0; c < K; ++c) q[c] = q[c] * inv;
  }
  /* alpha points at this (token, head): one value or K channel values */
  for (int c = 0; c < K; ++c) a[c] = alpha_mode == ORACLE_ALPHA_PER_CHANNEL ? (real)alpha[c] : (real)alpha[0];
  token_step(K, V, S, q, k, v, a, beta, u->scale, o);
}

/* The head's channels of x / conv rows: q, then k, then v. */
static size_t *head_channels(const unit_ctx *u, int h) {
  const int K = u->K, V = u->V, H = u->H;
  size_t *chan = malloc(sizeof(size_t) * (2 * K + V));
  for (int i = 0; i < K; ++i) chan[i] = (size_t)h * K + i;                    /* q */
  for (int i = 0; i < K; ++i) chan[K + i] = (size_t)H * K + (size_t)h * K + i; /* k */
  for (int i = 0; i < V; ++i) chan[2 * K + i] = (size_t)2 * H * K + (size_t)h * V + i; /* v */
  return chan;
}

/* Fold n tokens (rows x[0..n)) of one request into head h. Returns error bits. */
static int fold_head(const unit_ctx *u, int h, int live_slot, int warm, int32_t n,
                     const uint16_t *x, const float *alpha, int alpha_mode,
                     const float *beta, uint16_t *out, double *out_exact,
                     double *state_exact, snap_rule rule) {
  const int K = u->K, V = u->V, H = u->H;
  const int nchan = 2 * K + V;
  int err = 0;
  size_t *chan = head_channels(u, h);

  real *S = malloc(sizeof(real) * (size_t)V * K);
  real (*R)[CONV_ROWS] = malloc(sizeof(real) * CONV_ROWS * nchan);
  real *y = malloc(sizeof(real) * nchan);
  real *a = malloc(sizeof(real) * K);
  real *o = malloc(sizeof(real) * V);

  if (warm) {
    const unsigned char *blk = ssm_block(u->pool, u->layer, live_slot);
    size_t base = (size_t)h * V * K;
    for (size_t i = 0; i < (size_t)V * K; ++i) S[i] = load_ssm(u->pool, blk, base + i);
    const uint16_t *cb = conv_block(u->pool, u->layer, live_slot);
    for (int i = 0; i < nchan; ++i)
      for (int j = 0; j < CONV_ROWS; ++j) R[i][j] = widen(cb[(size_t)j * u->C + chan[i]]);
  } else {
    for (size_t i = 0; i < (size_t)V * K; ++i) S[i] = 0;
    for (int i = 0; i < nchan; ++i)
      for (int j = 0; j < CONV_ROWS; ++j) R[i][j] = 0;
  }

  int boundaries = 0;
  for (int32_t t = 0; t < n; ++t) {
    const float *at = alpha + ((size_t)t * H + h) * (alpha_mode == ORACLE_ALPHA_PER_CHANNEL ? K : 1);
    step_token(u, chan, nchan, S, R, x + (size_t)t * u->C, at, alpha_mode,
               (real)beta[(size_t)t * H + h], y, a, o, NULL);
    for (int r = 0; r < V; ++r) {
      size_t oi = ((size_t)t * H + h) * V + r;
      out[oi] = oracle_bf16_round((double)o[r]);
      if (out_exact) out_exact[oi] = (double)o[r];
    }
    /* snapshot after this token? */
    int dst = 0, take = 0;
    if (rule.mode == 1) {
      int64_t len = (int64_t)rule.start_len + t + 1;
      if (len % rule.interval == 0) {
        dst = rule.track[(rule.next + boundaries) & 1];
        ++boundaries;
        take = 1;
      }
    } else if (rule.mode == 2) {
      if (rule.seq_len_after % rule.interval == 0) {
        dst = rule.track[rule.next & 1];
        take = 1;
      }
    }
    if (take && dst > 0) {
      if (dst >= u->pool->slots) err |= 2;
      else store_head(u, dst, h, S, R, chan, nchan);
    }
  }
  store_head(u, live_slot, h, S, R, chan, nchan);
  if (state_exact)
    for (size_t i = 0; i < (size_t)V * K; ++i) state_exact[(size_t)h * V * K + i] = (double)S[i];
  free(chan); free(S); free(R); free(y); free(a); free(o);
  return err;
}

static int pool_ok(const oracle_pool *p, int layer) {
  return p && p->ssm && p->conv && p->layers > 0 && p->slots > 0 && p->heads > 0 &&
         p->head_k > 0 && p->head_v > 0 && layer >= 0 && layer < p->layers &&
         (p->ssm_dtype == ORACLE_SSM_F32 || p->ssm_dtype == ORACLE_SSM_BF16);
}

int oracle_prefill(const oracle_pool *pool, int32_t layer, int32_t batch,
                   const int32_t *cu_seqlens, const int32_t *slot_table,
                   const int32_t *has_initial_state, const int32_t *start_len,
                   const uint16_t *x, const uint16_t *conv_w, const float *alpha,
                   int32_t alpha_mode, const float *beta, float scale, uint32_t flags,
                   uint16_t *out, int32_t snap_interval, const int32_t *track_slots,
                   const int32_t *next_track_idx, double *out_exact, double *state_exact) {
  if (!pool_ok(pool, layer) || batch < 0 || snap_interval < 0) return 4;
  unit_ctx u = {pool, layer, pool->head_k, pool->head_v, pool->heads, conv_channels(pool),
                conv_w, (real)scale, flags};
  const int H = pool->heads;
  int err = 0;
#pragma omp parallel for collapse(2) reduction(| : err) schedule(dynamic)
  for (int b = 0; b < batch; ++b) {
    for (int h = 0; h < H; ++h) {
      int32_t t0 = cu_seqlens[b], n = cu_seqlens[b + 1] - cu_seqlens[b];
      int slot = slot_table[b];
      double *se = state_exact ? state_exact + (size_t)b * H * u.V * u.K : NULL;
      if (slot <= 0 || slot >= pool->slots) {
        if (slot >= pool->slots) err |= 1;
        for (int32_t t = 0; t < n; ++t)
          for (int r = 0; r < u.V; ++r) {
            size_t oi = ((size_t)(t0 + t) * H + h) * u.V + r;
            out[oi] = 0;
            if (out_exact) out_exact[oi] = 0;
          }
        continue;
      }
      snap_rule rule = {0};
      if (snap_interval > 0 && track_slots) {
        rule.mode = 1;
        rule.interval = snap_interval;
        rule.start_len = start_len ? start_len[b] : 0;
        rule.track[0] = track_slots[2 * b];
        rule.track[1] = track_slots[2 * b + 1];
        rule.next = next_track_idx ? next_track_idx[b] : 0;
      }
      size_t aoff = (size_t)t0 * H * (alpha_mode == ORACLE_ALPHA_PER_CHANNEL ? u.K : 1);
      err |= fold_head(&u, h, slot, has_initial_state ? has_initial_state[b] != 0 : 0, n,
                       x + (size_t)t0 * u.C, alpha + aoff, alpha_mode, beta + (size_t)t0 * H,
                       out + (size_t)t0 * H * u.V,
                       out_exact ? out_exact + (size_t)t0 * H * u.V : NULL, se, rule);
    }
  }
  return err;
}

int oracle_decode_step(const oracle_pool *pool, int32_t layer, int32_t batch,
                       const int32_t *slot_table, const uint16_t *x,
                       const uint16_t *conv_w, const float *alpha, int32_t alpha_mode,
                       const float *beta, float scale, uint32_t flags, uint16_t *out,
                       const int32_t *seq_len_after, int32_t track_interval,
                       const int32_t *track_slots, const int32_t *next_track_idx,
                       double *out_exact, double *state_exact) {
  if (!pool_ok(pool, layer) || batch < 0 || track_interval < 0) return 4;
  unit_ctx u = {pool, layer, pool->head_k, pool->head_v, pool->heads, conv_channels(pool),
                conv_w, (real)scale, flags};
  const int H = pool->heads;
  int err = 0;
#pragma omp parallel for collapse(2) reduction(| : err) schedule(dynamic)
  for (int b = 0; b < batch; ++b) {
    for (int h = 0; h < H; ++h) {
      int slot = slot_table[b];
      double *se = state_exact ? state_exact + (size_t)b * H * u.V * u.K : NULL;
      if (slot <= 0 || slot >= pool->slots) {
        if (slot >= pool->slots) err |= 1;
        for (int r = 0; r < u.V; ++r) {
          size_t oi = ((size_t)b * H + h) * u.V + r;
          out[oi] = 0;
          if (out_exact) out_exact[oi] = 0;
        }
        continue;
      }
      snap_rule rule = {0};
      if (track_interval > 0 && track_slots) {
        rule.mode = 2;
        rule.interval = track_interval;
        rule.seq_len_after = seq_len_after[b];
        rule.track[0] = track_slots[2 * b];
        rule.track[1] = track_slots[2 * b + 1];
        rule.next = next_track_idx ? next_track_idx[b] : 0;
      }
      size_t aoff = (size_t)b * H * (alpha_mode == ORACLE_ALPHA_PER_CHANNEL ? u.K : 1);
      err |= fold_head(&u, h, slot, 1, 1, x + (size_t)b * u.C, alpha + aoff, alpha_mode,
                       beta + (size_t)b * H, out + (size_t)b * H * u.V,
                       out_exact ? out_exact + (size_t)b * H * u.V : NULL, se, rule);
    }
  }
  return err;
}

/* ------------------------------------------------- speculative verify ---- */

/* A draft tree is valid when every parent is -1 (the live state) or an earlier
 * node, so that visiting nodes in index order visits parents first. */
static int tree_ok(const int32_t *parent, int32_t nodes) {
  for (int32_t n = 0; n < nodes; ++n)
    if (parent[n] < -1 || parent[n] >= n) return 0;
  return 1;
}

static unsigned char *node_ssm_block(const oracle_pool *p, void *node_ssm, int32_t nodes, int b, int n) {
  return (unsigned char *)node_ssm + ((size_t)b * nodes + n) * ssm_block_elems(p) * ssm_esize(p);
}
static uint16_t *node_conv_block(const oracle_pool *p, uint16_t *node_conv, int32_t nodes, int b, int n) {
  return node_conv + ((size_t)b * nodes + n) * CONV_ROWS * conv_channels(p);
}

/* Verify a draft tree for one layer without updating the live slot (page
 * "SGLang之MambaRadixCache机制", section 8.3: disable_state_update, one result per
 * draft position into an intermediate buffer; section 9.6: retrieve_parent_token,
 * parent before child, parent -1 reads the main state).  Node n of request b
 * starts from its parent's stored state and conv rows (the live slot's for -1),
 * takes token x[b][n], and stores its state (rounded to the pool dtype) and conv
 * rows into node_ssm[b][n], node_conv[b][n]; out[b][n] gets o.  Shapes: parent
 * [B][T], x [B][T][C], alpha [B][T][H] or [B][T][H][K], beta [B][T][H], out
 * [B][T][H][V], node_ssm [B][T][H][V][K] (pool ssm dtype), node_conv [B][T][3][C].
 * A request with an invalid tree or live slot gets zero outputs and no node
 * writes; error bits 8 (tree) and 1 (live slot >= slots). */
int oracle_verify_tree(const oracle_pool *pool, int32_t layer, int32_t batch, int32_t nodes,
                       const int32_t *slot_table, const int32_t *parent, const uint16_t *x,
                       const uint16_t *conv_w, const float *alpha, int32_t alpha_mode,
                       const float *beta, float scale, uint32_t flags, uint16_t *out,
                       void *node_ssm, uint16_t *node_conv, double *out_exact) {
  if (!pool_ok(pool, layer) || batch < 0 || nodes < 1) return 4;
  unit_ctx u = {pool, layer, pool->head_k, pool->head_v, pool->heads, conv_channels(pool),
                conv_w, (real)scale, flags};
  const int H = pool->heads, K = u.K, V = u.V, nchan = 2 * K + V;
  const size_t aw = alpha_mode == ORACLE_ALPHA_PER_CHANNEL ? (size_t)K : 1;
  int err = 0;
#pragma omp parallel for collapse(2) reduction(| : err) schedule(dynamic)
  for (int b = 0; b < batch; ++b) {
    for (int h = 0; h < H; ++h) {
      const int32_t *par = parent + (size_t)b * nodes;
      const int slot = slot_table[b];
      const int ok_tree = tree_ok(par, nodes);
      if (slot <= 0 || slot >= pool->slots || !ok_tree) {
        if (slot >= pool->slots) err |= 1;
        if (!ok_tree) err |= 8;
        for (int32_t n = 0; n < nodes; ++n)
          for (int r = 0; r < V; ++r) {
            size_t oi = (((size_t)b * nodes + n) * H + h) * V + r;
            out[oi] = 0;
            if (out_exact) out_exact[oi] = 0;
          }
        continue;
      }
      size_t *chan = head_channels(&u, h);
      real *S = malloc(sizeof(real) * (size_t)V * K);
      real (*R)[CONV_ROWS] = malloc(sizeof(real) * CONV_ROWS * nchan);
      real *y = malloc(sizeof(real) * nchan);
      real *a = malloc(sizeof(real) * K);
      real *o = malloc(sizeof(real) * V);
      const size_t hb = (size_t)h * V * K;
      for (int32_t n = 0; n < nodes; ++n) {
        const int p = par[n];
        /* the parent's state and conv rows: the live slot or an earlier node */
        const unsigned char *sblk = p < 0 ? ssm_block(pool, layer, slot) : node_ssm_block(pool, node_ssm, nodes, b, p);
        const uint16_t *cblk = p < 0 ? conv_block(pool, layer, slot) : node_conv_block(pool, node_conv, nodes, b, p);
        for (size_t i = 0; i < (size_t)V * K; ++i) S[i] = load_ssm(pool, sblk, hb + i);
        for (int i = 0; i < nchan; ++i)
          for (int j = 0; j < CONV_ROWS; ++j) R[i][j] = widen(cblk[(size_t)j * u.C + chan[i]]);
        const size_t tok = (size_t)b * nodes + n;
        step_token(&u, chan, nchan, S, R, x + tok * u.C, alpha + (tok * H + h) * aw, alpha_mode,
                   (real)beta[tok * H + h], y, a, o, NULL);
        for (int r = 0; r < V; ++r) {
          size_t oi = (tok * H + h) * V + r;
          out[oi] = oracle_bf16_round((double)o[r]);
          if (out_exact) out_exact[oi] = (double)o[r];
        }
        unsigned char *dblk = node_ssm_block(pool, node_ssm, nodes, b, n);
        for (size_t i = 0; i < (size_t)V * K; ++i) store_ssm(pool, dblk, hb + i, S[i]);
        uint16_t *dc = node_conv_block(pool, node_conv, nodes, b, n);
        for (int j = 0; j < CONV_ROWS; ++j)
          for (int i = 0; i < nchan; ++i) dc[(size_t)j * u.C + chan[i]] = oracle_bf16_round((double)R[i][j]);
      }
      free(chan); free(S); free(R); free(y); free(a); free(o);
    }
  }
  return err;
}

/* Copy a node's whole block (every head's state and all conv channels) into a
 * slot of the layer. */
static void copy_node(const oracle_pool *p, int layer, const void *node_ssm, const uint16_t *node_conv,
                      int32_t nodes, int b, int n, int dst) {
  memcpy(ssm_block(p, layer, dst), node_ssm_block(p, (void *)node_ssm, nodes, b, n),
         ssm_block_elems(p) * ssm_esize(p));
  memcpy(conv_block(p, layer, dst), node_conv_block(p, (uint16_t *)node_conv, nodes, b, n),
         (size_t)CONV_ROWS * conv_channels(p) * 2);
}

/* Commit the accepted step (page "SGLang之MambaRadixCache机制", section 8.4:
 * main_state[layer, slot] = buffer[layer, req, accepted_step]; section 8.6: when
 * the accepted tokens cross the track interval, the ping-pong track buffer is
 * updated too).  accepted[b] is the last accepted node (-1: nothing accepted,
 * nothing written).  Its depth d (1 + its parent's depth, 0 for the live state)
 * is the number of tokens it folds.  For each length L = seq_len_before[b] + i,
 * 0 < i <= d, with L % track_interval == 0 (track_interval > 0), the node at
 * depth i on the accepted path is copied to track_slots[2b + ((next_track_idx[b]
 * + j) & 1)] for the j-th such length, as the prefill snapshots do.  Error bits:
 * 1 live slot >= slots, 2 track slot >= slots, 8 invalid tree or accepted node. */
int oracle_accept_scatter(const oracle_pool *pool, int32_t layer, int32_t batch, int32_t nodes,
                          const int32_t *slot_table, const int32_t *parent, const int32_t *accepted,
                          const int32_t *seq_len_before, int32_t track_interval,
                          const int32_t *track_slots, const int32_t *next_track_idx,
                          const void *node_ssm, const uint16_t *node_conv) {
  if (!pool_ok(pool, layer) || batch < 0 || nodes < 1 || track_interval < 0) return 4;
  int err = 0;
  for (int b = 0; b < batch; ++b) {
    const int32_t *par = parent + (size_t)b * nodes;
    const int acc = accepted[b], slot = slot_table[b];
    if (acc == -1) continue;
    if (acc < -1 || acc >= nodes || !tree_ok(par, nodes)) {
      err |= 8;
      continue;
    }
    if (slot <= 0 || slot >= pool->slots) {
      if (slot >= pool->slots) err |= 1;
      continue;
    }
    /* the accepted path, root first */
    int depth = 0;
    for (int n = acc; n >= 0; n = par[n]) ++depth;
    int *path = malloc(sizeof(int) * (depth + 1));
    { int i = depth; for (int n = acc; n >= 0; n = par[n]) path[--i] = n; }
    if (track_interval > 0 && track_slots) {
      int j = 0;
      for (int i = 1; i <= depth; ++i) {
        int64_t len = (int64_t)seq_len_before[b] + i;
        if (len % track_interval != 0) continue;
        int dst = track_slots[2 * b + (((next_track_idx ? next_track_idx[b] : 0) + j) & 1)];
        ++j;
        if (dst <= 0) continue;
        if (dst >= pool->slots) { err |= 2; continue; }
        copy_node(pool, layer, node_ssm, node_conv, nodes, b, path[i - 1], dst);
      }
    }
    copy_node(pool, layer, node_ssm, node_conv, nodes, b, acc, slot);
    free(path);
  }
  return err;
}

/* --------------------------------------------------------- ReplaySSM ring ---- */

/* Element offsets into the ring arrays of (layer, slot, head, position). */
static size_t ring_row(const oracle_pool *p, const oracle_ring *r, int layer, int slot, int h, int t) {
  return (((size_t)layer * p->slots + slot) * p->heads + h) * r->positions + t;
}

int oracle_ring_bytes(const oracle_pool *pool, int32_t positions, int32_t alpha_mode,
                      size_t bytes[5]) {
  if (!pool || positions <= 0 || (alpha_mode != ORACLE_ALPHA_PER_HEAD && alpha_mode != ORACLE_ALPHA_PER_CHANNEL))
    return 4;
  const size_t rows = (size_t)pool->layers * pool->slots * pool->heads * positions;
  bytes[0] = rows * pool->head_k * 2;                                         /* rawk */
  bytes[1] = rows * pool->head_v * 2;                                         /* rawv */
  bytes[2] = rows * (alpha_mode == ORACLE_ALPHA_PER_CHANNEL ? pool->head_k : 1) * 4;  /* g */
  bytes[3] = rows * 4;                                                        /* beta */
  bytes[4] = (size_t)pool->layers * pool->slots * positions * conv_channels(pool) * 2;  /* xrow */
  return 0;
}

static int ring_ok(const oracle_pool *p, const oracle_ring *r, int32_t alpha_mode) {
  return r && r->positions > 0 && r->alpha_mode == alpha_mode && r->rawk && r->rawv && r->g &&
         r->beta && r->xrow && p;
}

/* Speculative verify of a draft chain with a ReplaySSM ring (page
 * "企业官网建设流程全解析", Kimi K3 notes, section "ReplaySSM": the verify still
 * produces every position's output but keeps no per-position state; it records
 * the inputs that regenerate the state: k before L2 normalisation and v before
 * the delta correction, both as they leave the conv, in bf16, the decay g and
 * beta in fp32).  Draft token t of request b follows token t-1 (t = 0 follows
 * the live slot).  out [B][D][H][V] equals D consecutive decode steps; the live
 * slot is only read.  Ring position t of the request's slot receives rawk, rawv,
 * g = alpha, beta, and the conv input row x_t (the conv state must advance with
 * the accepted tokens; post-conv values cannot give it back). */
int oracle_replay_verify(const oracle_pool *pool, const oracle_ring *ring, int32_t layer,
                         int32_t batch, int32_t draft, const int32_t *slot_table,
                         const uint16_t *x, const uint16_t *conv_w, const float *alpha,
                         int32_t alpha_mode, const float *beta, float scale, uint32_t flags,
                         uint16_t *out, double *out_exact) {
  if (!pool_ok(pool, layer) || batch < 0 || draft < 1 || !ring_ok(pool, ring, alpha_mode) ||
      draft > ring->positions)
    return 4;
  unit_ctx u = {pool, layer, pool->head_k, pool->head_v, pool->heads, conv_channels(pool),
                conv_w, (real)scale, flags};
  const int H = pool->heads, K = u.K, V = u.V, nchan = 2 * K + V;
  const size_t aw = alpha_mode == ORACLE_ALPHA_PER_CHANNEL ? (size_t)K : 1;
  int err = 0;
#pragma omp parallel for collapse(2) reduction(| : err) schedule(dynamic)
  for (int b = 0; b < batch; ++b) {
    for (int h = 0; h < H; ++h) {
      const int slot = slot_table[b];
      if (slot <= 0 || slot >= pool->slots) {
        if (slot >= pool->slots) err |= 1;
        for (int t = 0; t < draft; ++t)
          for (int r = 0; r < V; ++r) {
            size_t oi = (((size_t)b * draft + t) * H + h) * V + r;
            out[oi] = 0;
            if (out_exact) out_exact[oi] = 0;
          }
        continue;
      }
      size_t *chan = head_channels(&u, h);
      real *S = malloc(sizeof(real) * (size_t)V * K);
      real (*R)[CONV_ROWS] = malloc(sizeof(real) * CONV_ROWS * nchan);
      real *y = malloc(sizeof(real) * nchan), *a = malloc(sizeof(real) * K);
      real *o = malloc(sizeof(real) * V), *raw = malloc(sizeof(real) * (K + V));
      const unsigned char *sblk = ssm_block(pool, layer, slot);
      const uint16_t *cblk = conv_block(pool, layer, slot);
      for (size_t i = 0; i < (size_t)V * K; ++i) S[i] = load_ssm(pool, sblk, (size_t)h * V * K + i);
      for (int i = 0; i < nchan; ++i)
        for (int j = 0; j < CONV_ROWS; ++j) R[i][j] = widen(cblk[(size_t)j * u.C + chan[i]]);
      for (int t = 0; t < draft; ++t) {
        const size_t tok = (size_t)b * draft + t;
        const uint16_t *xt = x + tok * u.C;
        step_token(&u, chan, nchan, S, R, xt, alpha + (tok * H + h) * aw, alpha_mode,
                   (real)beta[tok * H + h], y, a, o, raw);
        for (int r = 0; r < V; ++r) {
          size_t oi = (tok * H + h) * V + r;
          out[oi] = oracle_bf16_round((double)o[r]);
          if (out_exact) out_exact[oi] = (double)o[r];
        }
        const size_t row = ring_row(pool, ring, layer, slot, h, t);
        for (int c = 0; c < K; ++c) ring->rawk[row * K + c] = oracle_bf16_round((double)raw[c]);
        for (int c = 0; c < V; ++c) ring->rawv[row * V + c] = oracle_bf16_round((double)raw[K + c]);
        for (size_t c = 0; c < aw; ++c) ring->g[row * aw + c] = alpha[(tok * H + h) * aw + c];
        ring->beta[row] = beta[tok * H + h];
        uint16_t *xr = ring->xrow + (((size_t)layer * pool->slots + slot) * ring->positions + t) * u.C;
        for (int i = 0; i < nchan; ++i) xr[chan[i]] = xt[chan[i]];
      }
      free(chan); free(S); free(R); free(y); free(a); free(o); free(raw);
    }
  }
  return err;
}

/* The exact-fold commit (same page and section: after acceptance only the
 * accepted prefix is replayed, in recurrent order, and the result is written
 * back to the slot; page "SGLang之MambaRadixCache机制解析", section 9.10: the
 * 256-boundary check happens during the replay).  accepted[b] tokens (0 .. ring
 * positions) are folded from ring positions 0 .. accepted-1 of the request's
 * slot: k = rawk normalised (flag), v = rawv, S' = S Diag(g), d = beta (v - S'k),
 * S = S' + d k^T, conv rows shifted through the x rows.  For every i in
 * [1, accepted] with (seq_len_before + i) % track_interval == 0 the state and
 * conv rows after token i go to track_slots[2b + ((next_track_idx[b] + j) & 1)]
 * for the j-th such i.  The state is rounded to the pool dtype only where it is
 * stored.  Error bits: 1 bad live slot, 2 bad track slot, 8 accepted outside
 * [0, positions]. */
int oracle_replay_commit(const oracle_pool *pool, const oracle_ring *ring, int32_t layer,
                         int32_t batch, const int32_t *slot_table, const int32_t *accepted,
                         int32_t alpha_mode, uint32_t flags, const int32_t *seq_len_before,
                         int32_t track_interval, const int32_t *track_slots,
                         const int32_t *next_track_idx) {
  if (!pool_ok(pool, layer) || batch < 0 || !ring_ok(pool, ring, alpha_mode) || track_interval < 0)
    return 4;
  unit_ctx u = {pool, layer, pool->head_k, pool->head_v, pool->heads, conv_channels(pool),
                NULL, 1, flags};
  const int H = pool->heads, K = u.K, V = u.V, nchan = 2 * K + V;
  const size_t aw = alpha_mode == ORACLE_ALPHA_PER_CHANNEL ? (size_t)K : 1;
  int err = 0;
#pragma omp parallel for collapse(2) reduction(| : err) schedule(dynamic)
  for (int b = 0; b < batch; ++b) {
    for (int h = 0; h < H; ++h) {
      const int slot = slot_table[b], n = accepted[b];
      if (n < 0 || n > ring->positions) {
        err |= 8;
        continue;
      }
      if (slot <= 0 || slot >= pool->slots) {
        if (slot >= pool->slots) err |= 1;
        continue;
      }
      if (n == 0) continue;
      size_t *chan = head_channels(&u, h);
      real *S = malloc(sizeof(real) * (size_t)V * K);
      real (*R)[CONV_ROWS] = malloc(sizeof(real) * CONV_ROWS * nchan);
      real *k = malloc(sizeof(real) * K), *v = malloc(sizeof(real) * V);
      real *a = malloc(sizeof(real) * K), *q = calloc(K, sizeof(real)), *o = malloc(sizeof(real) * V);
      const unsigned char *sblk = ssm_block(pool, layer, slot);
      const uint16_t *cblk = conv_block(pool, layer, slot);
      for (size_t i = 0; i < (size_t)V * K; ++i) S[i] = load_ssm(pool, sblk, (size_t)h * V * K + i);
      for (int i = 0; i < nchan; ++i)
        for (int j = 0; j < CONV_ROWS; ++j) R[i][j] = widen(cblk[(size_t)j * u.C + chan[i]]);
      int crossings = 0;
      for (int t = 0; t < n; ++t) {
        const size_t row = ring_row(pool, ring, layer, slot, h, t);
        for (int c = 0; c < K; ++c) k[c] = widen(ring->rawk[row * K + c]);
        for (int c = 0; c < V; ++c) v[c] = widen(ring->rawv[row * V + c]);
        if (flags & ORACLE_L2NORM_K) {
          real ss = 0;
          for (int c = 0; c < K; ++c) ss += k[c] * k[c];
          real inv = 1 / sqrt(ss + (real)L2_EPS);
          for (int c = 0; c < K; ++c) k[c] = k[c] * inv;
        }
        for (int c = 0; c < K; ++c) a[c] = (real)ring->g[row * aw + (aw == 1 ? 0 : c)];
        token_step(K, V, S, q, k, v, a, (real)ring->beta[row], 0, o);   /* output unused */
        const uint16_t *xr = ring->xrow + (((size_t)layer * pool->slots + slot) * ring->positions + t) * u.C;
        for (int i = 0; i < nchan; ++i) {
          R[i][0] = R[i][1];
          R[i][1] = R[i][2];
          R[i][2] = widen(xr[chan[i]]);
        }
        if (track_interval > 0 && track_slots &&
            ((int64_t)seq_len_before[b] + t + 1) % track_interval == 0) {
          const int dst = track_slots[2 * b + (((next_track_idx ? next_track_idx[b] : 0) + crossings) & 1)];
          ++crossings;
          if (dst >= pool->slots) err |= 2;
          else if (dst > 0) store_head(&u, dst, h, S, R, chan, nchan);
        }
      }
      store_head(&u, slot, h, S, R, chan, nchan);
      free(chan); free(S); free(R); free(k); free(v); free(a); free(q); free(o);
    }
  }
  return err;
}

/* ---------------------------------------------------------------- copies ---- */

static void copy_slot(const oracle_pool *p, int layer, int src, int dst) {
  size_t sb = ssm_block_elems(p) * ssm_esize(p);
  memmove(ssm_block(p, layer, dst), ssm_block(p, layer, src), sb);
  size_t cb = (size_t)CONV_ROWS * conv_channels(p) * 2;
  memmove(conv_block(p, layer, dst), conv_block(p, layer, src), cb);
}

int oracle_track_snapshot(const oracle_pool *pool, int32_t layer_begin, int32_t layer_end,
                          int32_t n, const int32_t *src_slots, const int32_t *dst_slots) {
  if (!pool || layer_begin < 0 || layer_end > pool->layers || layer_begin > layer_end || n < 0)
    return 4;
  int err = 0;
  for (int32_t i = 0; i < n; ++i) {
    int src = src_slots[i], dst = dst_slots[i];
    if (dst <= 0) continue;
    if (src <= 0 || src >= pool->slots || dst >= pool->slots) {
      err |= 2;
      continue;
    }
    if (src == dst) continue;
    for (int l = layer_begin; l < layer_end; ++l) copy_slot(pool, l, src, dst);
  }
  return err;
}

/* restore_linear_state_slots: for each op with a restore request, copy the
 * checkpoint slot into the live slot across all layers and report RESTORED (1);
 * a request whose source is missing or out of range reports COLD_START (0);
 * an op without a request leaves has_initial_state untouched. */
int oracle_restore_slots(const oracle_pool *pool, int32_t n_ops, const oracle_restore_op *ops,
                         int64_t *has_initial_state) {
  if (!pool || n_ops < 0) return 4;
  for (int32_t i = 0; i < n_ops; ++i) {
    const oracle_restore_op *op = &ops[i];
    if (!op->restore_requested) continue;
    int src = op->restore_src_slot_id, dst = op->linear_state_id;
    if (src < 1 || src >= pool->slots || dst < 1 || dst >= pool->slots) {
      has_initial_state[i] = 0;
      continue;
    }
    if (src != dst)
      for (int l = 0; l < pool->layers; ++l) copy_slot(pool, l, src, dst);
    has_initial_state[i] = 1;
  }
  return 0;
}
