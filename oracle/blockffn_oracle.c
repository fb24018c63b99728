/*
 * blockffn_oracle.c -- plain, slow CPU oracle of the BlockFFN layer (forward and backward).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It includes no HIP header and shares no code, table
 * or helper with the GPU library.
 *
 * What it computes (sources: the BlockFFN write-up on lsdiaocha.cn, §2 core
 * design and §4 acceleration kernel; the abstract of "BlockFFN: Towards
 * End-Side Acceleration-Friendly Mixture-of-Experts with Chunk-Level
 * Activation Sparsity", arXiv 2507.08771):
 *
 *   router   z_i = sum_k W_r[i][k] x_k + b_i
 *            a_i = max(z_i, 0)                      (ReLU; expert i active iff z_i > 0)
 *            g_i = s_i a_i / sqrt(mean_i(a_i^2) + eps)   (RMSNorm over the E outputs)
 *   expert   E_i(x) = W_out[i] Swish(W_in[i] x),  Swish(u) = u / (1 + e^-u)
 *   layer    y = sum over active i, ascending, of g_i E_i(x)
 *   chunk    U_c = union of the active sets of the L tokens of chunk c
 *   stats    token-level sparsity, chunk-level sparsity, experts-per-token
 *            histogram, consecutive-token expert reuse
 *   backward the gradients of a scalar loss with respect to x and every
 *            parameter, by the chain rule through the definitions above
 *            (the write-up §2 calls the ReLU + RMSNorm router fully
 *            differentiable; the abstract: differentiable, flexible routing)
 *
 * Every sum is accumulated in double, in the plain index order written
 * below, with no blocking or reordering.  Inputs are read in their stored
 * precision (IEEE binary32, or bfloat16 = the upper 16 bits of a binary32)
 * and widened here.  Every function is pinned by CPU tests against brute
 * force, closed forms, invariants and special cases that reduce to library
 * routines; none is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_MAX_HIST 129

typedef struct oracle_stats {
  int64_t n_tokens, n_chunks, n_experts, chunk_len;
  int64_t active_pairs; /* sum over tokens of |M_t| */
  int64_t union_sum;    /* sum over chunks of |U_c| */
  int64_t reuse_num;    /* sum over t >= 1 of |M_t and M_{t-1}| */
  int64_t reuse_den;    /* sum over t >= 1 of |M_{t-1}| */
  int64_t hist[ORACLE_MAX_HIST]; /* hist[k] = number of tokens with k active experts */
} oracle_stats_t;

/* Element idx of a stored array, widened to double. */
static double widen(const void *base, int64_t idx, int dtype) {
  if (dtype == ORACLE_F32) return (double)((const float *)base)[idx];
  uint32_t bits = ((uint32_t)((const uint16_t *)base)[idx]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static int mask_words(int E) { return (E + 63) / 64; }

static int mask_bit(const uint64_t *m, int i) { return (int)((m[i / 64] >> (i % 64)) & 1u); }

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * Router (write-up §2: ReLU then RMSNorm; abstract: "a router integrating ReLU
 * activation and RMSNorm").  For each token t writes the pre-activations
 * z[t][E], the gates g[t][E] and the activation pattern mask[t][W] (bit i of
 * word i/64 set iff z_i > 0).  The RMS is taken over all E router outputs,
 * inactive ones included.  rms_scale may be NULL (unit scale), b_router NULL
 * (no bias).
 */
int oracle_route(int32_t d, int32_t E, int32_t dtype, const void *x, int64_t T,
                 const void *w_router, const float *b_router, const float *rms_scale,
                 double eps, double *z_out, double *g_out, uint64_t *mask_out) {
  if (d <= 0 || E <= 0 || T < 0) return -1;
  const int W = mask_words(E);
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    double *z = z_out + t * E;
    double *g = g_out + t * E;
    uint64_t *m = mask_out + t * W;
    for (int w = 0; w < W; ++w) m[w] = 0;
    for (int i = 0; i < E; ++i) {
      double acc = 0.0;
      for (int k = 0; k < d; ++k)
        acc += widen(w_router, (int64_t)i * d + k, dtype) * widen(x, t * d + k, dtype);
      if (b_router) acc += (double)b_router[i];
      z[i] = acc;
      if (acc > 0.0) m[i / 64] |= (uint64_t)1 << (i % 64);
    }
    double ms = 0.0;
    for (int i = 0; i < E; ++i) {
      double a = z[i] > 0.0 ? z[i] : 0.0;
      ms += a * a;
    }
    ms /= (double)E;
    const double denom = sqrt(ms + eps);
    for (int i = 0; i < E; ++i) {
      double a = z[i] > 0.0 ? z[i] : 0.0;
      double s = rms_scale ? (double)rms_scale[i] : 1.0;
      g[i] = s * a / denom;
    }
  }
  return 0;
}

/*
 * Baseline routers for comparison (the MoE architecture blog on
 * intelliparadigm.com: §2.1 gives the Switch Transformer router as a
 * softmax over x W_r with TOP-K selection, K usually 2; §5.1 gives ReMoE as
 * G(x) = ReLU(x W_g) with the output divided by the sum of G).  Same z as
 * oracle_route (bias included); rms_scale and eps are not used.
 *   kind 1 (top-k softmax): p = softmax over all E of z (shifted by max z);
 *          the k largest z are selected, lower index first among equal z;
 *          g_i = p_i for the selected experts, 0 elsewhere; mask = selected
 *   kind 2 (ReLU, sum-normalised): a = max(z, 0), g_i = a_i / sum_j a_j
 *          (0 when no expert fires); mask bit i = [z_i > 0]
 */
int oracle_route_with(int32_t d, int32_t E, int32_t dtype, const void *x, int64_t T, const void *w_router,
                      const float *b_router, int32_t kind, int32_t top_k, double *z_out, double *g_out,
                      uint64_t *mask_out) {
  if (d <= 0 || E <= 0 || T < 0 || (kind != 1 && kind != 2) || (kind == 1 && (top_k < 1 || top_k > E)))
    return -1;
  const int W = mask_words(E);
  /* z exactly as the BlockFFN router computes it; its gates are overwritten below */
  int err = oracle_route(d, E, dtype, x, T, w_router, b_router, NULL, 0.0, z_out, g_out, mask_out);
  if (err) return err;
#pragma omp parallel
  {
    uint8_t *taken = (uint8_t *)malloc((size_t)E);
    if (!taken) {
#pragma omp atomic write
      err = -2;
    }
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      const double *z = z_out + t * E;
      double *g = g_out + t * E;
      uint64_t *m = mask_out + t * W;
      for (int w = 0; w < W; ++w) m[w] = 0;
      for (int i = 0; i < E; ++i) g[i] = 0.0;
      if (!taken) continue;
      if (kind == 1) {
        double zmax = z[0];
        for (int i = 1; i < E; ++i)
          if (z[i] > zmax) zmax = z[i];
        double sum = 0.0;
        for (int i = 0; i < E; ++i) sum += exp(z[i] - zmax);
        for (int i = 0; i < E; ++i) taken[i] = 0;
        for (int r = 0; r < top_k; ++r) {
          int best = -1;
          for (int i = 0; i < E; ++i)
            if (!taken[i] && (best < 0 || z[i] > z[best])) best = i;
          taken[best] = 1;
          g[best] = exp(z[best] - zmax) / sum;
          m[best / 64] |= (uint64_t)1 << (best % 64);
        }
      } else {
        double sum = 0.0;
        for (int i = 0; i < E; ++i) sum += z[i] > 0.0 ? z[i] : 0.0;
        for (int i = 0; i < E; ++i) {
          if (z[i] > 0.0) {
            g[i] = z[i] / sum;
            m[i / 64] |= (uint64_t)1 << (i % 64);
          }
        }
      }
    }
    free(taken);
  }
  return err;
}

/*
 * One expert on one token (write-up §2: a non-gated MLP with Swish):
 * u = W_in[i] x (d_e values), h = Swish(u), e = W_out[i] h (d values).
 * w_in_i points at W_in[i] ([d_e][d]) and w_out_i at W_out[i] ([d][d_e]);
 * x_off is the element offset of the token in x.
 */
static void expert_eval(int d, int de, int dtype, const void *x, int64_t x_off,
                        const void *w_in, int64_t w_in_off, const void *w_out, int64_t w_out_off,
                        double *h, double *e) {
  for (int j = 0; j < de; ++j) {
    double u = 0.0;
    for (int k = 0; k < d; ++k)
      u += widen(w_in, w_in_off + (int64_t)j * d + k, dtype) * widen(x, x_off + k, dtype);
    h[j] = u / (1.0 + exp(-u));
  }
  for (int k = 0; k < d; ++k) {
    double acc = 0.0;
    for (int j = 0; j < de; ++j) acc += widen(w_out, w_out_off + (int64_t)k * de + j, dtype) * h[j];
    e[k] = acc;
  }
}

/* Exported for the expert special-case pins: e[d] = E_i(x_t). */
int oracle_expert(int32_t d, int32_t de, int32_t dtype, const void *x, int64_t t,
                  const void *w_in, const void *w_out, int32_t i, double *e_out) {
  double *h = (double *)malloc(sizeof(double) * (size_t)de);
  if (!h) return -2;
  expert_eval(d, de, dtype, x, t * d, w_in, (int64_t)i * de * d, w_out, (int64_t)i * d * de, h, e_out);
  free(h);
  return 0;
}

/*
 * Per-token layer output: y_t = sum over i in M_t, ascending, of g[t][i] E_i(x_t).
 * Experts outside the pattern are skipped (their gate is exactly zero).
 */
int oracle_forward_tokens(int32_t d, int32_t E, int32_t de, int32_t dtype, const void *x, int64_t T,
                          const void *w_in, const void *w_out, const double *g,
                          const uint64_t *mask, double *y) {
  const int W = mask_words(E);
  int err = 0;
#pragma omp parallel
  {
    double *h = (double *)malloc(sizeof(double) * (size_t)de);
    double *e = (double *)malloc(sizeof(double) * (size_t)d);
    if (!h || !e) {
#pragma omp atomic write
      err = -2;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
      double *yt = y + t * d;
      for (int k = 0; k < d; ++k) yt[k] = 0.0;
      if (!h || !e) continue;
      for (int i = 0; i < E; ++i) {
        if (!mask_bit(mask + t * W, i)) continue;
        expert_eval(d, de, dtype, x, t * d, w_in, (int64_t)i * de * d, w_out, (int64_t)i * d * de, h, e);
        for (int k = 0; k < d; ++k) yt[k] += g[t * E + i] * e[k];
      }
    }
    free(h);
    free(e);
  }
  return err;
}

/*
 * Chunk evaluation (write-up §4): for every chunk, run every expert of the
 * chunk's union list on every token of the chunk and weight it by the token's
 * own gate, which masks out the pairs the token did not activate:
 * y_t = sum over s < count[c] of g[t][list[c][s]] E_{list[c][s]}(x_t).
 */
int oracle_forward_chunks(int32_t d, int32_t E, int32_t de, int32_t dtype, const void *x, int64_t T,
                          int32_t L, const void *w_in, const void *w_out, const double *g,
                          const int32_t *count, const int32_t *list, double *y) {
  if (L <= 0 || T % L != 0) return -1;
  int err = 0;
#pragma omp parallel
  {
    double *h = (double *)malloc(sizeof(double) * (size_t)de);
    double *e = (double *)malloc(sizeof(double) * (size_t)d);
    if (!h || !e) {
#pragma omp atomic write
      err = -2;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
      const int64_t c = t / L;
      double *yt = y + t * d;
      for (int k = 0; k < d; ++k) yt[k] = 0.0;
      if (!h || !e) continue;
      for (int s = 0; s < count[c]; ++s) {
        const int i = list[c * E + s];
        expert_eval(d, de, dtype, x, t * d, w_in, (int64_t)i * de * d, w_out, (int64_t)i * d * de, h, e);
        for (int k = 0; k < d; ++k) yt[k] += g[t * E + i] * e[k];
      }
    }
    free(h);
    free(e);
  }
  return err;
}

/* Dense evaluation: every expert on every token, y_t = sum over all i of g[t][i] E_i(x_t). */
int oracle_forward_dense(int32_t d, int32_t E, int32_t de, int32_t dtype, const void *x, int64_t T,
                         const void *w_in, const void *w_out, const double *g, double *y) {
  int err = 0;
#pragma omp parallel
  {
    double *h = (double *)malloc(sizeof(double) * (size_t)de);
    double *e = (double *)malloc(sizeof(double) * (size_t)d);
    if (!h || !e) {
#pragma omp atomic write
      err = -2;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
      double *yt = y + t * d;
      for (int k = 0; k < d; ++k) yt[k] = 0.0;
      if (!h || !e) continue;
      for (int i = 0; i < E; ++i) {
        expert_eval(d, de, dtype, x, t * d, w_in, (int64_t)i * de * d, w_out, (int64_t)i * d * de, h, e);
        for (int k = 0; k < d; ++k) yt[k] += g[t * E + i] * e[k];
      }
    }
    free(h);
    free(e);
  }
  return err;
}

/*
 * Chunk union (write-up §4; abstract: chunk-level sparsity is about the union
 * of the parameters several consecutive tokens activate).  Chunks are the
 * aligned, non-overlapping runs of L tokens.  umask[c] is the OR of the
 * chunk's token masks, count[c] its number of set bits, list[c][0..count)
 * the set bits in ascending order and list[c][count..E) = -1.
 */
int oracle_union(int32_t E, const uint64_t *mask, int64_t T, int32_t L, uint64_t *umask,
                 int32_t *count, int32_t *list) {
  if (E <= 0 || L <= 0 || T % L != 0) return -1;
  const int W = mask_words(E);
  const int64_t C = T / L;
  for (int64_t c = 0; c < C; ++c) {
    for (int w = 0; w < W; ++w) {
      uint64_t u = 0;
      for (int64_t t = c * L; t < (c + 1) * L; ++t) u |= mask[t * W + w];
      umask[c * W + w] = u;
    }
    int n = 0;
    for (int i = 0; i < E; ++i)
      if (mask_bit(umask + c * W, i)) list[c * E + n++] = i;
    count[c] = n;
    for (int s = n; s < E; ++s) list[c * E + s] = -1;
  }
  return 0;
}

static int64_t count_bits(const uint64_t *m, int E) {
  int64_t n = 0;
  for (int i = 0; i < E; ++i) n += mask_bit(m, i);
  return n;
}

/*
 * Sparsity statistics (abstract and write-up §3: token-level and 8-token
 * chunk-level sparsity; write-up §5: expert reuse between consecutive tokens
 * and the distribution of experts per token).  TLS = 1 - active_pairs/(T E),
 * CLS_L = 1 - union_sum/(C E), reuse = reuse_num/reuse_den.
 */
int oracle_stats(int32_t E, const uint64_t *mask, int64_t T, int32_t L, oracle_stats_t *out) {
  if (E <= 0 || E >= ORACLE_MAX_HIST || L <= 0 || T % L != 0) return -1;
  const int W = mask_words(E);
  const int64_t C = T / L;
  memset(out, 0, sizeof *out);
  out->n_tokens = T;
  out->n_chunks = C;
  out->n_experts = E;
  out->chunk_len = L;
  uint64_t *u = (uint64_t *)calloc((size_t)W, sizeof(uint64_t));
  if (!u) return -2;
  for (int64_t t = 0; t < T; ++t) {
    const int64_t n = count_bits(mask + t * W, E);
    out->active_pairs += n;
    out->hist[n] += 1;
    if (t >= 1) {
      int64_t both = 0;
      for (int i = 0; i < E; ++i) both += mask_bit(mask + t * W, i) & mask_bit(mask + (t - 1) * W, i);
      out->reuse_num += both;
      out->reuse_den += count_bits(mask + (t - 1) * W, E);
    }
  }
  for (int64_t c = 0; c < C; ++c) {
    for (int w = 0; w < W; ++w) u[w] = 0;
    for (int64_t t = c * L; t < (c + 1) * L; ++t)
      for (int w = 0; w < W; ++w) u[w] |= mask[t * W + w];
    out->union_sum += count_bits(u, E);
  }
  free(u);
  return 0;
}

/*
 * Layer backward: the chain rule through the forward above, for a scalar loss
 * whose gradient with respect to y is dy[T][d] (binary32).  Per token t, with
 * r = (ms + eps)^(-1/2) and a_i = max(z_i, 0):
 *
 *   for each active i:  u = W_in[i] x,  sig = 1 / (1 + e^-u),  h = u sig,
 *                       q = W_out[i]^T dy,  dg_i = q . h
 *                       du = g_i q sig (1 + u (1 - sig))    (Swish' = sig (1 + u (1 - sig)))
 *                       dW_out[i] += g_i dy h^T,  dW_in[i] += du x^T,  dx += W_in[i]^T du
 *   ds_i += dg_i a_i r
 *   dr    = sum_i dg_i s_i a_i,   dms = -dr r^3 / 2           (r = (ms + eps)^(-1/2))
 *   da_i  = dg_i s_i r + dms 2 a_i / E                        (ms = sum_i a_i^2 / E)
 *   dz_i  = da_i [z_i > 0]                                    (ReLU)
 *   db   += dz,  dW_r += dz x^T,  dx += W_r^T dz
 *
 * Inactive experts have a_i = g_i = 0 and dz_i = 0: they contribute nothing,
 * so only active pairs are visited.  The gates and pattern are recomputed
 * here exactly as oracle_route computes them.
 *
 * dz_extra ([T][E] or NULL) is a gradient with respect to z from other
 * terms of the loss (the CLS-aware objectives below); it is added to dz for
 * every (token, expert), active or not, before dz reaches db, dW_r and dx.
 *
 * Outputs are double and overwritten: dx[T][d], dw_router[E][d], db[E],
 * ds[E], dw_in[E][de][d], dw_out[E][d][de], dz[T][E] and dg[T][E] (dg_i for
 * active pairs, 0 elsewhere).  expert_sel (E bytes) and token_sel (T bytes)
 * may restrict which dw_in / dw_out blocks and which dx rows are computed
 * (NULL = all; unselected entries are left at 0).  Every sum over tokens runs
 * in ascending token order and every sum over experts in ascending expert
 * order; the per-pair quantities are recomputed where they are needed.
 */
/* One active pair (t, i) of the backward: u = W_in[i] x_t, h = Swish(u),
 * q = W_out[i]^T dy_t and du = g q Swish'(u) (d_e values each). */
static void pair_backward(int d, int de, int dtype, const void *x, int64_t t, const void *w_in,
                          const void *w_out, int i, const float *dy, double g, double *h, double *q,
                          double *du) {
  for (int j = 0; j < de; ++j) {
    double u = 0.0;
    for (int k = 0; k < d; ++k)
      u += widen(w_in, ((int64_t)i * de + j) * d + k, dtype) * widen(x, t * d + k, dtype);
    double qj = 0.0;
    for (int k = 0; k < d; ++k) qj += widen(w_out, ((int64_t)i * d + k) * de + j, dtype) * (double)dy[t * d + k];
    const double sig = 1.0 / (1.0 + exp(-u));
    h[j] = u * sig;
    q[j] = qj;
    du[j] = g * qj * sig * (1.0 + u * (1.0 - sig));
  }
}

int oracle_backward(int32_t d, int32_t E, int32_t de, int32_t dtype, const void *x, int64_t T,
                    const void *w_router, const float *b_router, const float *rms_scale, double eps,
                    const void *w_in, const void *w_out, const float *dy, const double *dz_extra,
                    const uint8_t *expert_sel, const uint8_t *token_sel,
                    double *dx, double *dw_router, double *db, double *ds, double *dw_in, double *dw_out,
                    double *dz, double *dg) {
  if (d <= 0 || E <= 0 || de <= 0 || T < 0) return -1;
  const int W = mask_words(E);
  double *z = (double *)malloc(sizeof(double) * (size_t)(T * E + 1));
  double *g = (double *)malloc(sizeof(double) * (size_t)(T * E + 1));
  double *dsc = (double *)malloc(sizeof(double) * (size_t)(T * E + 1));
  uint64_t *m = (uint64_t *)malloc(sizeof(uint64_t) * (size_t)(T * W + 1));
  if (!z || !g || !dsc || !m) {
    free(z); free(g); free(dsc); free(m);
    return -2;
  }
  oracle_route(d, E, dtype, x, T, w_router, b_router, rms_scale, eps, z, g, m);
  int err = 0;

#pragma omp parallel
  {
    double *h = (double *)malloc(sizeof(double) * (size_t)de);
    double *q = (double *)malloc(sizeof(double) * (size_t)de);
    double *du = (double *)malloc(sizeof(double) * (size_t)de);
    const int ok = h && q && du;
    if (!ok) {
#pragma omp atomic write
      err = -2;
    }

    /* 1. per token: dg for the active pairs, then the RMSNorm and ReLU backward */
#pragma omp for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
      double ms = 0.0;
      for (int i = 0; i < E; ++i) {
        const double a = z[t * E + i] > 0.0 ? z[t * E + i] : 0.0;
        ms += a * a;
      }
      const double r = 1.0 / sqrt(ms / (double)E + eps); /* the gates' 1 / RMS */
      double dr = 0.0;
      for (int i = 0; i < E; ++i) {
        double dgi = 0.0;
        if (mask_bit(m + t * W, i) && ok) {
          pair_backward(d, de, dtype, x, t, w_in, w_out, i, dy, g[t * E + i], h, q, du);
          for (int j = 0; j < de; ++j) dgi += q[j] * h[j];
        }
        const double a = z[t * E + i] > 0.0 ? z[t * E + i] : 0.0;
        const double s = rms_scale ? (double)rms_scale[i] : 1.0;
        dg[t * E + i] = dgi;
        dsc[t * E + i] = dgi * a * r;
        dr += dgi * s * a;
      }
      const double dms = -0.5 * dr * r * r * r;
      for (int i = 0; i < E; ++i) {
        const double a = z[t * E + i] > 0.0 ? z[t * E + i] : 0.0;
        const double s = rms_scale ? (double)rms_scale[i] : 1.0;
        const double da = dg[t * E + i] * s * r + dms * 2.0 * a / (double)E;
        dz[t * E + i] = (z[t * E + i] > 0.0 ? da : 0.0) + (dz_extra ? dz_extra[t * E + i] : 0.0);
      }
    }

    /* 2. router parameter gradients: sums over tokens, ascending */
#pragma omp for schedule(static)
    for (int i = 0; i < E; ++i) {
      double sb = 0.0, ss = 0.0;
      for (int64_t t = 0; t < T; ++t) {
        sb += dz[t * E + i];
        ss += dsc[t * E + i];
      }
      db[i] = sb;
      ds[i] = ss;
      for (int k = 0; k < d; ++k) {
        double acc = 0.0;
        for (int64_t t = 0; t < T; ++t) acc += dz[t * E + i] * widen(x, t * d + k, dtype);
        dw_router[(int64_t)i * d + k] = acc;
      }
    }

    /* 3. expert weight gradients: per expert, sums over its active tokens, ascending */
#pragma omp for schedule(dynamic, 1)
    for (int i = 0; i < E; ++i) {
      double *gi = dw_in + (int64_t)i * de * d;
      double *go = dw_out + (int64_t)i * d * de;
      for (int64_t n = 0; n < (int64_t)de * d; ++n) gi[n] = go[n] = 0.0;
      if ((expert_sel && !expert_sel[i]) || !ok) continue;
      for (int64_t t = 0; t < T; ++t) {
        if (!mask_bit(m + t * W, i)) continue;
        const double gti = g[t * E + i];
        pair_backward(d, de, dtype, x, t, w_in, w_out, i, dy, gti, h, q, du);
        for (int k = 0; k < d; ++k)
          for (int j = 0; j < de; ++j) go[(int64_t)k * de + j] += gti * (double)dy[t * d + k] * h[j];
        for (int j = 0; j < de; ++j)
          for (int k = 0; k < d; ++k) gi[(int64_t)j * d + k] += du[j] * widen(x, t * d + k, dtype);
      }
    }

    /* 4. input gradient: per token, experts ascending, then the router term */
#pragma omp for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
      double *dxt = dx + t * d;
      for (int k = 0; k < d; ++k) dxt[k] = 0.0;
      if ((token_sel && !token_sel[t]) || !ok) continue;
      for (int i = 0; i < E; ++i) {
        if (!mask_bit(m + t * W, i)) continue;
        pair_backward(d, de, dtype, x, t, w_in, w_out, i, dy, g[t * E + i], h, q, du);
        for (int k = 0; k < d; ++k) {
          double acc = 0.0;
          for (int j = 0; j < de; ++j) acc += widen(w_in, ((int64_t)i * de + j) * d + k, dtype) * du[j];
          dxt[k] += acc;
        }
      }
      for (int k = 0; k < d; ++k) {
        double acc = 0.0;
        for (int i = 0; i < E; ++i) acc += dz[t * E + i] * widen(w_router, (int64_t)i * d + k, dtype);
        dxt[k] += acc;
      }
    }
    free(h);
    free(q);
    free(du);
  }
  free(z);
  free(g);
  free(dsc);
  free(m);
  return err;
}

/*
 * CLS-aware training objectives (BlockFFN write-up §3).  With the sharp
 * sigmoid p_{t,i} = sigma(alpha z_{t,i}) as the soft activation pattern:
 *
 *   activation locality: binary cross-entropy between each token's soft
 *     pattern and the next token's activation pattern (the pattern sequence
 *     shifted left by one token), over every consecutive pair of the stream:
 *       L_AL = 1 / ((T - 1) E) * sum_{t < T-1} sum_i BCE(p_{t,i}, [z_{t+1,i} > 0])
 *       BCE(p, y) = -(y log p + (1 - y) log(1 - p)) = softplus(s) - y s, s = alpha z
 *   chunk sparsification: the probability that expert i fires for at least
 *     one token of chunk c, averaged over chunks and experts:
 *       L_CS = 1 / (C E) * sum_c sum_i (1 - prod_{t in c} (1 - p_{t,i}))
 *
 * Writes loss[0] = L_AL, loss[1] = L_CS and, when dz is non-NULL, the
 * gradient dz = w_al dL_AL/dz + w_cs dL_CS/dz ([T][E]):
 *   dL_AL/dz_{t,i} = alpha (p_{t,i} - y_{t,i}) / ((T - 1) E)   (t < T - 1; the target has no gradient)
 *   dL_CS/dz_{t,i} = alpha p (1 - p) prod_{t' in c, t' != t} (1 - p_{t',i}) / (C E)
 * z is the router pre-activation (as oracle_route writes it).
 */
static double softplus(double s) { return s > 0.0 ? s + log1p(exp(-s)) : log1p(exp(s)); }

int oracle_cls_losses(int32_t E, const double *z, int64_t T, int32_t L, double alpha, double w_al, double w_cs,
                      double *loss, double *dz) {
  if (E <= 0 || L <= 0 || T < 0 || T % L != 0) return -1;
  const int64_t C = T / L;
  const double n_al = (double)(T - 1) * (double)E;
  double al = 0.0, cs = 0.0;
  for (int64_t t = 0; t + 1 < T; ++t)
    for (int i = 0; i < E; ++i) {
      const double s = alpha * z[t * E + i];
      const double y = z[(t + 1) * E + i] > 0.0 ? 1.0 : 0.0;
      al += softplus(s) - y * s;
    }
  for (int64_t c = 0; c < C; ++c)
    for (int i = 0; i < E; ++i) {
      double q = 1.0;
      for (int64_t t = c * L; t < (c + 1) * L; ++t) q *= 1.0 - 1.0 / (1.0 + exp(-alpha * z[t * E + i]));
      cs += 1.0 - q;
    }
  loss[0] = T > 1 ? al / n_al : 0.0;
  loss[1] = C > 0 ? cs / ((double)C * (double)E) : 0.0;
  if (!dz) return 0;
  for (int64_t t = 0; t < T; ++t) {
    const int64_t c = t / L;
    for (int i = 0; i < E; ++i) {
      const double p = 1.0 / (1.0 + exp(-alpha * z[t * E + i]));
      double g = 0.0;
      if (t + 1 < T) {
        const double y = z[(t + 1) * E + i] > 0.0 ? 1.0 : 0.0;
        g += w_al * alpha * (p - y) / n_al;
      }
      double others = 1.0;
      for (int64_t u = c * L; u < (c + 1) * L; ++u)
        if (u != t) others *= 1.0 - 1.0 / (1.0 + exp(-alpha * z[u * E + i]));
      g += w_cs * alpha * p * (1.0 - p) * others / ((double)C * (double)E);
      dz[t * E + i] = g;
    }
  }
  return 0;
}
