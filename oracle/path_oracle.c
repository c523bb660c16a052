/*
 * path_oracle.c -- plain, slow fp64 CPU oracle for PaTH attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; only the tests, the smoke check and the bench's CPU-baseline
 * leg do.  It shares no code, header, table or helper with the HIP library.
 *
 * What it computes (PaTH summary, gist.science/ko/paper/2505.16381, section 2
 * "core mechanism"): causal softmax attention whose logit for query i and key
 * j <= i is
 *
 *     z_ij = scale * k_j^T (H_{j+1} H_{j+2} ... H_i) q_i  (+ PaTH-FoX bias)
 *     H_s  = I - beta_s w_s w_s^T
 *
 * The product is written in increasing s from left to right: this is the order
 * fixed by the summary's inference rule (section 3: cached keys are updated in
 * place with the newest transition, k_j <- H_t k_j, which gives
 * (H_i...H_{j+1} k_j)^T q_i).  The empty product (j = i) is the identity.
 *
 * PaTH-FoX (same page, section 2 "PaTH-FoX"): the additive forget bias
 * sum_{s=j+1..i} f_s is added to the scaled logit before the softmax.
 *
 * The logits of one query row are produced by a downward scan: a running
 * vector r starts at q_i; key j is scored against r, and only then is H_j
 * applied to r.  No d x d matrix and no L x L matrix is ever formed (the
 * lecture notes on PaTH, "idea" block, warn that the naive form needs one d x d
 * product chain per score pair).  The softmax is the plain two-pass one:
 * max, then sum of exponentials, then the weighted sum of values.
 *
 * Pins that tie this file to the pages and to mathematics (not to itself) live
 * in tests/test_oracle_pins.py.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL 1
#define ORACLE_ENOMEM 2

/* ------------------------------------------------------------------ basics */

static double dot(const double* a, const double* b, int64_t n) {
  double s = 0.0;
  for (int64_t t = 0; t < n; ++t) s += a[t] * b[t];
  return s;
}

/* r <- (I - beta w w^T) r : one Householder-like transition (summary, section 2). */
static void apply_h(double* r, const double* w, double beta, int64_t d) {
  double c = beta * dot(w, r, d);
  for (int64_t t = 0; t < d; ++t) r[t] -= c * w[t];
}

/*
 * Logits of query row i of one (batch, head): z[j] for j = 0..i.
 * K, W are [L, d]; beta, logf are [L]; logf may be NULL (plain PaTH).
 * r is caller scratch of length d.
 */
static void row_logits(const double* q_i, const double* K, const double* W, const double* beta,
                       const double* logf, int64_t i, int64_t d, double scale, double* r, double* z) {
  memcpy(r, q_i, (size_t)d * sizeof(double));
  double bias = 0.0; /* sum_{s=j+1..i} f_s */
  for (int64_t j = i; j >= 0; --j) {
    z[j] = scale * dot(K + j * d, r, d) + bias;
    apply_h(r, W + j * d, beta[j], d);
    if (logf) bias += logf[j];
  }
}

/* Exact two-pass softmax of z[0..n-1] applied to V [n, d]; lse = m + ln(sum exp(z - m)). */
static void softmax_rows(const double* z, int64_t n, const double* V, int64_t d, double* o, double* lse) {
  double m = -INFINITY;
  for (int64_t j = 0; j < n; ++j)
    if (z[j] > m) m = z[j];
  double l = 0.0;
  for (int64_t j = 0; j < n; ++j) l += exp(z[j] - m);
  for (int64_t t = 0; t < d; ++t) o[t] = 0.0;
  for (int64_t j = 0; j < n; ++j) {
    double p = exp(z[j] - m) / l;
    const double* vj = V + j * d;
    for (int64_t t = 0; t < d; ++t) o[t] += p * vj[t];
  }
  *lse = m + log(l);
}

static int resolve_threads(int nthreads) {
  if (nthreads > 0) return nthreads;
  long n = sysconf(_SC_NPROCESSORS_ONLN);
  return n > 0 ? (int)n : 1;
}

/* ------------------------------------------------------------------ prefill */

typedef struct {
  const double *q, *k, *v, *w, *beta, *logf;
  int64_t BH, L, d, nrows;
  const int64_t* rows;
  double scale;
  double *out, *lse;
  int64_t next; /* shared work counter, one item = (bh, row) */
} fwd_job;

static void* fwd_worker(void* arg) {
  fwd_job* J = (fwd_job*)arg;
  double* r = (double*)malloc((size_t)J->d * sizeof(double));
  double* z = (double*)malloc((size_t)(J->L > 0 ? J->L : 1) * sizeof(double));
  if (!r || !z) {
    free(r);
    free(z);
    return (void*)1;
  }
  const int64_t total = J->BH * J->nrows;
  for (;;) {
    int64_t item = __atomic_fetch_add(&J->next, 1, __ATOMIC_RELAXED);
    if (item >= total) break;
    int64_t bh = item / J->nrows, ri = item % J->nrows;
    int64_t i = J->rows ? J->rows[ri] : ri;
    const int64_t base = bh * J->L;
    row_logits(J->q + (base + i) * J->d, J->k + base * J->d, J->w + base * J->d, J->beta + base,
               J->logf ? J->logf + base : NULL, i, J->d, J->scale, r, z);
    softmax_rows(z, i + 1, J->v + base * J->d, J->d, J->out + (bh * J->nrows + ri) * J->d,
                 J->lse + bh * J->nrows + ri);
  }
  free(r);
  free(z);
  return NULL;
}

/*
 * PaTH (or PaTH-FoX when logf != NULL) forward for BH independent (batch, head)
 * slices.  q,k,v,w: [BH, L, d]; beta, logf: [BH, L].
 * rows == NULL: every row 0..L-1 (nrows must equal L); otherwise only the listed
 * rows, each in [0, L).  out: [BH, nrows, d]; lse: [BH, nrows].
 */
int path_oracle_fwd(const double* q, const double* k, const double* v, const double* w,
                    const double* beta, const double* logf, int64_t BH, int64_t L, int64_t d,
                    double scale, const int64_t* rows, int64_t nrows, double* out, double* lse,
                    int nthreads) {
  if (BH < 0 || L < 0 || d <= 0 || nrows < 0) return ORACLE_EINVAL;
  if (!rows && nrows != L) return ORACLE_EINVAL;
  if (rows)
    for (int64_t r = 0; r < nrows; ++r)
      if (rows[r] < 0 || rows[r] >= L) return ORACLE_EINVAL;
  if (BH == 0 || nrows == 0) return ORACLE_OK;
  fwd_job J = {q, k, v, w, beta, logf, BH, L, d, nrows, rows, scale, out, lse, 0};
  int nt = resolve_threads(nthreads);
  if ((int64_t)nt > BH * nrows) nt = (int)(BH * nrows);
  pthread_t* th = (pthread_t*)malloc((size_t)nt * sizeof(pthread_t));
  if (!th) return ORACLE_ENOMEM;
  int rc = ORACLE_OK;
  for (int t = 0; t < nt; ++t) pthread_create(&th[t], NULL, fwd_worker, &J);
  for (int t = 0; t < nt; ++t) {
    void* ret = NULL;
    pthread_join(th[t], &ret);
    if (ret) rc = ORACLE_ENOMEM;
  }
  free(th);
  return rc;
}

/* ------------------------------------------------------------------ backward */
/*
 * Gradients of the forward above for an upstream gradient dO of the outputs
 * (loss = sum_i dO_i . o_i).  The pages print no backward pass (the lecture
 * notes only warn, under "limitations", that it is costlier than RoPE's); this is
 * the chain rule applied to the definition and nothing else:
 *
 *   p_ij = softmax_j(z_ij)                 dv_j  = sum_i p_ij dO_i
 *   D_i  = sum_j p_ij (dO_i . v_j)         dz_ij = p_ij (dO_i . v_j - D_i)
 *
 *   a_{j,s} = H_{s-1} ... H_{j+1} k_j   (key j carried up to just below s; a_{j,j+1} = k_j)
 *   g_{s,i} = H_{s+1} ... H_i q_i       (query i carried down to just above s; g_{i,i} = q_i)
 *
 * Because every H is symmetric, z_ij = scale a_{j,s}^T H_s g_{s,i} + bias_ij for
 * any s in (j, i], and z_ij = scale k_j . g_{j,i} + bias_ij.  Hence
 *
 *   dq_i  = scale sum_{j<=i} dz_ij a_{j,i+1}
 *   dk_j  = scale sum_{i>=j} dz_ij g_{j,i}
 *   dH_s  = scale sum_{j<s<=i} dz_ij a_{j,s} g_{s,i}^T      (d x d; only dH_s w_s and
 *                                                           dH_s^T w_s are formed)
 *   H_s = I - beta_s w_s w_s^T:  dbeta_s = -w_s^T dH_s w_s,
 *                                dw_s    = -beta_s (dH_s + dH_s^T) w_s
 *   PaTH-FoX, bias_ij = sum_{s=j+1..i} f_s:  df_s = sum_{j<s<=i} dz_ij.
 */
typedef struct {
  const double *q, *k, *v, *w, *beta, *logf, *dout;
  int64_t BH, L, d;
  double scale;
  double *dq, *dk, *dv, *dw, *dbeta, *dlogf;
  int64_t next; /* shared work counter, one item = one (batch, head) */
} bwd_job;

static void bwd_one(const bwd_job* J, int64_t bh, double* P, double* dZ, double* G, double* A, double* r,
                    double* gw, double* aw, double* cu, double* cv) {
  const int64_t L = J->L, d = J->d, base = bh * L;
  const double *Q = J->q + base * d, *K = J->k + base * d, *V = J->v + base * d, *W = J->w + base * d;
  const double *beta = J->beta + base, *logf = J->logf ? J->logf + base : NULL, *dO = J->dout + base * d;
  double *dq = J->dq + base * d, *dk = J->dk + base * d, *dv = J->dv + base * d, *dw = J->dw + base * d;
  double *dbeta = J->dbeta + base, *dlogf = J->dlogf ? J->dlogf + base : NULL;
  const double scale = J->scale;

  /* probabilities: logits of each row, then the exact softmax */
  for (int64_t i = 0; i < L; ++i) {
    double* z = P + i * L;
    row_logits(Q + i * d, K, W, beta, logf, i, d, scale, r, z);
    double m = -INFINITY, l = 0.0;
    for (int64_t j = 0; j <= i; ++j)
      if (z[j] > m) m = z[j];
    for (int64_t j = 0; j <= i; ++j) l += exp(z[j] - m);
    for (int64_t j = 0; j <= i; ++j) z[j] = exp(z[j] - m) / l;
  }
  /* dv, D, dz */
  memset(dv, 0, (size_t)(L * d) * sizeof(double));
  for (int64_t i = 0; i < L; ++i) {
    const double* p = P + i * L;
    double D = 0.0;
    for (int64_t j = 0; j <= i; ++j) {
      const double dp = dot(dO + i * d, V + j * d, d);
      dZ[i * L + j] = dp;
      D += p[j] * dp;
      for (int64_t t = 0; t < d; ++t) dv[j * d + t] += p[j] * dO[i * d + t];
    }
    for (int64_t j = 0; j <= i; ++j) dZ[i * L + j] = p[j] * (dZ[i * L + j] - D);
  }
  /* carried queries g_{s,i} (G[(i L + s) d]) and keys a_{j,s} (A[(j (L+1) + s) d]) */
  for (int64_t i = 0; i < L; ++i) {
    memcpy(r, Q + i * d, (size_t)d * sizeof(double));
    for (int64_t s = i; s >= 0; --s) {
      memcpy(G + (i * L + s) * d, r, (size_t)d * sizeof(double));
      apply_h(r, W + s * d, beta[s], d);
    }
  }
  for (int64_t j = 0; j < L; ++j) {
    memcpy(r, K + j * d, (size_t)d * sizeof(double));
    for (int64_t s = j + 1; s <= L; ++s) {
      memcpy(A + (j * (L + 1) + s) * d, r, (size_t)d * sizeof(double));
      if (s < L) apply_h(r, W + s * d, beta[s], d);
    }
  }
  /* dq, dk */
  for (int64_t i = 0; i < L; ++i) {
    for (int64_t t = 0; t < d; ++t) dq[i * d + t] = 0.0;
    for (int64_t j = 0; j <= i; ++j) {
      const double c = scale * dZ[i * L + j];
      const double* a = A + (j * (L + 1) + i + 1) * d;
      for (int64_t t = 0; t < d; ++t) dq[i * d + t] += c * a[t];
    }
  }
  for (int64_t j = 0; j < L; ++j) {
    for (int64_t t = 0; t < d; ++t) dk[j * d + t] = 0.0;
    for (int64_t i = j; i < L; ++i) {
      const double c = scale * dZ[i * L + j];
      const double* g = G + (i * L + j) * d;
      for (int64_t t = 0; t < d; ++t) dk[j * d + t] += c * g[t];
    }
  }
  /* dH_s w_s and dH_s^T w_s over the pairs j < s <= i, then dbeta, dw, df */
  for (int64_t s = 0; s < L; ++s) {
    const double* ws = W + s * d;
    for (int64_t i = s; i < L; ++i) gw[i] = dot(G + (i * L + s) * d, ws, d);
    for (int64_t j = 0; j < s; ++j) aw[j] = dot(A + (j * (L + 1) + s) * d, ws, d);
    for (int64_t t = 0; t < d; ++t) cu[t] = cv[t] = 0.0;
    double df = 0.0;
    for (int64_t j = 0; j < s; ++j) {
      double c = 0.0; /* sum_i dz_ij (g_{s,i} . w_s) */
      for (int64_t i = s; i < L; ++i) c += dZ[i * L + j] * gw[i];
      const double* a = A + (j * (L + 1) + s) * d;
      for (int64_t t = 0; t < d; ++t) cu[t] += scale * c * a[t];
    }
    for (int64_t i = s; i < L; ++i) {
      double c = 0.0; /* sum_j dz_ij (a_{j,s} . w_s) */
      for (int64_t j = 0; j < s; ++j) {
        c += dZ[i * L + j] * aw[j];
        df += dZ[i * L + j];
      }
      const double* g = G + (i * L + s) * d;
      for (int64_t t = 0; t < d; ++t) cv[t] += scale * c * g[t];
    }
    dbeta[s] = -dot(ws, cu, d);
    for (int64_t t = 0; t < d; ++t) dw[s * d + t] = -beta[s] * (cu[t] + cv[t]);
    if (dlogf) dlogf[s] = df;
  }
}

static void* bwd_worker(void* arg) {
  bwd_job* J = (bwd_job*)arg;
  const int64_t L = J->L, d = J->d;
  double* P = (double*)malloc((size_t)(L * L) * sizeof(double));
  double* dZ = (double*)malloc((size_t)(L * L) * sizeof(double));
  double* G = (double*)malloc((size_t)(L * L * d) * sizeof(double));
  double* A = (double*)malloc((size_t)(L * (L + 1) * d) * sizeof(double));
  double* r = (double*)malloc((size_t)(3 * d + 2 * L) * sizeof(double)); /* r, gw, aw, cu, cv */
  void* ret = NULL;
  if (!P || !dZ || !G || !A || !r) {
    ret = (void*)1;
  } else {
    for (;;) {
      int64_t bh = __atomic_fetch_add(&J->next, 1, __ATOMIC_RELAXED);
      if (bh >= J->BH) break;
      bwd_one(J, bh, P, dZ, G, A, r, r + d, r + d + L, r + d + 2 * L, r + 2 * d + 2 * L);
    }
  }
  free(P);
  free(dZ);
  free(G);
  free(A);
  free(r);
  return ret;
}

/*
 * Backward of path_oracle_fwd over all rows.  Inputs as there plus dout [BH, L, d].
 * Outputs dq, dk, dv, dw [BH, L, d]; dbeta [BH, L]; dlogf [BH, L] (only when logf != NULL).
 * Memory: about (2 L^2 + 2 L^2 d) doubles per worker thread.
 */
int path_oracle_bwd(const double* q, const double* k, const double* v, const double* w, const double* beta,
                    const double* logf, const double* dout, int64_t BH, int64_t L, int64_t d, double scale,
                    double* dq, double* dk, double* dv, double* dw, double* dbeta, double* dlogf, int nthreads) {
  if (BH < 0 || L < 0 || d <= 0) return ORACLE_EINVAL;
  if ((logf == NULL) != (dlogf == NULL)) return ORACLE_EINVAL;
  if (BH == 0 || L == 0) return ORACLE_OK;
  bwd_job J = {q, k, v, w, beta, logf, dout, BH, L, d, scale, dq, dk, dv, dw, dbeta, dlogf, 0};
  int nt = resolve_threads(nthreads);
  if ((int64_t)nt > BH) nt = (int)BH;
  pthread_t* th = (pthread_t*)malloc((size_t)nt * sizeof(pthread_t));
  if (!th) return ORACLE_ENOMEM;
  int rc = ORACLE_OK;
  for (int t = 0; t < nt; ++t) pthread_create(&th[t], NULL, bwd_worker, &J);
  for (int t = 0; t < nt; ++t) {
    void* ret = NULL;
    pthread_join(th[t], &ret);
    if (ret) rc = ORACLE_ENOMEM;
  }
  free(th);
  return rc;
}

/* Logits z[0..i] of one row of one (batch, head) slice; K, W: [L, d], beta, logf: [L]. */
int path_oracle_row_logits(const double* q_i, const double* K, const double* W, const double* beta,
                           const double* logf, int64_t i, int64_t d, double scale, double* z) {
  if (i < 0 || d <= 0) return ORACLE_EINVAL;
  double* r = (double*)malloc((size_t)d * sizeof(double));
  if (!r) return ORACLE_ENOMEM;
  row_logits(q_i, K, W, beta, logf, i, d, scale, r, z);
  free(r);
  return ORACLE_OK;
}

/* out = H_lo H_{lo+1} ... H_hi x   (H_hi is applied first; empty product when hi < lo). */
int path_oracle_transport(const double* x, const double* W, const double* beta, int64_t lo, int64_t hi,
                          int64_t d, double* out) {
  if (d <= 0) return ORACLE_EINVAL;
  memcpy(out, x, (size_t)d * sizeof(double));
  for (int64_t s = hi; s >= lo; --s) apply_h(out, W + s * d, beta[s], d);
  return ORACLE_OK;
}

/* ------------------------------------------------------------------ decode */

typedef struct {
  double *kc, *vc, *fc;
  int64_t BH, cap, t0, nsteps, d;
  const double *qs, *ks, *vs, *ws, *betas, *fs;
  double scale;
  double *out, *lse;
  int64_t next;
} dec_job;

static void* dec_worker(void* arg) {
  dec_job* J = (dec_job*)arg;
  const int64_t d = J->d;
  double* z = (double*)malloc((size_t)(J->t0 + J->nsteps) * sizeof(double));
  if (!z) return (void*)1;
  for (;;) {
    int64_t bh = __atomic_fetch_add(&J->next, 1, __ATOMIC_RELAXED);
    if (bh >= J->BH) break;
    double* Kc = J->kc + bh * J->cap * d;
    double* Vc = J->vc + bh * J->cap * d;
    double* Fc = J->fc ? J->fc + bh * J->cap : NULL;
    for (int64_t s = 0; s < J->nsteps; ++s) {
      const int64_t t = J->t0 + s;
      const int64_t tok = s * J->BH + bh;
      const double* w = J->ws + tok * d;
      const double beta = J->betas[tok];
      /* Inference rule (summary, section 3): every cached key j < t takes the
         newest transition in place; the new key enters untransformed. */
      for (int64_t j = 0; j < t; ++j) apply_h(Kc + j * d, w, beta, d);
      memcpy(Kc + t * d, J->ks + tok * d, (size_t)d * sizeof(double));
      memcpy(Vc + t * d, J->vs + tok * d, (size_t)d * sizeof(double));
      /* PaTH-FoX (section 2): slot j carries the forget bias sum_{s=j+1..t} f_s,
         grown in place by the newest gate like the keys; the new slot starts at 0. */
      if (Fc) {
        for (int64_t j = 0; j < t; ++j) Fc[j] += J->fs[tok];
        Fc[t] = 0.0;
      }
      const double* qt = J->qs + tok * d;
      for (int64_t j = 0; j <= t; ++j) z[j] = J->scale * dot(Kc + j * d, qt, d) + (Fc ? Fc[j] : 0.0);
      softmax_rows(z, t + 1, Vc, d, J->out + tok * d, J->lse + tok);
    }
  }
  free(z);
  return NULL;
}

/*
 * nsteps decode steps for BH independent slices.  kc, vc: [BH, cap, d], the first
 * t0 slots hold the current cache; they are updated in place and slots
 * t0..t0+nsteps-1 are appended.  qs,ks,vs,ws: [nsteps, BH, d]; betas: [nsteps, BH].
 * PaTH-FoX: fc [BH, cap] per-slot forget bias (first t0 slots current, updated in
 * place) and fs [nsteps, BH] the new tokens' gates; both NULL for plain PaTH.
 * out: [nsteps, BH, d]; lse: [nsteps, BH].
 */
int path_oracle_decode(double* kc, double* vc, double* fc, int64_t BH, int64_t cap, int64_t t0, int64_t nsteps,
                       const double* qs, const double* ks, const double* vs, const double* ws,
                       const double* betas, const double* fs, int64_t d, double scale, double* out, double* lse,
                       int nthreads) {
  if (BH < 0 || cap < 0 || t0 < 0 || nsteps < 0 || d <= 0 || t0 + nsteps > cap) return ORACLE_EINVAL;
  if ((fc == NULL) != (fs == NULL)) return ORACLE_EINVAL;
  if (BH == 0 || nsteps == 0) return ORACLE_OK;
  dec_job J = {kc, vc, fc, BH, cap, t0, nsteps, d, qs, ks, vs, ws, betas, fs, scale, out, lse, 0};
  int nt = resolve_threads(nthreads);
  if ((int64_t)nt > BH) nt = (int)BH;
  pthread_t* th = (pthread_t*)malloc((size_t)nt * sizeof(pthread_t));
  if (!th) return ORACLE_ENOMEM;
  int rc = ORACLE_OK;
  for (int t = 0; t < nt; ++t) pthread_create(&th[t], NULL, dec_worker, &J);
  for (int t = 0; t < nt; ++t) {
    void* ret = NULL;
    pthread_join(th[t], &ret);
    if (ret) rc = ORACLE_ENOMEM;
  }
  free(th);
  return rc;
}

/* ------------------------------------------------------------------ prefill -> decode cache */

/*
 * Key cache after a prompt of L tokens (summary, section 3, inference rule): once the
 * prompt has been consumed, every cached key has taken each later transition in
 * place, so slot j holds H_{L-1} ... H_{j+2} H_{j+1} k_j (H_{j+1} applied first;
 * slot L-1 holds k_{L-1} itself).  Then q^T slot_j = k_j^T H_{j+1} ... H_{L-1} q, the
 * unscaled logit a query at position L-1 gives key j.
 * K, W: [L, d]; beta: [L].  Writes rows j0 .. j1-1 of the cache into out [(j1 - j0), d].
 */
int path_oracle_cache_keys(const double* K, const double* W, const double* beta, int64_t L, int64_t d,
                           int64_t j0, int64_t j1, double* out) {
  if (L < 0 || d <= 0 || j0 < 0 || j1 < j0 || j1 > L) return ORACLE_EINVAL;
  for (int64_t j = j0; j < j1; ++j) {
    double* r = out + (j - j0) * d;
    memcpy(r, K + j * d, (size_t)d * sizeof(double));
    for (int64_t s = j + 1; s < L; ++s) apply_h(r, W + s * d, beta[s], d);
  }
  return ORACLE_OK;
}

/*
 * PaTH-FoX part of the same cache: slot j's forget bias after a prompt of L tokens,
 * sum_{s=j+1..L-1} f_s (0 for the last slot), summed from s = j+1 upwards.
 */
int path_oracle_cache_bias(const double* logf, int64_t L, double* out) {
  if (L < 0) return ORACLE_EINVAL;
  for (int64_t j = 0; j < L; ++j) {
    double b = 0.0;
    for (int64_t s = j + 1; s < L; ++s) b += logf[s];
    out[j] = b;
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------ chunk quantities */

/*
 * Compact (UT) form of a run of transitions (summary, section 3 "UT transform"):
 * H_0 H_1 ... H_{n-1} = I - W^T T^{-1} W with W = [w_0; ...; w_{n-1}] (n x d) and T
 * the upper-triangular matrix with diagonal 1/beta_s and strict upper part
 * (W W^T)_{st}.  We never form 1/beta: T^{-1} = A^{-1} diag(beta) with
 * A = I + diag(beta) * strict_upper(W W^T), a unit upper-triangular matrix solved
 * here by plain back substitution, column by column.  tinv: n x n, row-major.
 */
int path_oracle_ut_tinv(const double* W, const double* beta, int64_t n, int64_t d, double* tinv) {
  if (n < 0 || d <= 0) return ORACLE_EINVAL;
  double* A = (double*)calloc((size_t)(n * n > 0 ? n * n : 1), sizeof(double));
  if (!A) return ORACLE_ENOMEM;
  for (int64_t s = 0; s < n; ++s)
    for (int64_t t = s + 1; t < n; ++t) A[s * n + t] = beta[s] * dot(W + s * d, W + t * d, d);
  /* Z = A^{-1}: Z[j][j] = 1, Z[i][j] = -sum_{k=i+1..j} A[i][k] Z[k][j] for i < j. */
  for (int64_t j = 0; j < n; ++j) {
    for (int64_t i = n - 1; i > j; --i) tinv[i * n + j] = 0.0;
    tinv[j * n + j] = 1.0;
    for (int64_t i = j - 1; i >= 0; --i) {
      double s = 0.0;
      for (int64_t k = i + 1; k <= j; ++k) s += A[i * n + k] * tinv[k * n + j];
      tinv[i * n + j] = -s;
    }
  }
  for (int64_t i = 0; i < n; ++i)
    for (int64_t j = 0; j < n; ++j) tinv[i * n + j] *= beta[j];
  free(A);
  return ORACLE_OK;
}

/* Explicit d x d product P = H_0 H_1 ... H_{n-1} (row-major), built as P <- P H_s. */
int path_oracle_householder_product(const double* W, const double* beta, int64_t n, int64_t d,
                                    double* P) {
  if (n < 0 || d <= 0) return ORACLE_EINVAL;
  double* pw = (double*)malloc((size_t)d * sizeof(double));
  if (!pw) return ORACLE_ENOMEM;
  for (int64_t a = 0; a < d; ++a)
    for (int64_t b = 0; b < d; ++b) P[a * d + b] = (a == b) ? 1.0 : 0.0;
  for (int64_t s = 0; s < n; ++s) {
    const double* w = W + s * d;
    for (int64_t a = 0; a < d; ++a) pw[a] = dot(P + a * d, w, d);
    for (int64_t a = 0; a < d; ++a)
      for (int64_t b = 0; b < d; ++b) P[a * d + b] -= beta[s] * pw[a] * w[b];
  }
  free(pw);
  return ORACLE_OK;
}

/*
 * Boundary-adjusted rows of one chunk of n tokens (summary, section 3,
 * "FlashAttention-style algorithm": precomputed boundary-adjusted query and key
 * rows), by their definitions:
 *   qtilde_a = H_0 H_1 ... H_a q_a            (chunk prefix, token a included)
 *   ktilde_b = H_{n-1} ... H_{b+1} k_b        (chunk suffix strictly after b)
 *   sintra[a][b] = k_b^T H_{b+1} ... H_a q_a  for b <= a (unscaled), 0 above the diagonal.
 * q, k, W: [n, d]; outputs qtilde, ktilde [n, d], sintra [n, n].
 */
int path_oracle_chunk_terms(const double* q, const double* k, const double* W, const double* beta,
                            int64_t n, int64_t d, double* qtilde, double* ktilde, double* sintra) {
  if (n < 0 || d <= 0) return ORACLE_EINVAL;
  double* r = (double*)malloc((size_t)d * sizeof(double));
  if (!r) return ORACLE_ENOMEM;
  for (int64_t a = 0; a < n; ++a) {
    /* The row scan gives sintra[a][*] and, after H_0, the prefix-adjusted query. */
    memcpy(r, q + a * d, (size_t)d * sizeof(double));
    for (int64_t b = a; b >= 0; --b) {
      sintra[a * n + b] = dot(k + b * d, r, d);
      apply_h(r, W + b * d, beta[b], d);
    }
    for (int64_t b = a + 1; b < n; ++b) sintra[a * n + b] = 0.0;
    memcpy(qtilde + a * d, r, (size_t)d * sizeof(double));
    /* ktilde_b = H_{n-1} ... H_{b+1} k_b : apply H_{b+1} first. */
    memcpy(ktilde + a * d, k + a * d, (size_t)d * sizeof(double));
    for (int64_t s = a + 1; s < n; ++s) apply_h(ktilde + a * d, W + s * d, beta[s], d);
  }
  free(r);
  return ORACLE_OK;
}

int path_oracle_abi_version(void) { return 1; }
