/*
 * CPU oracle for the HSTU block forward with a paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library; both follow the same written
 * definition independently.
 *
 * What it computes (all arithmetic in double; inputs are float values, which
 * in bf16 workloads are exactly representable in bf16):
 *
 *   HSTU block ("How Generative Recommenders Are Redefining RecSys at Scale",
 *   section HSTU: softmax replaced by SiLU-based weighting, a relative
 *   attention bias, elementwise gating before the output projection), with
 *   the equations
 *       x^   = LayerNorm(x)                       (over d, biased variance, no affine)
 *       [U|V|Q|K] = SiLU(x^ . W1)                 (column chunks, head-major inside)
 *       o_i  = (1/n) sum_{j in M(i)} SiLU(q_i.k_j + rab[b(i-j)]) v_j    (per head)
 *       g    = LayerNorm(o) (*) U                 (over all heads concatenated)
 *       y    = x + g . W2
 *   M(i) = {j <= i} for history queries, {j < history length} u {i} for
 *   candidate queries; b(delta) = min(nb-1, floor(4 log2(1+delta))).
 *
 *   Multitask ranking head (see oracle_head): per scored row and task, a
 *   Linear -> ReLU -> Linear perceptron giving the task's logit.
 *
 *   KV cache ("Deploying an HSTU Generative Recommender with NVIDIA
 *   Dynamo-Triton": a paged KV data table with lookup, allocation, append and
 *   eviction, LRU-style eviction of older users when space is tight; the
 *   attention reads the cache directly): an allocator with a FIFO free-page
 *   queue, whole-user LRU eviction, and a canonical state dump.
 *
 * Sums run in ascending index order.  OpenMP splits only independent outputs
 * (rows, (user, head, query) triples); it does not change any summation.
 * Build: gcc -O2 -fopenmp -fPIC -shared (no -ffast-math).
 *
 * Compile-time ORACLE_MUTANT=k plants one deliberate mistake (used only by
 * the tests that prove the pins catch such mistakes).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

#define OK 0
#define ERR_INVALID 1
#define ERR_NO_SPACE 2
#define ERR_UNKNOWN_USER 3

/* threads an OpenMP region of the oracle uses */
int oracle_threads(void) { return omp_get_max_threads(); }
/* sets that number (n >= 1), e.g. 1 for a single-threaded timing */
void oracle_set_threads(int n) { omp_set_num_threads(n < 1 ? 1 : n); }

/* ------------------------------------------------------------------------ */
/* elementwise pieces                                                        */
/* ------------------------------------------------------------------------ */

/* SiLU(z) = z * sigmoid(z) = z / (1 + e^-z) */
double oracle_silu(double z) {
#if ORACLE_MUTANT == 1
  return z / (1.0 + exp(z)); /* planted: wrong sign in the exponent */
#else
  return z / (1.0 + exp(-z));
#endif
}

/* LayerNorm without affine: (x - mean) / sqrt(var + eps), biased variance. */
void oracle_layer_norm(const double *x, int n, double eps, double *out) {
  double mean = 0.0;
  for (int k = 0; k < n; ++k) mean += x[k];
  mean /= n;
  double var = 0.0;
  for (int k = 0; k < n; ++k) var += (x[k] - mean) * (x[k] - mean);
  var /= n;
#if ORACLE_MUTANT == 2
  double inv = 1.0 / sqrt(var); /* planted: eps dropped */
#else
  double inv = 1.0 / sqrt(var + eps);
#endif
  for (int k = 0; k < n; ++k) out[k] = (x[k] - mean) * inv;
}

/* Relative-position bucket b(delta) = min(nb - 1, floor(4 * log2(1 + delta))),
 * evaluated exactly: floor(4 log2 m) = floor(log2(m^4)) = bit length of m^4
 * minus one, with m = 1 + delta. */
int oracle_bucket(int64_t delta, int num_buckets) {
  if (delta < 0) return -1;
  unsigned __int128 m = (unsigned __int128)(delta + 1);
  unsigned __int128 p = m * m * m * m;
  int b = 0;
  while ((p >> (b + 1)) != 0) ++b;
#if ORACLE_MUTANT == 3
  b = b / 2; /* planted: wrong bucket scale */
#endif
  return b < num_buckets - 1 ? b : num_buckets - 1;
}

/* Visibility of key position j to query position i for a user whose first
 * `hist` positions are history and the rest candidates. */
static int visible(int64_t i, int64_t j, int64_t hist) {
#if ORACLE_MUTANT == 4
  return j <= i; /* planted: candidates see each other (plain causal) */
#else
  if (j == i) return 1;
  return j < i && j < hist;
#endif
}

/* ------------------------------------------------------------------------ */
/* attention over a jagged batch                                             */
/* ------------------------------------------------------------------------ */

/*
 * q      [N_new][H][dh]   queries of the new tokens (user u's new tokens are
 *                          rows q_off[u] .. q_off[u+1]-1, at positions
 *                          start[u] .. start[u] + t_u - 1)
 * k, v   [sum L_u][H][dh] every key/value of user u (positions 0..L_u-1) at
 *                          rows kv_off[u] .. kv_off[u+1]-1
 * n_targets[u]             T_u: the last T_u positions are candidates
 * norm_n[u]                n_u
 * rab[num_buckets]         bias table of the layer (shared by the heads)
 * o      [N_new][H][dh]   output (A V), already divided by n_u
 */
int oracle_attention(int B, int H, int dh, const int64_t *q_off, const int64_t *start,
                     const int64_t *kv_off, const int64_t *n_targets, const double *norm_n,
                     const double *q, const double *k, const double *v, const double *rab,
                     int num_buckets, double *o) {
  if (B < 0 || H <= 0 || dh <= 0 || num_buckets <= 0) return ERR_INVALID;
  for (int u = 0; u < B; ++u) {
    int64_t t_u = q_off[u + 1] - q_off[u];
    int64_t L_u = kv_off[u + 1] - kv_off[u];
    if (t_u < 0 || L_u < 0 || start[u] < 0 || start[u] + t_u > L_u) return ERR_INVALID;
    if (n_targets[u] < 0 || n_targets[u] > L_u) return ERR_INVALID;
  }
  int64_t n_new = q_off[B];
  int64_t total = n_new * H;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t task = 0; task < total; ++task) {
    int64_t row = task / H;
    int h = (int)(task % H);
    int u = 0;
    while (q_off[u + 1] <= row) ++u;
    int64_t L_u = kv_off[u + 1] - kv_off[u];
    int64_t hist = L_u - n_targets[u];
    int64_t i = start[u] + (row - q_off[u]);
    const double *qi = q + (row * H + h) * dh;
    double *oi = o + (row * H + h) * dh;
    for (int e = 0; e < dh; ++e) oi[e] = 0.0;
    for (int64_t j = 0; j < L_u; ++j) {
      if (!visible(i, j, hist)) continue;
      const double *kj = k + ((kv_off[u] + j) * H + h) * dh;
      const double *vj = v + ((kv_off[u] + j) * H + h) * dh;
      double s = 0.0;
      for (int e = 0; e < dh; ++e) s += qi[e] * kj[e];
#if ORACLE_MUTANT == 5
      /* planted: bias dropped */
#elif ORACLE_MUTANT == 6
      s += rab[oracle_bucket(i - j + 1, num_buckets)]; /* planted: off-by-one distance */
#else
      s += rab[oracle_bucket(i - j, num_buckets)];
#endif
      double w = oracle_silu(s);
      for (int e = 0; e < dh; ++e) oi[e] += w * vj[e];
    }
#if ORACLE_MUTANT == 7
    double n = norm_n[u] + 1.0; /* planted: wrong normalizer */
#else
    double n = norm_n[u];
#endif
    for (int e = 0; e < dh; ++e) oi[e] /= n;
  }
  return OK;
}

/* ------------------------------------------------------------------------ */
/* one HSTU layer                                                            */
/* ------------------------------------------------------------------------ */

/*
 * x        [N_new][d] double  layer input of the new tokens (jagged by q_off)
 * w1       [d][4*H*dh] float  f1, used as x^ . W1; column chunks U, V, Q, K
 * w2       [H*dh][d] float    f2
 * rab      [num_buckets] float
 * start[u]                    c_u: cached positions of user u (new tokens follow)
 * hist_k/v [sum c_u][H][dh] double  cached K/V of each user, rows hist_off[u]..
 * Outputs (double; any may be NULL except y):
 *   xhat [N_new][d], u/v/q/k [N_new][H*dh], o [N_new][H*dh], g [N_new][H*dh], y [N_new][d]
 */
int oracle_layer(int B, int d, int H, int dh, double eps, const int64_t *q_off,
                 const int64_t *start, const int64_t *n_targets, const double *norm_n,
                 const double *x, const float *w1, const float *w2, const float *rab,
                 int num_buckets, const int64_t *hist_off, const double *hist_k,
                 const double *hist_v, double *xhat_out, double *u_out, double *v_out,
                 double *q_out, double *k_out, double *o_out, double *g_out, double *y) {
  if (B < 0 || d <= 0 || H <= 0 || dh <= 0 || !y) return ERR_INVALID;
  for (int u = 0; u < B; ++u)
    if (hist_off[u + 1] - hist_off[u] != start[u]) return ERR_INVALID;
  const int inner = H * dh;
  const int64_t n_new = q_off[B];
  double *xh = (double *)malloc(sizeof(double) * (size_t)(n_new * d + 1));
  double *s = (double *)malloc(sizeof(double) * (size_t)(n_new * 4 * inner + 1));
  double *o = (double *)malloc(sizeof(double) * (size_t)(n_new * inner + 1));
  double *g = (double *)malloc(sizeof(double) * (size_t)(n_new * inner + 1));
  int64_t *kv_off = (int64_t *)malloc(sizeof(int64_t) * (size_t)(B + 1));
  if (!xh || !s || !o || !g || !kv_off) return ERR_INVALID;

  /* 1. pre-norm */
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n_new; ++r) {
    double tmp[d];
    for (int c = 0; c < d; ++c) tmp[c] = x[r * d + c];
    oracle_layer_norm(tmp, d, eps, xh + r * d);
  }
  /* 2. f1 then SiLU */
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n_new; ++r) {
    for (int c = 0; c < 4 * inner; ++c) {
      double z = 0.0;
      for (int kk = 0; kk < d; ++kk) {
#if ORACLE_MUTANT == 8
        z += xh[r * d + kk] * (double)w1[(int64_t)c * d + kk]; /* planted: W1 read transposed */
#else
        z += xh[r * d + kk] * (double)w1[(int64_t)kk * 4 * inner + c];
#endif
      }
      s[r * 4 * inner + c] = oracle_silu(z);
    }
  }
  /* 3. split [U|V|Q|K]; 4. full K/V sequence of each user = cached + new */
  kv_off[0] = 0;
  for (int u = 0; u < B; ++u) kv_off[u + 1] = kv_off[u] + start[u] + (q_off[u + 1] - q_off[u]);
  double *kf = (double *)malloc(sizeof(double) * (size_t)(kv_off[B] * inner + 1));
  double *vf = (double *)malloc(sizeof(double) * (size_t)(kv_off[B] * inner + 1));
  double *qn = (double *)malloc(sizeof(double) * (size_t)(n_new * inner + 1));
  if (!kf || !vf || !qn) return ERR_INVALID;
  for (int u = 0; u < B; ++u) {
    for (int64_t j = 0; j < start[u]; ++j)
      for (int c = 0; c < inner; ++c) {
        kf[(kv_off[u] + j) * inner + c] = hist_k[(hist_off[u] + j) * inner + c];
        vf[(kv_off[u] + j) * inner + c] = hist_v[(hist_off[u] + j) * inner + c];
      }
    for (int64_t r = q_off[u]; r < q_off[u + 1]; ++r) {
      int64_t j = start[u] + (r - q_off[u]);
      const double *sr = s + r * 4 * inner;
      for (int c = 0; c < inner; ++c) {
#if ORACLE_MUTANT == 9
        /* planted: Q and K chunks swapped */
        qn[r * inner + c] = sr[3 * inner + c];
        kf[(kv_off[u] + j) * inner + c] = sr[2 * inner + c];
#else
        qn[r * inner + c] = sr[2 * inner + c];
        kf[(kv_off[u] + j) * inner + c] = sr[3 * inner + c];
#endif
        vf[(kv_off[u] + j) * inner + c] = sr[1 * inner + c];
      }
    }
  }
  /* 5. attention */
  {
    double *rabd = (double *)malloc(sizeof(double) * (size_t)num_buckets);
    if (!rabd) return ERR_INVALID;
    for (int b = 0; b < num_buckets; ++b) rabd[b] = (double)rab[b];
    int rc = oracle_attention(B, H, dh, q_off, start, kv_off, n_targets, norm_n, qn, kf, vf,
                              rabd, num_buckets, o);
    free(rabd);
    if (rc != OK) return rc;
  }
  /* 6. LayerNorm over the concatenated heads, gate by U */
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n_new; ++r) {
    double ln[inner];
    oracle_layer_norm(o + r * inner, inner, eps, ln);
    for (int c = 0; c < inner; ++c) {
#if ORACLE_MUTANT == 10
      g[r * inner + c] = ln[c] * s[r * 4 * inner + 1 * inner + c]; /* planted: gate by V */
#else
      g[r * inner + c] = ln[c] * s[r * 4 * inner + 0 * inner + c];
#endif
    }
  }
  /* 7. f2 plus residual */
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n_new; ++r) {
    for (int c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int kk = 0; kk < inner; ++kk) acc += g[r * inner + kk] * (double)w2[(int64_t)kk * d + c];
#if ORACLE_MUTANT == 11
      y[r * d + c] = acc; /* planted: residual dropped */
#else
      y[r * d + c] = x[r * d + c] + acc;
#endif
    }
  }
  for (int64_t r = 0; r < n_new; ++r) {
    int u = 0;
    while (q_off[u + 1] <= r) ++u;
    int64_t j = start[u] + (r - q_off[u]);
    for (int c = 0; c < inner; ++c) {
      if (u_out) u_out[r * inner + c] = s[r * 4 * inner + c];
      if (v_out) v_out[r * inner + c] = vf[(kv_off[u] + j) * inner + c];
      if (q_out) q_out[r * inner + c] = qn[r * inner + c];
      if (k_out) k_out[r * inner + c] = kf[(kv_off[u] + j) * inner + c];
      if (o_out) o_out[r * inner + c] = o[r * inner + c];
      if (g_out) g_out[r * inner + c] = g[r * inner + c];
    }
    if (xhat_out)
      for (int c = 0; c < d; ++c) xhat_out[r * d + c] = xh[r * d + c];
  }
  free(xh); free(s); free(o); free(g); free(kv_off); free(kf); free(vf); free(qn);
  return OK;
}

/* ------------------------------------------------------------------------ */
/* multitask ranking head ("NVIDIA Dynamo-Triton Gets End-to-End HSTU      */
/* Generative Recommender Workflow", section Recommendation as sequence      */
/* modeling: in the HSTU ranking example the blocks process the sequence    */
/* and a prediction head yields multitask ranking outputs).  The pages name */
/* no tasks or head shape; the reading here: for each scored row y (a row   */
/* of the last block's output) and task t, a two-layer perceptron           */
/*   z_t = c_t + sum_j w_t[j] * ReLU(b_t[j] + sum_k y[k] * A_t[k][j])        */
/* with A_t [d][hidden], b_t, w_t [hidden] and c_t; z is the task's logit.   */
/* ------------------------------------------------------------------------ */
int oracle_head(const double *y, int64_t y_rows, int d, const int32_t *rows, int64_t n_rows, int tasks,
                int hidden, const double *a, const double *b, const double *w, const double *c,
                double *logits) {
  if (!y || d <= 0 || tasks <= 0 || hidden <= 0 || n_rows < 0 || (n_rows > 0 && (!rows || !logits)))
    return ERR_INVALID;
  for (int64_t r = 0; r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= y_rows) return ERR_INVALID;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n_rows; ++r) {
#if ORACLE_MUTANT == 16
    const double *yr = y + r * d; /* planted: the row list ignored */
#else
    const double *yr = y + (int64_t)rows[r] * d;
#endif
    for (int t = 0; t < tasks; ++t) {
      const double *at = a + (int64_t)t * d * hidden;
#if ORACLE_MUTANT == 15
      double z = c[0]; /* planted: task 0's output bias for every task */
#else
      double z = c[t];
#endif
      for (int j = 0; j < hidden; ++j) {
#if ORACLE_MUTANT == 13
        double pre = 0.0; /* planted: hidden bias dropped */
#else
        double pre = b[(int64_t)t * hidden + j];
#endif
        for (int k = 0; k < d; ++k) {
#if ORACLE_MUTANT == 14
          pre += yr[k] * at[(int64_t)j * d + k]; /* planted: A_t read transposed */
#else
          pre += yr[k] * at[(int64_t)k * hidden + j];
#endif
        }
#if ORACLE_MUTANT == 12
        double h = pre < 0.0 ? pre : 0.0; /* planted: ReLU's sign flipped */
#else
        double h = pre > 0.0 ? pre : 0.0;
#endif
        z += w[(int64_t)t * hidden + j] * h;
      }
      logits[r * tasks + t] = z;
    }
  }
  return OK;
}

/* ------------------------------------------------------------------------ */
/* backward of one HSTU layer (training: every position of every user is    */
/* computed; no cache)                                                       */
/* ------------------------------------------------------------------------ */
/*
 * Gradients of a scalar loss with dL/dY = dy, by the chain rule through the
 * forward above ("How Generative Recommenders Are Redefining RecSys at
 * Scale", section HSTU support: HSTU training; the forward equations as in
 * oracle_layer):
 *   dW2 = g^T dy,  dg = dy W2^T,  dU = dg * LN(o),  dLN(o) = dg * U
 *   do  = LN'(o) applied to dLN(o):  rstd (dz - mean(dz) - z mean(dz z))
 *   per visible pair (i, j) of a user and head, z = q_i.k_j + rab[b(i-j)]:
 *     dP = do_i . v_j / n,  dv_j += SiLU(z) do_i / n,
 *     dz = dP SiLU'(z) with SiLU'(z) = s(z) (1 + z (1 - s(z))), s = sigmoid,
 *     dq_i += dz k_j,  dk_j += dz q_i,  drab[b(i-j)] += dz
 *   da = [dU|dV|dQ|dK],  ds = da * SiLU'(x^ W1),  dW1 = x^T ds
 *   dx = LN'(x) applied to ds W1^T, plus dy (the residual)
 * Inputs in double: x [N][d], w1 [d][4 inner], w2 [inner][d], rab [nb],
 * dy [N][d]; users' rows by q_off, positions 0.. (start = 0).
 * Outputs: dx [N][d], dw1 [d][4 inner], dw2 [inner][d], drab [nb].
 */
static double sigm(double z) { return 1.0 / (1.0 + exp(-z)); }

static double silu_grad(double z) {
  double s = sigm(z);
#if ORACLE_MUTANT == 17
  return s; /* planted: SiLU' taken as the sigmoid */
#else
  return s * (1.0 + z * (1.0 - s));
#endif
}

/* dx = rstd (dyv - mean(dyv) - yv mean(dyv yv)) for y = LayerNorm(x) = (x - mu) rstd */
static void ln_backward(const double *yv, const double *dyv, int n, double rstd, double *dxv) {
  double m1 = 0.0, m2 = 0.0;
  for (int c = 0; c < n; ++c) {
    m1 += dyv[c];
    m2 += dyv[c] * yv[c];
  }
  m1 /= n;
  m2 /= n;
  for (int c = 0; c < n; ++c) {
#if ORACLE_MUTANT == 18
    dxv[c] = rstd * (dyv[c] - yv[c] * m2); /* planted: the mean term dropped */
#else
    dxv[c] = rstd * (dyv[c] - m1 - yv[c] * m2);
#endif
  }
}

static double row_ln(const double *x, int n, double eps, double *y) {
  double mu = 0.0, var = 0.0;
  for (int c = 0; c < n; ++c) mu += x[c];
  mu /= n;
  for (int c = 0; c < n; ++c) var += (x[c] - mu) * (x[c] - mu);
  var /= n;
  double rstd = 1.0 / sqrt(var + eps);
  for (int c = 0; c < n; ++c) y[c] = (x[c] - mu) * rstd;
  return rstd;
}

int oracle_layer_backward(int B, int d, int H, int dh, double eps, const int64_t *q_off,
                          const int64_t *n_targets, const double *norm_n, const double *x,
                          const double *w1, const double *w2, const double *rab, int num_buckets,
                          const double *dy, double *dx, double *dw1, double *dw2, double *drab) {
  if (B < 0 || d <= 0 || H <= 0 || dh <= 0 || num_buckets <= 0) return ERR_INVALID;
  for (int u = 0; u < B; ++u) {
    int64_t L = q_off[u + 1] - q_off[u];
    if (L < 0 || n_targets[u] < 0 || n_targets[u] > L) return ERR_INVALID;
  }
  const int inner = H * dh, w = 4 * inner;
  const int64_t N = q_off[B];
  size_t nd = (size_t)(N * d + 1), nw = (size_t)(N * w + 1), ni = (size_t)(N * inner + 1);
  double *xh = calloc(nd, sizeof(double)), *xr = calloc((size_t)N + 1, sizeof(double));
  double *z1 = calloc(nw, sizeof(double)), *a = calloc(nw, sizeof(double));
  double *o = calloc(ni, sizeof(double)), *lo = calloc(ni, sizeof(double));
  double *orr = calloc((size_t)N + 1, sizeof(double)), *g = calloc(ni, sizeof(double));
  double *dg = calloc(ni, sizeof(double)), *dov = calloc(ni, sizeof(double));
  double *da = calloc(nw, sizeof(double)), *dxh = calloc(nd, sizeof(double));
  if (!xh || !xr || !z1 || !a || !o || !lo || !orr || !g || !dg || !dov || !da || !dxh) return ERR_INVALID;

  /* forward, keeping what the backward needs */
  for (int64_t r = 0; r < N; ++r) xr[r] = row_ln(x + r * d, d, eps, xh + r * d);
  for (int64_t r = 0; r < N; ++r)
    for (int c = 0; c < w; ++c) {
      double s = 0.0;
      for (int k = 0; k < d; ++k) s += xh[r * d + k] * w1[(int64_t)k * w + c];
      z1[r * w + c] = s;
      a[r * w + c] = s * sigm(s);
    }
  for (int u = 0; u < B; ++u) {
    int64_t r0 = q_off[u], L = q_off[u + 1] - r0, hist = L - n_targets[u];
    for (int h = 0; h < H; ++h)
      for (int64_t i = 0; i < L; ++i) {
        const double *qi = a + (r0 + i) * w + 2 * inner + h * dh;
        double *oi = o + (r0 + i) * inner + h * dh;
        for (int64_t j = 0; j < L; ++j) {
          if (!visible(i, j, hist)) continue;
          const double *kj = a + (r0 + j) * w + 3 * inner + h * dh;
          const double *vj = a + (r0 + j) * w + 1 * inner + h * dh;
          double z = rab[oracle_bucket(i - j, num_buckets)];
          for (int e = 0; e < dh; ++e) z += qi[e] * kj[e];
          double p = z * sigm(z) / norm_n[u];
          for (int e = 0; e < dh; ++e) oi[e] += p * vj[e];
        }
      }
  }
  for (int64_t r = 0; r < N; ++r) {
    orr[r] = row_ln(o + r * inner, inner, eps, lo + r * inner);
    for (int c = 0; c < inner; ++c) g[r * inner + c] = lo[r * inner + c] * a[r * w + c];
  }

  /* f2 and the gate */
  for (int c = 0; c < inner; ++c)
    for (int k = 0; k < d; ++k) {
      double s = 0.0;
      for (int64_t r = 0; r < N; ++r) s += g[r * inner + c] * dy[r * d + k];
      dw2[(int64_t)c * d + k] = s;
    }
  for (int64_t r = 0; r < N; ++r) {
    for (int c = 0; c < inner; ++c) {
      double s = 0.0;
      for (int k = 0; k < d; ++k) s += dy[r * d + k] * w2[(int64_t)c * d + k];
      dg[r * inner + c] = s;
      da[r * w + c] = s * lo[r * inner + c];            /* dU */
    }
    double dln[inner];
    for (int c = 0; c < inner; ++c) dln[c] = dg[r * inner + c] * a[r * w + c];
    ln_backward(lo + r * inner, dln, inner, orr[r], dov + r * inner);
  }

  /* attention */
  for (int b = 0; b < num_buckets; ++b) drab[b] = 0.0;
  for (int u = 0; u < B; ++u) {
    int64_t r0 = q_off[u], L = q_off[u + 1] - r0, hist = L - n_targets[u];
    double n = norm_n[u];
    for (int h = 0; h < H; ++h)
      for (int64_t i = 0; i < L; ++i) {
        const double *qi = a + (r0 + i) * w + 2 * inner + h * dh;
        const double *doi = dov + (r0 + i) * inner + h * dh;
        double *dqi = da + (r0 + i) * w + 2 * inner + h * dh;
        for (int64_t j = 0; j < L; ++j) {
          if (!visible(i, j, hist)) continue;
          const double *kj = a + (r0 + j) * w + 3 * inner + h * dh;
          const double *vj = a + (r0 + j) * w + 1 * inner + h * dh;
          double *dkj = da + (r0 + j) * w + 3 * inner + h * dh;
          double *dvj = da + (r0 + j) * w + 1 * inner + h * dh;
          int bk = oracle_bucket(i - j, num_buckets);
          double z = rab[bk], dp = 0.0;
          for (int e = 0; e < dh; ++e) {
            z += qi[e] * kj[e];
            dp += doi[e] * vj[e];
          }
          dp /= n;
          double p = z * sigm(z);
#if ORACLE_MUTANT == 20
          for (int e = 0; e < dh; ++e) dvj[e] += p * doi[e]; /* planted: 1/n dropped in dV */
#else
          for (int e = 0; e < dh; ++e) dvj[e] += p * doi[e] / n;
#endif
          double dz = dp * silu_grad(z);
          for (int e = 0; e < dh; ++e) {
            dqi[e] += dz * kj[e];
            dkj[e] += dz * qi[e];
          }
#if ORACLE_MUTANT == 19
          drab[oracle_bucket(i - j + 1, num_buckets)] += dz; /* planted: bias gradient to the wrong bucket */
#else
          drab[bk] += dz;
#endif
        }
      }
  }

  /* f1 and the pre-norm */
  for (int64_t r = 0; r < N; ++r)
    for (int c = 0; c < w; ++c) da[r * w + c] *= silu_grad(z1[r * w + c]);
  for (int k = 0; k < d; ++k)
    for (int c = 0; c < w; ++c) {
      double s = 0.0;
      for (int64_t r = 0; r < N; ++r) s += xh[r * d + k] * da[r * w + c];
      dw1[(int64_t)k * w + c] = s;
    }
  for (int64_t r = 0; r < N; ++r) {
    for (int k = 0; k < d; ++k) {
      double s = 0.0;
      for (int c = 0; c < w; ++c) s += da[r * w + c] * w1[(int64_t)k * w + c];
      dxh[r * d + k] = s;
    }
    ln_backward(xh + r * d, dxh + r * d, d, xr[r], dx + r * d);
#if ORACLE_MUTANT != 21
    for (int k = 0; k < d; ++k) dx[r * d + k] += dy[r * d + k];
#endif
    /* (mutant 21, planted: the residual's gradient dropped) */
  }
  free(xh); free(xr); free(z1); free(a); free(o); free(lo); free(orr); free(g);
  free(dg); free(dov); free(da); free(dxh);
  return OK;
}
