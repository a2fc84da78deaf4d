/*
 * norm_oracle.c -- plain double-precision CPU oracle for row-wise LayerNorm and RMSNorm,
 * forward and backward, with an optional residual add in front of the norm.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's CPU-baseline
 * leg may load or call this file. It shares no code, header, table or helper with the HIP
 * library; the two are compared element by element on identical input bits.
 *
 * What is computed is the textbook definition of each operation, evaluated in double
 * precision on the exact input values (bf16, fp16 or fp32 bit patterns widened exactly):
 *
 *   Sources (web pages):
 *   [P1] "PyTorch atinge desempenho SOTA em normalização com torch.compile"
 *        (matsubara.tec.br):
 *        para. 2  -- LayerNorm normalises with the mean and the variance taken along one
 *                    dimension, then scales by the trainable gamma (weight) and shifts by
 *                    beta (bias); RMSNorm uses the root mean square instead and has no beta.
 *        para. 3  -- the forward pass is a reduction along the contiguous dimension plus
 *                    pointwise work.
 *        para. 7  -- the backward pass produces dX, dW and, for LayerNorm, dB.
 *        paras. 8-10 -- fusing, splitting and re-ordering these reductions changes only the
 *                    order of the same sums, not their value; so the oracle is the plain,
 *                    unsplit definition.
 *
 *   [P3] "Towards Free Normalization: Fusing Normalization into GEMM and Attention Kernels"
 *        (brifing.si): items 3-4 and 9-10 -- a norm whose output is the input of a matrix
 *        product, fused into that product; the oracle evaluates the unfused composition.
 *        Item 5 -- norms fused around an attention kernel; the oracle normalises the query
 *        and key vectors, then evaluates softmax attention from its definition.
 *
 *   Readings taken where the pages say nothing (each is also listed in the design notes):
 *     - variance is the biased estimator (divide by N);
 *     - eps is added inside the square root, for both kinds;
 *     - RMSNorm subtracts no mean and has no bias;
 *     - the backward takes X and recomputes its own mean and rstd (it never uses a saved
 *       statistic from the device);
 *     - residual variant: h = R + X is rounded once to the input dtype (RNE) and the norm is
 *       applied to that rounded h, because the backward re-reads the stored h; the residual
 *       gradient equals the input gradient, plus an optional incoming gradient of h.
 *
 * Parallelism: rows (forward, dX) and column blocks (dW, dB) are split over OpenMP threads.
 * Every output value is computed by exactly one thread in the definition's own order (rows
 * ascending for the column sums), so results do not depend on the thread count.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -fPIC -shared (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_LAYERNORM = 0, OR_RMSNORM = 1 };
/* attention without a norm on its queries and keys (the unfused composition's second step) */
enum { OR_NO_NORM = -1 };
/* dtype: the storage type of every tensor, or OR_BF16_F32W / OR_F16_F32W = bf16 / fp16
 * activations and gradients (X, R, dY, dH) with fp32 weight and bias (their gradients are then
 * fp32 too). */
enum { OR_F32 = 0, OR_BF16 = 1, OR_BF16_F32W = 2, OR_F16 = 3, OR_F16_F32W = 4 };

enum {
  OR_OK = 0,
  OR_BAD_ARG = 1,
  OR_NO_MEMORY = 2,
};

/* ---- number formats ---------------------------------------------------------------- */

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
static double or_bf16_bits_to_double(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. Normal values are
 * (1024 + f) * 2^(e - 25), subnormals f * 2^-24; e = 31 holds the infinities and NaNs. */
static double or_f16_bits_to_double(uint16_t b) {
  const int sign = b >> 15, e = (b >> 10) & 31, f = b & 1023;
  double v;
  if (e == 31)
    v = f ? NAN : INFINITY;
  else if (e == 0)
    v = ldexp((double)f, -24);
  else
    v = ldexp((double)(1024 + f), e - 25);
  return sign ? -v : v;
}

static double or_load(int dtype, const void *base, int64_t idx) {
  if (dtype == OR_F32) {
    float f;
    memcpy(&f, (const char *)base + idx * 4, sizeof f);
    return (double)f;
  }
  uint16_t b;
  memcpy(&b, (const char *)base + idx * 2, sizeof b);
  return dtype == OR_F16 ? or_f16_bits_to_double(b) : or_bf16_bits_to_double(b);
}

/* Round a double to the nearest bf16 value, ties to even, in one step from the double
 * (no detour through binary32). bf16 keeps 8 significant bits and binary32's exponent range;
 * the smallest subnormal step is 2^-133 and the largest finite value is (2 - 2^-7) * 2^127. */
static double or_round_to_bf16(double v) {
  if (v != v || v == 0.0 || isinf(v)) return v;
  double a = fabs(v);
  int e;
  (void)frexp(a, &e);      /* a = m * 2^e with m in [0.5, 1) */
  int q = e - 8;           /* weight of the last kept bit */
  if (q < -133) q = -133;  /* subnormal range: fixed step */
  double r = nearbyint(ldexp(a, -q)); /* default rounding mode: to nearest, ties to even */
  double out = ldexp(r, q);
  if (out > 3.3895313892515355e38) out = INFINITY;
  return v < 0 ? -out : out;
}

/* Round a double to the nearest fp16 value, ties to even, in one step from the double. fp16
 * keeps 11 significant bits; the smallest subnormal step is 2^-24 and the largest finite value
 * 65504 = (2 - 2^-10) * 2^15; what rounds beyond it becomes infinity. */
static double or_round_to_f16(double v) {
  if (v != v || v == 0.0 || isinf(v)) return v;
  double a = fabs(v);
  int e;
  (void)frexp(a, &e);     /* a = m * 2^e with m in [0.5, 1) */
  int q = e - 11;         /* weight of the last kept bit */
  if (q < -24) q = -24;   /* subnormal range: fixed step */
  double k = nearbyint(ldexp(a, -q));
  double out = ldexp(k, q);
  if (out > 65504.0) out = INFINITY;
  return v < 0 ? -out : out;
}

/* storage type of the activations, and of the weight and bias, for a call's dtype */
static int or_act(int dtype) {
  return dtype == OR_BF16_F32W ? OR_BF16 : dtype == OR_F16_F32W ? OR_F16 : dtype;
}
static int or_wt(int dtype) {
  return (dtype == OR_BF16_F32W || dtype == OR_F16_F32W) ? OR_F32 : dtype;
}

static double or_round_to_dtype(int dtype, double v) {
  if (dtype == OR_F32) return (double)(float)v; /* C conversion: round to nearest even */
  if (dtype == OR_F16) return or_round_to_f16(v);
  return or_round_to_bf16(v);
}

/* bit pattern of the fp16 nearest to v (used by tests to pin the rounding rule) */
static uint16_t or_f16_bits(double v) {
  if (v != v) return (uint16_t)0x7E00;
  const double r = or_round_to_f16(v);
  const uint16_t sign = signbit(r) ? 0x8000 : 0;
  const double a = fabs(r);
  if (isinf(a)) return sign | 0x7C00;
  if (a < ldexp(1.0, -14)) return sign | (uint16_t)ldexp(a, 24); /* subnormal or zero */
  int e;
  const double m = frexp(a, &e); /* a = m * 2^e, m in [0.5, 1): biased exponent e + 14 */
  return sign | (uint16_t)((e + 14) << 10) | (uint16_t)(ldexp(m, 11) - 1024.0);
}

/* bit pattern of the bf16 nearest to v (used by tests to pin the rounding rule) */
static uint16_t or_bf16_bits(double v) {
  float f = (float)or_round_to_bf16(v); /* exact: the value is a bf16, hence a binary32 */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if (v != v) return (uint16_t)0x7FC0;
  return (uint16_t)(u >> 16);
}

/* ---- argument checks ----------------------------------------------------------------- */

static int or_check(int kind, int dtype, int64_t M, int64_t N, int64_t r0, int64_t r1,
                    double eps) {
  if (kind != OR_LAYERNORM && kind != OR_RMSNORM) return OR_BAD_ARG;
  if (dtype < OR_F32 || dtype > OR_F16_F32W) return OR_BAD_ARG;
  if (M < 0 || N <= 0) return OR_BAD_ARG;
  if (r0 < 0 || r1 < r0 || r1 > M) return OR_BAD_ARG;
  if (!(eps >= 0.0)) return OR_BAD_ARG;
  return OR_OK;
}

/* ---- per-row pieces -------------------------------------------------------------------- */

/* Row i of the norm's input, in double: X, or round(R + X) for the residual variant. */
static void or_input_row(int dtype, int64_t N, int64_t i, const void *X, const void *R,
                         double *x) {
  for (int64_t j = 0; j < N; ++j) {
    double v = or_load(dtype, X, i * N + j);
    if (R) v = or_round_to_dtype(dtype, or_load(dtype, R, i * N + j) + v);
    x[j] = v;
  }
}

/* Statistics of one row [P1 para. 2]. LayerNorm: mean, then the biased variance as the mean
 * of squared deviations from that mean (two passes). RMSNorm: mean of squares, mean = 0.
 * rstd = 1 / sqrt(statistic + eps). */
static void or_row_stats(int kind, int64_t N, const double *x, double eps, double *mean,
                         double *rstd) {
  if (kind == OR_LAYERNORM) {
    double s = 0.0;
    for (int64_t j = 0; j < N; ++j) s += x[j];
    double mu = s / (double)N;
    double q = 0.0;
    for (int64_t j = 0; j < N; ++j) q += (x[j] - mu) * (x[j] - mu);
    double var = q / (double)N;
    *mean = mu;
    *rstd = 1.0 / sqrt(var + eps);
  } else {
    double q = 0.0;
    for (int64_t j = 0; j < N; ++j) q += x[j] * x[j];
    double ms = q / (double)N;
    *mean = 0.0;
    *rstd = 1.0 / sqrt(ms + eps);
  }
}

/* ---- forward ------------------------------------------------------------------------- */

/*
 * Forward over rows [r0, r1) of an M x N row-major input.
 *   X     : input bits (the activation type of dtype), M*N
 *   R     : residual bits (activation type), M*N, or NULL
 *   W     : weight bits (the weight type of dtype), N
 *   B     : bias bits (weight type), N, or NULL (LayerNorm only; NULL means zero bias)
 *   Y     : out, (r1-r0)*N doubles, unrounded
 *   H     : out, (r1-r0)*N doubles holding round(R + X), or NULL (only with R)
 *   mean  : out, (r1-r0) doubles, or NULL (0 for RMSNorm)
 *   rstd  : out, (r1-r0) doubles, or NULL
 * Returns 0, or nonzero on a bad argument / allocation failure.
 */
int oracle_fwd_rows(int kind, int dtype, int64_t M, int64_t N, int64_t r0, int64_t r1,
                    const void *X, const void *R, const void *W, const void *B, double eps,
                    double *Y, double *H, double *mean, double *rstd) {
  int st = or_check(kind, dtype, M, N, r0, r1, eps);
  if (st) return st;
  if (!X || !W || !Y) return OR_BAD_ARG;
  if (kind == OR_RMSNORM && B) return OR_BAD_ARG;
  if (H && !R) return OR_BAD_ARG;
  int fail = 0;
#pragma omp parallel
  {
    double *x = (double *)malloc((size_t)N * sizeof(double));
    if (!x) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for schedule(static)
    for (int64_t i = r0; i < r1; ++i) {
      if (!x) continue;
      int64_t o = i - r0;
      or_input_row(or_act(dtype), N, i, X, R, x);
      if (H)
        for (int64_t j = 0; j < N; ++j) H[o * N + j] = x[j];
      double mu, rs;
      or_row_stats(kind, N, x, eps, &mu, &rs);
      for (int64_t j = 0; j < N; ++j) {
        double w = or_load(or_wt(dtype), W, j);
        double b = B ? or_load(or_wt(dtype), B, j) : 0.0;
        double xhat = (kind == OR_LAYERNORM) ? (x[j] - mu) * rs : x[j] * rs;
        Y[o * N + j] = (kind == OR_LAYERNORM) ? xhat * w + b : xhat * w;
      }
      if (mean) mean[o] = mu;
      if (rstd) rstd[o] = rs;
    }
    free(x);
  }
  return fail ? OR_NO_MEMORY : OR_OK;
}

/* ---- backward ------------------------------------------------------------------------ */

/*
 * Backward over rows [r0, r1) [P1 para. 7].
 *   X   : the norm's input bits (for the residual variant: the stored h), M*N
 *   dY  : gradient of the norm output, M*N
 *   dH  : optional incoming gradient of the residual output h, M*N, added to dX; or NULL
 *   W   : weight bits, N
 *   dX  : out, (r1-r0)*N doubles, or NULL (the residual gradient dR is the same array)
 *   dW  : out, N doubles: sum over rows r0..r1-1 of dY * xhat, or NULL
 *   dB  : out, N doubles: sum over rows r0..r1-1 of dY (LayerNorm only), or NULL
 *
 * With g = dY * w, xhat the normalised input and rstd the row's 1/sqrt(stat + eps):
 *   LayerNorm: dX = rstd * (g - mean_j(g) - xhat * mean_j(g * xhat))
 *   RMSNorm  : dX = rstd * (g - xhat * mean_j(g * xhat))
 * These are the derivatives of the forward definitions above with the statistics treated
 * as functions of the row.
 */
int oracle_bwd_rows(int kind, int dtype, int64_t M, int64_t N, int64_t r0, int64_t r1,
                    const void *X, const void *dY, const void *dH, const void *W, double eps,
                    double *dX, double *dW, double *dB) {
  int st = or_check(kind, dtype, M, N, r0, r1, eps);
  if (st) return st;
  if (!X || !dY || !W) return OR_BAD_ARG;
  if (kind == OR_RMSNORM && dB) return OR_BAD_ARG;
  int64_t rows = r1 - r0;
  double *mu = (double *)malloc((size_t)(rows > 0 ? rows : 1) * sizeof(double));
  double *rs = (double *)malloc((size_t)(rows > 0 ? rows : 1) * sizeof(double));
  if (!mu || !rs) {
    free(mu);
    free(rs);
    return OR_NO_MEMORY;
  }
  int fail = 0;

  /* per-row statistics and dX */
#pragma omp parallel
  {
    double *x = (double *)malloc((size_t)N * sizeof(double));
    double *xh = (double *)malloc((size_t)N * sizeof(double));
    double *g = (double *)malloc((size_t)N * sizeof(double));
    if (!x || !xh || !g) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for schedule(static)
    for (int64_t i = r0; i < r1; ++i) {
      if (!x || !xh || !g) continue;
      int64_t o = i - r0;
      or_input_row(or_act(dtype), N, i, X, NULL, x);
      or_row_stats(kind, N, x, eps, &mu[o], &rs[o]);
      if (!dX) continue;
      double sg = 0.0, sgx = 0.0;
      for (int64_t j = 0; j < N; ++j) {
        xh[j] = (kind == OR_LAYERNORM) ? (x[j] - mu[o]) * rs[o] : x[j] * rs[o];
        g[j] = or_load(or_act(dtype), dY, i * N + j) * or_load(or_wt(dtype), W, j);
        sg += g[j];
        sgx += g[j] * xh[j];
      }
      double c1 = sg / (double)N;
      double c2 = sgx / (double)N;
      for (int64_t j = 0; j < N; ++j) {
        double d = (kind == OR_LAYERNORM) ? rs[o] * (g[j] - c1 - xh[j] * c2)
                                          : rs[o] * (g[j] - xh[j] * c2);
        if (dH) d += or_load(or_act(dtype), dH, i * N + j);
        dX[o * N + j] = d;
      }
    }
    free(x);
    free(xh);
    free(g);
  }

  /* column sums dW = sum_i dY*xhat and dB = sum_i dY, rows in ascending order */
  if (!fail && (dW || dB)) {
#pragma omp parallel
    {
      int nt = 1, t = 0;
#ifdef _OPENMP
      nt = omp_get_num_threads();
      t = omp_get_thread_num();
#endif
      int64_t per = (N + nt - 1) / nt;
      int64_t j0 = (int64_t)t * per;
      int64_t j1 = j0 + per < N ? j0 + per : N;
      if (j0 < j1) {
        int64_t w = j1 - j0;
        double *aw = (double *)calloc((size_t)w, sizeof(double));
        double *ab = (double *)calloc((size_t)w, sizeof(double));
        if (!aw || !ab) {
#pragma omp atomic write
          fail = 1;
        } else {
          for (int64_t i = r0; i < r1; ++i) {
            int64_t o = i - r0;
            for (int64_t j = j0; j < j1; ++j) {
              double x = or_load(or_act(dtype), X, i * N + j);
              double xhat = (kind == OR_LAYERNORM) ? (x - mu[o]) * rs[o] : x * rs[o];
              double dy = or_load(or_act(dtype), dY, i * N + j);
              aw[j - j0] += dy * xhat;
              ab[j - j0] += dy;
            }
          }
          for (int64_t j = j0; j < j1; ++j) {
            if (dW) dW[j] = aw[j - j0];
            if (dB) dB[j] = ab[j - j0];
          }
        }
        free(aw);
        free(ab);
      }
    }
  }
  free(mu);
  free(rs);
  return fail ? OR_NO_MEMORY : OR_OK;
}

/* ---- the norm followed by a linear projection ---------------------------------------- */

/*
 * out = Norm(X) * L^T + c over rows [r0, r1): a pre-norm projection, the operation that a
 * normalisation fused into the following matrix product ("Towards Free Normalization: Fusing
 * Normalization into GEMM and Attention Kernels", brifing.si, items 3-4 and 9-10) has to
 * reproduce. Evaluated as its definition: the row's normalised output in double (the forward
 * above, with gamma and beta, unrounded), then one dot product with each row of L.
 *   X     : M*K input bits (the activation type of dtype)
 *   W, B  : the norm's gamma and beta (the weight type of dtype), K each; B may be NULL
 *   L     : Nout*K projection bits (the activation type of dtype), row j = output column j
 *   c     : Nout fp32 projection bias, or NULL (zero)
 *   out   : (r1-r0)*Nout doubles, unrounded
 */
int oracle_norm_linear_rows(int kind, int dtype, int64_t M, int64_t K, int64_t Nout,
                            int64_t r0, int64_t r1, const void *X, const void *W,
                            const void *B, const void *L, const float *c, double eps,
                            double *out) {
  int st = or_check(kind, dtype, M, K, r0, r1, eps);
  if (st) return st;
  if (Nout <= 0 || !X || !W || !L || !out) return OR_BAD_ARG;
  if (kind == OR_RMSNORM && B) return OR_BAD_ARG;
  const int64_t n = r1 - r0;
  double *y = (double *)malloc((size_t)(n ? n : 1) * (size_t)K * sizeof(double));
  if (!y) return OR_NO_MEMORY;
  st = oracle_fwd_rows(kind, dtype, M, K, r0, r1, X, NULL, W, B, eps, y, NULL, NULL, NULL);
  if (st) {
    free(y);
    return st;
  }
  const int act = or_act(dtype);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < Nout; ++j) {
    for (int64_t o = 0; o < n; ++o) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k) acc += y[o * K + k] * or_load(act, L, j * K + k);
      out[o * Nout + j] = acc + (c ? (double)c[j] : 0.0);
    }
  }
  free(y);
  return OR_OK;
}

/* ---- norms on the queries and keys of an attention ----------------------------------- */

/* One query or key vector of D bf16 values at Xb + off, normalised like a row of length D
 * (or copied, for OR_NO_NORM) with the D-entry gamma W and beta B (bf16 bits; B may be NULL). */
static void or_qk_row(int kind, int64_t D, const void *Xb, int64_t off, const void *W,
                      const void *B, double eps, double *out) {
  for (int64_t d = 0; d < D; ++d) out[d] = or_load(OR_BF16, Xb, off + d);
  if (kind == OR_NO_NORM) return;
  double mu, rs;
  or_row_stats(kind, D, out, eps, &mu, &rs);
  for (int64_t d = 0; d < D; ++d) {
    double w = or_load(OR_BF16, W, d);
    double b = B ? or_load(OR_BF16, B, d) : 0.0;
    out[d] = (kind == OR_LAYERNORM) ? (out[d] - mu) * rs * w + b : out[d] * rs * w;
  }
}

/*
 * Attention whose queries and keys are normalised first [P3 item 5: norms fused around an
 * attention kernel]. Reading: the norm applies to every query vector and every key vector of
 * every head along the head dimension D (QK-norm), with one gamma (and, for LayerNorm, beta)
 * of D entries for the queries and one for the keys, shared by all heads; V is used as given.
 * Then, per query head, softmax attention by its definition:
 *   logit(i, j) = scale * sum_d q'(i, d) k'(j, d),  over keys j visible to query i
 *                 (all S keys, or j <= i when causal),
 *   O(i, :)     = sum_j softmax_j(logit(i, .)) V(j, :),
 *   lse(i)      = log sum_j exp(logit(i, j)).
 * Grouped heads: query head h reads key and value head h / (Hq / Hk).
 *
 * Layout: Q [B][S][Hq][D], K and V [B][S][Hk][D], all bf16 bits; Wq, Bq, Wk, Bk D bf16 bits
 * each (Bq, Bk NULL for RMSNorm; all four NULL for OR_NO_NORM). Computes query positions
 * s0 .. s1-1 of batch b and query head h:
 *   O   : out, (s1-s0)*D doubles, unrounded
 *   lse : out, (s1-s0) doubles, or NULL
 * Returns 0, or nonzero on a bad argument / allocation failure.
 */
int oracle_norm_attention(int kind, int64_t B, int64_t S, int64_t Hq, int64_t Hk, int64_t D,
                          int64_t b, int64_t h, int64_t s0, int64_t s1, const void *Q,
                          const void *K, const void *V, const void *Wq, const void *Bq,
                          const void *Wk, const void *Bk, double eps, double scale, int causal,
                          double *O, double *lse) {
  if (kind != OR_LAYERNORM && kind != OR_RMSNORM && kind != OR_NO_NORM) return OR_BAD_ARG;
  if (B <= 0 || S <= 0 || Hq <= 0 || Hk <= 0 || D <= 0 || Hq % Hk != 0) return OR_BAD_ARG;
  if (b < 0 || b >= B || h < 0 || h >= Hq || s0 < 0 || s1 < s0 || s1 > S) return OR_BAD_ARG;
  if (!Q || !K || !V || !O || !(eps >= 0.0)) return OR_BAD_ARG;
  if (kind == OR_NO_NORM && (Wq || Bq || Wk || Bk)) return OR_BAD_ARG;
  if (kind != OR_NO_NORM && (!Wq || !Wk)) return OR_BAD_ARG;
  if (kind == OR_RMSNORM && (Bq || Bk)) return OR_BAD_ARG;
  const int64_t hk = h / (Hq / Hk);
  const int64_t nk = causal ? s1 : S; /* keys any of these queries sees */
  double *kn = (double *)malloc((size_t)(nk ? nk : 1) * (size_t)D * sizeof(double));
  if (!kn) return OR_NO_MEMORY;
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < nk; ++j)
    or_qk_row(kind, D, K, ((b * S + j) * Hk + hk) * D, Wk, Bk, eps, kn + j * D);
  int fail = 0;
#pragma omp parallel
  {
    double *qn = (double *)malloc((size_t)D * sizeof(double));
    double *p = (double *)malloc((size_t)(nk ? nk : 1) * sizeof(double));
    if (!qn || !p) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for schedule(static)
    for (int64_t i = s0; i < s1; ++i) {
      if (!qn || !p) continue;
      or_qk_row(kind, D, Q, ((b * S + i) * Hq + h) * D, Wq, Bq, eps, qn);
      const int64_t n = causal ? i + 1 : S;
      double mx = -INFINITY;
      for (int64_t j = 0; j < n; ++j) {
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += qn[d] * kn[j * D + d];
        p[j] = scale * dot;
        if (p[j] > mx) mx = p[j];
      }
      /* softmax with its largest logit taken out of every exponent (the same ratios) */
      double z = 0.0;
      for (int64_t j = 0; j < n; ++j) {
        p[j] = exp(p[j] - mx);
        z += p[j];
      }
      for (int64_t d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int64_t j = 0; j < n; ++j)
          acc += p[j] * or_load(OR_BF16, V, ((b * S + j) * Hk + hk) * D + d);
        O[(i - s0) * D + d] = acc / z;
      }
      if (lse) lse[i - s0] = mx + log(z);
    }
    free(qn);
    free(p);
  }
  free(kn);
  return fail ? OR_NO_MEMORY : OR_OK;
}

/* ---- helpers exposed for pins ---------------------------------------------------------- */

/* Widen count values of the given dtype to double. */
int oracle_decode(int dtype, const void *bits, int64_t count, double *out) {
  if ((dtype != OR_F32 && dtype != OR_BF16 && dtype != OR_F16) || count < 0 ||
      (count && (!bits || !out)))
    return OR_BAD_ARG;
  for (int64_t k = 0; k < count; ++k) out[k] = or_load(dtype, bits, k);
  return OR_OK;
}

/* Round count doubles to bf16 bit patterns (nearest, ties to even). */
int oracle_round_bf16(const double *in, int64_t count, uint16_t *out) {
  if (count < 0 || (count && (!in || !out))) return OR_BAD_ARG;
  for (int64_t k = 0; k < count; ++k) out[k] = or_bf16_bits(in[k]);
  return OR_OK;
}

/* Round count doubles to fp16 bit patterns (nearest, ties to even). */
int oracle_round_f16(const double *in, int64_t count, uint16_t *out) {
  if (count < 0 || (count && (!in || !out))) return OR_BAD_ARG;
  for (int64_t k = 0; k < count; ++k) out[k] = or_f16_bits(in[k]);
  return OR_OK;
}

/* Number of OpenMP threads a parallel region will use (1 without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Set the OpenMP thread count for later calls (ignored without OpenMP). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
