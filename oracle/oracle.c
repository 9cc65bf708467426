/*
 * oracle.c — plain, slow, fp64 CPU oracle for the max-shifted log-sum-exp family.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
 * in __graft_entry__.py and the CPU-baseline leg of bench.py may load or call
 * this library.  It shares no code, header, table or helper with the HIP path
 * under log_softmax_reductions_amd/csrc, and neither side includes the other.
 *
 * Every function takes the same fp32 arrays the GPU path receives, widens each
 * element to double and evaluates the plain definition written out, with one
 * OpenMP loop over independent outputs (rows, output elements or samples) and
 * nothing else reordered.  glibc's double exp/log/tanh/sqrt are used as-is.
 *
 * Sources (three kernel-benchmark transcripts, cited by page and passage):
 *   [LSE0]  POPCORNBENCH FW-GLM-5-1 l1_p29, "torch.logsumexp(x, dim=0)" for an
 *           (R,B,D) tensor: task statement and the per-(b,d) max / sum / log plan.
 *   [LSM]   POPCORNBENCH Kimi-K2.6 l1_p24, "LogSoftmax over dim=1": the opening
 *           formula x_i - max - log sum exp(x_j - max), the online recurrence
 *           and the pairwise (max, sum) combine, and the multi-block-per-row idea.
 *   [CHAIN] POPCORNBENCH Kimi-K2.6 l2_p92, "Conv2d -> GroupNorm -> Tanh ->
 *           Hardswish -> residual add -> LogSumExp(dim=1)": the model's forward,
 *           the GroupNorm definition (population variance per (sample, group))
 *           and the Hardswish formula x * relu6(x + 3) / 6.
 *
 * Non-finite conventions (the pages leave them open; these are the readings of
 * log(sum(exp(x))) taken literally):
 *   - an entry equal to -inf contributes exp(-inf) = 0, i.e. it is ignored;
 *   - all entries -inf:   LSE = log(0) = -inf;
 *   - any entry +inf:     LSE = +inf (unless a NaN is present);
 *   - any entry NaN:      LSE = NaN.
 *   log_softmax is x - LSE(row) elementwise, so an all -inf row gives NaN and a
 *   row holding +inf gives -inf at finite entries and NaN at the +inf entries.
 *
 * Status: every function returns 0 on success and a negative value on a bad
 * argument (null pointer, negative size); nothing is allocated except the
 * per-sample conv scratch of oracle_fused_chain (freed before return).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_BAD_ARG (-1)
#define ORACLE_NO_MEM (-2)

static int clamp_threads(int nthreads) { return nthreads < 1 ? 1 : nthreads; }

/* log(sum_i exp(p[i*stride])) for n values, by the plain definition with the
 * largest finite-or-infinite value factored out so that exp never overflows:
 *   LSE = M + log(sum_i exp(v_i - M)),  M = max_i v_i.       [LSE0] task plan
 * M = -inf means every term is exp(-inf) = 0; M = +inf means the sum itself is
 * +inf; a NaN anywhere makes the sum NaN. */
static double lse_strided(const float *p, int64_t n, int64_t stride) {
  int has_nan = 0;
  double m = -INFINITY;
  for (int64_t i = 0; i < n; ++i) {
    double v = (double)p[i * stride];
    if (isnan(v))
      has_nan = 1;
    else if (v > m)
      m = v;
  }
  if (has_nan) return NAN;
  if (isinf(m)) return m;
  double s = 0.0;
  for (int64_t i = 0; i < n; ++i) s += exp((double)p[i * stride] - m);
  return m + log(s);
}

/* O1 — logsumexp over the leading axis of a row-major (R, inner) array:
 *   out[j] = log(sum_{r<R} exp(x[r*inner + j])).        [LSE0] task statement
 * An (R,B,D) tensor reduced over dim 0 is the case inner = B*D. */
int oracle_lse_axis0(const float *x, int64_t R, int64_t inner, double *out,
                     int nthreads) {
  if (!x || !out || R < 1 || inner < 0) return ORACLE_BAD_ARG;
#pragma omp parallel for schedule(static) num_threads(clamp_threads(nthreads))
  for (int64_t j = 0; j < inner; ++j) out[j] = lse_strided(x + j, R, inner);
  return 0;
}

/* O2 — row-wise log_softmax of a row-major (rows, cols) array:
 *   lse[r]  = log(sum_c exp(x[r,c]))
 *   y[r,c]  = x[r,c] - lse[r]                       [LSM] opening formula
 * Either output pointer may be NULL when that output is not wanted. */
int oracle_log_softmax_rows(const float *x, int64_t rows, int64_t cols,
                            double *y, double *lse, int nthreads) {
  if (!x || rows < 0 || cols < 1 || (!y && !lse)) return ORACLE_BAD_ARG;
#pragma omp parallel for schedule(dynamic, 1) num_threads(clamp_threads(nthreads))
  for (int64_t r = 0; r < rows; ++r) {
    const float *row = x + r * cols;
    double L = lse_strided(row, cols, 1);
    if (lse) lse[r] = L;
    if (y) {
      double *yr = y + r * cols;
      for (int64_t c = 0; c < cols; ++c) yr[c] = (double)row[c] - L;
    }
  }
  return 0;
}

/* O2b — row-wise softmax, the non-log form:
 *   y[r,c] = exp(x[r,c] - lse[r]) = exp(x[r,c]) / sum_c exp(x[r,c])
 * [LSM] the standard-softmax variant it mentions (write exp(x - max), then
 * divide by the sum). */
int oracle_softmax_rows(const float *x, int64_t rows, int64_t cols, double *y,
                        int nthreads) {
  if (!x || !y || rows < 0 || cols < 1) return ORACLE_BAD_ARG;
#pragma omp parallel for schedule(dynamic, 1) num_threads(clamp_threads(nthreads))
  for (int64_t r = 0; r < rows; ++r) {
    const float *row = x + r * cols;
    const double L = lse_strided(row, cols, 1);
    double *yr = y + r * cols;
    for (int64_t c = 0; c < cols; ++c) yr[c] = exp((double)row[c] - L);
  }
  return 0;
}

/* O1b — logsumexp over the middle axis of a row-major (outer, R, inner) array:
 *   out[o, j] = log(sum_r exp(x[o, r, j]))
 * outer = 1 is O1; the chain's channel reduction of an (N, C, H, W) tensor is
 * outer = N, R = C, inner = H * W.     [LSE0] task statement, [CHAIN] the
 * logsumexp over dim 1 of the residual sum. */
int oracle_lse_axis(const float *x, int64_t outer, int64_t R, int64_t inner,
                    double *out, int nthreads) {
  if (!x || !out || outer < 0 || R < 1 || inner < 0) return ORACLE_BAD_ARG;
#pragma omp parallel for schedule(static) num_threads(clamp_threads(nthreads))
  for (int64_t i = 0; i < outer * inner; ++i) {
    const int64_t o = i / inner, j = i - o * inner;
    out[i] = lse_strided(x + o * R * inner + j, R, inner);
  }
  return 0;
}

/* O2c — log_softmax over the middle axis of (outer, R, inner):
 *   y[o, r, j] = x[o, r, j] - log(sum_r' exp(x[o, r', j]))      [LSM] formula */
int oracle_log_softmax_axis(const float *x, int64_t outer, int64_t R,
                            int64_t inner, double *y, int nthreads) {
  if (!x || !y || outer < 0 || R < 1 || inner < 0) return ORACLE_BAD_ARG;
#pragma omp parallel for schedule(static) num_threads(clamp_threads(nthreads))
  for (int64_t i = 0; i < outer * inner; ++i) {
    const int64_t o = i / inner, j = i - o * inner;
    const float *base = x + o * R * inner + j;
    const double L = lse_strided(base, R, inner);
    for (int64_t r = 0; r < R; ++r)
      y[(o * R + r) * inner + j] = (double)base[r * inner] - L;
  }
  return 0;
}

/* O3a — the (max, sum) pair of every chunk of every row.       [LSM] the
 * multi-block-per-row idea: each block reduces a portion of the row to its
 * local max and sum, which a second phase combines.
 *   chunk k of row r covers columns [k*chunk, min((k+1)*chunk, cols));
 *   m[r,k] = largest non-NaN entry of the chunk (-inf when there is none);
 *   s[r,k] = sum over the chunk of exp(x - m): 0 when m = -inf (all terms are
 *            exp(-inf)); otherwise an entry equal to m counts exactly 1 (so a
 *            chunk holding +inf gives s = the number of +inf entries); NaN when
 *            the chunk holds a NaN.
 * Hence LSE(chunk) = m + log(s) in every case.  nchunks = ceil(cols / chunk). */
int oracle_lse_chunk_partials(const float *x, int64_t rows, int64_t cols,
                              int64_t chunk, double *m_out, double *s_out,
                              int nthreads) {
  if (!x || !m_out || !s_out || rows < 0 || cols < 1 || chunk < 1)
    return ORACLE_BAD_ARG;
  const int64_t nchunks = (cols + chunk - 1) / chunk;
#pragma omp parallel for schedule(dynamic, 1) num_threads(clamp_threads(nthreads))
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t k = 0; k < nchunks; ++k) {
      const int64_t c0 = k * chunk;
      const int64_t c1 = (c0 + chunk < cols) ? c0 + chunk : cols;
      const float *p = x + r * cols;
      double m = -INFINITY;
      int has_nan = 0;
      for (int64_t c = c0; c < c1; ++c) {
        double v = (double)p[c];
        if (isnan(v))
          has_nan = 1;
        else if (v > m)
          m = v;
      }
      double s = 0.0;
      if (has_nan) {
        s = NAN;
      } else if (m == -INFINITY) {
        s = 0.0; /* every term is exp(-inf) = 0 */
      } else {
        for (int64_t c = c0; c < c1; ++c) {
          double v = (double)p[c];
          s += (v == m) ? 1.0 : exp(v - m);
        }
      }
      m_out[r * nchunks + k] = m;
      s_out[r * nchunks + k] = s;
    }
  }
  return 0;
}

/* O3b — merge k (max, sum) pairs per row into the row's logsumexp.  [LSM] the
 * pairwise combine (m1,s1),(m2,s2) -> (M, s1*exp(m1-M) + s2*exp(m2-M)) with
 * M = max(m1,m2), applied to all k pairs at once:
 *   M = max_k m_k;  S = sum_k s_k * w_k,  w_k = 1 if m_k == M else exp(m_k - M);
 *   lse = M + log(S).
 * Writing w_k = 1 for m_k == M is the literal value exp(0) and keeps the
 * identity (-inf, 0) and (+inf, n) pairs free of inf - inf.  A NaN in any m or
 * s makes the result NaN.  Either output pointer M_out / S_out may be NULL. */
int oracle_lse_merge(const double *m, const double *s, int64_t rows, int64_t k,
                     double *lse, double *M_out, double *S_out) {
  if (!m || !s || !lse || rows < 0 || k < 1) return ORACLE_BAD_ARG;
  for (int64_t r = 0; r < rows; ++r) {
    const double *mr = m + r * k, *sr = s + r * k;
    double M = -INFINITY;
    int has_nan = 0;
    for (int64_t i = 0; i < k; ++i) {
      if (isnan(mr[i]) || isnan(sr[i]))
        has_nan = 1;
      else if (mr[i] > M)
        M = mr[i];
    }
    double S = 0.0;
    if (has_nan) {
      M = NAN;
      S = NAN;
    } else {
      for (int64_t i = 0; i < k; ++i)
        S += sr[i] * ((mr[i] == M) ? 1.0 : exp(mr[i] - M));
    }
    if (M_out) M_out[r] = M;
    if (S_out) S_out[r] = S;
    lse[r] = has_nan ? NAN : (isinf(M) ? M : M + log(S));
  }
  return 0;
}

/* Hardswish as the chain's page writes it: h(t) = t * relu6(t + 3) / 6,
 * relu6(u) = min(max(u, 0), 6).                                     [CHAIN] */
double oracle_hardswish(double t) {
  double u = t + 3.0;
  if (u < 0.0) u = 0.0;
  if (u > 6.0) u = 6.0;
  return t * u / 6.0;
}

/* Direct cross-correlation with bias, nn.Conv2d semantics with stride 1, no
 * padding, dilation 1, one group:                 [CHAIN] the conv's shapes
 *   conv[n,o,h,w] = b[o] + sum_{c<Cin, i<K, j<K} W[o,c,i,j] * x[n,c,h+i,w+j]
 * for h < H-K+1, w < W-K+1, written to a double array of shape
 * (N, Cout, H-K+1, W-K+1).  b may be NULL (no bias). */
static void conv_one_sample(const float *xn, const float *w, const float *b,
                            int64_t Cin, int64_t H, int64_t W, int64_t Cout,
                            int64_t K, double *outn) {
  const int64_t Ho = H - K + 1, Wo = W - K + 1;
  for (int64_t o = 0; o < Cout; ++o) {
    for (int64_t h = 0; h < Ho; ++h) {
      for (int64_t x0 = 0; x0 < Wo; ++x0) {
        double acc = b ? (double)b[o] : 0.0;
        for (int64_t c = 0; c < Cin; ++c)
          for (int64_t i = 0; i < K; ++i)
            for (int64_t j = 0; j < K; ++j)
              acc += (double)w[((o * Cin + c) * K + i) * K + j] *
                     (double)xn[(c * H + h + i) * W + x0 + j];
        outn[(o * Ho + h) * Wo + x0] = acc;
      }
    }
  }
}

int oracle_conv2d(const float *x, const float *w, const float *b, int64_t N,
                  int64_t Cin, int64_t H, int64_t W, int64_t Cout, int64_t K,
                  double *out, int nthreads) {
  if (!x || !w || !out || N < 0 || Cin < 1 || Cout < 1 || K < 1 || H < K ||
      W < K)
    return ORACLE_BAD_ARG;
  const int64_t Ho = H - K + 1, Wo = W - K + 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(clamp_threads(nthreads))
  for (int64_t n = 0; n < N; ++n)
    conv_one_sample(x + n * Cin * H * W, w, b, Cin, H, W, Cout, K,
                    out + n * Cout * Ho * Wo);
  return 0;
}

/* O4 — the whole chain, one sample at a time:                       [CHAIN]
 *   v0   = conv2d(x, W, b)                         (N, Cout, Ho, Wo)
 *   for each sample n and group g (Cout/G consecutive channels):
 *     mean = average of v0 over the group's channels and all Ho*Wo pixels,
 *     var  = average of (v0 - mean)^2 over the same values (population
 *            variance, no Bessel correction), computed in two passes;
 *   v1   = (v0 - mean) / sqrt(var + eps) * gamma[c] + beta[c]   (GroupNorm)
 *   v2   = tanh(v1)
 *   v3   = hardswish(v2)
 *   v4   = v0 + v3                                 (residual add)
 *   out[n,0,h,w] = log(sum_c exp(v4[n,c,h,w]))      (logsumexp over dim 1)
 * gamma / beta may be NULL (meaning 1 and 0).  mean_out / rstd_out, if not
 * NULL, receive mean and 1/sqrt(var+eps) per (n, g), row-major (N, G). */
int oracle_fused_chain(const float *x, const float *w, const float *b,
                       const float *gamma, const float *beta, int64_t N,
                       int64_t Cin, int64_t H, int64_t W, int64_t Cout,
                       int64_t K, int64_t G, double eps, double *out,
                       double *mean_out, double *rstd_out, int nthreads) {
  if (!x || !w || !out || N < 0 || Cin < 1 || Cout < 1 || K < 1 || H < K ||
      W < K || G < 1 || Cout % G != 0 || !(eps >= 0.0))
    return ORACLE_BAD_ARG;
  const int64_t Ho = H - K + 1, Wo = W - K + 1, P = Ho * Wo, Cg = Cout / G;
  int status = 0;
#pragma omp parallel num_threads(clamp_threads(nthreads))
  {
    double *v = (double *)malloc((size_t)(Cout * P) * sizeof(double));
    double *col = (double *)malloc((size_t)Cout * sizeof(double));
    double *mean_g = (double *)malloc((size_t)G * sizeof(double));
    double *rstd_g = (double *)malloc((size_t)G * sizeof(double));
    if (!v || !col || !mean_g || !rstd_g) {
#pragma omp atomic write
      status = ORACLE_NO_MEM;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t n = 0; n < N; ++n) {
      if (!v || !col || !mean_g || !rstd_g) continue;
      conv_one_sample(x + n * Cin * H * W, w, b, Cin, H, W, Cout, K, v);
      /* GroupNorm statistics, two passes per (n, g). */
      for (int64_t g = 0; g < G; ++g) {
        const double *vg = v + g * Cg * P;
        const int64_t cnt = Cg * P;
        double sum = 0.0;
        for (int64_t i = 0; i < cnt; ++i) sum += vg[i];
        const double mu = sum / (double)cnt;
        double sq = 0.0;
        for (int64_t i = 0; i < cnt; ++i) sq += (vg[i] - mu) * (vg[i] - mu);
        const double var = sq / (double)cnt;
        mean_g[g] = mu;
        rstd_g[g] = 1.0 / sqrt(var + eps);
        if (mean_out) mean_out[n * G + g] = mu;
        if (rstd_out) rstd_out[n * G + g] = rstd_g[g];
      }
      /* Per pixel: normalise, activate, add the residual, logsumexp over c. */
      for (int64_t p = 0; p < P; ++p) {
        int has_nan = 0;
        double m = -INFINITY;
        for (int64_t c = 0; c < Cout; ++c) {
          const int64_t g = c / Cg;
          const double v0 = v[c * P + p];
          const double ga = gamma ? (double)gamma[c] : 1.0;
          const double be = beta ? (double)beta[c] : 0.0;
          const double v1 = (v0 - mean_g[g]) * rstd_g[g] * ga + be;
          const double v4 = v0 + oracle_hardswish(tanh(v1));
          col[c] = v4;
          if (isnan(v4))
            has_nan = 1;
          else if (v4 > m)
            m = v4;
        }
        double r;
        if (has_nan) {
          r = NAN;
        } else if (isinf(m)) {
          r = m;
        } else {
          double s = 0.0;
          for (int64_t c = 0; c < Cout; ++c) s += exp(col[c] - m);
          r = m + log(s);
        }
        out[n * P + p] = r;
      }
    }
    free(v);
    free(col);
    free(mean_g);
    free(rstd_g);
  }
  return status;
}

/* Number of OpenMP threads a parallel region would use (for reporting). */
int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
