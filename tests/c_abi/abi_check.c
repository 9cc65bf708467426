/* abi_check.c — the C ABI of include/lse.h driven from plain C, with no
 * Python and no torch in the process: device buffers from hipMalloc, one
 * hipStream_t, results copied back and compared with the fp64 oracle
 * (oracle/oracle.c, linked in: this is test code).
 *
 *   abi_check --host     validation paths only (no GPU needed)
 *   abi_check --oracle   the oracle's functions alone, against closed forms
 *                        and each other (no GPU; the CPU suite also runs it
 *                        built with AddressSanitizer and UBSan)
 *   abi_check            every call on the GPU against the oracle
 *
 * Inputs come from a SplitMix64 stream (uniforms, Box-Muller normals): the
 * same host arrays go to the library and to the oracle.  Tolerance as in the
 * Python parity tests: |gpu - ref| <= atol + rtol |ref| for finite refs,
 * the same class (-inf, +inf, NaN) otherwise.  Exit status 0 = all passed. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "lse.h"

/* oracle/oracle.c */
int oracle_lse_axis0(const float *x, int64_t R, int64_t inner, double *out, int nthreads);
int oracle_log_softmax_rows(const float *x, int64_t rows, int64_t cols, double *y,
                            double *lse, int nthreads);
int oracle_softmax_rows(const float *x, int64_t rows, int64_t cols, double *y, int nthreads);
int oracle_lse_axis(const float *x, int64_t outer, int64_t R, int64_t inner, double *out,
                    int nthreads);
int oracle_log_softmax_axis(const float *x, int64_t outer, int64_t R, int64_t inner,
                            double *y, int nthreads);
int oracle_fused_chain(const float *x, const float *w, const float *b, const float *gamma,
                       const float *beta, int64_t N, int64_t Cin, int64_t H, int64_t W,
                       int64_t Cout, int64_t K, int64_t G, double eps, double *out,
                       double *mean_out, double *rstd_out, int nthreads);
int oracle_lse_chunk_partials(const float *x, int64_t rows, int64_t cols, int64_t chunk,
                              double *m_out, double *s_out, int nthreads);
int oracle_lse_merge(const double *m, const double *s, int64_t rows, int64_t k, double *lse,
                     double *M_out, double *S_out);
int oracle_conv2d(const float *x, const float *w, const float *b, int64_t N, int64_t Cin,
                  int64_t H, int64_t W, int64_t Cout, int64_t K, double *out, int nthreads);
double oracle_hardswish(double t);

static int g_fail = 0;

#define CHECK_HIP(call)                                                              \
  do {                                                                               \
    hipError_t e_ = (call);                                                          \
    if (e_ != hipSuccess) {                                                          \
      fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__,    \
              __LINE__);                                                             \
      exit(2);                                                                       \
    }                                                                                \
  } while (0)

#define EXPECT(cond, what)                                                           \
  do {                                                                               \
    if (!(cond)) {                                                                   \
      fprintf(stderr, "FAILED: %s (%s:%d)\n", what, __FILE__, __LINE__);             \
      ++g_fail;                                                                      \
    }                                                                                \
  } while (0)

/* ------------------------------------------------------------- inputs */
static uint64_t g_state;
static uint64_t splitmix64(void) {
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static double uniform01(void) { return (double)(splitmix64() >> 11) * 0x1.0p-53; }
static float *normal_array(int64_t n, double sigma, uint64_t seed) {
  float *a = (float *)malloc((size_t)n * sizeof(float));
  g_state = seed;
  for (int64_t i = 0; i < n; ++i) {
    const double u1 = 1.0 - uniform01(), u2 = uniform01();
    a[i] = (float)(sigma * sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2));
  }
  return a;
}
static float *uniform_array(int64_t n, double bound, uint64_t seed) {
  float *a = (float *)malloc((size_t)n * sizeof(float));
  g_state = seed;
  for (int64_t i = 0; i < n; ++i) a[i] = (float)(bound * (2.0 * uniform01() - 1.0));
  return a;
}

/* ------------------------------------------------------------- helpers */
static float *to_device(const float *h, int64_t n) {
  float *d = NULL;
  CHECK_HIP(hipMalloc((void **)&d, (size_t)(n > 0 ? n : 1) * sizeof(float)));
  if (h && n > 0) CHECK_HIP(hipMemcpy(d, h, (size_t)n * sizeof(float), hipMemcpyHostToDevice));
  return d;
}
static float *from_device(const float *d, int64_t n) {
  float *h = (float *)malloc((size_t)n * sizeof(float));
  CHECK_HIP(hipMemcpy(h, d, (size_t)n * sizeof(float), hipMemcpyDeviceToHost));
  return h;
}

static void compare(const char *what, const float *got, const double *ref, int64_t n,
                    double atol, double rtol) {
  int64_t bad = 0;
  double worst = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    const double g = got[i], r = ref[i];
    int ok;
    if (isfinite(r)) {
      const double err = fabs(g - r);
      ok = isfinite(g) && err <= atol + rtol * fabs(r);
      if (isfinite(g) && err > worst) worst = err;
    } else if (isnan(r)) {
      ok = isnan(g);
    } else {
      ok = (g == r);
    }
    if (!ok) {
      if (bad < 3) fprintf(stderr, "  %s[%lld]: gpu %.9g ref %.9g\n", what, (long long)i, g, r);
      ++bad;
    }
  }
  printf("%-34s n=%-9lld max |err| %.3g  %s\n", what, (long long)n, worst, bad ? "FAIL" : "ok");
  if (bad) ++g_fail;
}

static void check_status(lse_status_t st, const char *what) {
  if (st != LSE_OK) {
    fprintf(stderr, "%s: %s: %s\n", what, lse_status_string(st), lse_last_error());
    ++g_fail;
  }
}

/* ------------------------------------------------------------- host-only */
static void host_checks(void) {
  float *fake = (float *)(uintptr_t)0x100000, *fake2 = (float *)(uintptr_t)0x900000000ull;
  EXPECT(lse_abi_version() == LSE_ABI_VERSION, "abi version");
  EXPECT(strcmp(lse_status_string(LSE_ERR_NULL), "LSE_ERR_NULL") == 0, "status string");
  EXPECT(lse_reduce_axis0(NULL, fake2, 3, 5, NULL) == LSE_ERR_NULL, "NULL x");
  EXPECT(strlen(lse_last_error()) > 0, "last error text");
  EXPECT(lse_reduce_axis0(fake, fake2, 0, 5, NULL) == LSE_ERR_SHAPE, "R = 0");
  EXPECT(lse_reduce_axis0(NULL, NULL, 3, 0, NULL) == LSE_OK, "empty call");
  EXPECT(log_softmax_rows(fake, fake, 4, 8, NULL, 0, NULL) == LSE_ERR_OVERLAP, "in place");
  EXPECT(log_softmax_rows(fake, fake2, 16, 393216, NULL, 0, NULL) == LSE_ERR_WORKSPACE,
         "missing workspace");
  EXPECT(log_softmax_rows_workspace_bytes(16, 393216) == 256 + 16 * 12 * 8, "workspace size");
  EXPECT(log_softmax_axis_strided(fake, fake2, 2, 3, 8, 24, 8, 24, 4, NULL) == LSE_ERR_SHAPE,
         "colliding output planes");
  EXPECT(log_softmax_rows_strided(fake, fake2, 4, 8, 7, 8, NULL, 0, NULL) == LSE_ERR_SHAPE,
         "row pitch below cols");
  EXPECT(fused_conv_gn_act_lse(fake, fake, NULL, NULL, NULL, 2, 8, 12, 12, 64, 5, 16, 1e-5f,
                               fake2, fake2, 1u << 20, NULL) == LSE_ERR_UNSUPPORTED,
         "unsupported kernel size");
  printf("%-34s %s\n", "host-side validation", g_fail ? "FAIL" : "ok");
}

/* ------------------------------------------------------------ oracle-only */
/* Every oracle function on small host arrays (edge sizes included), checked
 * against facts that do not restate its formula: closed forms, sums of
 * probabilities, agreement between independent entry points, a delta-filter
 * conv.  Run with the sanitizers by the CPU suite. */
static int close_to(double a, double b, double tol) {
  if (isnan(a) || isnan(b)) return isnan(a) && isnan(b);
  if (isinf(a) || isinf(b)) return a == b;
  return fabs(a - b) <= tol * (1.0 + fabs(b));
}

static void oracle_checks(void) {
  const double inf = INFINITY;
  /* axis 0: R equal values -> v + log R; two values -> max + log1p(exp(-|a - b|)) */
  {
    float x[15];
    for (int i = 0; i < 15; ++i) x[i] = 1.25f;
    double out[3];
    EXPECT(oracle_lse_axis0(x, 5, 3, out, 1) == 0, "lse_axis0 status");
    for (int j = 0; j < 3; ++j) EXPECT(close_to(out[j], 1.25 + log(5.0), 1e-14), "R equal values");
    const float y[2] = {3.0f, -1.0f};
    EXPECT(oracle_lse_axis0(y, 2, 1, out, 1) == 0, "two values status");
    EXPECT(close_to(out[0], 3.0 + log1p(exp(-4.0)), 1e-14), "two values");
    const float sp[8] = {-(float)inf, (float)inf, NAN, 0.0f,    /* plane 0 */
                         -(float)inf, 1.0f, (float)inf, NAN};   /* plane 1 */
    double o4[4];
    EXPECT(oracle_lse_axis0(sp, 2, 4, o4, 1) == 0, "special status");
    EXPECT(o4[0] == -inf && o4[1] == inf && isnan(o4[2]) && isnan(o4[3]), "special values");
    EXPECT(oracle_lse_axis0(NULL, 2, 4, o4, 1) < 0, "NULL rejected");
  }
  /* rows: exp(y) sums to 1, x - y is the row's LSE; softmax sums to 1 */
  {
    const int64_t rows = 4, cols = 37;
    float *x = normal_array(rows * cols, 3.0, 11);
    double *y = malloc(sizeof(double) * rows * cols), lse[4];
    EXPECT(oracle_log_softmax_rows(x, rows, cols, y, lse, 2) == 0, "log_softmax status");
    for (int64_t r = 0; r < rows; ++r) {
      double t = 0.0;
      for (int64_t c = 0; c < cols; ++c) t += exp(y[r * cols + c]);
      EXPECT(close_to(t, 1.0, 1e-13), "sum exp(log_softmax) = 1");
      EXPECT(close_to((double)x[r * cols + 5] - y[r * cols + 5], lse[r], 1e-13), "x - y = lse");
    }
    EXPECT(oracle_softmax_rows(x, rows, cols, y, 2) == 0, "softmax status");
    for (int64_t r = 0; r < rows; ++r) {
      double t = 0.0;
      for (int64_t c = 0; c < cols; ++c) t += y[r * cols + c];
      EXPECT(close_to(t, 1.0, 1e-13), "softmax sums to 1");
    }
    /* chunk partials merged = the row LSE, for chunkings that do and do not divide cols */
    const int64_t chunks[3] = {1, 7, 37};
    for (int k = 0; k < 3; ++k) {
      const int64_t nch = (cols + chunks[k] - 1) / chunks[k];
      double *m = malloc(sizeof(double) * rows * nch), *sm = malloc(sizeof(double) * rows * nch);
      double merged[4];
      EXPECT(oracle_lse_chunk_partials(x, rows, cols, chunks[k], m, sm, 2) == 0, "partials");
      EXPECT(oracle_lse_merge(m, sm, rows, nch, merged, NULL, NULL) == 0, "merge");
      for (int64_t r = 0; r < rows; ++r) EXPECT(close_to(merged[r], lse[r], 1e-13), "merged LSE");
      free(m);
      free(sm);
    }
    free(x);
    free(y);
  }
  /* middle axis: each outer slab is an axis-0 problem; log_softmax columns sum to 1 */
  {
    const int64_t outer = 3, R = 4, inner = 5;
    float *x = normal_array(outer * R * inner, 2.0, 12);
    double out[15], ref[5], y[60];
    EXPECT(oracle_lse_axis(x, outer, R, inner, out, 2) == 0, "lse_axis status");
    for (int64_t o = 0; o < outer; ++o) {
      EXPECT(oracle_lse_axis0(x + o * R * inner, R, inner, ref, 1) == 0, "slab status");
      for (int64_t j = 0; j < inner; ++j)
        EXPECT(close_to(out[o * inner + j], ref[j], 1e-15), "slab LSE");
    }
    EXPECT(oracle_log_softmax_axis(x, outer, R, inner, y, 2) == 0, "lsm_axis status");
    for (int64_t o = 0; o < outer; ++o)
      for (int64_t j = 0; j < inner; ++j) {
        double t = 0.0;
        for (int64_t r = 0; r < R; ++r) t += exp(y[(o * R + r) * inner + j]);
        EXPECT(close_to(t, 1.0, 1e-13), "axis log_softmax sums to 1");
      }
    free(x);
  }
  /* conv with a delta filter copies a shifted input channel plus the bias;
   * hardswish at its kinks; the chain with gamma = beta = 0 is LSE_c(conv) */
  {
    const int64_t N = 2, Cin = 3, H = 6, W = 7, Cout = 4, K = 3, Ho = 4, Wo = 5;
    float *x = normal_array(N * Cin * H * W, 1.0, 13);
    float w[4 * 3 * 9] = {0}, b[4] = {0.5f, -0.25f, 1.0f, 0.0f}, z[4] = {0};
    for (int64_t o = 0; o < Cout; ++o) w[(o * Cin + o % Cin) * 9 + 4] = 1.0f;  /* centre tap */
    double conv[2 * 4 * 4 * 5], chain[2 * 4 * 5], mean[4], rstd[4];
    EXPECT(oracle_conv2d(x, w, b, N, Cin, H, W, Cout, K, conv, 2) == 0, "conv status");
    for (int64_t n = 0; n < N; ++n)
      for (int64_t o = 0; o < Cout; ++o)
        for (int64_t h = 0; h < Ho; ++h)
          for (int64_t q = 0; q < Wo; ++q)
            EXPECT(conv[((n * Cout + o) * Ho + h) * Wo + q] ==
                       (double)x[((n * Cin + o % Cin) * H + h + 1) * W + q + 1] + (double)b[o],
                   "delta-filter conv");
    EXPECT(oracle_hardswish(-3.0) == 0.0 && oracle_hardswish(3.0) == 3.0 &&
               oracle_hardswish(0.0) == 0.0 && oracle_hardswish(-4.0) == 0.0 &&
               oracle_hardswish(5.0) == 5.0 && close_to(oracle_hardswish(1.0), 4.0 / 6.0, 1e-15),
           "hardswish kinks");
    EXPECT(oracle_fused_chain(x, w, b, z, z, N, Cin, H, W, Cout, K, 2, 1e-5, chain, mean, rstd,
                              2) == 0, "chain status");
    for (int64_t n = 0; n < N; ++n)
      for (int64_t p = 0; p < Ho * Wo; ++p) {
        double m = -INFINITY, t = 0.0;
        for (int64_t o = 0; o < Cout; ++o) m = fmax(m, conv[(n * Cout + o) * Ho * Wo + p]);
        for (int64_t o = 0; o < Cout; ++o) t += exp(conv[(n * Cout + o) * Ho * Wo + p] - m);
        EXPECT(close_to(chain[n * Ho * Wo + p], m + log(t), 1e-13), "chain = LSE_c(conv)");
      }
    for (int g = 0; g < 4; ++g) EXPECT(isfinite(mean[g]) && rstd[g] > 0.0, "group moments");
    free(x);
  }
  printf("%-34s %s\n", "oracle functions", g_fail ? "FAIL" : "ok");
}

/* ------------------------------------------------------------- GPU cases */
static void case_axis0(hipStream_t s) {
  const int64_t R = 7, inner = 1000, n = R * inner;
  float *x = normal_array(n, 2.0, 11), *dx = to_device(x, n), *dout = to_device(NULL, inner);
  double *ref = (double *)malloc(inner * sizeof(double));
  check_status(lse_reduce_axis0(dx, dout, R, inner, s), "lse_reduce_axis0");
  CHECK_HIP(hipStreamSynchronize(s));
  float *got = from_device(dout, inner);
  oracle_lse_axis0(x, R, inner, ref, 0);
  compare("lse_reduce_axis0 (7, 1000)", got, ref, inner, 1e-5, 2e-6);
  free(x); free(ref); free(got);
  CHECK_HIP(hipFree(dx)); CHECK_HIP(hipFree(dout));
}

/* Few outputs over many planes with a workspace (column split), and the same
   call without one. */
static void case_axis0_ws(hipStream_t s) {
  const int64_t R = 300000, inner = 12, n = R * inner;
  float *x = normal_array(n, 2.0, 14), *dx = to_device(x, n), *dout = to_device(NULL, inner);
  float *dy = to_device(NULL, n);
  double *ref = (double *)malloc(inner * sizeof(double));
  const size_t wl = lse_axis_workspace_bytes(1, R, inner, 0);
  const size_t wm = lse_axis_workspace_bytes(1, R, inner, 1);
  EXPECT(wl > 0 && wm > wl, "few-output workspace sizes");
  void *ws = NULL;
  CHECK_HIP(hipMalloc(&ws, wm));
  EXPECT(lse_reduce_axis0_ws(dx, dout, R, inner, NULL, 0, s) == LSE_ERR_WORKSPACE,
         "missing workspace");
  check_status(lse_reduce_axis0_ws(dx, dout, R, inner, ws, wl, s), "lse_reduce_axis0_ws");
  CHECK_HIP(hipStreamSynchronize(s));
  float *got = from_device(dout, inner);
  oracle_lse_axis0(x, R, inner, ref, 0);
  compare("lse_reduce_axis0_ws (300000, 12)", got, ref, inner, 1e-5, 2e-6);
  free(got);
  check_status(lse_reduce_axis0(dx, dout, R, inner, s), "lse_reduce_axis0 few outputs");
  CHECK_HIP(hipStreamSynchronize(s));
  got = from_device(dout, inner);
  compare("lse_reduce_axis0 (300000, 12)", got, ref, inner, 1e-5, 2e-6);
  free(got);
  double *yref = (double *)malloc(n * sizeof(double));
  check_status(log_softmax_axis_strided_ws(dx, dy, 1, R, inner, n, inner, n, inner, ws, wm, s),
               "log_softmax_axis_strided_ws");
  CHECK_HIP(hipStreamSynchronize(s));
  got = from_device(dy, n);
  oracle_log_softmax_axis(x, 1, R, inner, yref, 0);
  compare("log_softmax_axis_strided_ws (1, 300000, 12)", got, yref, n, 1e-5, 2e-6);
  free(got); free(x); free(ref); free(yref);
  CHECK_HIP(hipFree(dx)); CHECK_HIP(hipFree(dout)); CHECK_HIP(hipFree(dy)); CHECK_HIP(hipFree(ws));
}

static void case_rows(hipStream_t s) {
  const int64_t rows = 3, cols = 100000, n = rows * cols;
  float *x = normal_array(n, 3.0, 12), *dx = to_device(x, n), *dy = to_device(NULL, n);
  const size_t wsb = log_softmax_rows_workspace_bytes(rows, cols);
  void *ws = NULL;
  CHECK_HIP(hipMalloc(&ws, wsb));
  double *ref = (double *)malloc(n * sizeof(double)), *lse = (double *)malloc(rows * 8);
  check_status(log_softmax_rows(dx, dy, rows, cols, ws, wsb, s), "log_softmax_rows");
  CHECK_HIP(hipStreamSynchronize(s));
  float *got = from_device(dy, n);
  oracle_log_softmax_rows(x, rows, cols, ref, lse, 0);
  compare("log_softmax_rows (3, 100000)", got, ref, n, 1e-5, 2e-6);
  free(got);
  check_status(softmax_rows(dx, dy, rows, cols, ws, wsb, s), "softmax_rows");
  CHECK_HIP(hipStreamSynchronize(s));
  got = from_device(dy, n);
  oracle_softmax_rows(x, rows, cols, ref, 0);
  compare("softmax_rows (3, 100000)", got, ref, n, 1e-37, 1e-5);
  free(got);

  /* per-chunk pairs and their merge */
  const int64_t chunk = 4096, k = lse_rows_num_chunks(cols, chunk);
  float *dp = to_device(NULL, rows * k * 2), *dl = to_device(NULL, rows);
  check_status(lse_rows_partial(dx, rows, cols, chunk, (lse_pair_t *)dp, s), "lse_rows_partial");
  check_status(lse_rows_merge((const lse_pair_t *)dp, rows, k, dl, s), "lse_rows_merge");
  CHECK_HIP(hipStreamSynchronize(s));
  got = from_device(dl, rows);
  compare("lse_rows_partial + merge", got, lse, rows, 1e-5, 2e-6);
  free(got); free(x); free(ref); free(lse);
  CHECK_HIP(hipFree(dx)); CHECK_HIP(hipFree(dy)); CHECK_HIP(hipFree(ws));
  CHECK_HIP(hipFree(dp)); CHECK_HIP(hipFree(dl));
}

static void case_strided(hipStream_t s) {
  /* (3, 20, 64) planes with a pitch of 80 floats; output rows with a pitch of 72 */
  const int64_t outer = 3, R = 20, inner = 64, pitch = 80, opitch = 72;
  const int64_t nbig = outer * R * pitch;
  float *big = normal_array(nbig, 3.0, 13), *dbig = to_device(big, nbig);
  float *x = (float *)malloc(outer * R * inner * sizeof(float));
  for (int64_t o = 0; o < outer; ++o)
    for (int64_t r = 0; r < R; ++r)
      memcpy(x + (o * R + r) * inner, big + (o * R + r) * pitch, inner * sizeof(float));
  float *dout = to_device(NULL, outer * opitch);
  CHECK_HIP(hipMemset(dout, 0, outer * opitch * sizeof(float)));
  check_status(lse_reduce_axis_strided(dbig, dout, outer, R, inner, R * pitch, pitch, opitch, s),
               "lse_reduce_axis_strided");
  float *dy = to_device(NULL, outer * R * inner);
  check_status(log_softmax_axis_strided(dbig, dy, outer, R, inner, R * pitch, pitch, R * inner,
                                        inner, s),
               "log_softmax_axis_strided");
  CHECK_HIP(hipStreamSynchronize(s));
  float *o = from_device(dout, outer * opitch), *got = (float *)malloc(outer * inner * 4);
  for (int64_t i = 0; i < outer; ++i) memcpy(got + i * inner, o + i * opitch, inner * 4);
  double *ref = (double *)malloc(outer * R * inner * sizeof(double));
  oracle_lse_axis(x, outer, R, inner, ref, 0);
  compare("lse_reduce_axis_strided", got, ref, outer * inner, 1e-5, 2e-6);
  int pad_ok = 1;
  for (int64_t i = 0; i < outer; ++i)
    for (int64_t j = inner; j < opitch; ++j) pad_ok &= (o[i * opitch + j] == 0.0f);
  EXPECT(pad_ok, "strided output padding untouched");
  free(got);
  got = from_device(dy, outer * R * inner);
  oracle_log_softmax_axis(x, outer, R, inner, ref, 0);
  compare("log_softmax_axis_strided", got, ref, outer * R * inner, 1e-5, 2e-6);
  free(big); free(x); free(o); free(got); free(ref);
  CHECK_HIP(hipFree(dbig)); CHECK_HIP(hipFree(dout)); CHECK_HIP(hipFree(dy));
}

static void case_chain(hipStream_t s) {
  const int64_t N = 2, Cin = 8, H = 12, W = 12, Cout = 64, K = 3, G = 16;
  const int64_t nx = N * Cin * H * W, nw = Cout * Cin * K * K, Ho = H - K + 1, Wo = W - K + 1;
  const double bound = 1.0 / sqrt((double)(Cin * K * K));
  float *x = normal_array(nx, 1.0, 14), *w = uniform_array(nw, bound, 15),
        *b = uniform_array(Cout, bound, 16);
  float *dx = to_device(x, nx), *dw = to_device(w, nw), *db = to_device(b, Cout);
  float *dout = to_device(NULL, N * Ho * Wo);
  const size_t wsb = fused_conv_gn_act_lse_workspace_bytes(N, Cin, H, W, Cout, K, G);
  void *ws = NULL;
  CHECK_HIP(hipMalloc(&ws, wsb));
  check_status(fused_conv_gn_act_lse(dx, dw, db, NULL, NULL, N, Cin, H, W, Cout, K, G, 1e-5f,
                                     dout, ws, wsb, s),
               "fused_conv_gn_act_lse");
  CHECK_HIP(hipStreamSynchronize(s));
  float *got = from_device(dout, N * Ho * Wo);
  double *ref = (double *)malloc(N * Ho * Wo * sizeof(double));
  oracle_fused_chain(x, w, b, NULL, NULL, N, Cin, H, W, Cout, K, G, 1e-5, ref, NULL, NULL, 0);
  compare("fused_conv_gn_act_lse (2,8,12,12)", got, ref, N * Ho * Wo, 1e-5, 5e-4);
  free(x); free(w); free(b); free(got); free(ref);
  CHECK_HIP(hipFree(dx)); CHECK_HIP(hipFree(dw)); CHECK_HIP(hipFree(db));
  CHECK_HIP(hipFree(dout)); CHECK_HIP(hipFree(ws));
}

int main(int argc, char **argv) {
  const int host_only = argc > 1 && strcmp(argv[1], "--host") == 0;
  const int oracle_only = argc > 1 && strcmp(argv[1], "--oracle") == 0;
  if (oracle_only) {
    oracle_checks();
    printf(g_fail ? "FAILURES: %d\n" : "ALL OK\n", g_fail);
    return g_fail ? 1 : 0;
  }
  host_checks();
  if (!host_only) {
    hipStream_t s;
    CHECK_HIP(hipSetDevice(0));
    CHECK_HIP(hipStreamCreate(&s));
    case_axis0(s);
    case_axis0_ws(s);
    case_rows(s);
    case_strided(s);
    case_chain(s);
    CHECK_HIP(hipStreamDestroy(s));
  }
  printf(g_fail ? "FAILURES: %d\n" : "ALL OK\n", g_fail);
  return g_fail ? 1 : 0;
}
