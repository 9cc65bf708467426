// lse_api.hip — the extern "C" entry points declared in include/lse.h.
// Every argument is checked on the host before anything is enqueued; the
// launchers in the kernel files assume checked arguments.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/lse.h"
#include "../../include/lse_testing.h"
#include "lse_internal.hpp"

#define LSE_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

lse_status_t fail(lse_status_t st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

lse_status_t ok() {
  g_last_error.clear();
  return LSE_OK;
}

lse_status_t from_hip(hipError_t e, const char *what) {
  if (e == hipSuccess) return ok();
  return fail(LSE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// a * b without int64 overflow (both >= 0); false on overflow.
bool mul_ok(int64_t a, int64_t b, int64_t *r) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *r = a * b;
  return true;
}

bool overlaps(const void *a, int64_t a_bytes, const void *b, int64_t b_bytes) {
  const uintptr_t a0 = (uintptr_t)a, a1 = a0 + (uintptr_t)a_bytes;
  const uintptr_t b0 = (uintptr_t)b, b1 = b0 + (uintptr_t)b_bytes;
  return a_bytes > 0 && b_bytes > 0 && a0 < b1 && b0 < a1;
}

constexpr int64_t kMaxElems = INT64_MAX / 16;  // keeps every byte offset in range
constexpr int64_t kMaxGrid = 0x7fffffff;
// Workgroups of 512 lanes whose work-items fit one dispatch (32-bit count).
constexpr int64_t kMaxWorkgroups512 = 0xffffffffll / 512;

// a + b (both >= 0) capped: false when the sum passes kMaxElems.
bool add_ok(int64_t a, int64_t b, int64_t *r) {
  if (a > kMaxElems || b > kMaxElems - a) return false;
  *r = a + b;
  return true;
}

// Elements from the first to one past the last element of a row-major
// (n1, n2, inner) array with strides s1, s2 and contiguous inner index:
// (n1 - 1) s1 + (n2 - 1) s2 + inner.  All sizes >= 1, strides >= 0.
bool span_ok(int64_t n1, int64_t s1, int64_t n2, int64_t s2, int64_t inner, int64_t *span) {
  int64_t a, b, t;
  return mul_ok(n1 - 1, s1, &a) && mul_ok(n2 - 1, s2, &b) && add_ok(a, b, &t) &&
         add_ok(t, inner, span);
}

}  // namespace

LSE_EXPORT const char *lse_status_string(int status) {
  switch (status) {
    case LSE_OK: return "LSE_OK";
    case LSE_ERR_NULL: return "LSE_ERR_NULL";
    case LSE_ERR_SHAPE: return "LSE_ERR_SHAPE";
    case LSE_ERR_WORKSPACE: return "LSE_ERR_WORKSPACE";
    case LSE_ERR_OVERLAP: return "LSE_ERR_OVERLAP";
    case LSE_ERR_HIP: return "LSE_ERR_HIP";
    case LSE_ERR_UNSUPPORTED: return "LSE_ERR_UNSUPPORTED";
    default: return "LSE_ERR_UNKNOWN";
  }
}

LSE_EXPORT const char *lse_last_error(void) { return g_last_error.c_str(); }

LSE_EXPORT int lse_abi_version(void) { return LSE_ABI_VERSION; }

LSE_EXPORT void lse_testing_set_spin_limit(uint32_t polls) { lse::set_spin_limit(polls); }

LSE_EXPORT void lse_testing_set_rows_reread(int enable) { lse::set_rows_reread(enable != 0); }

LSE_EXPORT lse_status_t lse_testing_set_chain_path(int path) {
  if (path < 0 || path > 3) return fail(LSE_ERR_SHAPE, "lse_testing_set_chain_path: 0..3");
  lse::set_chain_path(path);
  return ok();
}

// ------------------------------------------------------------------ case A
LSE_EXPORT lse_status_t lse_reduce_axis0(const float *x, float *out, int64_t R, int64_t inner,
                                         hipStream_t stream) {
  if (R < 1) return fail(LSE_ERR_SHAPE, "lse_reduce_axis0: R = %lld must be >= 1", (long long)R);
  if (inner < 0)
    return fail(LSE_ERR_SHAPE, "lse_reduce_axis0: inner = %lld must be >= 0", (long long)inner);
  int64_t total;
  if (!mul_ok(R, inner, &total) || total > kMaxElems)
    return fail(LSE_ERR_SHAPE, "lse_reduce_axis0: R * inner overflows");
  if (inner == 0) return ok();
  if (!x || !out) return fail(LSE_ERR_NULL, "lse_reduce_axis0: x and out must be non-NULL");
  if (overlaps(x, total * 4, out, inner * 4))
    return fail(LSE_ERR_OVERLAP, "lse_reduce_axis0: out overlaps x");
  if ((inner + 63) / 64 > kMaxGrid)
    return fail(LSE_ERR_SHAPE, "lse_reduce_axis0: inner too large for one launch");
  const lse::AxisDims d{1, R, inner, R * inner, inner, inner, 0};
  return from_hip(lse::launch_lse_axis(x, out, d, stream), "lse_reduce_axis0 launch");
}

// ------------------------------------------------------------ middle axis
// Checks a strided axis call: x[o xso + r xsr + j], output y[o yso + r ysr + j]
// (logsumexp: ysr = 0 and R_out = 1).  Writes must not collide, so
// consecutive output planes / outer blocks may not overlap (ysr >= inner,
// yso >= (R_out - 1) ysr + inner); x's span and the output's span must be
// disjoint (checked on the byte ranges, conservatively).
static lse_status_t check_axis(const char *who, const void *x, const void *out, int64_t outer,
                               int64_t R, int64_t inner, int64_t xso, int64_t xsr, int64_t yso,
                               int64_t ysr, bool lsm, int64_t *total) {
  if (outer < 0 || R < 1 || inner < 0)
    return fail(LSE_ERR_SHAPE, "%s: need outer >= 0, R >= 1, inner >= 0 (got %lld, %lld, %lld)",
                who, (long long)outer, (long long)R, (long long)inner);
  if (xso < 0 || xsr < 0 || yso < 0 || ysr < 0)
    return fail(LSE_ERR_SHAPE, "%s: strides must be >= 0", who);
  int64_t t;
  if (!mul_ok(outer, R, &t) || !mul_ok(t, inner, total) || *total > kMaxElems)
    return fail(LSE_ERR_SHAPE, "%s: outer * R * inner overflows", who);
  if (*total == 0) return LSE_OK;
  const int64_t r_out = lsm ? R : 1;
  if (r_out > 1 && ysr < inner)
    return fail(LSE_ERR_SHAPE, "%s: output planes overlap (stride %lld < inner %lld)", who,
                (long long)ysr, (long long)inner);
  int64_t plane_span;
  if (!span_ok(r_out, ysr, 1, 0, inner, &plane_span))
    return fail(LSE_ERR_SHAPE, "%s: output extent overflows", who);
  if (outer > 1 && yso < plane_span)
    return fail(LSE_ERR_SHAPE, "%s: output blocks overlap (outer stride %lld < %lld)", who,
                (long long)yso, (long long)plane_span);
  int64_t xspan, yspan;
  if (!span_ok(outer, xso, R, xsr, inner, &xspan) || !span_ok(outer, yso, r_out, ysr, inner, &yspan))
    return fail(LSE_ERR_SHAPE, "%s: strided extent overflows", who);
  if (!x || !out) return fail(LSE_ERR_NULL, "%s: NULL pointer", who);
  if (overlaps(x, xspan * 4, out, yspan * 4))
    return fail(LSE_ERR_OVERLAP, "%s: output overlaps x", who);
  if ((outer * inner + 63) / 64 > kMaxGrid)
    return fail(LSE_ERR_SHAPE, "%s: too many outputs for one launch", who);
  return LSE_OK;
}

LSE_EXPORT lse_status_t lse_reduce_axis_strided(const float *x, float *out, int64_t outer,
                                                int64_t R, int64_t inner,
                                                int64_t x_stride_outer, int64_t x_stride_r,
                                                int64_t out_stride_outer, hipStream_t stream) {
  int64_t total;
  const lse_status_t st = check_axis("lse_reduce_axis", x, out, outer, R, inner, x_stride_outer,
                                     x_stride_r, out_stride_outer, 0, false, &total);
  if (st != LSE_OK) return st;
  if (total == 0) return ok();
  const lse::AxisDims d{outer, R, inner, x_stride_outer, x_stride_r, out_stride_outer, 0};
  return from_hip(lse::launch_lse_axis(x, out, d, stream), "lse_reduce_axis launch");
}

LSE_EXPORT lse_status_t lse_reduce_axis(const float *x, float *out, int64_t outer, int64_t R,
                                        int64_t inner, hipStream_t stream) {
  int64_t xso = 0;  // negative sizes are reported by the strided call's checks
  if (!mul_ok(R, inner, &xso) && R >= 1 && inner >= 0)
    return fail(LSE_ERR_SHAPE, "lse_reduce_axis: outer * R * inner overflows");
  return lse_reduce_axis_strided(x, out, outer, R, inner, xso, inner, inner, stream);
}

LSE_EXPORT lse_status_t log_softmax_axis_strided(const float *x, float *y, int64_t outer,
                                                 int64_t R, int64_t inner,
                                                 int64_t x_stride_outer, int64_t x_stride_r,
                                                 int64_t y_stride_outer, int64_t y_stride_r,
                                                 hipStream_t stream) {
  int64_t total;
  const lse_status_t st =
      check_axis("log_softmax_axis", x, y, outer, R, inner, x_stride_outer, x_stride_r,
                 y_stride_outer, y_stride_r, true, &total);
  if (st != LSE_OK) return st;
  if (total == 0) return ok();
  const lse::AxisDims d{outer, R, inner, x_stride_outer, x_stride_r, y_stride_outer, y_stride_r};
  return from_hip(lse::launch_log_softmax_axis(x, y, d, stream), "log_softmax_axis launch");
}

LSE_EXPORT lse_status_t log_softmax_axis(const float *x, float *y, int64_t outer, int64_t R,
                                         int64_t inner, hipStream_t stream) {
  int64_t so = 0;  // negative sizes are reported by the strided call's checks
  if (!mul_ok(R, inner, &so) && R >= 1 && inner >= 0)
    return fail(LSE_ERR_SHAPE, "log_softmax_axis: outer * R * inner overflows");
  return log_softmax_axis_strided(x, y, outer, R, inner, so, inner, so, inner, stream);
}

// ------------------------------------------------- axis calls with a workspace
LSE_EXPORT size_t lse_axis_workspace_bytes(int64_t outer, int64_t R, int64_t inner,
                                           int log_softmax) {
  int64_t t, total;
  if (outer < 1 || R < 1 || inner < 1 || !mul_ok(outer, R, &t) || !mul_ok(t, inner, &total) ||
      total > kMaxElems)
    return 0;
  return lse::axis_workspace_bytes(outer, R, inner, log_softmax != 0);
}

// The workspace of an axis call: required when the call's sizes take a split
// path, and disjoint from x and the output.
static lse_status_t check_axis_ws(const char *who, const void *x, const void *out, int64_t outer,
                                  int64_t R, int64_t inner, int64_t xso, int64_t xsr,
                                  int64_t yso, int64_t ysr, bool lsm, const void *ws,
                                  size_t ws_bytes) {
  const size_t need = lse::axis_workspace_bytes(outer, R, inner, lsm);
  if (need == 0) return LSE_OK;
  if (!ws) return fail(LSE_ERR_WORKSPACE, "%s: needs %zu workspace bytes", who, need);
  if (ws_bytes < need)
    return fail(LSE_ERR_WORKSPACE, "%s: workspace %zu < required %zu", who, ws_bytes, need);
  int64_t xspan, yspan;
  span_ok(outer, xso, R, xsr, inner, &xspan);  // checked by check_axis
  span_ok(outer, yso, lsm ? R : 1, ysr, inner, &yspan);
  if (overlaps(ws, (int64_t)need, x, xspan * 4) || overlaps(ws, (int64_t)need, out, yspan * 4))
    return fail(LSE_ERR_OVERLAP, "%s: workspace overlaps x or the output", who);
  return LSE_OK;
}

LSE_EXPORT lse_status_t lse_reduce_axis_strided_ws(const float *x, float *out, int64_t outer,
                                                   int64_t R, int64_t inner,
                                                   int64_t x_stride_outer, int64_t x_stride_r,
                                                   int64_t out_stride_outer, void *ws,
                                                   size_t ws_bytes, hipStream_t stream) {
  const char *who = "lse_reduce_axis_strided_ws";
  int64_t total;
  lse_status_t st = check_axis(who, x, out, outer, R, inner, x_stride_outer, x_stride_r,
                               out_stride_outer, 0, false, &total);
  if (st != LSE_OK) return st;
  if (total == 0) return ok();
  st = check_axis_ws(who, x, out, outer, R, inner, x_stride_outer, x_stride_r, out_stride_outer,
                     0, false, ws, ws_bytes);
  if (st != LSE_OK) return st;
  const lse::AxisDims d{outer, R, inner, x_stride_outer, x_stride_r, out_stride_outer, 0};
  return from_hip(lse::launch_lse_axis(x, out, d, stream, true, ws), who);
}

LSE_EXPORT lse_status_t lse_reduce_axis0_ws(const float *x, float *out, int64_t R, int64_t inner,
                                            void *ws, size_t ws_bytes, hipStream_t stream) {
  int64_t xso = 0;  // negative sizes are reported by the strided call's checks
  if (!mul_ok(R, inner, &xso) && R >= 1 && inner >= 0)
    return fail(LSE_ERR_SHAPE, "lse_reduce_axis0_ws: R * inner overflows");
  return lse_reduce_axis_strided_ws(x, out, 1, R, inner, xso, inner, inner, ws, ws_bytes, stream);
}

LSE_EXPORT lse_status_t log_softmax_axis_strided_ws(const float *x, float *y, int64_t outer,
                                                    int64_t R, int64_t inner,
                                                    int64_t x_stride_outer, int64_t x_stride_r,
                                                    int64_t y_stride_outer, int64_t y_stride_r,
                                                    void *ws, size_t ws_bytes,
                                                    hipStream_t stream) {
  const char *who = "log_softmax_axis_strided_ws";
  int64_t total;
  lse_status_t st = check_axis(who, x, y, outer, R, inner, x_stride_outer, x_stride_r,
                               y_stride_outer, y_stride_r, true, &total);
  if (st != LSE_OK) return st;
  if (total == 0) return ok();
  st = check_axis_ws(who, x, y, outer, R, inner, x_stride_outer, x_stride_r, y_stride_outer,
                     y_stride_r, true, ws, ws_bytes);
  if (st != LSE_OK) return st;
  const lse::AxisDims d{outer, R, inner, x_stride_outer, x_stride_r, y_stride_outer, y_stride_r};
  return from_hip(lse::launch_log_softmax_axis(x, y, d, stream, true, ws), who);
}

// ------------------------------------------------------------------ case B
static lse_status_t check_rows(const char *who, int64_t rows, int64_t cols, int64_t *total) {
  if (rows < 0) return fail(LSE_ERR_SHAPE, "%s: rows = %lld must be >= 0", who, (long long)rows);
  if (cols < 1) return fail(LSE_ERR_SHAPE, "%s: cols = %lld must be >= 1", who, (long long)cols);
  if (!mul_ok(rows, cols, total) || *total > kMaxElems)
    return fail(LSE_ERR_SHAPE, "%s: rows * cols overflows", who);
  return LSE_OK;
}

LSE_EXPORT lse_status_t log_softmax_rows_plan(int64_t cols, int64_t *nchunks, int64_t *chunk) {
  if (cols < 1) return fail(LSE_ERR_SHAPE, "log_softmax_rows_plan: cols must be >= 1");
  if (!nchunks || !chunk) return fail(LSE_ERR_NULL, "log_softmax_rows_plan: NULL output");
  const lse::RowsPlan p = lse::rows_plan(cols);
  *nchunks = p.nchunks;
  *chunk = p.nchunks == 1 ? cols : p.chunk;
  return ok();
}

LSE_EXPORT size_t log_softmax_rows_workspace_bytes(int64_t rows, int64_t cols) {
  int64_t total;
  if (rows < 0 || cols < 1 || !mul_ok(rows, cols, &total)) return 0;
  return lse::rows_workspace_bytes(rows, cols);
}

static lse_status_t rows_call(const char *who, bool softmax, const float *x, float *y,
                              int64_t rows, int64_t cols, int64_t ldx, int64_t ldy, void *ws,
                              size_t ws_bytes, hipStream_t stream) {
  int64_t total;
  lse_status_t st = check_rows(who, rows, cols, &total);
  if (st != LSE_OK) return st;
  if (ldx < cols || ldy < cols)
    return fail(LSE_ERR_SHAPE, "%s: ldx = %lld and ldy = %lld must be >= cols = %lld", who,
                (long long)ldx, (long long)ldy, (long long)cols);
  if (rows == 0) return ok();
  int64_t xspan, yspan;
  if (!span_ok(rows, ldx, 1, 0, cols, &xspan) || !span_ok(rows, ldy, 1, 0, cols, &yspan))
    return fail(LSE_ERR_SHAPE, "%s: rows * ld overflows", who);
  if (!x || !y) return fail(LSE_ERR_NULL, "%s: x and y must be non-NULL", who);
  if (((uintptr_t)x | (uintptr_t)y) & 3u)
    return fail(LSE_ERR_SHAPE, "%s: x and y must be 4-byte aligned (float)", who);
  if (overlaps(x, xspan * 4, y, yspan * 4))
    return fail(LSE_ERR_OVERLAP, "%s: y overlaps x (in-place is not supported)", who);
  const lse::RowsPlan p = lse::rows_plan(cols);
  if (p.nchunks > lse::kRowsMaxChunks)
    return fail(LSE_ERR_SHAPE, "%s: cols = %lld too long", who, (long long)cols);
  int64_t wgs;
  if (!mul_ok(rows, p.nchunks, &wgs) || wgs > kMaxGrid)
    return fail(LSE_ERR_SHAPE, "%s: rows * chunks = too many workgroups", who);
  if (p.nchunks > 1) {
    const size_t need = lse::rows_workspace_bytes(rows, cols);
    if (!ws) return fail(LSE_ERR_WORKSPACE, "%s: needs %zu workspace bytes", who, need);
    if (ws_bytes < need)
      return fail(LSE_ERR_WORKSPACE, "%s: workspace %zu < required %zu", who, ws_bytes, need);
    if (overlaps(ws, (int64_t)need, x, xspan * 4) || overlaps(ws, (int64_t)need, y, yspan * 4))
      return fail(LSE_ERR_OVERLAP, "%s: workspace overlaps x or y", who);
  }
  return from_hip(lse::launch_log_softmax_rows(x, y, rows, cols, ldx, ldy, ws, stream, softmax),
                  who);
}

LSE_EXPORT lse_status_t log_softmax_rows(const float *x, float *y, int64_t rows, int64_t cols,
                                         void *ws, size_t ws_bytes, hipStream_t stream) {
  return rows_call("log_softmax_rows", false, x, y, rows, cols, cols, cols, ws, ws_bytes,
                   stream);
}

LSE_EXPORT lse_status_t log_softmax_rows_noalloc(const float *x, float *y, int64_t rows,
                                                 int64_t cols, hipStream_t stream) {
  const char *who = "log_softmax_rows_noalloc";
  int64_t total;
  lse_status_t st = check_rows(who, rows, cols, &total);
  if (st != LSE_OK) return st;
  const size_t need = lse::rows_workspace_bytes(rows, cols);
  if (need > lse::kNoAllocScratchBytes)
    return fail(LSE_ERR_WORKSPACE,
                "%s: rows x chunks = %lld x %lld needs %zu bytes of scratch; the static scratch "
                "holds %zu (131040 row-chunk pairs); use log_softmax_rows with a workspace",
                who, (long long)rows, (long long)lse::rows_plan(cols).nchunks, need,
                lse::kNoAllocScratchBytes);
  void *ws = nullptr;
  if (need > 0 && rows > 0) {
    const hipError_t e = lse::noalloc_scratch(&ws);
    if (e != hipSuccess) return from_hip(e, "log_softmax_rows_noalloc: scratch address");
  }
  return rows_call(who, false, x, y, rows, cols, cols, cols, ws, need, stream);
}

LSE_EXPORT lse_status_t softmax_rows(const float *x, float *y, int64_t rows, int64_t cols,
                                     void *ws, size_t ws_bytes, hipStream_t stream) {
  return rows_call("softmax_rows", true, x, y, rows, cols, cols, cols, ws, ws_bytes, stream);
}

LSE_EXPORT lse_status_t log_softmax_rows_strided(const float *x, float *y, int64_t rows,
                                                 int64_t cols, int64_t ldx, int64_t ldy,
                                                 void *ws, size_t ws_bytes,
                                                 hipStream_t stream) {
  return rows_call("log_softmax_rows", false, x, y, rows, cols, ldx, ldy, ws, ws_bytes, stream);
}

LSE_EXPORT lse_status_t softmax_rows_strided(const float *x, float *y, int64_t rows,
                                             int64_t cols, int64_t ldx, int64_t ldy, void *ws,
                                             size_t ws_bytes, hipStream_t stream) {
  return rows_call("softmax_rows", true, x, y, rows, cols, ldx, ldy, ws, ws_bytes, stream);
}

LSE_EXPORT int64_t lse_rows_num_chunks(int64_t cols, int64_t chunk) {
  if (cols < 1 || chunk < 1) return -1;
  return (cols + chunk - 1) / chunk;
}

LSE_EXPORT lse_status_t lse_rows_partial(const float *x, int64_t rows, int64_t cols,
                                         int64_t chunk, lse_pair_t *partials,
                                         hipStream_t stream) {
  int64_t total;
  lse_status_t st = check_rows("lse_rows_partial", rows, cols, &total);
  if (st != LSE_OK) return st;
  if (chunk < 1)
    return fail(LSE_ERR_SHAPE, "lse_rows_partial: chunk = %lld must be >= 1", (long long)chunk);
  if (rows == 0) return ok();
  if (!x || !partials) return fail(LSE_ERR_NULL, "lse_rows_partial: NULL pointer");
  if (((uintptr_t)x | (uintptr_t)partials) & 3u)
    return fail(LSE_ERR_SHAPE, "lse_rows_partial: x and partials must be 4-byte aligned");
  const int64_t k = (cols + chunk - 1) / chunk;
  int64_t wgs;
  if (!mul_ok(rows, k, &wgs) || wgs > kMaxGrid)
    return fail(LSE_ERR_SHAPE, "lse_rows_partial: rows * chunks = too many workgroups");
  if (k > kMaxWorkgroups512)  // one row's chunks must fit one dispatch
    return fail(LSE_ERR_SHAPE, "lse_rows_partial: %lld chunks per row exceed one launch",
                (long long)k);
  if (overlaps(x, total * 4, partials, wgs * 8))
    return fail(LSE_ERR_OVERLAP, "lse_rows_partial: partials overlap x");
  return from_hip(lse::launch_lse_rows_partial(x, rows, cols, cols, chunk, partials, stream),
                  "lse_rows_partial launch");
}

LSE_EXPORT lse_status_t lse_rows_merge(const lse_pair_t *partials, int64_t rows,
                                       int64_t nchunks, float *row_lse, hipStream_t stream) {
  if (rows < 0) return fail(LSE_ERR_SHAPE, "lse_rows_merge: rows must be >= 0");
  if (nchunks < 1) return fail(LSE_ERR_SHAPE, "lse_rows_merge: nchunks must be >= 1");
  int64_t total;
  if (!mul_ok(rows, nchunks, &total) || total > kMaxElems)
    return fail(LSE_ERR_SHAPE, "lse_rows_merge: rows * nchunks overflows");
  if (rows == 0) return ok();
  if (!partials || !row_lse) return fail(LSE_ERR_NULL, "lse_rows_merge: NULL pointer");
  if ((rows + 3) / 4 > kMaxGrid) return fail(LSE_ERR_SHAPE, "lse_rows_merge: too many rows");
  if (overlaps(partials, total * 8, row_lse, rows * 4))
    return fail(LSE_ERR_OVERLAP, "lse_rows_merge: row_lse overlaps partials");
  return from_hip(lse::launch_lse_rows_merge(partials, rows, nchunks, row_lse, stream),
                  "lse_rows_merge launch");
}

// ------------------------------------------------------------------ case C
static lse_status_t check_chain(int64_t N, int64_t Cin, int64_t H, int64_t W, int64_t Cout,
                                int64_t K, int64_t groups) {
  if (N < 0) return fail(LSE_ERR_SHAPE, "fused_conv_gn_act_lse: N must be >= 0");
  if (Cin < 1 || Cout < 1 || K < 1 || groups < 1)
    return fail(LSE_ERR_SHAPE, "fused_conv_gn_act_lse: Cin, Cout, K, groups must be >= 1");
  if (H < K || W < K) return fail(LSE_ERR_SHAPE, "fused_conv_gn_act_lse: H, W must be >= K");
  if (Cout % groups != 0)
    return fail(LSE_ERR_SHAPE, "fused_conv_gn_act_lse: Cout %% groups != 0");
  if (H > 65536 || W > 65536) return fail(LSE_ERR_SHAPE, "fused_conv_gn_act_lse: H, W > 65536");
  int64_t t;
  if (!mul_ok(N, Cin, &t) || !mul_ok(t, H, &t) || !mul_ok(t, W, &t) || t > kMaxElems)
    return fail(LSE_ERR_SHAPE, "fused_conv_gn_act_lse: input size overflows");
  const int64_t tiles = ((H - K + 2) / 2) * ((W - K + 128) / 128);  // 2 x 128 pixel tiles
  if (!mul_ok(N, tiles, &t) || t > 0xffffffffll)  // workgroups: one or two tiles each
    return fail(LSE_ERR_SHAPE, "fused_conv_gn_act_lse: N x tiles too large for one launch");
  if (K != 3 || Cin != 8 || Cout != 64 || (16 % groups) != 0)
    return fail(LSE_ERR_UNSUPPORTED,
                "fused_conv_gn_act_lse: this build implements K=3, Cin=8, Cout=64 and groups "
                "in {1,2,4,8,16} (got K=%lld Cin=%lld Cout=%lld groups=%lld)",
                (long long)K, (long long)Cin, (long long)Cout, (long long)groups);
  return LSE_OK;
}

LSE_EXPORT size_t fused_conv_gn_act_lse_workspace_bytes(int64_t N, int64_t Cin, int64_t H,
                                                        int64_t W, int64_t Cout, int64_t K,
                                                        int64_t groups) {
  if (N < 0 || Cin < 1 || Cout < 1 || K < 1 || groups < 1 || H < K || W < K) return 0;
  return lse::conv_chain_workspace_bytes(N, Cin, H, W, Cout, K, groups);
}

LSE_EXPORT lse_status_t fused_conv_gn_act_lse(const float *x, const float *w, const float *b,
                                              const float *gamma, const float *beta, int64_t N,
                                              int64_t Cin, int64_t H, int64_t W, int64_t Cout,
                                              int64_t K, int64_t groups, float eps, float *out,
                                              void *ws, size_t ws_bytes, hipStream_t stream) {
  lse_status_t st = check_chain(N, Cin, H, W, Cout, K, groups);
  if (st != LSE_OK) return st;
  if (!(eps >= 0.0f)) return fail(LSE_ERR_SHAPE, "fused_conv_gn_act_lse: eps must be >= 0");
  if (N == 0) return ok();
  if (!x || !w || !out) return fail(LSE_ERR_NULL, "fused_conv_gn_act_lse: x, w, out required");
  const size_t need = lse::conv_chain_workspace_bytes(N, Cin, H, W, Cout, K, groups);
  if (!ws) return fail(LSE_ERR_WORKSPACE, "fused_conv_gn_act_lse: needs %zu bytes", need);
  if (ws_bytes < need)
    return fail(LSE_ERR_WORKSPACE, "fused_conv_gn_act_lse: workspace %zu < required %zu",
                ws_bytes, need);
  const int64_t in_bytes = N * Cin * H * W * 4;
  const int64_t out_bytes = N * (H - K + 1) * (W - K + 1) * 4;
  // every input (x, w, b, gamma, beta) against both buffers the call writes
  const void *ins[5] = {x, w, b, gamma, beta};
  const int64_t in_sizes[5] = {in_bytes, Cout * Cin * K * K * 4, Cout * 4, Cout * 4, Cout * 4};
  bool clash = overlaps(ws, (int64_t)need, out, out_bytes);
  for (int i = 0; i < 5; ++i)
    clash = clash || (ins[i] && (overlaps(ins[i], in_sizes[i], out, out_bytes) ||
                                 overlaps(ins[i], in_sizes[i], ws, (int64_t)need)));
  if (clash)
    return fail(LSE_ERR_OVERLAP, "fused_conv_gn_act_lse: out / workspace overlap an input");
  return from_hip(lse::launch_conv_chain(x, w, b, gamma, beta, N, Cin, H, W, Cout, K, groups,
                                         eps, out, ws, stream),
                  "fused_conv_gn_act_lse launch");
}
