/*
 * lse.h — C ABI of the MI355X (gfx950) max-shifted log-sum-exp engine.
 *
 * Every operation here evaluates  LSE(v) = m + log(sum_i exp(v_i - m)),
 * m = max_i v_i, over some set of fp32 values, in one of three layouts.
 * Sources, cited by page and passage (three kernel-benchmark transcripts):
 *   [LSE0]  POPCORNBENCH FW-GLM-5-1 l1_p29 — torch.logsumexp(x, dim=0) on an
 *           (R,B,D) tensor; the benchmark spec and the max / sum / log plan.
 *   [LSM]   POPCORNBENCH Kimi-K2.6 l1_p24 — LogSoftmax over dim 1 of
 *           (4096, 393216); the opening formula, the online (max, sum)
 *           recurrence, the pairwise combine and the multi-block-per-row idea.
 *   [CHAIN] POPCORNBENCH Kimi-K2.6 l2_p92 — Conv2d -> GroupNorm -> Tanh ->
 *           Hardswish -> residual add -> LogSumExp over dim 1.
 *
 * Conventions for every entry point:
 *   - Data pointers are DEVICE pointers the caller owns (allocated with
 *     hipMalloc or a framework allocator on the current device).  The library
 *     never allocates, frees or synchronises; every call only enqueues kernels
 *     on `stream` (0 = the null stream) and returns.
 *   - All tensors are fp32, dense and row-major (C order).  Sizes are int64.
 *     Pointers of the row calls (log_softmax_rows, softmax_rows,
 *     lse_rows_partial and their forms) must be 4-byte aligned, the natural
 *     alignment of float (LSE_ERR_SHAPE otherwise); the other calls accept
 *     any alignment.  Rows go through 128-bit loads and stores from their
 *     first 16-byte boundary on, with a few single-value loads and stores
 *     for the head and tail of a row that does not start or end on one.
 *   - Arguments are validated on the host before anything is enqueued; on any
 *     failure nothing is launched, a status != LSE_OK is returned and
 *     lse_last_error() describes it (thread-local string, valid until the next
 *     call on the same thread).  LSE_ERR_HIP reports a failed launch.
 *   - Non-finite values follow log(sum(exp(v))) literally: -inf entries are
 *     ignored (exp(-inf) = 0); all entries -inf gives -inf; any +inf gives
 *     +inf; any NaN gives NaN.  log_softmax is x - LSE(row) elementwise.
 *   - Outputs must not overlap inputs (LSE_ERR_OVERLAP where detectable).
 *   - Concurrent calls that share a workspace race; give each in-flight call
 *     its own workspace.
 */
#ifndef LSE_MI355X_H
#define LSE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* One (max, sum) partial of a set of values: LSE(set) = m + log(s).
 *   m = largest non-NaN value (-inf if none);
 *   s = sum of exp(v - m): 0 when m = -inf; when m = +inf, the number of +inf
 *       values; NaN when the set holds a NaN.
 * The identity of the combine is {-inf, 0}.                 [LSM] pairwise combine */
typedef struct lse_pair_t {
  float m;
  float s;
} lse_pair_t;

typedef enum lse_status_t {
  LSE_OK = 0,
  LSE_ERR_NULL = 1,        /* a required pointer is NULL                       */
  LSE_ERR_SHAPE = 2,       /* a size is out of range or inconsistent           */
  LSE_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required       */
  LSE_ERR_OVERLAP = 4,     /* an output overlaps an input                      */
  LSE_ERR_HIP = 5,         /* the HIP runtime reported an error on launch      */
  LSE_ERR_UNSUPPORTED = 6  /* valid request outside what this build implements */
} lse_status_t;

/* Short static name of a status code ("LSE_OK", ...). */
const char *lse_status_string(int status);
/* Detail of the last failure on the calling thread ("" if none). */
const char *lse_last_error(void);
/* ABI version of this header (bumped on any incompatible change). */
int lse_abi_version(void);
#define LSE_ABI_VERSION 1

/* ---------------------------------------------------------------- case A
 * logsumexp over the leading axis.                   [LSE0] task statement
 *   out[j] = LSE_{r < R} x[r * inner + j],   0 <= j < inner.
 * x: (R, inner) row-major, i.e. an (R, B, D) tensor reduced over dim 0 has
 * inner = B * D.  out: inner floats.  R >= 1, inner >= 0 (inner == 0 is a
 * no-op).  out must not overlap x. */
lse_status_t lse_reduce_axis0(const float *x, float *out, int64_t R,
                              int64_t inner, hipStream_t stream);

/* The same reduction over the middle axis of a row-major (outer, R, inner)
 * array; outer = 1 is lse_reduce_axis0.  An (N, C, H, W) tensor reduced over
 * dim 1 is outer = N, R = C, inner = H * W.   [LSE0] task statement; [CHAIN]
 * the logsumexp over dim 1.
 *   lse_reduce_axis:  out[o * inner + j] = LSE_r x[(o * R + r) * inner + j]
 *                     (out: outer x inner floats)
 *   log_softmax_axis: y[(o*R + r)*inner + j] = x[...] - LSE_r' x[(o*R + r')*inner + j]
 *                     (y: same shape as x; x is read once when R <= 256 and
 *                     inner, x and y allow 16-byte vectors, or R <= 128
 *                     otherwise; twice beyond)
 * outer, inner >= 0 (0 is a no-op), R >= 1; outputs must not overlap x. */
lse_status_t lse_reduce_axis(const float *x, float *out, int64_t outer,
                             int64_t R, int64_t inner, hipStream_t stream);
lse_status_t log_softmax_axis(const float *x, float *y, int64_t outer,
                              int64_t R, int64_t inner, hipStream_t stream);
/* Strided forms of the two calls above, for views into larger buffers (a
 * slice of planes or of the inner run, a padded channel pitch).  Strides are
 * in elements, >= 0; the inner index is contiguous:
 *   lse_reduce_axis_strided:  out[o * out_stride_outer + j]
 *                               = LSE_r x[o * x_stride_outer + r * x_stride_r + j]
 *   log_softmax_axis_strided: y[o * y_stride_outer + r * y_stride_r + j]
 *                               = x[o * x_stride_outer + r * x_stride_r + j] - LSE_r' (...)
 * The contiguous calls are x_stride_outer = R inner, x_stride_r = inner (and
 * the same for y; out_stride_outer = inner).  Outputs may not collide:
 * y_stride_r >= inner when R > 1, and the outer stride of the output is at
 * least the extent of one outer block ((R - 1) y_stride_r + inner, or inner
 * for logsumexp) when outer > 1; otherwise LSE_ERR_SHAPE.  x may overlap
 * itself (it is only read).  The whole address range of the output may not
 * intersect that of x (LSE_ERR_OVERLAP, even where the two would interleave
 * without sharing an element).  Columns are read and written 4 at a time
 * with 16-byte accesses whenever x and the output are 4-byte aligned and
 * inner >= 4 (at any 4-byte phase and any stride: the last 4 columns of a
 * run whose inner is not a multiple of 4 are read as one access and only the
 * columns not covered before are written); other layouts take one value at a
 * time. */
lse_status_t lse_reduce_axis_strided(const float *x, float *out, int64_t outer,
                                     int64_t R, int64_t inner,
                                     int64_t x_stride_outer, int64_t x_stride_r,
                                     int64_t out_stride_outer, hipStream_t stream);
lse_status_t log_softmax_axis_strided(const float *x, float *y, int64_t outer,
                                      int64_t R, int64_t inner,
                                      int64_t x_stride_outer, int64_t x_stride_r,
                                      int64_t y_stride_outer, int64_t y_stride_r,
                                      hipStream_t stream);

/* The axis calls above with a caller's workspace, for few outputs over many
 * planes (the logsumexp over dim 0 of (R, B, D) with B D small and R large):
 * there the calls without a workspace leave most of the GPU idle, since the
 * planes of one output run can only be split across the waves of one
 * workgroup.  With a workspace the planes of each run of outputs are split
 * across workgroups whose per-output (max, sum) pairs are merged by a second
 * launch in a fixed order (log_softmax then writes y in a third launch, so x
 * is read twice there); contiguous (R, inner) blocks of short runs split the
 * same way along the block; and long contiguous last-axis rows take the
 * split-row kernels of case B.  The reduction each output receives is the same as
 * without a workspace; only the order of the additions differs.
 *   lse_axis_workspace_bytes: bytes the call with these sizes needs (0 when
 *     none of the split paths applies, in which case ws may be NULL);
 *     log_softmax != 0 for log_softmax_axis_strided_ws.  0 for invalid sizes.
 *   ws: device memory of at least that many bytes, not overlapping x or the
 *     output; its contents on entry are irrelevant and it is scratch until
 *     the call's launches on `stream` have finished.  Concurrent calls need
 *     separate workspaces.  Missing or too small: LSE_ERR_WORKSPACE; other
 *     arguments and errors as for the calls without a workspace.
 *                  [LSE0] task statement; [LSM] the two-phase (max, sum) merge. */
size_t lse_axis_workspace_bytes(int64_t outer, int64_t R, int64_t inner,
                                int log_softmax);
lse_status_t lse_reduce_axis0_ws(const float *x, float *out, int64_t R,
                                 int64_t inner, void *ws, size_t ws_bytes,
                                 hipStream_t stream);
lse_status_t lse_reduce_axis_strided_ws(const float *x, float *out, int64_t outer,
                                        int64_t R, int64_t inner,
                                        int64_t x_stride_outer, int64_t x_stride_r,
                                        int64_t out_stride_outer, void *ws,
                                        size_t ws_bytes, hipStream_t stream);
lse_status_t log_softmax_axis_strided_ws(const float *x, float *y, int64_t outer,
                                         int64_t R, int64_t inner,
                                         int64_t x_stride_outer, int64_t x_stride_r,
                                         int64_t y_stride_outer, int64_t y_stride_r,
                                         void *ws, size_t ws_bytes,
                                         hipStream_t stream);

/* ---------------------------------------------------------------- case B
 * Row-wise log_softmax over the last axis.           [LSM] opening formula
 *   y[r, c] = x[r, c] - LSE_c x[r, :],   (rows, cols) row-major.
 * Rows longer than one workgroup's register tile are split across several
 * workgroups whose (max, sum) partials are merged through `ws`
 *                                           [LSM] multi-block-per-row idea.
 * Rows of up to 128 such chunks (4M columns) read x once; longer rows take
 * three launches (chunk pairs, a merge per row, the write), reading x twice.
 * ws: device workspace of at least log_softmax_rows_workspace_bytes(rows,
 * cols) bytes (0 for short rows, in which case ws may be NULL).  Its contents
 * on entry are irrelevant: the call clears what it uses with a kernel on
 * `stream`.  y must not overlap x (no in-place).  rows >= 0, cols >= 1. */
size_t log_softmax_rows_workspace_bytes(int64_t rows, int64_t cols);
lse_status_t log_softmax_rows(const float *x, float *y, int64_t rows,
                              int64_t cols, void *ws, size_t ws_bytes,
                              hipStream_t stream);
/* log_softmax_rows for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation, launches and results as
 * log_softmax_rows on the same (rows, cols), but the split rows' pair
 * workspace is a static device array inside the library (1 MiB per GPU the
 * library runs on, held until the process ends) instead of a caller buffer.
 * It allocates nothing.  Calls whose pairs exceed that array (rows x
 * ceil(cols / 32768) > 131040 for rows of up to 128 chunks, e.g. more than
 * 10920 rows of 393216 columns; rows x (ceil(cols / 16384) + 1) > 131040 for
 * longer rows) return LSE_ERR_WORKSPACE with nothing launched.  All calls on one
 * GPU share the array: calls that overlap on one GPU (other streams, other
 * threads) race and must not be enqueued concurrently; consecutive calls on
 * one stream are fine (each clears what it uses with a kernel). */
lse_status_t log_softmax_rows_noalloc(const float *x, float *y, int64_t rows,
                                      int64_t cols, hipStream_t stream);
/* Row-wise softmax, the non-log form: y[r, c] = exp(x[r, c] - LSE_c x[r, :]).
 * Same layout, split and workspace (log_softmax_rows_workspace_bytes) as
 * log_softmax_rows.                          [LSM] the standard-softmax variant */
lse_status_t softmax_rows(const float *x, float *y, int64_t rows, int64_t cols,
                          void *ws, size_t ws_bytes, hipStream_t stream);
/* A split row's workgroups wait for each other's (max, sum) pairs; one that
 * has waited about 50 us computes the missing pairs itself from x, with the
 * same arithmetic in the same order as their owners, so the results are
 * bit-identical whichever workgroup computes a pair.
 *
 * log_softmax_rows / softmax_rows over rows that sit ldx (x) and ldy (y)
 * elements apart, e.g. the first cols columns of a wider matrix: row r of x
 * starts at x + r * ldx.  ldx, ldy >= cols (else LSE_ERR_SHAPE); the
 * workspace is the same as for the contiguous call.  The address ranges
 * spanned by x and y may not intersect (LSE_ERR_OVERLAP).  The 16-byte
 * path needs ldx, ldy and cols to be multiples of 4. */
lse_status_t log_softmax_rows_strided(const float *x, float *y, int64_t rows,
                                      int64_t cols, int64_t ldx, int64_t ldy,
                                      void *ws, size_t ws_bytes,
                                      hipStream_t stream);
lse_status_t softmax_rows_strided(const float *x, float *y, int64_t rows,
                                  int64_t cols, int64_t ldx, int64_t ldy,
                                  void *ws, size_t ws_bytes, hipStream_t stream);
/* The split log_softmax_rows will use for a row length: *nchunks workgroups
 * per row, each covering *chunk consecutive columns (the last may be short).
 * Host-only; enqueues nothing. */
lse_status_t log_softmax_rows_plan(int64_t cols, int64_t *nchunks,
                                   int64_t *chunk);

/* Case B building blocks: per-chunk partials, then their merge.  Together
 * they give the row logsumexp of a row split across workgroups (or across
 * devices, by merging gathered partials).     [LSM] multi-block-per-row idea
 *   lse_rows_num_chunks(cols, chunk) = ceil(cols / chunk)  (-1 if invalid).
 *   lse_rows_partial: partials[r * nchunks + k] = the lse_pair_t of columns
 *     [k*chunk, min((k+1)*chunk, cols)) of row r.  chunk >= 1.
 *   lse_rows_merge: row_lse[r] = LSE of the nchunks pairs of row r:
 *     M = max_k m_k, S = sum_k s_k * (m_k == M ? 1 : exp(m_k - M)),
 *     row_lse = M + log(S)  (= M when M is +-inf, NaN if any pair has NaN).
 *                                                  [LSM] pairwise combine */
int64_t lse_rows_num_chunks(int64_t cols, int64_t chunk);
lse_status_t lse_rows_partial(const float *x, int64_t rows, int64_t cols,
                              int64_t chunk, lse_pair_t *partials,
                              hipStream_t stream);
lse_status_t lse_rows_merge(const lse_pair_t *partials, int64_t rows,
                            int64_t nchunks, float *row_lse,
                            hipStream_t stream);

/* ---------------------------------------------------------------- case C
 * The chain conv2d -> GroupNorm -> tanh -> hardswish -> residual add ->
 * logsumexp over channels, fused.                [CHAIN] the model's forward
 *   v0  = conv2d(x, w, b)   stride 1, no padding: (N, Cout, Ho, Wo),
 *         Ho = H - K + 1, Wo = W - K + 1
 *   v1  = GroupNorm(v0; groups, eps, gamma, beta)  (population variance over
 *         the Cout/groups channels and Ho*Wo pixels of each (sample, group))
 *   v4  = v0 + hardswish(tanh(v1)),  hardswish(t) = t * min(max(t+3,0),6) / 6
 *   out[n, 0, h, w] = LSE_c v4[n, c, h, w]          (N, 1, Ho, Wo)
 * x (N, Cin, H, W); w (Cout, Cin, K, K); b (Cout) or NULL; gamma, beta (Cout)
 * or NULL (meaning 1 and 0).  This build implements K == 3, Cin == 8,
 * Cout == 64 and groups dividing 64 into groups of 4 channels or more
 * (LSE_ERR_UNSUPPORTED otherwise).  ws: at least
 * fused_conv_gn_act_lse_workspace_bytes(...) bytes; on return (once the
 * stream has run the call) its first 2 * N * groups floats hold the
 * per-(n, g) mean followed by the per-(n, g) 1/sqrt(var + eps).
 * The conv runs once when a sample's 2 x 256-pixel tile pairs number at most
 * half of what the device can hold resident (one launch whose workgroups wait
 * for their sample's statistics); larger samples take two launches, the
 * first publishing the statistics, the second recomputing the conv and
 * applying them (the conv runs twice; nothing waits).  Both give identical
 * results.  A workgroup whose wait runs out (about 0.5 ms, e.g. when other
 * work holds the GPU) leaves its tiles to the launch's last workgroup, which
 * finishes them once every statistic is in: results are the same either way
 * and never depend on scheduling. */
size_t fused_conv_gn_act_lse_workspace_bytes(int64_t N, int64_t Cin, int64_t H,
                                             int64_t W, int64_t Cout,
                                             int64_t K, int64_t groups);
lse_status_t fused_conv_gn_act_lse(const float *x, const float *w,
                                   const float *b, const float *gamma,
                                   const float *beta, int64_t N, int64_t Cin,
                                   int64_t H, int64_t W, int64_t Cout,
                                   int64_t K, int64_t groups, float eps,
                                   float *out, void *ws, size_t ws_bytes,
                                   hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LSE_MI355X_H */
