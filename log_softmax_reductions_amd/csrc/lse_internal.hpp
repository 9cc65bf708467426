// lse_internal.hpp — host-side interface between the C ABI (lse_api.hip) and
// the kernel launchers.  Launchers assume validated arguments and return the
// hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lse {

// ---------------------------------------------------------------- case A
// Geometry of an axis reduction, strides in elements: x[o * xso + r * xsr + j]
// for o < outer, r < R, j < inner (j contiguous).  The logsumexp output is
// out[o * yso + j]; the log_softmax output is y[o * yso + r * ysr + j].
struct AxisDims {
  int64_t outer, R, inner;
  int64_t xso, xsr;
  int64_t yso, ysr;
};
// with_ws: the call comes from an entry point that takes a workspace, and ws
// holds at least axis_workspace_bytes(d.outer, d.R, d.inner, lsm) bytes (ws
// may be null when that is 0).
hipError_t launch_lse_axis(const float *x, float *out, const AxisDims &d, hipStream_t stream,
                           bool with_ws = false, void *ws = nullptr);
hipError_t launch_log_softmax_axis(const float *x, float *y, const AxisDims &d,
                                   hipStream_t stream, bool with_ws = false, void *ws = nullptr);
// Workspace of the entry points that take one: enough for whichever of the
// split paths (column split, split rows) the call's sizes can take; 0 when
// none of them splits.
size_t axis_workspace_bytes(int64_t outer, int64_t R, int64_t inner, bool lsm);

// Few outputs over many planes (lse_cols.hip): the planes of each tile of
// columns split across workgroups.  launch_cols returns false when the call
// does not take this path; otherwise e is the launch status.
size_t cols_workspace_bytes(const AxisDims &d, bool lsm);
bool launch_cols(const float *x, float *out, const AxisDims &d, bool lsm, bool with_ws, void *ws,
                 hipStream_t stream, hipError_t &e);

// Contiguous (R, inner) blocks with a short inner run (lse_blocks.hip): each
// block read as one flat run through LDS.  launch_blocks returns false when
// the call does not take this path; otherwise e is the launch status.
size_t blocks_workspace_bytes(const AxisDims &d, bool lsm);
bool launch_blocks(const float *x, float *out, const AxisDims &d, bool lsm, bool with_ws,
                   void *ws, hipStream_t stream, hipError_t &e);

// ---------------------------------------------------------------- case B
// Tile geometry of the row kernels (overridable at build time for sweeps).
#ifndef LSE_ROWS_THREADS
#define LSE_ROWS_THREADS 512
#endif
#ifndef LSE_ROWS_MAX_VPL
#define LSE_ROWS_MAX_VPL 32
#endif
#ifndef LSE_ROWS_SPLIT_VPL
#define LSE_ROWS_SPLIT_VPL 64   // floats per lane of a log_softmax_rows / softmax_rows chunk
#endif
constexpr int kRowsThreads = LSE_ROWS_THREADS;  // lanes per workgroup
constexpr int kRowsMaxVpl = LSE_ROWS_MAX_VPL;   // floats held per lane
constexpr int64_t kRowsTile = (int64_t)kRowsThreads * kRowsMaxVpl;  // 16384 columns
// Chunk of the split log_softmax / softmax rows: 32768 columns (128 KiB)
// per workgroup measured 5 % faster than 16384 on (4096, 393216).
constexpr int64_t kRowsSplitTile = (int64_t)kRowsThreads * LSE_ROWS_SPLIT_VPL;
static_assert(LSE_ROWS_SPLIT_VPL % 4 == 0 && LSE_ROWS_SPLIT_VPL >= LSE_ROWS_MAX_VPL &&
                  LSE_ROWS_MAX_VPL <= 32,
              "register tiles: up to 32 floats per lane, the split chunk at least that");
constexpr int64_t kRowsMaxChunks = 1 << 20;

// Split workspace: a 256-byte header, then rows * nchunks packed pairs.
struct RowsWsHeader {
  uint32_t reserved;
  uint32_t helped;   // chunk pairs computed by a sibling workgroup, not their owner
  uint32_t pad[62];
};
static_assert(sizeof(RowsWsHeader) == 256, "header is 256 bytes");

struct RowsPlan {
  int64_t nchunks;
  int64_t chunk;
};
RowsPlan rows_plan(int64_t cols);
size_t rows_workspace_bytes(int64_t rows, int64_t cols);

// Row r of x starts at x + r * ldx, of y at y + r * ldy (ld >= cols).
hipError_t launch_log_softmax_rows(const float *x, float *y, int64_t rows, int64_t cols,
                                   int64_t ldx, int64_t ldy, void *ws, hipStream_t stream,
                                   bool softmax = false);
// keep: x is read again by a later launch (cached loads instead of non-temporal).
hipError_t launch_lse_rows_partial(const float *x, int64_t rows, int64_t cols, int64_t ldx,
                                   int64_t chunk, void *partials, hipStream_t stream,
                                   bool keep = false);
hipError_t launch_lse_rows_merge(const void *partials, int64_t rows,
                                 int64_t nchunks, float *row_lse,
                                 hipStream_t stream);
// One workgroup per row, no workspace: out[r * ldo] = LSE of row r, and
// log_softmax / softmax of rows of any length (rows longer than the register
// tile re-read x).
hipError_t launch_rows_lse(const float *x, int64_t rows, int64_t cols, int64_t ldx, float *out,
                           int64_t ldo, hipStream_t stream);
hipError_t launch_log_softmax_rows_no_ws(const float *x, float *y, int64_t rows, int64_t cols,
                                         int64_t ldx, int64_t ldy, hipStream_t stream,
                                         bool softmax = false);
// Axis reductions whose (R, inner) blocks are short contiguous rows (inner 2
// or 4, planes contiguous in a block, R * inner <= 1024 and a multiple of 4,
// block pitches multiples of 4): the short-row segments with interleaved
// outputs.  False when the call does not fit; otherwise e is the launch status.
bool launch_axis_seg(const float *x, float *out, const AxisDims &d, bool lsm,
                     hipStream_t stream, hipError_t &e);
void set_spin_limit(uint32_t polls);
void set_rows_reread(bool on);
uint32_t chain_spin_limit();

// Static device scratch of log_softmax_rows_noalloc: a 256-byte header plus
// (1 MiB - 256) / 8 = 131040 packed pairs.  noalloc_scratch() returns its
// address on the current device (resolved once per device).
constexpr size_t kNoAllocScratchBytes = size_t(1) << 20;
hipError_t noalloc_scratch(void **ptr);

// ---------------------------------------------------------------- case C
// Test hook: 0 automatic, 1 fused, 2 statistics + recomputing apply,
// 3 statistics + staged apply (per host thread).
void set_chain_path(int path);
size_t conv_chain_workspace_bytes(int64_t N, int64_t Cin, int64_t H, int64_t W,
                                  int64_t Cout, int64_t K, int64_t groups);
hipError_t launch_conv_chain(const float *x, const float *w, const float *b,
                             const float *gamma, const float *beta, int64_t N,
                             int64_t Cin, int64_t H, int64_t W, int64_t Cout,
                             int64_t K, int64_t groups, float eps, float *out,
                             void *ws, hipStream_t stream);

}  // namespace lse
