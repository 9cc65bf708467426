// lse_cols.hip — logsumexp and log_softmax over the middle axis of an
// (outer, R, inner) array when the axis kernels' 4-output lanes would leave
// the GPU short of waves: few outputs (outer x inner) over many planes (the
// logsumexp over dim 0 of (R, B, D) with R in the hundreds of thousands and
// B D in the tens, say), or narrow inner runs over a few thousand outer
// blocks.
//
// POPCORNBENCH FW-GLM-5-1 l1_p29 (torch.logsumexp over dim 0 of (R,B,D)): every
// output is an independent max-shifted sum over its R values.  With one lane
// per 4 outputs, few outputs leave almost every lane of the GPU idle, and a
// run of fewer than 256 outputs gives a wave's load of one plane only a few
// bytes.  Here:
//   * LPP lanes (a power of two up to 64) share each plane of a tile of
//     4 LPP columns, so a wave reads 64 / LPP consecutive planes per load
//     instruction and each load of a packed (R, inner) array is one contiguous
//     span of up to 1 KiB; each lane folds its 4 columns' running (m, s) over
//     blocks of 4 planes (fold_block: exact max, one rescale per block).
//   * The planes of a tile are split into chunks, one workgroup each; with a
//     workspace the chunks' (m, s) pairs are merged by a second launch (fixed
//     chunk order, so results do not depend on timing).  Without one (the
//     entry points that take none) each tile is one chunk.
//   * Inside a workgroup the pairs of lanes sharing columns are merged with
//     xor shuffles, then the 4 waves' through LDS, always in the same order.
//   * log_softmax: (x - M) - log S is written by the same workgroup, which
//     reads its planes again (one chunk per tile), or by an apply launch over
//     the chunks after the merge launch has stored each column's (M, log S);
//     the pair launch then reads x with cached loads, so that part of the
//     second read can come from the Infinity Cache.
#include <type_traits>

#include "lse_device.hpp"
#include "lse_fold.hpp"
#include "lse_internal.hpp"

namespace lse {
namespace {

#ifndef LSE_COLS_A4
#define LSE_COLS_A4 1      // log_softmax runs off the 16-byte grid: 16-byte accesses at 4-byte alignment
#endif
// (logsumexp keeps one value per access there: 16-byte accesses at differing
// 4-byte phases measured 7-25 % slower for it, and up to 25 % faster for the
// log_softmax launches)
#ifndef LSE_COLS_WAVES
#define LSE_COLS_WAVES 4   // waves per workgroup
#endif
#ifndef LSE_COLS_U
#define LSE_COLS_U 4       // plane steps loaded before they are folded
#endif
constexpr int kColsWaves = LSE_COLS_WAVES;
constexpr int kColsThreads = kColsWaves * kWave;
constexpr int kColsU = LSE_COLS_U;
#ifndef LSE_COLS_MAX_OUTPUTS
#define LSE_COLS_MAX_OUTPUTS 32768   // without a workspace: up to this many outputs
#endif
#ifndef LSE_COLS_MAX_WAVES
#define LSE_COLS_MAX_WAVES 1024      // with one: while the axis kernels would get this few waves
#endif
#ifndef LSE_COLS_NARROW
#define LSE_COLS_NARROW 128          // ... for inner runs up to this wide,
#endif
#ifndef LSE_COLS_WIDE_MAX_WAVES
#define LSE_COLS_WIDE_MAX_WAVES 64   // ... and this few for wider ones
#endif
#ifndef LSE_COLS_LSM_MAX_WAVES
#define LSE_COLS_LSM_MAX_WAVES 64    // ... and, with more waves than this,
#endif
#ifndef LSE_COLS_LSM_MINR
#define LSE_COLS_LSM_MINR 1024       // ... log_softmax over at least this many planes
#endif
#ifndef LSE_COLS_OFFGRID_MINR
#define LSE_COLS_OFFGRID_MINR 768    // ... logsumexp off the 16-byte grid over at least this many
#endif
#ifndef LSE_COLS_MIN_PLANES_LOW
#define LSE_COLS_MIN_PLANES_LOW 128  // chunks down to this many planes when few workgroups
#endif
#ifndef LSE_COLS_MINR
#define LSE_COLS_MINR 64             // ... over at least this many planes
#endif
#ifndef LSE_COLS_TARGET_GROUPS
#define LSE_COLS_TARGET_GROUPS 2048  // workgroups the chunking aims for
#endif
#ifndef LSE_COLS_LSM_KEEP
#define LSE_COLS_LSM_KEEP 1          // log_softmax pairs read x with cached loads
#endif
#ifndef LSE_COLS_MIN_ITERS
#define LSE_COLS_MIN_ITERS 4         // ... and at least this many loop trips per lane
#endif
#ifndef LSE_COLS_MIN_PLANES
#define LSE_COLS_MIN_PLANES 512      // planes per chunk at least
#endif

// kColsPartialKeep: the pairs of a log_softmax, whose apply launch reads x
// again (cached loads, so that x may still be in the Infinity Cache).
enum ColsMode { kColsPartial = 0, kColsLse = 1, kColsLsm = 2, kColsPartialKeep = 3 };

typedef float v4f16 __attribute__((ext_vector_type(4)));

// How a lane's 4 columns are read and written: one 16-byte access at 16-byte
// alignment (kColA16: x, y, inner and the strides all multiples of 4 floats)
// or at 4-byte alignment (kColA4: inner >= 4; the run's last vector, which
// would pass its end, is read as the run's last 4 values, those the lane
// before holds counted as -inf, and written value by value), or one value per
// access (kColScalar: inner < 4).
enum ColLayout { kColA16 = 0, kColA4 = 1, kColScalar = 2 };
typedef float v4a4c __attribute__((ext_vector_type(4), aligned(4)));

// Column e (0..3) of lane cl within a tile of 4 LPP columns: vector lanes hold
// 4 consecutive columns, scalar lanes every LPP-th column.
template <int LPP, int LAY>
__device__ __forceinline__ int tile_col(int cl, int e) {
  return LAY != kColScalar ? 4 * cl + e : cl + LPP * e;
}

// The lane's 4 values of one plane row p (the tile's first column); columns
// at or past ncols read -inf.
template <int LPP, int LAY, bool NT>
__device__ __forceinline__ void cols_load(const float *p, int cl, int64_t ncols, float (&v)[4]) {
  const float ninf = -__builtin_inff();
  if constexpr (LAY == kColA16) {  // ncols % 4 == 0: a vector is wholly in or out
    if (4 * cl < ncols) {
      const v4f16 *q = reinterpret_cast<const v4f16 *>(p + 4 * cl);
      const v4f16 t = NT ? __builtin_nontemporal_load(q) : *q;
      v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = ninf;
    }
  } else if constexpr (LAY == kColA4) {
    const int j = 4 * cl;
    if (j + 4 <= ncols) {
      const v4a4c *q = reinterpret_cast<const v4a4c *>(p + j);
      const v4a4c t = NT ? __builtin_nontemporal_load(q) : *q;
      v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    } else if (j < ncols) {
      // the run's last 4 values (p + ncols - 4 is in the plane: inner >= 4)
      const v4a4c *q = reinterpret_cast<const v4a4c *>(p + ncols - 4);
      const v4a4c t = NT ? __builtin_nontemporal_load(q) : *q;
      const int64_t rem = ncols - j;  // 1..3 of them are this lane's
      v[0] = rem == 3 ? t.y : (rem == 2 ? t.z : t.w);
      v[1] = rem == 3 ? t.z : (rem == 2 ? t.w : ninf);
      v[2] = rem == 3 ? t.w : ninf;
      v[3] = ninf;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = ninf;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = tile_col<LPP, kColScalar>(cl, e);
      v[e] = (j < ncols) ? (NT ? __builtin_nontemporal_load(p + j) : p[j]) : ninf;
    }
  }
}

template <int LPP, int LAY>
__device__ __forceinline__ void cols_store(float *p, int cl, int64_t ncols, const float (&r)[4]) {
  if constexpr (LAY == kColA16) {
    if (4 * cl < ncols)
      __builtin_nontemporal_store(v4f16{r[0], r[1], r[2], r[3]}, reinterpret_cast<v4f16 *>(p + 4 * cl));
  } else if constexpr (LAY == kColA4) {
    const int j = 4 * cl;
    if (j + 4 <= ncols) {
      __builtin_nontemporal_store(v4a4c{r[0], r[1], r[2], r[3]}, reinterpret_cast<v4a4c *>(p + j));
    } else {
#pragma unroll
      for (int e = 0; e < 3; ++e)
        if (j + e < ncols) __builtin_nontemporal_store(r[e], p + j + e);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = tile_col<LPP, kColScalar>(cl, e);
      if (j < ncols) __builtin_nontemporal_store(r[e], p + j);
    }
  }
}

// y = (x - M) - log S over the lane's planes r, r + STEP, ... < r1, kColsU
// planes loaded before any is written.
template <int LPP, int LAY, int STEP>
__device__ __forceinline__ void cols_write(const float *xt, float *yt, int64_t xsr, int64_t ysr,
                                           int64_t r, int64_t r1, int cl, int64_t ncols,
                                           const float (&fm)[4], const float (&fl)[4]) {
  for (; r < r1; r += STEP * kColsU) {
    float q[kColsU][4];
#pragma unroll
    for (int u = 0; u < kColsU; ++u)
      if (r + u * STEP < r1) cols_load<LPP, LAY, true>(xt + (r + u * STEP) * xsr, cl, ncols, q[u]);
#pragma unroll
    for (int u = 0; u < kColsU; ++u) {
      if (r + u * STEP < r1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) q[u][e] = (q[u][e] - fm[e]) - fl[e];
        cols_store<LPP, LAY>(yt + (r + u * STEP) * ysr, cl, ncols, q[u]);
      }
    }
  }
}

// Merge of the running pairs of lanes whose index differs only in bits >=
// log2(LPP) (the lanes that hold the same columns): every such lane ends with
// the same (M, S), each step combining the same two values.
template <int LPP>
__device__ __forceinline__ void merge_lanes(float &m, float &s) {
  float M = m;
#pragma unroll
  for (int k = LPP; k < kWave; k <<= 1) M = fmaxf(M, __shfl_xor(M, k));
  float S = fold_weighted(m, s, M);
#pragma unroll
  for (int k = LPP; k < kWave; k <<= 1) S += __shfl_xor(S, k);
  m = M;
  s = S;
}

// Workgroup (o, tile t, chunk c) of an (outer, ctiles, chunks) grid, chunk
// fastest: folds planes [c rc, min(R, (c + 1) rc)) of the tile's columns.
//   kColsPartial: pairs[((o ctiles + t) C + col) chunks + c] = the chunk's
//                 (m, s) per column (each column's chunks contiguous)
//   kColsLse (one chunk): out[o yso + j] = m + log s
//   kColsLsm (one chunk): y[o yso + r ysr + j] = (x - m) - log s, re-reading x
template <int LPP, int LAY, int MODE>
__global__ __launch_bounds__(kColsThreads) void axis_cols_kernel(
    const float *__restrict__ x, float *__restrict__ out, AxisDims d, int64_t ctiles,
    int64_t chunks, int64_t rc, float2 *__restrict__ pairs) {
  constexpr int kGroups = kWave / LPP;          // planes per wave and step
  constexpr int kStep = kColsWaves * kGroups;   // planes per workgroup and step
  constexpr int C = 4 * LPP;                    // columns per tile
  __shared__ float2 lds_pair[kColsWaves][C];
  __shared__ float2 lds_fin[C];
  const int64_t b = blockIdx.x;
  const int64_t c = b % chunks;
  const int64_t ot = b / chunks;
  const int64_t t = ot % ctiles;
  const int64_t o = ot / ctiles;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int cl = lane % LPP;
  const int g = wave * kGroups + lane / LPP;  // the lane's plane within a step
  const int64_t j0 = t * C;
  const int64_t ncols = d.inner - j0;
  const int64_t r0 = c * rc;
  const int64_t r1 = (d.R - r0 < rc) ? d.R : r0 + rc;
  const float *xt = x + o * d.xso + j0;
  const int64_t xsr = d.xsr;
  // log_softmax reads its planes again: keep them cached
  constexpr bool kNt = MODE != kColsLsm && MODE != kColsPartialKeep;
  constexpr bool kPartial = MODE == kColsPartial || MODE == kColsPartialKeep;
  float m[4], s[4], comp[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    m[e] = -__builtin_inff();
    s[e] = 0.0f;
    comp[e] = 0.0f;
  }
  for (int64_t r = r0 + g; r < r1; r += kStep * kColsU) {
    float v[4][kColsU];
#pragma unroll
    for (int u = 0; u < kColsU; ++u) {
      const int64_t rr = r + u * kStep;
      float q[4];
      if (rr < r1) {
        cols_load<LPP, LAY, kNt>(xt + rr * xsr, cl, ncols, q);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) q[e] = -__builtin_inff();
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e][u] = q[e];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) fold_block_c<kColsU>(v[e], m[e], s[e], comp[e]);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    s[e] = fold_total(s[e], comp[e]);
    merge_lanes<LPP>(m[e], s[e]);
  }
  if (lane < LPP) {
#pragma unroll
    for (int e = 0; e < 4; ++e) lds_pair[wave][tile_col<LPP, LAY>(cl, e)] = make_float2(m[e], s[e]);
  }
  __syncthreads();
  for (int col = threadIdx.x; col < C; col += kColsThreads) {
    float M = lds_pair[0][col].x;
#pragma unroll
    for (int w = 1; w < kColsWaves; ++w) M = fmaxf(M, lds_pair[w][col].x);
    float S = 0.0f;
#pragma unroll
    for (int w = 0; w < kColsWaves; ++w) S += fold_weighted(lds_pair[w][col].x, lds_pair[w][col].y, M);
    if constexpr (kPartial) {
      pairs[(ot * C + col) * chunks + c] = make_float2(M, S);
    } else if constexpr (MODE == kColsLse) {
      if (col < ncols) out[o * d.yso + j0 + col] = M + logf(S);
    } else {
      lds_fin[col] = make_float2(M, logf(S));
    }
  }
  if constexpr (MODE == kColsLsm) {
    __syncthreads();
    float fm[4], fl[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float2 f = lds_fin[tile_col<LPP, LAY>(cl, e)];
      fm[e] = f.x;
      fl[e] = f.y;
    }
    float *yt = out + o * d.yso + j0;
    cols_write<LPP, LAY, kStep>(xt, yt, xsr, d.ysr, r0 + g, r1, cl, ncols, fm, fl);
  }
}

// WAVES waves per (o, t, column) of the tiles (1 or 4; 256-lane workgroups):
// lane i of the column's lanes folds its chunk pairs i, i + 64 WAVES, ... in
// order (4 loads in flight), then the pairs of the wave's lanes and of the
// column's waves merge (the same order on every call).  LSM stores (M, log S)
// per column for the apply launch, else writes the logsumexp.
template <bool LSM, int WAVES>
__global__ __launch_bounds__(256) void axis_cols_merge_kernel(const float2 *__restrict__ pairs,
                                                              float *__restrict__ out,
                                                              float2 *__restrict__ fin,
                                                              AxisDims d, int64_t ctiles,
                                                              int64_t chunks, int C) {
  constexpr int kLanes = WAVES * kWave;  // lanes per column
  __shared__ float2 lds[4];
  const int64_t i = (int64_t)blockIdx.x * (4 / WAVES) + threadIdx.x / kLanes;  // (o, t, column)
  const int tc = threadIdx.x % kLanes;
  if (i >= d.outer * ctiles * C) return;  // whole columns
  const int64_t ot = i / C;
  const int col = (int)(i - ot * C);
  const int64_t t = ot % ctiles;
  const int64_t o = ot / ctiles;
  const int64_t j = t * C + col;
  if (j >= d.inner) return;  // whole columns
  const float2 *p = pairs + i * chunks;
  float m = -__builtin_inff(), s = 0.0f;
  for (int64_t k0 = tc; k0 < chunks; k0 += 4 * kLanes) {
    float2 q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      q[u] = (k0 + u * kLanes < chunks) ? p[k0 + u * kLanes] : make_float2(-__builtin_inff(), 0.0f);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float mn = fmaxf(m, q[u].x);
      s = fold_weighted(m, s, mn) + fold_weighted(q[u].x, q[u].y, mn);
      m = mn;
    }
  }
  merge_lanes<1>(m, s);
  if constexpr (WAVES > 1) {
    const int w = threadIdx.x / kWave;
    if (threadIdx.x % kWave == 0) lds[w] = make_float2(m, s);
    __syncthreads();
    m = lds[0].x;
#pragma unroll
    for (int v = 1; v < WAVES; ++v) m = fmaxf(m, lds[v].x);
    float S = 0.0f;
#pragma unroll
    for (int v = 0; v < WAVES; ++v) S += fold_weighted(lds[v].x, lds[v].y, m);
    s = S;
  }
  if (tc == 0) {
    if constexpr (LSM)
      fin[i] = make_float2(m, logf(s));
    else
      out[o * d.yso + j] = m + logf(s);
  }
}

// log_softmax over the chunks' planes from the merged (M, log S) per column,
// on the grid of the partial launch.
template <int LPP, int LAY>
__global__ __launch_bounds__(kColsThreads) void axis_cols_apply_kernel(
    const float *__restrict__ x, float *__restrict__ y, AxisDims d, int64_t ctiles,
    int64_t chunks, int64_t rc, const float2 *__restrict__ fin) {
  constexpr int kGroups = kWave / LPP;
  constexpr int kStep = kColsWaves * kGroups;
  constexpr int C = 4 * LPP;
  const int64_t b = blockIdx.x;
  const int64_t c = b % chunks;
  const int64_t ot = b / chunks;
  const int64_t t = ot % ctiles;
  const int64_t o = ot / ctiles;
  const int lane = threadIdx.x % kWave;
  const int cl = lane % LPP;
  const int g = (threadIdx.x / kWave) * kGroups + lane / LPP;
  const int64_t j0 = t * C;
  const int64_t ncols = d.inner - j0;
  const int64_t r0 = c * rc;
  const int64_t r1 = (d.R - r0 < rc) ? d.R : r0 + rc;
  float fm[4], fl[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float2 f = fin[ot * C + tile_col<LPP, LAY>(cl, e)];
    fm[e] = f.x;
    fl[e] = f.y;
  }
  const float *xt = x + o * d.xso + j0;
  float *yt = y + o * d.yso + j0;
  cols_write<LPP, LAY, kStep>(xt, yt, d.xsr, d.ysr, r0 + g, r1, cl, ncols, fm, fl);
}

struct ColsPlan {
  int lpp;
  int64_t ctiles, chunks, rc;
};

// The column-split plan of a call, or false when the call keeps the other
// axis kernels.  with_ws: the caller can supply cols_workspace_bytes().
bool cols_plan(const AxisDims &d, bool lsm, bool with_ws, ColsPlan &p) {
  if (d.outer < 1 || d.inner < 1 || d.R < LSE_COLS_MINR) return false;
  int lpp = 1;
  while (lpp < kWave && 4 * lpp < d.inner) lpp *= 2;
  const int64_t C = 4 * lpp;
  p.lpp = lpp;
  p.ctiles = (d.inner + C - 1) / C;
  const int64_t groups = d.outer * p.ctiles;
  if (!with_ws) {
    if (d.outer * d.inner > LSE_COLS_MAX_OUTPUTS) return false;
    // One workgroup per tile: more lanes than the plane split (at most 16
    // waves on a run of outputs, ceil(inner / 4) lanes of each busy) only
    // while a tile holds the whole inner run of at most 32 columns.
    if (lpp > 8 || p.ctiles > 1) return false;
    p.chunks = 1;
  } else {
    // The axis kernels give each lane 4 outputs, a wave 256 of one run per
    // plane: they are left the call when that gives them enough waves, or,
    // for runs wider than LSE_COLS_NARROW columns (each wave reading 512 B or
    // more per plane), a moderate number of them; and, for log_softmax over up
    // to 256 planes, which they read once, unless it leaves them hardly any.
    const int64_t waves = (d.outer * ((d.inner + 3) / 4) + kWave - 1) / kWave;
    const int64_t max_waves =
        d.inner <= LSE_COLS_NARROW ? LSE_COLS_MAX_WAVES : LSE_COLS_WIDE_MAX_WAVES;
    if (waves > max_waves || groups > (int64_t(1) << 24)) return false;
    // Beyond hardly any waves, shorter reductions over runs that the axis
    // kernels read well stay with them: log_softmax (one launch there, three
    // here) over runs wider than 16 columns that are off the 16-byte grid or
    // wider than LSE_COLS_NARROW, and logsumexp over runs off the grid
    // (scalar lanes here, 16-byte ones there).
    const bool grid16 = d.inner % 4 == 0;
    if (waves > LSE_COLS_LSM_MAX_WAVES) {
      if (lsm && d.R < LSE_COLS_LSM_MINR && d.inner > 16 &&
          !(grid16 && d.inner <= LSE_COLS_NARROW))
        return false;
      if (!lsm && !grid16 && d.R < LSE_COLS_OFFGRID_MINR) return false;
    }
    const int64_t step = (int64_t)kColsWaves * (kWave / lpp) * kColsU * LSE_COLS_MIN_ITERS;
    // Chunks of at least LSE_COLS_MIN_PLANES planes while that still gives
    // half the target workgroups, else down to LSE_COLS_MIN_PLANES_LOW.
    int64_t min_planes = step > LSE_COLS_MIN_PLANES ? step : LSE_COLS_MIN_PLANES;
    if (groups * (d.R / min_planes) < LSE_COLS_TARGET_GROUPS / 2)
      min_planes = step > LSE_COLS_MIN_PLANES_LOW ? step : LSE_COLS_MIN_PLANES_LOW;
    int64_t k = (LSE_COLS_TARGET_GROUPS + groups - 1) / groups;
    const int64_t kmax = d.R / min_planes;
    if (k > kmax) k = kmax;
    p.chunks = k < 1 ? 1 : k;
    // One chunk per tile is only worth it while a tile holds the whole
    // inner run (wider runs give the plane-split kernels more lanes).
    if (p.chunks == 1 && p.ctiles > 1) return false;
  }
  p.rc = (d.R + p.chunks - 1) / p.chunks;
  p.chunks = (d.R + p.rc - 1) / p.rc;  // no empty last chunk
  return true;
}

size_t cols_ws_bytes(const AxisDims &d, const ColsPlan &p, bool lsm) {
  if (p.chunks <= 1) return 0;
  const int64_t cols = d.outer * p.ctiles * 4 * p.lpp;
  return (size_t)(cols * p.chunks * 8 + (lsm ? cols * 8 : 0));
}

template <int LPP, int LAY>
hipError_t launch_cols_t(const float *x, float *out, const AxisDims &d, bool lsm,
                         const ColsPlan &p, void *ws, hipStream_t stream) {
  const dim3 grid((uint32_t)(d.outer * p.ctiles * p.chunks));
  const dim3 block(kColsThreads);
  if (p.chunks == 1) {
    if (lsm)
      hipLaunchKernelGGL((axis_cols_kernel<LPP, LAY, kColsLsm>), grid, block, 0, stream, x, out, d,
                         p.ctiles, p.chunks, p.rc, nullptr);
    else
      hipLaunchKernelGGL((axis_cols_kernel<LPP, LAY, kColsLse>), grid, block, 0, stream, x, out, d,
                         p.ctiles, p.chunks, p.rc, nullptr);
    return hipGetLastError();
  }
  constexpr int C = 4 * LPP;
  auto *pairs = reinterpret_cast<float2 *>(ws);
  float2 *fin = pairs + d.outer * p.ctiles * p.chunks * C;
  if (lsm && LSE_COLS_LSM_KEEP)
    hipLaunchKernelGGL((axis_cols_kernel<LPP, LAY, kColsPartialKeep>), grid, block, 0, stream, x,
                       out, d, p.ctiles, p.chunks, p.rc, pairs);
  else
    hipLaunchKernelGGL((axis_cols_kernel<LPP, LAY, kColsPartial>), grid, block, 0, stream, x, out,
                       d, p.ctiles, p.chunks, p.rc, pairs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // a workgroup per column for long chunk lists, else a wave per column
  const int64_t ncol = d.outer * p.ctiles * C;
  const bool wide = p.chunks > 4 * kWave;
  const dim3 mgrid((uint32_t)(wide ? ncol : (ncol + 3) / 4));
  if (lsm) {
    if (wide)
      hipLaunchKernelGGL((axis_cols_merge_kernel<true, 4>), mgrid, dim3(256), 0, stream, pairs,
                         out, fin, d, p.ctiles, p.chunks, C);
    else
      hipLaunchKernelGGL((axis_cols_merge_kernel<true, 1>), mgrid, dim3(256), 0, stream, pairs,
                         out, fin, d, p.ctiles, p.chunks, C);
  } else {
    if (wide)
      hipLaunchKernelGGL((axis_cols_merge_kernel<false, 4>), mgrid, dim3(256), 0, stream, pairs,
                         out, fin, d, p.ctiles, p.chunks, C);
    else
      hipLaunchKernelGGL((axis_cols_merge_kernel<false, 1>), mgrid, dim3(256), 0, stream, pairs,
                         out, fin, d, p.ctiles, p.chunks, C);
  }
  e = hipGetLastError();
  if (e != hipSuccess || !lsm) return e;
  hipLaunchKernelGGL((axis_cols_apply_kernel<LPP, LAY>), grid, block, 0, stream, x, out, d,
                     p.ctiles, p.chunks, p.rc, fin);
  return hipGetLastError();
}

template <int LAY>
hipError_t launch_cols_v(const float *x, float *out, const AxisDims &d, bool lsm,
                         const ColsPlan &p, void *ws, hipStream_t stream) {
  switch (p.lpp) {
    case 1: return launch_cols_t<1, LAY>(x, out, d, lsm, p, ws, stream);
    case 2: return launch_cols_t<2, LAY>(x, out, d, lsm, p, ws, stream);
    case 4: return launch_cols_t<4, LAY>(x, out, d, lsm, p, ws, stream);
    case 8: return launch_cols_t<8, LAY>(x, out, d, lsm, p, ws, stream);
    case 16: return launch_cols_t<16, LAY>(x, out, d, lsm, p, ws, stream);
    case 32: return launch_cols_t<32, LAY>(x, out, d, lsm, p, ws, stream);
    case 64: return launch_cols_t<64, LAY>(x, out, d, lsm, p, ws, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t cols_workspace_bytes(const AxisDims &d, bool lsm) {
  ColsPlan p;
  return cols_plan(d, lsm, true, p) ? cols_ws_bytes(d, p, lsm) : 0;
}

bool launch_cols(const float *x, float *out, const AxisDims &d, bool lsm, bool with_ws, void *ws,
                 hipStream_t stream, hipError_t &e) {
  ColsPlan p;
  if (!cols_plan(d, lsm, with_ws, p)) return false;
  if (p.chunks > 1 && ws == nullptr) return false;  // the caller passed no workspace after all
  const uintptr_t a = (uintptr_t)x | (uintptr_t)out;
  const int64_t st = d.inner | d.xso | d.xsr | (lsm ? (d.yso | d.ysr) : 0);
  const bool vec = (st % 4 == 0) && ((lsm ? a : (uintptr_t)x) % 16 == 0);
  if (vec)
    e = launch_cols_v<kColA16>(x, out, d, lsm, p, ws, stream);
  else if (d.inner >= 4 && lsm && LSE_COLS_A4)
    e = launch_cols_v<kColA4>(x, out, d, lsm, p, ws, stream);
  else
    e = launch_cols_v<kColScalar>(x, out, d, lsm, p, ws, stream);
  return true;
}

}  // namespace lse
