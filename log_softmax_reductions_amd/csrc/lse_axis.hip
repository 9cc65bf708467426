// lse_axis.hip — logsumexp and log_softmax over the middle axis of a row-major
// (outer, R, inner) array; outer = 1 is the leading axis of (R, B, D).
//
// POPCORNBENCH FW-GLM-5-1 l1_p29 (torch.logsumexp over dim 0 of (R,B,D)): each
// output (b,d) is independent; out = max + log(sum(exp(x - max))) over the R
// values.  That page gives one thread per output and rejects 128-bit loads
// because a thread's R values sit a whole plane apart.  Here the vector axis
// is the contiguous inner index instead: lane l owns 4 consecutive inner
// outputs, and for each plane r one wave issues a single 1 KiB contiguous
// global_load_dwordx4 span.  All RB planes of a block are issued before any
// is used and stay in VGPRs, so the max and the sum are an exact two-pass over
// registers with no cross-lane traffic.  R > RB streams blocks of RB planes,
// merging the running (max, sum) per output.  The same layout with outer > 1
// is the channel reduction of an (N, C, H, W) tensor (outer = N, R = C,
// inner = H W), the logsumexp over dim 1 on POPCORNBENCH Kimi-K2.6 l2_p92.
//
// log_softmax over R > 32 planes, and logsumexp over long R with few outputs,
// split the planes of one run of outputs across the waves of a workgroup
// (axis_split_kernel below): each wave keeps at most 16 planes x 4 outputs per
// lane in VGPRs, and the waves' (max, sum) pairs are merged in LDS.
//
// Layouts off the 16-byte grid (x or the output at another 4-byte phase, or
// inner not a multiple of 4) keep the 4-column lanes: 16-byte accesses at
// 4-byte alignment, and the last lane of each run reads the run's last 4
// columns and writes only those its neighbour does not (ua_columns).
//
// A contiguous last axis (inner = 1) runs as rows (lse_rows.hip), contiguous
// blocks of short runs as flat sweeps (lse_blocks.hip), and few outputs over
// many planes as the column split (lse_cols.hip).
//
// Running state per output: m = max so far, s = sum of exp(v - c(m)) with the
// shift c(m) = m when m is finite and 0 when m is +-inf (all values -inf, or
// some +inf), which makes m + log(s) the literal log(sum(exp(v))) in every
// case: -inf -> log 0 = -inf, +inf -> log(inf) = +inf, NaN -> NaN, and
// (v - m) - log(s) the literal v - LSE for log_softmax.
#include <type_traits>

#include "lse_device.hpp"
#include "lse_fold.hpp"
#include "lse_internal.hpp"

namespace lse {
namespace {

#ifndef LSE_AXIS0_THREADS
#define LSE_AXIS0_THREADS 64   // one wave per workgroup measured fastest
#endif
#ifndef LSE_AXIS0_W
#define LSE_AXIS0_W 4   // outputs per lane on the 128-bit path (4 or 8)
#endif
#ifndef LSE_AXIS0_RBMAX
#define LSE_AXIS0_RBMAX 32   // planes held in registers at once
#endif
#ifndef LSE_AXIS0_NT_LOAD
#define LSE_AXIS0_NT_LOAD 1   // x is read exactly once: non-temporal loads
#endif
#ifndef LSE_AXIS_LSM_THREADS
#define LSE_AXIS_LSM_THREADS 128   // log_softmax writes R planes: two waves per workgroup
#endif
#ifndef LSE_AXIS_NT_STORE
#define LSE_AXIS_NT_STORE 1   // log_softmax output is not re-read here: non-temporal stores
#endif
#ifndef LSE_AXIS_SPLIT_RBW
#define LSE_AXIS_SPLIT_RBW 16   // planes per wave held in registers by the plane-split kernel
#endif
#ifndef LSE_AXIS_SPLIT_LSM_NT_LOAD
#define LSE_AXIS_SPLIT_LSM_NT_LOAD 0   // the log_softmax split reads x with cached loads
#endif
#ifndef LSE_AXIS_SPLIT_WAVES
#define LSE_AXIS_SPLIT_WAVES 8   // waves per workgroup: G = max(1, this / P) groups
#endif
#ifndef LSE_AXIS_LSM_SPLIT_MINR
#define LSE_AXIS_LSM_SPLIT_MINR 33   // log_softmax: plane split from this R up
#endif
#ifndef LSE_AXIS_LSE_SPLIT_MINR
#define LSE_AXIS_LSE_SPLIT_MINR 33   // logsumexp: plane split from this R up ...
#endif
#ifndef LSE_AXIS_LSE_SPLIT_MAXWAVES
#define LSE_AXIS_LSE_SPLIT_MAXWAVES 256   // ... when one wave per 256 outputs gives this few
#endif
#ifndef LSE_AXIS_LSE_SPLIT_TARGET
#define LSE_AXIS_LSE_SPLIT_TARGET 2048   // waves the logsumexp split aims for
#endif
constexpr int kAxis0Threads = LSE_AXIS0_THREADS;
constexpr int kLsmThreads = LSE_AXIS_LSM_THREADS;
constexpr int kMaxAxisThreads = kAxis0Threads > kLsmThreads ? kAxis0Threads : kLsmThreads;
constexpr int kVecW = LSE_AXIS0_W;

// Four floats as one 16-byte access at an address known only to be 4-byte
// aligned (gfx950 accepts dword-aligned 16-byte accesses).
typedef float v4a4 __attribute__((ext_vector_type(4), aligned(4)));

// W consecutive values of one plane into column i of v (64-bit loads for W = 2,
// 128-bit loads for W >= 4; A4: p is only 4-byte aligned).
template <int W, int RB, bool NT = LSE_AXIS0_NT_LOAD, bool A4 = false>
__device__ __forceinline__ void load_plane(const float *p, float (&v)[W][RB], int i) {
  if constexpr (W == 1) {
    v[0][i] = *p;
  } else if constexpr (W == 2) {
    const float2 t = *reinterpret_cast<const float2 *>(p);
    v[0][i] = t.x; v[1][i] = t.y;
  } else {
#pragma unroll
    for (int h = 0; h < W / 4; ++h) {
      typedef float v4a16 __attribute__((ext_vector_type(4)));
      typedef std::conditional_t<A4, v4a4, v4a16> v4f;
      v4f t;
      if constexpr (NT)
        t = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(p + 4 * h));
      else
        t = *reinterpret_cast<const v4f *>(p + 4 * h);
      v[4 * h][i] = t.x; v[4 * h + 1][i] = t.y; v[4 * h + 2][i] = t.z; v[4 * h + 3][i] = t.w;
    }
  }
}

// Each kernel takes its strides from the call's AxisDims when STR, else it
// uses those of a contiguous (outer, R, inner) array, so that the x and y
// offsets are one expression to the compiler (shared address arithmetic, fewer
// VGPRs).  They are written out as scalar locals in every kernel: read through
// a reference to the by-value kernel argument (a helper, a struct) they cost
// the plane-split kernel ~75 VGPRs.

#ifndef LSE_AXIS_XCD_REMAP
#define LSE_AXIS_XCD_REMAP 1
#endif
// Workgroups are handed to the 8 XCDs round robin (workgroup b to XCD b % 8),
// each XCD with its own L2.  When x or a plane's byte stride is not aligned to
// the 128-byte cache line, neighbouring output runs share the line at their
// boundary in every plane, and neighbours on different XCDs both fetch it
// (measured: 1.11 x the algorithmic bytes read).  Such calls deal the runs to
// the XCDs in 8 contiguous ranges, neighbours on one XCD: workgroup b takes run
// (b % 8) F + b / 8, F = grid / 8, for b < 8 F (a bijection; the last grid % 8
// keep their index).  With aligned planes the plain order measured faster.
__device__ __forceinline__ int64_t xcd_block(const float *x, int64_t plane_stride) {
  const int64_t b = blockIdx.x;
#if LSE_AXIS_XCD_REMAP
  if (plane_stride % 32 != 0 || ((uintptr_t)x & 127) != 0) {  // uniform
    const int64_t f = gridDim.x / 8;
    if (b < 8 * f) return (b % 8) * f + b / 8;
  }
#endif
  return b;
}

// One lane = W consecutive inner outputs of one outer index; NT threads per
// workgroup (the launch's block size: a constant, where blockDim.x would be
// read from the dispatch packet with a vector load).  UA: W = 4 over a ragged
// inner run (ceil(inner / 4) lanes per outer index; see ua_columns).
template <int W, int NT, bool UA = false>
__device__ __forceinline__ bool axis_item(const AxisDims &d, const float *x, int64_t plane_stride,
                                          int64_t &o, int64_t &q) {
  // W > 1 and !UA: inner % W == 0 by dispatch
  const int64_t nq = UA ? (d.inner + 3) / 4 : d.inner / W;
  const int64_t item = xcd_block(x, plane_stride) * NT + threadIdx.x;
  if (item >= d.outer * nq) return false;
  o = (d.outer == 1) ? 0 : item / nq;
  q = item - o * nq;
  return true;
}

// Ragged inner runs (UA): lane q's 4 columns start at 4 q, except the last
// lane of a run whose inner % 4 != 0, which reads the run's last 4 columns
// (inner >= 4 by dispatch) and owns only the columns from `skip` on (the
// others belong to its neighbour).  Every load stays inside the plane.
__device__ __forceinline__ int64_t ua_columns(const AxisDims &d, int64_t q, int &skip) {
  int64_t j0 = 4 * q;
  skip = 0;
  if (j0 + 4 > d.inner) {
    skip = (int)(j0 + 4 - d.inner);
    j0 = d.inner - 4;
  }
  return j0;
}

// Load planes r0 .. r0 + nb - 1 (nb <= RB, `stride` elements apart) of W
// lanes' outputs into v, padding with the identity -inf; all loads are issued
// before any is used.
template <int RB, int W, bool NT = LSE_AXIS0_NT_LOAD, bool A4 = false>
__device__ __forceinline__ void load_block(const float *base, int64_t stride, int64_t nb,
                                           float (&v)[W][RB]) {
  if (nb == RB) {
#pragma unroll
    for (int i = 0; i < RB; ++i) load_plane<W, RB, NT, A4>(base + (int64_t)i * stride, v, i);
  } else {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      if (i < nb) {
        load_plane<W, RB, NT, A4>(base + (int64_t)i * stride, v, i);
      } else {
#pragma unroll
        for (int w = 0; w < W; ++w) v[w][i] = -__builtin_inff();
      }
    }
  }
}

template <int W>
__device__ __forceinline__ void store_w(float *p, const float (&r)[W]) {
  if constexpr (W == 1) {
    *p = r[0];
  } else if constexpr (W == 2) {
    *reinterpret_cast<float2 *>(p) = make_float2(r[0], r[1]);
  } else {
#pragma unroll
    for (int h = 0; h < W / 4; ++h)
      *reinterpret_cast<float4 *>(p + 4 * h) =
          make_float4(r[4 * h], r[4 * h + 1], r[4 * h + 2], r[4 * h + 3]);
  }
}

#ifndef LSE_AXIS0_SADDR
#define LSE_AXIS0_SADDR 1
#endif
// load_block for 128-bit lanes whose x offsets, o xso + q W elements, fit 32
// bits as bytes: plane i's pointer is uniform (scalar registers) and the lane
// adds one 32-bit byte offset, so a load is a scalar base plus a vector offset.
// The 64-bit per-lane form leaves the compiler one 64-bit vector offset per
// plane (RB = 32: 64 VGPRs, 208 in all, 2 waves per SIMD).
template <int RB, bool NT = LSE_AXIS0_NT_LOAD, bool A4 = false>
__device__ __forceinline__ void load_block_s(const float *plane0, int64_t stride, int64_t nb,
                                             uint32_t off, float (&v)[4][RB]) {
  typedef float v4a16 __attribute__((ext_vector_type(4)));
  typedef std::conditional_t<A4, v4a4, v4a16> v4f;
  typedef __attribute__((address_space(1))) const char gbyte;
  typedef __attribute__((address_space(1))) const v4f gv4f;
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    if (nb == RB || i < nb) {
      // Empty asm statements pin the plane pointer to scalar registers and the
      // offset to one vector register at each load.
      gbyte *p = (gbyte *)(plane0 + (int64_t)i * stride);
      asm volatile("" : "+s"(p));
      uint32_t ok = off;
      asm volatile("" : "+v"(ok));
      v4f t;
      if constexpr (NT)
        t = __builtin_nontemporal_load((gv4f *)(p + ok));
      else
        t = *(gv4f *)(p + ok);
      v[0][i] = t.x; v[1][i] = t.y; v[2][i] = t.z; v[3][i] = t.w;
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) v[w][i] = -__builtin_inff();
    }
  }
}

// Store 4 outputs at a 4-byte aligned p: one 16-byte store, or, for the last
// lane of a ragged run (skip > 0), only the columns it owns.
__device__ __forceinline__ void store4_ua(float *p, const float (&r)[4], int skip) {
  if (skip == 0) {
    *reinterpret_cast<v4a4 *>(p) = v4a4{r[0], r[1], r[2], r[3]};
  } else {
#pragma unroll
    for (int w = 1; w < 4; ++w)
      if (w >= skip) p[w] = r[w];
  }
}

// store4_ua with non-temporal 16-byte stores when NT.
template <bool NT>
__device__ __forceinline__ void store4_ua_nt(float *p, const float (&r)[4], int skip) {
  if (NT && skip == 0)
    __builtin_nontemporal_store(v4a4{r[0], r[1], r[2], r[3]}, reinterpret_cast<v4a4 *>(p));
  else
    store4_ua(p, r, skip);
}

// out[o, j] = LSE_r x[o, r, j].  OFF32: W = 4 and every lane's x offset fits
// 32 bits as bytes (load_block_s).  UA: W = 4 on a ragged or only 4-byte
// aligned layout (ua_columns; 16-byte accesses at 4-byte alignment).
template <int RB, int W, bool STR, bool OFF32 = false, bool UA = false>
__global__ __launch_bounds__(kMaxAxisThreads) void lse_axis_kernel(
    const float *__restrict__ x, float *__restrict__ out, AxisDims d) {
  static_assert(!UA || W == 4, "ragged runs take 4 columns per lane");
  const int64_t st_xsr = STR ? d.xsr : d.inner;
  int64_t o, q;
  if (!axis_item<W, kAxis0Threads, UA>(d, x, st_xsr, o, q)) return;
  const int64_t st_xso = STR ? d.xso : d.R * d.inner;
  const int64_t st_yso = STR ? d.yso : d.inner;
  const int64_t R = d.R;
  int skip = 0;
  const int64_t j0 = UA ? ua_columns(d, q, skip) : q * W;
  float m[W], s[W], comp[W];
#pragma unroll
  for (int w = 0; w < W; ++w) {
    m[w] = -__builtin_inff();
    s[w] = 0.0f;
    comp[w] = 0.0f;
  }
  if constexpr (OFF32) {
    static_assert(W == 4, "scalar-base loads are 128-bit");
    const uint32_t off = (uint32_t)(o * st_xso + j0) * 4u;
    for (int64_t r0 = 0; r0 < R; r0 += RB) {
      float v[W][RB];
      load_block_s<RB, LSE_AXIS0_NT_LOAD != 0, UA>(x + r0 * st_xsr, st_xsr,
                                                   (R - r0 < RB) ? (R - r0) : RB, off, v);
#pragma unroll
      for (int w = 0; w < W; ++w) fold_block_c<RB>(v[w], m[w], s[w], comp[w]);
    }
  } else {
    const float *xo = x + o * st_xso + j0;
    for (int64_t r0 = 0; r0 < R; r0 += RB) {
      float v[W][RB];
      load_block<RB, W, LSE_AXIS0_NT_LOAD != 0, UA>(xo + r0 * st_xsr, st_xsr,
                                                    (R - r0 < RB) ? (R - r0) : RB, v);
#pragma unroll
      for (int w = 0; w < W; ++w) fold_block_c<RB>(v[w], m[w], s[w], comp[w]);
    }
  }
  float r[W];
#pragma unroll
  for (int w = 0; w < W; ++w) r[w] = m[w] + logf(fold_total(s[w], comp[w]));
  if constexpr (UA)
    store4_ua(out + o * st_yso + j0, r, skip);
  else
    store_w<W>(out + o * st_yso + j0, r);
}

#ifndef LSE_AXIS_WALK
#define LSE_AXIS_WALK 1   // wide aligned logsumexp over many planes walks them (lse_axis_walk_kernel)
#endif
#ifndef LSE_AXIS_WALK_COMP
#define LSE_AXIS_WALK_COMP 1   // the walk's column sums with Kahan compensation
#endif
#ifndef LSE_AXIS_WALK_VL
#define LSE_AXIS_WALK_VL 4   // 16-byte loads per lane and plane
#endif
#ifndef LSE_AXIS_WALK_THREADS
#define LSE_AXIS_WALK_THREADS 512
#endif
#ifndef LSE_AXIS_WALK_MINR
#define LSE_AXIS_WALK_MINR 33   // from here up the walk measured faster than blocks of 32 planes
#endif
#ifndef LSE_AXIS_WALK_MIN_BLOCKS
#define LSE_AXIS_WALK_MIN_BLOCKS 512   // workgroups the walk needs to fill the GPU
#endif
constexpr int kWalkThreads = LSE_AXIS_WALK_THREADS;
constexpr int kWalkVl = LSE_AXIS_WALK_VL;
#ifndef LSE_AXIS_WALK_NARROW
#define LSE_AXIS_WALK_NARROW 1   // half-width tiles (VL / 2) when wide ones give too few workgroups
#endif
// Outputs per workgroup for VL 16-byte vectors per lane.
template <int VL>
constexpr int64_t walk_cols() { return (int64_t)kWalkThreads * 4 * VL; }
// Sums against the lane's reference value that stay inside [kWalkLo, kWalkHi]
// are kept: nothing that matters has under- or overflowed, and c and log s
// (|log s| <= 16.7) cancel by at most a few ulps of 16 when added.
constexpr float kWalkLo = 9.5367431640625e-07f;  // 2^-20
constexpr float kWalkHi = 16777216.0f;           // 2^24

// Exact fold of one value into a running (m, s): fold_block with one plane.
__device__ __forceinline__ void fold_one(float v, float &m, float &s) {
  const float mn = fmaxf(m, v);
  const float c = safe_shift(mn);
  const float acc = (s == 0.0f) ? 0.0f : s * exp_base2(safe_shift(m) - c);
  m = mn;
  s = acc + exp_base2(v - c);
}

// out[o, j] = LSE_r x[o, r, j] for wide aligned planes, planes visited one at a
// time.  A workgroup owns walk_cols<VL>() consecutive outputs; wave w reads the
// contiguous 64 x 4 x VL outputs' span of each plane (lane l its VL vectors
// 256 outputs apart), so the workgroup streams walk_cols<VL>() x 4 bytes contiguous
// per plane, where the register-block kernel has each wave touch RB planes
// 1 KiB at a time.
//
// A column's R values no longer sit in registers together, and a running max
// per column would cost a rescale exponential per new max.  Instead every
// column of a lane is summed against one reference c, the largest of the
// lane's plane-0 values: s = sum_r exp(x_r - c), one exponential per value,
// and LSE = c + log s, the same quantity (its closed forms, a single finite
// value or R equal ones, hold exactly only for a column whose values equal c;
// otherwise to rounding, like any other result).  A lane whose
// sums all stay inside [2^-20, 2^24] is done: no term that matters under- or
// overflowed, and the final sum loses at most a few ulps.  Any other lane (a
// column more than ~14 below or ~16 above c, a non-finite value or reference)
// redoes its columns, one vector at a time, with the exact running fold of
// fold_block, which also gives the special-value results.
template <int VL, bool STR, bool UA = false>
__global__ __launch_bounds__(kWalkThreads) void lse_axis_walk_kernel(
    const float *__restrict__ x, float *__restrict__ out, AxisDims d) {
  typedef float v4a16 __attribute__((ext_vector_type(4)));
  typedef std::conditional_t<UA, v4a4, v4a16> v4f;  // UA: 4-byte aligned planes
  constexpr int NV = 4 * VL;
  const int64_t st_xsr = STR ? d.xsr : d.inner;
  const int64_t st_xso = STR ? d.xso : d.R * d.inner;
  const int64_t st_yso = STR ? d.yso : d.inner;
  constexpr int64_t kWalkCols = walk_cols<VL>();
  const int64_t tiles = (d.inner + kWalkCols - 1) / kWalkCols;
  const int64_t b = blockIdx.x;
  const int64_t o = (d.outer == 1) ? 0 : b / tiles;
  const int64_t t = b - o * tiles;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x & (kWave - 1);
  // The tile's first output; this lane's vector k starts jl + 4 kWave k past it.
  const int64_t tb = t * kWalkCols;
  const uint32_t jl = (uint32_t)wave * (kWave * 4 * VL) + 4 * lane;
  // A ragged last tile clamps every vector that would pass the end onto the
  // plane's last 4 columns (inner >= 4): loads stay in bounds, a vector wholly
  // past the end is not stored, and one that straddles it (UA: inner % 4 != 0)
  // stores only its own columns.  Offsets within a tile fit 32 bits, so every
  // load is a uniform plane pointer plus a 32-bit lane offset.
  const bool full = tb + kWalkCols <= d.inner;  // uniform
  uint32_t off[VL];  // byte offsets within the tile
#pragma unroll
  for (int k = 0; k < VL; ++k) {
    const uint32_t j = jl + 4 * kWave * k;
    off[k] = 4 * ((full || tb + j + 4 <= d.inner) ? j : (uint32_t)(d.inner - 4 - tb));
  }
  const float *xt = x + o * st_xso + tb;
  const int64_t R = d.R;

  typedef __attribute__((address_space(1))) const char gbyte;
  typedef __attribute__((address_space(1))) const v4f gv4f;
  auto load = [&](float (&v)[NV], const float *plane) {
    // The empty asm statements pin the plane pointer to scalar registers and
    // the lane offsets to 32-bit vector registers at the loads, so each load
    // is one scalar base plus a 32-bit offset.  Without them, loop strength
    // reduction keeps one 64-bit vector pointer per load (32 VGPRs).
    gbyte *p = (gbyte *)plane;
    asm volatile("" : "+s"(p));
#pragma unroll
    for (int k = 0; k < VL; ++k) {
      uint32_t ok = off[k];
      asm volatile("" : "+v"(ok));
      const v4f q = __builtin_nontemporal_load((gv4f *)(p + ok));
      v[4 * k] = q.x; v[4 * k + 1] = q.y; v[4 * k + 2] = q.z; v[4 * k + 3] = q.w;
    }
  };
  float va[NV], s[NV], cs[NV];
  load(va, xt);
  float lm = va[0];  // the lane's reference c
#pragma unroll
  for (int i = 1; i < NV; ++i) lm = fmaxf(lm, va[i]);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    s[i] = 0.0f;
    cs[i] = 0.0f;
  }
  // Each term joins its column's sum with Kahan's compensation cs: over
  // thousands of planes most terms sit far below the sum and plain addition
  // would round them away (0.78 of the tolerance at R = 8192, sigma 3).  A
  // non-finite term makes the sum NaN here, which sends the lane to the
  // exact redo below.
  auto acc = [&](const float (&v)[NV]) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      if constexpr (LSE_AXIS_WALK_COMP) {
        const float y = exp_base2(v[i] - lm) - cs[i];
        const float t = s[i] + y;
        cs[i] = (t - s[i]) - y;
        s[i] = t;
      } else {
        s[i] += exp_base2(v[i] - lm);
      }
    }
  };
  acc(va);
  for (int64_t r = 1; r < R; ++r) {
    load(va, xt + r * st_xsr);
    acc(va);
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) s[i] -= cs[i];
  float lo = s[0], hi = s[0], tot = 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    lo = fminf(lo, s[i]);
    hi = fmaxf(hi, s[i]);
    tot += s[i];  // a NaN sum survives here (fminf and fmaxf drop it)
  }
  float *op = out + o * st_yso + tb;
  if (lo >= kWalkLo && hi <= kWalkHi && tot <= kWalkHi * NV) {
#pragma unroll
    for (int k = 0; k < VL; ++k) {
      const uint32_t j = jl + 4 * kWave * k;
      if (full || tb + j + 4 <= d.inner) {
        v4f q;
#pragma unroll
        for (int e = 0; e < 4; ++e) q[e] = lm + logf(s[4 * k + e]);
        *reinterpret_cast<v4f *>(op + j) = q;
      } else if (UA && tb + j < d.inner) {
        float q[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) q[e] = lm + logf(s[4 * k + e]);
        const uint32_t j4 = off[k] / 4;  // the run's last 4 columns
        store4_ua(op + j4, q, (int)(j - j4));
      }
    }
  } else {
    // Rare: this lane's columns again, exactly, one vector of 4 at a time.
    for (int k = 0; k < VL; ++k) {
      const uint32_t j = jl + 4 * kWave * k;
      if (!(full || tb + j < d.inner)) continue;
      const uint32_t j4 = off[k] / 4;  // == j unless the vector straddles the end
      float m4[4], s4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        m4[e] = -__builtin_inff();
        s4[e] = 0.0f;
      }
      for (int64_t r = 0; r < R; ++r) {
        const v4f q = *reinterpret_cast<const v4f *>(xt + r * st_xsr + j4);
#pragma unroll
        for (int e = 0; e < 4; ++e) fold_one(q[e], m4[e], s4[e]);
      }
      float res[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) res[e] = m4[e] + logf(s4[e]);
      if (j4 == j)
        *reinterpret_cast<v4f *>(op + j) = v4f{res[0], res[1], res[2], res[3]};
      else
        store4_ua(op + j4, res, (int)(j - j4));
    }
  }
}

#ifndef LSE_AXIS_LSM_OFF32_NT
#define LSE_AXIS_LSM_OFF32_NT 1   // the 32-bit-offset log_softmax kernel stores non-temporally
#endif
// Store 4 values at a uniform plane pointer plus a 32-bit lane byte offset
// (the store form of load_block_s).  A4: only 4-byte aligned; skip > 0 (the
// last lane of a ragged run, see ua_columns): only the columns from skip on.
template <bool NT, bool A4 = false>
__device__ __forceinline__ void store4_s(float *plane, uint32_t off, const float (&r)[4],
                                         int skip = 0) {
  typedef float v4a16 __attribute__((ext_vector_type(4)));
  typedef std::conditional_t<A4, v4a4, v4a16> v4f;
  typedef __attribute__((address_space(1))) char gbyte_w;
  typedef __attribute__((address_space(1))) v4f gv4f_w;
  typedef __attribute__((address_space(1))) float gf_w;
  gbyte_w *p = (gbyte_w *)plane;
  asm volatile("" : "+s"(p));
  uint32_t ok = off;
  asm volatile("" : "+v"(ok));
  if (!A4 || skip == 0) {
    const v4f t = {r[0], r[1], r[2], r[3]};
    if constexpr (NT)
      __builtin_nontemporal_store(t, (gv4f_w *)(p + ok));
    else
      *(gv4f_w *)(p + ok) = t;
  } else {
#pragma unroll
    for (int w = 1; w < 4; ++w)
      if (w >= skip) *(gf_w *)(p + ok + 4 * w) = r[w];
  }
}

// y[o, r, j] = x[o, r, j] - LSE_r' x[o, r', j].  With R <= RB the R values stay
// in registers between the reduction and the write (one read, one write);
// otherwise a streaming reduction pass and a write pass (two reads).  OFF32:
// W = 4 and every lane's x and y offsets fit 32 bits as bytes (scalar plane
// pointers, as in load_block_s).  UA: W = 4 on a ragged or only 4-byte aligned
// layout (ua_columns).
template <int RB, int W, bool STR, bool OFF32 = false, bool UA = false>
__global__ __launch_bounds__(kMaxAxisThreads) void log_softmax_axis_kernel(
    const float *__restrict__ x, float *__restrict__ y, AxisDims d) {
  static_assert(!UA || W == 4, "ragged runs take 4 columns per lane");
  const int64_t st_xsr = STR ? d.xsr : d.inner;
  int64_t o, q;
  if (!axis_item<W, kLsmThreads, UA>(d, x, st_xsr, o, q)) return;
  const int64_t st_xso = STR ? d.xso : d.R * d.inner;
  const int64_t st_ysr = STR ? d.ysr : d.inner;
  const int64_t st_yso = STR ? d.yso : d.R * d.inner;
  const int64_t R = d.R;
  int skip = 0;
  const int64_t j0 = UA ? ua_columns(d, q, skip) : q * W;
  const float *xo = x + o * st_xso + j0;
  float *yo = y + o * st_yso + j0;
  const uint32_t xoff = (uint32_t)(o * st_xso + j0) * 4u;
  const uint32_t yoff = (uint32_t)(o * st_yso + j0) * 4u;
  // Planes r0 .. r0 + nb - 1 into v.
  auto load = [&](int64_t r0, int64_t nb, float (&v)[W][RB]) {
    if constexpr (OFF32)
      load_block_s<RB, LSE_AXIS0_NT_LOAD != 0, UA>(x + r0 * st_xsr, st_xsr, nb, xoff, v);
    else
      load_block<RB, W, LSE_AXIS0_NT_LOAD != 0, UA>(xo + r0 * st_xsr, st_xsr, nb, v);
  };
  float m[W], s[W];
#pragma unroll
  for (int w = 0; w < W; ++w) {
    m[w] = -__builtin_inff();
    s[w] = 0.0f;
  }
  float v[W][RB];
  if (R <= RB) {  // uniform
    load(0, R, v);
#pragma unroll
    for (int w = 0; w < W; ++w) fold_block<RB>(v[w], m[w], s[w]);
  } else {
    float comp[W];
#pragma unroll
    for (int w = 0; w < W; ++w) comp[w] = 0.0f;
    for (int64_t r0 = 0; r0 < R; r0 += RB) {
      load(r0, (R - r0 < RB) ? (R - r0) : RB, v);
#pragma unroll
      for (int w = 0; w < W; ++w) fold_block_c<RB>(v[w], m[w], s[w], comp[w]);
    }
#pragma unroll
    for (int w = 0; w < W; ++w) s[w] = fold_total(s[w], comp[w]);
  }
  float lns[W];
#pragma unroll
  for (int w = 0; w < W; ++w) lns[w] = logf(s[w]);
  for (int64_t r0 = 0; r0 < R; r0 += RB) {
    const int64_t nb = (R - r0 < RB) ? (R - r0) : RB;
    if (R > RB) load(r0, nb, v);
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      if (i < nb) {
        float r[W];
#pragma unroll
        for (int w = 0; w < W; ++w) r[w] = (v[w][i] - m[w]) - lns[w];
        if constexpr (OFF32)
          store4_s<LSE_AXIS_LSM_OFF32_NT != 0, UA>(y + (r0 + i) * st_ysr, yoff, r, skip);
        else if constexpr (UA)
          store4_ua(yo + (r0 + i) * st_ysr, r, skip);
        else
          store_w<W>(yo + (r0 + i) * st_ysr, r);
      }
    }
  }
}

template <int W>
__device__ __forceinline__ void store_w_nt(float *p, const float (&r)[W]) {
  if constexpr (W < 4) {
    store_w<W>(p, r);
  } else {
    typedef float v4f __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int h = 0; h < W / 4; ++h) {
      v4f t = {r[4 * h], r[4 * h + 1], r[4 * h + 2], r[4 * h + 3]};
      __builtin_nontemporal_store(t, reinterpret_cast<v4f *>(p + 4 * h));
    }
  }
}

// Plane-split variant of both reductions: a workgroup has G x P waves.  The P
// waves of one group cover the same 64 x W outputs, and wave p takes the
// contiguous slice of per = ceil(R / P) planes starting at p * per; the G
// groups cover consecutive runs of outputs, so each plane is read as one
// contiguous G x 64 x W span per workgroup.  Each wave folds its slice (blocks
// of RBW planes) into per-output (m, s) pairs, the P pairs of a group meet in
// LDS and every wave of the group merges them into the same (M, S) with the
// rule of fold_block.  With per <= RBW a wave's planes stay in VGPRs from the
// load to the log_softmax write (one read, one write of x's bytes), and a lane
// holds RBW x W values instead of R x W, so more waves fit on a SIMD to keep
// loads in flight.  Larger R reads x a second time for the write.
template <int RBW, int W, int P, int G, bool LSM, bool STR, bool UA = false, bool OFF32 = false>
__global__ __launch_bounds__(kWave * P * G) void axis_split_kernel(
    const float *__restrict__ x, float *__restrict__ out, AxisDims d) {
  static_assert(!UA || W == 4, "ragged runs take 4 columns per lane");
  static_assert(!OFF32 || W == 4, "scalar plane pointers take 4 columns per lane");
  const int64_t st_xsr = STR ? d.xsr : d.inner;
  const int64_t st_xso = STR ? d.xso : d.R * d.inner;
  const int64_t st_ysr = STR ? d.ysr : d.inner;
  const int64_t st_yso = STR ? d.yso : (LSM ? d.R * d.inner : d.inner);
  // log_softmax's split measured faster with cached loads (neighbouring
  // workgroups share the cache lines at their segment boundaries).
  constexpr bool kSplitNt = LSM ? (LSE_AXIS_SPLIT_LSM_NT_LOAD != 0) : (LSE_AXIS0_NT_LOAD != 0);
  __shared__ float lds_m[G][P][W][kWave];
  __shared__ float lds_s[G][P][W][kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wv = wid % P, grp = wid / P;
  const int64_t R = d.R;
  // W > 1 and !UA: inner % W == 0 by dispatch; UA: ragged runs (ua_columns)
  const int64_t nq = UA ? (d.inner + 3) / 4 : d.inner / W;
  const int64_t item = (xcd_block(x, st_xsr) * G + grp) * kWave + lane;
  const bool valid = item < d.outer * nq;
  int64_t o = 0, q = 0;
  if (valid) {
    o = (d.outer == 1) ? 0 : item / nq;
    q = item - o * nq;
  }
  int skip = 0;
  const int64_t j0 = UA ? ua_columns(d, q, skip) : q * W;
  const int64_t per = (R + P - 1) / P;
  const int64_t r0 = (int64_t)wv * per;
  int64_t nr = R - r0;  // planes of this wave's slice (0 for the last waves when P > R)
  nr = nr < 0 ? 0 : (nr > per ? per : nr);
  const int64_t xoff = o * st_xso + j0 + r0 * st_xsr;
  const int64_t yoff = o * st_yso + j0 + r0 * st_ysr;  // == xoff when contiguous
  const float *xs = x + xoff;
  // OFF32: plane pointers in scalar registers plus one 32-bit lane byte
  // offset each for x and y (load_block_s, store4_s).
  const uint32_t xo32 = (uint32_t)((o * st_xso + j0) * 4);
  const uint32_t yo32 = (uint32_t)((o * st_yso + j0) * 4);

  float m[W], s[W];
#pragma unroll
  for (int w = 0; w < W; ++w) {
    m[w] = -__builtin_inff();
    s[w] = 0.0f;
  }
  float v[W][RBW];
  const bool resident = per <= RBW;  // uniform
  float comp[W];
#pragma unroll
  for (int w = 0; w < W; ++w) comp[w] = 0.0f;
  for (int64_t b = 0; b < nr; b += RBW) {
    const int64_t nb = valid ? ((nr - b < RBW) ? (nr - b) : RBW) : 0;
    if constexpr (OFF32)
      load_block_s<RBW, kSplitNt, UA>(x + (r0 + b) * st_xsr, st_xsr, nb, xo32, v);
    else
      load_block<RBW, W, kSplitNt, UA>(xs + b * st_xsr, st_xsr, nb, v);
#pragma unroll
    for (int w = 0; w < W; ++w) fold_block_c<RBW>(v[w], m[w], s[w], comp[w]);
  }
#pragma unroll
  for (int w = 0; w < W; ++w) s[w] = fold_total(s[w], comp[w]);
#pragma unroll
  for (int w = 0; w < W; ++w) {
    lds_m[grp][wv][w][lane] = m[w];
    lds_s[grp][wv][w][lane] = s[w];
  }
  __syncthreads();
  // Merge the P pairs in the same order in every wave: identical (M, S).
#pragma unroll
  for (int w = 0; w < W; ++w) {
    float mm = lds_m[grp][0][w][lane];
#pragma unroll
    for (int p = 1; p < P; ++p) mm = fmaxf(mm, lds_m[grp][p][w][lane]);
    const float c = safe_shift(mm);
    float acc = 0.0f;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const float sp = lds_s[grp][p][w][lane];
      // A pair that counted nothing is skipped: its weight may be inf.
      if (sp != 0.0f) acc += sp * exp_base2(safe_shift(lds_m[grp][p][w][lane]) - c);
    }
    m[w] = mm;
    s[w] = acc;
  }
  if (!valid) return;
  if constexpr (!LSM) {
    if (wv == 0) {
      float r[W];
#pragma unroll
      for (int w = 0; w < W; ++w) r[w] = m[w] + logf(s[w]);
      if constexpr (UA)
        store4_ua(out + o * st_yso + j0, r, skip);
      else
        store_w<W>(out + o * st_yso + j0, r);
    }
  } else {
    float lns[W];
#pragma unroll
    for (int w = 0; w < W; ++w) lns[w] = logf(s[w]);
    float *ys = out + yoff;
    for (int64_t b = 0; b < nr; b += RBW) {
      const int64_t nb = (nr - b < RBW) ? (nr - b) : RBW;
      if (!resident) {
        if constexpr (OFF32)
          load_block_s<RBW, kSplitNt, UA>(x + (r0 + b) * st_xsr, st_xsr, nb, xo32, v);
        else
          load_block<RBW, W, kSplitNt, UA>(xs + b * st_xsr, st_xsr, nb, v);
      }
#pragma unroll
      for (int i = 0; i < RBW; ++i) {
        if (i < nb) {
          float r[W];
#pragma unroll
          for (int w = 0; w < W; ++w) r[w] = (v[w][i] - m[w]) - lns[w];
          if constexpr (OFF32)
            store4_s<LSE_AXIS_NT_STORE != 0, UA>(out + (r0 + b + i) * st_ysr, yo32, r, skip);
          else if constexpr (UA)
            store4_ua_nt<LSE_AXIS_NT_STORE != 0>(ys + (b + i) * st_ysr, r, skip);
          else if constexpr (LSE_AXIS_NT_STORE)
            store_w_nt<W>(ys + (b + i) * st_ysr, r);
          else
            store_w<W>(ys + (b + i) * st_ysr, r);
        }
      }
    }
  }
}

// Workgroups per CU, capped through the LDS each one reserves: 160 KiB per CU,
// allocated in 1280-byte granules, so a reservation of (160 KiB / c) rounded
// down to a granule lets exactly c workgroups share a CU (c + 1 do not fit).
constexpr int kLdsPerCu = 163840;
constexpr size_t occupancy_lds(int c) { return c > 0 ? (size_t)(kLdsPerCu / c) / 1280 * 1280 : 0; }

#ifndef LSE_AXIS0_CAP
#define LSE_AXIS0_CAP 1
#endif
// One-wave logsumexp workgroups per CU for RB planes (RB 128-bit loads in
// flight per wave).  With as many waves as the VGPRs allow, the memory system
// receives more outstanding loads than it turns into bandwidth, and the kernel
// slows: same-box sweeps of the cap over (R, 2048, 4096) and channel layouts
// measured the fastest at 6 waves per CU for RB = 32 (192 KiB in flight per
// CU; 12 allowed by VGPRs: 184 -> 173 us on (32, 2048, 4096)) and RB = 16
// (102 -> 91 us on (16, 2048, 4096)), 9 for RB = 8 (102 -> 92 us on (8, 4096,
// 4096)) and 16 for RB = 4 (105 -> 97 us on (4, 8192, 4096)).
constexpr int axis0_waves_per_cu(int rb) {
  return !LSE_AXIS0_CAP ? 0 : rb >= 16 ? 6 : rb == 8 ? 9 : 16;
}
// Two-wave log_softmax workgroups per CU (128-bit path with 32-bit offsets and
// non-temporal stores), the fastest of a same-box sweep over 3 .. 8: 3 for
// RB = 32 ((32, 2048, 4096): 371 us; 403 us at the VGPR limit of 6), 4 for
// RB = 16 ((16, 2048, 4096): 188 us; 200-212 us at 6-8), 6 for RB = 8 ((8,
// 4096, 4096): 178 us; 184 us at 4 and 8).
constexpr int lsm_groups_per_cu(int rb) {
  return !LSE_AXIS0_CAP ? 0 : rb == 32 ? 3 : rb == 16 ? 4 : rb == 8 ? 6 : 0;
}

#ifndef LSE_AXIS_UA
#define LSE_AXIS_UA 1   // ragged / 4-byte aligned layouts take the 128-bit kernels (ua_columns)
#endif
// The register-block kernels: vec = every plane and output row on a 16-byte
// boundary (inner and strides multiples of 4); otherwise, with 4-byte aligned
// x and output, inner >= 4 and lane offsets within 32 bits, the same kernels
// with 16-byte accesses at 4-byte alignment and the ragged last lane of each
// run clamped (UA); else one column per lane.
template <int RB, bool LSM, bool STR>
hipError_t launch_rb(const float *x, float *out, const AxisDims &d, bool vec,
                     hipStream_t stream) {
  // Largest lane offsets, in bytes, of x and of y.
  const int64_t xspan = ((d.outer - 1) * (STR ? d.xso : d.R * d.inner) + d.inner) * 4;
  const int64_t yspan =
      LSM ? ((d.outer - 1) * (STR ? d.yso : d.R * d.inner) + d.inner) * 4 : 0;
  const bool off32 = LSE_AXIS0_SADDR && kVecW == 4 && xspan <= (int64_t)0xffffffff &&
                     yspan <= (int64_t)0xffffffff;
  const bool ua = !vec && LSE_AXIS_UA && off32 && d.inner >= 4 &&
                  (((uintptr_t)x | (uintptr_t)out) & 3u) == 0;
  const int64_t items = d.outer * (vec ? d.inner / kVecW : ua ? (d.inner + 3) / 4 : d.inner);
  if constexpr (LSM) {
    const dim3 grid((uint32_t)((items + kLsmThreads - 1) / kLsmThreads));
    const size_t lds = (vec || ua) ? occupancy_lds(lsm_groups_per_cu(RB)) : 0;
    if (vec && off32)
      hipLaunchKernelGGL((log_softmax_axis_kernel<RB, 4, STR, true>), grid, dim3(kLsmThreads), lds,
                         stream, x, out, d);
    else if (vec)
      hipLaunchKernelGGL((log_softmax_axis_kernel<RB, kVecW, STR>), grid, dim3(kLsmThreads), lds,
                         stream, x, out, d);
    else if (ua)
      hipLaunchKernelGGL((log_softmax_axis_kernel<RB, 4, STR, true, true>), grid, dim3(kLsmThreads),
                         lds, stream, x, out, d);
    else
      hipLaunchKernelGGL((log_softmax_axis_kernel<RB, 1, STR>), grid, dim3(kLsmThreads), 0, stream,
                         x, out, d);
  } else {
    const dim3 grid((uint32_t)((items + kAxis0Threads - 1) / kAxis0Threads));
    const size_t lds = (vec || ua) ? occupancy_lds(axis0_waves_per_cu(RB)) : 0;
    if (vec && off32)
      hipLaunchKernelGGL((lse_axis_kernel<RB, 4, STR, true>), grid, dim3(kAxis0Threads), lds, stream,
                         x, out, d);
    else if (vec)
      hipLaunchKernelGGL((lse_axis_kernel<RB, kVecW, STR>), grid, dim3(kAxis0Threads), lds, stream, x,
                         out, d);
    else if (ua)
      hipLaunchKernelGGL((lse_axis_kernel<RB, 4, STR, true, true>), grid, dim3(kAxis0Threads), lds,
                         stream, x, out, d);
    else
      hipLaunchKernelGGL((lse_axis_kernel<RB, 1, STR>), grid, dim3(kAxis0Threads), 0, stream, x, out,
                         d);
  }
  return hipGetLastError();
}

#ifndef LSE_AXIS_SPLIT_OFF32
#define LSE_AXIS_SPLIT_OFF32 1   // the strided plane split with scalar plane pointers (load_block_s)
#endif
template <int RBW, int W, int P, bool LSM, bool STR>
hipError_t launch_split(const float *x, float *out, const AxisDims &d, bool ua,
                        hipStream_t stream) {
  constexpr int G = (LSE_AXIS_SPLIT_WAVES / P) > 1 ? (LSE_AXIS_SPLIT_WAVES / P) : 1;
  const int64_t items = d.outer * (ua ? (d.inner + 3) / 4 : d.inner / W);
  const dim3 grid((uint32_t)((items + kWave * G - 1) / (kWave * G)));
  // Largest lane offsets, in bytes, of x and of the output.
  const int64_t xspan = ((d.outer - 1) * (STR ? d.xso : d.R * d.inner) + d.inner) * 4;
  const int64_t yspan =
      ((d.outer - 1) * (STR ? d.yso : (LSM ? d.R * d.inner : d.inner)) + d.inner) * 4;
  // Strided calls only: with separate x and y strides the 64-bit form keeps
  // both planes' addresses live (144-168 VGPRs, a spill at 16 waves), and the
  // scalar plane pointers measured 8-49 % faster on padded views ((4, 256,
  // 65536) with a 64-float pad: 3539 -> 5270 GB/s); on dense calls they ran
  // up to 5 % slower ((128, 64, 15876): 214 -> 224 us), so those keep it.
  const bool off32 = LSE_AXIS_SPLIT_OFF32 && STR && W == 4 && xspan <= (int64_t)0xffffffff &&
                     yspan <= (int64_t)0xffffffff;
  if (off32 && ua)
    hipLaunchKernelGGL((axis_split_kernel<RBW, 4, P, G, LSM, STR, true, true>), grid,
                       dim3(kWave * P * G), 0, stream, x, out, d);
  else if (off32)
    hipLaunchKernelGGL((axis_split_kernel<RBW, 4, P, G, LSM, STR, false, true>), grid,
                       dim3(kWave * P * G), 0, stream, x, out, d);
  else if (ua)
    hipLaunchKernelGGL((axis_split_kernel<RBW, 4, P, G, LSM, STR, true>), grid,
                       dim3(kWave * P * G), 0, stream, x, out, d);
  else
    hipLaunchKernelGGL((axis_split_kernel<RBW, W, P, G, LSM, STR>), grid, dim3(kWave * P * G), 0,
                       stream, x, out, d);
  return hipGetLastError();
}

template <int RBW, bool LSM, bool STR>
hipError_t launch_split_p(int P, const float *x, float *out, const AxisDims &d, bool ua,
                          hipStream_t stream) {
  switch (P) {
    case 1: return launch_split<RBW, kVecW, 1, LSM, STR>(x, out, d, ua, stream);
    case 2: return launch_split<RBW, kVecW, 2, LSM, STR>(x, out, d, ua, stream);
    case 4: return launch_split<RBW, kVecW, 4, LSM, STR>(x, out, d, ua, stream);
    case 8: return launch_split<RBW, kVecW, 8, LSM, STR>(x, out, d, ua, stream);
    default: return launch_split<RBW, kVecW, 16, LSM, STR>(x, out, d, ua, stream);
  }
}

// Launches the plane walk with VL vectors per lane if its tiling suits d
// (true, launch status in e); false leaves the call to other kernels.
template <int VL, bool STR>
bool launch_walk(const float *x, float *out, const AxisDims &d, bool ua, hipStream_t stream,
                 hipError_t &e) {
  constexpr int64_t cols = walk_cols<VL>();
  const int64_t tiles = (d.inner + cols - 1) / cols;
  if (d.outer * tiles < LSE_AXIS_WALK_MIN_BLOCKS || tiles * cols * 8 > d.inner * 9 ||
      d.outer * tiles > 0x7fffffff)
    return false;
  if (ua)
    hipLaunchKernelGGL((lse_axis_walk_kernel<VL, STR, true>), dim3((uint32_t)(d.outer * tiles)),
                       dim3(kWalkThreads), 0, stream, x, out, d);
  else
    hipLaunchKernelGGL((lse_axis_walk_kernel<VL, STR>), dim3((uint32_t)(d.outer * tiles)),
                       dim3(kWalkThreads), 0, stream, x, out, d);
  e = hipGetLastError();
  return true;
}

template <bool LSM, bool STR>
hipError_t launch_axis_t(const float *x, float *out, const AxisDims &d, hipStream_t stream) {
  if (d.inner == 0 || d.outer == 0) return hipSuccess;
  const int64_t R = d.R;
  const uintptr_t a = (uintptr_t)x | (uintptr_t)out;
  // Every plane and output row must start on the vector boundary too.
  const int64_t st = d.inner | d.xso | d.xsr | d.yso | (LSM ? d.ysr : 0);
  const bool vec = (st % kVecW == 0) && (a % 16 == 0);
  // Off the 16-byte grid: the same 4-column lanes with 16-byte accesses at
  // 4-byte alignment and each run's ragged end clamped (ua_columns).
  const bool ua = !vec && LSE_AXIS_UA && kVecW == 4 && d.inner >= 4 && (a & 3u) == 0;
  constexpr int RBW = LSE_AXIS_SPLIT_RBW;
  if ((vec || ua) && LSM && R >= LSE_AXIS_LSM_SPLIT_MINR) {
    // log_softmax: the fewest waves (a power of two up to 16) whose slices of
    // ceil(R / P) planes fit RBW registers each, so x is read once up to
    // R = 16 RBW.
    int P = 1;
    while (P < 16 && (int64_t)P * RBW < R) P *= 2;
    return launch_split_p<RBW, true, STR>(P, x, out, d, ua, stream);
  }
  const int64_t waves = (d.outer * ((d.inner + kVecW - 1) / kVecW) + kWave - 1) / kWave;
  if ((vec || ua) && !LSM && R >= LSE_AXIS_LSE_SPLIT_MINR &&
      waves <= LSE_AXIS_LSE_SPLIT_MAXWAVES) {
    // logsumexp over long R with few outputs: one wave per 256 outputs would
    // leave most of the GPU idle, so P waves share each output run, each
    // streaming at least 8 planes.
    int P = 1;
    while (P < 16 && waves * P < LSE_AXIS_LSE_SPLIT_TARGET) P *= 2;
    while (P > 1 && R < 8 * (int64_t)P) P /= 2;
    if (P > 1) return launch_split_p<RBW, false, STR>(P, x, out, d, ua, stream);
  }
#if LSE_AXIS_WALK
  if constexpr (!LSM) {
    if ((vec || ua) && R >= LSE_AXIS_WALK_MINR) {
      // Many wide aligned planes: the plane walk, with the widest tile that
      // still gives enough workgroups and at most 1/8 padding.  Up to 32
      // planes the register-block kernel below is as fast or faster.
      hipError_t e = hipErrorInvalidValue;
      if (launch_walk<kWalkVl, STR>(x, out, d, ua, stream, e)) return e;
#if LSE_AXIS_WALK_NARROW
      // Half-width tiles (16 KiB per plane and workgroup) still beat the
      // register-block kernel (the channel layout (128, 64, 15876): 5890 ->
      // 6480 GB/s); quarter-width ones measured 8 % slower than it.
      if constexpr (kWalkVl >= 2)
        if (launch_walk<kWalkVl / 2, STR>(x, out, d, ua, stream, e)) return e;
#endif
    }
  }
#endif
  if (R <= 4) return launch_rb<4, LSM, STR>(x, out, d, vec, stream);
  if (R <= 8 || LSE_AXIS0_RBMAX <= 8) return launch_rb<8, LSM, STR>(x, out, d, vec, stream);
  if (R <= 16 || LSE_AXIS0_RBMAX <= 16) return launch_rb<16, LSM, STR>(x, out, d, vec, stream);
  if (LSM && R > 32 && R <= 128) {
    // log_softmax that the 4-column lanes cannot take (inner < 4, or x or y
    // off the 4-byte grid) keeps all R values in registers for the write:
    // narrow the per-lane vector so that R x W stays at 128 values (2 outputs
    // per lane up to 64 planes, 1 up to 128) instead of reading x twice.
    const bool two = R <= 64 && st % 2 == 0 && a % 8 == 0;
    const int64_t items = d.outer * (two ? d.inner / 2 : d.inner);
    const dim3 grid((uint32_t)((items + kLsmThreads - 1) / kLsmThreads));
    if (two)
      hipLaunchKernelGGL((log_softmax_axis_kernel<64, 2, STR>), grid, dim3(kLsmThreads), 0, stream,
                         x, out, d);
    else
      hipLaunchKernelGGL((log_softmax_axis_kernel<128, 1, STR>), grid, dim3(kLsmThreads), 0,
                         stream, x, out, d);
    return hipGetLastError();
  }
  return launch_rb<32, LSM, STR>(x, out, d, vec, stream);
}

// Outputs per launch: every kernel above runs at most 4 work-items per output
// (the plane split: P waves per run of 4-column lanes), so 2^29 outputs keep a
// dispatch's work-item count within 32 bits.
constexpr int64_t kMaxAxisOutputs = int64_t(1) << 29;

// Contiguous calls take instantiations whose strides derive from R and inner.
// Larger calls run as several launches of the strided instantiation over
// consecutive outer blocks, or over 2^29-column slices of the inner run.
template <bool LSM>
hipError_t launch_axis(const float *x, float *out, const AxisDims &d, hipStream_t stream) {
  if (d.outer * d.inner > kMaxAxisOutputs) {
    hipError_t e = hipSuccess;
    if (d.inner <= kMaxAxisOutputs) {
      const int64_t ob = kMaxAxisOutputs / d.inner;
      for (int64_t o0 = 0; o0 < d.outer && e == hipSuccess; o0 += ob) {
        AxisDims s = d;
        s.outer = (d.outer - o0 < ob) ? (d.outer - o0) : ob;
        e = launch_axis_t<LSM, true>(x + o0 * d.xso, out + o0 * d.yso, s, stream);
      }
    } else {
      for (int64_t o = 0; o < d.outer && e == hipSuccess; ++o)
        for (int64_t j0 = 0; j0 < d.inner && e == hipSuccess; j0 += kMaxAxisOutputs) {
          AxisDims s = d;
          s.outer = 1;
          s.inner = (d.inner - j0 < kMaxAxisOutputs) ? (d.inner - j0) : kMaxAxisOutputs;
          e = launch_axis_t<LSM, true>(x + o * d.xso + j0, out + o * d.yso + j0, s, stream);
        }
    }
    return e;
  }
  const bool contiguous = d.xsr == d.inner && (d.outer == 1 || d.xso == d.R * d.inner) &&
                          (LSM ? (d.ysr == d.inner && (d.outer == 1 || d.yso == d.R * d.inner))
                               : (d.outer == 1 || d.yso == d.inner));
  return contiguous ? launch_axis_t<LSM, false>(x, out, d, stream)
                    : launch_axis_t<LSM, true>(x, out, d, stream);
}

}  // namespace

// A reduction over a contiguous last axis (inner = 1, unit R stride) is a row
// reduction: the row kernels read each row as contiguous spans (short rows a
// segment of a wave each, long ones a workgroup or several), where the axis
// kernels would give each lane a row of its own and read it value by value.
static bool as_rows(const AxisDims &d, bool lsm) {
  return d.inner == 1 && d.xsr == 1 && (!lsm || d.ysr == 1) && d.outer <= 0x7fffffff;
}

#ifndef LSE_AXIS_COLS
#define LSE_AXIS_COLS 1   // few outputs over many planes take the column split (lse_cols.hip)
#endif
#ifndef LSE_AXIS_BLOCKS
#define LSE_AXIS_BLOCKS 1 // contiguous blocks with short inner runs read flat (lse_blocks.hip)
#endif
#ifndef LSE_AXIS_SEG
#define LSE_AXIS_SEG 1    // short (R, 2 or 4) blocks take the short-row segments (lse_rows.hip)
#endif
#ifndef LSE_AXIS_ROWS_SPLIT_MAX_ROWS
#define LSE_AXIS_ROWS_SPLIT_MAX_ROWS 1024   // logsumexp rows split with a workspace up to here
#endif
#ifndef LSE_AXIS_ROWS_SPLIT_OFFGRID
#define LSE_AXIS_ROWS_SPLIT_OFFGRID 1   // ... and any number of rows off the 16-byte grid
#endif
// Long last-axis logsumexp rows with a workspace: per-chunk pairs of the row
// register tile, then one merge per row (few rows only: many rows fill the
// GPU one workgroup per row).
// Also any number of rows that the one-workgroup-per-row kernel would read
// one value per access (off the 16-byte grid): the chunk pairs read them as
// 16-byte vectors at their own phase.
static bool lse_rows_split(const AxisDims &d, const float *x) {
  const bool vec = d.R % 4 == 0 && d.xso % 4 == 0 && (uintptr_t)x % 16 == 0;
  return (d.outer <= LSE_AXIS_ROWS_SPLIT_MAX_ROWS || (!vec && LSE_AXIS_ROWS_SPLIT_OFFGRID)) &&
         d.R > kRowsTile && (d.outer == 1 || d.yso == 1);
}

size_t axis_workspace_bytes(int64_t outer, int64_t R, int64_t inner, bool lsm) {
  if (outer < 1 || R < 1 || inner < 1) return 0;
  const AxisDims d{outer, R, inner, R * inner, inner, lsm ? R * inner : inner, lsm ? inner : 0};
  size_t n = LSE_AXIS_COLS ? cols_workspace_bytes(d, lsm) : 0;
  if (LSE_AXIS_BLOCKS) {
    const size_t k = blocks_workspace_bytes(d, lsm);
    if (k > n) n = k;
  }
  if (inner == 1) {
    size_t r = 0;
    if (lsm) {
      r = rows_workspace_bytes(outer, R);
    } else if (R > kRowsTile) {  // lse_rows_split, whatever the alignment
      r = (size_t)outer * (size_t)((R + kRowsTile - 1) / kRowsTile) * sizeof(float2);
    }
    if (r > n) n = r;
  }
  return n;
}

hipError_t launch_lse_axis(const float *x, float *out, const AxisDims &d, hipStream_t stream,
                           bool with_ws, void *ws) {
  if (as_rows(d, false)) {
    if (with_ws && ws != nullptr && lse_rows_split(d, x)) {
      const int64_t nchunks = (d.R + kRowsTile - 1) / kRowsTile;
      const hipError_t e = launch_lse_rows_partial(x, d.outer, d.R, d.xso, kRowsTile, ws, stream);
      if (e != hipSuccess) return e;
      return launch_lse_rows_merge(ws, d.outer, nchunks, out, stream);
    }
    return launch_rows_lse(x, d.outer, d.R, d.xso, out, d.yso, stream);
  }
  hipError_t e = hipSuccess;
  if (LSE_AXIS_SEG && launch_axis_seg(x, out, d, false, stream, e)) return e;
  if (LSE_AXIS_BLOCKS && launch_blocks(x, out, d, false, with_ws, ws, stream, e)) return e;
  if (LSE_AXIS_COLS && launch_cols(x, out, d, false, with_ws, ws, stream, e)) return e;
  return launch_axis<false>(x, out, d, stream);
}

hipError_t launch_log_softmax_axis(const float *x, float *y, const AxisDims &d,
                                   hipStream_t stream, bool with_ws, void *ws) {
  if (as_rows(d, true)) {
    if (with_ws && ws != nullptr && rows_plan(d.R).nchunks > 1 &&
        d.outer * rows_plan(d.R).nchunks <= 0x7fffffff)
      return launch_log_softmax_rows(x, y, d.outer, d.R, d.xso, d.yso, ws, stream);
    return launch_log_softmax_rows_no_ws(x, y, d.outer, d.R, d.xso, d.yso, stream);
  }
  hipError_t e = hipSuccess;
  if (LSE_AXIS_SEG && launch_axis_seg(x, y, d, true, stream, e)) return e;
  if (LSE_AXIS_BLOCKS && launch_blocks(x, y, d, true, with_ws, ws, stream, e)) return e;
  if (LSE_AXIS_COLS && launch_cols(x, y, d, true, with_ws, ws, stream, e)) return e;
  return launch_axis<true>(x, y, d, stream);
}

}  // namespace lse
