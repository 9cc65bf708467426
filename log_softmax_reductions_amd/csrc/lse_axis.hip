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
// Running state per output: m = max so far, s = sum of exp(v - c(m)) with the
// shift c(m) = m when m is finite and 0 when m is +-inf (all values -inf, or
// some +inf), which makes m + log(s) the literal log(sum(exp(v))) in every
// case: -inf -> log 0 = -inf, +inf -> log(inf) = +inf, NaN -> NaN, and
// (v - m) - log(s) the literal v - LSE for log_softmax.
#include "lse_device.hpp"
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
#ifndef LSE_AXIS_LSM64_W
#define LSE_AXIS_LSM64_W 4   // outputs per lane of log_softmax when 32 < R <= 64
#endif
#ifndef LSE_AXIS_LSM_THREADS
#define LSE_AXIS_LSM_THREADS 128   // log_softmax writes R planes: two waves per workgroup
#endif
constexpr int kAxis0Threads = LSE_AXIS0_THREADS;
constexpr int kLsmThreads = LSE_AXIS_LSM_THREADS;
constexpr int kMaxAxisThreads = kAxis0Threads > kLsmThreads ? kAxis0Threads : kLsmThreads;
constexpr int kVecW = LSE_AXIS0_W;

__device__ __forceinline__ float safe_shift(float m) { return is_finite(m) ? m : 0.0f; }

// Fold one block of NB planes (values v[0..NB)) into the running (m, s).
template <int NB>
__device__ __forceinline__ void fold_block(const float (&v)[NB], float &m, float &s) {
  float bm = v[0];
#pragma unroll
  for (int i = 1; i < NB; ++i) bm = fmaxf(bm, v[i]);
  const float mn = fmaxf(m, bm);
  const float c = safe_shift(mn);
  // s == 0 means nothing counted yet: skip the rescale (its factor may be inf).
  float acc = (s == 0.0f) ? 0.0f : s * exp_base2(safe_shift(m) - c);
#pragma unroll
  for (int i = 0; i < NB; ++i) acc += exp_base2(v[i] - c);
  m = mn;
  s = acc;
}

// W consecutive values of one plane into column i of v (64-bit loads for W = 2,
// 128-bit loads for W >= 4).
template <int W, int RB>
__device__ __forceinline__ void load_plane(const float *p, float (&v)[W][RB], int i) {
  if constexpr (W == 1) {
    v[0][i] = *p;
  } else if constexpr (W == 2) {
    const float2 t = *reinterpret_cast<const float2 *>(p);
    v[0][i] = t.x; v[1][i] = t.y;
  } else {
#pragma unroll
    for (int h = 0; h < W / 4; ++h) {
#if LSE_AXIS0_NT_LOAD
      typedef float v4f __attribute__((ext_vector_type(4)));
      const v4f t = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(p + 4 * h));
#else
      const float4 t = *reinterpret_cast<const float4 *>(p + 4 * h);
#endif
      v[4 * h][i] = t.x; v[4 * h + 1][i] = t.y; v[4 * h + 2][i] = t.z; v[4 * h + 3][i] = t.w;
    }
  }
}

// One lane = W consecutive inner outputs of one outer index.
template <int W>
__device__ __forceinline__ bool axis_item(int64_t outer, int64_t R, int64_t inner, int64_t &o,
                                          int64_t &q) {
  const int64_t nq = inner / W;  // W > 1: inner % W == 0 by dispatch
  const int64_t item = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (item >= outer * nq) return false;
  o = (outer == 1) ? 0 : item / nq;
  q = item - o * nq;
  return true;
}

// Load planes r0 .. r0 + nb - 1 (nb <= RB) of W lanes' outputs into v,
// padding with the identity -inf; all loads are issued before any is used.
template <int RB, int W>
__device__ __forceinline__ void load_block(const float *base, int64_t inner, int64_t nb,
                                           float (&v)[W][RB]) {
  if (nb == RB) {
#pragma unroll
    for (int i = 0; i < RB; ++i) load_plane<W>(base + (int64_t)i * inner, v, i);
  } else {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      if (i < nb) {
        load_plane<W>(base + (int64_t)i * inner, v, i);
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

// out[o, j] = LSE_r x[o, r, j]
template <int RB, int W>
__global__ __launch_bounds__(kMaxAxisThreads) void lse_axis_kernel(
    const float *__restrict__ x, float *__restrict__ out, int64_t outer, int64_t R,
    int64_t inner) {
  int64_t o, q;
  if (!axis_item<W>(outer, R, inner, o, q)) return;
  const float *xo = x + o * R * inner + q * W;
  float m[W], s[W];
#pragma unroll
  for (int w = 0; w < W; ++w) {
    m[w] = -__builtin_inff();
    s[w] = 0.0f;
  }
  for (int64_t r0 = 0; r0 < R; r0 += RB) {
    float v[W][RB];
    load_block<RB, W>(xo + r0 * inner, inner, (R - r0 < RB) ? (R - r0) : RB, v);
#pragma unroll
    for (int w = 0; w < W; ++w) fold_block<RB>(v[w], m[w], s[w]);
  }
  float r[W];
#pragma unroll
  for (int w = 0; w < W; ++w) r[w] = m[w] + logf(s[w]);
  store_w<W>(out + o * inner + q * W, r);
}

// y[o, r, j] = x[o, r, j] - LSE_r' x[o, r', j].  With R <= RB the R values stay
// in registers between the reduction and the write (one read, one write);
// otherwise a streaming reduction pass and a write pass (two reads).
template <int RB, int W>
__global__ __launch_bounds__(kMaxAxisThreads) void log_softmax_axis_kernel(
    const float *__restrict__ x, float *__restrict__ y, int64_t outer, int64_t R,
    int64_t inner) {
  int64_t o, q;
  if (!axis_item<W>(outer, R, inner, o, q)) return;
  const int64_t off = o * R * inner + q * W;
  float m[W], s[W];
#pragma unroll
  for (int w = 0; w < W; ++w) {
    m[w] = -__builtin_inff();
    s[w] = 0.0f;
  }
  float v[W][RB];
  if (R <= RB) {  // uniform
    load_block<RB, W>(x + off, inner, R, v);
#pragma unroll
    for (int w = 0; w < W; ++w) fold_block<RB>(v[w], m[w], s[w]);
  } else {
    for (int64_t r0 = 0; r0 < R; r0 += RB) {
      load_block<RB, W>(x + off + r0 * inner, inner, (R - r0 < RB) ? (R - r0) : RB, v);
#pragma unroll
      for (int w = 0; w < W; ++w) fold_block<RB>(v[w], m[w], s[w]);
    }
  }
  float lns[W];
#pragma unroll
  for (int w = 0; w < W; ++w) lns[w] = logf(s[w]);
  for (int64_t r0 = 0; r0 < R; r0 += RB) {
    const int64_t nb = (R - r0 < RB) ? (R - r0) : RB;
    if (R > RB) load_block<RB, W>(x + off + r0 * inner, inner, nb, v);
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      if (i < nb) {
        float r[W];
#pragma unroll
        for (int w = 0; w < W; ++w) r[w] = (v[w][i] - m[w]) - lns[w];
        store_w<W>(y + off + (r0 + i) * inner, r);
      }
    }
  }
}

template <int RB, bool LSM>
hipError_t launch_rb(const float *x, float *out, int64_t outer, int64_t R, int64_t inner,
                     bool vec, hipStream_t stream) {
  const int64_t items = outer * (vec ? inner / kVecW : inner);
  const dim3 grid((uint32_t)((items + kAxis0Threads - 1) / kAxis0Threads));
  if constexpr (LSM) {
    const dim3 lgrid((uint32_t)((items + kLsmThreads - 1) / kLsmThreads));
    if (vec)
      hipLaunchKernelGGL((log_softmax_axis_kernel<RB, kVecW>), lgrid, dim3(kLsmThreads), 0,
                         stream, x, out, outer, R, inner);
    else
      hipLaunchKernelGGL((log_softmax_axis_kernel<RB, 1>), lgrid, dim3(kLsmThreads), 0, stream,
                         x, out, outer, R, inner);
  } else {
    if (vec)
      hipLaunchKernelGGL((lse_axis_kernel<RB, kVecW>), grid, dim3(kAxis0Threads), 0, stream, x,
                         out, outer, R, inner);
    else
      hipLaunchKernelGGL((lse_axis_kernel<RB, 1>), grid, dim3(kAxis0Threads), 0, stream, x, out,
                         outer, R, inner);
  }
  return hipGetLastError();
}

template <bool LSM>
hipError_t launch_axis(const float *x, float *out, int64_t outer, int64_t R, int64_t inner,
                       hipStream_t stream) {
  if (inner == 0 || outer == 0) return hipSuccess;
  const uintptr_t a = (uintptr_t)x | (uintptr_t)out;
  const bool vec = (inner % kVecW == 0) && (a % 16 == 0);
  if (R <= 4) return launch_rb<4, LSM>(x, out, outer, R, inner, vec, stream);
  if (R <= 8 || LSE_AXIS0_RBMAX <= 8) return launch_rb<8, LSM>(x, out, outer, R, inner, vec, stream);
  if (R <= 16 || LSE_AXIS0_RBMAX <= 16)
    return launch_rb<16, LSM>(x, out, outer, R, inner, vec, stream);
  if (LSM && R > 32 && R <= 64 && LSE_AXIS_LSM64_W == 4 && vec) {
    const dim3 grid((uint32_t)((outer * (inner / 4) + kLsmThreads - 1) / kLsmThreads));
    hipLaunchKernelGGL((log_softmax_axis_kernel<64, 4>), grid, dim3(kLsmThreads), 0, stream,
                       x, out, outer, R, inner);
    return hipGetLastError();
  }
  if (LSM && R > 32 && R <= 128) {
    // log_softmax keeps all R values in registers for the write: narrow the
    // per-lane vector so that R x W stays at 128 values (2 outputs per lane
    // up to 64 planes, 1 up to 128) instead of reading x twice.
    const int64_t items = outer * (R <= 64 && inner % 2 == 0 && a % 8 == 0 ? inner / 2 : inner);
    const dim3 grid((uint32_t)((items + kLsmThreads - 1) / kLsmThreads));
    if (R <= 64 && inner % 2 == 0 && a % 8 == 0)
      hipLaunchKernelGGL((log_softmax_axis_kernel<64, 2>), grid, dim3(kLsmThreads), 0, stream,
                         x, out, outer, R, inner);
    else
      hipLaunchKernelGGL((log_softmax_axis_kernel<128, 1>), grid, dim3(kLsmThreads), 0,
                         stream, x, out, outer, R, inner);
    return hipGetLastError();
  }
  return launch_rb<32, LSM>(x, out, outer, R, inner, vec, stream);
}

}  // namespace

hipError_t launch_lse_axis(const float *x, float *out, int64_t outer, int64_t R, int64_t inner,
                           hipStream_t stream) {
  return launch_axis<false>(x, out, outer, R, inner, stream);
}

hipError_t launch_log_softmax_axis(const float *x, float *y, int64_t outer, int64_t R,
                                   int64_t inner, hipStream_t stream) {
  return launch_axis<true>(x, y, outer, R, inner, stream);
}

}  // namespace lse
