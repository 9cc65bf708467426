// lse_axis0.hip — logsumexp over the leading axis of an (R, inner) array.
//
// POPCORNBENCH FW-GLM-5-1 l1_p29 (torch.logsumexp over dim 0 of (R,B,D)): each
// output (b,d) is independent; out = max + log(sum(exp(x - max))) over the R
// values.  That page gives one thread per output and rejects 128-bit loads
// because a thread's R values sit a whole plane apart.  Here the vector axis
// is the contiguous inner index instead: lane l owns outputs 4l..4l+3, and for
// each plane r one wave issues a single 1 KiB contiguous global_load_dwordx4
// span.  All RB planes of a block are issued before any is used and stay in
// VGPRs, so the max and the sum are an exact two-pass over registers with no
// cross-lane traffic.  R > RB streams blocks of RB planes, merging the running
// (max, sum) per output.
//
// Running state per output: m = max so far, s = sum of exp(v - c(m)) with the
// shift c(m) = m when m is finite and 0 when m is +-inf (all values -inf, or
// some +inf), which makes m + log(s) the literal log(sum(exp(v))) in every
// case: -inf -> log 0 = -inf, +inf -> log(inf) = +inf, NaN -> NaN.
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
constexpr int kAxis0Threads = LSE_AXIS0_THREADS;
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

// W consecutive values of one plane into column i of v (128-bit loads for W >= 4).
template <int W, int RB>
__device__ __forceinline__ void load_plane(const float *p, float (&v)[W][RB], int i) {
  if constexpr (W == 1) {
    v[0][i] = *p;
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

template <int RB, int W>
__global__ __launch_bounds__(kAxis0Threads) void lse_axis0_kernel(
    const float *__restrict__ x, float *__restrict__ out, int64_t R, int64_t inner) {
  const int64_t nq = inner / W;  // W > 1: inner % W == 0 by dispatch
  const int64_t q = (int64_t)blockIdx.x * kAxis0Threads + threadIdx.x;
  if (q >= nq) return;
  float m[W], s[W];
#pragma unroll
  for (int w = 0; w < W; ++w) {
    m[w] = -__builtin_inff();
    s[w] = 0.0f;
  }
  for (int64_t r0 = 0; r0 < R; r0 += RB) {
    const int64_t nb = (R - r0 < RB) ? (R - r0) : RB;
    float v[W][RB];
    const float *base = x + r0 * inner + q * W;
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
          for (int w = 0; w < W; ++w) v[w][i] = -__builtin_inff();  // identity
        }
      }
    }
#pragma unroll
    for (int w = 0; w < W; ++w) fold_block<RB>(v[w], m[w], s[w]);
  }
  float r[W];
#pragma unroll
  for (int w = 0; w < W; ++w) r[w] = m[w] + logf(s[w]);
  if constexpr (W == 1) {
    out[q] = r[0];
  } else {
#pragma unroll
    for (int h = 0; h < W / 4; ++h)
      *reinterpret_cast<float4 *>(out + q * W + 4 * h) =
          make_float4(r[4 * h], r[4 * h + 1], r[4 * h + 2], r[4 * h + 3]);
  }
}

template <int RB>
hipError_t launch_rb(const float *x, float *out, int64_t R, int64_t inner, bool vec,
                     hipStream_t stream) {
  const int64_t items = vec ? inner / kVecW : inner;
  const int64_t blocks = (items + kAxis0Threads - 1) / kAxis0Threads;
  if (vec)
    hipLaunchKernelGGL((lse_axis0_kernel<RB, kVecW>), dim3((uint32_t)blocks), dim3(kAxis0Threads),
                       0, stream, x, out, R, inner);
  else
    hipLaunchKernelGGL((lse_axis0_kernel<RB, 1>), dim3((uint32_t)blocks), dim3(kAxis0Threads),
                       0, stream, x, out, R, inner);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lse_axis0(const float *x, float *out, int64_t R, int64_t inner,
                            hipStream_t stream) {
  if (inner == 0) return hipSuccess;
  const bool vec = (inner % kVecW == 0) && ((uintptr_t)x % 16 == 0) && ((uintptr_t)out % 16 == 0);
  if (R <= 4) return launch_rb<4>(x, out, R, inner, vec, stream);
  if (R <= 8 || LSE_AXIS0_RBMAX <= 8) return launch_rb<8>(x, out, R, inner, vec, stream);
  if (R <= 16 || LSE_AXIS0_RBMAX <= 16) return launch_rb<16>(x, out, R, inner, vec, stream);
  return launch_rb<32>(x, out, R, inner, vec, stream);
}

}  // namespace lse
