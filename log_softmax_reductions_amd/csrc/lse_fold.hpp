// lse_fold.hpp — the running (m, s) fold for long streams of planes.
//
// fold_block (lse_device.hpp) adds each exponential straight into the running
// sum.  Over thousands of blocks the sum grows far above most of its terms,
// and a term below half an ulp of it is rounded away entirely: a one-sided
// loss (about 4.5e-5 of S for 18750 N(0, 9) values per lane, above the 2e-6
// relative tolerance).  Here a block's terms are summed on their own first,
// and the block sum is added to the rescaled running sum with a compensation
// term (Kahan's summation: the rounding error of each addition is carried
// into the next).  The first block of a stream (s = 0) gives exactly
// fold_block's bits, so streams of one block are unchanged.
#pragma once

#include "lse_device.hpp"

namespace lse {

#ifndef LSE_FOLD_COMP
#define LSE_FOLD_COMP 1   // 0: the plain fold_block (for comparisons)
#endif

template <int NB>
__device__ __forceinline__ void fold_block_c(const float (&v)[NB], float &m, float &s,
                                             float &comp) {
  if constexpr (LSE_FOLD_COMP == 0) {
    fold_block<NB>(v, m, s);
    comp = 0.0f;
    return;
  }
  float bm = v[0];
#pragma unroll
  for (int i = 1; i < NB; ++i) bm = fmaxf(bm, v[i]);
  const float mn = fmaxf(m, bm);
  const float c = safe_shift(mn);
  float b = 0.0f;
#pragma unroll
  for (int i = 0; i < NB; ++i) b += exp_base2(v[i] - c);
  if (s == 0.0f) {  // nothing counted yet: the rescale factor may be inf
    m = mn;
    s = b;
    comp = 0.0f;
    return;
  }
  const float sc = exp_base2(safe_shift(m) - c);
  const float base = s * sc;
  m = mn;
  if (!is_finite(base) || !is_finite(b)) {  // +-inf or NaN: no compensation
    s = base + b;
    comp = 0.0f;
    return;
  }
  const float y = b - comp * sc;
  const float t = base + y;
  comp = (t - base) - y;
  s = t;
}

// The compensated total of a stream folded by fold_block_c.
__device__ __forceinline__ float fold_total(float s, float comp) {
  return is_finite(s) ? s - comp : s;
}

}  // namespace lse
