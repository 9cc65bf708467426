// lse_device.hpp — device building blocks shared by the gfx950 kernels:
// wave64 all-reductions on DPP row permutes plus the gfx950 permlane swaps,
// a workgroup all-reduce through LDS, the (max, sum) pair and its packing
// into one 64-bit word for cross-workgroup publication.
//
// The pair follows the pairwise combine on POPCORNBENCH Kimi-K2.6 l1_p24
// (LogSoftmax over dim 1): (m1,s1),(m2,s2) -> (M, s1 e^(m1-M) + s2 e^(m2-M)),
// M = max(m1,m2), with the weight of a term whose m equals M written as the
// exact 1 it is.  That keeps the identity (-inf, 0) and (+inf, n) pairs free of
// inf - inf, the NaN that page's own 32-lane reduction runs into when most
// lanes hold no data.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lse {

constexpr int kWave = 64;
constexpr float kLog2e = 1.44269504088896340736f;  // log2(e)

__device__ __forceinline__ uint32_t fbits(float v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ float bitsf(uint32_t v) { return __builtin_bit_cast(float, v); }

// exp(d) through the hardware base-2 exponential: 2^(d * log2 e).  Used for the
// bulk sums, where d = v - m <= 0 and the terms that matter have |d| small, so
// the rounding of d * log2 e costs well under an ulp of the sum.
__device__ __forceinline__ float exp_base2(float d) {
  return __builtin_amdgcn_exp2f(d * kLog2e);
}

__device__ __forceinline__ bool is_finite(float v) { return __builtin_isfinite(v); }

// ----------------------------------------------------------------- wave64
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return bitsf(__builtin_amdgcn_update_dpp(0u, fbits(v), CTRL, 0xF, 0xF, false));
}

struct OpMax {
  __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct OpSum {
  __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};

// All-reduce inside aligned segments of G lanes (G a power of two, 1..64):
// every lane ends with op over its segment, bitwise identical in every lane of
// the segment (each step combines the same two values, only in swapped operand
// order), and no value crosses a segment boundary.
template <int G, class Op>
__device__ __forceinline__ float seg_allreduce(float v, Op op) {
  static_assert(G >= 1 && G <= kWave && (G & (G - 1)) == 0, "segment of 1..64 lanes");
  if constexpr (G >= 2) v = op(v, dpp_mov<0xB1>(v));   // quad_perm [1,0,3,2]: lane ^ 1
  if constexpr (G >= 4) v = op(v, dpp_mov<0x4E>(v));   // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (G >= 8) v = op(v, dpp_mov<0x141>(v));  // row_half_mirror: the quads of 8
  if constexpr (G >= 16) v = op(v, dpp_mov<0x140>(v)); // row_mirror: halves of a 16-lane row
  if constexpr (G >= 32) {
    // v_permlane16_swap: the returned pair holds, in every lane, the values of
    // rows (0,1) or (2,3) of its row pair, so op of the two is the 32-lane result.
    auto p = __builtin_amdgcn_permlane16_swap(fbits(v), fbits(v), false, false);
    v = op(bitsf(p[0]), bitsf(p[1]));
  }
  if constexpr (G >= 64) {
    // v_permlane32_swap: the pair holds lane l % 32 and lane 32 + l % 32.
    auto q = __builtin_amdgcn_permlane32_swap(fbits(v), fbits(v), false, false);
    v = op(bitsf(q[0]), bitsf(q[1]));
  }
  return v;
}

// All-reduce over the lanes of a G-lane segment that agree mod LPC (powers of
// two, LPC <= G): LPC = 1 is seg_allreduce; otherwise the quad permute for
// lane ^ 2, then inside each 16-lane row a rotation by 8 (lane ^ 8) and by 4
// (after which every lane holds its residue class mod 4 of the row), and the
// permlane swaps for lane ^ 16 and lane ^ 32.  Every lane of a set ends with
// bitwise the same value (each step combines the same values in either order).
template <int LPC, int G, class Op>
__device__ __forceinline__ float coset_allreduce(float v, Op op) {
  static_assert(LPC >= 1 && LPC <= G && G <= kWave, "sets inside a segment");
  if constexpr (LPC == 1) {
    return seg_allreduce<G>(v, op);
  } else {
    if constexpr (LPC == 2 && G >= 4) v = op(v, dpp_mov<0x4E>(v));  // lane ^ 2
    if constexpr (G >= 16) {
      if constexpr (LPC <= 4) {
        v = op(v, dpp_mov<0x128>(v));  // row_ror:8 = lane ^ 8
        v = op(v, dpp_mov<0x124>(v));  // row_ror:4: the row's residue classes mod 4
      } else if constexpr (LPC == 8) {
        v = op(v, dpp_mov<0x128>(v));
      }
    } else if constexpr (G == 8 && LPC <= 4) {
      v = op(v, __shfl_xor(v, 4));  // lane ^ 4 inside an 8-lane segment
    }
    if constexpr (G >= 32 && LPC <= 16) {
      auto p = __builtin_amdgcn_permlane16_swap(fbits(v), fbits(v), false, false);
      v = op(bitsf(p[0]), bitsf(p[1]));
    }
    if constexpr (G >= 64 && LPC <= 32) {
      auto q = __builtin_amdgcn_permlane32_swap(fbits(v), fbits(v), false, false);
      v = op(bitsf(q[0]), bitsf(q[1]));
    }
    return v;
  }
}

// All 64 lanes end with op over the wave.
template <class Op>
__device__ __forceinline__ float wave_allreduce(float v, Op op) {
  return seg_allreduce<kWave>(v, op);
}

// Workgroup all-reduce of NW waves through `lds` (NW floats).  Every thread
// gets the same value; the trailing barrier lets the caller reuse `lds`.
template <int NW, class Op>
__device__ __forceinline__ float block_allreduce(float v, Op op, float *lds) {
  v = wave_allreduce(v, op);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x % kWave) == 0) lds[w] = v;
  __syncthreads();
  float r = lds[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = op(r, lds[i]);
  __syncthreads();
  return r;
}

// ------------------------------------------------------------------ pairs
// Term of the sum for a value v against the set's max m (m = max of the
// non-NaN values).  For finite m this is exp(v - m) (v = -inf gives 0, NaN
// gives NaN).  For m = -inf every non-NaN value is -inf and contributes 0; for
// m = +inf a +inf value contributes exactly 1 and a finite one 0.
__device__ __forceinline__ float pair_term_general(float v, float m) {
  if (v == m) return (m == -__builtin_inff()) ? 0.0f : 1.0f;
  return expf(v - m);
}

// The same term when m is known to be +-inf: v == m counts 1 for m = +inf
// and 0 for m = -inf, a NaN stays NaN, and anything else is exp(-inf) = 0.
__device__ __forceinline__ float pair_term_nonfinite(float v, float m) {
  const float hit = (m > 0.0f) ? 1.0f : 0.0f;
  return (v == m) ? hit : ((v != v) ? v : 0.0f);
}

// Weight of a partial whose max is mk inside a merge whose max is M.
__device__ __forceinline__ float merge_weight(float mk, float M) {
  return (mk == M) ? 1.0f : expf(mk - M);
}

// Shift of a running sum whose max is m: m itself when finite, 0 for +-inf
// (then exp(v - 0) counts a +inf value as inf and a -inf one as 0, and the
// final m + log s is +inf or -inf as it should be).
__device__ __forceinline__ float safe_shift(float m) { return is_finite(m) ? m : 0.0f; }

// Fold one block of NB values v[0..NB) of one output into its running (m, s):
// s is kept relative to safe_shift(m); a NaN value makes s NaN (fmaxf drops
// it from m), and m + log s is the logsumexp of everything folded.
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

// Weight-and-add step of merging running pairs (m_p, s_p) kept by fold_block
// into the merged max M: s_p exp(m_p - M) relative to safe_shift(M); a pair
// that counted nothing is skipped (its weight may be inf).
__device__ __forceinline__ float fold_weighted(float mp, float sp, float M) {
  return (sp != 0.0f) ? sp * exp_base2(safe_shift(mp) - safe_shift(M)) : 0.0f;
}

// Packed pair for single-word publication: low 32 bits m, high 32 bits s.  A
// real pair never packs to 0 (m = +0 implies s >= 1), so 0 means "not yet
// written" in a cleared workspace.
__device__ __forceinline__ uint64_t pack_pair(float m, float s) {
  return (uint64_t)fbits(m) | ((uint64_t)fbits(s) << 32);
}
__device__ __forceinline__ float pair_m(uint64_t p) { return bitsf((uint32_t)p); }
__device__ __forceinline__ float pair_s(uint64_t p) { return bitsf((uint32_t)(p >> 32)); }

// Publish p into an empty (zero) slot; false if the slot was already written.
__device__ __forceinline__ bool publish_pair_once(uint64_t *slot, uint64_t p) {
  uint64_t expected = 0;
  return __hip_atomic_compare_exchange_strong(slot, &expected, p, __ATOMIC_RELAXED,
                                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_pair_agent(const uint64_t *slot) {
  return __hip_atomic_load(const_cast<uint64_t *>(slot), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace lse
