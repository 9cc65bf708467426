// lse_rows.hip — row-wise log_softmax (and softmax) over long rows whose
// columns are contiguous (rows may sit any pitch ldx / ldy apart), and the
// per-chunk (max, sum) partial / merge building blocks.
//
// POPCORNBENCH Kimi-K2.6 l1_p24 (LogSoftmax over dim 1 of (4096, 393216)):
//   y_i = x_i - max - log(sum_j exp(x_j - max)); the minimum traffic is one
//   read and one write of the array; one row is 1.5 MiB; a row can be split
//   across blocks that each reduce their portion to a local (max, sum) and a
//   second phase combines them.  That page stays with one block per row and
//   re-reads the row for the write pass, and its warp-shuffle combine returns
//   NaN once idle lanes holding (-inf, 0) meet.
//
// Design here (gfx950):
//   * A workgroup of 512 lanes owns one chunk of up to 32768 columns and keeps
//     it in VGPRs (64 floats per lane, 16 non-temporal global_load_dwordx4 per
//     lane; each wave owns one contiguous 16 KiB run of the chunk), so the
//     chunk is read from HBM exactly once and written exactly once.  Full
//     chunks are stored through a raw buffer resource with the nt | sc1
//     cache-policy bits; partial chunks with non-temporal global stores.
//   * Exact chunk max (DPP/permlane wave reduce + LDS), then the sum of
//     exp(x - max) over the registers: one exponential per element.
//   * A row of k > 1 chunks: each workgroup publishes its pair as one packed
//     64-bit word (agent-scope compare-and-swap from 0), wave 0 polls the
//     row's k words, and every workgroup of the row merges the same k pairs in
//     the same order (so all get the bitwise-same row LSE) and writes its
//     chunk of y from registers.  A workgroup that has waited 50 us computes
//     any still-missing sibling pair itself from x, in its register tile with
//     the owner's own code (so the pair is bit-identical whoever computes it),
//     then reloads its own chunk; the first writer of a slot wins.  No global
//     counter is touched and no workgroup can wait on one that never starts,
//     whatever the dispatch order.
//   * Rows off the 16-byte grid (odd lengths, views at another 4-byte phase,
//     pitches not a multiple of 4): the register tile is framed on the output
//     row's first 128-byte line, so the stores stay aligned 16-byte buffer
//     stores, and the loads read x at its own 4-byte phase as 16-byte
//     accesses; the at most 31 columns before the frame and 3 after its last
//     whole vector are one extra value per lane for lanes 0..33 of wave 0.
//   * The write is y = (x - M) - log(S): x - M is exact for the large entries,
//     so the result keeps its accuracy when |M| is large.
//   * Rows of up to 1024 columns are one segment of 1-64 lanes each, several
//     rows per wave (rows_seg_kernel), with segment-wide DPP / permlane
//     reductions and no LDS; the last-axis reductions of the axis calls run
//     here too (logsumexp alone: one value per row).
//   * Rows of more than 128 chunks, whose chunks may not all be resident at
//     once to wait for each other, take three launches: chunk pairs (cached
//     loads), a merge per row, the write from the merged (M, log S), reading x
//     twice.
//   * A launch covers at most kMaxRowsWorkgroups workgroups (its work-item
//     count must fit 32 bits); longer grids are split into launches over
//     consecutive rows.
#include <atomic>
#include <type_traits>

#include "lse_device.hpp"
#include "lse_internal.hpp"

namespace lse {
namespace {

constexpr int kNW = kRowsThreads / kWave;  // waves per workgroup
#ifndef LSE_ROWS_SLEEP
#define LSE_ROWS_SLEEP 8          // s_sleep argument between polls (x 64 clocks)
#endif
#ifndef LSE_ROWS_NT_LOAD
#define LSE_ROWS_NT_LOAD 1        // x is read once from HBM: non-temporal loads
#endif
#ifndef LSE_ROWS_NT_STORE
#define LSE_ROWS_NT_STORE 1       // y is never re-read: non-temporal stores
#endif
#ifndef LSE_ROWS_KEEP_FOR_APPLY
#define LSE_ROWS_KEEP_FOR_APPLY 1  // three-launch rows: the pair launch reads x with cached loads
#endif
#ifndef LSE_ROWS_WAIT_MAX_CHUNKS
// Rows of up to this many chunks merge by waiting for their sibling
// workgroups; longer ones (more than 4M columns) take three launches, since a
// row's chunks may then not all fit on the GPU at once and the waiting
// workgroups would fall back to recomputing their siblings' pairs (one row of
// 153 chunks waiting: 12 % slower than three launches; rows of 65-128 chunks:
// 1-56 % faster, e.g. (64, 2200000) 3900 -> 5300 GB/s).
#define LSE_ROWS_WAIT_MAX_CHUNKS 128
#endif
constexpr uint32_t kDefaultSpinLimit = 1u << 24;
// Poll limit of the split rows' and the conv chain's waits, per host thread
// (a test hook: 0 forces every pair through the helping path).
thread_local uint32_t h_spin_limit = kDefaultSpinLimit;
// Test hook: split rows through the MALL re-read kernel (aligned rows only).
thread_local bool h_rows_reread = false;
// Workgroups of kRowsThreads lanes per launch: the dispatch's work-item count
// (workgroups x lanes) must fit 32 bits.
constexpr int64_t kMaxRowsWorkgroups = 0xffffffffll / kRowsThreads;

#ifndef LSE_ROWS_WAVE_CONTIG
#define LSE_ROWS_WAVE_CONTIG 1
#endif
// Float4 index of register vector q of thread t within a chunk.  Either way a
// wave's access per q is one contiguous 1 KiB.  Here each wave owns one
// contiguous run of VPL / 4 KiB (16 KiB for a 32768-column chunk): 2.3 %
// faster on (4096, 393216) than the 8 waves tiling 8 KiB per q
// (LSE_ROWS_WAVE_CONTIG=0).
template <int VPL>
__device__ __forceinline__ int64_t vec4_index(int q, int t) {
#if LSE_ROWS_WAVE_CONTIG
  return ((int64_t)(t / kWave) * (VPL / 4) + q) * kWave + (t % kWave);
#else
  return (int64_t)q * kRowsThreads + t;
#endif
}

// Four floats loaded or stored as one 16-byte access at an address that is
// only known to be 4-byte aligned (gfx950 accepts dword-aligned 16-byte
// accesses).
typedef float v4a4 __attribute__((ext_vector_type(4), aligned(4)));

// Load a chunk of `len` values starting at p into v (lane-strided so that each
// wave's load is one contiguous span), padding with -inf.  A full chunk (the
// common case) takes an unchecked path.  p needs 4-byte alignment only (a
// row whose output is line-aligned and input is not loads 16 bytes at x's own
// phase); len is a multiple of 4.
template <int VPL, bool VEC, bool A16 = true, bool NT = LSE_ROWS_NT_LOAD != 0>
__device__ __forceinline__ void load_chunk(const float *__restrict__ p, int64_t len,
                                           float (&v)[VPL]) {
  typedef float v4a16 __attribute__((ext_vector_type(4)));
  typedef std::conditional_t<A16, v4a16, v4a4> v4;  // A16: p is 16-byte aligned
  const int t = threadIdx.x;
  if constexpr (VEC) {
    if (len == (int64_t)VPL * kRowsThreads) {
      const v4 *p4 = reinterpret_cast<const v4 *>(p);
#pragma unroll
      for (int q = 0; q < VPL / 4; ++q) {
        v4 f;
        if constexpr (NT)
          f = __builtin_nontemporal_load(p4 + vec4_index<VPL>(q, t));
        else
          f = p4[vec4_index<VPL>(q, t)];
        v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
      }
      return;
    }
#pragma unroll
    for (int q = 0; q < VPL / 4; ++q) {
      const int64_t idx = vec4_index<VPL>(q, t) * 4;
      if (idx < len) {
        const v4 f = *reinterpret_cast<const v4 *>(p + idx);
        v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * q + e] = -__builtin_inff();
      }
    }
  } else {
    static_assert(VEC, "chunks are loaded as aligned tiles (SpanSplit covers the rest)");
  }
}

typedef float v4f __attribute__((ext_vector_type(4)));

// y is written once and never re-read here: non-temporal 128-bit stores.
__device__ __forceinline__ void store4(float *p, float a, float b, float c, float d) {
#if LSE_ROWS_NT_STORE
  __builtin_nontemporal_store(v4f{a, b, c, d}, reinterpret_cast<v4f *>(p));
#else
  *reinterpret_cast<float4 *>(p) = make_float4(a, b, c, d);
#endif
}

// The output of one value: log_softmax (x - M) - log S, or softmax
// exp(x - M) * (1 / S); `k` is log S or 1 / S accordingly.
template <bool SOFTMAX>
__device__ __forceinline__ float out_value(float v, float M, float k) {
  if constexpr (SOFTMAX)
    return exp_base2(v - M) * k;
  else
    return (v - M) - k;
}

// Full chunks are stored through a raw buffer resource, which lets the store
// carry the sc1 cache-policy bit beside nt (aux word 18 = nt | sc1): 1 % faster
// on (4096, 393216) than the plain non-temporal global store (aux 2, nt alone,
// measured equal to it; no bits at all -5.5 %).  -1 keeps the global store.
#ifndef LSE_ROWS_STORE_AUX
#define LSE_ROWS_STORE_AUX 18
#endif

template <int VPL, bool VEC, bool SOFTMAX>
__device__ __forceinline__ void store_chunk(float *__restrict__ p, int64_t len,
                                            const float (&v)[VPL], float M, float k) {
  const int t = threadIdx.x;
#if LSE_ROWS_STORE_AUX >= 0
  if constexpr (VEC) {
    if (len == (int64_t)VPL * kRowsThreads) {
      // 0x00020000: the 32-bit data format of a raw buffer on gfx9 parts.
      const __amdgpu_buffer_rsrc_t r =
          __builtin_amdgcn_make_buffer_rsrc(p, 0, (int)(len * 4), 0x00020000);
#pragma unroll
      for (int q = 0; q < VPL / 4; ++q) {
        const v4f o = {out_value<SOFTMAX>(v[4 * q], M, k), out_value<SOFTMAX>(v[4 * q + 1], M, k),
                       out_value<SOFTMAX>(v[4 * q + 2], M, k),
                       out_value<SOFTMAX>(v[4 * q + 3], M, k)};
        __builtin_amdgcn_raw_buffer_store_b128(o, r, (int)(vec4_index<VPL>(q, t) * 16), 0,
                                               LSE_ROWS_STORE_AUX);
      }
      return;
    }
  }
#endif
  if constexpr (VEC) {
    const bool full = (len == (int64_t)VPL * kRowsThreads);
#pragma unroll
    for (int q = 0; q < VPL / 4; ++q) {
      const int64_t idx = vec4_index<VPL>(q, t) * 4;
      if (full || idx < len)
        store4(p + idx, out_value<SOFTMAX>(v[4 * q], M, k), out_value<SOFTMAX>(v[4 * q + 1], M, k),
               out_value<SOFTMAX>(v[4 * q + 2], M, k), out_value<SOFTMAX>(v[4 * q + 3], M, k));
    }
  } else {
    static_assert(VEC, "chunks are stored as aligned tiles (store_chunk_b32 otherwise)");
  }
}

// log S for log_softmax, 1 / S for softmax.
template <bool SOFTMAX>
__device__ __forceinline__ float out_scale(float S) {
  if constexpr (SOFTMAX)
    return 1.0f / S;
  else
    return logf(S);
}

// A span of values [p, p + len) whose start is 4-byte but not necessarily
// line aligned (an odd row length, a pitch that is not a multiple of 32
// floats, a base off a 128-byte boundary): h <= 31 values before the first
// 128-byte boundary of the frame pointer f (the output row, or the input
// when there is none), then a body of a multiple of 4 values, then tail <= 3
// values.  The body goes through the register tile with line-aligned 16-byte
// accesses on the frame's side; the head and tail values (at most 34) ride
// in one extra register of lanes 0 .. 33 of wave 0.
struct SpanSplit {
  int h, tail;
  int64_t body;
  __device__ __forceinline__ SpanSplit(const float *f, int64_t len) {
    h = (int)((32u - (uint32_t)(((uintptr_t)f >> 2) & 31u)) & 31u);
    if ((int64_t)h > len) h = (int)len;
    body = (len - h) & ~(int64_t)3;
    tail = (int)(len - h - body);
  }
};

// This lane's extra value of a span p (-inf and col = -1 if it holds none):
// lanes 0 .. h-1 take the head when `head`, the next lanes the tail when
// `tail` (wave 0 only: at most 34 values).
__device__ __forceinline__ float extra_value(const float *__restrict__ p, const SpanSplit &sp,
                                             bool head, bool tail, int64_t &col) {
  const int l = threadIdx.x;
  const int nh = head ? sp.h : 0, nt = tail ? sp.tail : 0;
  col = -1;
  if (l < nh)
    col = l;
  else if (l - nh < nt)
    col = sp.h + sp.body + (l - nh);
  return col >= 0 ? p[col] : -__builtin_inff();
}

// The chunk's pair (exact max, sum of exp(v - max)); identical in every lane.
// One running max and one running sum per lane, over e = 0 .. VPL-1 in order
// (a wave issues dependent VALU operations back to back, so more accumulators
// would buy no latency hiding), then the lane's extra value when EXTRA (the
// head / tail of a span that is not 16-byte aligned, -inf in lanes without
// one), then the workgroup reductions.
template <int VPL, bool EXTRA = false>
__device__ __forceinline__ void chunk_pair(const float (&v)[VPL], float *red, float &m,
                                           float &s, float xe = 0.0f) {
  float lm = v[0];
#pragma unroll
  for (int e = 1; e < VPL; ++e) lm = fmaxf(lm, v[e]);
  if constexpr (EXTRA) lm = fmaxf(lm, xe);
  m = block_allreduce<kNW>(lm, OpMax{}, red);
  float ls = 0.0f;
  if (is_finite(m)) {  // uniform branch: m is the same in every lane
#pragma unroll
    for (int e = 0; e < VPL; ++e) ls += exp_base2(v[e] - m);
    if constexpr (EXTRA) ls += exp_base2(xe - m);
  } else {
#pragma unroll
    for (int e = 0; e < VPL; ++e) ls += pair_term_nonfinite(v[e], m);
    if constexpr (EXTRA) ls += pair_term_nonfinite(xe, m);
  }
  s = block_allreduce<kNW>(ls, OpSum{}, red);
}

// chunk_pair of a chunk that is not in this workgroup's registers (a
// sibling's, computed by the helping path): the same values reach the same
// lanes and meet the same operations in the same order (the running max and
// the running sum over e = 0 .. VPL-1, then the lane's extra value when
// EXTRA, the same workgroup reductions), so the pair is bit-identical to the
// one the chunk's owner computes.  The tile is streamed twice (max, then sum)
// instead of held.  VEC: p is 4-byte aligned and len a multiple of 4.
template <int VPL, bool VEC, bool EXTRA>
__device__ __forceinline__ void chunk_pair_streamed(const float *__restrict__ p, int64_t len,
                                                    float xe, float *red, float &m, float &s) {
  const int t = threadIdx.x;
  // Value e = 4 q + r of lane t: VEC, element r of float4 vec4_index<VPL>(q, t)
  // (one pointer stepped by kStep4 float4 per q); otherwise element
  // e * kRowsThreads + t.  -inf past len, as load_chunk pads.
#if LSE_ROWS_WAVE_CONTIG
  constexpr int64_t kStep4 = kWave;
#else
  constexpr int64_t kStep4 = kRowsThreads;
#endif
  // !EXTRA: a chunk of an aligned row (16-byte aligned p); EXTRA: x's own phase.
  typedef float v4a16 __attribute__((ext_vector_type(4)));
  typedef std::conditional_t<EXTRA, v4a4, v4a16> v4;
  const v4 *p4;
  int64_t idx;
  auto start = [&]() {
    p4 = reinterpret_cast<const v4 *>(p) + vec4_index<VPL>(0, t);
    idx = VEC ? vec4_index<VPL>(0, t) * 4 : (int64_t)t;
  };
  auto values = [&](float (&f)[4]) {
    if constexpr (VEC) {
      if (idx < len) {
        const v4 g = *p4;
        f[0] = g.x; f[1] = g.y; f[2] = g.z; f[3] = g.w;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) f[r] = -__builtin_inff();
      }
      p4 += kStep4;
      idx += 4 * kStep4;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        f[r] = (idx < len) ? p[idx] : -__builtin_inff();
        idx += kRowsThreads;
      }
    }
  };
  start();
  float lm;
  {
    float f[4];
    values(f);
    lm = fmaxf(fmaxf(fmaxf(f[0], f[1]), f[2]), f[3]);
  }
#pragma unroll 1
  for (int q = 1; q < VPL / 4; ++q) {
    float f[4];
    values(f);
#pragma unroll
    for (int r = 0; r < 4; ++r) lm = fmaxf(lm, f[r]);
  }
  if constexpr (EXTRA) lm = fmaxf(lm, xe);
  m = block_allreduce<kNW>(lm, OpMax{}, red);
  start();
  float ls = 0.0f;
  const bool fin = is_finite(m);
#pragma unroll 1
  for (int q = 0; q < VPL / 4; ++q) {
    float f[4];
    values(f);
#pragma unroll
    for (int r = 0; r < 4; ++r) ls += fin ? exp_base2(f[r] - m) : pair_term_nonfinite(f[r], m);
  }
  if constexpr (EXTRA) ls += fin ? exp_base2(xe - m) : pair_term_nonfinite(xe, m);
  s = block_allreduce<kNW>(ls, OpSum{}, red);
}

// The pair of a chunk streamed from memory by the whole workgroup: an exact
// max pass, then a sum pass (the second read is served by cache).  Used for
// chunks longer than the register tile.
__device__ __forceinline__ void stream_chunk_pair(const float *__restrict__ p, int64_t len,
                                                  float *red, float &m, float &s) {
  float lm = -__builtin_inff();
  for (int64_t i = threadIdx.x; i < len; i += kRowsThreads) lm = fmaxf(lm, p[i]);
  m = block_allreduce<kNW>(lm, OpMax{}, red);
  float ls = 0.0f;
  if (is_finite(m)) {
    // compensated: over thousands of terms per lane the small ones would be
    // rounded away against the running sum
    float lc = 0.0f;
    for (int64_t i = threadIdx.x; i < len; i += kRowsThreads) {
      const float y = exp_base2(p[i] - m) - lc;
      const float t = ls + y;
      lc = (t - ls) - y;
      ls = t;
    }
    ls -= lc;
  } else {
    for (int64_t i = threadIdx.x; i < len; i += kRowsThreads) ls += pair_term_general(p[i], m);
  }
  s = block_allreduce<kNW>(ls, OpSum{}, red);
}

// Merge the k pairs at pairs[0..k) held by one wave; every lane returns the
// same (M, S).  Lanes stride over the pairs; the order is fixed.
__device__ __forceinline__ void wave_merge_pairs(const uint64_t *pairs, int64_t k, float &M,
                                                 float &S) {
  const int lane = threadIdx.x % kWave;
  float lm = -__builtin_inff();
  bool nan_seen = false;
  for (int64_t j = lane; j < k; j += kWave) {
    const uint64_t p = load_pair_agent(pairs + j);
    const float mj = pair_m(p), sj = pair_s(p);
    nan_seen |= (mj != mj) || (sj != sj);
    lm = fmaxf(lm, mj);
  }
  M = wave_allreduce(lm, OpMax{});
  float ls = 0.0f;
  for (int64_t j = lane; j < k; j += kWave) {
    const uint64_t p = load_pair_agent(pairs + j);
    ls += pair_s(p) * merge_weight(pair_m(p), M);
  }
  S = wave_allreduce(ls, OpSum{});
  if (__builtin_amdgcn_ballot_w64(nan_seen) != 0) {
    M = __builtin_nanf("");
    S = __builtin_nanf("");
  }
}

// How long a workgroup waits for its siblings before computing their pairs
// itself, in ticks of the 100 MHz real-time counter (50 us; a real wait is a
// few microseconds).
constexpr uint64_t kHelpTicks = 5000ull;

// Wave 0 polls until all k pair words of a row are non-zero (true), or the
// poll limit or the time threshold runs out (false).
__device__ __forceinline__ bool wave_wait_pairs(const uint64_t *pairs, int64_t k,
                                                uint32_t limit) {
  const int lane = threadIdx.x % kWave;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (uint32_t it = 0;; ++it) {
    bool missing = false;
    for (int64_t j = lane; j < k; j += kWave) missing |= (load_pair_agent(pairs + j) == 0);
    if (__builtin_amdgcn_ballot_w64(missing) == 0) return true;
    if (it >= limit || __builtin_amdgcn_s_memrealtime() - t0 > kHelpTicks) return false;
    __builtin_amdgcn_s_sleep(LSE_ROWS_SLEEP);
  }
}

// One workgroup = one (row, chunk).  SPLIT: rows of nchunks > 1 chunks whose
// pairs are merged through the workspace.  !SPLIT: one workgroup per row.
//
// Split rows: blockIdx.x, in row-major order, picks the (row, chunk), so the
// chunks of a row are dispatched together and the workgroups in flight
// stream one contiguous region of x and y.  (Giving each of the 8 XCDs its
// own run of whole rows instead was measured 30% slower.)  Each workgroup
// publishes its pair with a compare-and-swap from 0 and waits for its
// siblings.  A workgroup that has waited kHelpTicks (or spin_limit polls)
// computes every still-missing sibling pair itself from x, which is
// read-only, and publishes it the same way; the first writer of a slot wins,
// so all workgroups of a row merge identical pairs.  Progress therefore never
// depends on the order or timing in which blocks are dispatched: no workgroup
// waits on one that has not started.
template <int VPL, bool VEC, bool SPLIT, bool SOFTMAX>
__global__ __launch_bounds__(kRowsThreads) void log_softmax_rows_kernel(
    const float *__restrict__ x, float *__restrict__ y, int64_t rows, int64_t cols,
    int64_t ldx, int64_t ldy, int64_t nchunks, int64_t chunk, RowsWsHeader *__restrict__ hdr,
    uint64_t *__restrict__ pairs, uint32_t spin_limit) {
  __shared__ float red[kNW];
  __shared__ int s_state;
  __shared__ float s_final[2];
  int64_t row, c;
  if constexpr (SPLIT) {
    const int64_t t = blockIdx.x;
    row = t / nchunks;
    c = t - row * nchunks;
  } else {
    row = blockIdx.x;
    c = 0;
  }
  const float *xrow = x + row * ldx;
  float *yrow = y + row * ldy;
  // VEC: every row of x and y 16-byte aligned with cols % 4 == 0; chunk c
  // covers columns [c chunk, ...).  Otherwise the chunks tile the row's body,
  // which starts sp.h columns in, where y's row reaches a 128-byte boundary
  // (so every store is a whole-line 16-byte store; the loads take x's own
  // phase), and the row's head and tail values ride as extra values with
  // chunk 0 and the last chunk.
  int64_t c0 = c * chunk, len;
  SpanSplit sp(yrow, cols);
  if constexpr (VEC) {
    len = (cols - c0 < chunk) ? (cols - c0) : chunk;
  } else {
    len = sp.body - c0;
    len = len < 0 ? 0 : (len < chunk ? len : chunk);
    c0 += sp.h;
  }
  const float *xr = xrow + c0;
  float *yr = yrow + c0;

  float v[VPL];
  load_chunk<VPL, true, VEC>(xr, len, v);
  float xe = 0.0f;
  int64_t xcol = -1;
  if constexpr (!VEC) xe = extra_value(xrow, sp, c == 0, c == nchunks - 1, xcol);
  float m, s;
  chunk_pair<VPL, !VEC>(v, red, m, s, xe);

  float M, lnS;
  if constexpr (SPLIT) {
    uint64_t *row_pairs = pairs + row * nchunks;
    // spin_limit == 0 is a test mode: the owner leaves its slot to the
    // helping path, so every pair of the row is computed by a helper.
    if (threadIdx.x == 0 && spin_limit != 0) publish_pair_once(row_pairs + c, pack_pair(m, s));
    for (;;) {
      if (threadIdx.x < kWave) {
        const bool all = wave_wait_pairs(row_pairs, nchunks, spin_limit);
        if (threadIdx.x == 0) s_state = all ? 1 : 0;
      }
      __syncthreads();
      if (s_state == 1) break;  // uniform: every thread read the same LDS word
      // Help: compute each still-missing sibling pair from x.
      for (int64_t j = 0; j < nchunks; ++j) {
        __syncthreads();
        if (threadIdx.x == 0) s_state = (load_pair_agent(row_pairs + j) == 0) ? 2 : 0;
        __syncthreads();
        if (s_state == 2) {
          int64_t j0 = j * chunk, lj;
          float hxe = 0.0f;
          if constexpr (VEC) {
            lj = (cols - j0 < chunk) ? (cols - j0) : chunk;
          } else {
            lj = sp.body - j0;
            lj = lj < 0 ? 0 : (lj < chunk ? lj : chunk);
            j0 += sp.h;
            int64_t hcol;
            hxe = extra_value(xrow, sp, j == 0, j == nchunks - 1, hcol);
          }
          float hm, hs;
          chunk_pair_streamed<VPL, true, !VEC>(xrow + j0, lj, hxe, red, hm, hs);
          if (threadIdx.x == 0 && publish_pair_once(row_pairs + j, pack_pair(hm, hs)))
            __hip_atomic_fetch_add(&hdr->helped, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      __syncthreads();
    }
    if (threadIdx.x < kWave) {
      float Mw, Sw;
      wave_merge_pairs(row_pairs, nchunks, Mw, Sw);
      if (threadIdx.x == 0) {
        s_final[0] = Mw;
        s_final[1] = out_scale<SOFTMAX>(Sw);
      }
    }
    __syncthreads();
    M = s_final[0];
    lnS = s_final[1];
  } else {
    M = m;
    lnS = out_scale<SOFTMAX>(s);
  }
  store_chunk<VPL, true, SOFTMAX>(yr, len, v, M, lnS);
  if constexpr (!VEC)
    if (xcol >= 0) yrow[xcol] = out_value<SOFTMAX>(xe, M, lnS);
}

// Clear n 64-bit words (the workspace header and pair slots); grid-stride, so
// any n fits a grid of at most kClearBlocks workgroups.
constexpr int64_t kClearBlocks = 4096;
__global__ __launch_bounds__(256) void clear_words_kernel(uint64_t *__restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0;
}
uint32_t clear_blocks(int64_t words) {
  const int64_t b = (words + 255) / 256;
  return (uint32_t)(b < kClearBlocks ? b : kClearBlocks);
}

// ------------------------------------------------------------ partial/merge
// One workgroup per (row, chunk) of a chunk that fits the register tile.
// KEEP: x is read again by a later launch (the three-launch rows): cached
// loads, so that it may still be in the Infinity Cache.
template <int VPL, bool VEC, bool KEEP = false>
__global__ __launch_bounds__(kRowsThreads) void lse_rows_partial_kernel(
    const float *__restrict__ x, int64_t cols, int64_t ldx, int64_t nchunks, int64_t chunk,
    float2 *__restrict__ partials) {
  constexpr bool kNt = LSE_ROWS_NT_LOAD != 0 && !KEEP;
  __shared__ float red[kNW];
  const int64_t t = blockIdx.x;
  const int64_t row = t / nchunks, c = t - row * nchunks;
  const int64_t c0 = c * chunk;
  const int64_t len = (cols - c0 < chunk) ? (cols - c0) : chunk;
  const float *xc = x + row * ldx + c0;
  float v[VPL];
  float m, s;
  if constexpr (VEC) {
    load_chunk<VPL, true, true, kNt>(xc, len, v);
    chunk_pair<VPL>(v, red, m, s);
  } else {  // the chunk's aligned body in the tile, its head and tail as extras
    const SpanSplit sp(xc, len);
    load_chunk<VPL, true, true, kNt>(xc + sp.h, sp.body, v);
    int64_t col;
    const float xe = extra_value(xc, sp, true, true, col);
    chunk_pair<VPL, true>(v, red, m, s, xe);
  }
  if (threadIdx.x == 0) partials[t] = make_float2(m, s);
}

// Chunks longer than the register tile.
__global__ __launch_bounds__(kRowsThreads) void lse_rows_partial_stream_kernel(
    const float *__restrict__ x, int64_t cols, int64_t ldx, int64_t nchunks, int64_t chunk,
    float2 *__restrict__ partials) {
  __shared__ float red[kNW];
  const int64_t t = blockIdx.x;
  const int64_t row = t / nchunks, c = t - row * nchunks;
  const int64_t c0 = c * chunk;
  const int64_t len = (cols - c0 < chunk) ? (cols - c0) : chunk;
  float m, s;
  stream_chunk_pair(x + row * ldx + c0, len, red, m, s);
  if (threadIdx.x == 0) partials[t] = make_float2(m, s);
}

// ---------------------------------------------------------- whole rows
// One workgroup per row and no workspace: the form the generic-axis calls
// take when they reduce a contiguous last axis (they have no workspace
// argument).  The logsumexp is written straight to out[row * ldo]; rows that
// fit the register tile are read once from registers, longer ones are read
// once with the online (max, sum) recurrence.  log_softmax / softmax of rows
// longer than the register tile take the pair the same way and then write y
// in a second pass over x.

// The logsumexp of one (max, sum) pair, with the merge's conventions.
__device__ __forceinline__ float pair_lse(float m, float s) {
  if (s != s) return __builtin_nanf("");
  return is_finite(m) ? m + logf(s) : m;
}

// stream_chunk_pair with 128-bit loads (VEC: p 16-byte aligned, len % 4 == 0).
template <bool VEC>
__device__ __forceinline__ void stream_row_pair(const float *__restrict__ p, int64_t len,
                                                float *red, float &m, float &s) {
  if constexpr (!VEC) {
    stream_chunk_pair(p, len, red, m, s);
  } else {
    const v4f *p4 = reinterpret_cast<const v4f *>(p);
    const int64_t n4 = len / 4;
    float lm = -__builtin_inff();
    for (int64_t i = threadIdx.x; i < n4; i += kRowsThreads) {
      const v4f f = p4[i];
      lm = fmaxf(lm, fmaxf(fmaxf(f.x, f.y), fmaxf(f.z, f.w)));
    }
    m = block_allreduce<kNW>(lm, OpMax{}, red);
    float ls = 0.0f;
    if (is_finite(m)) {
      for (int64_t i = threadIdx.x; i < n4; i += kRowsThreads) {
        const v4f f = p4[i];
        ls += (exp_base2(f.x - m) + exp_base2(f.y - m)) + (exp_base2(f.z - m) + exp_base2(f.w - m));
      }
    } else {
      for (int64_t i = threadIdx.x; i < n4; i += kRowsThreads) {
        const v4f f = p4[i];
        ls += (pair_term_general(f.x, m) + pair_term_general(f.y, m)) +
              (pair_term_general(f.z, m) + pair_term_general(f.w, m));
      }
    }
    s = block_allreduce<kNW>(ls, OpSum{}, red);
  }
}

#ifndef LSE_ROWS_STREAM_ONLINE
#define LSE_ROWS_STREAM_ONLINE 1   // whole streamed rows: one pass with the online recurrence
#endif

// Running pair of one lane: fold values into (m, s) with the online
// recurrence of the log_softmax page: a new maximum rescales the sum by
// exp(m_old - m_new), then each value adds exp(v - m).  The same conventions
// as chunk_pair: m is the largest non-NaN value, s counts +inf values when
// m = +inf, is 0 while m = -inf, and becomes NaN with any NaN.  Finite terms
// join s with Kahan's compensation c (a lane may add millions of them, most
// far below s, which plain addition would round away); total() is the
// compensated sum.
struct OnlinePair {
  float m = -__builtin_inff(), s = 0.0f, c = 0.0f;
  __device__ __forceinline__ void rescale_to(float mn) {
    if (mn != m) {  // m < mn: exp(m - mn) is 0 when m = -inf or mn = +inf
      const float f = exp_base2(m - mn);
      s *= f;
      c *= f;
      m = mn;
    }
  }
  __device__ __forceinline__ void add_finite(float g) {
    const float y = g - c;
    const float t = s + y;
    c = is_finite(t) ? (t - s) - y : 0.0f;
    s = t;
  }
  __device__ __forceinline__ void add4(float a, float b, float c4, float d) {
    rescale_to(fmaxf(m, fmaxf(fmaxf(a, b), fmaxf(c4, d))));
    if (is_finite(m)) {
      add_finite((exp_base2(a - m) + exp_base2(b - m)) + (exp_base2(c4 - m) + exp_base2(d - m)));
    } else {
      s += (pair_term_nonfinite(a, m) + pair_term_nonfinite(b, m)) +
           (pair_term_nonfinite(c4, m) + pair_term_nonfinite(d, m));
      c = 0.0f;
    }
  }
  __device__ __forceinline__ void add1(float a) {
    rescale_to(fmaxf(m, a));
    if (is_finite(m)) {
      add_finite(exp_base2(a - m));
    } else {
      s += pair_term_nonfinite(a, m);
      c = 0.0f;
    }
  }
  __device__ __forceinline__ float total() const { return is_finite(s) ? s - c : s; }
};

// The pair of a whole row read once: each lane folds its strided values with
// OnlinePair, then the lanes' pairs are merged (weights exp(m_lane - M)).
template <bool VEC>
__device__ __forceinline__ void online_row_pair(const float *__restrict__ p, int64_t len,
                                                float *red, float &M, float &S) {
  OnlinePair op;
  if constexpr (VEC) {
    const v4f *p4 = reinterpret_cast<const v4f *>(p);
    const int64_t n4 = len / 4;
    int64_t i = threadIdx.x;
    constexpr int U = 4;  // loads in flight per lane
    for (; i + (U - 1) * kRowsThreads < n4; i += U * kRowsThreads) {
      v4f f[U];
#pragma unroll
      for (int u = 0; u < U; ++u) f[u] = __builtin_nontemporal_load(p4 + i + u * kRowsThreads);
#pragma unroll
      for (int u = 0; u < U; ++u) op.add4(f[u].x, f[u].y, f[u].z, f[u].w);
    }
    for (; i < n4; i += kRowsThreads) {
      const v4f f = __builtin_nontemporal_load(p4 + i);
      op.add4(f.x, f.y, f.z, f.w);
    }
  } else {
    for (int64_t i = threadIdx.x; i < len; i += kRowsThreads) op.add1(p[i]);
  }
  M = block_allreduce<kNW>(op.m, OpMax{}, red);
  const float w = (op.m == M) ? 1.0f : exp_base2(op.m - M);
  S = block_allreduce<kNW>(op.total() * w, OpSum{}, red);
}

// ------------------------------------------------- MALL re-read variant
// The split log_softmax in the form that re-reads x for the write instead of
// keeping the chunk in registers (selected through the test hook, for the
// comparison with the register-resident kernel): pass 1 folds the chunk with
// the online (max, sum) recurrence, four 16-byte loads in flight per lane
// and cached (so that the re-read can hit the L2 or the Infinity Cache),
// using few registers, so that more workgroups fit; the pairs meet as in the
// register-resident kernel; pass 2 reads the chunk again and writes y.
// Aligned rows only (16-byte x and y rows, cols and the chunk multiples of 4).
__device__ __forceinline__ void cached_chunk_pair(const float *__restrict__ p, int64_t len,
                                                  float *red, float &M, float &S) {
  OnlinePair op;
  const v4f *p4 = reinterpret_cast<const v4f *>(p);
  const int64_t n4 = len / 4;
  int64_t i = threadIdx.x;
  constexpr int U = 4;  // loads in flight per lane
  for (; i + (U - 1) * kRowsThreads < n4; i += U * kRowsThreads) {
    v4f f[U];
#pragma unroll
    for (int u = 0; u < U; ++u) f[u] = p4[i + u * kRowsThreads];
#pragma unroll
    for (int u = 0; u < U; ++u) op.add4(f[u].x, f[u].y, f[u].z, f[u].w);
  }
  for (; i < n4; i += kRowsThreads) {
    const v4f f = p4[i];
    op.add4(f.x, f.y, f.z, f.w);
  }
  M = block_allreduce<kNW>(op.m, OpMax{}, red);
  const float w = (op.m == M) ? 1.0f : exp_base2(op.m - M);
  S = block_allreduce<kNW>(op.total() * w, OpSum{}, red);
}

template <bool SOFTMAX>
__global__ __launch_bounds__(kRowsThreads) void log_softmax_rows_reread_kernel(
    const float *__restrict__ x, float *__restrict__ y, int64_t cols, int64_t ldx, int64_t ldy,
    int64_t nchunks, int64_t chunk, RowsWsHeader *__restrict__ hdr,
    uint64_t *__restrict__ pairs, uint32_t spin_limit) {
  __shared__ float red[kNW];
  __shared__ int s_state;
  __shared__ float s_final[2];
  const int64_t t = blockIdx.x;
  const int64_t row = t / nchunks, c = t - row * nchunks;
  const int64_t c0 = c * chunk;
  const int64_t len = (cols - c0 < chunk) ? (cols - c0) : chunk;
  const float *xr = x + row * ldx + c0;
  float *yr = y + row * ldy + c0;
  float m, s;
  cached_chunk_pair(xr, len, red, m, s);
  uint64_t *row_pairs = pairs + row * nchunks;
  if (threadIdx.x == 0 && spin_limit != 0) publish_pair_once(row_pairs + c, pack_pair(m, s));
  for (;;) {
    if (threadIdx.x < kWave) {
      const bool all = wave_wait_pairs(row_pairs, nchunks, spin_limit);
      if (threadIdx.x == 0) s_state = all ? 1 : 0;
    }
    __syncthreads();
    if (s_state == 1) break;
    for (int64_t j = 0; j < nchunks; ++j) {  // help: missing sibling pairs from x
      __syncthreads();
      if (threadIdx.x == 0) s_state = (load_pair_agent(row_pairs + j) == 0) ? 2 : 0;
      __syncthreads();
      if (s_state == 2) {
        const int64_t j0 = j * chunk;
        float hm, hs;
        cached_chunk_pair(x + row * ldx + j0, (cols - j0 < chunk) ? (cols - j0) : chunk, red, hm,
                          hs);
        if (threadIdx.x == 0 && publish_pair_once(row_pairs + j, pack_pair(hm, hs)))
          __hip_atomic_fetch_add(&hdr->helped, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();
  }
  if (threadIdx.x < kWave) {
    float Mw, Sw;
    wave_merge_pairs(row_pairs, nchunks, Mw, Sw);
    if (threadIdx.x == 0) {
      s_final[0] = Mw;
      s_final[1] = out_scale<SOFTMAX>(Sw);
    }
  }
  __syncthreads();
  const float M = s_final[0], k = s_final[1];
  const v4f *x4 = reinterpret_cast<const v4f *>(xr);
  const int64_t n4 = len / 4;
  int64_t i = threadIdx.x;
  constexpr int U = 4;
  for (; i + (U - 1) * kRowsThreads < n4; i += U * kRowsThreads) {
    v4f f[U];
#pragma unroll
    for (int u = 0; u < U; ++u) f[u] = x4[i + u * kRowsThreads];
#pragma unroll
    for (int u = 0; u < U; ++u)
      store4(yr + 4 * (i + u * kRowsThreads), out_value<SOFTMAX>(f[u].x, M, k),
             out_value<SOFTMAX>(f[u].y, M, k), out_value<SOFTMAX>(f[u].z, M, k),
             out_value<SOFTMAX>(f[u].w, M, k));
  }
  for (; i < n4; i += kRowsThreads) {
    const v4f f = x4[i];
    store4(yr + 4 * i, out_value<SOFTMAX>(f.x, M, k), out_value<SOFTMAX>(f.y, M, k),
           out_value<SOFTMAX>(f.z, M, k), out_value<SOFTMAX>(f.w, M, k));
  }
}

template <bool VEC>
__device__ __forceinline__ void whole_row_pair(const float *__restrict__ p, int64_t len,
                                               float *red, float &m, float &s) {
#if LSE_ROWS_STREAM_ONLINE
  online_row_pair<VEC>(p, len, red, m, s);
#else
  stream_row_pair<VEC>(p, len, red, m, s);
#endif
}

template <int VPL, bool VEC>
__global__ __launch_bounds__(kRowsThreads) void rows_lse_kernel(const float *__restrict__ x,
                                                                int64_t cols, int64_t ldx,
                                                                float *__restrict__ out,
                                                                int64_t ldo) {
  __shared__ float red[kNW];
  const int64_t row = blockIdx.x;
  const float *xrow = x + row * ldx;
  float v[VPL];
  float m, s;
  if constexpr (VEC) {
    load_chunk<VPL, true>(xrow, cols, v);
    chunk_pair<VPL>(v, red, m, s);
  } else {  // the row's aligned body in the tile, its head and tail as extras
    const SpanSplit sp(xrow, cols);
    load_chunk<VPL, true>(xrow + sp.h, sp.body, v);
    int64_t col;
    const float xe = extra_value(xrow, sp, true, true, col);
    chunk_pair<VPL, true>(v, red, m, s, xe);
  }
  if (threadIdx.x == 0) out[row * ldo] = pair_lse(m, s);
}

template <bool VEC>
__global__ __launch_bounds__(kRowsThreads) void rows_lse_stream_kernel(
    const float *__restrict__ x, int64_t cols, int64_t ldx, float *__restrict__ out,
    int64_t ldo) {
  __shared__ float red[kNW];
  const int64_t row = blockIdx.x;
  float m, s;
  whole_row_pair<VEC>(x + row * ldx, cols, red, m, s);
  if (threadIdx.x == 0) out[row * ldo] = pair_lse(m, s);
}

#ifndef LSE_ROWS_SEG_MAX
#define LSE_ROWS_SEG_MAX 1024   // rows up to this many columns take a segment of a wave
#endif
#ifndef LSE_ROWS_SEG_A8
#define LSE_ROWS_SEG_A8 1  // rows of 2..32 values at differing phases: 8-byte accesses
#endif
// (same box, GB/s logsumexp / log_softmax, one value -> 8 bytes per access:
// 3 columns 3908 / 3378 -> 4886 / 4014, 17 columns 3568 / 3395 -> 3600 / 3857;
// from 99 columns on 8-byte accesses measured 6-15 % slower)
#ifndef LSE_ROWS_LSE_SEG_MAX
#define LSE_ROWS_LSE_SEG_MAX 2048  // logsumexp-only rows up to this long take a segment,
#endif
#ifndef LSE_ROWS_LSE_SEG_VEC_MAX
#define LSE_ROWS_LSE_SEG_VEC_MAX 3072  // ... and up to 4096 unless 16-byte aligned and longer than this
#endif
// (same box, GB/s: (200000, 2049) 4520 -> 6485, (50000, 2500) 5342 -> 6467, (131072, 3072)
// 6373 -> 6640, (100000, 4096) at a 4-byte offset 6360 -> 6561; aligned (100000, 4096) 7104 ->
// 6551 in a segment, so it keeps the workgroup kernel)
// Interleaved blocks (axis calls with inner > 1) take a wave-wide segment up
// to 64 values per lane: the axis kernels they would fall back to read such
// blocks 8-16 bytes per plane and lane.
constexpr int64_t kSegInterleavedMax = 64 * 64;
static_assert(LSE_ROWS_SEG_MAX >= 1 && LSE_ROWS_SEG_MAX <= 16 * 64,
              "a wave-wide segment holds at most 16 values per lane");
constexpr int kSegWaves = 4;    // waves per workgroup of the short-row kernel
#ifndef LSE_ROWS_SEG_VALUES_LSE
#define LSE_ROWS_SEG_VALUES_LSE 16  // values per lane in flight, row logsumexp only
#endif
#ifndef LSE_ROWS_SEG_VALUES_ROWS
#define LSE_ROWS_SEG_VALUES_ROWS 4  // values per lane in flight, (log-)softmax rows
#endif
enum RowsOut { kOutLogSoftmax = 0, kOutSoftmax = 1, kOutLse = 2 };
// Rows a segment takes per wave: enough that each lane has the values above
// in flight before the first reduction.
constexpr int seg_rows_per_pass(int vpl, int out) {
  const int target = out == kOutLse ? LSE_ROWS_SEG_VALUES_LSE : LSE_ROWS_SEG_VALUES_ROWS;
  return vpl >= target ? 1 : target / vpl;
}

// Short rows: a segment of G lanes (a power of two, 1..64) per row, 64 / G
// rows per wave (NR passes of them), kSegWaves waves per workgroup.  Lane s of
// a segment holds the row's 4-value vectors q G + s, padding with -inf: one
// 16-byte access each, at 16-byte alignment (kSegA16) or at the 4-byte phase
// all rows share (kSegA4: a view one float off the grid), or, when rows sit at
// differing phases, its values q G + s one per access (16-byte accesses
// straddling lines measured up to 18 % slower there).  Each load instruction
// of a segment reads one contiguous span of its row and, for packed rows
// (pitch = cols), the wave's load is one contiguous span across its rows.  The row's max and sum are all-reductions inside the
// segment (DPP and permlane swaps): no LDS, no barrier, no idle lanes for rows
// of a few to a thousand columns.  OUT picks the result: log_softmax or softmax
// rows from the registers, or the row's logsumexp alone (y[row * ldy]).  Same
// pair arithmetic as chunk_pair.
enum SegLayout {
  kSegA16 = 0,    // x, y 16-byte aligned, cols and pitches multiples of 4
  kSegA4 = 1,     // cols and pitches multiples of 4, x or y at another 4-byte phase
  kSegScalar = 2,  // rows at differing phases, one value per access
  kSegA8 = 3       // rows at differing phases, 8-byte accesses at 4-byte alignment
};
typedef float v2a4 __attribute__((ext_vector_type(2), aligned(4)));

// 16-byte load / non-temporal store at 4-byte alignment (gfx950 accepts
// dword-aligned 16-byte global accesses).
__device__ __forceinline__ v4a4 load4_a4(const float *p) {
#if LSE_ROWS_NT_LOAD
  return __builtin_nontemporal_load(reinterpret_cast<const v4a4 *>(p));
#else
  return *reinterpret_cast<const v4a4 *>(p);
#endif
}
__device__ __forceinline__ void store4_a4(float *p, float a, float b, float c, float d) {
  __builtin_nontemporal_store(v4a4{a, b, c, d}, reinterpret_cast<v4a4 *>(p));
}

// INNER > 1 (2, or a power of two from 4, 16-byte layouts only): each row is
// an (R, INNER) block of an axis reduction over R with INNER interleaved
// outputs.  INNER = 2: value e of a lane's 4-value vector belongs to output
// e % 2, and every lane keeps a (max, sum) for both.  INNER >= 4: a lane's
// vectors all start at the same column 4 (s % (INNER / 4)) of their planes
// (G is a multiple of INNER / 4), so value e belongs to output that + e % 4,
// and the lanes holding the same outputs (s equal mod INNER / 4) reduce
// together.
template <int G, int VPL, int NR, int LAY, int OUT, int INNER = 1>
__global__ __launch_bounds__(kWave * kSegWaves) void rows_seg_kernel(
    const float *__restrict__ x, float *__restrict__ y, int64_t rows, int64_t cols, int64_t ldx,
    int64_t ldy) {
  static_assert(INNER == 1 || (LAY != kSegScalar && LAY != kSegA8 && (INNER & (INNER - 1)) == 0),
                "interleaved outputs need 4-value vectors");
  constexpr int NACC = INNER >= 4 ? 4 : INNER;  // outputs a lane holds
  constexpr int LPC = INNER >= 4 ? INNER / 4 : 1;  // lanes per plane; s % LPC picks the outputs
  static_assert(G % LPC == 0, "a segment covers whole planes");
  constexpr bool SOFTMAX = OUT == kOutSoftmax;
  constexpr int kPerLoad = LAY == kSegScalar ? 1 : (LAY == kSegA8 ? 2 : 4);  // values per load
  constexpr int kSegs = kWave / G;                     // segments per wave
  const int lane = threadIdx.x % kWave;
  const int s = lane % G;
  const int64_t row0 =
      ((int64_t)blockIdx.x * kSegWaves + threadIdx.x / kWave) * (int64_t)(kSegs * NR);
  if (row0 >= rows) return;  // whole waves
  // Pass j of the wave covers rows row0 + j kSegs .. + kSegs - 1, one per
  // segment; segments past the last row hold -inf and store nothing.
  float v[NR][VPL];
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const int64_t row = row0 + j * kSegs + lane / G;
    const bool live = row < rows;
    const float *xr = x + (live ? row : row0) * ldx;
#pragma unroll
    for (int q = 0; q < VPL / kPerLoad; ++q) {
      const int64_t idx = ((int64_t)q * G + s) * kPerLoad;
      float *vq = &v[j][kPerLoad * q];
      if constexpr (LAY == kSegA16) {
        if (live && idx < cols) {  // cols % 4 == 0: a vector is wholly in or out
#if LSE_ROWS_NT_LOAD
          const v4f f = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(xr + idx));
#else
          const v4f f = *reinterpret_cast<const v4f *>(xr + idx);
#endif
          vq[0] = f.x; vq[1] = f.y; vq[2] = f.z; vq[3] = f.w;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) vq[r] = -__builtin_inff();
        }
      } else if constexpr (LAY == kSegA4) {
        if (live && idx < cols) {  // cols % 4 == 0: a vector is wholly in or out
          const v4a4 f = load4_a4(xr + idx);
          vq[0] = f.x; vq[1] = f.y; vq[2] = f.z; vq[3] = f.w;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) vq[r] = -__builtin_inff();
        }
      } else if constexpr (LAY == kSegA8) {
        if (live && idx + 2 <= cols) {
#if LSE_ROWS_NT_LOAD
          const v2a4 f = __builtin_nontemporal_load(reinterpret_cast<const v2a4 *>(xr + idx));
#else
          const v2a4 f = *reinterpret_cast<const v2a4 *>(xr + idx);
#endif
          vq[0] = f.x; vq[1] = f.y;
        } else {  // the last value of an odd row, or past the row
          vq[0] = (live && idx < cols) ? xr[idx] : -__builtin_inff();
          vq[1] = -__builtin_inff();
        }
      } else {
#if LSE_ROWS_NT_LOAD
        vq[0] = (live && idx < cols) ? __builtin_nontemporal_load(xr + idx) : -__builtin_inff();
#else
        vq[0] = (live && idx < cols) ? xr[idx] : -__builtin_inff();
#endif
      }
    }
  }
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    float M[NACC], S[NACC];
#pragma unroll
    for (int c = 0; c < NACC; ++c) {
      float lm = v[j][c];
#pragma unroll
      for (int e = c + NACC; e < VPL; e += NACC) lm = fmaxf(lm, v[j][e]);
      M[c] = coset_allreduce<LPC, G>(lm, OpMax{});
      float ls = 0.0f;
      if (is_finite(M[c])) {  // the same in every lane holding output c
#pragma unroll
        for (int e = c; e < VPL; e += NACC) ls += exp_base2(v[j][e] - M[c]);
      } else {
#pragma unroll
        for (int e = c; e < VPL; e += NACC) ls += pair_term_nonfinite(v[j][e], M[c]);
      }
      S[c] = coset_allreduce<LPC, G>(ls, OpSum{});
    }
    const int64_t row = row0 + j * kSegs + lane / G;
    if (row >= rows) continue;
    if constexpr (OUT == kOutLse) {
      if constexpr (INNER == 1) {
        if (s == 0) y[row * ldy] = pair_lse(M[0], S[0]);
      } else if constexpr (INNER >= 4) {
        // The G / LPC lanes of a set share its 4 outputs: lane s writes output
        // s / LPC of its set, and s / LPC + G / LPC, ... when the set has
        // fewer than 4 lanes.
        constexpr int kSetLanes = G / LPC;
#pragma unroll
        for (int c0 = 0; c0 < 4; c0 += kSetLanes) {
          const int cs = c0 + s / LPC;
          if (cs < 4) {
            float mc = M[0], sc = S[0];
#pragma unroll
            for (int c = 1; c < 4; ++c) {
              mc = (cs == c) ? M[c] : mc;
              sc = (cs == c) ? S[c] : sc;
            }
            y[row * ldy + 4 * (s % LPC) + cs] = pair_lse(mc, sc);
          }
        }
      } else {
        // lane s of the segment writes outputs s, s + G, ... (G < INNER for
        // blocks of fewer than 4 planes)
#pragma unroll
        for (int c0 = 0; c0 < INNER; c0 += G) {
          const int cs = c0 + s;
          if (cs < INNER) {
            float mc = M[0], sc = S[0];
#pragma unroll
            for (int c = 1; c < INNER; ++c) {
              mc = (cs == c) ? M[c] : mc;
              sc = (cs == c) ? S[c] : sc;
            }
            y[row * ldy + cs] = pair_lse(mc, sc);
          }
        }
      }
    } else {
      float k[NACC];
#pragma unroll
      for (int c = 0; c < NACC; ++c) k[c] = out_scale<SOFTMAX>(S[c]);
      float *yr = y + row * ldy;
#pragma unroll
      for (int q = 0; q < VPL / kPerLoad; ++q) {
        const int64_t idx = ((int64_t)q * G + s) * kPerLoad;
        const float *vq = &v[j][kPerLoad * q];
        if (idx < cols) {
          if constexpr (LAY == kSegScalar) {
            yr[idx] = out_value<SOFTMAX>(vq[0], M[0], k[0]);
          } else if constexpr (LAY == kSegA8) {
            const float o0 = out_value<SOFTMAX>(vq[0], M[0], k[0]);
            if (idx + 2 <= cols)
              __builtin_nontemporal_store(v2a4{o0, out_value<SOFTMAX>(vq[1], M[0], k[0])},
                                          reinterpret_cast<v2a4 *>(yr + idx));
            else
              yr[idx] = o0;
          } else {
            float o[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = out_value<SOFTMAX>(vq[r], M[r % NACC], k[r % NACC]);
            if constexpr (LAY == kSegA16)
              store4(yr + idx, o[0], o[1], o[2], o[3]);
            else
              store4_a4(yr + idx, o[0], o[1], o[2], o[3]);
          }
        }
      }
    }
  }
}

template <bool VEC, bool SOFTMAX>
__global__ __launch_bounds__(kRowsThreads) void rows_stream_write_kernel(
    const float *__restrict__ x, float *__restrict__ y, int64_t cols, int64_t ldx,
    int64_t ldy) {
  __shared__ float red[kNW];
  const int64_t row = blockIdx.x;
  const float *xr = x + row * ldx;
  float *yr = y + row * ldy;
  float M, S;
  whole_row_pair<VEC>(xr, cols, red, M, S);
  const float k = out_scale<SOFTMAX>(S);
  if constexpr (VEC) {
    const v4f *x4 = reinterpret_cast<const v4f *>(xr);
    const int64_t n4 = cols / 4;
    int64_t i = threadIdx.x;
    constexpr int U = 4;  // loads in flight per lane
    for (; i + (U - 1) * kRowsThreads < n4; i += U * kRowsThreads) {
      v4f f[U];
#pragma unroll
      for (int u = 0; u < U; ++u) f[u] = __builtin_nontemporal_load(x4 + i + u * kRowsThreads);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t j = 4 * (i + u * kRowsThreads);
        store4(yr + j, out_value<SOFTMAX>(f[u].x, M, k), out_value<SOFTMAX>(f[u].y, M, k),
               out_value<SOFTMAX>(f[u].z, M, k), out_value<SOFTMAX>(f[u].w, M, k));
      }
    }
    for (; i < n4; i += kRowsThreads) {
      const v4f f = __builtin_nontemporal_load(x4 + i);
      store4(yr + 4 * i, out_value<SOFTMAX>(f.x, M, k), out_value<SOFTMAX>(f.y, M, k),
             out_value<SOFTMAX>(f.z, M, k), out_value<SOFTMAX>(f.w, M, k));
    }
  } else {
    for (int64_t i = threadIdx.x; i < cols; i += kRowsThreads)
      yr[i] = out_value<SOFTMAX>(xr[i], M, k);
  }
}

// One wave per row, 4 rows per workgroup: merges the row's nchunks chunk pairs.
// OUT = kOutLse writes the row's logsumexp to out[row]; kOutLogSoftmax /
// kOutSoftmax write the pair (M, log S) / (M, 1 / S) of the row to
// ((float2 *)out)[row] for rows_apply_kernel.
template <int OUT>
__global__ __launch_bounds__(256) void lse_rows_merge_kernel(const float2 *__restrict__ partials,
                                                             int64_t rows, int64_t nchunks,
                                                             float *__restrict__ out) {
  const int64_t row = (int64_t)blockIdx.x * (256 / kWave) + threadIdx.x / kWave;
  if (row >= rows) return;  // whole wave exits together
  const int lane = threadIdx.x % kWave;
  const float2 *pr = partials + row * nchunks;
  float lm = -__builtin_inff();
  bool nan_seen = false;
  for (int64_t j = lane; j < nchunks; j += kWave) {
    const float2 p = pr[j];
    nan_seen |= (p.x != p.x) || (p.y != p.y);
    lm = fmaxf(lm, p.x);
  }
  const float M = wave_allreduce(lm, OpMax{});
  float ls = 0.0f;
  for (int64_t j = lane; j < nchunks; j += kWave) {
    const float2 p = pr[j];
    ls += p.y * merge_weight(p.x, M);
  }
  const float S = wave_allreduce(ls, OpSum{});
  if (lane == 0) {
    const bool nan = __builtin_amdgcn_ballot_w64(nan_seen) != 0;
    if constexpr (OUT == kOutLse) {
      out[row] = nan ? __builtin_nanf("") : (is_finite(M) ? M + logf(S) : M);
    } else {
      const float k = nan ? __builtin_nanf("") : out_scale<OUT == kOutSoftmax>(S);
      reinterpret_cast<float2 *>(out)[row] = make_float2(M, k);
    }
  }
}

// Running merge of pair (mk, sk) into (m, s), both in the chunk pairs'
// convention (s relative to m; +inf counted, -inf and NaN-free as in
// chunk_pair): the same in either operand order, bit for bit.
__device__ __forceinline__ void merge_pair_into(float &m, float &s, float mk, float sk) {
  const float mn = fmaxf(m, mk);
  s = s * merge_weight(m, mn) + sk * merge_weight(mk, mn);
  m = mn;
}

// lse_rows_merge_kernel for rows of many chunks: one 256-lane workgroup per
// row, lane i merging chunks i, i + 256, ... (4 loads in flight) in one pass,
// then the lanes' pairs merge across the wave and the 4 waves in a fixed
// order.  A NaN anywhere makes the sum NaN, and the row's result NaN.
template <int OUT>
__global__ __launch_bounds__(256) void rows_merge_wide_kernel(const float2 *__restrict__ partials,
                                                              int64_t nchunks,
                                                              float *__restrict__ out) {
  __shared__ float2 lds[4];
  const int64_t row = blockIdx.x;
  const float2 *pr = partials + row * nchunks;
  float m = -__builtin_inff(), s = 0.0f;
  for (int64_t k0 = threadIdx.x; k0 < nchunks; k0 += 4 * 256) {
    float2 q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      q[u] = (k0 + u * 256 < nchunks) ? pr[k0 + u * 256] : make_float2(-__builtin_inff(), 0.0f);
#pragma unroll
    for (int u = 0; u < 4; ++u) merge_pair_into(m, s, q[u].x, q[u].y);
  }
#pragma unroll
  for (int k = 1; k < kWave; k <<= 1) {
    const float mo = __shfl_xor(m, k), so = __shfl_xor(s, k);
    merge_pair_into(m, s, mo, so);
  }
  if (threadIdx.x % kWave == 0) lds[threadIdx.x / kWave] = make_float2(m, s);
  __syncthreads();
  if (threadIdx.x == 0) {
    float M = lds[0].x, S = lds[0].y;
#pragma unroll
    for (int w = 1; w < 4; ++w) merge_pair_into(M, S, lds[w].x, lds[w].y);
    const bool nan = S != S;
    if constexpr (OUT == kOutLse) {
      out[row] = nan ? __builtin_nanf("") : (is_finite(M) ? M + logf(S) : M);
    } else {
      const float k = nan ? __builtin_nanf("") : out_scale<OUT == kOutSoftmax>(S);
      reinterpret_cast<float2 *>(out)[row] = make_float2(M, k);
    }
  }
}

// Row merges: a wave per row, or a workgroup per row past 256 chunks.
#ifndef LSE_ROWS_MERGE_WIDE
#define LSE_ROWS_MERGE_WIDE 256
#endif
template <int OUT>
hipError_t launch_rows_merge(const float2 *partials, int64_t rows, int64_t nchunks, float *out,
                             hipStream_t stream) {
  const int64_t per = (OUT == kOutLse) ? 1 : 2;  // floats of output per row
  if (nchunks > LSE_ROWS_MERGE_WIDE) {
    return for_row_batches(rows, 0xffffffffll / 256, [&](int64_t r0, int64_t nr) {
      hipLaunchKernelGGL(rows_merge_wide_kernel<OUT>, dim3((uint32_t)nr), dim3(256), 0, stream,
                         partials + r0 * nchunks, nchunks, out + r0 * per);
      return hipGetLastError();
    });
  }
  return for_row_batches(rows, 4 * (0xffffffffll / 256), [&](int64_t r0, int64_t nr) {
    hipLaunchKernelGGL(lse_rows_merge_kernel<OUT>, dim3((uint32_t)((nr + 3) / 4)), dim3(256), 0,
                       stream, partials + r0 * nchunks, nr, nchunks, out + r0 * per);
    return hipGetLastError();
  });
}

// Third launch of a row split into more chunks than can wait for each other:
// y = out_value(x, M, k) over one kRowsTile chunk of one row per workgroup,
// from the row's merged (M, k).  VEC: x, y 16-byte aligned, cols and pitches
// multiples of 4.
template <bool VEC, bool SOFTMAX>
__global__ __launch_bounds__(kRowsThreads) void rows_apply_kernel(
    const float *__restrict__ x, float *__restrict__ y, int64_t cols, int64_t ldx, int64_t ldy,
    int64_t nchunks, const float2 *__restrict__ fin) {
  constexpr int kVec = (int)(kRowsTile / (4 * kRowsThreads));  // float4 per lane
  const int64_t b = blockIdx.x;
  const int64_t row = b / nchunks;
  const int64_t c0 = (b - row * nchunks) * kRowsTile;
  const int64_t len = (cols - c0 < kRowsTile) ? cols - c0 : kRowsTile;
  const float2 f = fin[row];
  const float *xr = x + row * ldx + c0;
  float *yr = y + row * ldy + c0;
  const int t = threadIdx.x;
  if constexpr (VEC) {
    v4f v[kVec];
#pragma unroll
    for (int q = 0; q < kVec; ++q) {
      const int64_t idx = ((int64_t)q * kRowsThreads + t) * 4;
      if (idx < len) v[q] = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(xr + idx));
    }
#pragma unroll
    for (int q = 0; q < kVec; ++q) {
      const int64_t idx = ((int64_t)q * kRowsThreads + t) * 4;
      if (idx < len)
        store4(yr + idx, out_value<SOFTMAX>(v[q].x, f.x, f.y), out_value<SOFTMAX>(v[q].y, f.x, f.y),
               out_value<SOFTMAX>(v[q].z, f.x, f.y), out_value<SOFTMAX>(v[q].w, f.x, f.y));
    }
  } else {
    for (int64_t i = t; i < len; i += kRowsThreads)
      yr[i] = out_value<SOFTMAX>(__builtin_nontemporal_load(xr + i), f.x, f.y);
  }
}

int vpl_for(int64_t len) {
  // smallest register tile (floats per lane) covering len columns
  if (len <= 4 * kRowsThreads) return 4;
  if (len <= 8 * kRowsThreads) return 8;
  if (len <= 16 * kRowsThreads) return 16;
  if (len <= 32 * kRowsThreads) return 32;
  return LSE_ROWS_SPLIT_VPL;  // a split chunk (up to kRowsSplitTile columns)
}

template <bool SPLIT, bool SOFTMAX>
hipError_t launch_rows_vpl(int vpl, bool vec, dim3 grid, const float *x, float *y, int64_t rows,
                           int64_t cols, int64_t ldx, int64_t ldy, int64_t nchunks,
                           int64_t chunk, RowsWsHeader *hdr, uint64_t *pairs,
                           uint32_t spin_limit, hipStream_t stream) {
#define LSE_ROWS_CASE(V)                                                                      \
  case V:                                                                                     \
    if (vec)                                                                                  \
      hipLaunchKernelGGL((log_softmax_rows_kernel<V, true, SPLIT, SOFTMAX>), grid,            \
                         dim3(kRowsThreads), 0, stream, x, y, rows, cols, ldx, ldy, nchunks,  \
                         chunk, hdr, pairs, spin_limit);                                      \
    else                                                                                      \
      hipLaunchKernelGGL((log_softmax_rows_kernel<V, false, SPLIT, SOFTMAX>), grid,           \
                         dim3(kRowsThreads), 0, stream, x, y, rows, cols, ldx, ldy, nchunks,  \
                         chunk, hdr, pairs, spin_limit);                                      \
    break;
  switch (vpl) {
    LSE_ROWS_CASE(4)
    LSE_ROWS_CASE(8)
    LSE_ROWS_CASE(16)
    LSE_ROWS_CASE(32)
#if LSE_ROWS_SPLIT_VPL > 32
    LSE_ROWS_CASE(LSE_ROWS_SPLIT_VPL)
#endif
    default:
      return hipErrorInvalidValue;
  }
#undef LSE_ROWS_CASE
  return hipGetLastError();
}

// Runs launch(r0, nr) over consecutive row ranges of at most max_rows rows,
// so that no single dispatch exceeds 32-bit work-item counts; stops at the
// first failed launch.
template <class F>
hipError_t for_row_batches(int64_t rows, int64_t max_rows, F launch) {
  if (max_rows < 1) return hipErrorInvalidConfiguration;  // one row alone is too large
  for (int64_t r0 = 0; r0 < rows; r0 += max_rows) {
    const int64_t nr = (rows - r0 < max_rows) ? (rows - r0) : max_rows;
    const hipError_t e = launch(r0, nr);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int G, int VPL, int OUT, int INNER>
void launch_seg(int lay, dim3 grid, hipStream_t stream, const float *x, float *y, int64_t rows,
                int64_t cols, int64_t ldx, int64_t ldy) {
  constexpr int NR = seg_rows_per_pass(VPL, OUT);
  const dim3 block(kWave * kSegWaves);
  if constexpr (INNER >= 4 && G % (INNER / 4) != 0)
    return;  // never chosen: a block of R >= 1 planes gives G >= INNER / 4
  else if (lay == kSegA16)
    hipLaunchKernelGGL((rows_seg_kernel<G, VPL, NR, kSegA16, OUT, INNER>), grid, block, 0, stream,
                       x, y, rows, cols, ldx, ldy);
  else if (lay == kSegA4)
    hipLaunchKernelGGL((rows_seg_kernel<G, VPL, NR, kSegA4, OUT, INNER>), grid, block, 0, stream,
                       x, y, rows, cols, ldx, ldy);
  else if constexpr (INNER == 1) {
    if (lay == kSegA8)
      hipLaunchKernelGGL((rows_seg_kernel<G, VPL, NR, kSegA8, OUT>), grid, block, 0, stream, x, y,
                         rows, cols, ldx, ldy);
    else
      hipLaunchKernelGGL((rows_seg_kernel<G, VPL, NR, kSegScalar, OUT>), grid, block, 0, stream,
                         x, y, rows, cols, ldx, ldy);
  }
}

// Rows of at most LSE_ROWS_SEG_MAX columns through rows_seg_kernel: the
// segment is the smallest power of two of lanes, up to a wave, whose 4 values
// per lane hold the row; a wave-wide segment holds 4, 8 or 16 values per lane.
// vec: x (and y, for the row outputs) 16-byte aligned, cols and the pitches
// multiples of 4.  For kOutLse, y[r * ldy] receives row r's logsumexp.
template <int OUT, int INNER = 1>
hipError_t launch_rows_seg(const float *x, float *y, int64_t rows, int64_t cols, int64_t ldx,
                           int64_t ldy, bool vec, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  if (cols < 1 || cols > (INNER > 1 || OUT == kOutLse ? kSegInterleavedMax : LSE_ROWS_SEG_MAX))
    return hipErrorInvalidValue;
  int g = 1;
  while (g < kWave && 4 * g < cols) g *= 2;
  int vpl = 4;
  if (g == kWave)
    while (vpl * kWave < cols) vpl *= 2;
  // 16-byte accesses when all rows share one 4-byte phase
  const bool one_phase = cols % 4 == 0 && ldx % 4 == 0 && (OUT == kOutLse || ldy % 4 == 0);
  const int lay = vec ? kSegA16
                : one_phase ? kSegA4
                : (LSE_ROWS_SEG_A8 && cols >= 2 && cols <= 32) ? kSegA8 : kSegScalar;
  if (INNER > 1 && (lay == kSegScalar || lay == kSegA8)) return hipErrorInvalidValue;
  if (INNER >= 4 && g < INNER / 4) return hipErrorInvalidValue;
  const int64_t rows_per_group = (int64_t)kSegWaves * (kWave / g) * seg_rows_per_pass(vpl, OUT);
  const int64_t max_groups = 0xffffffffll / (kWave * kSegWaves);  // 32-bit work-item count
  return for_row_batches(rows, max_groups * rows_per_group, [&](int64_t r0, int64_t nr) {
    const dim3 grid((uint32_t)((nr + rows_per_group - 1) / rows_per_group));
    const float *xb = x + r0 * ldx;
    float *yb = y + r0 * ldy;
    switch (g == kWave ? kWave * vpl : g) {
      case 1: launch_seg<1, 4, OUT, INNER>(lay, grid, stream, xb, yb, nr, cols, ldx, ldy); break;
      case 2: launch_seg<2, 4, OUT, INNER>(lay, grid, stream, xb, yb, nr, cols, ldx, ldy); break;
      case 4: launch_seg<4, 4, OUT, INNER>(lay, grid, stream, xb, yb, nr, cols, ldx, ldy); break;
      case 8: launch_seg<8, 4, OUT, INNER>(lay, grid, stream, xb, yb, nr, cols, ldx, ldy); break;
      case 16: launch_seg<16, 4, OUT, INNER>(lay, grid, stream, xb, yb, nr, cols, ldx, ldy); break;
      case 32: launch_seg<32, 4, OUT, INNER>(lay, grid, stream, xb, yb, nr, cols, ldx, ldy); break;
      case 4 * kWave: launch_seg<64, 4, OUT, INNER>(lay, grid, stream, xb, yb, nr, cols, ldx, ldy); break;
      case 8 * kWave: launch_seg<64, 8, OUT, INNER>(lay, grid, stream, xb, yb, nr, cols, ldx, ldy); break;
      case 16 * kWave: launch_seg<64, 16, OUT, INNER>(lay, grid, stream, xb, yb, nr, cols, ldx, ldy); break;
      case 32 * kWave:
        if constexpr (INNER > 1 || OUT == kOutLse) {
          launch_seg<64, 32, OUT, INNER>(lay, grid, stream, xb, yb, nr, cols, ldx, ldy);
          break;
        } else {
          return hipErrorInvalidValue;
        }
      case 64 * kWave:
        if constexpr (INNER > 1 || OUT == kOutLse) {
          launch_seg<64, 64, OUT, INNER>(lay, grid, stream, xb, yb, nr, cols, ldx, ldy);
          break;
        } else {
          return hipErrorInvalidValue;
        }
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  });
}

// ---------------------------------------------------------- multi-row
// Rows of 6144-16384 columns, at least 8192 of them: one 512-lane workgroup
// per row would hold only 12-32 values per lane (24-64 KiB per workgroup, its
// two reductions and barriers amortized over few bytes).  Here
// RPW rows share a workgroup, 512 / RPW lanes each with 64 values per lane (up
// to 128 KiB per workgroup, as the 32768-column rows): the row's waves
// all-reduce its max and sum through LDS, and y is written from the registers.
// (Same box, log_softmax GB/s: (50000, 8192) 5434 -> 5950, (25000, 16384) 4997
// -> 5527, (40000, 10000) 5469 -> 5783; rows of 4100 columns, half of each
// row's lanes idle, 5628 -> 5275, and (128, 16384), half the workgroups, 2185 ->
// 1698, keep one workgroup per row.)
#ifndef LSE_ROWS_MULTI
#define LSE_ROWS_MULTI 1
#endif
#ifndef LSE_ROWS_MULTI_A4
#define LSE_ROWS_MULTI_A4 1   // ... also rows off the 16-byte grid
#endif
#ifndef LSE_ROWS_MULTI_LSE
#define LSE_ROWS_MULTI_LSE 1  // ... and the row logsumexp
#endif
template <int RPW, int OUT, bool A4>
__global__ __launch_bounds__(kRowsThreads) void rows_multi_kernel(const float *__restrict__ x,
                                                                  float *__restrict__ y,
                                                                  int64_t rows, int64_t cols,
                                                                  int64_t ldx, int64_t ldy) {
  // A4: rows at their own 4-byte phase (an odd length or pitch, an offset
  // view): the row's lanes share it, so 16-byte accesses at 4-byte alignment
  // over the row's whole vectors; its last cols % 4 values ride in up to
  // three extra registers of the lane that would hold the next vector.
  constexpr int kLanes = kRowsThreads / RPW;  // lanes per row
  constexpr int kWpr = kLanes / kWave;        // waves per row
  constexpr int VPL = 64;
  constexpr bool SOFTMAX = OUT == kOutSoftmax;
  const float ninf = -__builtin_inff();
  __shared__ float red[kNW];
  const int t = threadIdx.x;
  const int r = t / kLanes, tl = t % kLanes;
  const int wave = t / kWave, lane = t % kWave;
  const int64_t row = (int64_t)blockIdx.x * RPW + r;
  const bool live = row < rows;
  const float *xr = x + (live ? row : 0) * ldx;
  const int64_t c4 = cols & ~(int64_t)3;  // the whole vectors
  float v[VPL];
#pragma unroll
  for (int q = 0; q < VPL / 4; ++q) {
    const int64_t idx = ((int64_t)q * kLanes + tl) * 4;  // a wave reads 1 KiB per q
    if (live && idx < c4) {
      v4f f;
      if constexpr (A4) {
        const v4a4 g = load4_a4(xr + idx);
        f = v4f{g.x, g.y, g.z, g.w};
      } else {
        f = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(xr + idx));
      }
      v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * q + e] = ninf;
    }
  }
  const int tail = (int)(cols - c4);
  const bool tail_lane = A4 && live && tail > 0 && tl == (int)((c4 / 4) % kLanes);
  float xt[3] = {ninf, ninf, ninf};
  if (tail_lane)
    for (int e = 0; e < tail; ++e) xt[e] = xr[c4 + e];
  float lm = fmaxf(xt[0], fmaxf(xt[1], xt[2]));
#pragma unroll
  for (int i = 0; i < VPL; ++i) lm = fmaxf(lm, v[i]);
  lm = wave_allreduce(lm, OpMax{});
  if (lane == 0) red[wave] = lm;
  __syncthreads();
  float M = red[r * kWpr];
#pragma unroll
  for (int w = 1; w < kWpr; ++w) M = fmaxf(M, red[r * kWpr + w]);
  __syncthreads();
  float ls[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (is_finite(M)) {
#pragma unroll
    for (int i = 0; i < VPL; ++i) ls[i % 4] += exp_base2(v[i] - M);
#pragma unroll
    for (int e = 0; e < 3; ++e) ls[e] += exp_base2(xt[e] - M);
  } else {
#pragma unroll
    for (int i = 0; i < VPL; ++i) ls[i % 4] += pair_term_nonfinite(v[i], M);
#pragma unroll
    for (int e = 0; e < 3; ++e) ls[e] += pair_term_nonfinite(xt[e], M);
  }
  const float lsum = wave_allreduce((ls[0] + ls[1]) + (ls[2] + ls[3]), OpSum{});
  if (lane == 0) red[wave] = lsum;
  __syncthreads();
  float S = red[r * kWpr];
#pragma unroll
  for (int w = 1; w < kWpr; ++w) S += red[r * kWpr + w];
  if (!live) return;
  if constexpr (OUT == kOutLse) {
    if (tl == 0) y[row * ldy] = pair_lse(M, S);
  } else {
    const float k = out_scale<SOFTMAX>(S);
    float *yr = y + row * ldy;
#pragma unroll
    for (int q = 0; q < VPL / 4; ++q) {
      const int64_t idx = ((int64_t)q * kLanes + tl) * 4;
      if (idx < c4) {
        const float o0 = out_value<SOFTMAX>(v[4 * q], M, k);
        const float o1 = out_value<SOFTMAX>(v[4 * q + 1], M, k);
        const float o2 = out_value<SOFTMAX>(v[4 * q + 2], M, k);
        const float o3 = out_value<SOFTMAX>(v[4 * q + 3], M, k);
        if constexpr (A4)
          store4_a4(yr + idx, o0, o1, o2, o3);
        else
          store4(yr + idx, o0, o1, o2, o3);
      }
    }
    if (tail_lane)
      for (int e = 0; e < tail; ++e)
        __builtin_nontemporal_store(out_value<SOFTMAX>(xt[e], M, k), yr + c4 + e);
  }
}

// Rows of 6144-16384 columns, at least 8192 of them, through
// rows_multi_kernel; false when the call does not fit.  vec: x and y rows
// 16-byte aligned with cols and the pitches multiples of 4.
template <int OUT>
bool launch_rows_multi(const float *x, float *y, int64_t rows, int64_t cols, int64_t ldx,
                       int64_t ldy, bool vec, hipStream_t stream, hipError_t &e) {
  if (!LSE_ROWS_MULTI || cols < 6144 || cols > 16384 || rows < 8192) return false;
  if (!vec && !LSE_ROWS_MULTI_A4) return false;
  const int rpw = cols <= 8192 ? 4 : 2;
  e = for_row_batches(rows, kMaxRowsWorkgroups * rpw, [&](int64_t r0, int64_t nr) {
    const dim3 grid((uint32_t)((nr + rpw - 1) / rpw)), block(kRowsThreads);
    const float *xb = x + r0 * ldx;
    float *yb = y + r0 * ldy;  // the row logsumexp: out[row * ldy]
    if (rpw == 4) {
      if (vec) hipLaunchKernelGGL((rows_multi_kernel<4, OUT, false>), grid, block, 0, stream, xb, yb, nr, cols, ldx, ldy);
      else hipLaunchKernelGGL((rows_multi_kernel<4, OUT, true>), grid, block, 0, stream, xb, yb, nr, cols, ldx, ldy);
    } else {
      if (vec) hipLaunchKernelGGL((rows_multi_kernel<2, OUT, false>), grid, block, 0, stream, xb, yb, nr, cols, ldx, ldy);
      else hipLaunchKernelGGL((rows_multi_kernel<2, OUT, true>), grid, block, 0, stream, xb, yb, nr, cols, ldx, ldy);
    }
    return hipGetLastError();
  });
  return true;
}

template <bool SOFTMAX>
hipError_t launch_rows_mode(const float *x, float *y, int64_t rows, int64_t cols, int64_t ldx,
                            int64_t ldy, void *ws, hipStream_t stream) {
  const RowsPlan p = rows_plan(cols);
  const bool vec = (cols % 4 == 0) && (p.chunk % 4 == 0) && (ldx % 4 == 0) &&
                   (ldy % 4 == 0) && ((uintptr_t)x % 16 == 0) && ((uintptr_t)y % 16 == 0);
  if (p.nchunks == 1 && cols <= LSE_ROWS_SEG_MAX)
    return launch_rows_seg<SOFTMAX ? kOutSoftmax : kOutLogSoftmax>(x, y, rows, cols, ldx, ldy,
                                                                   vec, stream);
  if (p.nchunks == 1) {
    hipError_t e = hipSuccess;
    if (launch_rows_multi<SOFTMAX ? kOutSoftmax : kOutLogSoftmax>(x, y, rows, cols, ldx, ldy, vec,
                                                                  stream, e))
      return e;
  }
  if (p.nchunks == 1) {
    return for_row_batches(rows, kMaxRowsWorkgroups, [&](int64_t r0, int64_t nr) {
      return launch_rows_vpl<false, SOFTMAX>(vpl_for(cols), vec, dim3((uint32_t)nr), x + r0 * ldx,
                                             y + r0 * ldy, nr, cols, ldx, ldy, 1, cols, nullptr,
                                             nullptr, 0u, stream);
    });
  }
  if (p.nchunks > LSE_ROWS_WAIT_MAX_CHUNKS) {
    // More chunks than can count on waiting for each other: the chunk pairs
    // of the register tile, a merge per row, then the write from the merged
    // (M, k) (x read twice).
    const int64_t nc = (cols + kRowsTile - 1) / kRowsTile;
    auto *part = reinterpret_cast<float2 *>(reinterpret_cast<char *>(ws) + sizeof(RowsWsHeader));
    float2 *fin = part + rows * nc;
    hipError_t e = launch_lse_rows_partial(x, rows, cols, ldx, kRowsTile, part, stream,
                                           LSE_ROWS_KEEP_FOR_APPLY != 0);
    if (e != hipSuccess) return e;
    e = launch_rows_merge<SOFTMAX ? kOutSoftmax : kOutLogSoftmax>(
        part, rows, nc, reinterpret_cast<float *>(fin), stream);
    if (e != hipSuccess) return e;
    return for_row_batches(rows, kMaxRowsWorkgroups / nc, [&](int64_t r0, int64_t nr) {
      const dim3 grid((uint32_t)(nr * nc));
      if (vec)
        hipLaunchKernelGGL((rows_apply_kernel<true, SOFTMAX>), grid, dim3(kRowsThreads), 0, stream,
                           x + r0 * ldx, y + r0 * ldy, cols, ldx, ldy, nc, fin + r0);
      else
        hipLaunchKernelGGL((rows_apply_kernel<false, SOFTMAX>), grid, dim3(kRowsThreads), 0,
                           stream, x + r0 * ldx, y + r0 * ldy, cols, ldx, ldy, nc, fin + r0);
      return hipGetLastError();
    });
  }
  auto *hdr = reinterpret_cast<RowsWsHeader *>(ws);
  auto *pairs = reinterpret_cast<uint64_t *>(reinterpret_cast<char *>(ws) + sizeof(RowsWsHeader));
  const int64_t words = (int64_t)(rows_workspace_bytes(rows, cols) / sizeof(uint64_t));
  hipLaunchKernelGGL(clear_words_kernel, dim3(clear_blocks(words)), dim3(256), 0, stream,
                     reinterpret_cast<uint64_t *>(ws), words);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint32_t spin = h_spin_limit;
  if (h_rows_reread && vec) {
    return for_row_batches(rows, kMaxRowsWorkgroups / p.nchunks, [&](int64_t r0, int64_t nr) {
      hipLaunchKernelGGL((log_softmax_rows_reread_kernel<SOFTMAX>), dim3((uint32_t)(nr * p.nchunks)),
                         dim3(kRowsThreads), 0, stream, x + r0 * ldx, y + r0 * ldy, cols, ldx,
                         ldy, p.nchunks, p.chunk, hdr, pairs + r0 * p.nchunks, spin);
      return hipGetLastError();
    });
  }
  return for_row_batches(rows, kMaxRowsWorkgroups / p.nchunks, [&](int64_t r0, int64_t nr) {
    return launch_rows_vpl<true, SOFTMAX>(vpl_for(p.chunk), vec, dim3((uint32_t)(nr * p.nchunks)),
                                          x + r0 * ldx, y + r0 * ldy, nr, cols, ldx, ldy,
                                          p.nchunks, p.chunk, hdr, pairs + r0 * p.nchunks, spin,
                                          stream);
  });
}

}  // namespace

void set_spin_limit(uint32_t polls) { h_spin_limit = polls; }
void set_rows_reread(bool on) { h_rows_reread = on; }
uint32_t chain_spin_limit() { return h_spin_limit; }

RowsPlan rows_plan(int64_t cols) {
  RowsPlan p;
  p.nchunks = (cols + kRowsSplitTile - 1) / kRowsSplitTile;
  if (p.nchunks < 1) p.nchunks = 1;
  // balance the chunks, keeping them a multiple of 4 columns
  int64_t chunk = (cols + p.nchunks - 1) / p.nchunks;
  chunk = (chunk + 3) / 4 * 4;
  if (chunk > kRowsSplitTile) chunk = kRowsSplitTile;
  p.chunk = chunk;
  p.nchunks = (cols + chunk - 1) / chunk;
  return p;
}

size_t rows_workspace_bytes(int64_t rows, int64_t cols) {
  const RowsPlan p = rows_plan(cols);
  if (p.nchunks <= 1) return 0;
  if (p.nchunks > LSE_ROWS_WAIT_MAX_CHUNKS)  // three launches: tile pairs, then (M, k) per row
    return sizeof(RowsWsHeader) +
           (size_t)rows * (size_t)((cols + kRowsTile - 1) / kRowsTile + 1) * sizeof(float2);
  return sizeof(RowsWsHeader) + (size_t)rows * (size_t)p.nchunks * sizeof(uint64_t);
}

hipError_t launch_log_softmax_rows(const float *x, float *y, int64_t rows, int64_t cols,
                                   int64_t ldx, int64_t ldy, void *ws, hipStream_t stream,
                                   bool softmax) {
  if (rows == 0) return hipSuccess;
  return softmax ? launch_rows_mode<true>(x, y, rows, cols, ldx, ldy, ws, stream)
                 : launch_rows_mode<false>(x, y, rows, cols, ldx, ldy, ws, stream);
}

hipError_t launch_lse_rows_partial(const float *x, int64_t rows, int64_t cols, int64_t ldx,
                                   int64_t chunk, void *partials, hipStream_t stream, bool keep) {
  if (rows == 0) return hipSuccess;
  const int64_t nchunks = (cols + chunk - 1) / chunk;
  const bool vec =
      (cols % 4 == 0) && (chunk % 4 == 0) && (ldx % 4 == 0) && ((uintptr_t)x % 16 == 0);
  const int vpl = chunk > kRowsTile ? 0 : vpl_for(chunk);
  return for_row_batches(rows, kMaxRowsWorkgroups / nchunks, [&](int64_t r0, int64_t nr) {
    const dim3 grid((uint32_t)(nr * nchunks));
    const float *xb = x + r0 * ldx;
    auto *out = reinterpret_cast<float2 *>(partials) + r0 * nchunks;
    if (vpl == 0) {
      hipLaunchKernelGGL(lse_rows_partial_stream_kernel, grid, dim3(kRowsThreads), 0, stream, xb,
                         cols, ldx, nchunks, chunk, out);
      return hipGetLastError();
    }
#define LSE_PART_CASE(V)                                                                       \
  case V:                                                                                      \
    if (vec && keep)                                                                           \
      hipLaunchKernelGGL((lse_rows_partial_kernel<V, true, true>), grid, dim3(kRowsThreads),   \
                         0, stream, xb, cols, ldx, nchunks, chunk, out);                       \
    else if (vec)                                                                              \
      hipLaunchKernelGGL((lse_rows_partial_kernel<V, true>), grid, dim3(kRowsThreads), 0,      \
                         stream, xb, cols, ldx, nchunks, chunk, out);                          \
    else if (keep)                                                                             \
      hipLaunchKernelGGL((lse_rows_partial_kernel<V, false, true>), grid, dim3(kRowsThreads),  \
                         0, stream, xb, cols, ldx, nchunks, chunk, out);                       \
    else                                                                                       \
      hipLaunchKernelGGL((lse_rows_partial_kernel<V, false>), grid, dim3(kRowsThreads), 0,     \
                         stream, xb, cols, ldx, nchunks, chunk, out);                          \
    break;
    switch (vpl) {
      LSE_PART_CASE(4)
      LSE_PART_CASE(8)
      LSE_PART_CASE(16)
      LSE_PART_CASE(32)
      default:
        return hipErrorInvalidValue;
    }
#undef LSE_PART_CASE
    return hipGetLastError();
  });
}

hipError_t launch_rows_lse(const float *x, int64_t rows, int64_t cols, int64_t ldx, float *out,
                           int64_t ldo, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const bool vec = (cols % 4 == 0) && (ldx % 4 == 0) && ((uintptr_t)x % 16 == 0);
  // Segments up to 2048 values, and up to 4096 for rows the workgroup kernel
  // reads one value per access (off the 16-byte grid) or that leave most of
  // its lanes with few values (up to 3072 columns).
  if (cols <= LSE_ROWS_LSE_SEG_MAX ||
      (cols <= kSegInterleavedMax && !(vec && cols > LSE_ROWS_LSE_SEG_VEC_MAX)))
    return launch_rows_seg<kOutLse>(x, out, rows, cols, ldx, ldo, vec, stream);
  if (LSE_ROWS_MULTI_LSE) {
    hipError_t e = hipSuccess;
    if (launch_rows_multi<kOutLse>(x, out, rows, cols, ldx, ldo, vec, stream, e)) return e;
  }
  return for_row_batches(rows, kMaxRowsWorkgroups, [&](int64_t r0, int64_t nr) {
    const dim3 grid((uint32_t)nr);
    const float *xb = x + r0 * ldx;
    float *ob = out + r0 * ldo;
    if (cols > kRowsTile) {
      if (vec)
        hipLaunchKernelGGL(rows_lse_stream_kernel<true>, grid, dim3(kRowsThreads), 0, stream, xb,
                           cols, ldx, ob, ldo);
      else
        hipLaunchKernelGGL(rows_lse_stream_kernel<false>, grid, dim3(kRowsThreads), 0, stream,
                           xb, cols, ldx, ob, ldo);
      return hipGetLastError();
    }
#define LSE_ROWLSE_CASE(V)                                                                     \
  case V:                                                                                      \
    if (vec)                                                                                   \
      hipLaunchKernelGGL((rows_lse_kernel<V, true>), grid, dim3(kRowsThreads), 0, stream, xb,  \
                         cols, ldx, ob, ldo);                                                  \
    else                                                                                       \
      hipLaunchKernelGGL((rows_lse_kernel<V, false>), grid, dim3(kRowsThreads), 0, stream, xb, \
                         cols, ldx, ob, ldo);                                                  \
    break;
    switch (vpl_for(cols)) {
      LSE_ROWLSE_CASE(4)
      LSE_ROWLSE_CASE(8)
      LSE_ROWLSE_CASE(16)
      LSE_ROWLSE_CASE(32)
      default:
        return hipErrorInvalidValue;
    }
#undef LSE_ROWLSE_CASE
    return hipGetLastError();
  });
}

hipError_t launch_log_softmax_rows_no_ws(const float *x, float *y, int64_t rows, int64_t cols,
                                         int64_t ldx, int64_t ldy, hipStream_t stream,
                                         bool softmax) {
  if (rows == 0) return hipSuccess;
  if (cols <= kRowsTile)  // one chunk per row: the register kernel needs no workspace
    return launch_log_softmax_rows(x, y, rows, cols, ldx, ldy, nullptr, stream, softmax);
  const bool vec = (cols % 4 == 0) && (ldx % 4 == 0) && (ldy % 4 == 0) &&
                   ((uintptr_t)x % 16 == 0) && ((uintptr_t)y % 16 == 0);
  return for_row_batches(rows, kMaxRowsWorkgroups, [&](int64_t r0, int64_t nr) {
    const dim3 grid((uint32_t)nr);
    const float *xb = x + r0 * ldx;
    float *yb = y + r0 * ldy;
#define LSE_ROWSTREAM(V, S)                                                                    \
  hipLaunchKernelGGL((rows_stream_write_kernel<V, S>), grid, dim3(kRowsThreads), 0, stream,    \
                     xb, yb, cols, ldx, ldy)
    if (vec) {
      if (softmax) LSE_ROWSTREAM(true, true); else LSE_ROWSTREAM(true, false);
    } else {
      if (softmax) LSE_ROWSTREAM(false, true); else LSE_ROWSTREAM(false, false);
    }
#undef LSE_ROWSTREAM
    return hipGetLastError();
  });
}

bool launch_axis_seg(const float *x, float *out, const AxisDims &d, bool lsm,
                     hipStream_t stream, hipError_t &e) {
  const int64_t cols = d.R * d.inner;
  const bool pow2 = d.inner >= 2 && d.inner <= 256 && (d.inner & (d.inner - 1)) == 0;
  if (!pow2 || d.xsr != d.inner || (lsm && d.ysr != d.inner) ||
      cols > kSegInterleavedMax || cols % 4 != 0 || d.xso % 4 != 0 || (lsm && d.yso % 4 != 0) ||
      d.outer < 1 || d.outer > 0x7fffffff)
    return false;
  // logsumexp over runs of 8+ outputs in blocks of at most 256 values: the
  // axis kernels' lanes, which need no cross-lane steps, measured faster
  // ((300000, 32, 8): 3410 against 3140 GB/s) unless the blocks have only a
  // few planes
  if (!lsm && d.inner >= 8 && cols <= 256 && d.R > 8) return false;
  const bool vec = ((uintptr_t)x % 16 == 0) && (!lsm || (uintptr_t)out % 16 == 0);
  auto go = [&](auto inner_c) {
    constexpr int I = decltype(inner_c)::value;
    return lsm ? launch_rows_seg<kOutLogSoftmax, I>(x, out, d.outer, cols, d.xso, d.yso, vec,
                                                    stream)
               : launch_rows_seg<kOutLse, I>(x, out, d.outer, cols, d.xso, d.yso, vec, stream);
  };
  switch (d.inner) {
    case 2: e = go(std::integral_constant<int, 2>{}); break;
    case 4: e = go(std::integral_constant<int, 4>{}); break;
    case 8: e = go(std::integral_constant<int, 8>{}); break;
    case 16: e = go(std::integral_constant<int, 16>{}); break;
    case 32: e = go(std::integral_constant<int, 32>{}); break;
    case 64: e = go(std::integral_constant<int, 64>{}); break;
    case 128: e = go(std::integral_constant<int, 128>{}); break;
    default: e = go(std::integral_constant<int, 256>{}); break;
  }
  return true;
}

hipError_t launch_lse_rows_merge(const void *partials, int64_t rows, int64_t nchunks,
                                 float *row_lse, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  return launch_rows_merge<kOutLse>(reinterpret_cast<const float2 *>(partials), rows, nchunks,
                                    row_lse, stream);
}

}  // namespace lse
