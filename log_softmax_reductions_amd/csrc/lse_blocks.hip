// lse_blocks.hip — logsumexp and log_softmax over the middle axis of an
// (outer, R, inner) array whose (R, inner) blocks are each one contiguous run
// of memory and whose inner run is short: 2 to 256 columns, such as a
// reduction over the channels of 7 x 7 feature maps.  A plane of such a block
// is a few hundred bytes, so kernels that give each lane columns of its own
// read it in short pieces, one value per access when the run is not a
// multiple of 4.
//
// POPCORNBENCH FW-GLM-5-1 l1_p29 (torch.logsumexp over a leading axis): each
// output is the max-shifted sum over its R values, which here lie inner
// floats apart inside the block.  The block is read as the flat run it is:
//   * 4 consecutive floats per lane, a workgroup's lanes covering a sweep of
//     W consecutive floats, W a multiple of both 4 and inner (the largest
//     such W up to 1024); the next sweep is W floats on, so every lane meets
//     the same 4 columns, (4 t + e) mod inner, on every sweep and keeps one
//     running (m, s) for each (16-byte accesses at the block's own 4-byte
//     phase, shared by all lanes);
//   * the W / inner partials of each column are merged in a fixed order
//     through LDS;
//   * with a workspace, a block's planes are split into chunks, one
//     workgroup each, whose (m, s) pairs per column are merged afterwards in
//     chunk order (a merge launch for logsumexp; for log_softmax each
//     workgroup of the apply launch merges its block's pairs itself, the same
//     way, and writes (x - M) - log S over its chunk; past 8 chunks a merge
//     launch with a wave per column does it for both).  Without one, one
//     workgroup takes a whole block, and log_softmax reads it again;
//   * log_softmax keeps its values in registers where they fit (the split-row
//     protocol of log_softmax_rows, per column): a block of up to 16 sweeps
//     of a 256- or 512-lane workgroup is that workgroup's, loaded once and
//     written from registers; a longer one (with a workspace) is split into
//     chunks of up to 16 sweeps of 512 lanes whose workgroups publish their
//     (m, s) per column into zeroed slots
//     (compare-and-swap from 0), wait for their siblings', merge them in
//     chunk order and write from registers.  A workgroup that has waited too
//     long computes every still-missing sibling chunk's pairs itself from x,
//     in the owner's order (the first writer of a slot wins), so progress
//     never depends on dispatch order and the results not on who computed a
//     pair.
#include "lse_device.hpp"
#include "lse_fold.hpp"
#include "lse_internal.hpp"

namespace lse {
namespace {

#ifndef LSE_BLK_MAX_INNER
#define LSE_BLK_MAX_INNER 256      // widest inner run the kernels take
#endif
#ifndef LSE_BLK_TARGET_GROUPS
#define LSE_BLK_TARGET_GROUPS 1024 // workgroups the chunking aims for
#endif
#ifndef LSE_BLK_MAX_CHUNKS
#define LSE_BLK_MAX_CHUNKS 4096    // chunks per block at most
#endif
#ifndef LSE_BLK_SERIAL_CHUNKS
#define LSE_BLK_SERIAL_CHUNKS 8    // up to this many, one thread per column merges them
#endif
#ifndef LSE_BLK_U
#define LSE_BLK_U 4                // 16-byte loads per lane in flight
#endif
#ifndef LSE_BLK_MIN_TRIPS
#define LSE_BLK_MIN_TRIPS 4        // chunks of at least this many U-sweep trips
#endif
#ifndef LSE_BLK_GATE
#define LSE_BLK_GATE 1             // 0: never; 1: the shapes measured faster here; 2: every eligible call
#endif
#ifndef LSE_BLK_NOWS_MIN_OUTER
#define LSE_BLK_NOWS_MIN_OUTER 512 // without a workspace: at least this many blocks
#endif
#ifndef LSE_BLK_MIN_BLOCK
#define LSE_BLK_MIN_BLOCK 2048     // gate 1: blocks of at least this many floats,
#endif
#ifndef LSE_BLK_GATE_INNER
#define LSE_BLK_GATE_INNER 128     // ... inner runs up to this wide,
#endif
#ifndef LSE_BLK_RESIDENT
#define LSE_BLK_RESIDENT 1         // log_softmax from registers (one chunk, or chunks that wait)
#endif
#ifndef LSE_BLK_RES_MAX_CHUNKS
#define LSE_BLK_RES_MAX_CHUNKS 32  // ... for blocks of at most this many 16-sweep chunks
#endif
#ifndef LSE_BLK_RES_MIN_GROUPS
#define LSE_BLK_RES_MIN_GROUPS 2048 // ... and at least this many workgroups,
#endif
#ifndef LSE_BLK_RES_FEW_CHUNKS
#define LSE_BLK_RES_FEW_CHUNKS 16  // ... or, for blocks of at most this many chunks,
#endif
#ifndef LSE_BLK_RES_FEW_GROUPS
#define LSE_BLK_RES_FEW_GROUPS 256 // ... at least this many (160 up to 8 chunks),
#endif
#ifndef LSE_BLK_RES_SLOTS
#define LSE_BLK_RES_SLOTS 512      // ... outside (1, 2) x the 512-lane workgroups resident at once
#endif
#ifndef LSE_BLK_SLEEP
#define LSE_BLK_SLEEP 8            // s_sleep argument between polls (x 64 clocks)
#endif
#ifndef LSE_BLK_BIG_BLOCK
#define LSE_BLK_BIG_BLOCK 65536    // ... or, for logsumexp, blocks of at least this many floats
#endif

constexpr int kBlkThreads = 256;
constexpr int kBlkU = LSE_BLK_U;
constexpr int kBlkMaxInner = LSE_BLK_MAX_INNER;
static_assert(kBlkMaxInner <= kBlkThreads, "a period of at most one workgroup");

enum BlkMode {
  kBlkPartial = 0,      // the chunk's (m, s) per column into the workspace
  kBlkPartialKeep = 1,  // the same, x read with cached loads (the apply reads it again)
  kBlkLse = 2,          // one chunk: the logsumexp
  kBlkLsm = 3           // one chunk: log_softmax, the block read again
};

typedef float v4b4 __attribute__((ext_vector_type(4), aligned(4)));

// Sweep geometry of an inner run: lp lanes cover one period of lcm(4, inner)
// floats, a workgroup's act = (256 / lp) lp lanes a sweep of 4 act floats.
struct BlkSweep {
  int lp, act, w;
};
__host__ __device__ inline BlkSweep blk_sweep(int inner, int threads = kBlkThreads) {
  const int g = (inner % 4 == 0) ? 4 : ((inner % 2 == 0) ? 2 : 1);
  BlkSweep s;
  s.lp = inner / g;
  s.act = (threads / s.lp) * s.lp;
  s.w = 4 * s.act;
  return s;
}

// The lane's 4 floats at j of a run ending at f (floats at or past f read as
// fill).
template <bool NT>
__device__ __forceinline__ void blk_load4(const float *p, int64_t j, int64_t f, float fill,
                                          float (&v)[4]) {
  if (j + 4 <= f) {
    const v4b4 *a = reinterpret_cast<const v4b4 *>(p + j);
    const v4b4 q = NT ? __builtin_nontemporal_load(a) : *a;
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      v[e] = (j + e < f) ? (NT ? __builtin_nontemporal_load(p + j + e) : p[j + e]) : fill;
  }
}

// y = (x - M_e) - L_e over the lane's floats j, j + w, ... < f1 of the block
// (M_e, L_e: its 4 columns'), kBlkU loads in flight.
__device__ __forceinline__ void blk_write(const float *xb, float *yb, int64_t j, int64_t f1, int w,
                                          const float (&fm)[4], const float (&fl)[4]) {
  for (; j < f1; j += (int64_t)w * kBlkU) {
    float q[kBlkU][4];
#pragma unroll
    for (int u = 0; u < kBlkU; ++u) blk_load4<true>(xb, j + (int64_t)u * w, f1, 0.0f, q[u]);
#pragma unroll
    for (int u = 0; u < kBlkU; ++u) {
      const int64_t jj = j + (int64_t)u * w;
      float r[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = (q[u][e] - fm[e]) - fl[e];
      if (jj + 4 <= f1) {
        __builtin_nontemporal_store(v4b4{r[0], r[1], r[2], r[3]}, reinterpret_cast<v4b4 *>(yb + jj));
      } else {
#pragma unroll
        for (int e = 0; e < 3; ++e)
          if (jj + e < f1) __builtin_nontemporal_store(r[e], yb + jj + e);
      }
    }
  }
}

// (M, log S) of column t < inner from the block's chunk pairs (fixed order).
__device__ __forceinline__ float2 blk_merge_pairs(const float2 *p, int64_t chunks) {
  float M = p[0].x;
  for (int64_t k = 1; k < chunks; ++k) M = fmaxf(M, p[k].x);
  float S = 0.0f;
  for (int64_t k = 0; k < chunks; ++k) S += fold_weighted(p[k].x, p[k].y, M);
  return make_float2(M, S);
}

// Merge of the nk partials of each column c < inner, which sit at part[c +
// k inner] (flat index 4 lane + e of the sweep), into res[c] = (M, S): G
// lanes per column, lane g folding partials g, g + G, ... (max first, then
// the weighted sum), then reduced across the G lanes; the same order on every
// call.  G = the largest power of two up to nk / 4 (at most 64).
template <int G, int NT>
__device__ __forceinline__ void blk_merge_g(const float2 *part, float2 *res, int inner, int nk,
                                            int t) {
  constexpr int kCpw = kWave / G;  // columns per wave and round
  const int lane = t % kWave, wave = t / kWave;
  const int g = lane % G;
  for (int c0 = wave * kCpw; c0 < inner; c0 += (NT / kWave) * kCpw) {
    const int c = c0 + lane / G;
    float m = -__builtin_inff();
    if (c < inner)
      for (int k = g; k < nk; k += G) m = fmaxf(m, part[c + k * inner].x);
    m = seg_allreduce<G>(m, OpMax{});
    float s = 0.0f;
    if (c < inner)
      for (int k = g; k < nk; k += G) s += fold_weighted(part[c + k * inner].x, part[c + k * inner].y, m);
    s = seg_allreduce<G>(s, OpSum{});
    if (g == 0 && c < inner) res[c] = make_float2(m, s);
  }
}

template <int NT = kBlkThreads>
__device__ __forceinline__ void blk_merge_cols(const float2 *part, float2 *res, int inner, int nk,
                                               int t) {
  const int q = nk / 4;
  if (q >= 64) blk_merge_g<64, NT>(part, res, inner, nk, t);
  else if (q >= 32) blk_merge_g<32, NT>(part, res, inner, nk, t);
  else if (q >= 16) blk_merge_g<16, NT>(part, res, inner, nk, t);
  else if (q >= 8) blk_merge_g<8, NT>(part, res, inner, nk, t);
  else if (q >= 4) blk_merge_g<4, NT>(part, res, inner, nk, t);
  else if (q >= 2) blk_merge_g<2, NT>(part, res, inner, nk, t);
  else blk_merge_g<1, NT>(part, res, inner, nk, t);
}

// Workgroup (o, c) of an (outer, chunks) grid, chunk fastest: planes
// [c rc, min(R, (c + 1) rc)) of block o (rc a multiple of 4, so every chunk
// starts on a period).  Lane t < act folds floats 4 t + k w .. + 3 of the
// chunk into the running pairs of columns (4 (t mod lp) + e) mod inner.
//   kBlkPartial(Keep): pairs[(o inner + col) chunks + c] = (m, s)
//   kBlkLse:           out[o yso + col] = m + log s
//   kBlkLsm:           y[o yso + k] = (x - m) - log s, reading the block again
template <int MODE>
__global__ __launch_bounds__(kBlkThreads) void axis_block_kernel(const float *__restrict__ x,
                                                                 float *__restrict__ out,
                                                                 AxisDims d, int64_t chunks,
                                                                 int64_t rc,
                                                                 float2 *__restrict__ pairs) {
  __shared__ float2 part[4 * kBlkThreads];
  __shared__ float2 res[kBlkMaxInner];
  float2 *tab = res;  // log_softmax: (M, log S) in place of (M, S)
  constexpr bool kNt = MODE == kBlkPartial || MODE == kBlkLse;  // else x is read again
  const int t = threadIdx.x;
  const int64_t b = blockIdx.x;
  const int64_t c = b % chunks;
  const int64_t o = b / chunks;
  const int inner = (int)d.inner;
  const BlkSweep sw = blk_sweep(inner);
  const int64_t r0 = c * rc;
  const int64_t r1 = (d.R - r0 < rc) ? d.R : r0 + rc;
  const int64_t f0 = r0 * inner, f1 = r1 * inner;
  const float *xb = x + o * d.xso;
  const float ninf = -__builtin_inff();
  float m[4], s[4], comp[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    m[e] = ninf;
    s[e] = 0.0f;
    comp[e] = 0.0f;
  }
  if (t < sw.act) {
    for (int64_t j = f0 + 4 * t; j < f1; j += (int64_t)sw.w * kBlkU) {
      float q[kBlkU][4];
#pragma unroll
      for (int u = 0; u < kBlkU; ++u) blk_load4<kNt>(xb, j + (int64_t)u * sw.w, f1, ninf, q[u]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float v[kBlkU];
#pragma unroll
        for (int u = 0; u < kBlkU; ++u) v[u] = q[u][e];
        fold_block_c<kBlkU>(v, m[e], s[e], comp[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) part[4 * t + e] = make_float2(m[e], fold_total(s[e], comp[e]));
  }
  __syncthreads();
  blk_merge_cols<kBlkThreads>(part, res, inner, sw.w / inner, t);
  __syncthreads();
  if (t < inner) {
    const float M = res[t].x, S = res[t].y;
    if constexpr (MODE == kBlkPartial || MODE == kBlkPartialKeep) {
      pairs[(o * inner + t) * chunks + c] = make_float2(M, S);
    } else if constexpr (MODE == kBlkLse) {
      out[o * d.yso + t] = M + logf(S);
    } else {
      tab[t] = make_float2(M, logf(S));
    }
  }
  if constexpr (MODE == kBlkLsm) {
    __syncthreads();
    if (t < sw.act) {
      float fm[4], fl[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float2 v = tab[(4 * (t % sw.lp) + e) % inner];
        fm[e] = v.x;
        fl[e] = v.y;
      }
      blk_write(xb, out + o * d.yso, f0 + 4 * t, f1, sw.w, fm, fl);
    }
  }
}

// logsumexp of a block's columns from their chunk pairs: one thread per
// (o, col), chunks merged in order.
__global__ __launch_bounds__(256) void axis_block_merge_kernel(const float2 *__restrict__ pairs,
                                                               float *__restrict__ out,
                                                               AxisDims d, int64_t chunks) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= d.outer * d.inner) return;
  const int64_t o = i / d.inner;
  const int64_t col = i - o * d.inner;
  const float2 f = blk_merge_pairs(pairs + i * chunks, chunks);
  out[o * d.yso + col] = f.x + logf(f.y);
}

// The same merge for long chunk lists: a wave per (o, col), lane l loading
// chunks l, l + 64, ..., l + 15 * 64 at once (one round of loads for up to
// 1024 chunks) and folding them into its running pair against one shared
// maximum, then the lanes' pairs reduced across the wave (the same order on
// every call).  LSM: fin[o inner + col] = (M, log S) for the apply launch;
// else the logsumexp into out.
constexpr int kBlkMergeQ = 16;
template <bool LSM>
__global__ __launch_bounds__(256) void axis_block_merge_wide_kernel(
    const float2 *__restrict__ pairs, float *__restrict__ out, float2 *__restrict__ fin,
    AxisDims d, int64_t chunks) {
  const int64_t i = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;  // (o, col)
  const int lane = threadIdx.x % kWave;
  if (i >= d.outer * d.inner) return;  // whole waves
  const float2 *p = pairs + i * chunks;
  float m = -__builtin_inff(), s = 0.0f;
  for (int64_t k0 = lane; k0 < chunks; k0 += kBlkMergeQ * kWave) {
    float2 q[kBlkMergeQ];
#pragma unroll
    for (int u = 0; u < kBlkMergeQ; ++u)
      q[u] = (k0 + u * kWave < chunks) ? p[k0 + u * kWave] : make_float2(-__builtin_inff(), 0.0f);
    float mn = m;
#pragma unroll
    for (int u = 0; u < kBlkMergeQ; ++u) mn = fmaxf(mn, q[u].x);
    float t = fold_weighted(m, s, mn);
#pragma unroll
    for (int u = 0; u < kBlkMergeQ; ++u) t += fold_weighted(q[u].x, q[u].y, mn);
    s = t;
    m = mn;
  }
  const float M = wave_allreduce(m, OpMax{});
  const float S = wave_allreduce(fold_weighted(m, s, M), OpSum{});
  if (lane == 0) {
    if constexpr (LSM) {
      fin[i] = make_float2(M, logf(S));
    } else {
      const int64_t o = i / d.inner;
      out[o * d.yso + (i - o * d.inner)] = M + logf(S);
    }
  }
}

// log_softmax over chunk c of block o (the pair launch's grid): the block's
// chunk pairs are merged first (the order of the merge kernel), or read
// merged from fin, then written.
__global__ __launch_bounds__(kBlkThreads) void axis_block_apply_kernel(
    const float *__restrict__ x, float *__restrict__ y, AxisDims d, int64_t chunks, int64_t rc,
    const float2 *__restrict__ pairs, const float2 *__restrict__ fin) {
  __shared__ float2 tab[kBlkMaxInner];
  const int t = threadIdx.x;
  const int64_t b = blockIdx.x;
  const int64_t c = b % chunks;
  const int64_t o = b / chunks;
  const int inner = (int)d.inner;
  const BlkSweep sw = blk_sweep(inner);
  if (t < inner) {
    if (fin != nullptr) {  // merged by axis_block_merge_wide_kernel
      tab[t] = fin[o * inner + t];
    } else {
      const float2 f = blk_merge_pairs(pairs + (o * inner + t) * chunks, chunks);
      tab[t] = make_float2(f.x, logf(f.y));
    }
  }
  __syncthreads();
  if (t >= sw.act) return;
  float fm[4], fl[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float2 v = tab[(4 * (t % sw.lp) + e) % inner];
    fm[e] = v.x;
    fl[e] = v.y;
  }
  const int64_t r0 = c * rc;
  const int64_t r1 = (d.R - r0 < rc) ? d.R : r0 + rc;
  blk_write(x + o * d.xso, y + o * d.yso, r0 * inner + 4 * t, r1 * inner, sw.w, fm, fl);
}

// ------------------------------------------------------- register-resident
// Sweeps per workgroup of the register-resident log_softmax: 16 x 4 floats
// per lane.
#ifndef LSE_BLK_RES_K
#define LSE_BLK_RES_K 16
#endif
constexpr int kBlkResK = LSE_BLK_RES_K;
// Lanes per workgroup of the register-resident log_softmax: 256 for blocks of
// up to 16 of their sweeps, 512 for larger ones and for split blocks.
constexpr int kBlkResWide = 2 * kBlkThreads;
#ifndef LSE_BLK_RES_WPE
#define LSE_BLK_RES_WPE 4          // waves per SIMD the split kernel's registers must allow (0: any)
#endif

// Fold of one chunk of K sweeps into per-lane pairs for its 4 columns, from
// nothing: exact max over the K values of each column slot, then their shifted
// sum in sweep order.  The owner folds its registers (blk_fold_fresh); a
// helper re-reads the chunk from x, one sweep at a time (blk_fold_fresh_mem):
// the same arithmetic in the same order, so both produce the same bits.
template <int K>
__device__ __forceinline__ void blk_fold_fresh(const float (&q)[K][4], float (&m)[4],
                                               float (&s)[4]) {
  float c[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float bm = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < K; ++k) bm = fmaxf(bm, q[k][e]);
    m[e] = bm;
    c[e] = safe_shift(bm);
    s[e] = 0.0f;
  }
#pragma unroll
  for (int k = 0; k < K; ++k) {
#pragma unroll
    for (int e = 0; e < 4; ++e) s[e] += exp_base2(q[k][e] - c[e]);
  }
}

template <int K>
__device__ __forceinline__ void blk_fold_fresh_mem(const float *xb, int64_t j, int64_t f, int w,
                                                   bool act, float (&m)[4], float (&s)[4]) {
  const float ninf = -__builtin_inff();
  float bm[4] = {ninf, ninf, ninf, ninf};
  if (act) {
#pragma unroll 1
    for (int k = 0; k < K; ++k) {
      float v[4];
      blk_load4<false>(xb, j + (int64_t)k * w, f, ninf, v);
#pragma unroll
      for (int e = 0; e < 4; ++e) bm[e] = fmaxf(bm[e], v[e]);
    }
  }
  float c[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    m[e] = bm[e];
    c[e] = safe_shift(bm[e]);
    s[e] = 0.0f;
  }
#pragma unroll 1
  for (int k = 0; k < K; ++k) {
    float v[4] = {ninf, ninf, ninf, ninf};
    if (act) blk_load4<false>(xb, j + (int64_t)k * w, f, ninf, v);
#pragma unroll
    for (int e = 0; e < 4; ++e) s[e] += exp_base2(v[e] - c[e]);
  }
}

// The chunk's (M, S) per column into res[0..inner) (through part and the
// column merge; trailing barrier included).
template <int NT>
__device__ __forceinline__ void blk_chunk_columns(const float (&m)[4], const float (&s)[4],
                                                  float2 *part, float2 *res, int inner,
                                                  const BlkSweep &sw, int t) {
  if (t < sw.act) {
#pragma unroll
    for (int e = 0; e < 4; ++e) part[4 * t + e] = make_float2(m[e], s[e]);
  }
  __syncthreads();
  blk_merge_cols<NT>(part, res, inner, sw.w / inner, t);
  __syncthreads();
}

// Wave 0 polls until all k slots are non-zero (true), or the poll limit or
// the time threshold (50 us of the 100 MHz real-time counter; a real wait is
// a few microseconds) runs out (false).
__device__ __forceinline__ bool blk_wait_slots(const uint64_t *slots, int64_t k, uint32_t limit) {
  const int lane = threadIdx.x % kWave;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (uint32_t it = 0;; ++it) {
    bool missing = false;
    for (int64_t j = lane; j < k; j += kWave) missing |= (load_pair_agent(slots + j) == 0);
    if (__builtin_amdgcn_ballot_w64(missing) == 0) return true;
    if (it >= limit || __builtin_amdgcn_s_memrealtime() - t0 > 5000ull) return false;
    __builtin_amdgcn_s_sleep(LSE_BLK_SLEEP);
  }
}

// log_softmax with the values in registers.  Workgroup (o, c) of an
// (outer, chunks) grid of NT-lane workgroups, chunk fastest, holds floats
// f0 + 4 t + k w (k < K) of chunk c (rc planes, a whole number of periods,
// rc inner <= K w).
//   !SPLIT (chunks = 1): the block's (M, S) per column come from this
//     workgroup alone.
//   SPLIT: slots[(o chunks + c) inner + col] receive the chunk's packed
//     (m, s) (zeroed beforehand); the workgroup waits for the block's other
//     chunks (or computes the missing ones itself), merges the block's pairs
//     per column in chunk order, and writes.  spin_limit 0 is a test mode in
//     which owners publish nothing, so every pair comes from a helper.
template <int K, bool SPLIT, int NT>
__global__ __launch_bounds__(NT)
#if LSE_BLK_RES_WPE
__attribute__((amdgpu_waves_per_eu(LSE_BLK_RES_WPE)))
#endif
void axis_block_resident_kernel(
    const float *__restrict__ x, float *__restrict__ y, AxisDims d, int64_t chunks, int64_t rc,
    uint64_t *__restrict__ slots, uint32_t spin_limit) {
  __shared__ float2 part[4 * NT];
  __shared__ float2 res[kBlkMaxInner];
  __shared__ int s_state;
  const int t = threadIdx.x;
  const int64_t b = blockIdx.x;
  const int64_t c = b % chunks;
  const int64_t o = b / chunks;
  const int inner = (int)d.inner;
  const BlkSweep sw = blk_sweep(inner, NT);
  const int64_t r0 = c * rc;
  const int64_t r1 = (d.R - r0 < rc) ? d.R : r0 + rc;
  const int64_t f0 = r0 * inner, f1 = r1 * inner;
  const float *xb = x + o * d.xso;
  const float ninf = -__builtin_inff();
  const bool act = t < sw.act;
  float q[K][4];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    if (act) {
      blk_load4<true>(xb, f0 + 4 * t + (int64_t)k * sw.w, f1, ninf, q[k]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) q[k][e] = ninf;
    }
  }
  float m[4], s[4];
  blk_fold_fresh<K>(q, m, s);
  blk_chunk_columns<NT>(m, s, part, res, inner, sw, t);
  if constexpr (SPLIT) {
    uint64_t *bs = slots + o * chunks * inner;
    if (t < inner && spin_limit != 0)
      publish_pair_once(bs + c * inner + t, pack_pair(res[t].x, res[t].y));
    for (;;) {
      if (t < kWave) {
        const bool all = blk_wait_slots(bs, chunks * inner, spin_limit);
        if (t == 0) s_state = all ? 1 : 0;
      }
      __syncthreads();
      if (s_state == 1) break;  // uniform: every thread read the same LDS word
      // Help: recompute each sibling chunk with a missing slot from x.
      for (int64_t j = 0; j < chunks; ++j) {
        __syncthreads();
        if (t == 0) s_state = 0;
        __syncthreads();
        if (t < inner && load_pair_agent(bs + j * inner + t) == 0) s_state = 2;
        __syncthreads();
        if (s_state != 2) continue;  // uniform, as above
        const int64_t hr0 = j * rc;
        const int64_t hf1 = ((d.R - hr0 < rc) ? d.R : hr0 + rc) * inner;
        const int64_t hj = hr0 * inner + 4 * t;
        float hm[4], hs[4];
        blk_fold_fresh_mem<K>(xb, hj, hf1, sw.w, act, hm, hs);
        blk_chunk_columns<NT>(hm, hs, part, res, inner, sw, t);
        if (t < inner) publish_pair_once(bs + j * inner + t, pack_pair(res[t].x, res[t].y));
      }
      __syncthreads();
    }
    if (t < inner) {
      float M = -__builtin_inff();
      for (int64_t j = 0; j < chunks; ++j) M = fmaxf(M, pair_m(load_pair_agent(bs + j * inner + t)));
      float S = 0.0f;
      for (int64_t j = 0; j < chunks; ++j) {
        const uint64_t p = load_pair_agent(bs + j * inner + t);
        S += fold_weighted(pair_m(p), pair_s(p), M);
      }
      res[t] = make_float2(M, logf(S));
    }
  } else if (t < inner) {
    res[t] = make_float2(res[t].x, logf(res[t].y));
  }
  __syncthreads();
  if (!act) return;
  float fm[4], fl[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float2 v = res[(4 * (t % sw.lp) + e) % inner];
    fm[e] = v.x;
    fl[e] = v.y;
  }
  float *yb = y + o * d.yso;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int64_t jj = f0 + 4 * t + (int64_t)k * sw.w;
    if (jj < f1) {
      float r[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = (q[k][e] - fm[e]) - fl[e];
      if (jj + 4 <= f1) {
        __builtin_nontemporal_store(v4b4{r[0], r[1], r[2], r[3]}, reinterpret_cast<v4b4 *>(yb + jj));
      } else {
#pragma unroll
        for (int e = 0; e < 3; ++e)
          if (jj + e < f1) __builtin_nontemporal_store(r[e], yb + jj + e);
      }
    }
  }
}

__global__ __launch_bounds__(256) void blk_clear_kernel(uint64_t *__restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0;
}

struct BlkPlan {
  int64_t chunks, rc;
  int mode, k, nt;
};

enum BlkLaunch { kLaunchFold = 0, kLaunchResident = 1, kLaunchResidentSplit = 2 };

// Workgroups of one launch: the dispatch's work-item count must fit 32 bits.
constexpr int64_t kMaxBlkGroups = 0xffffffffLL / kBlkThreads;

// The block plan of a call, or false when the call keeps the other axis
// kernels.  with_ws: the caller can supply blocks_workspace_bytes().
bool blk_plan(const AxisDims &d, bool lsm, bool with_ws, BlkPlan &p) {
  if (LSE_BLK_GATE == 0) return false;
  if (d.outer < 1 || d.R < 1 || d.inner < 2 || d.inner > kBlkMaxInner) return false;
  if (d.xsr != d.inner || (lsm && d.ysr != d.inner)) return false;
  if (d.R * d.inner > (int64_t(1) << 40)) return false;
  const BlkSweep sw = blk_sweep((int)d.inner);
  const int64_t n = d.R * d.inner;
  p.k = 0;
  if (lsm && LSE_BLK_RESIDENT) {
    // one workgroup per block, held in registers: 256 lanes with 4, 8 or 16
    // sweeps, else 512 lanes with 16 (wider workgroups leave most lanes of a
    // small block idle: (40000, 200, 13) 5900 -> 3700 GB/s)
    const BlkSweep rs = blk_sweep((int)d.inner, kBlkThreads);
    const BlkSweep rw = blk_sweep((int)d.inner, kBlkResWide);
    const int64_t cap[4] = {4LL * rs.w, 8LL * rs.w, 16LL * rs.w, (int64_t)kBlkResK * rw.w};
    const int ks[4] = {4, 8, 16, kBlkResK};
    for (int i = 0; i < 4; ++i) {
      const int nt = i < 3 ? kBlkThreads : kBlkResWide;
      if (n <= cap[i] && d.outer <= 0xffffffffLL / nt) {
        p.chunks = 1;
        p.rc = d.R;
        p.k = ks[i];
        p.nt = nt;
        p.mode = kLaunchResident;
        return true;
      }
    }
    // chunks of at most kBlkResK sweeps of 512 lanes, of near-equal whole
    // periods, that wait for each other; on grids of several workgroups per
    // slot (with about one, loading and waiting do not overlap across
    // workgroups), or of blocks of few chunks (same box, GB/s, fold path ->
    // resident: (256, 2048, 49) 3430 -> 4240, (64, 8000, 25) 2820 -> 3610,
    // (32, 30000, 5) 1560 -> 1920; 640 workgroups of 16 chunks -9 %)
    if (with_ws) {
      const int64_t per = (int64_t)rw.lp * 4 / d.inner;  // planes per period
      const int64_t rc_max = (int64_t)kBlkResK * rw.w / d.inner;
      int64_t chunks = (d.R + rc_max - 1) / rc_max;
      int64_t rc = (d.R + chunks - 1) / chunks;
      rc = (rc + per - 1) / per * per;
      chunks = (d.R + rc - 1) / rc;
      // grids of fewer workgroups: blocks of few chunks, most CUs busy, and
      // not just past one round of resident workgroups (whose last blocks
      // would then run alone)
      const int64_t g = d.outer * chunks;
      const bool few = chunks <= LSE_BLK_RES_FEW_CHUNKS &&
                       g >= (chunks <= 8 ? 160 : LSE_BLK_RES_FEW_GROUPS) &&
                       (g <= LSE_BLK_RES_SLOTS || g >= 2 * LSE_BLK_RES_SLOTS);
      if (chunks <= LSE_BLK_RES_MAX_CHUNKS && (g >= LSE_BLK_RES_MIN_GROUPS || few) &&
          d.outer * chunks <= 0xffffffffLL / kBlkResWide) {
        p.chunks = chunks;
        p.rc = rc;
        p.k = kBlkResK;
        p.nt = kBlkResWide;
        p.mode = kLaunchResidentSplit;
        return true;
      }
    }
  }
  // chunks of whole periods (4 planes) and at least LSE_BLK_MIN_TRIPS trips
  const int64_t trip = (int64_t)sw.w * kBlkU;
  int64_t min_planes = (LSE_BLK_MIN_TRIPS * trip + d.inner - 1) / d.inner;
  min_planes = (min_planes + 3) / 4 * 4;
  p.chunks = 1;
  if (with_ws) {
    int64_t k = (LSE_BLK_TARGET_GROUPS + d.outer - 1) / d.outer;
    const int64_t kmax = d.R / min_planes;
    if (k > kmax) k = kmax;
    if (k > LSE_BLK_MAX_CHUNKS) k = LSE_BLK_MAX_CHUNKS;
    p.chunks = k < 1 ? 1 : k;
  } else if (d.outer < LSE_BLK_NOWS_MIN_OUTER) {
    return false;
  }
  p.rc = ((d.R + p.chunks - 1) / p.chunks + 3) / 4 * 4;
  p.chunks = (d.R + p.rc - 1) / p.rc;
  if (d.outer * p.chunks > kMaxBlkGroups) return false;
  p.mode = kLaunchFold;
  return true;
}

// Which calls take the blocks (measured against the axis kernels, the column
// split and the plane split on the same shapes): blocks of at least
// LSE_BLK_MIN_BLOCK floats (smaller ones leave most of a sweep's lanes idle
// and make workgroups too short), any number of them; then inner
// runs up to LSE_BLK_GATE_INNER, with a workspace only off the 16-byte grid
// (on it the axis kernels and the column split were about as fast), except
// logsumexp over blocks of LSE_BLK_BIG_BLOCK floats or more, which the
// blocks read faster whatever the run (wider runs the axis kernels read well
// otherwise, and their log_softmax reads x once), and log_softmax over blocks
// of LSE_BLK_LSM_BIG floats or more (few long blocks, where both read x twice:
// 2-12 % faster there, 5-23 % slower on blocks of 1-2 M floats).
#ifndef LSE_BLK_LSM_BIG
#define LSE_BLK_LSM_BIG 4194304
#endif
bool blk_wanted(const AxisDims &d, bool lsm, bool with_ws, const float *x, const float *out) {
  if (LSE_BLK_GATE == 2) return true;
  const int64_t n = d.R * d.inner;
  if (n < LSE_BLK_MIN_BLOCK) return false;
  const bool big_lse = !lsm && n >= LSE_BLK_BIG_BLOCK;
  if (d.inner > LSE_BLK_GATE_INNER) return big_lse;
  if (LSE_BLK_LSM_BIG && lsm && n >= LSE_BLK_LSM_BIG) return true;
  const uintptr_t a = (uintptr_t)x | (lsm ? (uintptr_t)out : 0);
  const int64_t st = d.inner | d.xso | (lsm ? d.yso : 0);
  const bool grid16 = st % 4 == 0 && a % 16 == 0;
  return !grid16 || !with_ws || big_lse;
}

size_t blk_ws_bytes(const AxisDims &d, const BlkPlan &p, bool lsm) {
  // fold: a float2 pair per column and chunk (and, merged by a wave per
  // column, a float2 (M, log S) per column for log_softmax); resident split:
  // a packed pair per column and chunk
  if (p.chunks <= 1) return 0;
  const size_t cols = (size_t)(d.outer * d.inner);
  const bool fin = lsm && p.mode == kLaunchFold && p.chunks > LSE_BLK_SERIAL_CHUNKS;
  return cols * (size_t)p.chunks * 8 + (fin ? cols * 8 : 0);
}

}  // namespace

size_t blocks_workspace_bytes(const AxisDims &d, bool lsm) {
  BlkPlan p;
  return blk_plan(d, lsm, true, p) ? blk_ws_bytes(d, p, lsm) : 0;
}

bool launch_blocks(const float *x, float *out, const AxisDims &d, bool lsm, bool with_ws,
                   void *ws, hipStream_t stream, hipError_t &e) {
  BlkPlan p;
  if (!blk_plan(d, lsm, with_ws, p) || !blk_wanted(d, lsm, with_ws, x, out)) return false;
  if (p.chunks > 1 && ws == nullptr) return false;
  const dim3 grid((uint32_t)(d.outer * p.chunks));
  const dim3 block(kBlkThreads);
  if (p.mode == kLaunchResident) {
    const dim3 rblock((uint32_t)p.nt);
    if (p.nt == kBlkResWide)
      hipLaunchKernelGGL((axis_block_resident_kernel<kBlkResK, false, kBlkResWide>), grid, rblock,
                         0, stream, x, out, d, p.chunks, p.rc, nullptr, 0u);
    else if (p.k == 4)
      hipLaunchKernelGGL((axis_block_resident_kernel<4, false, kBlkThreads>), grid, rblock, 0,
                         stream, x, out, d, p.chunks, p.rc, nullptr, 0u);
    else if (p.k == 8)
      hipLaunchKernelGGL((axis_block_resident_kernel<8, false, kBlkThreads>), grid, rblock, 0,
                         stream, x, out, d, p.chunks, p.rc, nullptr, 0u);
    else
      hipLaunchKernelGGL((axis_block_resident_kernel<16, false, kBlkThreads>), grid, rblock, 0,
                         stream, x, out, d, p.chunks, p.rc, nullptr, 0u);
    e = hipGetLastError();
    return true;
  }
  if (p.mode == kLaunchResidentSplit) {
    auto *slots = reinterpret_cast<uint64_t *>(ws);
    const int64_t words = d.outer * p.chunks * d.inner;
    const int64_t cb = (words + 255) / 256;
    hipLaunchKernelGGL(blk_clear_kernel, dim3((uint32_t)(cb < 4096 ? cb : 4096)), dim3(256), 0,
                       stream, slots, words);
    e = hipGetLastError();
    if (e != hipSuccess) return true;
    hipLaunchKernelGGL((axis_block_resident_kernel<kBlkResK, true, kBlkResWide>), grid,
                       dim3(kBlkResWide), 0, stream, x, out, d, p.chunks, p.rc, slots,
                       chain_spin_limit());
    e = hipGetLastError();
    return true;
  }
  auto *pairs = reinterpret_cast<float2 *>(ws);
  if (p.chunks > 1) {
    if (lsm)
      hipLaunchKernelGGL((axis_block_kernel<kBlkPartialKeep>), grid, block, 0, stream, x, out, d,
                         p.chunks, p.rc, pairs);
    else
      hipLaunchKernelGGL((axis_block_kernel<kBlkPartial>), grid, block, 0, stream, x, out, d,
                         p.chunks, p.rc, pairs);
  } else if (lsm) {
    hipLaunchKernelGGL((axis_block_kernel<kBlkLsm>), grid, block, 0, stream, x, out, d, p.chunks,
                       p.rc, pairs);
  } else {
    hipLaunchKernelGGL((axis_block_kernel<kBlkLse>), grid, block, 0, stream, x, out, d, p.chunks,
                       p.rc, pairs);
  }
  e = hipGetLastError();
  if (e != hipSuccess || p.chunks == 1) return true;
  const int64_t cols = d.outer * d.inner;
  float2 *fin = nullptr;
  if (p.chunks > LSE_BLK_SERIAL_CHUNKS) {  // a wave per column
    const dim3 mgrid((uint32_t)((cols + 3) / 4));
    if (lsm) {
      fin = pairs + cols * p.chunks;
      hipLaunchKernelGGL((axis_block_merge_wide_kernel<true>), mgrid, dim3(256), 0, stream, pairs,
                         out, fin, d, p.chunks);
    } else {
      hipLaunchKernelGGL((axis_block_merge_wide_kernel<false>), mgrid, dim3(256), 0, stream, pairs,
                         out, fin, d, p.chunks);
    }
    e = hipGetLastError();
    if (e != hipSuccess || !lsm) return true;
  } else if (!lsm) {
    hipLaunchKernelGGL(axis_block_merge_kernel, dim3((uint32_t)((cols + 255) / 256)), dim3(256), 0,
                       stream, pairs, out, d, p.chunks);
    e = hipGetLastError();
    return true;
  }
  hipLaunchKernelGGL(axis_block_apply_kernel, grid, block, 0, stream, x, out, d, p.chunks, p.rc,
                     pairs, fin);
  e = hipGetLastError();
  return true;
}

}  // namespace lse
