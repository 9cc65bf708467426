// conv_chain.hip — conv2d 3x3 -> GroupNorm -> tanh -> hardswish -> residual
// add -> logsumexp over channels, fused around the conv on fp32 MFMA (as
// Winograd F(2x2, 3x3), or a direct implicit GEMM when LSE_CHAIN_WINO=0).
//
// POPCORNBENCH Kimi-K2.6 l2_p92: the model's forward is x_conv = conv(x);
// GroupNorm (mean and population variance per (sample, group) over the
// group's channels and all pixels); tanh; hardswish x * relu6(x + 3) / 6;
// x_conv + that; logsumexp over dim 1 with keepdim.  That page keeps the conv
// in the vendor library and runs a stats kernel plus a one-block-per-pixel
// epilogue over the materialised conv output.  Here the conv output is never
// written to memory and the conv runs once:
//
//   each workgroup of 8 waves takes a pair of 2 x 128 pixel tiles of one
//   sample (pair = workgroup index, in sample order); waves 0-3
//   stage and convolve one tile, waves 4-7 the other, on MFMA into registers
//   (64 accumulators per lane, so four waves fit on a SIMD); the pair
//   publishes each tile's per-group (mean, M2), waits until every tile of
//   its sample has published, merges the sample's statistics in fp64, and
//   runs normalise, tanh, hardswish, residual and the 64-channel logsumexp
//   on the accumulators it still holds, writing one float per pixel.
//
// The wait normally ends within microseconds: the hardware starts workgroups
// in index order (dealt round robin to the XCDs), and every workgroup
// publishes before it waits, so the tiles of a sample that has a waiting
// workgroup are all held by running workgroups soon after, which needs only
// as many co-resident workgroups as a sample has tile pairs (32 for 126 x 126;
// hundreds fit).  Progress never depends on that order, though.  Each workgroup
// counts its arrival (after publishing) on a per-sample word; one whose wait
// runs out (kChainWaitTicks, or the test hook's poll limit) counts itself
// deferred on the same word: if every pair of its sample has arrived by then
// the statistics are complete and it carries on, otherwise it records its
// pair in the sample's queue and exits, which frees its slot for the pairs
// still to come.  The sample's last arrival sees the deferrals made before
// it and finishes those pairs itself after its own (conv, merge, epilogue;
// nothing left to wait for).  The two counts share one 64-bit word, so every
// deferral is either seen by the last arrival or sees it.  A sample with more
// tile pairs than half of what the device holds at once takes two launches
// instead: one publishes the statistics, the next recomputes the conv and
// applies them (the conv runs twice, nothing waits; the results are
// identical).
//
// Direct form (conv_tile), GEMM shape per sample: D[c][p] = sum_k W[c][k] *
// patch[k][p] with c the 64 output channels (M), p the pixels (N) and
// k = (ci, kh, kw), 72 values (K).  The Winograd form (conv_tile_wino) has
// the same operand roles with p a 2 x 2 output block and K the 8 input
// channels, once per Winograd position.
// v_mfma_f32_16x16x4_f32 operands, lane l = 0..63, i = l % 16, q = l / 16:
//   A (16x4):  lane l holds A[i][q]          -> W[16t + i][4s + q]
//   B (4x16):  lane l holds B[q][i]          -> patch[4s + q][pixel i]
//   D (16x16): lane l holds D[4q + r][i], r = 0..3
// so each lane's accumulator of M-tile t holds channels 16t + 4q + r of one
// pixel: a whole quad of 4 consecutive channels.  With groups of 4k channels,
// a group's statistics reduce inside 16-lane DPP rows, and a pixel's 64
// channels are 16 values in-lane plus the 4 lanes i, i+16, i+32, i+48 (two
// permlane swaps).
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "lse_device.hpp"
#include "lse_internal.hpp"

namespace lse {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kCin = 8, kCout = 64, kKs = 3, kKdim = kCin * kKs * kKs;  // 72
constexpr int kKSteps = kKdim / 4;                                       // 18
constexpr int kMT = kCout / 16;                                          // 4 M-tiles
constexpr int kTileH = 2, kTileW = 128;                                  // output pixels
constexpr int kLdsH = kTileH + kKs - 1;                                  // 4 input rows
constexpr int kLdsW = kTileW + 4;     // 130 input columns needed, padded to 33 float4
constexpr int kF4PerRow = kLdsW / 4;                                     // 33
constexpr int kStageF4 = kCin * kLdsH * kF4PerRow;                       // 1056
constexpr int kNB = 4;   // 16-pixel blocks per wave: 4 waves x 4 x 16 = 2 x 128
constexpr int kThreads = 256;  // one tile's team of 4 waves
#ifndef LSE_CHAIN_HELD
#define LSE_CHAIN_HELD 1024   // statistics words held in registers per workgroup while polling
#endif
#ifndef LSE_CHAIN_TEAMS
#define LSE_CHAIN_TEAMS 2   // tiles (teams of 4 waves) per workgroup: 1 or 2
#endif
constexpr int kTeams = LSE_CHAIN_TEAMS;
static_assert(kTeams == 1 || kTeams == 2, "one or two tiles per workgroup");
// W in LDS, one 72-value row per output channel padded to 76 floats: the A
// fragment read of a K-step (lane l -> row 16t + l % 16, column 9 (l / 16) plus
// a per-step constant, see conv_tile) then hits 64 distinct banks
// (12 (l % 16) + 9 (l / 16) is distinct mod 64 for the 64 lanes).
constexpr int kWStride = kKdim + 4;                                      // 76
constexpr int kWF4 = kCout * kKdim / 4;                                  // 1152 float4

#ifndef LSE_CHAIN_WINO
#define LSE_CHAIN_WINO 1   // the 3x3 contraction as Winograd F(2x2, 3x3) on MFMA
#endif
constexpr bool kWino = LSE_CHAIN_WINO != 0;
#ifndef LSE_CHAIN_WINO_SB
#define LSE_CHAIN_WINO_SB 2   // scheduling barriers in the Winograd loop: 1 per row of M, 2 also per M-tile
#endif
static_assert(!kWino || kTeams == 2, "the Winograd weight staging uses one thread per (o, ci)");
// Transformed weights U in LDS in MFMA fragment order [p][ks][t][lane]: p the
// 16 Winograd positions, ks the half of the 8 input channels, t the M-tile,
// lane 16 q + i holding U[p][16 t + i][4 ks + q].
constexpr int kWinoU = 16 * 2 * kMT * kWave;                             // 8192 floats
constexpr int kWLds = kWino ? kWinoU : kCout * kWStride;

struct ChainWsHeader {
  uint32_t reserved;   // 0
  uint32_t deferred;   // pairs finished by their sample's last arrival
  uint32_t pad[62];
};

struct ChainArgs {
  const float *x, *w, *b, *gamma, *beta;
  int32_t N, H, W, Ho, Wo, G, log2G, tiles_w, tiles;
  float eps;
  uint32_t spin_limit;
  uint32_t block_base;   // pair index (over all samples) of this launch's first workgroup
  uint32_t xcd_order;    // 1: consecutive pairs on one XCD (xcd_pair)
  uint32_t stage_first;  // pair index of the first pair whose conv tiles sit in `stage`
  float *stage;          // kStats with staging, kApplyStaged: conv tiles of this batch
  float *out;
  float *mean;           // (N, G), written by tile 0 of each sample
  float *rstd;           // (N, G)
  ChainWsHeader *hdr;
  uint64_t *stats;       // (N, tiles, G) packed (mean, -M2); 0 = not yet written
  uint64_t *arrivals;    // (N): low 32 bits pairs arrived, high 32 bits pairs deferred
  uint32_t *queue;       // (N, pairs per sample): deferred pair + 1, in deferral order
};

// Row-of-16 all-reduce (lanes sharing l / 16) on DPP only.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0x141>(v);
  v += dpp_mov<0x140>(v);
  return v;
}

// Combine across the 4 lanes i, i+16, i+32, i+48 (the same pixel).
template <class Op>
__device__ __forceinline__ float across_quads(float v, Op op) {
  auto p = __builtin_amdgcn_permlane16_swap(fbits(v), fbits(v), false, false);
  v = op(bitsf(p[0]), bitsf(p[1]));
  auto q = __builtin_amdgcn_permlane32_swap(fbits(v), fbits(v), false, false);
  return op(bitsf(q[0]), bitsf(q[1]));
}

// hardswish(tanh(z)), taking y = 2 log2(e) z (the scale is folded into the
// normalisation's multiply-add).  tanh(z) = 1 - 2 r with r = 1 / (2^y + 1) in
// [0, 1] (exp overflow gives r = 0, t = 1; underflow r = 1, t = -1), and
// hardswish(t) = t * min(max(t + 3, 0), 6) / 6 = t (t + 3) / 6 on [-1, 1],
// where the clamp never binds; in r that is (2 - 5 r + 2 r^2) / 3, two fmas.
// The absolute error is a few 1e-7, far inside the chain's tolerance.
__device__ __forceinline__ float hardswish_of_tanh_scaled(float y) {
  const float r = __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(y) + 1.0f);
  return fmaf(r, fmaf(r, 2.0f / 3.0f, -5.0f / 3.0f), 2.0f / 3.0f);
}

// log2(e) x hardswish(tanh(z)) from the same y = 2 log2(e) z: the polynomial
// in r with its coefficients scaled by log2(e).
__device__ __forceinline__ float hardswish_of_tanh_scaled_log2e(float y) {
  const float r = __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(y) + 1.0f);
  return fmaf(r, fmaf(r, 2.0f / 3.0f * kLog2e, -5.0f / 3.0f * kLog2e), 2.0f / 3.0f * kLog2e);
}

// The x tile of sample n at (h0, w0): 8 channels x 4 rows x 132 columns.  It
// is loaded into registers with every global load of the tile in flight at
// once (128-bit loads when rows are 16-byte aligned), then stored to LDS, so
// a tile costs one memory latency and the next tile's loads can be in flight
// while the current one is on the MFMAs.  Columns past W and rows past H read
// as 0 and feed only masked pixels.
constexpr int kStageIters = (kStageF4 + kThreads - 1) / kThreads;        // 5

struct XRegs {
  float4 v[kStageIters];
};

__device__ __forceinline__ void load_x(const ChainArgs &a, int64_t n, int h0, int w0,
                                       XRegs &xr, int tid) {
  const float *xn = a.x + n * (int64_t)kCin * a.H * a.W;
  const bool vec = ((a.W & 3) == 0) && (((uintptr_t)a.x & 15) == 0);
#pragma unroll
  for (int it = 0; it < kStageIters; ++it) {
    const int f = tid + it * kThreads;
    float4 val = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (f < kStageF4) {
      const int row = f / kF4PerRow, c4 = f - row * kF4PerRow;
      const int ci = row / kLdsH, r = row - ci * kLdsH;
      const int hh = h0 + r, ww = w0 + 4 * c4;
      if (hh < a.H) {
        const float *src = xn + ((int64_t)ci * a.H + hh) * a.W + ww;
        if (vec && ww + 3 < a.W) {
          val = *reinterpret_cast<const float4 *>(src);
        } else {
          if (ww < a.W) val.x = src[0];
          if (ww + 1 < a.W) val.y = src[1];
          if (ww + 2 < a.W) val.z = src[2];
          if (ww + 3 < a.W) val.w = src[3];
        }
      }
    }
    xr.v[it] = val;
  }
}

__device__ __forceinline__ void store_x(const XRegs &xr, float *xs, int tid) {
#pragma unroll
  for (int it = 0; it < kStageIters; ++it) {
    const int f = tid + it * kThreads;
    if (f < kStageF4) *reinterpret_cast<float4 *>(xs + 4 * f) = xr.v[it];
  }
}

// W (64 x 72, contiguous) through registers into LDS rows of kWStride floats;
// the loads do not depend on the tile, so they are issued first.
template <int NT>
struct WRegs {
  static constexpr int kIters = (kWF4 + NT - 1) / NT;   // 5 for 256 threads, 3 for 512
  float4 v[kIters];
};

template <int NT>
__device__ __forceinline__ void load_w(const float *__restrict__ w, WRegs<NT> &wr) {
  const bool vec = ((uintptr_t)w & 15) == 0;
#pragma unroll
  for (int it = 0; it < WRegs<NT>::kIters; ++it) {
    const int f = threadIdx.x + it * NT;
    float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (f < kWF4) {
      if (vec) {
        v = reinterpret_cast<const float4 *>(w)[f];
      } else {
        v.x = w[4 * f]; v.y = w[4 * f + 1]; v.z = w[4 * f + 2]; v.w = w[4 * f + 3];
      }
    }
    wr.v[it] = v;
  }
}

template <int NT>
__device__ __forceinline__ void store_w(const WRegs<NT> &wr, float *wl) {
#pragma unroll
  for (int it = 0; it < WRegs<NT>::kIters; ++it) {
    const int f = threadIdx.x + it * NT;
    if (f < kWF4) {
      const int o = f / (kKdim / 4), c4 = f - o * (kKdim / 4);
      *reinterpret_cast<float4 *>(wl + o * kWStride + 4 * c4) = wr.v[it];
    }
  }
}

// The wave's conv tile: acc[blk][t] for its kNB 16-pixel blocks and 4 M-tiles,
// bias included.  Outer-product order: each K-step reads 4 A fragments (W)
// and 4 B fragments (x patches) from LDS and issues 16 MFMAs.
//
// K is visited in the order that makes every LDS offset a lane constant plus
// a compile-time constant: in K-step s, lane quarter q (the MFMA's K row)
// takes input channel ci = 4 (s / 9) + q and filter tap s % 9 = (kh, kw), i.e.
// k = 9 ci + 3 kh + kw of W's (Cout, Cin, 3, 3) layout.  A and B use the same
// order, so the sum over K is the same set of products.  The W reads stay on
// 64 distinct banks (row stride 76: 12 li + 9 q covers every bank once).
__device__ __forceinline__ void conv_tile(const ChainArgs &a, const float *xs, const float *wl,
                                          int pr, int pc0, f32x4 (&acc)[kNB][kMT]) {
  const int lane = threadIdx.x % kWave;
  const int li = lane % 16, q = lane / 16;
#pragma unroll
  for (int t = 0; t < kMT; ++t) {
    f32x4 bias;
#pragma unroll
    for (int r = 0; r < 4; ++r) bias[r] = a.b ? a.b[16 * t + 4 * q + r] : 0.0f;
#pragma unroll
    for (int blk = 0; blk < kNB; ++blk) acc[blk][t] = bias;
  }
  const float *xb = xs + q * (kLdsH * kLdsW) + pr * kLdsW + pc0 + li;
  const float *wa = wl + li * kWStride + 9 * q;
#pragma unroll
  for (int s = 0; s < kKSteps; ++s) {
    const int cib = 4 * (s / 9), kh = (s % 9) / 3, kw = s % 3;  // compile-time per step
    const int boff = (cib * kLdsH + kh) * kLdsW + kw;
    const int aoff = 9 * cib + 3 * kh + kw;
    float af[kMT], bf[kNB];
#pragma unroll
    for (int t = 0; t < kMT; ++t) af[t] = wa[16 * t * kWStride + aoff];
#pragma unroll
    for (int blk = 0; blk < kNB; ++blk) bf[blk] = xb[boff + 16 * blk];
#pragma unroll
    for (int blk = 0; blk < kNB; ++blk)
#pragma unroll
      for (int t = 0; t < kMT; ++t)
        acc[blk][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[t], bf[blk], acc[blk][t], 0, 0, 0);
  }
}

// Winograd F(2x2, 3x3) (Lavin and Gray, "Fast Algorithms for Convolutional
// Neural Networks"): a 2 x 2 block of outputs of the 3 x 3 correlation is
// Y = A^T [(G g G^T) . (B^T d B)] A over the block's 4 x 4 input window d, with
//   B^T = [1 0 -1 0; 0 1 1 0; 0 -1 1 0; 0 1 0 -1],
//   G   = [1 0 0; 1/2 1/2 1/2; 1/2 -1/2 1/2; 0 0 1],
//   A^T = [1 1 1 0; 0 1 -1 -1],
// so per block and output channel o the 16 products at positions p are sums
// over the input channels, M[p][o] = sum_ci U[p][o][ci] V[p][ci] (U = G g G^T
// per (o, ci), V = B^T d B per ci): 16 GEMMs with K = 8 instead of one with
// K = 72, 2.25 times fewer multiply-adds.  The transforms are exact up to
// fp32 rounding (coefficients 0, +-1, +-1/2).

// W arrives as (o, ci, kh, kw) rows of 9; thread o * 8 + ci holds its 3 x 3
// filter (loaded at the workgroup's start, with x) and writes its 16 U values.
struct WinoW {
  float g[9];
};

__device__ __forceinline__ void load_w(const float *__restrict__ w, WinoW &r) {
  const float *g = w + threadIdx.x * 9;  // 512 threads = 64 x 8 filters
#pragma unroll
  for (int k = 0; k < 9; ++k) r.g[k] = g[k];
}

__device__ __forceinline__ void store_w(const WinoW &r, float *ul) {
  const int o = threadIdx.x / kCin, ci = threadIdx.x % kCin;
  const int t = o / 16, i = o % 16, ks = ci / 4, q = ci % 4;
  float h[4][3];  // G g
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    const float g0 = r.g[c], g1 = r.g[3 + c], g2 = r.g[6 + c];
    h[0][c] = g0;
    h[1][c] = 0.5f * (g0 + g1 + g2);
    h[2][c] = 0.5f * (g0 - g1 + g2);
    h[3][c] = g2;
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const float u[4] = {h[a][0], 0.5f * (h[a][0] + h[a][1] + h[a][2]),
                        0.5f * (h[a][0] - h[a][1] + h[a][2]), h[a][2]};
#pragma unroll
    for (int b = 0; b < 4; ++b)
      ul[(((4 * a + b) * 2 + ks) * kMT + t) * kWave + 16 * q + i] = u[b];
  }
}

// The wave's 16 Winograd blocks (MFMA N = 16: lane i takes block i, output
// rows 0-1 and columns 32 twave + 2 i + {0, 1} of the tile) for all 64 output
// channels.  acc[2 dy + dx][t] ends as the conv output (bias included) at
// (dy, dx) of the lane's block, channels 16 t + 4 q + r: the layout of
// conv_tile with the pixel of (blk, lane) moved.  Row a of M at a time: the
// lane builds V for its input channels q and 4 + q (B^T rows need two input
// rows), then per M-tile 8 MFMAs give M[4 a + j] for j = 0..3, which fold
// into Y by A (columns) and A^T (row a's sign).
__device__ __forceinline__ void conv_tile_wino(const ChainArgs &a, const float *xs,
                                               const float *ul, int twave,
                                               f32x4 (&acc)[kNB][kMT]) {
  const int lane = threadIdx.x % kWave;
  const int li = lane % 16, q = lane / 16;
#pragma unroll
  for (int t = 0; t < kMT; ++t) {
    f32x4 bias;
#pragma unroll
    for (int r = 0; r < 4; ++r) bias[r] = a.b ? a.b[16 * t + 4 * q + r] : 0.0f;
#pragma unroll
    for (int blk = 0; blk < kNB; ++blk) acc[blk][t] = bias;
  }
  const float *xq = xs + q * (kLdsH * kLdsW) + 2 * (16 * twave + li);
  const float *uq = ul + lane;
#pragma unroll
  for (int ar = 0; ar < 4; ++ar) {
    // Row ar of B^T d combines input rows (r0, r1) with sign sg: d_r0 + sg d_r1.
    const int r0 = (ar == 0) ? 0 : (ar == 2 ? 2 : 1);
    const int r1 = (ar == 0) ? 2 : (ar == 3 ? 3 : (ar == 1 ? 2 : 1));
    const float sg = (ar == 1) ? 1.0f : -1.0f;
    float v[2][4];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const float *xc = xq + ks * (4 * kLdsH * kLdsW);
      const float2 p0 = *reinterpret_cast<const float2 *>(xc + r0 * kLdsW);
      const float2 p1 = *reinterpret_cast<const float2 *>(xc + r0 * kLdsW + 2);
      const float2 n0 = *reinterpret_cast<const float2 *>(xc + r1 * kLdsW);
      const float2 n1 = *reinterpret_cast<const float2 *>(xc + r1 * kLdsW + 2);
      const float e0 = fmaf(sg, n0.x, p0.x), e1 = fmaf(sg, n0.y, p0.y);
      const float e2 = fmaf(sg, n1.x, p1.x), e3 = fmaf(sg, n1.y, p1.y);
      v[ks][0] = e0 - e2;
      v[ks][1] = e1 + e2;
      v[ks][2] = e2 - e1;
      v[ks][3] = e1 - e3;
    }
#pragma unroll
    for (int t = 0; t < kMT; ++t) {
      f32x4 m[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) m[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          m[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(
              uq[(((4 * ar + j) * 2 + ks) * kMT + t) * kWave], v[ks][j], m[j], 0, 0, 0);
      const f32x4 P0 = m[0] + m[1] + m[2];  // (M A) column 0 of row ar
      const f32x4 P1 = m[1] - m[2] - m[3];  // column 1
      if (ar <= 2) {                        // A^T row 0: rows 0, 1, 2 with +1
        acc[0][t] += P0;
        acc[1][t] += P1;
      }
      if (ar == 1) {                        // A^T row 1: +1, -1, -1 on rows 1, 2, 3
        acc[2][t] += P0;
        acc[3][t] += P1;
      } else if (ar >= 2) {
        acc[2][t] -= P0;
        acc[3][t] -= P1;
      }
#if LSE_CHAIN_WINO_SB >= 2
      __builtin_amdgcn_sched_barrier(0);
#endif
    }
#if LSE_CHAIN_WINO_SB >= 1
    __builtin_amdgcn_sched_barrier(0);
#endif
  }
}

// Tile-statistics word: low 32 bits the tile mean, high 32 bits -M2.  M2 >= 0,
// so the high word always has its sign bit set and a written word is never 0.
__device__ __forceinline__ uint64_t pack_stats(float mean, float m2) {
  return (uint64_t)fbits(mean) | ((uint64_t)fbits(-m2) << 32);
}

// Values counted in group statistics for tile j: 4 channels per quad, qpg
// quads per group, times the tile's valid pixels.  Only the last tile row and
// the last tile column can be partial, so no division is needed when the
// sample is one tile wide.
__device__ __forceinline__ double tile_count(const ChainArgs &a, int j, int qpg, int tiles_h) {
  int th, tw;
  if (a.tiles_w == 1) {
    th = j;
    tw = 0;
  } else {
    th = j / a.tiles_w;
    tw = j - th * a.tiles_w;
  }
  const int vr = (th == tiles_h - 1) ? a.Ho - th * kTileH : kTileH;
  const int vc = (tw == a.tiles_w - 1) ? a.Wo - tw * kTileW : kTileW;
  return (double)(4 * qpg) * (double)vr * (double)vc;
}

// How long a workgroup waits for its sample's statistics before it defers its
// pair: 0.5 ms of the 100 MHz real-time counter (a sample's tiles normally
// publish within a few microseconds of each other).
constexpr uint64_t kChainWaitTicks = 50000ull;
// Statistics words a thread keeps in registers from its last poll.
constexpr int kHeldPer = LSE_CHAIN_HELD / (kTeams * kThreads);

// Tile-relative pixel of accumulator block blk in lane i of team wave w:
// direct conv, row w / 2 and 16-pixel block blk of the wave's 64 columns;
// Winograd, (dy, dx) = (blk / 2, blk % 2) of the lane's 2 x 2 block.
__device__ __forceinline__ void pixel_of(int blk, int li, int wave, int &dh, int &dw) {
  if constexpr (kWino) {
    dh = blk / 2;
    dw = 32 * wave + 2 * li + blk % 2;
  } else {
    dh = wave / 2;
    dw = (wave % 2) * 64 + 16 * blk + li;
  }
}

__device__ __forceinline__ void tile_valid(const ChainArgs &a, int tile, bool (&valid)[kNB],
                                           int wave) {
  const int th = tile / a.tiles_w, tw = tile - th * a.tiles_w;
  const int li = threadIdx.x % 16;
#pragma unroll
  for (int blk = 0; blk < kNB; ++blk) {
    int dh, dw;
    pixel_of(blk, li, wave, dh, dw);
    valid[blk] = (th * kTileH + dh < a.Ho) && (tw * kTileW + dw < a.Wo);
  }
}

// Poll until every tile of sample n has published its statistics words
// (true) or the wait runs out (false: kChainWaitTicks or the poll limit);
// called by the whole workgroup (NT threads), every thread returns the same
// verdict.  Thread t polls words t, t + NT, ... of the sample's (tile, group)
// block, one round trip per poll; the first kHeldPer of them stay in wd.  A
// poll's verdict is the OR of one ballot per wave through LDS, so every wave
// leaves the loop together.
template <int NT, class Lds>
__device__ __forceinline__ bool wait_stats(const ChainArgs &a, int64_t n, Lds &L,
                                           uint64_t (&wd)[kHeldPer]) {
  constexpr int kWaves = NT / kWave;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const uint64_t *ws = a.stats + n * a.tiles * a.G;
  const int words = a.tiles * a.G;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (uint32_t it = 0;; ++it) {
    bool missing = false;
#pragma unroll
    for (int j = 0; j < kHeldPer; ++j) {
      const int idx = threadIdx.x + NT * j;
      wd[j] = (idx < words) ? load_pair_agent(ws + idx) : 1ull;
      missing |= (wd[j] == 0);
    }
    // Words past the held ones (samples of more than kHeldPer x NT words):
    // eight loads in flight per thread instead of one round trip per word.
    int idx = threadIdx.x + NT * kHeldPer;
    for (; idx + NT * 7 < words; idx += NT * 8) {
      uint64_t w8[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) w8[u] = load_pair_agent(ws + idx + NT * u);
#pragma unroll
      for (int u = 0; u < 8; ++u) missing |= (w8[u] == 0);
    }
    for (; idx < words; idx += NT) missing |= (load_pair_agent(ws + idx) == 0);
    const bool late =
        it >= a.spin_limit || __builtin_amdgcn_s_memrealtime() - t0 > kChainWaitTicks;
    const uint64_t mb = __builtin_amdgcn_ballot_w64(missing);
    const uint64_t lb = __builtin_amdgcn_ballot_w64(late);
    // Double-buffered by poll parity: a wave can only rewrite a slot after
    // every wave has passed the next poll's barrier, i.e. has read it.
    if (lane == 0) L.flags[it & 1][wave] = (mb != 0 ? 1u : 0u) | (lb != 0 ? 2u : 0u);
    __syncthreads();
    uint32_t f = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) f |= L.flags[it & 1][w];
    if ((f & 1u) == 0) return true;
    if (f & 2u) return false;
    __builtin_amdgcn_s_sleep(8);
  }
}

// Merge the sample's statistics (all words present; the first kHeldPer per
// thread in wd, as left by wait_stats) into the epilogue's per-channel table
// L.sc / L.sh; ends with a barrier.  Per thread in fp64: C = sum n_j,
// S1 = sum n_j mean_j, S2 = sum (M2_j + n_j mean_j^2) over its words, which
// all belong to group t % G; lanes of a wave with the same group are combined
// by xor shuffles, the waves in LDS (fixed order: the result is
// deterministic); per group mean = S1 / C, M2 = S2 - C mean^2,
// rstd = 1 / sqrt(M2 / C + eps).
template <int NT, class Lds>
__device__ __forceinline__ void merge_stats(const ChainArgs &a, int64_t n,
                                            const uint64_t (&wd)[kHeldPer], bool write_global,
                                            float ga, float be, Lds &L) {
  constexpr int kWaves = NT / kWave;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int qpg = 16 / a.G;
  const int tiles_h = a.tiles / a.tiles_w;
  const uint64_t *ws = a.stats + n * a.tiles * a.G;
  const int words = a.tiles * a.G;
  double C = 0.0, S1 = 0.0, S2 = 0.0;
  auto add = [&](int idx, uint64_t w) {
    const double c = tile_count(a, idx >> a.log2G, qpg, tiles_h);  // G is a power of 2
    const double m = (double)bitsf((uint32_t)w);
    C += c;
    S1 += c * m;
    S2 += -(double)bitsf((uint32_t)(w >> 32)) + c * m * m;
  };
#pragma unroll
  for (int j = 0; j < kHeldPer; ++j) {
    const int idx = threadIdx.x + NT * j;
    if (idx < words) add(idx, wd[j]);
  }
  // The rest in the same order, eight loads in flight at a time.
  int idx = threadIdx.x + NT * kHeldPer;
  for (; idx + NT * 7 < words; idx += NT * 8) {
    uint64_t w8[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) w8[u] = load_pair_agent(ws + idx + NT * u);
#pragma unroll
    for (int u = 0; u < 8; ++u) add(idx + NT * u, w8[u]);
  }
  for (; idx < words; idx += NT) add(idx, load_pair_agent(ws + idx));
  for (int o = kWave / 2; o >= a.G; o >>= 1) {  // lanes l, l ^ o share a group while o >= G
    C += __shfl_xor(C, o);
    S1 += __shfl_xor(S1, o);
    S2 += __shfl_xor(S2, o);
  }
  if (lane < a.G) {
    L.mrg[wave][lane][0] = C;
    L.mrg[wave][lane][1] = S1;
    L.mrg[wave][lane][2] = S2;
  }
  __syncthreads();
  if (threadIdx.x < kCout) {
    // Thread c = channel c: its group's statistics (the 4 qpg threads of a
    // group add the same values in the same order), folded with gamma, beta
    // (ga, be: this thread's channel, loaded at kernel start) and tanh's
    // 2 log2(e) into the epilogue's one multiply-add: 2 log2(e) z = v sc + sh.
    const int c = threadIdx.x, g = (c / 4) / (16 / a.G);
    double Cg = 0.0, S1g = 0.0, S2g = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      Cg += L.mrg[w][g][0];
      S1g += L.mrg[w][g][1];
      S2g += L.mrg[w][g][2];
    }
    const double MU = S1g / Cg;
    const double M2 = fmax(S2g - Cg * MU * MU, 0.0);
    const float fm = (float)MU, fr = (float)(1.0 / sqrt(M2 / Cg + (double)a.eps));
    const float sc = fr * ga;
    L.sc[c] = sc * (2.0f * kLog2e);
    L.sh[c] = (be - fm * sc) * (2.0f * kLog2e);
    if (write_global && c % (4 * (16 / a.G)) == 0) {
      a.mean[n * a.G + g] = fm;
      a.rstd[n * a.G + g] = fr;
    }
  }
  __syncthreads();
}

#ifndef LSE_CHAIN_PAIR_WAVES_PER_EU
#define LSE_CHAIN_PAIR_WAVES_PER_EU 4
#endif

// LDS scratch of the 8-wave pair workgroup besides the x and W tiles.
struct PairLds {
  float wmean[kTeams * kThreads / kWave][16];  // per wave and group: mean, M2, count
  float wm2[kTeams * kThreads / kWave][16];
  float wcnt[kTeams * kThreads / kWave];
  double mrg[kTeams * kThreads / kWave][16][3];  // per wave and group: C, S1, S2
  uint32_t flags[2][kTeams * kThreads / kWave];  // per poll parity and wave: 1 missing, 2 gave up
  // per channel, read 4 at a time: 2 log2(e) z = conv * sc + sh, z the tanh input
  alignas(16) float sc[kCout];
  alignas(16) float sh[kCout];
};


// tile_epilogue with the per-channel scale and shift read from LDS (four
// consecutive channels per read) instead of held in 32 registers.
__device__ __forceinline__ void tile_epilogue_lds(const ChainArgs &a, int64_t n, int tile,
                                                  const f32x4 (&acc)[kNB][kMT],
                                                  const bool (&valid)[kNB], const PairLds &L,
                                                  int wave) {
  const int lane = threadIdx.x % kWave;
  const int li = lane % 16, q = lane / 16;
  const int th = tile / a.tiles_w, tw = tile - th * a.tiles_w;
#pragma unroll
  for (int blk = 0; blk < kNB; ++blk) {
    // w = log2(e) u, u = v + hardswish(tanh(GN(v))): one fma folds the
    // residual add into the scaling.
    float w[kMT][4];
#pragma unroll
    for (int t = 0; t < kMT; ++t) {
      const f32x4 sc = *reinterpret_cast<const f32x4 *>(&L.sc[16 * t + 4 * q]);
      const f32x4 sh = *reinterpret_cast<const f32x4 *>(&L.sh[16 * t + 4 * q]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = acc[blk][t][r];
        w[t][r] = fmaf(v, kLog2e, hardswish_of_tanh_scaled_log2e(fmaf(v, sc[r], sh[r])));
      }
    }
    // The logsumexp of the pixel's 64 values without the max shift: the sum
    // of exp(u) = 2^w itself.  Where that sum lies in [2^-60, 2^60] no term
    // overflowed and none that matters underflowed, and each term is off by
    // at most |u| x 2^-24 relative (the rounding of w), so log S is within a
    // few 1e-7 of the shifted form.  Any other pixel (huge or tiny values, a
    // non-finite one) is done again with the max shift; the wave takes that
    // branch only if one of its pixels needs it.
    float s = 0.0f;
#pragma unroll
    for (int t = 0; t < kMT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) s += __builtin_amdgcn_exp2f(w[t][r]);
    const float S = across_quads(s, OpSum{});
    const bool redo = !(S >= 0x1p-60f && S <= 0x1p60f);  // NaN included
    float res = logf(S);
    if (__builtin_amdgcn_ballot_w64(redo) != 0) {
      float m = -__builtin_inff();
#pragma unroll
      for (int t = 0; t < kMT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) m = fmaxf(m, w[t][r]);
      const float Mw = across_quads(m, OpMax{});  // log2(e) x the max
      const float c2 = is_finite(Mw) ? Mw : 0.0f;
      float s2 = 0.0f;
#pragma unroll
      for (int t = 0; t < kMT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) s2 += __builtin_amdgcn_exp2f(w[t][r] - c2);
      const float S2 = across_quads(s2, OpSum{});
      // LSE = ln 2 (Mw + log2 S2); a non-finite Mw passes through.
      if (redo) res = is_finite(Mw) ? (Mw + __builtin_log2f(S2)) * 0.693147180559945309f : Mw;
      if (redo && (S2 != S2)) res = S2;
    }
    if (q == 0 && valid[blk]) {
      int dh, dw;
      pixel_of(blk, li, wave, dh, dw);
      a.out[(n * a.Ho + th * kTileH + dh) * (int64_t)a.Wo + tw * kTileW + dw] = res;
    }
  }
}

// Sum over the lanes whose quads share a GroupNorm group, for per-lane,
// per-M-tile values x[t] already summed over their 16-lane row (row r holds
// quad 4t + r of M-tile t): qpg = 2 pairs rows (0,1) and (2,3), qpg = 4 joins
// all four rows, qpg = 8 and 16 also join M-tiles.  Every lane ends with the
// sum of its own quad's group.
__device__ __forceinline__ void group_sum(float (&x)[kMT], int qpg) {
  if (qpg >= 2) {
#pragma unroll
    for (int t = 0; t < kMT; ++t) {
      auto p = __builtin_amdgcn_permlane16_swap(fbits(x[t]), fbits(x[t]), false, false);
      x[t] = bitsf(p[0]) + bitsf(p[1]);
    }
  }
  if (qpg >= 4) {
#pragma unroll
    for (int t = 0; t < kMT; ++t) {
      auto p = __builtin_amdgcn_permlane32_swap(fbits(x[t]), fbits(x[t]), false, false);
      x[t] = bitsf(p[0]) + bitsf(p[1]);
    }
  }
  if (qpg >= 8) {
    x[0] = x[1] = x[0] + x[1];
    x[2] = x[3] = x[2] + x[3];
  }
  if (qpg >= 16) x[0] = x[1] = x[2] = x[3] = x[0] + x[2];
}

// Per-group (mean, M2) of both tiles of a pair, one team of 4 waves per tile
// (team 1 idle when the pair has no second tile).  Each wave reduces its
// quarter tile on its own (DPP rows and permlane swaps, two passes: mean, then
// M2 about it) and leaves (count, mean, M2) per group in LDS; after the one
// barrier wave 0 combines tile A's four waves and wave 1 tile B's with the
// pairwise update of (count, mean, M2) and publishes one word per group.
__device__ __forceinline__ void publish_pair_stats(const ChainArgs &a, int64_t n, int tA, int tB,
                                                   bool hasB, bool active,
                                                   const f32x4 (&acc)[kNB][kMT],
                                                   const bool (&valid)[kNB], PairLds &L) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int li = lane % 16, q = lane / 16;
  const int qpg = 16 / a.G;
  if (active) {
    int px = 0;  // valid pixels of the wave's strip (lanes 0..15 cover its columns)
#pragma unroll
    for (int blk = 0; blk < kNB; ++blk)
      px += __builtin_popcountll(__builtin_amdgcn_ballot_w64(valid[blk]) & 0xFFFFull);
    const float cnt = (float)(4 * qpg * px);
    float mu[kMT], m2[kMT];
#pragma unroll
    for (int t = 0; t < kMT; ++t) {
      float sacc = 0.0f;
#pragma unroll
      for (int blk = 0; blk < kNB; ++blk)
        if (valid[blk])
#pragma unroll
          for (int r = 0; r < 4; ++r) sacc += acc[blk][t][r];
      mu[t] = row16_sum(sacc);
    }
    group_sum(mu, qpg);
    const float inv_cnt = (px > 0) ? 1.0f / cnt : 0.0f;  // one division for the 4 groups
#pragma unroll
    for (int t = 0; t < kMT; ++t) {
      mu[t] *= inv_cnt;
      float sacc = 0.0f;
#pragma unroll
      for (int blk = 0; blk < kNB; ++blk)
        if (valid[blk])
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float d = acc[blk][t][r] - mu[t];
            sacc = fmaf(d, d, sacc);
          }
      m2[t] = row16_sum(sacc);
    }
    group_sum(m2, qpg);
    if (li == 0) {
#pragma unroll
      for (int t = 0; t < kMT; ++t) {
        if ((4 * t + q) % qpg == 0) {  // one writer per group
          const int g = (4 * t + q) / qpg;
          L.wmean[wave][g] = mu[t];
          L.wm2[wave][g] = m2[t];
        }
      }
      if (q == 0) L.wcnt[wave] = cnt;
    }
  }
  __syncthreads();
  const int rt = wave;  // wave 0 combines team 0, wave 1 team 1
  if (rt < kTeams && lane < a.G && (rt == 0 || hasB)) {
    const int g = lane, tile = rt ? tB : tA;
    float N = 0.0f, mean = 0.0f, M2 = 0.0f;
#pragma unroll
    for (int w = 4 * rt; w < 4 * rt + 4; ++w) {
      const float nw = L.wcnt[w];
      if (nw > 0.0f) {
        const float delta = L.wmean[w][g] - mean, Nn = N + nw;
        mean += delta * (nw / Nn);
        M2 += L.wm2[w][g] + delta * delta * (N * nw / Nn);
        N = Nn;
      }
    }
    __hip_atomic_store(a.stats + (n * a.tiles + tile) * a.G + g, pack_stats(mean, M2),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// One workgroup of 8 waves = a pair of tiles (A = 2p, B = 2p + 1) of one
// sample.  Waves 0-3 stage and convolve tile A, waves 4-7 tile B, at the same
// time; each wave holds the 64 accumulators of its quarter tile, so four
// waves fit on a SIMD and one wave's MFMAs overlap others' staging, waiting
// and epilogue.  W staging and the wait for the sample's statistics are paid
// once per pair.
//   kFused: pairs in workgroup order (sample order); publish, wait for the
//           sample, merge, epilogue (one launch; used while a sample's pairs
//           fit on the GPU at once, see launch_conv_chain).
//   kStats: publish only (and, when a.stage is set, store the pair's conv
//           tiles there).  kApply: the statistics are complete (published by
//           a kStats launch): merge, epilogue.  kStats + kApply compute the
//           conv twice but never wait on another workgroup.
//   kApplyStaged: as kApply, but the conv tiles are read back from a.stage
//           (written by the kStats launch just before) instead of recomputed.
// In every mode a workgroup whose wait runs out computes the missing tile
// statistics of its sample itself (see the file comment).
enum ChainMode { kFused = 0, kStats = 1, kApply = 2, kApplyStaged = 3 };

// Staged conv tiles of one pair: 8 waves x 16 accumulator vectors x 64 lanes
// of float4 = 128 KiB, in register order, so that each wave's store or load
// of one accumulator vector is one contiguous 1 KiB.
constexpr int64_t kStageF4PerPair = (int64_t)kTeams * (kThreads / kWave) * kNB * kMT * kWave;
__device__ __forceinline__ f32x4 *stage_slot(const ChainArgs &a, uint32_t pair) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  return reinterpret_cast<f32x4 *>(a.stage) + (int64_t)(pair - a.stage_first) * kStageF4PerPair +
         (int64_t)wave * (kNB * kMT * kWave) + lane;
}

// Stage the pair of tiles of sample n with index pr (team 0: tile 2 pr, team
// 1: tile 2 pr + 1) and convolve it into acc; the caller must have passed a
// barrier since the last reads of xs.  Inactive waves (no second tile) get
// zero accumulators and no valid pixels.
__device__ __forceinline__ void stage_and_convolve(const ChainArgs &a, int64_t n, uint32_t pr,
                                                   int team, int tid, int twave, float *xs,
                                                   const float *wl, f32x4 (&acc)[kNB][kMT],
                                                   bool (&valid)[kNB]) {
  const int tile = kTeams * (int)pr + team;
  const bool active = tile < a.tiles;  // uniform per wave
  if (active) {
    XRegs xr;
    const int th = tile / a.tiles_w, tw = tile - th * a.tiles_w;
    load_x(a, n, th * kTileH, tw * kTileW, xr, tid);
    store_x(xr, xs, tid);
  }
  __syncthreads();
  if (active) {
    if constexpr (kWino)
      conv_tile_wino(a, xs, wl, twave, acc);
    else
      conv_tile(a, xs, wl, twave / 2, (twave % 2) * 64, acc);
    tile_valid(a, tile, valid, twave);
  }
}

// The epilogue's per-channel table from a sample's merged mean / rstd in the
// workspace head (written by chain_merge_kernel), with merge_stats' formula:
// the same floats in, so the same table out.  Ends with a barrier.
template <class Lds>
__device__ __forceinline__ void stats_table(const ChainArgs &a, int64_t n, float ga, float be,
                                            Lds &L) {
  if (threadIdx.x < kCout) {
    const int c = threadIdx.x, g = (c / 4) / (16 / a.G);
    const float fm = a.mean[n * a.G + g], fr = a.rstd[n * a.G + g];
    const float sc = fr * ga;
    L.sc[c] = sc * (2.0f * kLog2e);
    L.sh[c] = (be - fm * sc) * (2.0f * kLog2e);
  }
  __syncthreads();
}

// Between the statistics and apply launches of the two-launch path: one
// workgroup per sample merges its tiles' statistics once (merge_stats, the
// fused path's arithmetic and order) and writes mean / rstd for the apply
// launch, instead of every apply workgroup merging them (a 600 x 520 sample
// has 23920 words at 16 groups).
__global__ __launch_bounds__(kTeams * kThreads) void chain_merge_kernel(ChainArgs a) {
  __shared__ PairLds L;
  const int64_t n = a.block_base + blockIdx.x;  // here: first sample of the launch + index
  // Every word was published by the statistics launch, which ended before
  // this one started: nothing to wait for.
  const uint64_t *ws = a.stats + n * a.tiles * a.G;
  const int words = a.tiles * a.G;
  uint64_t wd[kHeldPer];
#pragma unroll
  for (int j = 0; j < kHeldPer; ++j) {
    const int idx = threadIdx.x + kTeams * kThreads * j;
    wd[j] = (idx < words) ? load_pair_agent(ws + idx) : 1ull;
  }
  merge_stats<kTeams * kThreads>(a, n, wd, true, 1.0f, 0.0f, L);
}

// Cold path of the sample's last arrival: finish the ndef pairs of sample n
// deferred before it (their statistics are all published).  Out of line so
// that nothing of it stays alive through the common path.
// ChainArgs is read from the kernel's argument segment (the kernel's only
// argument, at offset 0): passed by value (or by its address), the compiler
// copied it to the call frame in scratch at the start of every workgroup (16
// bytes per lane: 33 MB of writes per launch of the (128, 8, 128, 128) chain,
// for a call that almost never happens).
__device__ __noinline__ void finish_deferred(const ChainArgs *ap, int64_t n, uint32_t ndef,
                                             float *xs_team, const float *wl, PairLds *Lp) {
  const ChainArgs &a = *ap;
  PairLds &L = *Lp;
  __shared__ uint32_t s_pair;
  const uint32_t groups = (uint32_t)(a.tiles + kTeams - 1) / kTeams;
  const int team = kTeams == 1 ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x / kThreads);
  const int tid = threadIdx.x - team * kThreads;
  const int twave = tid / kWave;
  float ga = 1.0f, be = 0.0f;
  if (threadIdx.x < kCout) {
    if (a.gamma) ga = a.gamma[threadIdx.x];
    if (a.beta) be = a.beta[threadIdx.x];
  }
  for (uint32_t d = 0; d < ndef; ++d) {
    __syncthreads();  // everyone has read s_pair / finished with xs
    if (threadIdx.x == 0) {
      // The entry is stored right after its deferral was counted: it shows up.
      uint32_t e;
      while ((e = __hip_atomic_load(a.queue + n * groups + d, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT)) == 0u)
        __builtin_amdgcn_s_sleep(2);
      s_pair = e - 1u;
      __hip_atomic_fetch_add(&a.hdr->deferred, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    const uint32_t qp = s_pair;
    f32x4 acc[kNB][kMT];
    bool valid[kNB];
    stage_and_convolve(a, n, qp, team, tid, twave, xs_team, wl, acc, valid);
    uint64_t wd[kHeldPer];
    while (!wait_stats<kTeams * kThreads>(a, n, L, wd)) {
    }
    merge_stats<kTeams * kThreads>(a, n, wd, qp == 0, ga, be, L);
    const int tile = kTeams * (int)qp + team;
    if (tile < a.tiles) tile_epilogue_lds(a, n, tile, acc, valid, L, twave);
  }
}

#ifndef LSE_CHAIN_XCD
#define LSE_CHAIN_XCD 1
#endif
// The pair of this workgroup within its launch.  Workgroups go to the 8 XCDs
// round robin (b to XCD b % 8), each with its own L2, and neighbouring pairs
// share the 2 input rows at their boundary (the 3 x 3 halo).  With xcd_order
// the launch's pairs are dealt to the XCDs in 8 contiguous ranges, so that
// neighbours, and all pairs of a sample, run on one XCD: pair
// (b % 8) F + b / 8, F = grid / 8, for b < 8 F (a bijection; the last grid % 8
// keep their index).  The host sets it when a sample's pairs fit half of one
// XCD (the fused launch waits on a sample's pairs) or for launches that never
// wait.
__device__ __forceinline__ uint32_t xcd_pair(const ChainArgs &a) {
  const uint32_t b = blockIdx.x;
  if (LSE_CHAIN_XCD && a.xcd_order) {
    const uint32_t f = gridDim.x / 8;
    if (b < 8 * f) return (b % 8) * f + b / 8;
  }
  return b;
}

template <int MODE>
__global__ __launch_bounds__(kTeams * kThreads)
__attribute__((amdgpu_waves_per_eu(LSE_CHAIN_PAIR_WAVES_PER_EU)))
void conv_chain_pair_kernel(ChainArgs a) {
  __shared__ alignas(16) float xs[kTeams][kCin * kLdsH * kLdsW];
  __shared__ alignas(16) float wl[kWLds];  // W rows, or U in fragment order (Winograd)
  __shared__ PairLds L;
  __shared__ uint32_t s_ndef, s_last;
  // W's and x's loads are in flight together.  The pair is the workgroup
  // index: an atomic ticket (pairs in the order workgroups start) put its
  // round trip before the x loads and measured 0.209 against 0.195 ms on
  // (128, 8, 128, 128), with bit-identical results.
  std::conditional_t<kWino, WinoW, WRegs<kTeams * kThreads>> wr;
  if constexpr (MODE != kApplyStaged) load_w(a.w, wr);
  const uint32_t pair = a.block_base + xcd_pair(a);
  const uint32_t groups = (uint32_t)(a.tiles + kTeams - 1) / kTeams;  // workgroups per sample
  const int64_t n = pair / groups;
  const uint32_t p = pair - (uint32_t)n * groups;
  const int tA = kTeams * (int)p, tB = tA + 1;
  const bool hasB = kTeams == 2 && tB < a.tiles;  // uniform

  const int team = kTeams == 1 ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x / kThreads);
  const int tid = threadIdx.x - team * kThreads;                           // within the team
  const int twave = tid / kWave;
  const bool active = team == 0 || hasB;                                   // uniform per wave
  const int tile = team ? tB : tA;

  f32x4 acc[kNB][kMT];
  bool valid[kNB];
  if constexpr (MODE == kApplyStaged) {
    if (active) {  // the conv tiles from the staging area
      const f32x4 *src = stage_slot(a, pair);
#pragma unroll
      for (int blk = 0; blk < kNB; ++blk)
#pragma unroll
        for (int t = 0; t < kMT; ++t) acc[blk][t] = src[(blk * kMT + t) * kWave];
      tile_valid(a, tile, valid, twave);
    }
  } else {
    XRegs xr;
    if (active) {
      const int th = tile / a.tiles_w, tw = tile - th * a.tiles_w;
      load_x(a, n, th * kTileH, tw * kTileW, xr, tid);
    }
    store_w(wr, wl);  // W rows, or U (Winograd)
    if (active) store_x(xr, xs[team], tid);
    __syncthreads();
    if (active) {
      if constexpr (kWino)
        conv_tile_wino(a, xs[team], wl, twave, acc);
      else
        conv_tile(a, xs[team], wl, twave / 2, (twave % 2) * 64, acc);
      tile_valid(a, tile, valid, twave);
    }
  }
  if constexpr (MODE == kFused || MODE == kStats)
    publish_pair_stats(a, n, tA, tB, hasB, active, acc, valid, L);
  if constexpr (MODE == kStats) {
    if (a.stage && active) {  // uniform per wave
      f32x4 *dst = stage_slot(a, pair);
#pragma unroll
      for (int blk = 0; blk < kNB; ++blk)
#pragma unroll
        for (int t = 0; t < kMT; ++t) dst[(blk * kMT + t) * kWave] = acc[blk][t];
    }
    return;
  }
  // This thread's channel of gamma / beta (threads < 64), loaded only now so
  // that they are not held through the conv.
  float ga = 1.0f, be = 0.0f;
  if (threadIdx.x < kCout) {
    if (a.gamma) ga = a.gamma[threadIdx.x];
    if (a.beta) be = a.beta[threadIdx.x];
  }
  if constexpr (MODE == kApply || MODE == kApplyStaged) {
    // The sample's mean / rstd were merged by chain_merge_kernel between the
    // launches: nothing to wait for, no per-workgroup merge.
    stats_table(a, n, ga, be, L);
    if (active) tile_epilogue_lds(a, n, tile, acc, valid, L, twave);
    return;
  }
  // Arrival (after this pair's statistics were published); the returned
  // counts are needed only after the epilogue, so the round trip overlaps
  // the wait.
  uint64_t arrived_before = 0;
  if (threadIdx.x == 0)
    arrived_before = __hip_atomic_fetch_add(a.arrivals + n, 1ull, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
  uint64_t wd[kHeldPer];
  // A poll limit of 0 (test hook) tries to defer without waiting.
  bool ok = a.spin_limit != 0 && wait_stats<kTeams * kThreads>(a, n, L, wd);  // uniform
  if (!ok) {
    if (threadIdx.x == 0) {
      const uint64_t st = __hip_atomic_fetch_add(a.arrivals + n, 1ull << 32, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
      const bool all_arrived = (uint32_t)st == groups;
      if (!all_arrived)  // the sample's last arrival finishes this pair
        __hip_atomic_store(a.queue + n * groups + (uint32_t)(st >> 32), p + 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      s_last = all_arrived ? 1u : 0u;
    }
    __syncthreads();
    if (s_last == 0) return;  // deferred
    // Every pair of the sample has arrived, so every statistic is published:
    // poll until all are visible (normally the first poll).
    while (!wait_stats<kTeams * kThreads>(a, n, L, wd)) {
    }
  }
  // The last arrival of the sample finishes the pairs deferred before it.
  if (threadIdx.x == 0)
    s_ndef = ((uint32_t)arrived_before + 1u == groups) ? (uint32_t)(arrived_before >> 32) : 0u;
  merge_stats<kTeams * kThreads>(a, n, wd, tA == 0, ga, be, L);  // barriers: s_ndef visible
  if (active) tile_epilogue_lds(a, n, tile, acc, valid, L, twave);
  const uint32_t ndef = s_ndef;
  if (ndef != 0)
    finish_deferred((const ChainArgs *)__builtin_amdgcn_kernarg_segment_ptr(), n, ndef, xs[team],
                    wl, &L);
}

// Clear n 64-bit words (the header, the statistics words and the queue);
// grid-stride, at most 4096 workgroups.
__global__ __launch_bounds__(256) void chain_clear_kernel(uint64_t *__restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0;
}

}  // namespace

namespace {
// Which launches compute the chain: one fused launch, or a statistics launch
// then an apply launch that recomputes the conv, or one that reads the conv
// tiles back from a staging area in the workspace (sized for the 256 MB
// Infinity Cache).
enum ChainPath { kPathAuto = 0, kPathFused = 1, kPathRecompute = 2, kPathStaged = 3 };
thread_local int h_chain_path = kPathAuto;  // test hook: force a path on this thread

constexpr size_t kStageBytesPerPair = (size_t)kStageF4PerPair * 16;  // 128 KiB
constexpr size_t kStageCapBytes = (size_t)192 << 20;  // staged samples per batch fit this
#ifndef LSE_CHAIN_STAGED_DEFAULT
#define LSE_CHAIN_STAGED_DEFAULT 0   // two-launch path: 1 stages, 0 recomputes the conv
#endif

}  // namespace
int64_t fused_pair_limit();
namespace {

struct ChainLayout {
  int64_t tiles_w, tiles, per_sample;
  int path;                // kPathFused, kPathRecompute or kPathStaged
  int64_t stage_samples;   // samples per staged batch
  size_t head, stats_off, arrivals_off, queue_off, stage_off, total;
};
ChainLayout chain_layout(int64_t N, int64_t H, int64_t W, int64_t K, int64_t groups) {
  ChainLayout L;
  const int64_t Ho = H - K + 1, Wo = W - K + 1;
  L.tiles_w = (Wo + kTileW - 1) / kTileW;
  L.tiles = ((Ho + kTileH - 1) / kTileH) * L.tiles_w;
  L.per_sample = (L.tiles + kTeams - 1) / kTeams;  // tile pairs = workgroups per sample
  const bool stage_fits = (size_t)L.per_sample * kStageBytesPerPair <= kStageCapBytes;
  const int forced = h_chain_path;
  if (forced == kPathFused || forced == kPathRecompute)
    L.path = forced;
  else if (forced == kPathStaged)
    L.path = stage_fits ? kPathStaged : kPathRecompute;
  else if (L.per_sample <= fused_pair_limit())
    L.path = kPathFused;
  else
    L.path = (LSE_CHAIN_STAGED_DEFAULT && stage_fits) ? kPathStaged : kPathRecompute;
  L.stage_samples = 0;
  if (L.path == kPathStaged) {
    L.stage_samples = (int64_t)(kStageCapBytes / ((size_t)L.per_sample * kStageBytesPerPair));
    if (L.stage_samples > N) L.stage_samples = N;
  }
  L.head = ((size_t)(2 * N * groups) * sizeof(float) + 255) / 256 * 256;  // mean, rstd
  L.stats_off = L.head + sizeof(ChainWsHeader);
  L.arrivals_off = L.stats_off + (size_t)(N * L.tiles * groups) * sizeof(uint64_t);
  L.queue_off = L.arrivals_off + (size_t)N * sizeof(uint64_t);
  // one queue slot per tile pair
  L.stage_off = L.queue_off + ((size_t)(N * L.per_sample) * 4 + 255) / 256 * 256;
  L.total = L.stage_off + (size_t)L.stage_samples * L.per_sample * kStageBytesPerPair;
  if (L.path != kPathStaged) L.total = L.queue_off + ((size_t)(N * L.per_sample) * 4 + 7) / 8 * 8;
  return L;
}
}  // namespace

void set_chain_path(int path) { h_chain_path = path; }

// The fused launch needs every pair of a sample resident at once (a waiting
// workgroup holds its slot).  It is used while a sample has at most half as
// many pairs as the current device can hold (the other half is headroom for
// other work sharing the GPU); larger samples take the two-launch path.
// Queried once per device.
int64_t fused_pair_limit() {
  static std::atomic<int64_t> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int64_t v = cached[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, conv_chain_pair_kernel<kFused>,
                                                   kTeams * kThreads, 0) != hipSuccess)
    return 0;  // unknown: always the two-launch path
  v = std::max<int64_t>(1, (int64_t)cus * per_cu / 2);
  cached[dev].store(v, std::memory_order_relaxed);
  return v;
}

size_t conv_chain_workspace_bytes(int64_t N, int64_t /*Cin*/, int64_t H, int64_t W,
                                  int64_t /*Cout*/, int64_t K, int64_t groups) {
  return chain_layout(N, H, W, K, groups).total;
}

hipError_t launch_conv_chain(const float *x, const float *w, const float *b, const float *gamma,
                             const float *beta, int64_t N, int64_t Cin, int64_t H, int64_t W,
                             int64_t Cout, int64_t K, int64_t groups, float eps, float *out,
                             void *ws, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  (void)Cin; (void)Cout;
  const ChainLayout L = chain_layout(N, H, W, K, groups);
  ChainArgs a;
  a.x = x; a.w = w; a.b = b; a.gamma = gamma; a.beta = beta;
  a.N = (int32_t)N;
  a.H = (int32_t)H; a.W = (int32_t)W;
  a.Ho = (int32_t)(H - K + 1); a.Wo = (int32_t)(W - K + 1);
  a.G = (int32_t)groups;
  a.log2G = 0;
  while ((1 << a.log2G) < a.G) ++a.log2G;
  a.tiles_w = (int32_t)L.tiles_w;
  a.tiles = (int32_t)L.tiles;
  a.eps = eps;
  a.spin_limit = chain_spin_limit();
  a.out = out;
  char *base = reinterpret_cast<char *>(ws);
  a.mean = reinterpret_cast<float *>(base);
  a.rstd = a.mean + N * groups;
  a.hdr = reinterpret_cast<ChainWsHeader *>(base + L.head);
  a.stats = reinterpret_cast<uint64_t *>(base + L.stats_off);
  a.arrivals = reinterpret_cast<uint64_t *>(base + L.arrivals_off);
  a.queue = reinterpret_cast<uint32_t *>(base + L.queue_off);
  a.block_base = 0;
  // Pairs of a sample on one XCD: always for the launches that never wait;
  // for the fused launch only while a sample holds at most half of one XCD's
  // resident pairs (its pairs then all run at once on that XCD).
  a.xcd_order = (L.path != kPathFused || L.per_sample * 8 <= fused_pair_limit()) ? 1u : 0u;
  // The header, the statistics words and the queue start at 0 (the staging
  // area is written before it is read).
  const size_t clear_end = L.path == kPathStaged ? L.stage_off : L.total;
  const int64_t words = (int64_t)((clear_end - L.head) / sizeof(uint64_t));
  const int64_t clear_blocks = std::min<int64_t>((words + 255) / 256, 4096);
  hipLaunchKernelGGL(chain_clear_kernel, dim3((uint32_t)clear_blocks), dim3(256), 0, stream,
                     reinterpret_cast<uint64_t *>(base + L.head), words);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t per_sample = L.per_sample;
  // Samples per launch: a dispatch's work-item count must fit 32 bits (and a
  // staged batch must fit the staging area).
  int64_t max_n = std::max<int64_t>(1, (0xffffffffll / (kTeams * kThreads)) / per_sample);
  if (L.path == kPathStaged) max_n = std::min(max_n, L.stage_samples);
  a.stage = L.path == kPathStaged ? reinterpret_cast<float *>(base + L.stage_off) : nullptr;
  const dim3 block(kTeams * kThreads);
  for (int64_t n0 = 0; n0 < N; n0 += max_n) {
    const int64_t nb = std::min(max_n, N - n0);
    const dim3 grid((uint32_t)(nb * per_sample));
    a.block_base = (uint32_t)(n0 * per_sample);
    a.stage_first = a.block_base;
    if (L.path == kPathFused) {
      hipLaunchKernelGGL(conv_chain_pair_kernel<kFused>, grid, block, 0, stream, a);
    } else {
      hipLaunchKernelGGL(conv_chain_pair_kernel<kStats>, grid, block, 0, stream, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      ChainArgs m = a;
      m.block_base = (uint32_t)n0;  // the merge takes samples, one workgroup each
      hipLaunchKernelGGL(chain_merge_kernel, dim3((uint32_t)nb), block, 0, stream, m);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if (L.path == kPathStaged)
        hipLaunchKernelGGL(conv_chain_pair_kernel<kApplyStaged>, grid, block, 0, stream, a);
      else
        hipLaunchKernelGGL(conv_chain_pair_kernel<kApply>, grid, block, 0, stream, a);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace lse
