// bench_copy.hip — device-to-device fp32 copies for the benchmark's copy
// ceiling (read n floats once, write them once): the same bytes as the
// row-wise log_softmax moves, with no arithmetic and no cross-workgroup
// traffic.  Not part of liblse.so; bench.py loads the library built from this
// file and reports the fastest variant.
//
//   variant 0 "tile":   the log_softmax kernel's own access pattern: 512-lane
//                       workgroups, each copying 32768 floats held in
//                       registers (16 non-temporal 128-bit loads per lane,
//                       each wave one contiguous 16 KiB run), stored through
//                       a raw buffer resource with the nt | sc1 policy bits;
//   variant 1 "stream": a grid-stride loop, 4 non-temporal 128-bit loads in
//                       flight per lane, non-temporal 128-bit stores;
//   variant 2 "plain":  one 128-bit load and store per work-item, default
//                       cache policy.
// bench_copy_capped runs "tile" with unused dynamic LDS per workgroup, which
// caps how many workgroups a CU holds (fewer requests in flight).
// n must be a multiple of 4 and both pointers 16-byte aligned; variant 0
// also needs n to be a multiple of 32768 (bench_copy returns -1 otherwise).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
constexpr int kWave = 64;
constexpr int kTileThreads = 512, kTileVec = 16;  // 16 float4 per lane
constexpr int64_t kTileFloats = (int64_t)kTileThreads * kTileVec * 4;  // 32768

__global__ __launch_bounds__(kTileThreads) void copy_tile(const v4f *__restrict__ x,
                                                          float *__restrict__ y) {
  const int t = threadIdx.x;
  const int64_t base4 = (int64_t)blockIdx.x * (kTileFloats / 4);
  v4f v[kTileVec];
#pragma unroll
  for (int q = 0; q < kTileVec; ++q)
    v[q] = __builtin_nontemporal_load(x + base4 + ((t / kWave) * kTileVec + q) * kWave + t % kWave);
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      y + base4 * 4, 0, (int)(kTileFloats * 4), 0x00020000);
#pragma unroll
  for (int q = 0; q < kTileVec; ++q)
    __builtin_amdgcn_raw_buffer_store_b128(v[q], r,
                                           (((t / kWave) * kTileVec + q) * kWave + t % kWave) * 16,
                                           0, 18);
}

__global__ __launch_bounds__(256) void copy_stream(const v4f *__restrict__ x, v4f *__restrict__ y,
                                                   int64_t n4) {
  constexpr int U = 4;
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + (U - 1) * stride < n4; i += U * stride) {
    v4f f[U];
#pragma unroll
    for (int u = 0; u < U; ++u) f[u] = __builtin_nontemporal_load(x + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) __builtin_nontemporal_store(f[u], y + i + u * stride);
  }
  for (; i < n4; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(x + i), y + i);
}

__global__ __launch_bounds__(256) void copy_plain(const v4f *__restrict__ x, v4f *__restrict__ y,
                                                  int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n4) y[i] = x[i];
}

}  // namespace

// "tile" with `lds_bytes` of dynamic LDS per workgroup (unused), which caps
// the workgroups resident per CU (160 KiB of LDS per CU).
extern "C" __attribute__((visibility("default"))) int bench_copy_capped(const float *x, float *y,
                                                                         int64_t n, int lds_bytes,
                                                                         hipStream_t stream) {
  if (n % kTileFloats != 0 || n / kTileFloats > 0x7fffffff || lds_bytes < 0 ||
      lds_bytes > 160 * 1024 || ((uintptr_t)x | (uintptr_t)y) % 16 != 0)
    return -1;
  hipLaunchKernelGGL(copy_tile, dim3((uint32_t)(n / kTileFloats)), dim3(kTileThreads),
                     (unsigned)lds_bytes, stream, reinterpret_cast<const v4f *>(x), y);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

extern "C" __attribute__((visibility("default"))) int bench_copy(const float *x, float *y,
                                                                  int64_t n, int variant,
                                                                  hipStream_t stream) {
  if (n % 4 != 0 || ((uintptr_t)x | (uintptr_t)y) % 16 != 0) return -1;
  const int64_t n4 = n / 4;
  if (variant == 0) {
    if (n % kTileFloats != 0 || n / kTileFloats > 0x7fffffff) return -1;
    hipLaunchKernelGGL(copy_tile, dim3((uint32_t)(n / kTileFloats)), dim3(kTileThreads), 0,
                       stream, reinterpret_cast<const v4f *>(x), y);
  } else if (variant == 1) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return -1;
    hipLaunchKernelGGL(copy_stream, dim3((uint32_t)(cus * 16)), dim3(256), 0, stream,
                       reinterpret_cast<const v4f *>(x), reinterpret_cast<v4f *>(y), n4);
  } else if (variant == 2) {
    if ((n4 + 255) / 256 > 0x7fffffff) return -1;
    hipLaunchKernelGGL(copy_plain, dim3((uint32_t)((n4 + 255) / 256)), dim3(256), 0, stream,
                       reinterpret_cast<const v4f *>(x), reinterpret_cast<v4f *>(y), n4);
  } else {
    return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
