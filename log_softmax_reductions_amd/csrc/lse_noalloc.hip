// lse_noalloc.hip — log_softmax_rows for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops): the split rows'
// (max, sum) pair workspace lives in a file-scope device array instead of a
// caller's buffer.
//
// The array is one per GPU the library runs on, held until the process ends.
// Host code never passes the array's name to a kernel (on the host that name
// is only a stand-in): the first call on each device, with that device
// current, resolves the device address with hipGetSymbolAddress and keeps it;
// every kernel argument uses that address.  Calls on one GPU share the array,
// so calls that overlap on one GPU (different streams, or different threads
// enqueueing concurrently) race; each call clears what it uses with a kernel
// on its stream before using it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "lse_internal.hpp"

namespace lse {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace lse
