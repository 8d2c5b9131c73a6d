// Device scratch of the no-allocation decode entry point
// (pkv_paged_decode_attn_noalloc): a file-scope device array that stands in
// for the caller's decode workspace, for callers that cannot allocate (code
// under HIP graph capture, tight serving loops, harnesses that forbid it).
//
// Each device the library runs on holds its own copy of the array for the
// life of the process. Host code never passes the array's name to a kernel
// (on the host it is only a stand-in for the symbol): the device address is
// looked up once per device with hipGetSymbolAddress, with that device
// current, and kept; the kernels take that address as their workspace.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "internal.hpp"
#include "pkv.h"

static __device__ __align__(256) char scratch[PKV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

}  // namespace

namespace pkv {

hipError_t noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      // this device's copy of the array, looked up with the device current
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace pkv
