// k_static_scratch.hip -- the device-resident scratch array behind
// ox_conv2d_fused_static, the convolution entry point that allocates
// nothing (for callers that cannot call hipMalloc: code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation).
//
// The array lives in the library's code object, one copy per GPU, for the
// life of the process.  In host code its name only stands in for the symbol;
// its device address on the current GPU comes from hipGetSymbolAddress,
// looked up once per device on the first call made with that device current,
// and kept.  Every call on one GPU shares that GPU's copy, which keeps the
// last call's contents: the split-K partials written there are fully
// rewritten before they are read, so nothing needs clearing, and calls that
// overlap on one GPU (two streams, two threads) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ox_internal.h"

namespace ox {

namespace {

constexpr size_t kScratchBytes = (size_t)32 << 20;   // 32 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

void* g_ptr[kMaxDevices];
int g_rc[kMaxDevices];
std::once_flag g_once[kMaxDevices];

}  // namespace

size_t static_scratch_bytes() { return kScratchBytes; }

int static_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev]() {
    void* p = nullptr;
    const hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_rc[dev] = (int)r;
    g_ptr[dev] = r == hipSuccess ? p : nullptr;
  });
  *ptr = g_ptr[dev];
  return g_rc[dev];
}

}  // namespace ox
