// workspace.hip -- per-(device, stream) scratch buffers for kernels that
// need device memory beyond their inputs and outputs (split-K partials).
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <utility>

#include "ox_internal.h"

namespace ox {

namespace {

struct Buf {
  void* ptr = nullptr;
  size_t bytes = 0;
};

std::mutex g_mu;
std::map<std::pair<int, void*>, Buf> g_bufs;

}  // namespace

void* stream_workspace(void* stream, size_t bytes) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  Buf& b = g_bufs[{dev, stream}];
  if (b.bytes >= bytes) return b.ptr;
  if (b.ptr) {
    // work already queued on this stream may still use the old buffer
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return nullptr;
    (void)hipFree(b.ptr);
    b.ptr = nullptr;
    b.bytes = 0;
  }
  size_t want = bytes < ((size_t)1 << 20) ? ((size_t)1 << 20) : bytes;
  void* p = nullptr;
  if (hipMalloc(&p, want) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  b.ptr = p;
  b.bytes = want;
  return p;
}

}  // namespace ox
