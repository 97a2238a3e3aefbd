// Host-side runtime helpers of libpagedattn: the static device scratch of
// the allocation-free decode entry point, and the synchronous copy the
// optional precondition checks read device tables with.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pagedattn_internal.h"
#include "pagedattn_runtime.h"

namespace {

// Scratch of paged_attention_decode_noalloc: the work plan and the split-K
// partials of one call.  Every device the library runs on holds its own copy
// until the process ends.  In host code `scratch` names a host-side stand-in
// of the symbol, not device memory: kernels get the device address that
// hipGetSymbolAddress returns for the current device (noalloc_scratch).
static __device__ __align__(256) char scratch[pa_internal::kNoallocScratchBytes];

std::mutex g_scratch_mutex;
void *g_scratch_ptr[pa_internal::kMaxDevices];

}  // namespace

namespace pa_internal {

int noalloc_scratch(void **ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 6;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    // once per device, with that device current
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return 6;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return 0;
}

int copy_to_host_sync(void *dst, const void *src, size_t bytes, void *stream) {
  if (bytes == 0) return 0;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(dst, src, bytes, hipMemcpyDefault, st) != hipSuccess) return 6;
  return hipStreamSynchronize(st) == hipSuccess ? 0 : 6;
}

}  // namespace pa_internal
