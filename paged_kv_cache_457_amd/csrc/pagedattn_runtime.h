// Internal interface of the host-side runtime helpers (pagedattn_runtime.hip)
// that the C ABI calls: the library's static device scratch for callers
// that cannot allocate, and the device-to-host copy of the optional
// precondition checks.  Kept apart from the launch interfaces so that
// adding these changes no kernel's sources.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace pa_internal {

// Bytes of the static device scratch that paged_attention_decode_noalloc
// uses in place of a caller's workspace (one copy per device).
constexpr size_t kNoallocScratchBytes = size_t(32) << 20;

// The current device's address of the static scratch, looked up once per
// device; 0 on success, PA_ERR_HIP (6) when the runtime fails.
int noalloc_scratch(void **ptr);

// Copies `bytes` from `src` (device memory, or host memory the device can
// reach) to the pageable host buffer `dst`, ordered on `stream`, and waits
// for it.  Used only by the PA_DEBUG_CHECKS=1 pass.  0 on success, 6 on a
// runtime error.
int copy_to_host_sync(void *dst, const void *src, size_t bytes, void *stream);

}  // namespace pa_internal
