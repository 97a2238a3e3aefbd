// Internal interface of the host-side runtime helpers (pagedattn_runtime.hip)
// that the C ABI calls: the library's static device scratch for callers
// that cannot allocate.  Kept apart from the launch interfaces so that
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

}  // namespace pa_internal
