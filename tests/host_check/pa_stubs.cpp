// Host-only stand-ins for the HIP side of libpagedattn, for building the C
// ABI's host code (pagedattn_api.cpp) with the address and undefined-
// behaviour sanitizers and no GPU.  Test infrastructure only.
//
// Every launch returns success without touching memory and records what it
// was given; the queries below report how many launches ran and the byte
// range of the workspace the last launch's plan and partials would span.
// The static scratch is a fixed stand-in address; the debug pass's device
// copy is a host memcpy (the tests hand it host arrays).
#include <cstdint>
#include <cstring>

#include "pagedattn_internal.h"
#include "pagedattn_prefill_launch.h"
#include "pagedattn_probe_launch.h"
#include "pagedattn_step_launch.h"
#include "pagedattn_runtime.h"

namespace {
int g_launches = 0;
uintptr_t g_lo = 0, g_hi = 0;

void span(const void *p, size_t bytes) {
  if (!p || bytes == 0) return;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  if (g_lo == 0 || a < g_lo) g_lo = a;
  if (a + bytes > g_hi) g_hi = a + bytes;
}

void decode_span(const pa_internal::DecodeLaunch &a, size_t plan_ints) {
  g_lo = g_hi = 0;
  span(a.plan, plan_ints * sizeof(int32_t));
  const size_t rows = (size_t)a.num_seqs * a.num_heads * a.max_parts;
  if (a.ws_acc) span(a.ws_acc, rows * a.head_dim * sizeof(float));
  if (a.ws_ml) span(a.ws_ml, rows * 2 * sizeof(float));
}
}  // namespace

namespace pa_internal {

int launch_decode(const DecodeLaunch &a) {
  ++g_launches;
  decode_span(a, kPlanHeader + (size_t)a.num_seqs * a.max_parts);
  return 0;
}
int launch_decode_read_probe(const DecodeLaunch &a) { return launch_decode(a); }
int launch_decode_step(const DecodeLaunch &a, const CacheLaunch &) { return launch_decode(a); }
int launch_decode_shared_prefix(const PrefixLaunch &p);
int launch_shared_prefix_step(const PrefixLaunch &p, const CacheLaunch &) {
  return launch_decode_shared_prefix(p);
}
int launch_decode_shared_prefix(const PrefixLaunch &p) {
  ++g_launches;
  decode_span(p.base, 0);
  // unit records, then nslots and seq_pre
  span(p.base.plan, (kPlanHeader + (size_t)kPrefixUnitInts * p.max_units) * sizeof(int32_t));
  span(p.nslots, (size_t)p.base.num_seqs * sizeof(int32_t));
  span(p.seq_pre, (size_t)p.base.num_seqs * sizeof(int32_t));
  return 0;
}
int launch_prefill(const PrefillLaunch &a) {
  ++g_launches;
  g_lo = g_hi = 0;
  span(a.plan, (kPlanHeader + (size_t)kPrefillPlanRecord * a.num_tokens * a.max_parts) *
                   sizeof(int32_t));
  span(a.nparts, (size_t)a.num_tokens * sizeof(int32_t));
  const size_t rows = (size_t)a.num_tokens * a.num_heads * a.max_parts;
  if (a.ws_acc) span(a.ws_acc, rows * a.head_dim * sizeof(float));
  if (a.ws_ml) span(a.ws_ml, rows * 2 * sizeof(float));
  return 0;
}
int launch_prefill_step(const PrefillLaunch &a, const CacheLaunch &) {
  return launch_prefill(a);
}
int launch_reshape_and_cache(const CacheLaunch &) { return ++g_launches, 0; }
int launch_reshape_and_cache_rope(const RopeLaunch &) { return ++g_launches, 0; }
int launch_copy_pages(const CopyLaunch &) { return ++g_launches, 0; }
int launch_hbm_probe(const void *, size_t, void *, void *) { return ++g_launches, 0; }
size_t hbm_probe_sink_bytes() { return 4096; }

int noalloc_scratch(void **ptr) {
  *ptr = reinterpret_cast<void *>(uintptr_t(1) << 40);
  return 0;
}

int copy_to_host_sync(void *dst, const void *src, size_t bytes, void *) {
  if (bytes) std::memcpy(dst, src, bytes);
  return 0;
}

}  // namespace pa_internal

extern "C" {
int pa_stub_launches(void) { return g_launches; }
// [lo, hi): the workspace bytes the last decode-family or prefill launch's
// plan and partials span (0, 0 when it had none)
void pa_stub_last_span(uintptr_t *lo, uintptr_t *hi) {
  *lo = g_lo;
  *hi = g_hi;
}
}
