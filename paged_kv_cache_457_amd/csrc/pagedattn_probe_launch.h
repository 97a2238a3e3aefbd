// Internal interface of the decode access-pattern read probe between the
// host-side C ABI and its HIP launch code, kept apart from the shared
// internal header so adding it changes no other kernel's sources.
#pragma once

#include "pagedattn_internal.h"

namespace pa_internal {

// The plan kernel alone (the unit list of a decode call, into a.plan).
int launch_decode_plan(const DecodeLaunch &a);
// The plan kernel, then the decode access-pattern read probe.
int launch_decode_read_probe(const DecodeLaunch &a);
// Whether the grouped-query (matrix-core) partition kernel runs one item
// per wavefront for this call (partition and table sizes only).
bool gqa_wave_items(const DecodeLaunch &a);

}  // namespace pa_internal
