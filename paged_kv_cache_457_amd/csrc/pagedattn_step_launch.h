// Internal interface of the fused decode step (cache write, then decode)
// between the host-side C ABI and its HIP launch code, kept apart from the
// shared internal header so adding it changes no other kernel's sources.
#pragma once

#include "pagedattn_internal.h"
#include "pagedattn_prefill_launch.h"

namespace pa_internal {

// The step's tokens to the cache and the decode call's plan in one launch,
// then the decode call's partition (and reduce) kernels.  cache.num_tokens
// is the call's num_seqs; returns 0 or the PA_ERR_HIP code.
int launch_decode_step(const DecodeLaunch &a, const CacheLaunch &cache);
// The same for shared-prefix decode: the step's tokens and the shared-prefix
// plan in one launch, then the unit kernel and the reduce.
int launch_shared_prefix_step(const PrefixLaunch &p, const CacheLaunch &cache);
// The shared-prefix plan alone (cache null) or with the step's cache write.
int launch_prefix_prep(const PrefixLaunch &p, const CacheLaunch *cache);
// A prefill step: the chunk rows to the cache and the prefill plan in one
// launch, then the attention (and reduce) kernels; cache.num_tokens is the
// call's num_tokens.
int launch_prefill_step(const PrefillLaunch &a, const CacheLaunch &cache);

}  // namespace pa_internal
