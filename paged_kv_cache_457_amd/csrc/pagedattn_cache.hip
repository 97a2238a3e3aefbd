// KV-cache write and the HBM read probe.
//
// Each decode step produces the next token together with the updated KV
// cache (tutorial page, section 4.3, step 3 of the iteration): the new
// token's K and V rows go to the page slot its sequence's page table gives.
#include "pagedattn_device.h"
#include "pagedattn_internal.h"

namespace {

using namespace pa_dev;

// ------------------------------------------------------------ cache write
// Grid (num_tokens), 256 threads.  Copies token t's K and V rows, all
// kv-heads, 16 bytes per lane, to page slot / bs at offset slot % bs.
__global__ __launch_bounds__(256) void pa_reshape_and_cache(
    const u32x4 *__restrict__ k, const u32x4 *__restrict__ v, u32x4 *__restrict__ k_pool,
    u32x4 *__restrict__ v_pool, const int64_t *__restrict__ slot_mapping, int num_kv_heads,
    int row_chunks, int block_size, int64_t num_slots) {
  const int t = blockIdx.x;
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t page = slot / block_size;
  const int64_t off = slot - page * block_size;
  const int total = num_kv_heads * row_chunks;
  for (int c = threadIdx.x; c < total; c += blockDim.x) {
    const int g = c / row_chunks;
    const int dc = c - g * row_chunks;
    const size_t src = ((size_t)t * num_kv_heads + g) * row_chunks + dc;
    const size_t dst = (((size_t)page * num_kv_heads + g) * block_size + off) * row_chunks + dc;
    k_pool[dst] = k[src];
    v_pool[dst] = v[src];
  }
}

// -------------------------------------------------------- HBM read probe
// Achievable read bandwidth: each of kProbeBlocks workgroups streams one
// contiguous slice of the buffer with non-temporal 16-byte loads, four
// 4 KiB rows in flight per workgroup.  Long per-workgroup streams measured
// faster on MI355X than a grid-stride sweep (7.0 vs 6.2-6.5 TB/s over 4 GiB).
constexpr int kProbeBlocks = 1024;
constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;

__global__ __launch_bounds__(kProbeThreads) void pa_hbm_probe(const u32x4 *__restrict__ buf,
                                                              size_t n16, size_t per_block,
                                                              uint32_t *__restrict__ sink) {
  const size_t lo = (size_t)blockIdx.x * per_block;
  const size_t hi = min(lo + per_block, n16);
  size_t i = lo + threadIdx.x;
  uint32_t x = 0;
  for (; i + (kProbeUnroll - 1) * kProbeThreads < hi; i += kProbeUnroll * kProbeThreads) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * kProbeThreads);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < hi; i += kProbeThreads) {
    const u32x4 a = __builtin_nontemporal_load(buf + i);
    x ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  sink[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = x;
}
}  // namespace

namespace pa_internal {

int launch_reshape_and_cache(const CacheLaunch &a) {
  hipStream_t st = reinterpret_cast<hipStream_t>(a.stream);
  const int row_chunks = a.head_dim * a.elem_bytes / 16;
  hipLaunchKernelGGL(pa_reshape_and_cache, dim3(a.num_tokens), dim3(256), 0, st,
                     reinterpret_cast<const u32x4 *>(a.k), reinterpret_cast<const u32x4 *>(a.v),
                     reinterpret_cast<u32x4 *>(a.k_pool), reinterpret_cast<u32x4 *>(a.v_pool),
                     a.slot_mapping, a.num_kv_heads, row_chunks, a.block_size,
                     (int64_t)a.num_blocks * a.block_size);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

size_t hbm_probe_sink_bytes() { return (size_t)kProbeBlocks * kProbeThreads * 4; }

int launch_hbm_probe(const void *buf, size_t bytes, void *sink, void *stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const size_t n16 = bytes / 16;
  hipLaunchKernelGGL(pa_hbm_probe, dim3(kProbeBlocks), dim3(kProbeThreads), 0, st,
                     reinterpret_cast<const u32x4 *>(buf), n16,
                     (n16 + kProbeBlocks - 1) / kProbeBlocks, reinterpret_cast<uint32_t *>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

}  // namespace pa_internal
