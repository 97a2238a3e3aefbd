// One new token's K and V rows into their cache slot: the body of the cache
// write, shared by the cache-write kernel and the decode step's preparation
// kernel (which writes the step's tokens beside its work plan).
#pragma once

#include "pagedattn_device.h"

namespace pa_dev {

// Threads that copy one token: 16 bytes each per pass.
constexpr int kCacheThreads = 256;
// Chunks per thread loaded before the slot is known (8 KiB of K and of V per
// token: 32 kv-heads of 128 bf16), so that the source reads and the slot read
// are in flight together.
constexpr int kCacheHeld = 2;

// Token t's rows (num_kv_heads * row_chunks 16-byte chunks each of K and V)
// to page slot / block_size at offset slot % block_size, by the kCacheThreads
// threads tid = 0 .. kCacheThreads - 1.  A slot outside [0, num_slots) writes
// nothing.
__device__ __forceinline__ void cache_write_token(
    int t, int tid, const u32x4 *__restrict__ k, const u32x4 *__restrict__ v,
    u32x4 *__restrict__ k_pool, u32x4 *__restrict__ v_pool,
    const int64_t *__restrict__ slot_mapping, int num_kv_heads, int row_chunks, int block_size,
    int64_t num_slots) {
  const int total = num_kv_heads * row_chunks;
  const u32x4 *k_row = k + (size_t)t * total;
  const u32x4 *v_row = v + (size_t)t * total;
  u32x4 kh[kCacheHeld], vh[kCacheHeld];
#pragma unroll
  for (int i = 0; i < kCacheHeld; ++i) {
    const int c = tid + i * kCacheThreads;
    if (c < total) {
      kh[i] = k_row[c];
      vh[i] = v_row[c];
    }
  }
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t page = slot / block_size;
  const int64_t off = slot - page * block_size;
  // chunk c of the token (kv-head c / row_chunks) to its slot row in that head's page
  auto dst = [&](int c) {
    const int g = c / row_chunks;
    const int dc = c - g * row_chunks;
    return (((size_t)page * num_kv_heads + g) * block_size + off) * row_chunks + dc;
  };
#pragma unroll
  for (int i = 0; i < kCacheHeld; ++i) {
    const int c = tid + i * kCacheThreads;
    if (c < total) {
      k_pool[dst(c)] = kh[i];
      v_pool[dst(c)] = vh[i];
    }
  }
  for (int c = tid + kCacheHeld * kCacheThreads; c < total; c += kCacheThreads) {
    k_pool[dst(c)] = k_row[c];
    v_pool[dst(c)] = v_row[c];
  }
}

}  // namespace pa_dev
