// Internal interface of the multi-token (prefill) attention between the
// host-side C ABI and its HIP launch code, kept apart from the decode
// interface so the two kernels' sources change independently.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace pa_internal {

// query rows of a prefill work item (token x head of one kv-head's group),
// and ints per prefill plan item: (sequence, first chunk token, partition,
// chunk's first row, chunk length, position of chunk token 0, whether every
// page the item reads lies in the pool, unused)
constexpr int kPrefillRows = 256;
constexpr int kPrefillPlanRecord = 8;
// keys of a prefill LDS tile; split-K partitions are whole tiles
constexpr int kPrefillKeyTile = 128;

struct PrefillLaunch {
  void *out;
  const void *q;
  const void *k_pool;
  const void *v_pool;
  const int32_t *block_tables;
  const int32_t *context_lens;
  const int32_t *query_start;  // [num_seqs + 1]
  int32_t *plan;               // item list written by the plan kernel
  int32_t *nparts;             // [num_tokens] key partitions of each row's block
  float *ws_ml;                // [num_tokens, num_heads, max_parts, 2]
  float *ws_acc;               // [num_tokens, num_heads, max_parts, head_dim]
  int part_tokens = 0;         // keys per partition (whole key tiles), 0: no split
  int max_parts = 1;
  int num_seqs, num_tokens, num_heads, num_kv_heads, head_dim, block_size;
  int max_blocks, num_blocks;
  float scale;
  void *stream;
  void *ev_begin;
  void *ev_end;
  const float *alibi = nullptr;  // [num_heads] ALiBi slopes, or none
};

// multi-token attention: plan kernel, then the persistent item pass
int launch_prefill(const PrefillLaunch &a);

}  // namespace pa_internal
