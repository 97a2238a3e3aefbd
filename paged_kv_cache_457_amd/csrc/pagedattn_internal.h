// Internal interface between the host-side C ABI (argument checks) and the
// HIP launch code.  Not installed; the public interface is include/pagedattn.h.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace pa_internal {

// Partitions are dealt to 4 wavefronts per workgroup, each holding one page
// id per lane.
constexpr int kMaxPartitionPages = 4 * 64;
// The plan: int32 [kPlanHeader + num_seqs * max_parts]; element 0 is the
// number of units, then one (sequence * max_parts + partition) per unit.
constexpr int kPlanHeader = 4;
constexpr int kMaxDevices = 64;
// Shared-prefix decode: query rows (members x heads of a group) one prefix
// unit serves, and the ints of one unit record in the plan.
constexpr int kPrefixRows = 32;
constexpr int kPrefixUnitInts = 5;

struct DecodeLaunch {
  void *out;
  const void *q;
  const void *k_pool;
  const void *v_pool;
  const int32_t *block_tables;
  const int32_t *context_lens;
  int32_t *plan;  // unit list written by the plan kernel
  // Partials, partition-major within a sequence: the rows one partition
  // of a sequence writes are adjacent.
  float *ws_ml;   // [S, max_parts, H, 2] (running max in log2 units, sum)
  float *ws_acc;  // [S, max_parts, H, D] unnormalised weighted V
  int num_seqs, num_heads, num_kv_heads, head_dim, block_size;
  int max_blocks, num_blocks, dtype;
  int part_pages;  // pages per partition (<= 64)
  int max_parts;   // ceil(max_blocks / part_pages)
  // partitions one item covers in the one-wave-per-item grouped-query form
  // (consecutive partitions of one sequence and kv-head, streamed by one
  // wave); 1 everywhere else.  The plan lists items of chain * part_pages
  // pages.
  int chain = 1;
  float scale;
  void *stream;
  void *ev_begin;
  void *ev_end;
  const float *alibi = nullptr;  // [num_heads] ALiBi slopes, or none
};

struct PrefixLaunch {
  DecodeLaunch base;            // max_parts holds the partial slots per sequence
  const int32_t *group_starts;  // [num_groups + 1]
  const int32_t *prefix_lens;   // [num_groups]
  int num_groups;
  int32_t *nslots;              // [num_seqs] slots each sequence fills
  int32_t *seq_pre;             // [num_seqs] shared prefix pages of its group
  long long max_units;          // bound on the plan's units
};

struct CacheLaunch {
  const void *k;
  const void *v;
  void *k_pool;
  void *v_pool;
  const int64_t *slot_mapping;
  int num_tokens, num_kv_heads, head_dim, block_size, num_blocks, elem_bytes;
  void *stream;
};

struct RopeLaunch {
  CacheLaunch cache;          // k, v, pools, slots, shapes, stream
  void *q;                    // [num_tokens, num_heads, head_dim], rotated in place
  const int64_t *positions;   // [num_tokens]
  const float *cos_sin;       // [max_position, rot_dim]: cosines, then sines
  int num_heads, rot_dim, max_position, neox;
};

struct CopyLaunch {
  const void *k_src;
  const void *v_src;
  void *k_dst;
  void *v_dst;
  const int64_t *mapping;  // [num_pairs, 2] (source page, destination page)
  int num_pairs;
  int64_t page_bytes;      // bytes of one page of one pool, all kv-heads
  int src_blocks, dst_blocks;
  void *stream;
};

// Each returns 0 on success or the PA_ERR_HIP code on a launch error.
int launch_decode(const DecodeLaunch &a);
// The partition pass for bf16 with 2, 4 or 8 query heads per kv-head, on
// the matrix cores; called by launch_decode.
int launch_partition_gqa(const DecodeLaunch &a, float scale_log2);
// Partitions per item of a decode call (DecodeLaunch::chain).
int decode_chain(const DecodeLaunch &a);
// Workgroups of `kernel` one compute unit holds at once (at least 1).
int blocks_per_cu(const void *kernel, int block_threads);
// Grid of a persistent kernel: what the current device holds at once
// (per_cu workgroups per compute unit), capped by the number of work items;
// 0 on a runtime error.
unsigned persistent_grid_items(long long items, int per_cu);
// Grid of the decode partition kernels: up to kDecodeGridRounds times what
// the device holds at once, capped by the bound on their items.  Past the
// resident workgroups the hardware dispatcher hands the largest-first list
// out as workgroups finish (measured on MI355X 3-10% faster than one
// persistent round for batches of unevenly long sequences); the cap bounds
// the workgroups that find no unit when few of the bound's units exist.
constexpr int kDecodeGridRounds = 8;
unsigned decode_grid(const DecodeLaunch &a, int per_cu);
// Shared-prefix decode: plan, unit pass and the final merge.
int launch_decode_shared_prefix(const PrefixLaunch &p);
int launch_prefix_plan(const PrefixLaunch &p);
int launch_prefix_units(const PrefixLaunch &p, float scale_log2);
int launch_reshape_and_cache(const CacheLaunch &a);
int launch_reshape_and_cache_rope(const RopeLaunch &r);
// Also PA_ERR_UNSUPPORTED (3) when a pointer is not device-accessible.
int launch_copy_pages(const CopyLaunch &a);
int launch_hbm_probe(const void *buf, size_t bytes, void *sink, void *stream);
size_t hbm_probe_sink_bytes();

}  // namespace pa_internal
