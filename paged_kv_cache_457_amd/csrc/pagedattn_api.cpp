// Host side of the C ABI declared in include/pagedattn.h: argument checks
// (all before any HIP call, so every rejection is testable without a GPU),
// workspace sizing, and hand-off to the launch code.
#include "pagedattn.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <vector>

#include "pagedattn_internal.h"
#include "pagedattn_probe_launch.h"
#include "pagedattn_step_launch.h"
#include "pagedattn_prefill_launch.h"
#include "pagedattn_runtime.h"

namespace {

// Default split (partition_size 0): the whole table when it holds at most
// kSinglePartitionTokens tokens; else the largest of 2048, 1024, 512, 256
// tokens that still gives at least kMinUnits (sequence, partition) units, so
// that a small batch of long sequences keeps every compute unit busy while a
// large batch reads long runs per unit (measured on MI355X: 2048-token
// partitions beat 1024 by 3% at 256 lognormal sequences and by 9% at 8 x
// 32768 tokens; 512 and below lose more).
constexpr int kMaxDefaultPartitionTokens = 2048;
constexpr int kMinDefaultPartitionTokens = 256;
constexpr int64_t kMinUnits = 128;
using pa_internal::kMaxPartitionPages;
using pa_internal::kPlanHeader;
static_assert(pa_internal::kNoallocScratchBytes == PA_NOALLOC_SCRATCH_BYTES,
              "the static scratch is the size the header states");

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool supported_dim(int d) { return d == 64 || d == 128; }
bool supported_bs(int bs) { return bs == 16 || bs == 32; }
bool supported_group(int g) { return g == 1 || g == 2 || g == 4 || g == 8; }
int elem_bytes(int dtype) { return dtype == PA_DTYPE_F32 ? 4 : 2; }

constexpr int kSinglePartitionTokens = 2048;  // one pass, no reduce launch

int partition_tokens(const pa_decode_dims *d, int32_t block_size) {
  if (d->partition_size != 0) return d->partition_size;
  const int64_t table_tokens = (int64_t)d->max_blocks_per_seq * block_size;
  if (table_tokens <= kSinglePartitionTokens) return (int)table_tokens;
  int pt = kMaxDefaultPartitionTokens;
  while (pt > kMinDefaultPartitionTokens &&
         (int64_t)d->num_seqs * ((table_tokens + pt - 1) / pt) < kMinUnits)
    pt /= 2;
  return pt;
}

// Shape checks that do not involve the kv-head count (the workspace and
// partition queries, which do not take it, apply only these).
int check_decode_shape(int32_t block_size, const pa_decode_dims *d) {
  if (!d) return PA_ERR_NULL;
  if (d->num_seqs < 0 || d->num_heads < 1 || d->max_blocks_per_seq < 1 || d->num_blocks < 1 ||
      d->reserved != 0 || d->partition_size < 0)
    return PA_ERR_SHAPE;
  if (d->dtype != PA_DTYPE_F32 && d->dtype != PA_DTYPE_BF16) return PA_ERR_UNSUPPORTED;
  if (!supported_dim(d->head_dim) || !supported_bs(block_size)) return PA_ERR_UNSUPPORTED;
  // context capacity must fit in int32 token counts
  if ((int64_t)d->max_blocks_per_seq * block_size > INT32_MAX) return PA_ERR_SHAPE;
  const int pt = partition_tokens(d, block_size);
  if (pt % block_size != 0 || pt / block_size > kMaxPartitionPages) return PA_ERR_SHAPE;
  return PA_OK;
}

// Shape checks of a decode call: the above, the head group, and the int32
// count of (sequence, partition, kv-head) work items.
int check_decode_dims(int32_t num_kv_heads, int32_t block_size, const pa_decode_dims *d) {
  const int rc = check_decode_shape(block_size, d);
  if (rc != PA_OK) return rc;
  if (num_kv_heads < 1 || d->num_heads % num_kv_heads != 0) return PA_ERR_SHAPE;
  if (!supported_group(d->num_heads / num_kv_heads)) return PA_ERR_UNSUPPORTED;
  const int pt = partition_tokens(d, block_size);
  const int64_t parts = ((int64_t)d->max_blocks_per_seq * block_size + pt - 1) / pt;
  if ((int64_t)d->num_seqs * parts * num_kv_heads > INT32_MAX) return PA_ERR_SHAPE;
  return PA_OK;
}

int max_partitions(int32_t block_size, const pa_decode_dims *d) {
  const int pp = partition_tokens(d, block_size) / block_size;
  return (d->max_blocks_per_seq + pp - 1) / pp;
}

// Workspace layout: the unit plan (int32, rounded up to 256 bytes), then,
// when a sequence can span more than one partition, the partials:
// fp32 accumulators [S, P, H, D] followed by (max, sum) pairs [S, P, H, 2].
size_t plan_bytes(int num_seqs, int parts) {
  const size_t b = ((size_t)kPlanHeader + (size_t)num_seqs * parts) * sizeof(int32_t);
  return (b + 255) / 256 * 256;
}
size_t partial_bytes(const pa_decode_dims *d, int parts) {
  if (parts <= 1) return 0;
  return (size_t)d->num_seqs * d->num_heads * parts * (size_t)(d->head_dim + 2) * sizeof(float);
}

// Shared-prefix decode: the default partition is kSharedPartitionTokens (a
// group's prefix unit is one long read, so it is split finer than plain
// decode splits a sequence).  Slots per sequence are prefix partitions
// then own-page partitions, each at most ceil(max_blocks / partition pages).
constexpr int kSharedPartitionTokens = 512;

int shared_partition_tokens(const pa_decode_dims *d, int32_t block_size) {
  if (d->partition_size != 0) return d->partition_size;
  const int64_t table_tokens = (int64_t)d->max_blocks_per_seq * block_size;
  return (int)(table_tokens < kSharedPartitionTokens ? table_tokens : kSharedPartitionTokens);
}
int prefix_slots(int32_t block_size, const pa_decode_dims *d) {
  const int pp = shared_partition_tokens(d, block_size) / block_size;
  return 2 * ((d->max_blocks_per_seq + pp - 1) / pp);
}
size_t prefix_plan_ints(int num_seqs, int slots) {
  return (size_t)kPlanHeader + (size_t)pa_internal::kPrefixUnitInts * num_seqs * slots +
         2 * (size_t)num_seqs;
}
size_t prefix_workspace_bytes(int32_t block_size, const pa_decode_dims *d) {
  const int ms = prefix_slots(block_size, d);
  const size_t plan = (prefix_plan_ints(d->num_seqs, ms) * sizeof(int32_t) + 255) / 256 * 256;
  return plan + (size_t)d->num_seqs * d->num_heads * ms * (size_t)(d->head_dim + 2) * sizeof(float);
}

// Prefill split-K default: enough (block, kv-head) items to keep every CU
// busy several rounds without splitting, else partitions that reach that
// many, of at least kMinPrefillPartition keys.
constexpr int64_t kPrefillTargetItems = 1024;
constexpr int kMinPrefillPartition = 1024;

int prefill_partition_tokens(int32_t num_kv_heads, int32_t block_size, const pa_prefill_dims *d) {
  const int64_t cap = (int64_t)d->max_blocks_per_seq * block_size;
  if (d->partition_size != 0) return d->partition_size >= cap ? 0 : d->partition_size;
  const int tok = pa_internal::kPrefillRows / (d->num_heads / num_kv_heads);
  const int64_t items = ((int64_t)d->num_tokens + tok - 1) / tok * num_kv_heads;
  if (items >= kPrefillTargetItems || items == 0) return 0;
  const int64_t parts = (kPrefillTargetItems + items - 1) / items;
  constexpr int64_t tile = pa_internal::kPrefillKeyTile;
  int64_t kp = ((cap + parts - 1) / parts + tile - 1) / tile * tile;
  if (kp < kMinPrefillPartition) kp = kMinPrefillPartition;
  return kp >= cap ? 0 : (int)kp;
}

int prefill_max_parts(int32_t num_kv_heads, int32_t block_size, const pa_prefill_dims *d) {
  const int pt = prefill_partition_tokens(num_kv_heads, block_size, d);
  const int64_t cap = (int64_t)d->max_blocks_per_seq * block_size;
  return pt ? (int)((cap + pt - 1) / pt) : 1;
}

// Shape checks shared by the prefill call and its workspace query.
int check_prefill_dims(int32_t num_kv_heads, int32_t block_size, const pa_prefill_dims *d) {
  if (!d) return PA_ERR_NULL;
  if (d->num_seqs < 0 || d->num_tokens < 0 || d->num_heads < 1 || num_kv_heads < 1 ||
      d->max_blocks_per_seq < 1 || d->num_blocks < 1 || d->partition_size < 0 ||
      d->partition_size % pa_internal::kPrefillKeyTile != 0)
    return PA_ERR_SHAPE;
  if (d->num_heads % num_kv_heads != 0) return PA_ERR_SHAPE;
  if (d->dtype != PA_DTYPE_BF16) return PA_ERR_UNSUPPORTED;  // matrix cores: bf16 only
  if (!supported_dim(d->head_dim) || !supported_bs(block_size) ||
      !supported_group(d->num_heads / num_kv_heads))
    return PA_ERR_UNSUPPORTED;
  if ((int64_t)d->max_blocks_per_seq * block_size > INT32_MAX) return PA_ERR_SHAPE;
  // rows of a sequence cannot exist without the sequence
  if (d->num_tokens > 0 && d->num_seqs == 0) return PA_ERR_SHAPE;
  // work items (block, partition, kv-head) are int32; there are at most
  // num_tokens * partitions of them
  const int64_t parts = prefill_max_parts(num_kv_heads, block_size, d);
  if ((int64_t)d->num_tokens * parts * num_kv_heads > INT32_MAX) return PA_ERR_SHAPE;
  return PA_OK;
}

size_t prefill_plan_bytes(int num_tokens, int parts) {
  const size_t ints = (size_t)kPlanHeader +
                      (size_t)pa_internal::kPrefillPlanRecord * num_tokens * parts + num_tokens;
  return (ints * sizeof(int32_t) + 255) / 256 * 256;
}

size_t prefill_workspace_bytes(int32_t num_kv_heads, int32_t block_size, const pa_prefill_dims *d) {
  const int parts = prefill_max_parts(num_kv_heads, block_size, d);
  size_t b = prefill_plan_bytes(d->num_tokens, parts);
  if (parts > 1)
    b += (size_t)d->num_tokens * d->num_heads * parts * (d->head_dim + 2) * sizeof(float);
  return b;
}

// ---------------------------------------------------------------------------
// PA_DEBUG_CHECKS=1: the device-side preconditions the kernels do not check
// (they skip or clamp instead), read back and checked on the host.  Debug
// only: each check copies the tables it needs to pageable host memory and
// waits for the stream, so it is not for graph capture or timing.  A
// violation returns PA_ERR_PRECONDITION and nothing is launched.
bool debug_checks() {
  const char *e = std::getenv("PA_DEBUG_CHECKS");
  return e && e[0] == '1' && e[1] == '\0';
}

template <class T>
bool read_back(std::vector<T> &dst, const T *src, size_t n, void *stream) {
  dst.resize(n);
  return pa_internal::copy_to_host_sync(dst.data(), src, n * sizeof(T), stream) == 0;
}

// Context lengths in [0, max_blocks * block_size]; the page ids a context
// uses (its first ceil(ctx / block_size) table entries) in [0, num_blocks).
int check_tables(const int32_t *block_tables, const int32_t *context_lens, int num_seqs,
                 int max_blocks, int num_blocks, int block_size, void *stream) {
  std::vector<int32_t> ctx, bt;
  if (!read_back(ctx, context_lens, num_seqs, stream) ||
      !read_back(bt, block_tables, (size_t)num_seqs * max_blocks, stream))
    return PA_ERR_HIP;
  const int64_t cap = (int64_t)max_blocks * block_size;
  for (int s = 0; s < num_seqs; ++s) {
    if (ctx[s] < 0 || ctx[s] > cap) return PA_ERR_PRECONDITION;
    const int64_t used = ((int64_t)ctx[s] + block_size - 1) / block_size;
    for (int64_t j = 0; j < used; ++j) {
      const int32_t b = bt[(size_t)s * max_blocks + j];
      if (b < 0 || b >= num_blocks) return PA_ERR_PRECONDITION;
    }
  }
  return PA_OK;
}

// Slots negative (no token) or in [0, num_blocks * block_size), and the
// non-negative ones distinct.
int check_slots(const int64_t *slot_mapping, int num_tokens, int num_blocks, int block_size,
                void *stream) {
  std::vector<int64_t> sl;
  if (!read_back(sl, slot_mapping, num_tokens, stream)) return PA_ERR_HIP;
  const int64_t slots = (int64_t)num_blocks * block_size;
  std::vector<int64_t> used;
  used.reserve(sl.size());
  for (const int64_t x : sl) {
    if (x < 0) continue;
    if (x >= slots) return PA_ERR_PRECONDITION;
    used.push_back(x);
  }
  std::sort(used.begin(), used.end());
  return std::adjacent_find(used.begin(), used.end()) == used.end() ? PA_OK
                                                                     : PA_ERR_PRECONDITION;
}

// Sharing groups: group_starts runs from 0 to num_seqs without decreasing;
// prefix_lens in [0, max_blocks * block_size]; the members of a group hold
// the same page ids in the prefix's whole pages, and those ids are in the
// pool (the prefix units read them through the group's first member).
int check_groups(const int32_t *group_starts, const int32_t *prefix_lens, int num_groups,
                 const int32_t *block_tables, int num_seqs, int max_blocks, int num_blocks,
                 int block_size, void *stream) {
  std::vector<int32_t> gs, pl, bt;
  if (!read_back(gs, group_starts, (size_t)num_groups + 1, stream) ||
      !read_back(pl, prefix_lens, num_groups, stream) ||
      !read_back(bt, block_tables, (size_t)num_seqs * max_blocks, stream))
    return PA_ERR_HIP;
  if (gs[0] != 0 || gs[num_groups] != num_seqs) return PA_ERR_PRECONDITION;
  for (int i = 0; i < num_groups; ++i) {
    if (gs[i + 1] < gs[i]) return PA_ERR_PRECONDITION;
    if (pl[i] < 0 || (int64_t)pl[i] > (int64_t)max_blocks * block_size)
      return PA_ERR_PRECONDITION;
    if (gs[i + 1] == gs[i]) continue;
    const int pages = pl[i] / block_size;
    const int32_t *first = &bt[(size_t)gs[i] * max_blocks];
    for (int j = 0; j < pages; ++j)
      if (first[j] < 0 || first[j] >= num_blocks) return PA_ERR_PRECONDITION;
    for (int m = gs[i] + 1; m < gs[i + 1]; ++m)
      if (!std::equal(first, first + pages, &bt[(size_t)m * max_blocks]))
        return PA_ERR_PRECONDITION;
  }
  return PA_OK;
}

// query_start runs from 0 to num_tokens without decreasing.
int check_query_start(const int32_t *query_start, int num_seqs, int num_tokens, void *stream) {
  std::vector<int32_t> qs;
  if (!read_back(qs, query_start, (size_t)num_seqs + 1, stream)) return PA_ERR_HIP;
  if (qs[0] != 0 || qs[num_seqs] != num_tokens) return PA_ERR_PRECONDITION;
  for (int s = 0; s < num_seqs; ++s)
    if (qs[s + 1] < qs[s]) return PA_ERR_PRECONDITION;
  return PA_OK;
}

// Page copies: no two pairs that are carried out (both pages inside their
// pools) name the same destination; within one pool no destination is also
// a source.
int check_copy_pairs(const int64_t *mapping, int num_pairs, int src_blocks, int dst_blocks,
                     bool same_pool, void *stream) {
  std::vector<int64_t> m;
  if (!read_back(m, mapping, (size_t)num_pairs * 2, stream)) return PA_ERR_HIP;
  std::vector<int64_t> src, dst;
  for (int i = 0; i < num_pairs; ++i) {
    const int64_t a = m[2 * (size_t)i], b = m[2 * (size_t)i + 1];
    if (a < 0 || a >= src_blocks || b < 0 || b >= dst_blocks) continue;  // skipped pair
    src.push_back(a);
    dst.push_back(b);
  }
  std::sort(dst.begin(), dst.end());
  if (std::adjacent_find(dst.begin(), dst.end()) != dst.end()) return PA_ERR_PRECONDITION;
  if (same_pool)
    for (const int64_t a : src)
      if (std::binary_search(dst.begin(), dst.end(), a)) return PA_ERR_PRECONDITION;
  return PA_OK;
}

// Where a decode call's work plan and split-K partials go: the caller's
// workspace, or the library's static device scratch.
enum class Workspace { kCaller, kStatic };

// cache: the decode step's new tokens (paged_attention_decode_step), written
// to the pools before the attention; its pointers are already checked.
int decode_impl(void *out, const void *q, const void *k_pool, const void *v_pool,
                const int32_t *block_tables, const int32_t *context_lens, int32_t num_kv_heads,
                float scale, int32_t block_size, const float *alibi, const pa_decode_dims *dims,
                bool read_probe = false, Workspace where = Workspace::kCaller,
                const pa_internal::CacheLaunch *cache = nullptr);
// cache: the step's chunk rows (paged_attention_prefill_step), written to
// the pools before the attention; its pointers are already checked.
int prefill_impl(void *out, const void *q, const void *k_pool, const void *v_pool,
                 const int32_t *block_tables, const int32_t *context_lens,
                 const int32_t *query_start, int32_t num_kv_heads, float scale,
                 int32_t block_size, const float *alibi, const pa_prefill_dims *dims,
                 const pa_internal::CacheLaunch *cache = nullptr);

// The cache write of a decode step's entry (one new token per sequence):
// checks its pointers and fills c; shape checks are the decode call's.
int step_cache(pa_internal::CacheLaunch *c, const void *k, const void *v,
               const int64_t *slot_mapping, void *k_pool, void *v_pool, int32_t num_kv_heads,
               int32_t block_size, const pa_decode_dims *dims) {
  const int rc = check_decode_dims(num_kv_heads, block_size, dims);
  if (rc != PA_OK) return rc;
  if (dims->num_seqs > 0) {
    if (!k || !v || !slot_mapping) return PA_ERR_NULL;
    if (!aligned(k, 16) || !aligned(v, 16) || !aligned(slot_mapping, 8)) return PA_ERR_ALIGN;
  }
  c->k = k;
  c->v = v;
  c->k_pool = k_pool;
  c->v_pool = v_pool;
  c->slot_mapping = slot_mapping;
  c->num_tokens = dims->num_seqs;
  c->num_kv_heads = num_kv_heads;
  c->head_dim = dims->head_dim;
  c->block_size = block_size;
  c->num_blocks = dims->num_blocks;
  c->elem_bytes = elem_bytes(dims->dtype);
  c->stream = dims->stream;
  return PA_OK;
}

// cache: the step's new tokens (paged_attention_decode_shared_prefix_step),
// written to the pools before the attention; its pointers are already checked.
int shared_prefix_impl(void *out, const void *q, const void *k_pool, const void *v_pool,
                       const int32_t *block_tables, const int32_t *context_lens,
                       int32_t num_kv_heads, float scale, int32_t block_size,
                       const int32_t *group_starts, const int32_t *prefix_lens,
                       int32_t num_groups, const pa_decode_dims *dims,
                       const pa_internal::CacheLaunch *cache) {
  if (!dims) return PA_ERR_NULL;
  int rc = check_decode_dims(num_kv_heads, block_size, dims);
  if (rc != PA_OK) return rc;
  if (dims->dtype != PA_DTYPE_BF16) return PA_ERR_UNSUPPORTED;  // matrix cores: bf16 only
  if (!std::isfinite(scale) || num_groups < 0) return PA_ERR_SHAPE;
  const int ms = prefix_slots(block_size, dims);
  if ((int64_t)dims->num_seqs * ms * num_kv_heads > INT32_MAX) return PA_ERR_SHAPE;
  if (dims->num_seqs == 0) return PA_OK;
  if (num_groups < 1) return PA_ERR_SHAPE;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens || !group_starts ||
      !prefix_lens)
    return PA_ERR_NULL;
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(group_starts, 4) ||
      !aligned(prefix_lens, 4))
    return PA_ERR_ALIGN;
  if (!dims->workspace || dims->workspace_bytes < prefix_workspace_bytes(block_size, dims) ||
      !aligned(dims->workspace, 16))
    return PA_ERR_WORKSPACE;
  if (debug_checks()) {
    rc = check_tables(block_tables, context_lens, dims->num_seqs, dims->max_blocks_per_seq,
                      dims->num_blocks, block_size, dims->stream);
    if (rc == PA_OK)
      rc = check_groups(group_starts, prefix_lens, num_groups, block_tables, dims->num_seqs,
                        dims->max_blocks_per_seq, dims->num_blocks, block_size, dims->stream);
    if (rc == PA_OK && cache)
      rc = check_slots(cache->slot_mapping, cache->num_tokens, dims->num_blocks, block_size,
                       dims->stream);
    if (rc != PA_OK) return rc;
  }
  int32_t *plan = static_cast<int32_t *>(dims->workspace);
  const size_t plan_ints = prefix_plan_ints(dims->num_seqs, ms);
  const size_t plan_bytes = (plan_ints * sizeof(int32_t) + 255) / 256 * 256;
  float *ws_acc = reinterpret_cast<float *>(static_cast<char *>(dims->workspace) + plan_bytes);

  pa_internal::PrefixLaunch p{};
  pa_internal::DecodeLaunch &a = p.base;
  a.out = out;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.plan = plan;
  a.ws_acc = ws_acc;
  a.ws_ml = ws_acc + (size_t)dims->num_seqs * dims->num_heads * ms * dims->head_dim;
  a.num_seqs = dims->num_seqs;
  a.num_heads = dims->num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = dims->head_dim;
  a.block_size = block_size;
  a.max_blocks = dims->max_blocks_per_seq;
  a.num_blocks = dims->num_blocks;
  a.dtype = dims->dtype;
  a.part_pages = shared_partition_tokens(dims, block_size) / block_size;
  a.max_parts = ms;
  a.scale = scale;
  a.stream = dims->stream;
  a.ev_begin = dims->timing_events[0];
  a.ev_end = dims->timing_events[1];
  p.group_starts = group_starts;
  p.prefix_lens = prefix_lens;
  p.num_groups = num_groups;
  p.nslots = plan + kPlanHeader + (size_t)pa_internal::kPrefixUnitInts * dims->num_seqs * ms;
  p.seq_pre = p.nslots + dims->num_seqs;
  p.max_units = (long long)dims->num_seqs * ms;
  return cache ? pa_internal::launch_shared_prefix_step(p, *cache)
               : pa_internal::launch_decode_shared_prefix(p);
}

}  // namespace

extern "C" {

size_t paged_attention_decode_workspace_bytes(int32_t block_size, const pa_decode_dims *dims) {
  // The size does not depend on the kv-head count, which the query does
  // not take; the call itself checks the head group and the item count.
  if (check_decode_shape(block_size, dims) != PA_OK) return SIZE_MAX;
  if (dims->num_seqs == 0) return 0;
  const int mp = max_partitions(block_size, dims);
  return plan_bytes(dims->num_seqs, mp) + partial_bytes(dims, mp);
}

size_t paged_attention_decode_shared_prefix_workspace_bytes(int32_t block_size,
                                                            const pa_decode_dims *dims) {
  if (check_decode_shape(block_size, dims) != PA_OK) return SIZE_MAX;
  if (dims->num_seqs == 0) return 0;
  return prefix_workspace_bytes(block_size, dims);
}

int paged_attention_decode_shared_prefix(void *out, const void *q, const void *k_pool,
                                         const void *v_pool, const int32_t *block_tables,
                                         const int32_t *context_lens, int32_t num_kv_heads,
                                         float scale, int32_t block_size,
                                         const int32_t *group_starts,
                                         const int32_t *prefix_lens, int32_t num_groups,
                                         const pa_decode_dims *dims) {
  return shared_prefix_impl(out, q, k_pool, v_pool, block_tables, context_lens, num_kv_heads,
                            scale, block_size, group_starts, prefix_lens, num_groups, dims,
                            nullptr);
}

int paged_attention_decode_shared_prefix_step(
    void *out, const void *q, const void *k, const void *v, const int64_t *slot_mapping,
    void *k_pool, void *v_pool, const int32_t *block_tables, const int32_t *context_lens,
    int32_t num_kv_heads, float scale, int32_t block_size, const int32_t *group_starts,
    const int32_t *prefix_lens, int32_t num_groups, const pa_decode_dims *dims) {
  if (!dims) return PA_ERR_NULL;
  pa_internal::CacheLaunch c{};
  const int rc = step_cache(&c, k, v, slot_mapping, k_pool, v_pool, num_kv_heads, block_size,
                            dims);
  if (rc != PA_OK) return rc;
  return shared_prefix_impl(out, q, k_pool, v_pool, block_tables, context_lens, num_kv_heads,
                            scale, block_size, group_starts, prefix_lens, num_groups, dims, &c);
}

int32_t paged_attention_decode_partition_tokens(int32_t block_size, const pa_decode_dims *dims) {
  if (check_decode_shape(block_size, dims) != PA_OK) return -1;
  return partition_tokens(dims, block_size);
}

int paged_attention_decode(void *out, const void *q, const void *k_pool, const void *v_pool,
                           const int32_t *block_tables, const int32_t *context_lens,
                           int32_t num_kv_heads, float scale, int32_t block_size,
                           const pa_decode_dims *dims) {
  return decode_impl(out, q, k_pool, v_pool, block_tables, context_lens, num_kv_heads, scale,
                     block_size, nullptr, dims);
}

int paged_attention_decode_noalloc(void *out, const void *q, const void *k_pool,
                                   const void *v_pool, const int32_t *block_tables,
                                   const int32_t *context_lens, int32_t num_kv_heads, float scale,
                                   int32_t block_size, const pa_decode_dims *dims) {
  return decode_impl(out, q, k_pool, v_pool, block_tables, context_lens, num_kv_heads, scale,
                     block_size, nullptr, dims, false, Workspace::kStatic);
}

int paged_attention_decode_alibi(void *out, const void *q, const void *k_pool,
                                 const void *v_pool, const int32_t *block_tables,
                                 const int32_t *context_lens, int32_t num_kv_heads, float scale,
                                 int32_t block_size, const float *alibi_slopes,
                                 const pa_decode_dims *dims) {
  if (!dims) return PA_ERR_NULL;
  const int rc = check_decode_dims(num_kv_heads, block_size, dims);
  if (rc != PA_OK) return rc;
  if (dims->num_seqs > 0 && !alibi_slopes) return PA_ERR_NULL;
  if (!aligned(alibi_slopes, 4)) return PA_ERR_ALIGN;
  return decode_impl(out, q, k_pool, v_pool, block_tables, context_lens, num_kv_heads, scale,
                     block_size, alibi_slopes, dims);
}

int paged_attention_decode_step(void *out, const void *q, const void *k, const void *v,
                                const int64_t *slot_mapping, void *k_pool, void *v_pool,
                                const int32_t *block_tables, const int32_t *context_lens,
                                int32_t num_kv_heads, float scale, int32_t block_size,
                                const pa_decode_dims *dims) {
  if (!dims) return PA_ERR_NULL;
  pa_internal::CacheLaunch c{};
  const int rc = step_cache(&c, k, v, slot_mapping, k_pool, v_pool, num_kv_heads, block_size,
                            dims);
  if (rc != PA_OK) return rc;
  return decode_impl(out, q, k_pool, v_pool, block_tables, context_lens, num_kv_heads, scale,
                     block_size, nullptr, dims, false, Workspace::kCaller, &c);
}

int paged_attention_decode_read_probe(void *out, const void *q, const void *k_pool,
                                      const void *v_pool, const int32_t *block_tables,
                                      const int32_t *context_lens, int32_t num_kv_heads,
                                      float scale, int32_t block_size,
                                      const pa_decode_dims *dims) {
  return decode_impl(out, q, k_pool, v_pool, block_tables, context_lens, num_kv_heads, scale,
                     block_size, nullptr, dims, true);
}

}  // extern "C"

namespace {

int decode_impl(void *out, const void *q, const void *k_pool, const void *v_pool,
                const int32_t *block_tables, const int32_t *context_lens, int32_t num_kv_heads,
                float scale, int32_t block_size, const float *alibi, const pa_decode_dims *dims,
                bool read_probe, Workspace where, const pa_internal::CacheLaunch *cache) {
  if (!dims) return PA_ERR_NULL;
  int rc = check_decode_dims(num_kv_heads, block_size, dims);
  if (rc != PA_OK) return rc;
  if (!std::isfinite(scale)) return PA_ERR_SHAPE;
  // the static scratch replaces the workspace: a caller's one is an error
  if (where == Workspace::kStatic && (dims->workspace || dims->workspace_bytes))
    return PA_ERR_WORKSPACE;
  if (dims->num_seqs == 0) return PA_OK;  // nothing is read or written; pointers may be NULL
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens) return PA_ERR_NULL;
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4))
    return PA_ERR_ALIGN;
  const int mp = max_partitions(block_size, dims);
  const size_t pb = plan_bytes(dims->num_seqs, mp);
  const size_t need = pb + partial_bytes(dims, mp);
  if (where == Workspace::kStatic && need > pa_internal::kNoallocScratchBytes)
    return PA_ERR_SCRATCH_LIMIT;
  if (where == Workspace::kCaller &&
      (!dims->workspace || dims->workspace_bytes < need || !aligned(dims->workspace, 16)))
    return PA_ERR_WORKSPACE;
  if (debug_checks()) {
    rc = check_tables(block_tables, context_lens, dims->num_seqs, dims->max_blocks_per_seq,
                      dims->num_blocks, block_size, dims->stream);
    if (rc == PA_OK && cache)
      rc = check_slots(cache->slot_mapping, cache->num_tokens, dims->num_blocks, block_size,
                       dims->stream);
    if (rc != PA_OK) return rc;
  }
  char *ws = nullptr;
  if (where == Workspace::kStatic) {
    // the scratch's address: the first HIP call of the path (the debug
    // pass aside), after every argument check
    void *p = nullptr;
    if (pa_internal::noalloc_scratch(&p) != 0) return PA_ERR_HIP;
    ws = static_cast<char *>(p);
  } else {
    ws = static_cast<char *>(dims->workspace);
  }
  float *ws_acc = nullptr;
  float *ws_ml = nullptr;
  if (mp > 1) {
    ws_acc = reinterpret_cast<float *>(ws + pb);
    ws_ml = ws_acc + (size_t)dims->num_seqs * dims->num_heads * mp * dims->head_dim;
  }

  pa_internal::DecodeLaunch a{};
  a.out = out;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.plan = reinterpret_cast<int32_t *>(ws);
  a.ws_ml = ws_ml;
  a.ws_acc = ws_acc;
  a.num_seqs = dims->num_seqs;
  a.num_heads = dims->num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = dims->head_dim;
  a.block_size = block_size;
  a.max_blocks = dims->max_blocks_per_seq;
  a.num_blocks = dims->num_blocks;
  a.dtype = dims->dtype;
  a.part_pages = partition_tokens(dims, block_size) / block_size;
  a.max_parts = mp;
  a.scale = scale;
  a.stream = dims->stream;
  a.ev_begin = dims->timing_events[0];
  a.ev_end = dims->timing_events[1];
  a.alibi = alibi;
  if (read_probe) return pa_internal::launch_decode_read_probe(a);
  return cache ? pa_internal::launch_decode_step(a, *cache) : pa_internal::launch_decode(a);
}

}  // namespace

extern "C" {

size_t paged_attention_prefill_workspace_bytes(int32_t num_kv_heads, int32_t block_size,
                                               const pa_prefill_dims *dims) {
  if (check_prefill_dims(num_kv_heads, block_size, dims) != PA_OK) return SIZE_MAX;
  if (dims->num_tokens == 0) return 0;
  return prefill_workspace_bytes(num_kv_heads, block_size, dims);
}

int32_t paged_attention_prefill_partition_tokens(int32_t num_kv_heads, int32_t block_size,
                                                 const pa_prefill_dims *dims) {
  if (check_prefill_dims(num_kv_heads, block_size, dims) != PA_OK) return -1;
  return prefill_partition_tokens(num_kv_heads, block_size, dims);
}

int paged_attention_prefill(void *out, const void *q, const void *k_pool, const void *v_pool,
                            const int32_t *block_tables, const int32_t *context_lens,
                            const int32_t *query_start, int32_t num_kv_heads, float scale,
                            int32_t block_size, const pa_prefill_dims *dims) {
  return prefill_impl(out, q, k_pool, v_pool, block_tables, context_lens, query_start,
                      num_kv_heads, scale, block_size, nullptr, dims);
}

int paged_attention_prefill_alibi(void *out, const void *q, const void *k_pool,
                                  const void *v_pool, const int32_t *block_tables,
                                  const int32_t *context_lens, const int32_t *query_start,
                                  int32_t num_kv_heads, float scale, int32_t block_size,
                                  const float *alibi_slopes, const pa_prefill_dims *dims) {
  if (!dims) return PA_ERR_NULL;
  const int rc = check_prefill_dims(num_kv_heads, block_size, dims);
  if (rc != PA_OK) return rc;
  if (dims->num_tokens > 0 && !alibi_slopes) return PA_ERR_NULL;
  if (!aligned(alibi_slopes, 4)) return PA_ERR_ALIGN;
  return prefill_impl(out, q, k_pool, v_pool, block_tables, context_lens, query_start,
                      num_kv_heads, scale, block_size, alibi_slopes, dims);
}

int paged_attention_prefill_step(void *out, const void *q, const void *k, const void *v,
                                 const int64_t *slot_mapping, void *k_pool, void *v_pool,
                                 const int32_t *block_tables, const int32_t *context_lens,
                                 const int32_t *query_start, int32_t num_kv_heads, float scale,
                                 int32_t block_size, const pa_prefill_dims *dims) {
  if (!dims) return PA_ERR_NULL;
  const int rc = check_prefill_dims(num_kv_heads, block_size, dims);
  if (rc != PA_OK) return rc;
  if (dims->num_tokens > 0) {
    if (!k || !v || !slot_mapping) return PA_ERR_NULL;
    if (!aligned(k, 16) || !aligned(v, 16) || !aligned(slot_mapping, 8)) return PA_ERR_ALIGN;
  }
  pa_internal::CacheLaunch c{};
  c.k = k;
  c.v = v;
  c.k_pool = k_pool;
  c.v_pool = v_pool;
  c.slot_mapping = slot_mapping;
  c.num_tokens = dims->num_tokens;
  c.num_kv_heads = num_kv_heads;
  c.head_dim = dims->head_dim;
  c.block_size = block_size;
  c.num_blocks = dims->num_blocks;
  c.elem_bytes = elem_bytes(dims->dtype);
  c.stream = dims->stream;
  return prefill_impl(out, q, k_pool, v_pool, block_tables, context_lens, query_start,
                      num_kv_heads, scale, block_size, nullptr, dims, &c);
}

}  // extern "C"

namespace {

int prefill_impl(void *out, const void *q, const void *k_pool, const void *v_pool,
                 const int32_t *block_tables, const int32_t *context_lens,
                 const int32_t *query_start, int32_t num_kv_heads, float scale,
                 int32_t block_size, const float *alibi, const pa_prefill_dims *dims,
                 const pa_internal::CacheLaunch *cache) {
  if (!dims) return PA_ERR_NULL;
  int rc = check_prefill_dims(num_kv_heads, block_size, dims);
  if (rc != PA_OK) return rc;
  if (!std::isfinite(scale)) return PA_ERR_SHAPE;
  if (dims->num_tokens == 0) return PA_OK;  // no rows: nothing is read or written
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens || !query_start)
    return PA_ERR_NULL;
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(query_start, 4))
    return PA_ERR_ALIGN;
  if (!dims->workspace ||
      dims->workspace_bytes < prefill_workspace_bytes(num_kv_heads, block_size, dims) ||
      !aligned(dims->workspace, 16))
    return PA_ERR_WORKSPACE;
  if (debug_checks()) {
    rc = check_query_start(query_start, dims->num_seqs, dims->num_tokens, dims->stream);
    if (rc == PA_OK)
      rc = check_tables(block_tables, context_lens, dims->num_seqs, dims->max_blocks_per_seq,
                        dims->num_blocks, block_size, dims->stream);
    if (rc == PA_OK && cache)
      rc = check_slots(cache->slot_mapping, cache->num_tokens, dims->num_blocks, block_size,
                       dims->stream);
    if (rc != PA_OK) return rc;
  }
  const int parts = prefill_max_parts(num_kv_heads, block_size, dims);
  const size_t pb = prefill_plan_bytes(dims->num_tokens, parts);
  pa_internal::PrefillLaunch a{};
  a.out = out;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.plan = static_cast<int32_t *>(dims->workspace);
  a.nparts = a.plan + kPlanHeader +
             (size_t)pa_internal::kPrefillPlanRecord * dims->num_tokens * parts;
  a.part_tokens = prefill_partition_tokens(num_kv_heads, block_size, dims);
  a.max_parts = parts;
  if (parts > 1) {
    a.ws_acc = reinterpret_cast<float *>(static_cast<char *>(dims->workspace) + pb);
    a.ws_ml = a.ws_acc + (size_t)dims->num_tokens * dims->num_heads * parts * dims->head_dim;
  }
  a.num_seqs = dims->num_seqs;
  a.num_tokens = dims->num_tokens;
  a.num_heads = dims->num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = dims->head_dim;
  a.block_size = block_size;
  a.max_blocks = dims->max_blocks_per_seq;
  a.num_blocks = dims->num_blocks;
  a.scale = scale;
  a.stream = dims->stream;
  a.ev_begin = dims->timing_events[0];
  a.ev_end = dims->timing_events[1];
  a.alibi = alibi;
  return cache ? pa_internal::launch_prefill_step(a, *cache) : pa_internal::launch_prefill(a);
}

}  // namespace

extern "C" {

int reshape_and_cache(const void *k, const void *v, void *k_pool, void *v_pool,
                      const int64_t *slot_mapping, const pa_cache_dims *dims) {
  if (!dims) return PA_ERR_NULL;
  if (dims->num_tokens < 0 || dims->num_kv_heads < 1 || dims->num_blocks < 1)
    return PA_ERR_SHAPE;
  if (dims->dtype != PA_DTYPE_F32 && dims->dtype != PA_DTYPE_BF16) return PA_ERR_UNSUPPORTED;
  if (!supported_dim(dims->head_dim) || !supported_bs(dims->block_size))
    return PA_ERR_UNSUPPORTED;
  if (dims->num_tokens == 0) return PA_OK;  // nothing to write; pointers may be NULL
  if (!k || !v || !k_pool || !v_pool || !slot_mapping) return PA_ERR_NULL;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(slot_mapping, 8))
    return PA_ERR_ALIGN;
  if (debug_checks()) {
    const int rc = check_slots(slot_mapping, dims->num_tokens, dims->num_blocks,
                               dims->block_size, dims->stream);
    if (rc != PA_OK) return rc;
  }
  pa_internal::CacheLaunch a{};
  a.k = k;
  a.v = v;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.slot_mapping = slot_mapping;
  a.num_tokens = dims->num_tokens;
  a.num_kv_heads = dims->num_kv_heads;
  a.head_dim = dims->head_dim;
  a.block_size = dims->block_size;
  a.num_blocks = dims->num_blocks;
  a.elem_bytes = elem_bytes(dims->dtype);
  a.stream = dims->stream;
  return pa_internal::launch_reshape_and_cache(a);
}

int reshape_and_cache_rope(void *q, const void *k, const void *v, void *k_pool, void *v_pool,
                           const int64_t *slot_mapping, const int64_t *positions,
                           const float *cos_sin, const pa_rope_dims *rope,
                           const pa_cache_dims *dims) {
  if (!dims || !rope) return PA_ERR_NULL;
  if (dims->num_tokens < 0 || dims->num_kv_heads < 1 || dims->num_blocks < 1 ||
      rope->num_heads < 1 || rope->max_position < 1 || rope->reserved != 0)
    return PA_ERR_SHAPE;
  if (dims->dtype != PA_DTYPE_F32 && dims->dtype != PA_DTYPE_BF16) return PA_ERR_UNSUPPORTED;
  if (!supported_dim(dims->head_dim) || !supported_bs(dims->block_size))
    return PA_ERR_UNSUPPORTED;
  if (rope->is_neox != 0 && rope->is_neox != 1) return PA_ERR_SHAPE;
  // rotary entries: even, within the head, whole 16-byte chunks per half
  const int per_chunk = 16 / elem_bytes(dims->dtype);
  if (rope->rot_dim < 2 || rope->rot_dim > dims->head_dim || rope->rot_dim % 2 != 0)
    return PA_ERR_SHAPE;
  if (rope->rot_dim % (2 * per_chunk) != 0) return PA_ERR_UNSUPPORTED;
  if ((int64_t)rope->max_position * rope->rot_dim > INT32_MAX) return PA_ERR_SHAPE;
  if (dims->num_tokens == 0) return PA_OK;  // nothing to write; pointers may be NULL
  if (!q || !k || !v || !k_pool || !v_pool || !slot_mapping || !positions || !cos_sin)
    return PA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(k_pool, 16) ||
      !aligned(v_pool, 16) || !aligned(slot_mapping, 8) || !aligned(positions, 8) ||
      !aligned(cos_sin, 16))
    return PA_ERR_ALIGN;
  if (debug_checks()) {
    const int rc = check_slots(slot_mapping, dims->num_tokens, dims->num_blocks,
                               dims->block_size, dims->stream);
    if (rc != PA_OK) return rc;
  }
  pa_internal::RopeLaunch r{};
  pa_internal::CacheLaunch &a = r.cache;
  a.k = k;
  a.v = v;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.slot_mapping = slot_mapping;
  a.num_tokens = dims->num_tokens;
  a.num_kv_heads = dims->num_kv_heads;
  a.head_dim = dims->head_dim;
  a.block_size = dims->block_size;
  a.num_blocks = dims->num_blocks;
  a.elem_bytes = elem_bytes(dims->dtype);
  a.stream = dims->stream;
  r.q = q;
  r.positions = positions;
  r.cos_sin = cos_sin;
  r.num_heads = rope->num_heads;
  r.rot_dim = rope->rot_dim;
  r.max_position = rope->max_position;
  r.neox = rope->is_neox;
  return pa_internal::launch_reshape_and_cache_rope(r);
}

int copy_blocks(const void *k_src, const void *v_src, void *k_dst, void *v_dst,
                const int64_t *block_mapping, const pa_copy_dims *dims) {
  if (!dims) return PA_ERR_NULL;
  if (dims->num_pairs < 0 || dims->num_kv_heads < 1 || dims->src_num_blocks < 1 ||
      dims->dst_num_blocks < 1 || dims->reserved != 0)
    return PA_ERR_SHAPE;
  if (dims->dtype != PA_DTYPE_F32 && dims->dtype != PA_DTYPE_BF16) return PA_ERR_UNSUPPORTED;
  if (!supported_dim(dims->head_dim) || !supported_bs(dims->block_size)) return PA_ERR_UNSUPPORTED;
  if (dims->num_pairs == 0) return PA_OK;  // nothing to copy; pointers may be NULL
  if (!k_src || !v_src || !k_dst || !v_dst || !block_mapping) return PA_ERR_NULL;
  if (!aligned(k_src, 16) || !aligned(v_src, 16) || !aligned(k_dst, 16) || !aligned(v_dst, 16) ||
      !aligned(block_mapping, 8))
    return PA_ERR_ALIGN;
  if (debug_checks()) {
    const int rc = check_copy_pairs(block_mapping, dims->num_pairs, dims->src_num_blocks,
                                    dims->dst_num_blocks, k_src == k_dst && v_src == v_dst,
                                    dims->stream);
    if (rc != PA_OK) return rc;
  }
  pa_internal::CopyLaunch a{};
  a.k_src = k_src;
  a.v_src = v_src;
  a.k_dst = k_dst;
  a.v_dst = v_dst;
  a.mapping = block_mapping;
  a.num_pairs = dims->num_pairs;
  a.page_bytes = (int64_t)dims->num_kv_heads * dims->block_size * dims->head_dim *
                 elem_bytes(dims->dtype);
  a.src_blocks = dims->src_num_blocks;
  a.dst_blocks = dims->dst_num_blocks;
  a.stream = dims->stream;
  return pa_internal::launch_copy_pages(a);
}

const char *pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "PA_OK: success";
    case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE: a size is out of range or inconsistent";
    case PA_ERR_UNSUPPORTED:
      return "PA_ERR_UNSUPPORTED: dtype, head_dim, block_size or head group not supported";
    case PA_ERR_ALIGN: return "PA_ERR_ALIGN: a pointer is misaligned";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: split-K workspace missing or too small";
    case PA_ERR_HIP: return "PA_ERR_HIP: the HIP runtime reported a launch error";
    case PA_ERR_PRECONDITION:
      return "PA_ERR_PRECONDITION: a device-side precondition does not hold (found by "
             "PA_DEBUG_CHECKS=1)";
    case PA_ERR_SCRATCH_LIMIT:
      return "PA_ERR_SCRATCH_LIMIT: the call needs more than the library's static scratch "
             "(PA_NOALLOC_SCRATCH_BYTES); use paged_attention_decode with a workspace";
  }
  return "unknown status";
}

size_t pa_hbm_read_probe_sink_bytes(void) { return pa_internal::hbm_probe_sink_bytes(); }

int pa_hbm_read_probe(const void *buf, size_t bytes, void *sink, void *stream) {
  if (!buf || !sink) return PA_ERR_NULL;
  if (bytes < 16 || bytes % 16 != 0) return PA_ERR_SHAPE;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return PA_ERR_ALIGN;
  return pa_internal::launch_hbm_probe(buf, bytes, sink, stream);
}

}  // extern "C"
