/*
 * libpagedattn -- paged decode and prefill attention, the KV-cache write and
 * the page copy for AMD Instinct MI355X (gfx950).
 *
 * What is computed (vLLM / PagedAttention pages):
 *   - The KV cache is cut into fixed-size pages of 16 or 32 tokens that sit
 *     anywhere in a physical page pool; a per-sequence page table maps
 *     logical page j to a physical page, and the attention kernel reads the
 *     pages through that table with no data movement and no padding
 *     (showapi.com article, section 2.1; tutorial page, section 4.2 and its
 *     page-table figure; pinggu.org thread, PagedAttention paragraph).
 *   - Each decode step produces the next token and the updated KV cache
 *     (tutorial page, section 4.3, step 3 of the iteration).
 * The pages give neither the attention formula nor a memory layout; this
 * library computes, per query head, softmax(q . K^T * scale) . V over the
 * sequence's context tokens, and fixes the layouts below.
 *
 * Layouts (all row-major and contiguous):
 *   q, out          [num_seqs, num_heads, head_dim]
 *   k_pool, v_pool  [num_blocks, num_kv_heads, block_size, head_dim]
 *                   token t of a sequence is at logical page t / block_size,
 *                   offset t % block_size; one (page, kv-head) is a
 *                   contiguous block_size * head_dim run of elements
 *   block_tables    int32 [num_seqs, max_blocks_per_seq]
 *   context_lens    int32 [num_seqs]
 *   k, v (new)      [num_tokens, num_kv_heads, head_dim]
 *   slot_mapping    int64 [num_tokens], slot = physical_page * block_size + offset
 * Query head h reads kv-head h / (num_heads / num_kv_heads).
 *
 * Ownership: every pointer is a device pointer owned by the caller
 * (including the workspace).  The library allocates nothing, keeps no
 * handle to caller memory, never synchronises, and launches all work on the
 * given stream (NULL = the null stream), so calls are stream-ordered and
 * re-entrant across streams.
 *
 * Errors: arguments are validated on the host before any HIP call; a
 * rejected call returns a nonzero PA_ERR_* code and touches nothing.  A
 * failed launch returns PA_ERR_HIP.  Faults inside a kernel surface, as with
 * any HIP call, at the caller's next synchronisation.
 *
 * Device-side preconditions (the contents of tables in device memory) are
 * not checked by default: the kernels skip out-of-pool page ids and slots
 * and clamp context lengths instead, as each call states.  With the
 * environment variable PA_DEBUG_CHECKS=1 every call first copies the device
 * tables it reads to host memory, waits for its stream, and returns
 * PA_ERR_PRECONDITION without launching anything when a precondition fails:
 *   - context lengths in [0, max_blocks_per_seq * block_size];
 *   - the page ids a context uses (its first ceil(L / block_size) table
 *     entries) in [0, num_blocks);
 *   - slots negative or in [0, num_blocks * block_size), the non-negative
 *     ones distinct;
 *   - query_start from 0 to num_tokens without decreasing; sharing groups
 *     from 0 to num_seqs without decreasing, prefix lengths within the
 *     table, members' prefix page ids equal and in the pool;
 *   - page copies: no repeated destination, and within one pool no
 *     destination that is also a source.
 * That pass synchronises and allocates host memory: it is for debugging,
 * not for graph capture or timing.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  PA_OK = 0,
  PA_ERR_NULL = 1,        /* a required pointer is NULL */
  PA_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
  PA_ERR_UNSUPPORTED = 3, /* valid but not built: dtype, head_dim, block_size, group */
  PA_ERR_ALIGN = 4,       /* a pointer is not 16-byte (tables: 4/8-byte) aligned */
  PA_ERR_WORKSPACE = 5,   /* workspace missing, too small or misaligned */
  PA_ERR_HIP = 6,         /* the HIP runtime reported a launch error */
  PA_ERR_SCRATCH_LIMIT = 7, /* paged_attention_decode_noalloc: the call needs more
                               than PA_NOALLOC_SCRATCH_BYTES of scratch */
  PA_ERR_PRECONDITION = 8   /* PA_DEBUG_CHECKS=1 found a device-side precondition
                               violated (see the file header) */
};

enum { PA_DTYPE_F32 = 0, PA_DTYPE_BF16 = 1 };

/* Shapes and launch context of paged_attention_decode. */
typedef struct pa_decode_dims {
  int32_t num_seqs;            /* >= 0; 0 is a no-op */
  int32_t num_heads;           /* query heads, a multiple of num_kv_heads */
  int32_t head_dim;            /* 64 or 128 */
  int32_t max_blocks_per_seq;  /* columns of block_tables, >= 1 */
  int32_t num_blocks;          /* pages in each pool, >= 1 */
  int32_t dtype;               /* PA_DTYPE_*: one type for q, out, k_pool, v_pool */
  int32_t partition_size;      /* tokens per split-K partition, a multiple of
                                  block_size, at most 256 pages; 0 = default: no
                                  split when max_blocks_per_seq * block_size
                                  <= 2048, else the largest of 2048, 1024, 512,
                                  256 that gives num_seqs * partitions >= 128
                                  (256 when none does) */
  int32_t reserved;            /* must be 0 */
  void *workspace;             /* device scratch, caller-owned, 16-byte aligned, at
                                  least paged_attention_decode_workspace_bytes();
                                  required whenever num_seqs > 0 (it holds the
                                  work plan and the split-K partials) */
  size_t workspace_bytes;
  void *stream;                /* hipStream_t */
  void *timing_events[2];      /* optional hipEvent_t pair (or NULLs): recorded at
                                  the partition kernel's own start and end (the
                                  kernel is launched through hipExtLaunchKernel),
                                  for measuring it alone */
} pa_decode_dims;

/*
 * Single-token decode attention over a paged KV cache: the attention step of
 * each decode iteration, reading the sequence's KV pages through its page
 * table in place, with no gather copy and no padding (showapi.com article,
 * section 2.1; tutorial page, section 4.2 and its page-table figure, and
 * section 4.3, step 3 of the iteration).  The formula is not on the pages;
 * the one below is standard softmax attention per query head.
 *
 * For sequence s with L = context_lens[s] (clamped to
 * [0, max_blocks_per_seq * block_size]) and every query head h:
 *   out[s,h,:] = sum_t w_t V_t,  w = softmax_t(scale * q[s,h,:] . K_t),
 * over tokens t = 0 .. L-1 read through block_tables[s, t / block_size].
 * L = 0 writes a zero row.  Block-table columns at or past ceil(L /
 * block_size) are never used (they may hold anything; the kernel may load
 * them, so the whole [num_seqs, max_blocks_per_seq] table must be readable).
 * Slots past L in the last page are never used in arithmetic (they may hold
 * anything, NaN included).
 *
 * num_kv_heads: kv-heads in the pools; num_heads / num_kv_heads must be
 *   1, 2, 4 or 8.
 * scale: the logit scale, typically 1/sqrt(head_dim).
 * block_size: tokens per page, 16 or 32.
 *
 * Sequences longer than partition_size tokens are split into partitions
 * whose partial (max, sum, weighted V) go to the workspace and are merged by
 * a log-sum-exp reduce kernel; the result is the same softmax up to fp32
 * rounding.  Accumulation is fp32; bf16 results are rounded to nearest even.
 * With bf16 and 2-8 query heads per kv-head the contractions run on the
 * matrix cores, with the softmax weights entering as a pair of bf16 terms
 * (about 16 significant bits).
 *
 * Launches, all on dims->stream: a one-workgroup plan kernel (orders the
 * (sequence, partition) work units by size into the workspace), the
 * partition kernel (timing_events bracket this one), and the reduce kernel
 * when some sequence can span more than one partition.  The result does not
 * depend on the order units run in: each output element is computed by one
 * fixed sequence of operations on its sequence's tokens.
 *
 * The workspace is required for every call with num_seqs > 0, also when no
 * sequence is split: besides the split-K partials it holds the work plan,
 * which the plan kernel writes on the device so the host never reads
 * context_lens.  block_size is a separate argument, as in the call's
 * published argument list; the pools' other dimensions are in dims.
 *
 * Device-side preconditions (checked only with PA_DEBUG_CHECKS=1): the
 * first ceil(L / block_size) entries of each used table row lie in
 * [0, num_blocks), and 0 <= L <= max_blocks_per_seq * block_size.  Without
 * the check, a page id outside that range is skipped by the kernel (its
 * tokens drop out of the softmax) instead of being read, and L is clamped.
 */
int paged_attention_decode(void *out, const void *q, const void *k_pool,
                           const void *v_pool, const int32_t *block_tables,
                           const int32_t *context_lens, int32_t num_kv_heads,
                           float scale, int32_t block_size,
                           const pa_decode_dims *dims);

/* Bytes of the static device scratch of paged_attention_decode_noalloc. */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * paged_attention_decode for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The work plan and the split-K partials go to a static device
 * buffer of PA_NOALLOC_SCRATCH_BYTES (32 MiB) instead of a caller's
 * workspace; the library allocates nothing and calls no allocating routine.
 * Every device the library runs on holds one such buffer from the first
 * call on it until the process ends.
 *
 * Arguments, layouts, results and launches are those of
 * paged_attention_decode, except:
 *   - dims->workspace must be NULL and dims->workspace_bytes 0
 *     (PA_ERR_WORKSPACE otherwise);
 *   - a call whose paged_attention_decode_workspace_bytes() exceeds
 *     PA_NOALLOC_SCRATCH_BYTES returns PA_ERR_SCRATCH_LIMIT before any HIP
 *     call (for example 256 sequences x 32 heads x 4 partitions of
 *     head_dim 128 need 17 MB and fit; 8 x 32 heads x 64 partitions need
 *     8.5 MB);
 *   - the first call on a device looks up the buffer's device address
 *     (hipGetSymbolAddress) with that device current; a failure there
 *     returns PA_ERR_HIP.
 * Every call on one device uses that device's one buffer, which keeps the
 * last call's contents; each call writes every plan entry and partial it
 * reads, so nothing needs clearing between calls.  Calls that overlap on one
 * device -- launched on different streams without ordering, or from several
 * host threads -- race on the buffer and give undefined results.  Calls
 * ordered on one stream are safe.
 */
int paged_attention_decode_noalloc(void *out, const void *q, const void *k_pool,
                                   const void *v_pool, const int32_t *block_tables,
                                   const int32_t *context_lens, int32_t num_kv_heads,
                                   float scale, int32_t block_size, const pa_decode_dims *dims);

/*
 * paged_attention_decode with ALiBi (the showapi.com article, section 4.1,
 * lists ALiBi among the position encodings the engine serves): the logit of
 * context token t for query head h gets alibi_slopes[h] * (t - (L - 1))
 * added, L - 1 being the query's own position, before the softmax.
 * alibi_slopes: device fp32 [num_heads], 4-byte aligned, required when
 * num_seqs > 0 (PA_ERR_NULL otherwise).  Everything else, workspace
 * included, is as for paged_attention_decode.
 */
int paged_attention_decode_alibi(void *out, const void *q, const void *k_pool,
                                 const void *v_pool, const int32_t *block_tables,
                                 const int32_t *context_lens, int32_t num_kv_heads, float scale,
                                 int32_t block_size, const float *alibi_slopes,
                                 const pa_decode_dims *dims);

/*
 * One decode step: the step's new tokens into the cache, then attention over
 * the updated cache.  Each iteration yields the next token together with the
 * updated KV cache (tutorial page, section 4.3, step 3), and the step's own
 * token is the last context position its attention reads (section 4.2).
 *
 * The result -- out and both pools -- is bit for bit that of
 *   reshape_and_cache(k, v, k_pool, v_pool, slot_mapping, cache dims), then
 *   paged_attention_decode(out, q, k_pool, v_pool, block_tables, context_lens,
 *                          num_kv_heads, scale, block_size, dims),
 * with cache dims = {num_tokens = dims->num_seqs, num_kv_heads,
 * dims->head_dim, block_size, dims->num_blocks, dims->dtype, dims->stream}.
 * k, v: device [num_seqs, num_kv_heads, head_dim] of dims->dtype, 16-byte
 * aligned (row s is sequence s's new token); slot_mapping: device int64
 * [num_seqs], 8-byte aligned, as for reshape_and_cache (a negative or
 * out-of-pool slot writes nothing; two equal slots are a precondition
 * violation).  Everything else, workspace included, is as for
 * paged_attention_decode; with num_seqs = 0 nothing is read or written.
 *
 * Launches, all on dims->stream: one kernel whose first workgroup writes the
 * work plan while the others write the new tokens (the plan reads only
 * context_lens, so the two are independent), then the partition kernel
 * (timing_events bracket this one) and the reduce kernel when some sequence
 * can span more than one partition: one launch fewer than the two calls.
 * PA_DEBUG_CHECKS=1 checks both calls' device-side preconditions.
 */
int paged_attention_decode_step(void *out, const void *q, const void *k, const void *v,
                                const int64_t *slot_mapping, void *k_pool, void *v_pool,
                                const int32_t *block_tables, const int32_t *context_lens,
                                int32_t num_kv_heads, float scale, int32_t block_size,
                                const pa_decode_dims *dims);

/*
 * Workspace bytes paged_attention_decode needs for these shapes, with
 * P = ceil(max_blocks_per_seq * block_size / partition_size):
 *   the work plan, 4 * (4 + num_seqs * P) rounded up to 256, plus, when
 *   P > 1, the split-K partials num_seqs * num_heads * P * (head_dim + 2) * 4.
 * 0 when num_seqs is 0.  Returns SIZE_MAX when the shapes are invalid.  The
 * size does not depend on the kv-head count, which is not an argument; the
 * call itself checks the head group and its count of work items.
 */
size_t paged_attention_decode_workspace_bytes(int32_t block_size,
                                              const pa_decode_dims *dims);

/*
 * The partition size, in tokens, paged_attention_decode uses for these
 * shapes (dims->partition_size, or the default when that is 0); -1 when the
 * shapes are invalid.
 */
int32_t paged_attention_decode_partition_tokens(int32_t block_size,
                                                const pa_decode_dims *dims);

/*
 * Decode attention for batches in which groups of consecutive sequences
 * share their first pages (vLLM / PagedAttention pages: in parallel
 * sampling the outputs of one request share the prefix's KV pages --
 * tutorial page, section 4.2).  The result is that of
 * paged_attention_decode on the same arguments; the shared pages are read
 * once per group (up to 32 query rows, members x query heads per kv-head,
 * per read) instead of once per sequence.
 *
 * group_starts  int32 [num_groups + 1], device: group i is sequences
 *               group_starts[i] .. group_starts[i + 1] - 1 (nondecreasing,
 *               group_starts[0] = 0, group_starts[num_groups] = num_seqs;
 *               sequences outside every group have no shared prefix)
 * prefix_lens   int32 [num_groups], device: tokens at the start of every
 *               member's context on the same physical pages; the first
 *               prefix_lens[i] / block_size table columns of every member
 *               hold the same page ids (tokens of a partial last page count
 *               as the members' own)
 * A member's own context may end inside the prefix (its tokens past its
 * context length are masked).  bf16 only (PA_ERR_UNSUPPORTED otherwise);
 * head groups of 1, 2, 4 or 8.  The workspace must hold
 * paged_attention_decode_shared_prefix_workspace_bytes(); dims, stream and
 * timing events as for paged_attention_decode (the events bracket the
 * pass over the units), except that partition_size 0 here means 512 tokens
 * (or the whole table when it is smaller).
 *
 * Launches: a plan kernel (prefix units per group chunk and partition,
 * own-page units per sequence, largest first), the unit pass (partials for
 * every unit) and the reduce kernel (merges each sequence's partials).
 */
int paged_attention_decode_shared_prefix(void *out, const void *q, const void *k_pool,
                                         const void *v_pool, const int32_t *block_tables,
                                         const int32_t *context_lens, int32_t num_kv_heads,
                                         float scale, int32_t block_size,
                                         const int32_t *group_starts,
                                         const int32_t *prefix_lens, int32_t num_groups,
                                         const pa_decode_dims *dims);

/*
 * One shared-prefix decode step: the step's new tokens into the cache, then
 * paged_attention_decode_shared_prefix over the updated cache (tutorial
 * page, section 4.3, step 3; the samples of a group share their prompt's
 * pages, section 4.2).  Bit for bit reshape_and_cache(k, v, k_pool, v_pool,
 * slot_mapping, cache dims) followed by paged_attention_decode_shared_prefix
 * with the other arguments, with k, v, slot_mapping and the cache dims as
 * for paged_attention_decode_step.  The first launch writes the shared-prefix
 * work plan in one workgroup and the new tokens in the others; the unit and
 * reduce kernels follow.  A group's shared pages are read-only for the step:
 * a member's new token goes to a page of its own (copy_blocks first when a
 * prefix ends inside a page).
 */
int paged_attention_decode_shared_prefix_step(
    void *out, const void *q, const void *k, const void *v, const int64_t *slot_mapping,
    void *k_pool, void *v_pool, const int32_t *block_tables, const int32_t *context_lens,
    int32_t num_kv_heads, float scale, int32_t block_size, const int32_t *group_starts,
    const int32_t *prefix_lens, int32_t num_groups, const pa_decode_dims *dims);

/*
 * Workspace bytes of paged_attention_decode_shared_prefix, with
 * P = ceil(max_blocks_per_seq * block_size / partition_size) (partition
 * size as that call resolves it):
 *   plan 4 * (4 + 10 * num_seqs * P + 2 * num_seqs) rounded up to 256, plus
 *   partials num_seqs * num_heads * 2P * (head_dim + 2) * 4.
 * 0 when num_seqs is 0; SIZE_MAX for invalid shapes.
 */
size_t paged_attention_decode_shared_prefix_workspace_bytes(int32_t block_size,
                                                            const pa_decode_dims *dims);

/* Shapes and launch context of paged_attention_prefill. */
typedef struct pa_prefill_dims {
  int32_t num_seqs;            /* >= 0 */
  int32_t num_tokens;          /* rows of q and out (query_start[num_seqs]), >= 0;
                                  0 is a no-op */
  int32_t num_heads;           /* query heads; num_heads / num_kv_heads in {1, 2, 4, 8} */
  int32_t head_dim;            /* 64 or 128 */
  int32_t max_blocks_per_seq;  /* columns of block_tables, >= 1 */
  int32_t num_blocks;          /* pages in each pool, >= 1 */
  int32_t dtype;               /* PA_DTYPE_BF16 (the only type built) */
  int32_t partition_size;      /* keys per split-K partition, a positive multiple
                                  of 128 (the kernel's key tile); 0 = default:
                                  no split when the step has
                                  at least 1024 (block, kv-head) work items, else
                                  partitions of max(1024, ceil(capacity / parts))
                                  keys with parts = ceil(1024 / items), capacity =
                                  max_blocks_per_seq * block_size (no split when
                                  that is not below the capacity) */
  void *workspace;             /* device scratch, caller-owned, 16-byte aligned, at
                                  least paged_attention_prefill_workspace_bytes();
                                  required whenever num_tokens > 0 (work plan and,
                                  with a split, the partials) */
  size_t workspace_bytes;
  void *stream;                /* hipStream_t */
  void *timing_events[2];      /* optional hipEvent_t pair, recorded at the
                                  attention kernel's own start and end */
} pa_prefill_dims;

/*
 * Multi-token attention over a paged KV cache: the prompt of a newly
 * admitted request, or a chunk of it, attended in one step (continuous
 * batching admits new requests into the running batch with pages allocated
 * for them: tutorial page, section 4.3, step 2; pinggu.org thread,
 * continuous batching).
 *
 * Rows query_start[s] .. query_start[s+1]-1 of q and out belong to sequence
 * s; with n = their count and L = context_lens[s] (clamped to
 * [0, max_blocks_per_seq * block_size]), the chunk is the sequence's last n
 * tokens, and its row i, at position p = L - n + i, attends to the tokens at
 * positions 0 .. p:
 *   out[query_start[s] + i, h, :] = sum_{t <= p} w_t V_t,
 *   w = softmax_{t <= p}(scale * q[query_start[s] + i, h, :] . K_t),
 * K, V of kv-head h / (num_heads / num_kv_heads), read through
 * block_tables[s, t / block_size].  The chunk's own K/V rows must already be
 * in the pools (reshape_and_cache of the same rows, earlier on the stream).
 * A single row per sequence is the decode step.  A row that sees no token
 * (p < 0, i.e. more rows than context) is written as zeros; tokens on pages
 * whose id is outside [0, num_blocks) are skipped.  Slots past L in the last
 * page are never used in arithmetic.
 *
 * Layouts: q, out [num_tokens, num_heads, head_dim] bf16; query_start int32
 * [num_seqs + 1], non-decreasing from 0 to num_tokens (values are clamped to
 * [0, num_tokens] on the device); pools, block_tables and context_lens as
 * for paged_attention_decode.  Rows of out outside every sequence's range are
 * not written.
 *
 * Arithmetic: q.K and P.V on the matrix cores in bf16 with fp32
 * accumulation; the softmax weights enter P.V rounded to bf16 (8
 * significant bits), their sum is kept in fp32.  Results are rounded to
 * nearest even.
 *
 * Launches, all on dims->stream: a one-workgroup plan kernel (cuts every
 * chunk into blocks of 256 / group consecutive tokens, and with a split each
 * block's keys into partitions, and orders the items by the keys they read,
 * most first, into the workspace), the attention pass (timing_events
 * bracket this one) and, with a split, a reduce kernel that merges each
 * row's partitions by log-sum-exp.  The result does not depend on the order
 * work items run in.
 */
int paged_attention_prefill(void *out, const void *q, const void *k_pool, const void *v_pool,
                            const int32_t *block_tables, const int32_t *context_lens,
                            const int32_t *query_start, int32_t num_kv_heads, float scale,
                            int32_t block_size, const pa_prefill_dims *dims);

/*
 * paged_attention_prefill with ALiBi: the logit of token t for the chunk
 * row at position p and query head h gets alibi_slopes[h] * (t - p) added.
 * alibi_slopes: device fp32 [num_heads], 4-byte aligned, required when
 * num_tokens > 0.  Everything else is as for paged_attention_prefill.
 */
int paged_attention_prefill_alibi(void *out, const void *q, const void *k_pool,
                                  const void *v_pool, const int32_t *block_tables,
                                  const int32_t *context_lens, const int32_t *query_start,
                                  int32_t num_kv_heads, float scale, int32_t block_size,
                                  const float *alibi_slopes, const pa_prefill_dims *dims);

/*
 * One chunked-prefill step in one call: the chunk's own K/V rows are written
 * to their page slots, then the chunk attends over the cache that now holds
 * them (the new tokens' KV goes to the cache before attention reads it:
 * tutorial page, section 4.3, step 2 and section 4.2).
 *
 * The result -- out and both pools -- is bit for bit that of
 *   reshape_and_cache(k, v, k_pool, v_pool, slot_mapping, cache dims), then
 *   paged_attention_prefill(out, q, k_pool, v_pool, block_tables,
 *                           context_lens, query_start, num_kv_heads, scale,
 *                           block_size, dims),
 * with cache dims = {num_tokens = dims->num_tokens, num_kv_heads,
 * dims->head_dim, block_size, dims->num_blocks, dims->dtype, dims->stream}.
 * k, v: device [num_tokens, num_kv_heads, head_dim] bf16, 16-byte aligned
 * (row r is the K/V of q's row r); slot_mapping: device int64 [num_tokens],
 * 8-byte aligned, as for reshape_and_cache (a negative or out-of-pool slot
 * writes nothing; two equal slots are a precondition violation).
 * Everything else, workspace included, is as for paged_attention_prefill;
 * with num_tokens = 0 nothing is read or written.
 *
 * Launches, all on dims->stream: one kernel whose first workgroup writes the
 * work plan while the others write the chunk's rows (the plan reads only
 * query_start and context_lens, so the two are independent), then the
 * attention pass (timing_events bracket this one) and, with a split, the
 * reduce kernel: one launch fewer than the two calls.  PA_DEBUG_CHECKS=1
 * checks both calls' device-side preconditions.
 */
int paged_attention_prefill_step(void *out, const void *q, const void *k, const void *v,
                                 const int64_t *slot_mapping, void *k_pool, void *v_pool,
                                 const int32_t *block_tables, const int32_t *context_lens,
                                 const int32_t *query_start, int32_t num_kv_heads, float scale,
                                 int32_t block_size, const pa_prefill_dims *dims);

/*
 * Workspace bytes of paged_attention_prefill, with P the partitions of the
 * capacity (1 without a split):
 *   plan 4 * (4 + 3 * num_tokens * P + num_tokens) rounded up to 256, plus,
 *   when P > 1, partials num_tokens * num_heads * P * (head_dim + 2) * 4.
 * 0 when num_tokens is 0; SIZE_MAX for invalid shapes.
 */
size_t paged_attention_prefill_workspace_bytes(int32_t num_kv_heads, int32_t block_size,
                                               const pa_prefill_dims *dims);

/*
 * The key partition paged_attention_prefill uses for these shapes
 * (dims->partition_size, or the default when that is 0; 0 = no split);
 * -1 for invalid shapes.
 */
int32_t paged_attention_prefill_partition_tokens(int32_t num_kv_heads, int32_t block_size,
                                                 const pa_prefill_dims *dims);

/* Shapes and launch context of reshape_and_cache. */
typedef struct pa_cache_dims {
  int32_t num_tokens;   /* >= 0; 0 is a no-op */
  int32_t num_kv_heads; /* >= 1 */
  int32_t head_dim;     /* 64 or 128 */
  int32_t block_size;   /* 16 or 32 */
  int32_t num_blocks;   /* pages in each pool */
  int32_t dtype;        /* PA_DTYPE_* of k, v and the pools */
  void *stream;         /* hipStream_t */
} pa_cache_dims;

/*
 * KV-cache write: each decode iteration yields the next token together with
 * the updated KV cache (tutorial page, section 4.3, step 3), and a token's
 * K/V lives in its sequence's page at the slot the page table maps its
 * position to (tutorial page, section 4.2, page-table figure; showapi.com
 * article, section 2.1).  The slot encoding is not on the pages; here
 * slot = physical_page * block_size + offset.
 *
 * For each token i with slot = slot_mapping[i] >= 0,
 *   k_pool[slot / block_size, :, slot % block_size, :] = k[i, :, :]
 *   v_pool[slot / block_size, :, slot % block_size, :] = v[i, :, :]
 * bit for bit (no conversion).  A negative slot means "no token" and is
 * skipped.  A slot at or past num_blocks * block_size is also skipped
 * rather than written.  Two tokens naming the same slot is a precondition
 * violation (the surviving value is unspecified); PA_DEBUG_CHECKS=1 reports
 * both as PA_ERR_PRECONDITION instead.  Pointers: k, v [num_tokens,
 * num_kv_heads, head_dim] and the pools 16-byte aligned, slot_mapping
 * 8-byte aligned, all device memory owned by the caller.
 */
int reshape_and_cache(const void *k, const void *v, void *k_pool, void *v_pool,
                      const int64_t *slot_mapping, const pa_cache_dims *dims);

/* Rotary position embedding parameters of reshape_and_cache_rope. */
typedef struct pa_rope_dims {
  int32_t num_heads;     /* query heads of q, >= 1 */
  int32_t rot_dim;       /* rotated entries per head: even, <= head_dim, a multiple
                            of 16 (bf16) or 8 (fp32); PA_ERR_UNSUPPORTED otherwise */
  int32_t max_position;  /* rows of cos_sin, >= 1 */
  int32_t is_neox;       /* 1: pairs (i, i + rot_dim/2); 0: pairs (2i, 2i + 1) */
  int32_t reserved;      /* must be 0 */
} pa_rope_dims;

/*
 * KV-cache write with rotary position embedding fused in (the showapi.com
 * article, section 4.1, lists RoPE among the position encodings the engine
 * serves).  For each token i with pos = positions[i] in [0, max_position):
 *   - every query head of q[i] ([num_tokens, num_heads, head_dim], device,
 *     same dtype as the pools) is rotated in place;
 *   - k[i] is rotated the same way and written, with v[i] unchanged, to
 *     slot_mapping[i] exactly as reshape_and_cache writes it (k itself is
 *     not modified; negative or out-of-pool slots write nothing).
 * Rotation of pair (a, b) with c = cos_sin[pos, j], s = cos_sin[pos,
 * rot_dim/2 + j]: (a c - b s, b c + a s), in fp32, rounded to the element
 * type (bf16: nearest even).  Pair j is entries (j, j + rot_dim/2) when
 * is_neox, else (2j, 2j + 1); entries past rot_dim are unchanged.
 * cos_sin: device fp32 [max_position, rot_dim], 16-byte aligned, filled by
 * the caller (for example cos and sin of pos * base^(-2j/rot_dim)).  A token whose position
 * is outside [0, max_position) is skipped entirely (q untouched, nothing
 * written).  positions: device int64 [num_tokens], 8-byte aligned.
 */
int reshape_and_cache_rope(void *q, const void *k, const void *v, void *k_pool, void *v_pool,
                           const int64_t *slot_mapping, const int64_t *positions,
                           const float *cos_sin, const pa_rope_dims *rope,
                           const pa_cache_dims *dims);

/* Shapes and launch context of copy_blocks. */
typedef struct pa_copy_dims {
  int32_t num_pairs;       /* rows of block_mapping, >= 0; 0 is a no-op */
  int32_t num_kv_heads;    /* >= 1 */
  int32_t head_dim;        /* 64 or 128 */
  int32_t block_size;      /* 16 or 32 */
  int32_t dtype;           /* PA_DTYPE_* of all four pools */
  int32_t src_num_blocks;  /* pages in k_src / v_src */
  int32_t dst_num_blocks;  /* pages in k_dst / v_dst */
  int32_t reserved;        /* must be 0 */
  void *stream;            /* hipStream_t */
} pa_copy_dims;

/*
 * Whole-page copy between pools (vLLM / PagedAttention pages: several
 * sequences may share prefix pages, so a sequence about to write into a
 * shared page first gets its own copy -- tutorial page, section 4.2; under
 * memory pressure a preempted sequence's KV pages move to a CPU-side pool
 * and back -- tutorial page, sections 4.4 and 4.5).
 *
 * For each pair i of block_mapping ([num_pairs, 2] int64: source page,
 * destination page), page block_mapping[i][0] of k_src / v_src (every
 * kv-head, [num_kv_heads, block_size, head_dim] elements) is copied bit for
 * bit to page block_mapping[i][1] of k_dst / v_dst.  Pools have the layout
 * of paged_attention_decode.  A pair with a page outside its pool (negative
 * included) is skipped.
 *
 * Memory: the four pools and block_mapping may be device memory or pinned
 * host memory (hipHostMalloc), so one call swaps pages out to a host pool,
 * back in, or copies within a device pool (source and destination pools the
 * same).  Pageable host memory gives PA_ERR_UNSUPPORTED.  Pointers are
 * classified with hipPointerGetAttributes after the argument checks.
 *
 * Preconditions: no two pairs name the same destination page; when source
 * and destination are the same pools, no destination page is also a
 * source page (the result would depend on the order of the copies).
 */
int copy_blocks(const void *k_src, const void *v_src, void *k_dst, void *v_dst,
                const int64_t *block_mapping, const pa_copy_dims *dims);

/* Static, human-readable text for a status code. */
const char *pa_status_string(int status);

/*
 * Measurement kernel: streams `bytes` (a multiple of 16, >= 16) of `buf`
 * with 16-byte loads and writes one 32-bit checksum per workgroup to
 * `sink` (at least pa_hbm_read_probe_sink_bytes() bytes).  Gives the
 * achievable HBM read bandwidth of the device the pools live on.
 */
int pa_hbm_read_probe(const void *buf, size_t bytes, void *sink, void *stream);
size_t pa_hbm_read_probe_sink_bytes(void);

/*
 * Measurement kernel: the access pattern of paged_attention_decode without
 * its arithmetic.  Takes the same arguments, checks and workspace, runs the
 * same plan kernel, and then reads exactly the K and V pages the partition
 * kernels would read, in their order and with their load shapes: items
 * (unit, kv-head) largest unit first, one workgroup of 4 wavefronts (8 for
 * bf16 with one query head per kv-head) per item with the unit's pages
 * dealt to the wavefronts in turn (or one
 * wavefront per item where the grouped-query kernel works that way: bf16
 * with 2-8 query heads per kv-head, partitions of at most 64 pages and a
 * table of at least 16 partitions; there an item is a run of up to four
 * consecutive partitions of at most 64 pages in all), each (page, kv-head)
 * run as 16-byte non-temporal loads.  Instead of attention it
 * stores, for each item, the XOR of every 16-byte word it loaded in the
 * first 16 bytes of the output row of the item's first query head
 * (h = kv-head * num_heads / num_kv_heads); nothing else in `out` is
 * written, and a sequence's items overwrite each other's word.
 * timing_events bracket the read kernel.  Its rate, the decode call's KV
 * bytes over its duration, is the read bandwidth the decode access pattern
 * reaches on the device: the ceiling for the partition kernels.
 */
int paged_attention_decode_read_probe(void *out, const void *q, const void *k_pool,
                                      const void *v_pool, const int32_t *block_tables,
                                      const int32_t *context_lens, int32_t num_kv_heads,
                                      float scale, int32_t block_size,
                                      const pa_decode_dims *dims);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
