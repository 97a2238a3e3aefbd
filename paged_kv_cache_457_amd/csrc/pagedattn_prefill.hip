// Paged multi-token attention: prefill and chunked prefill (bf16, matrix cores).
//
// Continuous batching admits a new request into the running batch with pages
// allocated for its prompt (tutorial page, section 4.3, step 2; pinggu
// thread, continuous batching).  Its prompt, or a chunk of it, is then
// attended in one step over the paged cache, after the cache write of the
// same step has put the chunk's K/V rows into their pages.  Row i of a
// sequence's chunk of n tokens is the token at position p = ctx - n + i; it
// sees the tokens at positions 0 .. p (causal), read through the block
// table like every decode step.
//
// Work item: (sequence, kv-head, block of TOK = kRows / G consecutive chunk
// tokens) = kRows query rows, row r = token r / G, query head g*G + r % G.
// Each of the workgroup's waves carries 32 rows as two 16-row MFMA tiles.
// Keys go through in tiles of kKeys that all waves share: the workgroup
// loads a tile's K and V rows straight from global memory into LDS
// (buffer_load_dwordx4 ... lds, no staging registers), double buffered: the
// next tile's loads are in flight while one tile is used.
//
//   q.K   S^T = K Q^T, v_mfma_f32_16x16x32_bf16: A = 16 keys x 32 head_dim
//         (one 16-byte LDS read per lane), B = 16 query rows (registers).
//         Lane 16*q4 + j gets S[key 4*q4 + r][row j].
//   P.V   O^T += V^T P^T, the same instruction with 32 keys as its reduction
//         dimension: B is P straight from two 16-key S tiles (lane-local;
//         the keys are taken in the order both operands agree on), A is V^T
//         from two transposing LDS reads (ds_read_b64_tr_b16).  Lane
//         16*q4 + j holds O^T[d = 16n + 4*q4 + r][row j], so the softmax
//         state of row j lives in the lanes that hold its output columns.
//
// Online softmax per row in log2 units with the scale folded in.  Keys at or
// past the item's last position, and keys on pages whose id is outside the
// pool, are loaded as zeros (so a poisoned slot never reaches a multiply) and
// masked to -inf in S; a tile that lies wholly below a wave's first position
// and on valid pages skips the per-key mask.
#include <type_traits>

#include "pagedattn_cache_row.h"
#include "pagedattn_device.h"
#include "pagedattn_internal.h"
#include "pagedattn_prefill_launch.h"
#include "pagedattn_step_launch.h"
#include "pagedattn_timed_launch.h"

namespace {

using namespace pa_dev;
using pa_internal::kPlanHeader;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kWaves = 8;           // two per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32 * kWaves;  // query rows of a work item
static_assert(kRows == pa_internal::kPrefillRows, "rows per work item");
constexpr int kKeys = pa_internal::kPrefillKeyTile;  // keys per LDS tile
constexpr float kRescaleLog2 = 8.f; // lazy rescale threshold of the running max
constexpr int kPlanThreads = 1024;
constexpr int kPlanRecord = pa_internal::kPrefillPlanRecord;  // ints per plan item
constexpr int kBuckets = kPlanThreads - 1;  // plan size classes (key tiles); the last is open-ended


template <int D, int BS, int G>
struct PrefillShape {
  static constexpr int ROW = 2 * D;                      // bytes per key row
  static constexpr int CPR = D / 8;                      // 16-byte chunks per row
  static constexpr int NC = D / 32;                      // q.K slabs
  static constexpr int NN = D / 16;                      // 16-column blocks of O
  static constexpr int TILE = kKeys * ROW;               // bytes of a K (or V) tile
  static constexpr int LOADS = TILE / (16 * kThreads);   // 16-byte loads per thread, K or V
  static constexpr int TOK = kRows / G;                  // chunk tokens per work item
  static constexpr int PPT = kKeys / BS;                 // pages per key tile
  static_assert(LOADS >= 1 && TILE % (16 * kThreads) == 0, "tile loads");
  static_assert(kRows % G == 0 && 32 % G == 0, "rows of a wave hold whole tokens");
};

// Position of 16-byte chunk c of key row r inside its LDS row.  Rows are
// unpadded; the chunk index is XOR-ed with a function of the row.  Measured
// on gfx950 (SQ_LDS_BANK_CONFLICT over single-pattern kernels), a 64-lane
// ds_read_b128 is served in four passes of 16 lanes, a pass being the
// lanes with equal (bit 5, bit 2 ^ bit 3 ^ bit 4) of the lane id, and a
// ds_read_b64_tr_b16 in two passes of 32 consecutive lanes, over 64 banks
// of 4 bytes.  Under that model these masks give the q.K operand reads and
// the transposing V reads no conflicts at all (verified by the counter);
// an earlier mask chosen for 16-lane passes of consecutive lanes cost four
// conflict cycles per q.K read.
template <int D>
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (D == 128) {
    return c ^ ((r & 7) << 1);
  } else {
    return c ^ (r & 7);
  }
}

// ------------------------------------------------------------------ plan
// One workgroup.  Every chunk is cut into blocks of `tok` consecutive
// tokens; with key partitions of kpart tokens (a multiple of kKeys; 0: no
// split) each block is further cut by its keys, one item per partition
// that holds keys the block sees.  plan[0] = item count; item k is the
// kPlanRecord ints at plan[kPlanHeader + kPlanRecord * k] (their order is
// given beside kPrefillPlanRecord), items ordered by the key tiles they
// read, most first (a sequence's blocks by its largest when they are close
// in size: sort_keys).  An item's page flag is set when no page it reads lies
// outside the pool: the wave that writes a sequence's items first finds
// the sequence's first such page (a flag left clear only sends the item
// down the per-key mask path).  With a split,
// nparts[row] is the number of partitions of the row's block (1: the item
// writes the row's output itself).  Valid chunks give at most max_items
// items; with overlapping chunks (an invalid query_start) the surplus is
// dropped, so nothing is written outside the plan.
//
// A wave takes one sequence at a time and its lanes the sequence's
// (block, partition) pairs, so a long chunk over a long context costs a
// few strided passes rather than one lane's serial loop.
__device__ __forceinline__ void prefill_plan_body(
    const int32_t *__restrict__ context_lens, const int32_t *__restrict__ query_start,
    const int32_t *__restrict__ block_tables, int max_blocks, int num_blocks, int block_size,
    int num_seqs, int num_tokens, int ctx_cap, int tok, int kpart, int max_parts, int max_items,
    int32_t *__restrict__ plan, int32_t *__restrict__ nparts) {
  constexpr int kPlanWaves = kPlanThreads / 64;
  __shared__ int s_count[kBuckets + 1];
  __shared__ int s_next[kBuckets + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int P = kpart ? max_parts : 1;  // partition slots per block
  for (int i = threadIdx.x; i <= kBuckets; i += kPlanThreads) s_count[i] = 0;
  if (kpart)  // rows outside every chunk: nothing to merge
    for (int i = threadIdx.x; i < num_tokens; i += kPlanThreads) nparts[i] = 1;
  __syncthreads();
  // chunk bounds, and the position of its first token
  auto chunk = [&](int s, int &a, int &n, int &p0) {
    a = min(max(query_start[s], 0), num_tokens);
    const int b = min(max(query_start[s + 1], a), num_tokens);
    n = b - a;
    p0 = min(max(context_lens[s], 0), ctx_cap) - n;
  };
  // keys the block starting at t0 sees, and its partitions
  auto keys = [&](int n, int p0, int t0) { return max(0, p0 + min(n, t0 + tok)); };
  // The keys an item of sequence (n, p0) is sorted by, given its own: the
  // sequence's total when its first block already sees half of them (a long
  // cached context under a short chunk), so that the sequence's blocks are
  // adjacent in the list.  With kv-head fastest, blocks of one (sequence,
  // kv-head) then run in the same round on the same XCD and read their
  // common keys through its L2 (Llama-2-7B chunked prefill, 8 x 1024 new
  // tokens after U[0, 3072] cached: 6-10% faster).  Where a sequence's blocks
  // differ more (a prompt with nothing cached), each item keeps its own size:
  // grouping them there cost 3-4% in balance.  Split items keep their own.
  auto sort_keys = [&](int n, int p0, int ke) {
    return !kpart && 2 * keys(n, p0, 0) >= max(0, p0 + n) ? max(0, p0 + n) : ke;
  };
  auto parts = [&](int kv_end) { return kpart && kv_end > 0 ? (kv_end + kpart - 1) / kpart : 1; };
  auto bucket = [&](int kv_end, int kp) {
    const int lo = kpart ? kp * kpart : 0;
    const int hi = kpart ? min(kv_end, lo + kpart) : kv_end;
    return hi <= lo ? 0 : min((hi - lo + kKeys - 1) / kKeys, kBuckets);
  };
  // visit(block start, partition, keys) for every item of sequence s
  auto items_of = [&](int s, auto visit) {
    int a, n, p0;
    chunk(s, a, n, p0);
    const int nb = (n + tok - 1) / tok;
    for (int j = lane; j < nb * P; j += 64) {
      const int b = P == 1 ? j : j / P, kp = j - b * P;
      const int ke = keys(n, p0, b * tok);
      if (kp < parts(ke)) visit(b * tok, kp, ke);
    }
    return a;
  };
  for (int s = wave; s < num_seqs; s += kPlanWaves) {
    int a0, n0, p00;
    chunk(s, a0, n0, p00);
    const int a = items_of(s, [&](int, int kp, int ke) {
      atomicAdd(&s_count[bucket(sort_keys(n0, p00, ke), kp)], 1);
    });
    if (kpart) {
      int a2, n, p0;
      chunk(s, a2, n, p0);
      for (int i = lane; i < n; i += 64) nparts[a + i] = parts(keys(n, p0, i - i % tok));
    }
  }
  __syncthreads();
  // first slot of each size class, largest class first: an exclusive scan
  // over thread t <-> class kBuckets - t (lane scan, then one over waves)
  {
    __shared__ int s_wave[kPlanWaves];
    const int t = threadIdx.x;
    const int v = s_count[kBuckets - t];
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane == 63) s_wave[wave] = x;
    __syncthreads();
    int before = 0;
    for (int k = 0; k < wave; ++k) before += s_wave[k];
    s_next[kBuckets - t] = before + x - v;
    if (t == kPlanThreads - 1) plan[0] = min(before + x, max_items);
  }
  __syncthreads();
  for (int s = wave; s < num_seqs; s += kPlanWaves) {
    int a, n, p0;
    chunk(s, a, n, p0);
    // first page of the sequence's keys whose id lies outside the pool; a
    // long table is read kScanBatch loads a lane at a time, all in flight
    // together
    constexpr int kScanBatch = 8;
    const int npg = (max(0, p0 + n) + block_size - 1) / block_size;
    const int32_t *row = block_tables + (size_t)s * max_blocks;
    int first_bad = 0x7fffffff;
    for (int pb = lane; pb < npg; pb += 64 * kScanBatch) {
      int id[kScanBatch];
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u) id[u] = pb + 64 * u < npg ? row[pb + 64 * u] : 0;
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u)
        if (pb + 64 * u < npg && (unsigned)id[u] >= (unsigned)num_blocks)
          first_bad = min(first_bad, pb + 64 * u);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) first_bad = min(first_bad, __shfl_xor(first_bad, o));
    items_of(s, [&](int t0, int kp, int ke) {
      const int k = atomicAdd(&s_next[bucket(sort_keys(n, p0, ke), kp)], 1);
      if (k >= max_items) return;
      // pages the item's key tiles span
      const int kt_hi = kpart ? min((ke + kKeys - 1) / kKeys, (kp + 1) * (kpart / kKeys))
                              : (ke + kKeys - 1) / kKeys;
      const int p_hi = min(kt_hi * (kKeys / block_size), (ke + block_size - 1) / block_size);
      int32_t *r = plan + kPlanHeader + kPlanRecord * k;
      r[0] = s;
      r[1] = t0;
      r[2] = kp;
      r[3] = a;
      r[4] = n;
      r[5] = p0;
      r[6] = first_bad >= p_hi;
      r[7] = 0;
    });
  }
}

__global__ __launch_bounds__(kPlanThreads) void pa_prefill_plan(
    const int32_t *__restrict__ context_lens, const int32_t *__restrict__ query_start,
    const int32_t *__restrict__ block_tables, int max_blocks, int num_blocks, int block_size,
    int num_seqs, int num_tokens, int ctx_cap, int tok, int kpart, int max_parts, int max_items,
    int32_t *__restrict__ plan, int32_t *__restrict__ nparts) {
  prefill_plan_body(context_lens, query_start, block_tables, max_blocks, num_blocks, block_size,
                    num_seqs, num_tokens, ctx_cap, tok, kpart, max_parts, max_items, plan,
                    nparts);
}

// A prefill step's first launch: workgroup 0 writes the plan while the
// others write the step's chunk rows to the cache, kPlanThreads /
// kCacheThreads rows each.  The plan reads only context lengths, the chunk
// bounds and the block table, so the two are independent; the attention
// kernel, launched after, sees both.
constexpr int kPrepTokens = kPlanThreads / kCacheThreads;

__global__ __launch_bounds__(kPlanThreads) void pa_prefill_step_prep(
    const int32_t *__restrict__ context_lens, const int32_t *__restrict__ query_start,
    const int32_t *__restrict__ block_tables, int max_blocks, int num_blocks, int block_size,
    int num_seqs, int num_tokens, int ctx_cap, int tok, int kpart, int max_parts, int max_items,
    int32_t *__restrict__ plan, int32_t *__restrict__ nparts, const u32x4 *__restrict__ k,
    const u32x4 *__restrict__ v, u32x4 *__restrict__ k_pool, u32x4 *__restrict__ v_pool,
    const int64_t *__restrict__ slot_mapping, int num_kv_heads, int row_chunks) {
  if (blockIdx.x == 0) {
    prefill_plan_body(context_lens, query_start, block_tables, max_blocks, num_blocks,
                      block_size, num_seqs, num_tokens, ctx_cap, tok, kpart, max_parts,
                      max_items, plan, nparts);
    return;
  }
  const int t = (blockIdx.x - 1) * kPrepTokens + threadIdx.x / kCacheThreads;
  if (t < num_tokens)
    cache_write_token(t, threadIdx.x % kCacheThreads, k, v, k_pool, v_pool, slot_mapping,
                      num_kv_heads, row_chunks, block_size, (int64_t)num_blocks * block_size);
}

// ------------------------------------------------------------- work item
// Four outputs as bf16 bits through the hardware conversion (round to
// nearest even, one instruction per pair).
__device__ __forceinline__ uint2 bf16x4_bits(float a, float b, float c, float d) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 lo = {(__bf16)a, (__bf16)b};
  const bf16x2 hi = {(__bf16)c, (__bf16)d};
  return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

__device__ __forceinline__ float rows_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float rows_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int D, int BS, int G, bool AL>
__device__ __forceinline__ void prefill_item(
    void *__restrict__ out, const void *__restrict__ q, const void *__restrict__ k_pool,
    const void *__restrict__ v_pool, const int32_t *__restrict__ block_tables, int num_heads,
    int num_kv_heads, int max_blocks, int num_blocks, float scale_log2,
    const float *__restrict__ alibi, int kpart, int max_parts, float *__restrict__ ws_ml,
    float *__restrict__ ws_acc, int rec, int g) {
  using Sh = PrefillShape<D, BS, G>;
  constexpr int ROW = Sh::ROW, CPR = Sh::CPR, NC = Sh::NC, NN = Sh::NN, TILE = Sh::TILE;
  constexpr int LOADS = Sh::LOADS, TOK = Sh::TOK, PPT = Sh::PPT;
  // two buffers of [K, V]; separate arrays, so the compiler can tell that
  // reads of one buffer need not wait for the loads filling the other
  __shared__ __attribute__((aligned(16))) char s_kv0[2][TILE];
  __shared__ __attribute__((aligned(16))) char s_kv1[2][TILE];
  auto kv_buf = [&](auto buf_c) -> char(*)[TILE] {
    if constexpr (decltype(buf_c)::value == 0) return s_kv0;
    else return s_kv1;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4 = lane >> 4;
  const int j16 = lane & 15;

  // the item's plan record (lane j holds field j; uniform once read out)
  const int s = __builtin_amdgcn_readlane(rec, 0);
  const int t0 = __builtin_amdgcn_readlane(rec, 1);    // first chunk token of the block
  const int kp = __builtin_amdgcn_readlane(rec, 2);    // key partition
  const int qa = __builtin_amdgcn_readlane(rec, 3);    // the chunk's first row of q
  const int n = __builtin_amdgcn_readlane(rec, 4);     // chunk length
  const int p0 = __builtin_amdgcn_readlane(rec, 5);    // position of chunk token 0
  const bool pages_ok = __builtin_amdgcn_readlane(rec, 6) != 0;  // no page outside the pool
  const int ntok = min(TOK, n - t0);                                  // tokens of this item
  const int kv_end = max(0, p0 + t0 + ntok);                          // keys the block sees
  // this item's key tiles [kt_lo, kt_hi): partition kp of the block's keys
  const int nparts_item = kpart && kv_end > 0 ? (kv_end + kpart - 1) / kpart : 1;
  const int kt_lo = kpart ? kp * (kpart / kKeys) : 0;
  const int kt_hi = kpart ? min((kv_end + kKeys - 1) / kKeys, (kp + 1) * (kpart / kKeys))
                          : (kv_end + kKeys - 1) / kKeys;
  const int npages = (kv_end + BS - 1) / BS;
  const int32_t *bt = block_tables + (size_t)s * max_blocks;

  // this wave's token range (rows 32*wave .. 32*wave + 31)
  const int first = 32 * wave / G;
  const int last = min(ntok - 1, (32 * wave + 31) / G);
  const bool wave_live = first < ntok;
  const int wmin = p0 + t0 + first;  // position of the wave's first token
  const int wmax = p0 + t0 + last;   // and of its last

  // The exponent argument is fma(s, c, -m) with the row max m taken over
  // raw scores, which needs c > 0: a negative scale negates q instead (exact
  // in bf16), and c is kept at least FLT_MIN so that masked -inf scores stay
  // -inf (a zero scale then gives equal weights, as it should).
  const bool negate = scale_log2 < 0.f;
  const float c = fmaxf(fabsf(scale_log2), 1.17549435e-38f);
  // With ALiBi the scores are first turned into scaled logits with the bias
  // slope * (key - position) added (log2 units), and the rest of the
  // softmax runs with a unit scale.
  const float cx = AL ? 1.f : c;

  // Page ids of key tile kt, lane j holding the tile's page j (other lanes
  // load in-row entries that go unused): one vector load, issued a tile
  // ahead of the loads that use it, so a tile's loads never wait on the
  // block table.  The first two tiles' ids are loaded before the query rows,
  // so that the first tile's loads wait on them alone.
  auto tile_ids = [&](int kt) { return bt[min(kt * PPT + lane, max_blocks - 1)]; };
  const int ids_first = tile_ids(kt_lo);
  int ids_next = tile_ids(kt_lo + 1);  // page ids of tile kt + 1 while tile kt is used

  // query rows as MFMA B operands, and each row's position (-1: not a row)
  bf16x8 qf[2][NC];
  int pos[2];
  float slope[2];  // ALiBi slope of each row tile's head, log2 units
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int row = 32 * wave + 16 * t + j16;
    const int tk = row / G;
    const bool live = tk < ntok;
    pos[t] = live ? p0 + t0 + tk : -1;
    slope[t] = AL ? alibi[g * G + row % G] * kLog2e : 0.f;
    const char *qrow = reinterpret_cast<const char *>(q) +
                       ((size_t)(qa + t0 + (live ? tk : 0)) * num_heads + g * G + row % G) * ROW;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (live) w = load16(qrow + 64 * cc + 16 * q4);
      if (negate) w ^= 0x80008000u;
      qf[t][cc] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // LDS offsets of this lane's operand reads; the 16-key sub-tile and the
  // key pair add whole-row multiples that leave the swizzle unchanged
  int koff[NC], voff[NN];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) koff[cc] = j16 * ROW + swz<D>(j16, 4 * cc + q4) * 16;
  const int vr = 4 * q4 + (j16 >> 2);
#pragma unroll
  for (int nb = 0; nb < NN; ++nb)
    voff[nb] = vr * ROW + swz<D>(vr, 2 * nb + ((j16 >> 1) & 1)) * 16 + (j16 & 1) * 8;

  // global -> registers -> LDS staging of key tiles
  const size_t page_stride = (size_t)num_kv_heads * BS * ROW;
  const char *kb = reinterpret_cast<const char *>(k_pool) + (size_t)g * BS * ROW;
  const char *vb = reinterpret_cast<const char *>(v_pool) + (size_t)g * BS * ROW;
  // Load l of a thread takes chunk l * kThreads + tid of the tile, whose
  // page within the tile is the same for the whole wave (a wave's 64 chunks
  // lie in one page): the table entry and page base are scalar, the lane
  // adds its offset inside the page.
  static_assert(CPR * BS >= 64, "a wave's chunks lie in one page");
  const int wtid = __builtin_amdgcn_readfirstlane(tid & ~63);
  int loff[LOADS], lkey[LOADS];
#pragma unroll
  for (int l = 0; l < LOADS; ++l) {
    const int ci = l * kThreads + tid;
    lkey[l] = ci / CPR;
    loff[l] = (lkey[l] % BS) * ROW + swz<D>(lkey[l], ci % CPR) * 16;
  }
  // Buffer-resource loads straight into LDS (buffer_load ... lds).  Unlike
  // the global form, the compiler does not treat them as possibly touching
  // LDS through a flat address, so its LDS-read waits inside the compute
  // below stay partial while a tile's loads are in flight.  The buffer's
  // range check supplies the zeros: a lane whose offset lies past the
  // resource's size receives zeros, with no branch.
  constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw 32-bit dwords, no swizzle
  constexpr int kOutOfRange = 0x7ffffff0;
  // Tile kt into buffer buf, straight from global memory into LDS: each load
  // instruction of a wave fills 64 consecutive 16-byte slots, lane i the
  // slot of chunk column i % CPR in row i / CPR of that span, which holds
  // the row's chunk swz(row, i % CPR) (the swizzle is an XOR, so it is its
  // own inverse).  ids holds the tile's page ids (tile_ids); fetch_one
  // issues load l of the LOADS a thread makes per tile.  Chunks of keys the
  // item does not see, or on pages outside the pool, are loaded as zeros
  // through the range check.
  auto fetch_one = [&](int kt, auto buf_c, int ids, int l) {
    const int pt = (l * kThreads + wtid) / CPR / BS;  // page within the tile (uniform)
    const int pj = kt * PPT + pt;
    const int bid = __builtin_amdgcn_readlane(ids, pt);
    const bool page_ok = pj < npages && (unsigned)bid < (unsigned)num_blocks;
    const bool ok = page_ok && kt * kKeys + lkey[l] < kv_end;
    const size_t base = (size_t)(page_ok ? bid : 0) * page_stride;
    const int span = (l * kThreads + wtid) / CPR * ROW;  // uniform LDS offset
    // the resource spans the head's rows of one page; an offset past it
    // reads zeros
    const auto rk = __builtin_amdgcn_make_buffer_rsrc((void *)(kb + base), 0, BS * ROW, kRsrcWord3);
    const auto rv = __builtin_amdgcn_make_buffer_rsrc((void *)(vb + base), 0, BS * ROW, kRsrcWord3);
    const int off = ok ? loff[l] : kOutOfRange;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_char *)kv_buf(buf_c)[0] + span, 16, off, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_char *)kv_buf(buf_c)[1] + span, 16, off, 0, 0, 0);
  };
  auto fetch = [&](int kt, auto buf_c, int ids) {
#pragma unroll
    for (int l = 0; l < LOADS; ++l) fetch_one(kt, buf_c, ids, l);
  };
  // tiles that hold no key the item does not see and no page outside the pool
  auto tile_clean = [&](int kt) { return pages_ok && (kt + 1) * kKeys <= kv_end; };

  // softmax state per row tile: running max m (scaled, log2 units), the
  // lane's partial sum, O^T columns
  float m[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f};
  f32x4 o[2][NN];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int nb = 0; nb < NN; ++nb) o[t][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // S^T for one 32-key half of a tile (two 16-key sub-tiles, both row tiles)
  // K operands of one 32-key part: two 16-key sub-tiles x NC head_dim slabs
  auto load_k = [&](const lds_char *ks, int h, bf16x8 (&ka)[2][NC]) {
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int cc = 0; cc < NC; ++cc)
        ka[st][cc] = *(const __attribute__((address_space(3))) bf16x8 *)(
            ks + (32 * h + 16 * st) * ROW + koff[cc]);
  };
  auto scores = [&](const bf16x8 (&ka)[2][NC], f32x4 (&sacc)[2][2]) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      sacc[st][0] = f32x4{0.f, 0.f, 0.f, 0.f};
      sacc[st][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        sacc[st][0] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[st][cc], qf[0][cc], sacc[st][0], 0, 0, 0);
        sacc[st][1] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[st][cc], qf[1][cc], sacc[st][1], 0, 0, 0);
      }
    }
  };
  // scores of keys a row does not see (past its position, or on a page
  // outside the pool) to -inf
  auto mask = [&](f32x4 (&sacc)[2][2], int kt, int h) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int k16 = 32 * h + 16 * st;    // first key of the sub-tile in the tile
      const int pj = kt * PPT + k16 / BS;  // a sub-tile lies in one page
      const bool page_ok =
          pj < npages && (pages_ok || (unsigned)bt[pj] < (unsigned)num_blocks);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kk = kt * kKeys + k16 + 4 * q4 + r;
          if (!(page_ok && kk <= pos[t])) sacc[st][t][r] = -INFINITY;
        }
    }
  };
  // ALiBi: scores -> scaled logits plus slope * (key - position)
  auto add_bias = [&](f32x4 (&sacc)[2][2], int kt, int h) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float sb = slope[t] * (float)(kt * kKeys + 32 * h + 4 * q4 - pos[t]);
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          sacc[st][t][r] = fmaf(sacc[st][t][r], c, fmaf(slope[t], (float)(16 * st + r), sb));
    }
  };
  // The running max moves only when some row's grows by more than
  // 2^kRescaleLog2 (weights stay below that bound, and the base cancels
  // between the weighted sum and the sum of weights).  The check compares
  // each lane's raw maximum with its row's threshold (m + kRescaleLog2) / c
  // and takes one ballot; the row-wide maximum is formed only in the rare
  // rescale.
  float thr[2] = {-INFINITY, -INFINITY};
  auto update_max = [&](const f32x4 (&sacc)[2][2]) {
    float mx[2];
    bool grow = false;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      mx[t] = fmaxf(fmaxf(fmaxf(sacc[0][t][0], sacc[0][t][1]), fmaxf(sacc[0][t][2], sacc[0][t][3])),
                    fmaxf(fmaxf(sacc[1][t][0], sacc[1][t][1]), fmaxf(sacc[1][t][2], sacc[1][t][3])));
      grow = grow || mx[t] > thr[t];
    }
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const float mn = fmaxf(m[t], rows_max(mx[t]) * cx);
        const float alpha = mn == -INFINITY ? 1.f : fast_exp2(m[t] - mn);
        m[t] = mn;
        thr[t] = (mn + kRescaleLog2) / cx;
        lsum[t] *= alpha;
#pragma unroll
        for (int nb = 0; nb < NN; ++nb) o[t][nb] *= alpha;
      }
    }
  };
  // weights as bf16 B operands (keys 4*q4 + r of sub-tile 0, then of 1).
  // With ALiBi the attention can rest on a handful of nearby keys, so there
  // the weights enter as a bf16 pair hi + lo (about 16 significant bits) at
  // the cost of a second instruction per tile.
  auto weights = [&](const f32x4 (&sacc)[2][2], i16x8 (&pb)[2], i16x8 (&pl)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float base = m[t] == -INFINITY ? 0.f : m[t];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = fast_exp2(fmaf(sacc[st][t][r], cx, -base));
          lsum[t] += p;
          const __bf16 hi = (__bf16)p;
          pb[t][4 * st + r] = __builtin_bit_cast(short, hi);
          if constexpr (AL) pl[t][4 * st + r] = __builtin_bit_cast(short, (__bf16)(p - (float)hi));
        }
    }
  };
  // V^T operands of one 32-key part: two transposing reads per 16 columns
  auto load_v = [&](const lds_char *vs, int h, bf16x8 (&va)[NN]) {
#pragma unroll
    for (int nb = 0; nb < NN; ++nb) {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4 *)(vs + 32 * h * ROW + voff[nb]));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4 *)(vs + (32 * h + 16) * ROW + voff[nb]));
      va[nb] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  // O^T += V^T P^T with the part's 32 keys as the reduction dimension
  auto pv = [&](const bf16x8 (&va)[NN], const i16x8 (&pb)[2], const i16x8 (&pl)[2]) {
#pragma unroll
    for (int nb = 0; nb < NN; ++nb) {
      o[0][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[nb], __builtin_bit_cast(bf16x8, pb[0]),
                                                         o[0][nb], 0, 0, 0);
      o[1][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[nb], __builtin_bit_cast(bf16x8, pb[1]),
                                                         o[1][nb], 0, 0, 0);
      if constexpr (AL) {
        o[0][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            va[nb], __builtin_bit_cast(bf16x8, pl[0]), o[0][nb], 0, 0, 0);
        o[1][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            va[nb], __builtin_bit_cast(bf16x8, pl[1]), o[1][nb], 0, 0, 0);
      }
    }
  };
  // One tile, in 32-key parts, software pipelined over the LDS reads: a
  // part's V operands are read at its start and used at its end, and the K
  // operands are read one part ahead.  Each part's scores are computed
  // before the previous part's exponentials and P.V, so those matrix
  // instructions can run beside the vector work.
  auto compute = [&](auto masked_c, auto buf_c, int kt, auto after_first_part) {
    constexpr bool kMasked = decltype(masked_c)::value;
    constexpr int kParts = kKeys / 32;
    const lds_char *ks = (const lds_char *)kv_buf(buf_c)[0];
    const lds_char *vs = (const lds_char *)kv_buf(buf_c)[1];
    f32x4 sc[2][2][2];     // scores of two parts in flight: [slot][sub-tile][row tile]
    bf16x8 ka[2][NC];      // K operands of one part
    bf16x8 va[NN];         // V^T operands of one part
    i16x8 pb[2], pl[2];
    // ALiBi's second weight operand leaves no registers for K one part ahead
    constexpr bool kAhead = !AL;
    load_k(ks, 0, ka);
    scores(ka, sc[0]);
    if constexpr (AL) add_bias(sc[0], kt, 0);
    if constexpr (kMasked) mask(sc[0], kt, 0);
    if constexpr (kAhead) load_k(ks, 1, ka);
    update_max(sc[0]);
#pragma unroll
    for (int h = 0; h < kParts; ++h) {
      // keep the scheduler from hoisting one part's LDS reads into another's
      // work, which would raise register pressure past the budget
      __builtin_amdgcn_sched_barrier(0);
      if (h == 1) {
        after_first_part();
        __builtin_amdgcn_sched_barrier(0);
      }
      load_v(vs, h, va);
      if (h + 1 < kParts) {
        if constexpr (!kAhead) load_k(ks, h + 1, ka);
        scores(ka, sc[(h + 1) & 1]);
        if constexpr (AL) add_bias(sc[(h + 1) & 1], kt, h + 1);
        if constexpr (kMasked) mask(sc[(h + 1) & 1], kt, h + 1);
      }
      weights(sc[h & 1], pb, pl);
      if (kAhead && h + 2 < kParts) load_k(ks, h + 2, ka);
      pv(va, pb, pl);
      if (h + 1 < kParts) update_max(sc[(h + 1) & 1]);
    }
  };
  // one key tile: start the loads of the next tile into the other buffer
  // (read before the last barrier), use this one; the barrier's fence waits
  // for the loads.  The buffer index is a compile-time constant, so every
  // LDS address is a lane offset plus an immediate.
  auto step = [&](auto masked_c, auto buf_c, int kt) {
    constexpr int buf = decltype(buf_c)::value;
    using Next = std::integral_constant<int, buf ^ 1>;
    // The two waves of a SIMD issue the next tile's loads at different
    // times: the first four waves right away, the other four after their
    // first 32-key part (or right away when they skip the tile), so that
    // while one waits for the load unit to take its loads the other
    // computes.
    const bool more = kt + 1 < kt_hi;
    const bool run = wave_live && kt * kKeys <= wmax;
    const bool early = wave < 4 || !run;
    const int ids = ids_next;
    if (more && early) fetch(kt + 1, Next{}, ids);
    if (more) ids_next = tile_ids(kt + 2);
    if (run)
      compute(masked_c, buf_c, kt, [&] {
        if (more && !early) fetch(kt + 1, Next{}, ids);
      });
    __syncthreads();
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using Clean = std::integral_constant<bool, false>;
  using Masked = std::integral_constant<bool, true>;

  // Each wave first runs the tiles that lie wholly below its first row's
  // position on valid pages (no per-key mask), then the rest.  Every wave
  // takes one barrier per tile, so the two loops of different waves stay in
  // step.  Buffer 0 holds the item's even tiles counted from kt_lo.
  if (kt_hi > kt_lo) {
    fetch(kt_lo, B0{}, ids_first);
    __syncthreads();
    const int clean_end = wave_live ? min(kt_hi, max(kt_lo, (wmin + 1) / kKeys)) : kt_lo;
    int kt = kt_lo;
    for (; kt + 1 < clean_end && tile_clean(kt) && tile_clean(kt + 1); kt += 2) {
      step(Clean{}, B0{}, kt);
      step(Clean{}, B1{}, kt + 1);
    }
    // kt - kt_lo is even here: the clean loop takes tiles in pairs
    for (; kt < kt_hi; kt += 2) {
      step(Masked{}, B0{}, kt);
      if (kt + 1 < kt_hi) step(Masked{}, B1{}, kt + 1);
    }
  }

  // Store: lane (q4, j) holds d = 16n + 4*q4 .. +3 of row j.  A block with
  // one key partition writes its normalised output; otherwise each item
  // writes its partition's (max, sum, unnormalised sum of weighted V) for
  // the reduce kernel.
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float L = rows_sum(lsum[t]);
    const int row = 32 * wave + 16 * t + j16;
    const int tk = row / G;
    if (tk >= ntok) continue;
    const size_t grow = (size_t)(qa + t0 + tk) * num_heads + g * G + row % G;
    if (nparts_item == 1) {
      const float inv = L > 0.f ? 1.f / L : 0.f;
      char *orow = reinterpret_cast<char *>(out) + grow * ROW;
#pragma unroll
      for (int nb = 0; nb < NN; ++nb)
        *reinterpret_cast<uint2 *>(orow + (16 * nb + 4 * q4) * 2) =
            bf16x4_bits(o[t][nb][0] * inv, o[t][nb][1] * inv, o[t][nb][2] * inv,
                        o[t][nb][3] * inv);
    } else {
      const size_t slot = grow * max_parts + kp;
      float *acc = ws_acc + slot * D;
#pragma unroll
      for (int nb = 0; nb < NN; ++nb)
        *reinterpret_cast<float4 *>(acc + 16 * nb + 4 * q4) =
            make_float4(o[t][nb][0], o[t][nb][1], o[t][nb][2], o[t][nb][3]);
      if (q4 == 0) {
        ws_ml[slot * 2] = m[t];
        ws_ml[slot * 2 + 1] = L;
      }
    }
  }
}

// Merge of the key partitions of the rows whose block was split: one wave
// per (row, query head), out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p.
// Lanes hold the partitions' (m, l) 64 at a time; each partition's weight
// is then broadcast while the lanes stream its D accumulator values.  With
// at most kReduceBatch partitions a lane loads its values of every
// partition, and the statistics, before using any of them, so the wave
// waits on memory once; the sums are taken in the same order either way.
constexpr int kReduceBatch = 16;

// A merged row: acc / L in bf16 (zeros where no key was seen).
template <int D>
__device__ __forceinline__ void store_row(void *out, long long rh, int lane,
                                          const float (&acc)[D / 64], float L) {
  constexpr int DPL = D / 64;
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t *dst = reinterpret_cast<uint16_t *>(out) + rh * D + lane * DPL;
  if constexpr (DPL == 2)
    *reinterpret_cast<uint32_t *>(dst) =
        BF16::round_bits(acc[0] * inv) | (BF16::round_bits(acc[1] * inv) << 16);
  else
    dst[0] = (uint16_t)BF16::round_bits(acc[0] * inv);
}

template <int D>
__global__ __launch_bounds__(256) void pa_prefill_reduce(
    void *__restrict__ out, const float *__restrict__ ws_ml, const float *__restrict__ ws_acc,
    const int32_t *__restrict__ nparts, int num_tokens, int num_heads, int max_parts) {
  constexpr int DPL = D / 64;  // outputs per lane
  using Vec = std::conditional_t<DPL == 2, float2, float>;
  const int lane = threadIdx.x & 63;
  const long long rh = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);  // (row, head)
  if (rh >= (long long)num_tokens * num_heads) return;
  const int np = min(nparts[rh / num_heads], max_parts);
  if (np <= 1) return;  // written by its item
  const float2 *ml = reinterpret_cast<const float2 *>(ws_ml) + rh * max_parts;
  float acc[DPL] = {}, L = 0.f;
  if (np <= kReduceBatch) {
    const float *a = ws_acc + rh * max_parts * D + lane * DPL;
    const float2 st = lane < np ? ml[lane] : make_float2(-INFINITY, 0.f);
    Vec v[kReduceBatch];
#pragma unroll
    for (int p = 0; p < kReduceBatch; ++p)
      if (p < np) v[p] = *reinterpret_cast<const Vec *>(a + (size_t)p * D);
    const float M = wave_max(st.x);
    if (M != -INFINITY) {
      const float w = lane < np ? fast_exp2(st.x - M) : 0.f;
      L = wave_sum(lane < np ? fmaf(st.y, w, 0.f) : 0.f);
#pragma unroll
      for (int p = 0; p < kReduceBatch; ++p) {
        if (p < np) {
          const float wq = __shfl(w, p);
          if constexpr (DPL == 2) {
            acc[0] = fmaf(v[p].x, wq, acc[0]);
            acc[1] = fmaf(v[p].y, wq, acc[1]);
          } else {
            acc[0] = fmaf(v[p], wq, acc[0]);
          }
        }
      }
    }
    store_row<D>(out, rh, lane, acc, L);
    return;
  }
  float M = -INFINITY;
  for (int p = lane; p < np; p += 64) M = fmaxf(M, ml[p].x);
  M = wave_max(M);
  if (M != -INFINITY) {
    const float *a = ws_acc + rh * max_parts * D + lane * DPL;
    for (int p0 = 0; p0 < np; p0 += 64) {
      float w = 0.f;
      if (p0 + lane < np) {
        const float2 st = ml[p0 + lane];
        w = fast_exp2(st.x - M);
        L = fmaf(st.y, w, L);
      }
      const int cnt = min(64, np - p0);
#pragma unroll 4
      for (int q = 0; q < cnt; ++q) {
        const float wq = __shfl(w, q);
        const Vec v = *reinterpret_cast<const Vec *>(a + (size_t)(p0 + q) * D);
        if constexpr (DPL == 2) {
          acc[0] = fmaf(v.x, wq, acc[0]);
          acc[1] = fmaf(v.y, wq, acc[1]);
        } else {
          acc[0] = fmaf(v, wq, acc[0]);
        }
      }
    }
    L = wave_sum(L);
  }
  store_row<D>(out, rh, lane, acc, L);
}

template <int D, int BS, int G, bool AL>
__global__ __launch_bounds__(kThreads, 2) void pa_prefill_gqa(
    void *__restrict__ out, const void *__restrict__ q, const void *__restrict__ k_pool,
    const void *__restrict__ v_pool, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ plan, int num_heads, int num_kv_heads, int max_blocks,
    int num_blocks, float scale_log2, const float *__restrict__ alibi, int kpart,
    int max_parts, float *__restrict__ ws_ml, float *__restrict__ ws_acc) {
  const int items = plan[0] * num_kv_heads;
  // an item's plan record, lane j holding field j; loaded one item ahead, so
  // an item starts without waiting on the plan (past the last item: the
  // first record, unused)
  auto record = [&](int it) {
    const int r = it < items ? it / num_kv_heads : 0;
    return plan[kPlanHeader + kPlanRecord * r + (int)(threadIdx.x & (kPlanRecord - 1))];
  };
  static_assert((kPlanRecord & (kPlanRecord - 1)) == 0, "record fields by lane mask");
  int it = snake_item(0);
  int rec = record(it);
  for (int k = 0; it < items; ++k) {
    const int it_next = snake_item(k + 1);
    const int rec_next = record(it_next);
    prefill_item<D, BS, G, AL>(out, q, k_pool, v_pool, block_tables, num_heads, num_kv_heads,
                               max_blocks, num_blocks, scale_log2, alibi, kpart, max_parts,
                               ws_ml, ws_acc, rec, it % num_kv_heads);
    __syncthreads();  // the next item reuses the LDS
    it = it_next;
    rec = rec_next;
  }
}

template <int D, int BS, int G, bool AL>
int launch_al(const pa_internal::PrefillLaunch &a) {
  hipStream_t st = reinterpret_cast<hipStream_t>(a.stream);
  auto kernel = pa_prefill_gqa<D, BS, G, AL>;
  static const int per_cu =
      pa_internal::blocks_per_cu(reinterpret_cast<const void *>(kernel), kThreads);
  // items <= num_tokens * max_parts (each block holds at least one token)
  const unsigned grid = pa_internal::persistent_grid_items(
      (long long)a.num_tokens * a.max_parts * a.num_kv_heads, per_cu);
  if (grid == 0) return 6;
  pa_internal::launch_timed(kernel, dim3(grid), dim3(kThreads), st, a.ev_begin, a.ev_end, a.out,
                            a.q, a.k_pool, a.v_pool,
                     a.block_tables, a.plan, a.num_heads, a.num_kv_heads, a.max_blocks,
                     a.num_blocks, a.scale * kLog2e, a.alibi, a.part_tokens, a.max_parts,
                     a.ws_ml, a.ws_acc);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

template <int D, int BS, int G>
int launch(const pa_internal::PrefillLaunch &a) {
  return a.alibi ? launch_al<D, BS, G, true>(a) : launch_al<D, BS, G, false>(a);
}

template <int D, int BS>
int by_group(const pa_internal::PrefillLaunch &a) {
  switch (a.num_heads / a.num_kv_heads) {
    case 1: return launch<D, BS, 1>(a);
    case 2: return launch<D, BS, 2>(a);
    case 4: return launch<D, BS, 4>(a);
    case 8: return launch<D, BS, 8>(a);
  }
  return 3;
}

}  // namespace

namespace pa_internal {

namespace {

// The plan launch of a prefill call, or with a cache write (cache not
// null), the step's preparation kernel that does both.
int run_prefill(const PrefillLaunch &a, const CacheLaunch *cache) {
  hipStream_t st = reinterpret_cast<hipStream_t>(a.stream);
  const int tok = kPrefillRows / (a.num_heads / a.num_kv_heads);
  if (cache) {
    const unsigned grid = 1 + (unsigned)((a.num_tokens + kPrepTokens - 1) / kPrepTokens);
    hipLaunchKernelGGL(pa_prefill_step_prep, dim3(grid), dim3(kPlanThreads), 0, st,
                       a.context_lens, a.query_start, a.block_tables, a.max_blocks,
                       a.num_blocks, a.block_size, a.num_seqs, a.num_tokens,
                       a.max_blocks * a.block_size, tok, a.part_tokens, a.max_parts,
                       a.num_tokens * a.max_parts, a.plan, a.nparts,
                       static_cast<const u32x4 *>(cache->k), static_cast<const u32x4 *>(cache->v),
                       static_cast<u32x4 *>(cache->k_pool), static_cast<u32x4 *>(cache->v_pool),
                       cache->slot_mapping, cache->num_kv_heads,
                       a.head_dim * cache->elem_bytes / 16);
  } else {
    hipLaunchKernelGGL(pa_prefill_plan, dim3(1), dim3(kPlanThreads), 0, st, a.context_lens,
                       a.query_start, a.block_tables, a.max_blocks, a.num_blocks, a.block_size,
                       a.num_seqs, a.num_tokens, a.max_blocks * a.block_size, tok,
                       a.part_tokens, a.max_parts, a.num_tokens * a.max_parts, a.plan, a.nparts);
  }
  if (hipGetLastError() != hipSuccess) return 6;
  // the attention kernel's launch records the timing events, if any
  int rc;
  if (a.head_dim == 64)
    rc = a.block_size == 16 ? by_group<64, 16>(a) : by_group<64, 32>(a);
  else
    rc = a.block_size == 16 ? by_group<128, 16>(a) : by_group<128, 32>(a);
  if (rc != 0) return rc;
  if (a.max_parts > 1) {
    const long long rows = (long long)a.num_tokens * a.num_heads;
    auto reduce = a.head_dim == 64 ? pa_prefill_reduce<64> : pa_prefill_reduce<128>;
    hipLaunchKernelGGL(reduce, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, a.out,
                       a.ws_ml, a.ws_acc, a.nparts, a.num_tokens, a.num_heads, a.max_parts);
    if (hipGetLastError() != hipSuccess) return 6;
  }
  return 0;
}

}  // namespace

int launch_prefill(const PrefillLaunch &a) { return run_prefill(a, nullptr); }

int launch_prefill_step(const PrefillLaunch &a, const CacheLaunch &cache) {
  return run_prefill(a, &cache);
}

}  // namespace pa_internal
