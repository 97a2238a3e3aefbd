// Paged decode attention, partition pass (VALU path) and log-sum-exp reduce.
//
// Method (vLLM / PagedAttention pages): the KV cache is a pool of fixed-size
// pages; a per-sequence page table maps logical to physical pages and the
// attention kernel reads the pages through that table directly, with no
// gather copy and no padding (showapi.com article, section 2.1; tutorial
// page, section 4.2).
//
// This file holds the VALU partition kernel (every dtype and head group;
// used for fp32 and for bf16 with one query head per kv-head), the reduce
// kernel that merges split-K partitions, and the dispatch that picks the
// partition kernel.  The grouped-query bf16 kernel on the matrix cores is
// in pagedattn_decode_gqa.hip.
//
// Lane layout of the VALU kernel: each (page, kv-head) run of
// block_size * head_dim elements is read as whole 16-byte chunks; lane l,
// load i takes chunk i*64 + l, so every load instruction covers 1 KiB of
// consecutive bytes.  With R = chunks per token row, a load instruction holds
// 64/R tokens and lane l always sees the same R-chunk column (l % R) of
// token rows (l / R) + i*64/R.  The partial q.K dot products of a row are
// summed across its R lanes with DPP row operations, so every lane of the
// row ends up holding the full logit.  Softmax is the online form (running
// max, rescaled running sum and accumulator) in log2 units, with log2(e)
// folded into the scale.
#include <atomic>

#include "pagedattn_cache_row.h"
#include "pagedattn_device.h"
#include "pagedattn_internal.h"
#include "pagedattn_probe_launch.h"
#include "pagedattn_step_launch.h"
#include "pagedattn_timed_launch.h"

namespace {

using namespace pa_dev;
using pa_internal::kMaxPartitionPages;
using pa_internal::kPlanHeader;

// ------------------------------------------------------ decode, partition pass
// One workgroup of NW wavefronts per unit (sequence s, kv-head g, partition
// p of at most part_pages pages).  The unit's pages are dealt to its waves
// in turn: wave w takes partition pages w, w + NW, w + 2 NW, ...  Each wave
// keeps a running (max, sum, V accumulator) for the G query heads of g over
// its own pages, with PF pages of K and V in flight; the NW partial states
// are merged through LDS at the end, which is the same log-sum-exp merge the
// reduce kernel applies across partitions.
//
// Scheduling: a plan kernel sorts the (sequence, partition) units by size,
// largest first, and a persistent grid (as many workgroups as the GPU holds
// at once) walks that list with the kv-head fastest; see pa_decode_plan and
// pa_decode_partition below.
template <class T, int D, int BS, int G>
struct DecodeShape {
  static constexpr int E = T::kPerChunk;       // elements per 16-byte chunk
  static constexpr int R = D / E;              // lanes (chunks) per token row
  static constexpr int TPI = 64 / R;           // token rows per load instruction
  static constexpr int NLD = BS / TPI;         // load instructions per page
  static constexpr int PAGE_BYTES = BS * D * T::kBytes;
  static_assert(NLD * 1024 == PAGE_BYTES, "a page is whole 1 KiB wave loads");
  // pages in flight per wave: two where the registers allow it
  static constexpr int PF = (NLD <= 4 && G <= 2) ? 2 : 1;
};

template <class T, int D, int BS, int G>
struct WaveSoftmax {
  using S = DecodeShape<T, D, BS, G>;
  float m[G];           // running max of the logits, log2 units (wave-uniform)
  float l[G];           // this lane's share of the running sum
  float acc[G][S::E];   // this lane's share of sum p * V over its d-chunk

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = -INFINITY;
      l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < S::E; ++e) acc[h][e] = 0.f;
    }
  }

  // Fold one page into the state.  tok0: logical index of the page's first
  // token; live: whether the page id was valid; rg: this lane's token-row
  // group.  Tokens at or past ctx get weight exactly 0 and their V is never
  // used in arithmetic (a masked slot may hold NaN).
  // With ALiBi, slope[h] (log2 units) times the token's distance behind the
  // query, (token - (ctx - 1)), is added to head h's logit.
  template <bool AL>
  __device__ __forceinline__ void page(const u32x4 (&qc)[G], const u32x4 (&kc)[S::NLD],
                                       const u32x4 (&vc)[S::NLD], int tok0, int ctx, bool live,
                                       int rg, float scale_log2, const float (&slope)[G]) {
    float lg[S::NLD][G];
#pragma unroll
    for (int i = 0; i < S::NLD; ++i)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        lg[i][h] = row_sum<S::R>(T::dot(qc[h], kc[i])) * scale_log2;
        if constexpr (AL)
          lg[i][h] = fmaf(slope[h], (float)(tok0 + i * S::TPI + rg - (ctx - 1)), lg[i][h]);
      }
    bool keep[S::NLD];
#pragma unroll
    for (int i = 0; i < S::NLD; ++i) {
      keep[i] = live && (tok0 + i * S::TPI + rg < ctx);
      if (!keep[i])
#pragma unroll
        for (int h = 0; h < G; ++h) lg[i][h] = -INFINITY;
    }
    float p[S::NLD][G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float pm = lg[0][h];
#pragma unroll
      for (int i = 1; i < S::NLD; ++i) pm = fmaxf(pm, lg[i][h]);
      pm = group_max<S::R>(pm);
      const float mn = fmaxf(m[h], pm);
      if (mn == -INFINITY) {
        // nothing live so far (only possible when page ids are invalid)
#pragma unroll
        for (int i = 0; i < S::NLD; ++i) p[i][h] = 0.f;
        continue;
      }
      const float alpha = fast_exp2(m[h] - mn);
      m[h] = mn;
      l[h] *= alpha;
#pragma unroll
      for (int e = 0; e < S::E; ++e) acc[h][e] *= alpha;
#pragma unroll
      for (int i = 0; i < S::NLD; ++i) {
        p[i][h] = fast_exp2(lg[i][h] - mn);
        l[h] += p[i][h];
      }
    }
#pragma unroll
    for (int i = 0; i < S::NLD; ++i) {
      float vf[S::E];
      T::unpack(vc[i], vf);
      if (!keep[i])
#pragma unroll
        for (int e = 0; e < S::E; ++e) vf[e] = 0.f;
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < S::E; ++e) acc[h][e] = fmaf(p[i][h], vf[e], acc[h][e]);
    }
  }
};

// One work unit: the G query heads of kv-head g over partition `part` of
// sequence s.  All threads of the workgroup call it with the same unit.
template <class T, int D, int BS, int G, int NW, bool AL>
__device__ __forceinline__ void decode_unit(
    void *__restrict__ out, const void *__restrict__ q, const void *__restrict__ k_pool,
    const void *__restrict__ v_pool, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ context_lens, float *__restrict__ ws_ml,
    float *__restrict__ ws_acc, int num_heads, int num_kv_heads, int max_blocks,
    int num_blocks, int part_pages, int max_parts, float scale_log2,
    const float *__restrict__ alibi, int s, int g, int part) {
  using S = DecodeShape<T, D, BS, G>;
  constexpr int E = S::E, R = S::R, NLD = S::NLD, PAGE_BYTES = S::PAGE_BYTES;
  __shared__ float s_ml[NW][G][2];
  __shared__ __attribute__((aligned(16))) float s_acc[NW][G][D];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int dc = lane % R;
  const int rg = lane / R;
  const int h0 = g * G;
  const int p_begin = part * part_pages;

  // Independent loads first: the context length, this wave's page ids (one
  // per lane; columns past the context are loaded but never used) and q.
  int ctx = context_lens[s];
  const int col = p_begin + wave + NW * lane;
  int my_bid = -1;
  if (wave + NW * lane < part_pages && col < max_blocks)
    my_bid = block_tables[(size_t)s * max_blocks + col];
  const size_t head_row_bytes = (size_t)D * T::kBytes;
  u32x4 qc[G];
  const char *q_b = reinterpret_cast<const char *>(q);
#pragma unroll
  for (int h = 0; h < G; ++h)
    qc[h] = load16(q_b + ((size_t)s * num_heads + h0 + h) * head_row_bytes + dc * 16);

  ctx = min(max(ctx, 0), max_blocks * BS);
  const int npages = (ctx + BS - 1) / BS;
  char *out_b = reinterpret_cast<char *>(out);
  if (ctx == 0) {
    if (part == 0 && wave == 0 && rg == 0) {
      float z[E];
#pragma unroll
      for (int e = 0; e < E; ++e) z[e] = 0.f;
#pragma unroll
      for (int h = 0; h < G; ++h)
        *reinterpret_cast<u32x4 *>(out_b + ((size_t)s * num_heads + h0 + h) * head_row_bytes +
                                   dc * 16) = T::pack(z);
    }
    return;
  }
  if (p_begin >= npages) return;
  const int np = min(npages - p_begin, part_pages);
  const int np_w = wave < np ? (np - wave + NW - 1) / NW : 0;  // this wave's pages

  WaveSoftmax<T, D, BS, G> st;
  st.init();
  float slope[G];
#pragma unroll
  for (int h = 0; h < G; ++h) slope[h] = AL ? alibi[h0 + h] * kLog2e : 0.f;
  const size_t page_stride = (size_t)num_kv_heads * PAGE_BYTES;
  const char *k_b = reinterpret_cast<const char *>(k_pool) + (size_t)g * PAGE_BYTES + lane * 16;
  const char *v_b = reinterpret_cast<const char *>(v_pool) + (size_t)g * PAGE_BYTES + lane * 16;

  // page j of this wave: its id, whether it is valid, and its loads
  auto fetch = [&](u32x4 (&kc)[NLD], u32x4 (&vc)[NLD], int j) -> bool {
    const int bid = __builtin_amdgcn_readlane(my_bid, j);
    const bool ok = (unsigned)bid < (unsigned)num_blocks;
    const size_t off = (size_t)(ok ? bid : 0) * page_stride;  // an invalid id reads page 0, unused
#pragma unroll
    for (int i = 0; i < NLD; ++i) kc[i] = load_kv16(k_b + off + i * 1024);
#pragma unroll
    for (int i = 0; i < NLD; ++i) vc[i] = load_kv16(v_b + off + i * 1024);
    return ok;
  };
  auto tok0 = [&](int j) { return (p_begin + wave + NW * j) * BS; };

  if constexpr (S::PF == 2) {
    // Two buffers, one page ahead.  Inside the loop every fetch is
    // unconditional, so the number of loads in flight is the same on every
    // path and the compiler's wait before a page's use lets the next page's
    // loads stay outstanding; the last one or two pages are done after it.
    if (np_w > 0) {
      u32x4 ka[NLD], va[NLD], kb[NLD], vb[NLD];
      bool oka = fetch(ka, va, 0), okb;
      int j = 0;
      for (; j + 2 < np_w; j += 2) {
        okb = fetch(kb, vb, j + 1);
        st.template page<AL>(qc, ka, va, tok0(j), ctx, oka, rg, scale_log2, slope);
        oka = fetch(ka, va, j + 2);
        st.template page<AL>(qc, kb, vb, tok0(j + 1), ctx, okb, rg, scale_log2, slope);
      }
      if (j + 1 < np_w) {
        okb = fetch(kb, vb, j + 1);
        st.template page<AL>(qc, ka, va, tok0(j), ctx, oka, rg, scale_log2, slope);
        st.template page<AL>(qc, kb, vb, tok0(j + 1), ctx, okb, rg, scale_log2, slope);
      } else {
        st.template page<AL>(qc, ka, va, tok0(j), ctx, oka, rg, scale_log2, slope);
      }
    }
  } else {
    for (int j = 0; j < np_w; ++j) {
      u32x4 kc[NLD], vc[NLD];
      const bool ok = fetch(kc, vc, j);
      st.template page<AL>(qc, kc, vc, tok0(j), ctx, ok, rg, scale_log2, slope);
    }
  }

  // this wave's totals: sum the row groups' shares
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st.l[h] = group_sum<R>(st.l[h]);
#pragma unroll
    for (int e = 0; e < E; ++e) st.acc[h][e] = group_sum<R>(st.acc[h][e]);
  }
  if (rg == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < E; e += 4)
        *reinterpret_cast<float4 *>(&s_acc[wave][h][dc * E + e]) =
            make_float4(st.acc[h][e], st.acc[h][e + 1], st.acc[h][e + 2], st.acc[h][e + 3]);
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s_ml[wave][h][0] = st.m[h];
      s_ml[wave][h][1] = st.l[h];
    }
  }
  __syncthreads();

  merge_waves<T, D, G, NW>(
      [&](int w, int h, int d) -> float4 {
        return *reinterpret_cast<const float4 *>(&s_acc[w][h][d]);
      },
      [&](int w, int h) { return s_ml[w][h][0]; }, [&](int w, int h) { return s_ml[w][h][1]; },
      npages <= part_pages, out_b + ((size_t)s * num_heads + h0) * head_row_bytes,
      ws_acc + (((size_t)s * max_parts + part) * num_heads + h0) * D,
      ws_ml + (((size_t)s * max_parts + part) * num_heads + h0) * 2);
}

// Partition kernel: a grid of up to kDecodeGridRounds times what the GPU
// holds at once walks the unit list the plan kernel wrote, largest units
// first, item i = (list[i / num_kv_heads], kv-head i % num_kv_heads), in the
// snake order of snake_item.  Workgroups past the resident ones start as
// earlier ones finish, so the hardware's dispatcher hands the list out
// greedily.  Kv-head fastest puts the heads of one unit on workgroups that
// start together on different XCDs (the hardware hands consecutive
// workgroups to the 8 XCDs in turn).
template <class T, int D, int BS, int G, int NW, bool AL>
__global__ __launch_bounds__(64 * NW) void pa_decode_partition(
    void *__restrict__ out, const void *__restrict__ q, const void *__restrict__ k_pool,
    const void *__restrict__ v_pool, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ context_lens, float *__restrict__ ws_ml,
    float *__restrict__ ws_acc, const int32_t *__restrict__ plan, int num_seqs, int num_heads,
    int num_kv_heads, int max_blocks, int num_blocks, int part_pages, int max_parts,
    float scale_log2, const float *__restrict__ alibi) {
  // the list holds num_seqs * max_parts entries, -1 past the last unit
  const long long bound = (long long)num_seqs * max_parts * num_kv_heads;
  for (int k = 0;; ++k) {
    const int it = snake_item(k);
    if (it >= bound) break;
    const int unit = plan[kPlanHeader + it / num_kv_heads];
    if (unit < 0) break;
    decode_unit<T, D, BS, G, NW, AL>(out, q, k_pool, v_pool, block_tables, context_lens, ws_ml,
                                     ws_acc, num_heads, num_kv_heads, max_blocks, num_blocks,
                                     part_pages, max_parts, scale_log2, alibi, unit / max_parts,
                                     it % num_kv_heads, unit % max_parts);
    __syncthreads();  // the next unit reuses the LDS the merge just read
  }
}

// ----------------------------------------------------------- decode, plan
// One workgroup orders the (sequence, partition) units for the partition
// kernels: a counting sort by page count, largest first, so the shortest
// units finish the pass and no workgroup starts a long unit at the end.  A
// sequence with context 0 gets one unit of size 0 (its output rows are
// written as zeros).  Layout: plan[0] = unit count, plan[kPlanHeader + k] =
// sequence * max_parts + partition for k below the count, -1 from there to
// num_seqs * max_parts, so a partition workgroup finds its unit, or that it
// has none, with one load.  Threads take candidate units (sequence,
// partition) in turn, so short batches of long sequences spread over the
// workgroup too.  Units of equal size are placed in arbitrary order; results
// do not depend on the order units run in.
constexpr int kPlanThreads = 1024;

// The plan, by one workgroup of kPlanThreads threads.
__device__ __forceinline__ void decode_plan_body(
    const int32_t *__restrict__ context_lens, int32_t *__restrict__ plan, int num_seqs,
    int ctx_cap, int block_size, int part_pages, int max_parts) {
  __shared__ int s_count[kMaxPartitionPages + 1];  // units per size 0..part_pages
  __shared__ int s_next[kMaxPartitionPages + 1];   // next free slot per size
  __shared__ int s_total;
  // size of candidate unit u = (sequence u / max_parts, partition u % max_parts):
  // its page count, 0 for the single unit of an empty sequence, -1 if none
  auto unit_size = [&](int u) {
    const int s = u / max_parts;
    const int p = u - s * max_parts;
    const int ctx = min(max(context_lens[s], 0), ctx_cap);
    const int np = (ctx + block_size - 1) / block_size;
    if (np == 0) return p == 0 ? 0 : -1;
    return p * part_pages < np ? min(part_pages, np - p * part_pages) : -1;
  };
  const int candidates = num_seqs * max_parts;
  for (int i = threadIdx.x; i <= part_pages; i += kPlanThreads) s_count[i] = 0;
  __syncthreads();
  for (int u = threadIdx.x; u < candidates; u += kPlanThreads) {
    const int z = unit_size(u);
    if (z >= 0) atomicAdd(&s_count[z], 1);
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    // first list position of each size, sizes taken from part_pages down to
    // 0: lane l owns positions l*per .. l*per + per - 1 of that walk
    const int lane = threadIdx.x;
    const int per = (part_pages + 64) / 64;
    int mine = 0;
    for (int k = 0; k < per; ++k) {
      const int i = lane * per + k;
      if (i <= part_pages) mine += s_count[part_pages - i];
    }
    int incl = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    int at = incl - mine;
    for (int k = 0; k < per; ++k) {
      const int i = lane * per + k;
      if (i <= part_pages) {
        s_next[part_pages - i] = at;
        at += s_count[part_pages - i];
      }
    }
    if (lane == 63) {
      plan[0] = incl;
      s_total = incl;
    }
  }
  __syncthreads();
  for (int u = threadIdx.x; u < candidates; u += kPlanThreads) {
    const int z = unit_size(u);
    if (z >= 0) plan[kPlanHeader + atomicAdd(&s_next[z], 1)] = u;
  }
  for (int k = s_total + threadIdx.x; k < candidates; k += kPlanThreads)
    plan[kPlanHeader + k] = -1;
}

__global__ __launch_bounds__(kPlanThreads) void pa_decode_plan(
    const int32_t *__restrict__ context_lens, int32_t *__restrict__ plan, int num_seqs,
    int ctx_cap, int block_size, int part_pages, int max_parts) {
  decode_plan_body(context_lens, plan, num_seqs, ctx_cap, block_size, part_pages, max_parts);
}

// A decode step's first launch: workgroup 0 writes the plan while the others
// write the step's new tokens to the cache, kPlanThreads / kCacheThreads
// tokens each.  The plan reads only context lengths, so the two are
// independent; the partition kernel, launched after, sees both.
constexpr int kPrepTokens = kPlanThreads / kCacheThreads;

__global__ __launch_bounds__(kPlanThreads) void pa_decode_step_prep(
    const int32_t *__restrict__ context_lens, int32_t *__restrict__ plan, int num_seqs,
    int ctx_cap, int block_size, int part_pages, int max_parts, const u32x4 *__restrict__ k,
    const u32x4 *__restrict__ v, u32x4 *__restrict__ k_pool, u32x4 *__restrict__ v_pool,
    const int64_t *__restrict__ slot_mapping, int num_tokens, int num_kv_heads, int row_chunks,
    int64_t num_slots) {
  if (blockIdx.x == 0) {
    decode_plan_body(context_lens, plan, num_seqs, ctx_cap, block_size, part_pages, max_parts);
    return;
  }
  const int t = (blockIdx.x - 1) * kPrepTokens + threadIdx.x / kCacheThreads;
  if (t < num_tokens)
    cache_write_token(t, threadIdx.x % kCacheThreads, k, v, k_pool, v_pool, slot_mapping,
                      num_kv_heads, row_chunks, block_size, num_slots);
}

// ------------------------------------------------- decode, log-sum-exp merge
// Grid (num_heads, num_seqs), kReduceWaves wavefronts.  Merges the
// partitions of sequences that span more than one:
//   M = max_p m_p,  w_p = 2^(m_p - M),  out = sum_p w_p acc_p / sum_p w_p l_p.
// Wave w folds partitions w, w + kReduceWaves, ... with eight partitions'
// loads in flight; lane l owns D/64 consecutive outputs; the waves' sums meet
// in LDS.
constexpr int kReduceWaves = 4;
constexpr int kReduceUnroll = 8;

// With nslots (shared-prefix decode) sequence s has nslots[s] partials,
// written by the prefix and suffix units, and every sequence is finished
// here, also with one partial or none (a zero row).
template <class T, int D>
__global__ __launch_bounds__(64 * kReduceWaves) void pa_decode_reduce(
    void *__restrict__ out, const float *__restrict__ ws_ml, const float *__restrict__ ws_acc,
    const int32_t *__restrict__ context_lens, const int32_t *__restrict__ nslots,
    int num_heads, int ctx_cap, int part_tokens, int max_parts) {
  constexpr int DPL = D / 64;  // output elements per lane
  __shared__ float s_o[kReduceWaves][D];
  __shared__ float s_l[kReduceWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  int nparts;
  if (nslots) {
    nparts = min(nslots[s], max_parts);
  } else {
    const int ctx = min(max(context_lens[s], 0), ctx_cap);
    nparts = (ctx + part_tokens - 1) / part_tokens;
    if (nparts <= 1) return;  // the partition pass wrote the output itself
  }
  // partial p of head h is row (s * max_parts + p) * num_heads + h
  const size_t row0 = (size_t)s * max_parts * num_heads + h;
  const size_t pstride = num_heads;  // rows between consecutive partials
  const float *ml = ws_ml + row0 * 2;
  const float *acc = ws_acc + row0 * D + lane * DPL;

  float M = -INFINITY;
  for (int p = lane; p < nparts; p += 64) M = fmaxf(M, ml[2 * p * pstride]);
  M = wave_max(M);

  float L = 0.f, o[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) o[j] = 0.f;
  if (M != -INFINITY) {
    for (int p0 = wave; p0 < nparts; p0 += kReduceWaves * kReduceUnroll) {
      float w[kReduceUnroll], lp[kReduceUnroll], a[kReduceUnroll][DPL];
#pragma unroll
      for (int u = 0; u < kReduceUnroll; ++u) {
        const int p = p0 + u * kReduceWaves;
        const bool in = p < nparts;
        w[u] = in ? ml[2 * p * pstride] : -INFINITY;
        lp[u] = in ? ml[2 * p * pstride + 1] : 0.f;
#pragma unroll
        for (int j = 0; j < DPL; ++j) a[u][j] = in ? acc[p * pstride * D + j] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kReduceUnroll; ++u) {
        const float sc = fast_exp2(w[u] - M);
        L = fmaf(lp[u], sc, L);
#pragma unroll
        for (int j = 0; j < DPL; ++j) o[j] = fmaf(a[u][j], sc, o[j]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < DPL; ++j) s_o[wave][lane * DPL + j] = o[j];
  if (lane == 0) s_l[wave] = L;
  __syncthreads();
  if (wave != 0) return;
  float Lt = 0.f;
#pragma unroll
  for (int w = 0; w < kReduceWaves; ++w) Lt += s_l[w];
  const float inv = Lt > 0.f ? 1.0f / Lt : 0.f;
  float r[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kReduceWaves; ++w) t += s_o[w][lane * DPL + j];
    r[j] = t * inv;
  }
  if constexpr (T::kBytes == 4) {
    float *dst = reinterpret_cast<float *>(out) + ((size_t)s * num_heads + h) * D + lane * DPL;
#pragma unroll
    for (int j = 0; j < DPL; ++j) dst[j] = r[j];
  } else {
    uint16_t *dst = reinterpret_cast<uint16_t *>(out) + ((size_t)s * num_heads + h) * D + lane * DPL;
#pragma unroll
    for (int j = 0; j < DPL; ++j) dst[j] = (uint16_t)BF16::round_bits(r[j]);
  }
}

// The same merge when every sequence has at most kFewParts partials (the
// host knows it from the table width and partition size): one wavefront
// per (sequence, query head), four heads per workgroup, each lane loading
// every partial's (max, sum) and its D/64 accumulator values at once; no
// LDS and no barrier.  Partials past nparts count as (-inf, 0, 0).
constexpr int kFewParts = 8;
constexpr int kFewHeadsPerBlock = 4;

template <class T, int D>
__global__ __launch_bounds__(64 * kFewHeadsPerBlock) void pa_decode_reduce_few(
    void *__restrict__ out, const float *__restrict__ ws_ml, const float *__restrict__ ws_acc,
    const int32_t *__restrict__ context_lens, const int32_t *__restrict__ nslots,
    int num_heads, int ctx_cap, int part_tokens, int max_parts) {
  constexpr int DPL = D / 64;  // output elements per lane
  const int lane = threadIdx.x & 63;
  const int h = blockIdx.x * kFewHeadsPerBlock + (threadIdx.x >> 6);
  const int s = blockIdx.y;
  if (h >= num_heads) return;
  int nparts;
  if (nslots) {
    nparts = min(nslots[s], max_parts);
  } else {
    const int ctx = min(max(context_lens[s], 0), ctx_cap);
    nparts = (ctx + part_tokens - 1) / part_tokens;
    if (nparts <= 1) return;  // the partition pass wrote the output itself
  }
  // partial p of head h is row (s * max_parts + p) * num_heads + h
  const size_t row0 = (size_t)s * max_parts * num_heads + h;
  const size_t pstride = num_heads;  // rows between consecutive partials
  const float *ml = ws_ml + row0 * 2;
  const float *acc = ws_acc + row0 * D + lane * DPL;
  float mp[kFewParts], lp[kFewParts], a[kFewParts][DPL];
#pragma unroll
  for (int p = 0; p < kFewParts; ++p) {
    const bool in = p < nparts;
    mp[p] = in ? ml[2 * p * pstride] : -INFINITY;
    lp[p] = in ? ml[2 * p * pstride + 1] : 0.f;
#pragma unroll
    for (int j = 0; j < DPL; ++j) a[p][j] = in ? acc[p * pstride * D + j] : 0.f;
  }
  float M = -INFINITY;
#pragma unroll
  for (int p = 0; p < kFewParts; ++p) M = fmaxf(M, mp[p]);
  float L = 0.f, o[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) o[j] = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int p = 0; p < kFewParts; ++p) {
      const float sc = fast_exp2(mp[p] - M);
      L = fmaf(lp[p], sc, L);
#pragma unroll
      for (int j = 0; j < DPL; ++j) o[j] = fmaf(a[p][j], sc, o[j]);
    }
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  const size_t o0 = ((size_t)s * num_heads + h) * D + lane * DPL;
  if constexpr (T::kBytes == 4) {
#pragma unroll
    for (int j = 0; j < DPL; ++j) reinterpret_cast<float *>(out)[o0 + j] = o[j] * inv;
  } else {
#pragma unroll
    for (int j = 0; j < DPL; ++j)
      reinterpret_cast<uint16_t *>(out)[o0 + j] = (uint16_t)BF16::round_bits(o[j] * inv);
  }
}

// The split-K merge of a decode call: the few-partials form when every
// sequence has at most kFewParts partials, else the four-wave form.
template <class T, int D>
int launch_reduce(const pa_internal::DecodeLaunch &a, const int32_t *nslots) {
  hipStream_t st = reinterpret_cast<hipStream_t>(a.stream);
  const int ctx_cap = a.max_blocks * a.block_size;
  const int part_tokens = a.part_pages * a.block_size;
  if (a.max_parts <= kFewParts) {
    const dim3 grid((a.num_heads + kFewHeadsPerBlock - 1) / kFewHeadsPerBlock, a.num_seqs);
    hipLaunchKernelGGL((pa_decode_reduce_few<T, D>), grid, dim3(64 * kFewHeadsPerBlock), 0, st,
                       a.out, a.ws_ml, a.ws_acc, a.context_lens, nslots, a.num_heads, ctx_cap,
                       part_tokens, a.max_parts);
  } else {
    hipLaunchKernelGGL((pa_decode_reduce<T, D>), dim3(a.num_heads, a.num_seqs),
                       dim3(64 * kReduceWaves), 0, st, a.out, a.ws_ml, a.ws_acc, a.context_lens,
                       nslots, a.num_heads, ctx_cap, part_tokens, a.max_parts);
  }
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

// Wavefronts per workgroup of the VALU partition kernel: 8 for bf16 with
// one query head per kv-head (measured on MI355X at the Llama-2-7B decode
// shape: 179.2 -> 178.0 us a step; 2 waves: 187.2 us), 4 for fp32 and for
// head groups, whose registers leave no room for two waves per SIMD without
// spilling.
template <class T, int G>
constexpr int valu_waves() {
  return T::kBytes == 2 && G == 1 ? 8 : 4;
}

template <class T, int D, int BS, int G, bool AL>
int launch_valu_al(const pa_internal::DecodeLaunch &a, float scale_log2) {
  hipStream_t st = reinterpret_cast<hipStream_t>(a.stream);
  constexpr int NW = valu_waves<T, G>();
  auto kernel = pa_decode_partition<T, D, BS, G, NW, AL>;
  static const int per_cu = pa_internal::blocks_per_cu(reinterpret_cast<const void *>(kernel),
                                                       64 * NW);
  const unsigned grid = pa_internal::decode_grid(a, per_cu);
  if (grid == 0) return 6;
  pa_internal::launch_timed(kernel, dim3(grid), dim3(64 * NW), st, a.ev_begin, a.ev_end, a.out,
                            a.q, a.k_pool, a.v_pool, a.block_tables, a.context_lens, a.ws_ml,
                            a.ws_acc,
                     a.plan, a.num_seqs, a.num_heads, a.num_kv_heads, a.max_blocks,
                     a.num_blocks, a.part_pages, a.max_parts, scale_log2, a.alibi);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

template <class T, int D, int BS, int G>
int launch_valu(const pa_internal::DecodeLaunch &a, float scale_log2) {
  return a.alibi ? launch_valu_al<T, D, BS, G, true>(a, scale_log2)
                 : launch_valu_al<T, D, BS, G, false>(a, scale_log2);
}

template <class T, int D, int BS>
int partition_pass(const pa_internal::DecodeLaunch &a, float scale_log2) {
  const int g = a.num_heads / a.num_kv_heads;
  if constexpr (T::kBytes == 2) {
    // bf16: one query head per kv-head here; head groups on the matrix cores
    if (g >= 2) return pa_internal::launch_partition_gqa(a, scale_log2);
    return launch_valu<T, D, BS, 1>(a, scale_log2);
  } else {
    switch (g) {
      case 1: return launch_valu<T, D, BS, 1>(a, scale_log2);
      case 2: return launch_valu<T, D, BS, 2>(a, scale_log2);
      case 4: return launch_valu<T, D, BS, 4>(a, scale_log2);
      case 8: return launch_valu<T, D, BS, 8>(a, scale_log2);
    }
    return 3;
  }
}

// The plan launch of a decode call, or with a cache write (c not null), the
// step's preparation kernel that does both.
int launch_plan_or_prep(const pa_internal::DecodeLaunch &a, const pa_internal::CacheLaunch *c) {
  if (!c) return pa_internal::launch_decode_plan(a);
  const int row_chunks = a.head_dim * c->elem_bytes / 16;
  const unsigned grid = 1 + (unsigned)((c->num_tokens + kPrepTokens - 1) / kPrepTokens);
  hipLaunchKernelGGL(pa_decode_step_prep, dim3(grid), dim3(kPlanThreads), 0,
                     reinterpret_cast<hipStream_t>(a.stream), a.context_lens, a.plan, a.num_seqs,
                     a.max_blocks * a.block_size, a.block_size, a.part_pages * a.chain,
                     (a.max_parts + a.chain - 1) / a.chain,
                     static_cast<const u32x4 *>(c->k), static_cast<const u32x4 *>(c->v),
                     static_cast<u32x4 *>(c->k_pool), static_cast<u32x4 *>(c->v_pool),
                     c->slot_mapping, c->num_tokens, c->num_kv_heads, row_chunks,
                     (int64_t)c->num_blocks * c->block_size);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

template <class T, int D>
int run_decode(const pa_internal::DecodeLaunch &a, const pa_internal::CacheLaunch *c) {
  const float scale_log2 = a.scale * kLog2e;
  if (launch_plan_or_prep(a, c) != 0) return 6;
  // the partition kernel's launch records the timing events, if any
  const int rc = a.block_size == 16 ? partition_pass<T, D, 16>(a, scale_log2)
                                    : partition_pass<T, D, 32>(a, scale_log2);
  if (rc != 0) return rc;
  if (a.max_parts > 1) return launch_reduce<T, D>(a, nullptr);
  return 0;
}

template <class T>
int dispatch_dim(const pa_internal::DecodeLaunch &a, const pa_internal::CacheLaunch *c) {
  return a.head_dim == 64 ? run_decode<T, 64>(a, c) : run_decode<T, 128>(a, c);
}

}  // namespace

namespace pa_internal {

int blocks_per_cu(const void *kernel, int block_threads) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, block_threads, 0) != hipSuccess)
    return 1;
  return n > 0 ? n : 1;
}

unsigned decode_grid(const DecodeLaunch &a, int per_cu) {
  return persistent_grid_items((long long)a.num_seqs * a.max_parts * a.num_kv_heads,
                               per_cu * kDecodeGridRounds);
}

unsigned persistent_grid_items(long long items, int per_cu) {
  // compute units of the current device, queried once per device
  static std::atomic<int> cus_of[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  int cus = dev < kMaxDevices ? cus_of[dev].load(std::memory_order_relaxed) : 0;
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      return 0;
    if (dev < kMaxDevices) cus_of[dev].store(cus, std::memory_order_relaxed);
  }
  const long long resident = (long long)cus * per_cu;
  return (unsigned)(resident < items ? resident : items);
}

namespace {

int shared_prefix(const PrefixLaunch &p, const CacheLaunch *cache) {
  const DecodeLaunch &a = p.base;
  int rc = launch_prefix_prep(p, cache);
  if (rc != 0) return rc;
  // the unit kernel's launch records the timing events, if any
  rc = launch_prefix_units(p, a.scale * kLog2e);
  if (rc != 0) return rc;
  return a.head_dim == 64 ? launch_reduce<BF16, 64>(a, p.nslots)
                          : launch_reduce<BF16, 128>(a, p.nslots);
}

}  // namespace

int launch_decode_shared_prefix(const PrefixLaunch &p) { return shared_prefix(p, nullptr); }

int launch_shared_prefix_step(const PrefixLaunch &p, const CacheLaunch &cache) {
  return shared_prefix(p, &cache);
}

int launch_decode_plan(const DecodeLaunch &a) {
  // units of a.chain partitions (one, except in the grouped-query kernel's
  // one-wave form)
  hipLaunchKernelGGL(pa_decode_plan, dim3(1), dim3(kPlanThreads), 0,
                     reinterpret_cast<hipStream_t>(a.stream), a.context_lens, a.plan, a.num_seqs,
                     a.max_blocks * a.block_size, a.block_size, a.part_pages * a.chain,
                     (a.max_parts + a.chain - 1) / a.chain);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

int launch_decode(const DecodeLaunch &call) {
  DecodeLaunch a = call;
  a.chain = decode_chain(call);
  return a.dtype == 0 ? dispatch_dim<F32>(a, nullptr) : dispatch_dim<BF16>(a, nullptr);
}

int launch_decode_step(const DecodeLaunch &call, const CacheLaunch &cache) {
  DecodeLaunch a = call;
  a.chain = decode_chain(call);
  return a.dtype == 0 ? dispatch_dim<F32>(a, &cache) : dispatch_dim<BF16>(a, &cache);
}

}  // namespace pa_internal
