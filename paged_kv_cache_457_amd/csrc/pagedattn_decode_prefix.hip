// Paged decode attention with shared prefixes (bf16, matrix cores).
//
// Parallel sampling keeps one prompt's KV cache on pages that all samples of
// the prompt share (tutorial page, section 4.2: several outputs of one
// request share the same prefix pages; showapi.com article, section 2.2).
// Plain decode reads such a page once per sample.  Here the samples of a
// group read each shared page once: the G query heads of every member form
// one grouped contraction over the shared pages (up to 32 query rows, two
// 16-row MFMA tiles), and each member's own pages past the prefix are a
// separate unit.  Every unit leaves partial (max, sum, accumulator) rows in
// the workspace and the reduce kernel merges a sequence's prefix and suffix
// partials by log-sum-exp, so the result is the same softmax as plain decode.
//
// Units (plan kernel, largest first):
//   prefix unit: members seq0 .. seq0 + nmem - 1 of one group (nmem * G <=
//                32 rows), pages [pb, pe) of the shared prefix, read through
//                seq0's table row (the members' rows agree there)
//   suffix unit: one sequence (nmem = 1), pages [pb, pe) past the prefix
// Each unit writes partial slot `slot` of its rows; a sequence's slots are
// its group's prefix partitions first, then its own suffix partitions.
//
// Lane layouts are those of the grouped-query kernel (pagedattn_decode_gqa
// .hip), with the head-group columns widened to member x head rows:
// tile t, lane 16*q4 + j holds query row 16*t + j = member (16t+j) / G, head
// g*G + (16t+j) % G.  Each query row masks the tokens at or past its own
// sequence's context.  V rows at or past the longest member's context are
// staged as zeros, so a poisoned slot (NaN) never reaches a multiply; a
// row's other masked tokens only multiply finite, live values by 0.
#include "pagedattn_cache_row.h"
#include "pagedattn_device.h"
#include "pagedattn_internal.h"
#include "pagedattn_step_launch.h"
#include "pagedattn_timed_launch.h"

namespace {

using namespace pa_dev;
using pa_internal::kMaxPartitionPages;
using pa_internal::kPlanHeader;
using pa_internal::kPrefixRows;
using pa_internal::kPrefixUnitInts;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kTiles = kPrefixRows / 16;

// ------------------------------------------------------------------ plan
// One workgroup.  Layout of the plan area:
//   plan[0]                          unit count
//   plan[1]                          prefix units (they come first)
//   plan[kPlanHeader + 5k .. +4]     unit k: seq0, nmem, pb, pe, slot
//   nslots[s]                        partial slots sequence s fills
//   seq_pre[s]                       shared prefix pages of s's group
//                                    (working array of the plan kernel)
// kLds: every sequence's context length and prefix pages, and every
// group's bounds, are kept in LDS (at most kPlanLds of each): the kernel
// reads its inputs in one round of global loads at its start and writes
// the plan at its end, with no global round trip between its phases.
// Otherwise (larger batches) seq_pre is the working array in global memory.
constexpr int kPlanThreads = 1024;
constexpr int kPlanLds = 2048;

template <bool kLds>
__device__ __forceinline__ void prefix_plan_body(
    const int32_t *__restrict__ context_lens, const int32_t *__restrict__ group_starts,
    const int32_t *__restrict__ prefix_lens, int num_groups, int num_seqs, int group_size,
    int ctx_cap, int block_size, int part_pages, int32_t *__restrict__ plan,
    int32_t *__restrict__ nslots, int32_t *__restrict__ seq_pre) {
  // size classes (pages per unit) of prefix units [0] and own units [1]
  __shared__ int s_count[2][kMaxPartitionPages + 1];
  __shared__ int s_next[2][kMaxPartitionPages + 1];
  constexpr int kL = kLds ? kPlanLds : 1;
  __shared__ int s_ctx[kL], s_pre[kL], s_gb[kL], s_ge[kL], s_gpre[kL];
  const int members_per_chunk = kPrefixRows / group_size;
  const int max_pages = ctx_cap / block_size;
  // group gi: its sequences [b, e) and its prefix pages
  auto load_group = [&](int gi, int &b, int &e, int &pre) {
    b = min(max(group_starts[gi], 0), num_seqs);
    e = min(max(group_starts[gi + 1], b), num_seqs);
    pre = min(max(prefix_lens[gi], 0), ctx_cap) / block_size;
  };
  auto group = [&](int gi, int &b, int &e, int &pre) {
    if constexpr (kLds) {
      b = s_gb[gi];
      e = s_ge[gi];
      pre = s_gpre[gi];
    } else {
      load_group(gi, b, e, pre);
    }
  };
  auto ctx_of = [&](int s) {
    if constexpr (kLds) return s_ctx[s];
    else return min(max(context_lens[s], 0), ctx_cap);
  };
  auto pre_of = [&](int s) {
    if constexpr (kLds) return s_pre[s];
    else return (int)seq_pre[s];
  };
  auto set_pre = [&](int s, int v) {
    if constexpr (kLds) s_pre[s] = v;
    else seq_pre[s] = v;
  };
  for (int i = threadIdx.x; i <= part_pages; i += kPlanThreads) s_count[0][i] = s_count[1][i] = 0;
  if constexpr (kLds) {
    for (int gi = threadIdx.x; gi < num_groups; gi += kPlanThreads)
      load_group(gi, s_gb[gi], s_ge[gi], s_gpre[gi]);
    for (int s = threadIdx.x; s < num_seqs; s += kPlanThreads)
      s_ctx[s] = min(max(context_lens[s], 0), ctx_cap);
  }
  for (int s = threadIdx.x; s < num_seqs; s += kPlanThreads) set_pre(s, 0);
  __syncthreads();
  for (int gi = threadIdx.x; gi < num_groups; gi += kPlanThreads) {
    int b, e, pre;
    group(gi, b, e, pre);
    for (int s = b; s < e; ++s) set_pre(s, pre);
  }
  __syncthreads();
  // pages of sequence s past its prefix
  auto own_pages = [&](int s) {
    return max(0, min((ctx_of(s) + block_size - 1) / block_size, max_pages) - pre_of(s));
  };
  // pass 1: count units per size; slots per sequence
  for (int gi = threadIdx.x; gi < num_groups; gi += kPlanThreads) {
    int b, e, pre;
    group(gi, b, e, pre);
    if (e == b) continue;
    pre = pre_of(b);
    const int chunks = (e - b + members_per_chunk - 1) / members_per_chunk;
    for (int p0 = 0; p0 < pre; p0 += part_pages)
      atomicAdd(&s_count[0][min(part_pages, pre - p0)], chunks);
  }
  for (int s = threadIdx.x; s < num_seqs; s += kPlanThreads) {
    const int own = own_pages(s);
    for (int p0 = 0; p0 < own; p0 += part_pages)
      atomicAdd(&s_count[1][min(part_pages, own - p0)], 1);
    nslots[s] = (pre_of(s) + part_pages - 1) / part_pages + (own + part_pages - 1) / part_pages;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int at = 0;
    for (int kind = 0; kind < 2; ++kind) {
      for (int z = part_pages; z >= 1; --z) {
        s_next[kind][z] = at;
        at += s_count[kind][z];
      }
      if (kind == 0) plan[1] = at;
    }
    plan[0] = at;
  }
  __syncthreads();
  // pass 2: write the records, prefix units first, each kind largest first
  auto put = [&](int kind, int seq0, int nmem, int pb, int pe, int slot) {
    int32_t *r = plan + kPlanHeader + kPrefixUnitInts * atomicAdd(&s_next[kind][pe - pb], 1);
    r[0] = seq0;
    r[1] = nmem;
    r[2] = pb;
    r[3] = pe;
    r[4] = slot;
  };
  for (int gi = threadIdx.x; gi < num_groups; gi += kPlanThreads) {
    int b, e, pre;
    group(gi, b, e, pre);
    if (e == b) continue;
    pre = pre_of(b);
    for (int s0 = b; s0 < e; s0 += members_per_chunk)
      for (int p0 = 0, k = 0; p0 < pre; p0 += part_pages, ++k)
        put(0, s0, min(members_per_chunk, e - s0), p0, min(pre, p0 + part_pages), k);
  }
  for (int s = threadIdx.x; s < num_seqs; s += kPlanThreads) {
    const int pre = pre_of(s);
    const int own = own_pages(s);
    const int slot0 = (pre + part_pages - 1) / part_pages;
    for (int p0 = 0, k = 0; p0 < own; p0 += part_pages, ++k)
      put(1, s, 1, pre + p0, pre + min(own, p0 + part_pages), slot0 + k);
  }
}

template <bool kLds>
__global__ __launch_bounds__(kPlanThreads) void pa_prefix_plan(
    const int32_t *__restrict__ context_lens, const int32_t *__restrict__ group_starts,
    const int32_t *__restrict__ prefix_lens, int num_groups, int num_seqs, int group_size,
    int ctx_cap, int block_size, int part_pages, int32_t *__restrict__ plan,
    int32_t *__restrict__ nslots, int32_t *__restrict__ seq_pre) {
  prefix_plan_body<kLds>(context_lens, group_starts, prefix_lens, num_groups, num_seqs,
                         group_size, ctx_cap, block_size, part_pages, plan, nslots, seq_pre);
}

// A shared-prefix decode step's first launch: workgroup 0 writes the plan
// while the others write the step's new tokens to the cache,
// kPlanThreads / kCacheThreads tokens each.  The plan reads only context
// lengths and the groups, so the two are independent; the unit kernel,
// launched after, sees both.
constexpr int kPrepTokens = kPlanThreads / kCacheThreads;

template <bool kLds>
__global__ __launch_bounds__(kPlanThreads) void pa_prefix_step_prep(
    const int32_t *__restrict__ context_lens, const int32_t *__restrict__ group_starts,
    const int32_t *__restrict__ prefix_lens, int num_groups, int num_seqs, int group_size,
    int ctx_cap, int block_size, int part_pages, int32_t *__restrict__ plan,
    int32_t *__restrict__ nslots, int32_t *__restrict__ seq_pre, const u32x4 *__restrict__ k,
    const u32x4 *__restrict__ v, u32x4 *__restrict__ k_pool, u32x4 *__restrict__ v_pool,
    const int64_t *__restrict__ slot_mapping, int num_kv_heads, int row_chunks,
    int64_t num_slots) {
  if (blockIdx.x == 0) {
    prefix_plan_body<kLds>(context_lens, group_starts, prefix_lens, num_groups, num_seqs,
                           group_size, ctx_cap, block_size, part_pages, plan, nslots, seq_pre);
    return;
  }
  const int t = (blockIdx.x - 1) * kPrepTokens + threadIdx.x / kCacheThreads;
  if (t < num_seqs)
    cache_write_token(t, threadIdx.x % kCacheThreads, k, v, k_pool, v_pool, slot_mapping,
                      num_kv_heads, row_chunks, block_size, num_slots);
}

// ------------------------------------------------------------ unit kernel
template <int D, int BS>
struct PrefixShape {
  static constexpr int GPP = BS / 16;          // 16-token granules per page
  static constexpr int NC = D / 32;            // 32-wide head_dim slabs (q.K)
  static constexpr int NN = D / 16;            // 16-wide head_dim blocks (P.V)
  static constexpr int ROW = D * 2;            // bytes per token row
  static constexpr int GBYTES = 16 * ROW;      // bytes of one granule of K or V
  static constexpr int NVLD = GBYTES / 1024;   // 1 KiB V loads per granule
  static constexpr int PITCH = ROW + 32;       // LDS row pitch of a staged V granule
  static constexpr int VBYTES = 16 * PITCH;    // per-wave LDS: staging, then partial O
  // the merge stores a wave's 16 x D partial O in head_dim slices that fit
  // its staging area
  static constexpr int PASSES = (16 * (D + 8) * 4 + VBYTES - 1) / VBYTES;
  static constexpr int DH = D / PASSES;        // head_dim columns per merge pass
  // row pitch of a stored slice: 8 floats of padding spread the 16 rows a
  // store instruction writes over all LDS banks
  static constexpr int DHP = DH + 8;
  static_assert(DH % 16 == 0 && 16 * DHP * 4 <= VBYTES, "merge slice");
};

template <int D>
struct PrefixGranule {
  bf16x8 k[D / 32];
  u32x4 v[16 * D * 2 / 1024];
  bool ok;
};

// One unit.  Wave roles: with two row tiles, waves [0, NW/2) carry tile 0
// and the others tile 1; with one tile all NW waves carry it.  The waves of
// a tile deal the unit's pages among themselves in turn, so every wave
// holds the state of one 16-row tile and a granule of K/V is loaded once
// per tile (the second load of a page by the other tile's waves, at about
// the same time in the same workgroup, is served by the caches).
// solo: each wave carries a unit of its own (a sequence's pages past its
// prefix: one tile), streams all of that unit's pages and writes its
// partial rows directly; the workgroup's waves then share no state beyond
// their barriers.  A wave with no unit passes nmem = 0 and pb = pe.
template <int D, int BS, int G, int NW>
__device__ __forceinline__ void prefix_unit(
    const void *__restrict__ q, const void *__restrict__ k_pool, const void *__restrict__ v_pool,
    const int32_t *__restrict__ block_tables, const int32_t *__restrict__ context_lens,
    float *__restrict__ ws_ml, float *__restrict__ ws_acc, int num_heads, int num_kv_heads,
    int max_blocks, int num_blocks, int max_slots, float scale_log2, int seq0, int nmem, int pb,
    int pe, int slot, int g, bool solo) {
  using S = PrefixShape<D, BS>;
  constexpr int GPP = S::GPP, NC = S::NC, NN = S::NN, ROW = S::ROW, NVLD = S::NVLD;
  constexpr int PITCH = S::PITCH, DH = S::DH, DHP = S::DHP;
  __shared__ __attribute__((aligned(16))) char s_wave[NW][S::VBYTES];
  __shared__ float s_ml[NW][16][2];
  // the unit's query rows as MFMA B operands: [tile (solo: wave)][slab][lane]
  // 16 bytes
  __shared__ __attribute__((aligned(16))) u32x4 s_q[NW][NC][64];
  static_assert(kTiles <= NW, "a query slot per tile");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q4 = lane >> 4;
  const int j16 = lane & 15;
  const int rows = nmem * G;                       // query rows of this unit (<= 32)
  const int ntiles = solo ? 1 : (rows + 15) / 16;  // 1 or 2, same for the whole workgroup
  const int wpt = solo ? 1 : ntiles == 2 ? NW / 2 : NW;  // waves per tile
  const int tile = solo ? 0 : wave / wpt;           // this wave's tile
  const int wslot = solo ? 0 : wave % wpt;          // its place among the tile's waves
  const int qslot = solo ? wave : tile;             // its query rows in s_q
  const int ctx_cap = max_blocks * BS;

  // q of both tiles to LDS (wave 0; solo: each wave its own), each row's
  // context length, the longest
  int ctx_max = 0, my_ctx = 0;
#pragma unroll
  for (int t = 0; t < kTiles; ++t) {
    if (solo && t > 0) break;
    const int r = 16 * t + j16;
    const bool live = r < rows;
    const int s = seq0 + (live ? r / G : 0);
    if (solo || wave == 0) {
      const char *qrow =
          reinterpret_cast<const char *>(q) + ((size_t)s * num_heads + g * G + r % G) * ROW;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (live) w = load16(qrow + 64 * c + 16 * q4);
        s_q[solo ? wave : t][c][lane] = w;
      }
    }
    const int c = live ? min(max(context_lens[s], 0), ctx_cap) : 0;
    ctx_max = max(ctx_max, c);
    if (t == tile) my_ctx = c;
  }
#pragma unroll
  for (int o2 = 32; o2 >= 1; o2 >>= 1) ctx_max = max(ctx_max, __shfl_xor(ctx_max, o2));

  // this wave's page ids: unit pages wslot, wslot + wpt, ..., one per lane
  // in two registers (its pages 0-63, then 64-127): with two tiles, wpt is
  // NW / 2 = 2 and a partition of up to kMaxPartitionPages = 256 pages gives
  // a wave up to 128 pages
  static_assert(kMaxPartitionPages <= 2 * 64 * (NW / 2), "two page ids per lane suffice");
  const int np = pe - pb;
  int my_bid = -1, my_bid_hi = -1;
  if (wslot + wpt * lane < np)
    my_bid = block_tables[(size_t)seq0 * max_blocks + pb + wslot + wpt * lane];
  if (wslot + wpt * (64 + lane) < np)
    my_bid_hi = block_tables[(size_t)seq0 * max_blocks + pb + wslot + wpt * (64 + lane)];
  const int np_w = wslot < np ? (np - wslot + wpt - 1) / wpt : 0;
  __syncthreads();  // s_q is written by wave 0 and read by all

  float m = -INFINITY, l = 0.f;
  f32x4 o[NN];
#pragma unroll
  for (int n = 0; n < NN; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const size_t page_stride = (size_t)num_kv_heads * BS * ROW;
  const char *k_b = reinterpret_cast<const char *>(k_pool) + (size_t)g * BS * ROW;
  const char *v_b = reinterpret_cast<const char *>(v_pool) + (size_t)g * BS * ROW;
  char *vs = s_wave[wave];
  const u32x4 *qt = &s_q[qslot][0][lane];

  auto fetch = [&](PrefixGranule<D> &gr, int jg) {
    const int jp = jg / GPP;  // this wave's page, uniform
    const int bid = __builtin_amdgcn_readlane(jp < 64 ? my_bid : my_bid_hi, jp & 63);
    gr.ok = (unsigned)bid < (unsigned)num_blocks;
    const size_t off = (size_t)(gr.ok ? bid : 0) * page_stride + (jg % GPP) * S::GBYTES;
    if (ntiles == 2) {
      // both row tiles' waves read each page: cached loads, so the second
      // read of a line finds it in the caches
#pragma unroll
      for (int c = 0; c < NC; ++c)
        gr.k[c] = __builtin_bit_cast(bf16x8, load16(k_b + off + j16 * ROW + 64 * c + 16 * q4));
#pragma unroll
      for (int i = 0; i < NVLD; ++i) gr.v[i] = load16(v_b + off + i * 1024 + 16 * lane);
    } else {
#pragma unroll
      for (int c = 0; c < NC; ++c)
        gr.k[c] = __builtin_bit_cast(bf16x8, load_kv16(k_b + off + j16 * ROW + 64 * c + 16 * q4));
#pragma unroll
      for (int i = 0; i < NVLD; ++i) gr.v[i] = load_kv16(v_b + off + i * 1024 + 16 * lane);
    }
  };

  auto process = [&](const PrefixGranule<D> &gr, int jg) {
    const int tok0 = (pb + wslot + wpt * (jg / GPP)) * BS + 16 * (jg % GPP);
#pragma unroll
    for (int i = 0; i < NVLD; ++i) {
      const int byte = i * 1024 + 16 * lane;
      const int row = byte / ROW;
      u32x4 w = gr.v[i];
      if (!gr.ok || tok0 + row >= ctx_max) w = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4 *>(vs + row * PITCH + byte % ROW) = w;
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(gr.k[c], __builtin_bit_cast(bf16x8, qt[64 * c]),
                                                    acc, 0, 0, 0);
    float sc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool keep = gr.ok && tok0 + 4 * q4 + r < my_ctx;
      sc[r] = keep ? acc[r] * scale_log2 : -INFINITY;
    }
    float pm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    pm = fmaxf(pm, __shfl_xor(pm, 16));
    pm = fmaxf(pm, __shfl_xor(pm, 32));
    // rows differ in context length, so a row may have nothing live yet
    const float mn = fmaxf(m, pm);
    const bool none = mn == -INFINITY;
    const float alpha = none ? 1.f : fast_exp2(m - mn);
    const float base = none ? 0.f : mn;
    m = mn;
    l *= alpha;
#pragma unroll
    for (int n = 0; n < NN; ++n) o[n] *= alpha;
    i16x4 phi, plo;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = fast_exp2(sc[r] - base);
      l += p;
      const __bf16 hi = (__bf16)p;
      const __bf16 lo = (__bf16)(p - (float)hi);
      phi[r] = __builtin_bit_cast(short, hi);
      plo[r] = __builtin_bit_cast(short, lo);
    }
    const int vbase = (4 * q4 + (j16 >> 2)) * PITCH + 8 * (j16 & 3);
#pragma unroll
    for (int n = 0; n < NN; ++n) {
      const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4 *)((lds_char *)vs + vbase + 32 * n));
      o[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, phi, o[n], 0, 0, 0);
      o[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, plo, o[n], 0, 0, 0);
    }
  };

  const int ng = np_w * GPP;
  if (ng > 0) {
    PrefixGranule<D> ga, gb;
    fetch(ga, 0);
    int j = 0;
    for (; j + 2 < ng; j += 2) {
      fetch(gb, j + 1);
      process(ga, j);
      fetch(ga, j + 2);
      process(gb, j + 1);
    }
    if (j + 1 < ng) {
      fetch(gb, j + 1);
      process(ga, j);
      process(gb, j + 1);
    } else {
      process(ga, j);
    }
  }

  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (solo) {
    // the wave's own partial rows: lane (q4, j) holds d = 16n + 4*q4 .. +3
    // of row j
    if (j16 < rows) {
      const size_t wrow =
          ((size_t)(seq0 + j16 / G) * max_slots + slot) * num_heads + g * G + j16 % G;
#pragma unroll
      for (int n = 0; n < NN; ++n)
        *reinterpret_cast<float4 *>(ws_acc + wrow * D + 16 * n + 4 * q4) =
            make_float4(o[n][0], o[n][1], o[n][2], o[n][3]);
      if (q4 == 0) {
        ws_ml[wrow * 2] = m;
        ws_ml[wrow * 2 + 1] = l;
      }
    }
    return;
  }
  // Merge: each tile's waves by log-sum-exp, through LDS, in head_dim slices
  // of DH columns (a wave's slice of its partial O fits its staging area).
  if (q4 == 0) {
    s_ml[wave][j16][0] = m;
    s_ml[wave][j16][1] = l;
  }
  float *s_acc = reinterpret_cast<float *>(vs);
#pragma unroll
  for (int h = 0; h < S::PASSES; ++h) {
    __syncthreads();  // staging areas (or the previous slice) no longer in use
#pragma unroll
    for (int n = 0; n < DH / 16; ++n) {
      const int nn = h * (DH / 16) + n;
      *reinterpret_cast<float4 *>(&s_acc[j16 * DHP + 16 * n + 4 * q4]) =
          make_float4(o[nn][0], o[nn][1], o[nn][2], o[nn][3]);
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < ntiles * 16 * (DH / 4); idx += 64 * NW) {
      const int t = idx / (16 * (DH / 4));
      const int j = (idx / (DH / 4)) % 16;
      const int d = (idx % (DH / 4)) * 4;
      const int r = 16 * t + j;
      if (r >= rows) continue;
      const int w0 = t * wpt;
      float M = -INFINITY;
      for (int w = w0; w < w0 + wpt; ++w) M = fmaxf(M, s_ml[w][j][0]);
      float L = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
      if (M != -INFINITY) {
        for (int w = w0; w < w0 + wpt; ++w) {
          const float sc = fast_exp2(s_ml[w][j][0] - M);
          L = fmaf(s_ml[w][j][1], sc, L);
          const float4 a = *reinterpret_cast<const float4 *>(
              reinterpret_cast<const float *>(s_wave[w]) + j * DHP + d);
          acc[0] = fmaf(a.x, sc, acc[0]);
          acc[1] = fmaf(a.y, sc, acc[1]);
          acc[2] = fmaf(a.z, sc, acc[2]);
          acc[3] = fmaf(a.w, sc, acc[3]);
        }
      }
      const size_t wrow =
          ((size_t)(seq0 + r / G) * max_slots + slot) * num_heads + g * G + r % G;
      *reinterpret_cast<float4 *>(ws_acc + wrow * D + h * DH + d) =
          make_float4(acc[0], acc[1], acc[2], acc[3]);
      if (h == 0 && d == 0) {
        ws_ml[wrow * 2] = M;
        ws_ml[wrow * 2 + 1] = L;
      }
    }
  }
}

// Kernel over the plan's units, snake order, on a grid of several rounds of
// resident workgroups.  Prefix units first, item i = (unit i / num_kv_heads,
// kv-head i % num_kv_heads), all NW waves on one unit; then the own units
// NW at a time, one per wave (solo), item = (NW consecutive units,
// kv-head).
template <int D, int BS, int G, int NW>
__global__ __launch_bounds__(64 * NW) void pa_decode_prefix_gqa(
    const void *__restrict__ q, const void *__restrict__ k_pool, const void *__restrict__ v_pool,
    const int32_t *__restrict__ block_tables, const int32_t *__restrict__ context_lens,
    float *__restrict__ ws_ml, float *__restrict__ ws_acc, const int32_t *__restrict__ plan,
    int num_heads, int num_kv_heads, int max_blocks, int num_blocks, int max_slots,
    float scale_log2, int solo_own) {
  const int units = plan[0];
  // own units run solo unless a unit can exceed the 128 page ids a single
  // wave holds (partitions of more than 128 pages)
  const int npre = solo_own ? plan[1] : units;
  const int pre_items = npre * num_kv_heads;
  const int items = pre_items + (units - npre + NW - 1) / NW * num_kv_heads;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int k = 0;; ++k) {
    const int it = snake_item(k);
    if (it >= items) break;
    const bool solo = it >= pre_items;
    const int i = solo ? it - pre_items : it;
    const int unit = solo ? npre + NW * (i / num_kv_heads) + wave : i / num_kv_heads;
    const bool has = unit < units;  // the last group of own units may be short
    // (index clamped: the record of a missing unit is not read past the list)
    const int32_t *u = plan + kPlanHeader + (size_t)kPrefixUnitInts * min(unit, units - 1);
    prefix_unit<D, BS, G, NW>(q, k_pool, v_pool, block_tables, context_lens, ws_ml, ws_acc,
                              num_heads, num_kv_heads, max_blocks, num_blocks, max_slots,
                              scale_log2, has ? u[0] : 0, has ? u[1] : 0, has ? u[2] : 0,
                              has ? u[3] : 0, has ? u[4] : 0, i % num_kv_heads, solo);
    __syncthreads();  // the next unit reuses the LDS
  }
}

constexpr int kWavesPerUnit = 4;

template <int D, int BS, int G>
int launch(const pa_internal::PrefixLaunch &p, float scale_log2) {
  const pa_internal::DecodeLaunch &a = p.base;
  hipStream_t st = reinterpret_cast<hipStream_t>(a.stream);
  auto kernel = pa_decode_prefix_gqa<D, BS, G, kWavesPerUnit>;
  static const int per_cu = pa_internal::blocks_per_cu(reinterpret_cast<const void *>(kernel),
                                                       64 * kWavesPerUnit);
  // several rounds of resident workgroups, as for the partition kernels
  const unsigned grid = pa_internal::persistent_grid_items(p.max_units * (long long)a.num_kv_heads,
                                                           per_cu * pa_internal::kDecodeGridRounds);
  if (grid == 0) return 6;
  pa_internal::launch_timed(kernel, dim3(grid), dim3(64 * kWavesPerUnit), st, a.ev_begin,
                            a.ev_end, a.q, a.k_pool, a.v_pool, a.block_tables, a.context_lens,
                            a.ws_ml, a.ws_acc, a.plan, a.num_heads, a.num_kv_heads,
                            a.max_blocks, a.num_blocks, a.max_parts, scale_log2,
                            a.part_pages <= 128 ? 1 : 0);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

template <int D, int BS>
int by_group(const pa_internal::PrefixLaunch &p, float scale_log2) {
  switch (p.base.num_heads / p.base.num_kv_heads) {
    case 1: return launch<D, BS, 1>(p, scale_log2);
    case 2: return launch<D, BS, 2>(p, scale_log2);
    case 4: return launch<D, BS, 4>(p, scale_log2);
    case 8: return launch<D, BS, 8>(p, scale_log2);
  }
  return 3;
}

}  // namespace

namespace pa_internal {

int launch_prefix_prep(const PrefixLaunch &p, const CacheLaunch *cache) {
  const DecodeLaunch &a = p.base;
  hipStream_t st = reinterpret_cast<hipStream_t>(a.stream);
  const bool lds = a.num_seqs <= kPlanLds && p.num_groups <= kPlanLds;
  if (cache) {
    auto kernel = lds ? pa_prefix_step_prep<true> : pa_prefix_step_prep<false>;
    const unsigned grid = 1 + (unsigned)((a.num_seqs + kPrepTokens - 1) / kPrepTokens);
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kPlanThreads), 0, st, a.context_lens,
                       p.group_starts, p.prefix_lens, p.num_groups, a.num_seqs,
                       a.num_heads / a.num_kv_heads, a.max_blocks * a.block_size, a.block_size,
                       a.part_pages, a.plan, p.nslots, p.seq_pre,
                       static_cast<const u32x4 *>(cache->k), static_cast<const u32x4 *>(cache->v),
                       static_cast<u32x4 *>(cache->k_pool), static_cast<u32x4 *>(cache->v_pool),
                       cache->slot_mapping, cache->num_kv_heads,
                       a.head_dim * cache->elem_bytes / 16,
                       (int64_t)cache->num_blocks * cache->block_size);
  } else {
    auto kernel = lds ? pa_prefix_plan<true> : pa_prefix_plan<false>;
    hipLaunchKernelGGL(kernel, dim3(1), dim3(kPlanThreads), 0, st, a.context_lens,
                       p.group_starts, p.prefix_lens, p.num_groups, a.num_seqs,
                       a.num_heads / a.num_kv_heads, a.max_blocks * a.block_size, a.block_size,
                       a.part_pages, a.plan, p.nslots, p.seq_pre);
  }
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

int launch_prefix_plan(const PrefixLaunch &p) { return launch_prefix_prep(p, nullptr); }

int launch_prefix_units(const PrefixLaunch &p, float scale_log2) {
  const DecodeLaunch &a = p.base;
  if (a.head_dim == 64)
    return a.block_size == 16 ? by_group<64, 16>(p, scale_log2) : by_group<64, 32>(p, scale_log2);
  return a.block_size == 16 ? by_group<128, 16>(p, scale_log2) : by_group<128, 32>(p, scale_log2);
}

}  // namespace pa_internal
