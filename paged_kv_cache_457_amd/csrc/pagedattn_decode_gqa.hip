// Paged decode attention, partition pass for grouped-query attention in bf16
// on the matrix cores (gfx950 MFMA).
//
// When G query heads share one kv-head (grouped-query attention; not on the
// vLLM / PagedAttention pages, which describe the paged cache itself: page
// table, fixed-size pages, attention reading pages through the table with no
// copy -- showapi.com article, section 2.1; tutorial page, section 4.2), one
// read of a K or V page serves G heads, so each page step is a small dense
// contraction: S = K q^T over head_dim, then O = V^T P^T over the page's
// tokens.  Both run on v_mfma instructions with the head group padded to 16
// columns; the pass stays bound by HBM, and the matrix cores take the
// multiply-adds off the vector ALUs.
//
// Work decomposition, scheduling and the merge of the NW waves' partial
// states are those of the VALU partition kernel (pagedattn_decode.hip):
// one workgroup of NW wavefronts per (sequence, kv-head, partition), pages
// dealt to the waves in turn, a persistent grid walking the plan kernel's
// largest-first unit list with the kv-head fastest.
//
// Lane layouts (lane l = 16*q4 + j16; 16x16 MFMA tiles):
// Tokens go through in granules of 16 (a 32-token page is two granules).
//   q.K   v_mfma_f32_16x16x32_bf16, one per 32-wide slab c of head_dim.
//         A = K rows: lane l holds K[token j16][32*c + 8*q4 .. +7] of the
//         granule, one 16-byte global load.  B = q^T: lane l holds
//         q[head j16][32*c + 8*q4 .. +7] (zero for j16 >= G).  Result: lane l
//         holds S[token 4*q4 + r][head j16], r = 0..3.
//   P.V   v_mfma_f32_16x16x16_bf16, one per 16-wide column block n of
//         head_dim, accumulating O^T[d][head].
//         B = P^T: lane l holds P[head j16][token 4*q4 + e] -- the q.K result
//         registers after exp, so P never moves between lanes.
//         A = V^T: lane l holds V[4*q4 + e][16*n + j16], e = 0..3, which is
//         one ds_read_b64_tr_b16 from the granule staged row-major in
//         LDS (within each 16-lane group, lane j of the read supplies 4
//         consecutive 16-bit values M[j][0..3] and lane i receives
//         M[4e + i/4][i%4], e = 0..3).  Result: lane l holds
//         O^T[16*n + 4*q4 + r][head j16], so the running max, sum and the
//         rescale of O are all per lane (per head).
// P enters the matrix cores as a bf16 pair hi + lo (hi = bf16(p), lo =
// bf16(p - hi)), two MFMAs per tile, so the weights carry about 16
// significant bits; the running sum uses the fp32 weights.
// Masked tokens (at or past the context length, or on an invalid page) get
// weight 0 and their V rows are written to LDS as zeros, so a poisoned slot
// (NaN) never reaches a multiply.
#include "pagedattn_device.h"
#include "pagedattn_internal.h"
#include "pagedattn_probe_launch.h"
#include "pagedattn_timed_launch.h"

namespace {

using namespace pa_dev;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) char lds_char;

template <int D, int BS, int G>
struct GqaShape {
  static_assert(G >= 2 && G <= 16, "head group padded to 16 MFMA columns");
  // The wave works in granules of 16 tokens (one MFMA tile of tokens): a
  // 32-token page is two granules with the same page id, so the prefetch
  // depth and the registers it needs do not depend on the page size.
  static constexpr int GPP = BS / 16;              // granules per page
  static constexpr int NC = D / 32;                // 32-wide head_dim slabs (q.K)
  static constexpr int NN = D / 16;                // 16-wide head_dim blocks (P.V)
  static constexpr int ROW = D * 2;                // bytes per token row
  static constexpr int GBYTES = 16 * ROW;          // bytes of one granule of K or V
  static constexpr int NVLD = GBYTES / 1024;       // 1 KiB V loads per granule
  // LDS row pitch of the staged V granule: 32 bytes of padding put the 8
  // rows a transposing read touches per half-wave in distinct banks
  static constexpr int PITCH = ROW + 32;
  static constexpr int VBYTES = 16 * PITCH;
  static constexpr int ACC_BYTES = G * D * 4;
  // per-wave LDS: the staged V granule, later reused for the wave's partial O
  static constexpr int WAVE_LDS = VBYTES > ACC_BYTES ? VBYTES : ACC_BYTES;
};

template <int D, int BS, int G>
struct GqaGranule {
  using S = GqaShape<D, BS, G>;
  bf16x8 k[S::NC];
  u32x4 v[S::NVLD];
  bool ok;
};

// In the one-wave-per-item form (below) one wave streams a run of
// consecutive partitions of its sequence and kv-head, up to kChainPages
// pages (one page id per lane) and kChainMax partitions, so the loads of
// the next partition are in flight while the last granules of one are
// used, and per-item startup is paid once per run.  The partials of all
// but the run's last partition wait in LDS until the run is streamed.
constexpr int kChainPages = 64;
constexpr int kChainMax = 4;

// WPI: wavefronts per item.  WPI == NW: the workgroup's NW waves deal the
// unit's pages among them and merge their states in LDS; the item is
// partition `item` of the sequence.  WPI == 1: each wave takes a whole item
// of its own, partitions chain * item .. chain * item + chain - 1 (at most
// 64 pages, one id per lane), streams their pages as one run with the
// granule prefetch crossing the partition edges, keeps each partition's
// result as it passes the partition's last page and writes them all at the
// end of the run, with no workgroup barrier.  Each partition's state
// starts afresh at its first page, so the results are those of one item
// per partition.
template <int D, int BS, int G, int NW, int WPI, bool AL>
__device__ __forceinline__ void decode_unit_gqa(
    void *__restrict__ out, const void *__restrict__ q, const void *__restrict__ k_pool,
    const void *__restrict__ v_pool, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ context_lens, float *__restrict__ ws_ml,
    float *__restrict__ ws_acc, int num_heads, int num_kv_heads, int max_blocks,
    int num_blocks, int part_pages, int max_parts, int chain, float scale_log2,
    const float *__restrict__ alibi, int s, int g, int item) {
  using S = GqaShape<D, BS, G>;
  constexpr int GPP = S::GPP, NC = S::NC, NN = S::NN, ROW = S::ROW, NVLD = S::NVLD;
  constexpr int PITCH = S::PITCH;
  __shared__ __attribute__((aligned(16))) char s_wave[NW][S::WAVE_LDS];
  __shared__ float s_ml[NW][G][2];
  // WPI == 1: partials of the run's earlier partitions, and (slot kPend)
  // the last partition's (max, sum)
  constexpr int kPend = WPI == 1 ? kChainMax - 1 : 0;
  __shared__ __attribute__((aligned(16))) float s_pend[WPI == 1 ? NW : 1][kPend > 0 ? kPend : 1][G * D];
  __shared__ float s_pend_ml[WPI == 1 ? NW : 1][kPend + 1][G][2];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // LDS region
  const int iw = WPI == 1 ? 0 : wave;  // this wave's place among the item's waves
  const int q4 = lane >> 4;
  const int j16 = lane & 15;
  const int h0 = g * G;
  const int item_pages = WPI == 1 ? chain * part_pages : part_pages;
  const int p_begin = item * item_pages;

  // Independent loads first: context length, this wave's page ids (one per
  // lane; columns past the context are loaded but never used) and q as the
  // B operand of the q.K tiles.
  int ctx = context_lens[s];
  const int col = p_begin + iw + WPI * lane;
  int my_bid = -1;
  if (iw + WPI * lane < item_pages && col < max_blocks)
    my_bid = block_tables[(size_t)s * max_blocks + col];
  bf16x8 qb[NC];
  {
    const char *qrow = reinterpret_cast<const char *>(q) + ((size_t)s * num_heads + h0 + j16) * ROW;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (j16 < G) w = load16(qrow + 64 * c + 16 * q4);
      qb[c] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // ALiBi: head j16's slope in log2 units (the padding heads past G add 0)
  const float slope = AL && j16 < G ? alibi[h0 + j16] * kLog2e : 0.f;

  ctx = min(max(ctx, 0), max_blocks * BS);
  const int npages = (ctx + BS - 1) / BS;
  char *out_b = reinterpret_cast<char *>(out);
  if (ctx == 0) {
    // the G output rows (contiguous) become zeros, 16 bytes per lane and step
    if (item == 0 && iw == 0) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      for (int off = lane * 16; off < G * ROW; off += 64 * 16)
        *reinterpret_cast<u32x4 *>(out_b + ((size_t)s * num_heads + h0) * ROW + off) = z;
    }
    return;
  }
  if (p_begin >= npages) return;
  const int np = min(npages - p_begin, item_pages);
  const int np_w = iw < np ? (np - iw + WPI - 1) / WPI : 0;

  // running state for head j16 (lanes j16 >= G carry a padding column)
  float m = -INFINITY;  // max of the logits so far, log2 units, same in all 4 lane groups
  float l = 0.f;        // this lane's share of the sum of weights
  f32x4 o[NN];          // O^T[16n + 4*q4 + r][head j16]
#pragma unroll
  for (int n = 0; n < NN; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const size_t page_stride = (size_t)num_kv_heads * BS * ROW;
  const char *k_b = reinterpret_cast<const char *>(k_pool) + (size_t)g * BS * ROW;
  const char *v_b = reinterpret_cast<const char *>(v_pool) + (size_t)g * BS * ROW;
  char *vs = s_wave[wave];

  // granule jg of this wave: page jg / GPP of the wave's pages, tokens
  // 16 * (jg % GPP) .. +15 of it
  auto fetch = [&](GqaGranule<D, BS, G> &gr, int jg) {
    const int bid = __builtin_amdgcn_readlane(my_bid, jg / GPP);
    gr.ok = (unsigned)bid < (unsigned)num_blocks;
    // an invalid id reads page 0, whose values are never used
    const size_t off = (size_t)(gr.ok ? bid : 0) * page_stride + (jg % GPP) * S::GBYTES;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      gr.k[c] = __builtin_bit_cast(bf16x8, load_kv16(k_b + off + j16 * ROW + 64 * c + 16 * q4));
#pragma unroll
    for (int i = 0; i < NVLD; ++i) gr.v[i] = load_kv16(v_b + off + i * 1024 + 16 * lane);
  };

  auto process = [&](const GqaGranule<D, BS, G> &gr, int jg) {
    const int tok0 = (p_begin + iw + WPI * (jg / GPP)) * BS + 16 * (jg % GPP);
    // stage V row-major in LDS; masked rows as zeros
#pragma unroll
    for (int i = 0; i < NVLD; ++i) {
      const int byte = i * 1024 + 16 * lane;
      const int row = byte / ROW;
      u32x4 w = gr.v[i];
      if (!gr.ok || tok0 + row >= ctx) w = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4 *>(vs + row * PITCH + byte % ROW) = w;
    }
    // logits S[token][head] of the granule's 16 tokens
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(gr.k[c], qb[c], acc, 0, 0, 0);
    float sc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool keep = gr.ok && tok0 + 4 * q4 + r < ctx;
      float x = acc[r] * scale_log2;
      if constexpr (AL) x = fmaf(slope, (float)(tok0 + 4 * q4 + r - (ctx - 1)), x);
      sc[r] = keep ? x : -INFINITY;
    }
    // online softmax for head j16: granule max over the 4 lane groups
    float pm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    pm = fmaxf(pm, __shfl_xor(pm, 16));
    pm = fmaxf(pm, __shfl_xor(pm, 32));
    const float mn = fmaxf(m, pm);
    if (mn == -INFINITY) return;  // nothing live yet (only with invalid page ids)
    const float alpha = fast_exp2(m - mn);
    m = mn;
    l *= alpha;
#pragma unroll
    for (int n = 0; n < NN; ++n) o[n] *= alpha;
    i16x4 phi, plo;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = fast_exp2(sc[r] - mn);
      l += p;
      const __bf16 hi = (__bf16)p;
      const __bf16 lo = (__bf16)(p - (float)hi);
      phi[r] = __builtin_bit_cast(short, hi);
      plo[r] = __builtin_bit_cast(short, lo);
    }
    // V^T operand rows: token 4*q4 + j16/4, columns 16n + 4*(j16%4)
    const int base = (4 * q4 + (j16 >> 2)) * PITCH + 8 * (j16 & 3);
#pragma unroll
    for (int n = 0; n < NN; ++n) {
      const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4 *)((lds_char *)vs + base + 32 * n));
      o[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, phi, o[n], 0, 0, 0);
      o[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, plo, o[n], 0, 0, 0);
    }
  };

  // WPI == 1: one wave holds a partition's whole state; lane (q4, j16) has
  // O^T[16n + 4*q4 + r][head j16] (O already summed over tokens by the
  // MFMAs) and its share of the sum of weights, first summed over the 4
  // lane groups.  The partials of the run's partitions before its last one
  // wait in LDS and all of the run's partials are written when the wave has
  // streamed the run: on MI355X writes issued while the pass streams its
  // reads cost about 1.3 us per MB written (8 x 32768 tokens at 512-token
  // partitions: 169 -> 159 us with the writes deferred), and few writes
  // come at the end of a run.
  auto hold_partials = [&](int k) {  // k-th partition of the run
    float lt = l + __shfl_xor(l, 16);
    lt += __shfl_xor(lt, 32);
    if (j16 < G) {
#pragma unroll
      for (int n = 0; n < NN; ++n)
        *reinterpret_cast<float4 *>(&s_pend[wave][k][j16 * D + 16 * n + 4 * q4]) =
            make_float4(o[n][0], o[n][1], o[n][2], o[n][3]);
      if (q4 == 0) {
        s_pend_ml[wave][k][j16][0] = m;
        s_pend_ml[wave][k][j16][1] = lt;
      }
    }
  };
  // [G][D] floats of LDS to the G heads' partial rows of partition `part`
  // (adjacent in the workspace), 16 bytes per lane and store, so that each
  // store instruction writes up to 1 KiB of whole rows
  auto write_rows = [&](const float *src, const float *src_ml, int part) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const size_t row0 = ((size_t)s * max_parts + part) * num_heads + h0;
    float *rows = ws_acc + row0 * D;
    constexpr int kChunks = G * D / 4;  // 16-byte chunks of the [G][D] block
#pragma unroll
    for (int i = 0; i < (kChunks + 63) / 64; ++i) {
      const int c = 64 * i + lane;
      if (kChunks % 64 == 0 || c < kChunks)
        *reinterpret_cast<float4 *>(rows + 4 * c) = *reinterpret_cast<const float4 *>(&src[4 * c]);
    }
    if (lane < 2 * G) ws_ml[row0 * 2 + lane] = src_ml[lane];
  };
  // The wave's final state: out rows when the sequence is one partition,
  // else the run's partials, the last partition's through the wave's
  // staging area ([head][d]; the V granule staged there has been read).
  const int part_first = p_begin / part_pages;
  auto store_wave = [&](int part) {
    if (npages > part_pages) {
      for (int k = 0; k < part - part_first; ++k)
        write_rows(s_pend[wave][k], &s_pend_ml[wave][k][0][0], part_first + k);
      float lt = l + __shfl_xor(l, 16);
      lt += __shfl_xor(lt, 32);
      float *st = reinterpret_cast<float *>(vs);
      if (j16 < G) {
#pragma unroll
        for (int n = 0; n < NN; ++n)
          *reinterpret_cast<float4 *>(&st[j16 * D + 16 * n + 4 * q4]) =
              make_float4(o[n][0], o[n][1], o[n][2], o[n][3]);
        if (q4 == 0) {
          s_pend_ml[wave][kPend][j16][0] = m;
          s_pend_ml[wave][kPend][j16][1] = lt;
        }
      }
      write_rows(st, &s_pend_ml[wave][kPend][0][0], part);
      return;
    }
    float lt = l + __shfl_xor(l, 16);
    lt += __shfl_xor(lt, 32);
    if (j16 < G) {
      const size_t row = (size_t)s * num_heads + h0 + j16;
      const float inv = lt > 0.f ? 1.0f / lt : 0.f;
#pragma unroll
      for (int n = 0; n < NN; ++n) {
        float v[4] = {o[n][0] * inv, o[n][1] * inv, o[n][2] * inv, o[n][3] * inv};
        BF16::store4(out_b + row * ROW + (16 * n + 4 * q4) * 2, v);
      }
    }
  };
  // granule index of the next partition's first granule, and the partition
  // the granules before it belong to.  Past the edge the state restarts
  // empty.
  const int pg = part_pages * GPP;
  int edge = pg;
  int part = part_first;
  auto at_edge = [&](int jg) {
    if constexpr (WPI == 1) {
      if (jg == edge) {
        hold_partials(part - part_first);
        ++part;
        edge += pg;
        m = -INFINITY;
        l = 0.f;
#pragma unroll
        for (int n = 0; n < NN; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };

  // One granule ahead; inside the loop every fetch is unconditional, so the
  // number of loads in flight is the same on every path and the wait before
  // a granule's use leaves the next one's loads outstanding.  A partition
  // edge before granule j is handled before the loads of granule j + 1 are
  // issued.
  const int ng = np_w * GPP;
  if (ng > 0) {
    GqaGranule<D, BS, G> ga, gb;
    fetch(ga, 0);
    int j = 0;
    for (; j + 2 < ng; j += 2) {
      at_edge(j);
      fetch(gb, j + 1);
      process(ga, j);
      at_edge(j + 1);
      fetch(ga, j + 2);
      process(gb, j + 1);
    }
    if (j + 1 < ng) {
      at_edge(j);
      fetch(gb, j + 1);
      process(ga, j);
      at_edge(j + 1);
      process(gb, j + 1);
    } else {
      at_edge(j);
      process(ga, j);
    }
  }

  if constexpr (WPI == 1) {
    store_wave(part);
    return;
  }
  // this wave's totals: the sum of weights over the 4 lane groups; O is
  // already summed over tokens by the MFMAs
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  // the V staging area becomes this wave's partial O (its own region)
  float *s_acc = reinterpret_cast<float *>(vs);
  if (j16 < G) {
#pragma unroll
    for (int n = 0; n < NN; ++n)
      *reinterpret_cast<float4 *>(&s_acc[j16 * D + 16 * n + 4 * q4]) =
          make_float4(o[n][0], o[n][1], o[n][2], o[n][3]);
    if (q4 == 0) {
      s_ml[wave][j16][0] = m;
      s_ml[wave][j16][1] = l;
    }
  }
  __syncthreads();
  merge_waves<BF16, D, G, NW>(
      [&](int w, int h, int d) -> float4 {
        return *reinterpret_cast<const float4 *>(
            reinterpret_cast<const float *>(s_wave[w]) + h * D + d);
      },
      [&](int w, int h) { return s_ml[w][h][0]; }, [&](int w, int h) { return s_ml[w][h][1]; },
      npages <= part_pages, out_b + ((size_t)s * num_heads + h0) * ROW,
      ws_acc + (((size_t)s * max_parts + part) * num_heads + h0) * D,
      ws_ml + (((size_t)s * max_parts + part) * num_heads + h0) * 2);
}

// Partition kernel over the plan's unit list (largest units first), item
// i = (list[i / num_kv_heads], kv-head i % num_kv_heads), in the snake order
// of snake_item.  WPI == NW: one item per workgroup step, on a grid of
// decode_grid; a unit is (sequence, partition).  WPI == 1: wave w of the
// workgroup's k-th step takes item NW * snake_item(k) + w, so the NW waves
// run consecutive items (the kv-heads of one unit) independently; a unit is
// (sequence, run of `chain` partitions).
// Two waves per SIMD: at most 256 registers (VGPRs and AGPRs) per lane.
template <int D, int BS, int G, int NW, int WPI, bool AL>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2))) void
pa_decode_partition_gqa(
    void *__restrict__ out, const void *__restrict__ q, const void *__restrict__ k_pool,
    const void *__restrict__ v_pool, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ context_lens, float *__restrict__ ws_ml,
    float *__restrict__ ws_acc, const int32_t *__restrict__ plan, int num_seqs, int num_heads,
    int num_kv_heads, int max_blocks, int num_blocks, int part_pages, int max_parts, int chain,
    float scale_log2, const float *__restrict__ alibi) {
  if constexpr (WPI == 1) {
    // the list holds num_seqs * max_units entries, -1 past the last unit
    const int max_units = (max_parts + chain - 1) / chain;
    const long long bound = (long long)num_seqs * max_units * num_kv_heads;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    for (int k = 0;; ++k) {
      const long long it = (long long)snake_item(k) * NW + wave;
      if (it >= bound) break;
      const int unit = plan[pa_internal::kPlanHeader + it / num_kv_heads];
      if (unit < 0) break;
      decode_unit_gqa<D, BS, G, NW, 1, AL>(out, q, k_pool, v_pool, block_tables, context_lens,
                                           ws_ml, ws_acc, num_heads, num_kv_heads, max_blocks,
                                           num_blocks, part_pages, max_parts, chain, scale_log2,
                                           alibi, unit / max_units, (int)(it % num_kv_heads),
                                           unit % max_units);
    }
  } else {
    // the list holds num_seqs * max_parts entries, -1 past the last unit
    const long long bound = (long long)num_seqs * max_parts * num_kv_heads;
    static_assert(WPI == NW, "an item takes one wave or the whole workgroup");
    for (int k = 0;; ++k) {
      const int it = snake_item(k);
      if (it >= bound) break;
      const int unit = plan[pa_internal::kPlanHeader + it / num_kv_heads];
      if (unit < 0) break;
      decode_unit_gqa<D, BS, G, NW, NW, AL>(out, q, k_pool, v_pool, block_tables, context_lens,
                                            ws_ml, ws_acc, num_heads, num_kv_heads, max_blocks,
                                            num_blocks, part_pages, max_parts, 1, scale_log2,
                                            alibi, unit / max_parts, it % num_kv_heads,
                                            unit % max_parts);
      __syncthreads();  // the next unit reuses the LDS the merge just read
    }
  }
}

constexpr int kWavesPerUnit = 4;

// One item per wave when a partition is at most kWaveItemPages pages and
// the table holds at least kWaveItemMinParts partitions: long sequences cut
// into many partitions, where each wave then streams a whole partition and
// no workgroup merge or barrier separates the items.  Measured on MI355X:
// 8 x 32768 tokens at 512-token partitions 187.7 -> 180.4 us a step, at
// 2048 171.3 -> 166.8 us.  Ragged batches whose tables hold few partitions
// keep the four-wave items, whose finer steps the dispatcher balances
// better (256 lognormal lengths at 1024-token partitions: 165.7 us against
// 180.2 us one item per wave; 128 shared-prefix samples at 512: 83.3 us
// against 95.5).
constexpr int kWaveItemPages = 64;
constexpr int kWaveItemMinParts = 16;

template <int D, int BS, int G, int WPI, bool AL>
int launch_al(const pa_internal::DecodeLaunch &a, float scale_log2) {
  hipStream_t st = reinterpret_cast<hipStream_t>(a.stream);
  auto kernel = pa_decode_partition_gqa<D, BS, G, kWavesPerUnit, WPI, AL>;
  static const int per_cu = pa_internal::blocks_per_cu(reinterpret_cast<const void *>(kernel),
                                                       64 * kWavesPerUnit);
  const long long items =
      (long long)a.num_seqs * ((a.max_parts + a.chain - 1) / a.chain) * a.num_kv_heads;
  const unsigned grid =
      WPI == 1 ? pa_internal::persistent_grid_items((items + kWavesPerUnit - 1) / kWavesPerUnit,
                                                    per_cu * pa_internal::kDecodeGridRounds)
               : pa_internal::decode_grid(a, per_cu);
  if (grid == 0) return 6;
  pa_internal::launch_timed(kernel, dim3(grid), dim3(64 * kWavesPerUnit), st, a.ev_begin,
                            a.ev_end, a.out, a.q, a.k_pool, a.v_pool, a.block_tables,
                            a.context_lens, a.ws_ml, a.ws_acc, a.plan,
                     a.num_seqs, a.num_heads, a.num_kv_heads, a.max_blocks, a.num_blocks,
                     a.part_pages, a.max_parts, WPI == 1 ? a.chain : 1, scale_log2, a.alibi);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

template <int D, int BS, int G, bool AL>
int launch_wpi(const pa_internal::DecodeLaunch &a, float scale_log2) {
  return pa_internal::gqa_wave_items(a)
             ? launch_al<D, BS, G, 1, AL>(a, scale_log2)
             : launch_al<D, BS, G, kWavesPerUnit, AL>(a, scale_log2);
}

template <int D, int BS, int G>
int launch(const pa_internal::DecodeLaunch &a, float scale_log2) {
  return a.alibi ? launch_wpi<D, BS, G, true>(a, scale_log2)
                 : launch_wpi<D, BS, G, false>(a, scale_log2);
}

template <int D, int BS>
int by_group(const pa_internal::DecodeLaunch &a, float scale_log2) {
  switch (a.num_heads / a.num_kv_heads) {
    case 2: return launch<D, BS, 2>(a, scale_log2);
    case 4: return launch<D, BS, 4>(a, scale_log2);
    case 8: return launch<D, BS, 8>(a, scale_log2);
  }
  return 3;
}

template <int D>
int by_block(const pa_internal::DecodeLaunch &a, float scale_log2) {
  return a.block_size == 16 ? by_group<D, 16>(a, scale_log2) : by_group<D, 32>(a, scale_log2);
}

}  // namespace

namespace pa_internal {

bool gqa_wave_items(const DecodeLaunch &a) {
  return a.part_pages <= kWaveItemPages && a.max_parts >= kWaveItemMinParts;
}

int decode_chain(const DecodeLaunch &a) {
  if (a.dtype != 1 || a.num_heads < 2 * a.num_kv_heads || !gqa_wave_items(a)) return 1;
  const int c = kChainPages / a.part_pages;
  return c < 1 ? 1 : c > kChainMax ? kChainMax : c;
}

int launch_partition_gqa(const DecodeLaunch &a, float scale_log2) {
  return a.head_dim == 64 ? by_block<64>(a, scale_log2) : by_block<128>(a, scale_log2);
}

}  // namespace pa_internal
