// HIP kernels for paged decode attention and the KV-cache write, gfx950.
//
// Method (vLLM / PagedAttention pages): the KV cache is a pool of fixed-size
// pages; a per-sequence page table maps logical to physical pages and the
// attention kernel reads the pages through that table directly, with no
// gather copy and no padding (showapi.com article, section 2.1; tutorial
// page, section 4.2).  Each decode step also appends the new token's K/V to
// the cache (tutorial page, section 4.3, step 3).
//
// Work decomposition: one 64-lane wavefront per (sequence, kv-head,
// partition of up to 64 pages).  A wavefront reads each (page, kv-head) run
// of block_size * head_dim elements as whole 16-byte chunks: lane l, load i
// takes chunk i*64 + l, so every load instruction covers 1 KiB of
// consecutive bytes.  With R = chunks per token row, a load instruction
// holds 64/R tokens and lane l always sees the same R-chunk column
// (l % R) of token rows (l / R) + i*64/R.  The partial q.K dot products of a
// row are summed across its R lanes with DPP row operations, so every lane
// of the row ends up holding the full logit.  Softmax is the online form
// (running max, rescaled running sum and accumulator) in log2 units, with
// log2(e) folded into the scale.  Sequences longer than one partition leave
// (max, sum, unnormalised V accumulation) per partition in the workspace,
// and a second kernel merges them by log-sum-exp.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedattn_internal.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// Reinterpret a 32-bit word as two bf16.  Takes the word by value: a
// bit-cast applied directly to an element of an ext_vector lvalue reads
// element 0 whatever the index (seen with this compiler), so always copy
// the element out first.
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

// ------------------------------------------------------------ element types
struct F32 {
  static constexpr int kBytes = 4;
  static constexpr int kPerChunk = 4;
  __device__ static void unpack(const u32x4 c, float *f) {
#pragma unroll
    for (int w = 0; w < 4; ++w) f[w] = __uint_as_float(c[w]);
  }
  __device__ static u32x4 pack(const float *f) {
    u32x4 c;
#pragma unroll
    for (int w = 0; w < 4; ++w) c[w] = __float_as_uint(f[w]);
    return c;
  }
  // q . k over one 16-byte chunk
  __device__ static float dot(const u32x4 qc, const u32x4 kc) {
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) acc = fmaf(__uint_as_float(qc[w]), __uint_as_float(kc[w]), acc);
    return acc;
  }
  // four consecutive outputs (16 bytes)
  __device__ static void store4(char *dst, const float *o) {
    *reinterpret_cast<float4 *>(dst) = make_float4(o[0], o[1], o[2], o[3]);
  }
};

struct BF16 {
  static constexpr int kBytes = 2;
  static constexpr int kPerChunk = 8;
  // a 32-bit word holds element 2w in its low half and 2w+1 in its high half
  __device__ static void unpack(const u32x4 c, float *f) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      f[2 * w] = __uint_as_float(c[w] << 16);
      f[2 * w + 1] = __uint_as_float(c[w] & 0xffff0000u);
    }
  }
  // fp32 -> bf16, round to nearest even; NaN stays a quiet NaN
  __device__ static uint32_t round_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  }
  __device__ static u32x4 pack(const float *f) {
    u32x4 c;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      c[w] = round_bits(f[2 * w]) | (round_bits(f[2 * w + 1]) << 16);
    return c;
  }
  // four consecutive outputs (8 bytes), rounded to nearest even
  __device__ static void store4(char *dst, const float *o) {
    *reinterpret_cast<uint2 *>(dst) = make_uint2(round_bits(o[0]) | (round_bits(o[1]) << 16),
                                                 round_bits(o[2]) | (round_bits(o[3]) << 16));
  }
  // q . k over one chunk with v_dot2_f32_bf16: products of bf16 pairs are
  // exact in fp32, accumulated in fp32
  __device__ static float dot(const u32x4 qc, const u32x4 kc) {
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qc[w]), as_bf16x2(kc[w]), acc, false);
    return acc;
  }
};

// ------------------------------------------------------- wavefront reductions
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the R consecutive lanes that share a token row (R = 8, 16, 32).
// quad_perm [1,0,3,2] and [2,3,0,1] sum each quad; row_half_mirror pairs
// the two quads of each 8-lane half; row_mirror pairs the two halves of the
// 16-lane row.  Every lane of the group gets the same bits (fp add commutes).
template <int R>
__device__ __forceinline__ float row_sum(float v) {
  static_assert(R == 8 || R == 16 || R == 32, "row width");
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  if constexpr (R >= 16) v += dpp<0x140>(v);
  if constexpr (R == 32) v += __shfl_xor(v, 16);
  return v;
}

// Reduce over the 64/R row groups (lanes with equal l % R).
template <int R>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (R <= 8) v += __shfl_xor(v, 8);
  if constexpr (R <= 16) v += __shfl_xor(v, 16);
  if constexpr (R <= 32) v += __shfl_xor(v, 32);
  return v;
}
template <int R>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (R <= 8) v = fmaxf(v, __shfl_xor(v, 8));
  if constexpr (R <= 16) v = fmaxf(v, __shfl_xor(v, 16));
  if constexpr (R <= 32) v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ u32x4 load16(const char *p) { return *reinterpret_cast<const u32x4 *>(p); }

// KV page chunks are read once per call: non-temporal loads keep them from
// displacing reusable lines in the caches (measured on MI355X at the
// Llama-2-7B decode shape: 200 us -> 182 us for the partition pass)
__device__ __forceinline__ u32x4 load_kv16(const char *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

// ------------------------------------------------------ decode, partition pass
// One workgroup of NW wavefronts per unit (sequence s, kv-head g, partition
// p of at most part_pages pages).  The unit's pages are dealt to its waves
// in turn: wave w takes partition pages w, w + NW, w + 2 NW, ...  Each wave
// keeps a running (max, sum, V accumulator) for the G query heads of g over
// its own pages, with PF pages of K and V in flight; the NW partial states
// are merged through LDS at the end, which is the same log-sum-exp merge the
// reduce kernel applies across partitions.
//
// Grid: 1-D, max_parts * num_seqs * num_kv_heads workgroups, ordered
// kv-head fastest, then sequence, then partition.  The hardware hands
// consecutive workgroups to the 8 XCDs in turn, so this order gives every
// XCD the same share of each sequence's heads whatever the spread of
// context lengths (partition-fastest order would send partition p of every
// sequence to one XCD).
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
  __device__ __forceinline__ void page(const u32x4 (&qc)[G], const u32x4 (&kc)[S::NLD],
                                       const u32x4 (&vc)[S::NLD], int tok0, int ctx, bool live,
                                       int rg, float scale_log2) {
    float lg[S::NLD][G];
#pragma unroll
    for (int i = 0; i < S::NLD; ++i)
#pragma unroll
      for (int h = 0; h < G; ++h) lg[i][h] = row_sum<S::R>(T::dot(qc[h], kc[i])) * scale_log2;
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

template <class T, int D, int BS, int G, int NW>
__global__ __launch_bounds__(64 * NW) void pa_decode_partition(
    void *__restrict__ out, const void *__restrict__ q, const void *__restrict__ k_pool,
    const void *__restrict__ v_pool, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ context_lens, float *__restrict__ ws_ml,
    float *__restrict__ ws_acc, int num_seqs, int num_heads, int num_kv_heads, int max_blocks,
    int num_blocks, int part_pages, int max_parts, float scale_log2) {
  using S = DecodeShape<T, D, BS, G>;
  constexpr int E = S::E, R = S::R, NLD = S::NLD, PAGE_BYTES = S::PAGE_BYTES;
  __shared__ float s_ml[NW][G][2];
  __shared__ __attribute__((aligned(16))) float s_acc[NW][G][D];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = blockIdx.x % num_kv_heads;
  const int sp = blockIdx.x / num_kv_heads;
  const int s = sp % num_seqs;
  const int part = sp / num_seqs;
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
        st.page(qc, ka, va, tok0(j), ctx, oka, rg, scale_log2);
        oka = fetch(ka, va, j + 2);
        st.page(qc, kb, vb, tok0(j + 1), ctx, okb, rg, scale_log2);
      }
      if (j + 1 < np_w) {
        okb = fetch(kb, vb, j + 1);
        st.page(qc, ka, va, tok0(j), ctx, oka, rg, scale_log2);
        st.page(qc, kb, vb, tok0(j + 1), ctx, okb, rg, scale_log2);
      } else {
        st.page(qc, ka, va, tok0(j), ctx, oka, rg, scale_log2);
      }
    }
  } else {
    for (int j = 0; j < np_w; ++j) {
      u32x4 kc[NLD], vc[NLD];
      const bool ok = fetch(kc, vc, j);
      st.page(qc, kc, vc, tok0(j), ctx, ok, rg, scale_log2);
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

  // merge the waves: thread t owns 4 consecutive outputs of one head
  const bool whole = npages <= part_pages;
  for (int idx = threadIdx.x; idx < G * D / 4; idx += 64 * NW) {
    const int h = idx / (D / 4);
    const int d = (idx % (D / 4)) * 4;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_ml[w][h][0]);
    float L = 0.f, o[4] = {0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float sc = fast_exp2(s_ml[w][h][0] - M);
        L = fmaf(s_ml[w][h][1], sc, L);
        const float4 a = *reinterpret_cast<const float4 *>(&s_acc[w][h][d]);
        o[0] = fmaf(a.x, sc, o[0]);
        o[1] = fmaf(a.y, sc, o[1]);
        o[2] = fmaf(a.z, sc, o[2]);
        o[3] = fmaf(a.w, sc, o[3]);
      }
    }
    if (whole) {
      const float inv = L > 0.f ? 1.0f / L : 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] *= inv;
      T::store4(out_b + ((size_t)s * num_heads + h0 + h) * head_row_bytes + d * T::kBytes, o);
    } else {
      const size_t row = ((size_t)s * num_heads + h0 + h) * max_parts + part;
      *reinterpret_cast<float4 *>(ws_acc + row * D + d) = make_float4(o[0], o[1], o[2], o[3]);
      if (d == 0) {
        ws_ml[row * 2] = M;
        ws_ml[row * 2 + 1] = L;
      }
    }
  }
}

// ------------------------------------------------- decode, log-sum-exp merge
// Grid (num_heads, num_seqs), 64 threads.  Merges the partitions of
// sequences that span more than one: M = max_p m_p, w_p = 2^(m_p - M),
// out = sum_p w_p acc_p / sum_p w_p l_p.
template <class T, int D>
__global__ __launch_bounds__(64) void pa_decode_reduce(
    void *__restrict__ out, const float *__restrict__ ws_ml, const float *__restrict__ ws_acc,
    const int32_t *__restrict__ context_lens, int num_heads, int ctx_cap, int part_tokens,
    int max_parts) {
  constexpr int DPL = D / 64;  // output elements per lane
  const int lane = threadIdx.x;
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  int ctx = context_lens[s];
  ctx = min(max(ctx, 0), ctx_cap);
  const int nparts = (ctx + part_tokens - 1) / part_tokens;
  if (nparts <= 1) return;
  const size_t row0 = ((size_t)s * num_heads + h) * max_parts;

  float M = -INFINITY;
  for (int p = lane; p < nparts; p += 64) M = fmaxf(M, ws_ml[(row0 + p) * 2]);
  M = wave_max(M);
  float L = 0.f;
  for (int p = lane; p < nparts; p += 64)
    L += ws_ml[(row0 + p) * 2 + 1] * fast_exp2(ws_ml[(row0 + p) * 2] - M);
  L = wave_sum(L);

  float o[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) o[j] = 0.f;
  for (int p = 0; p < nparts; ++p) {
    const float w = fast_exp2(ws_ml[(row0 + p) * 2] - M);
    const float *a = ws_acc + (row0 + p) * D + lane * DPL;
#pragma unroll
    for (int j = 0; j < DPL; ++j) o[j] = fmaf(w, a[j], o[j]);
  }
  const float inv = 1.0f / L;
  if constexpr (T::kBytes == 4) {
    float *dst = reinterpret_cast<float *>(out) + ((size_t)s * num_heads + h) * D + lane * DPL;
#pragma unroll
    for (int j = 0; j < DPL; ++j) dst[j] = o[j] * inv;
  } else {
    uint16_t *dst = reinterpret_cast<uint16_t *>(out) + ((size_t)s * num_heads + h) * D + lane * DPL;
#pragma unroll
    for (int j = 0; j < DPL; ++j) dst[j] = (uint16_t)BF16::round_bits(o[j] * inv);
  }
}

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

// ------------------------------------------------------------- dispatch
constexpr int kWavesPerUnit = 4;

template <class T, int D, int BS, int G>
int run_decode(const pa_internal::DecodeLaunch &a) {
  hipStream_t st = reinterpret_cast<hipStream_t>(a.stream);
  const float scale_log2 = a.scale * kLog2e;
  if (a.ev_begin) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(a.ev_begin), st);
  dim3 grid((unsigned)a.max_parts * a.num_kv_heads * a.num_seqs);
  hipLaunchKernelGGL((pa_decode_partition<T, D, BS, G, kWavesPerUnit>), grid,
                     dim3(64 * kWavesPerUnit), 0, st, a.out, a.q,
                     a.k_pool, a.v_pool, a.block_tables, a.context_lens, a.ws_ml, a.ws_acc,
                     a.num_seqs, a.num_heads, a.num_kv_heads, a.max_blocks, a.num_blocks, a.part_pages,
                     a.max_parts, scale_log2);
  if (hipGetLastError() != hipSuccess) return 6;
  if (a.ev_end) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(a.ev_end), st);
  if (a.max_parts > 1) {
    hipLaunchKernelGGL((pa_decode_reduce<T, D>), dim3(a.num_heads, a.num_seqs), dim3(64), 0, st,
                       a.out, a.ws_ml, a.ws_acc, a.context_lens, a.num_heads,
                       a.max_blocks * BS, a.part_pages * BS, a.max_parts);
    if (hipGetLastError() != hipSuccess) return 6;
  }
  return 0;
}

template <class T, int D, int BS>
int dispatch_group(const pa_internal::DecodeLaunch &a) {
  switch (a.num_heads / a.num_kv_heads) {
    case 1: return run_decode<T, D, BS, 1>(a);
    case 2: return run_decode<T, D, BS, 2>(a);
    case 4: return run_decode<T, D, BS, 4>(a);
    case 8: return run_decode<T, D, BS, 8>(a);
  }
  return 3;
}

template <class T, int D>
int dispatch_block(const pa_internal::DecodeLaunch &a) {
  return a.block_size == 16 ? dispatch_group<T, D, 16>(a) : dispatch_group<T, D, 32>(a);
}

template <class T>
int dispatch_dim(const pa_internal::DecodeLaunch &a) {
  return a.head_dim == 64 ? dispatch_block<T, 64>(a) : dispatch_block<T, 128>(a);
}

}  // namespace

namespace pa_internal {

int launch_decode(const DecodeLaunch &a) {
  return a.dtype == 0 ? dispatch_dim<F32>(a) : dispatch_dim<BF16>(a);
}

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
                     reinterpret_cast<const u32x4 *>(buf), n16, (n16 + kProbeBlocks - 1) / kProbeBlocks,
                     reinterpret_cast<uint32_t *>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

}  // namespace pa_internal
