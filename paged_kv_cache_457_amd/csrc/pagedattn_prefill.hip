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
// stages a tile's K and V rows in LDS (double buffered; the next tile's
// global loads are in flight in registers while the current tile is used).
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
// pool, are staged as zeros (so a poisoned slot never reaches a multiply) and
// masked to -inf in S; a tile that lies wholly below a wave's first position
// and on valid pages skips the per-key mask.
#include <type_traits>

#include "pagedattn_device.h"
#include "pagedattn_internal.h"

namespace {

using namespace pa_dev;
using pa_internal::kPlanHeader;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32 * kWaves;  // query rows of a work item
constexpr int kKeys = 64;           // keys per LDS tile
constexpr int kBuckets = 1024;      // plan size classes (key tiles); the last is open-ended
constexpr int kPlanThreads = 1024;

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
// unpadded; XOR-ing the chunk index with a function of the row spreads the
// 16 rows one q.K operand read touches, and the 8 rows each half of a
// transposing V read touches, over all banks.
template <int D>
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (D == 128)
    return c ^ (((r & 7) << 1) | ((r >> 3) & 1));
  else
    return c ^ ((((r >> 1) & 3) << 1) | ((r >> 3) & 1));
}

// ------------------------------------------------------------------ plan
// One workgroup.  plan[0] = item count; item k is plan[kPlanHeader + 2k]
// (sequence) and plan[kPlanHeader + 2k + 1] (first chunk token), items
// ordered by the key tiles they read, most first.  Every chunk token is in
// exactly one item, so there are at most num_tokens items.
__global__ __launch_bounds__(kPlanThreads) void pa_prefill_plan(
    const int32_t *__restrict__ context_lens, const int32_t *__restrict__ query_start,
    int num_seqs, int num_tokens, int ctx_cap, int tok, int32_t *__restrict__ plan) {
  __shared__ int s_count[kBuckets + 1];
  __shared__ int s_next[kBuckets + 1];
  for (int i = threadIdx.x; i <= kBuckets; i += kPlanThreads) s_count[i] = 0;
  __syncthreads();
  // chunk length, and the position of its first token
  auto chunk = [&](int s, int &n, int &p0) {
    const int a = min(max(query_start[s], 0), num_tokens);
    const int b = min(max(query_start[s + 1], a), num_tokens);
    n = b - a;
    p0 = min(max(context_lens[s], 0), ctx_cap) - n;
  };
  auto bucket = [&](int n, int p0, int t0) {
    const int kv_end = p0 + min(n, t0 + tok);  // keys the item's last token sees
    return kv_end <= 0 ? 0 : min((kv_end + kKeys - 1) / kKeys, kBuckets);
  };
  for (int s = threadIdx.x; s < num_seqs; s += kPlanThreads) {
    int n, p0;
    chunk(s, n, p0);
    for (int t0 = 0; t0 < n; t0 += tok) atomicAdd(&s_count[bucket(n, p0, t0)], 1);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int at = 0;
    for (int z = kBuckets; z >= 0; --z) {
      s_next[z] = at;
      at += s_count[z];
    }
    plan[0] = at;
  }
  __syncthreads();
  for (int s = threadIdx.x; s < num_seqs; s += kPlanThreads) {
    int n, p0;
    chunk(s, n, p0);
    for (int t0 = 0; t0 < n; t0 += tok) {
      int32_t *r = plan + kPlanHeader + 2 * atomicAdd(&s_next[bucket(n, p0, t0)], 1);
      r[0] = s;
      r[1] = t0;
    }
  }
}

// ------------------------------------------------------------- work item
template <int D, int BS, int G>
__device__ __forceinline__ void prefill_item(
    void *__restrict__ out, const void *__restrict__ q, const void *__restrict__ k_pool,
    const void *__restrict__ v_pool, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ context_lens, const int32_t *__restrict__ query_start,
    int num_tokens, int num_heads, int num_kv_heads, int max_blocks, int num_blocks,
    float scale_log2, int s, int t0, int g) {
  using Sh = PrefillShape<D, BS, G>;
  constexpr int ROW = Sh::ROW, CPR = Sh::CPR, NC = Sh::NC, NN = Sh::NN, TILE = Sh::TILE;
  constexpr int LOADS = Sh::LOADS, TOK = Sh::TOK, PPT = Sh::PPT;
  __shared__ __attribute__((aligned(16))) char s_kv[2][2][TILE];  // [buffer][K, V]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4 = lane >> 4;
  const int j16 = lane & 15;

  // the sequence's chunk (uniform)
  const int qa = min(max(query_start[s], 0), num_tokens);
  const int qb = min(max(query_start[s + 1], qa), num_tokens);
  const int n = qb - qa;
  const int p0 = min(max(context_lens[s], 0), max_blocks * BS) - n;  // position of chunk token 0
  const int ntok = min(TOK, n - t0);                                  // tokens of this item
  const int kv_end = max(0, p0 + t0 + ntok);                          // keys the item sees
  const int ntiles = (kv_end + kKeys - 1) / kKeys;
  const int npages = (kv_end + BS - 1) / BS;
  const int32_t *bt = block_tables + (size_t)s * max_blocks;

  // this wave's token range (rows 32*wave .. 32*wave + 31)
  const int first = 32 * wave / G;
  const int last = min(ntok - 1, (32 * wave + 31) / G);
  const bool wave_live = first < ntok;
  const int wmin = p0 + t0 + first;  // position of the wave's first token
  const int wmax = p0 + t0 + last;   // and of its last

  // query rows as MFMA B operands, and each row's position (-1: not a row)
  bf16x8 qf[2][NC];
  int pos[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int row = 32 * wave + 16 * t + j16;
    const int tk = row / G;
    const bool live = tk < ntok;
    pos[t] = live ? p0 + t0 + tk : -1;
    const char *qrow = reinterpret_cast<const char *>(q) +
                       ((size_t)(qa + t0 + (live ? tk : 0)) * num_heads + g * G + row % G) * ROW;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (live) w = load16(qrow + 64 * c + 16 * q4);
      qf[t][c] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // global -> registers -> LDS staging of key tiles
  const size_t page_stride = (size_t)num_kv_heads * BS * ROW;
  const char *kb = reinterpret_cast<const char *>(k_pool) + (size_t)g * BS * ROW;
  const char *vb = reinterpret_cast<const char *>(v_pool) + (size_t)g * BS * ROW;
  u32x4 rk[LOADS], rv[LOADS];
  unsigned okbits = 0;
  auto fetch = [&](int kt) {
    okbits = 0;
#pragma unroll
    for (int l = 0; l < LOADS; ++l) {
      const int ci = l * kThreads + tid;
      const int key = ci / CPR;
      const int kk = kt * kKeys + key;
      const int pj = kk / BS;
      const int bid = pj < npages ? bt[pj] : -1;
      const bool ok = kk < kv_end && (unsigned)bid < (unsigned)num_blocks;
      okbits |= (unsigned)ok << l;
      const size_t off = (size_t)(ok ? bid : 0) * page_stride + (kk % BS) * ROW + (ci % CPR) * 16;
      rk[l] = load16(kb + off);
      rv[l] = load16(vb + off);
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int l = 0; l < LOADS; ++l) {
      const int ci = l * kThreads + tid;
      const int key = ci / CPR;
      const bool ok = (okbits >> l) & 1u;
      const int at = key * ROW + swz<D>(key, ci % CPR) * 16;
      const u32x4 z = {0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4 *>(&s_kv[buf][0][at]) = ok ? rk[l] : z;
      *reinterpret_cast<u32x4 *>(&s_kv[buf][1][at]) = ok ? rv[l] : z;
    }
  };
  // pages of tile kt that are valid (uniform)
  auto tile_pages_ok = [&](int kt) {
    bool ok = true;
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int pj = kt * PPT + j;
      if (pj < npages) ok = ok && (unsigned)bt[pj] < (unsigned)num_blocks;
    }
    return ok;
  };

  float m[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f};
  f32x4 o[2][NN];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int nb = 0; nb < NN; ++nb) o[t][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](auto masked_c, int buf, int kt) {
    constexpr bool kMasked = decltype(masked_c)::value;
    const lds_char *ks = (const lds_char *)s_kv[buf][0];
    const lds_char *vs = (const lds_char *)s_kv[buf][1];
    // S^T for the tile's four 16-key sub-tiles and both row tiles
    f32x4 sacc[4][2];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      sacc[st][0] = f32x4{0.f, 0.f, 0.f, 0.f};
      sacc[st][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int r = 16 * st + j16;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const bf16x8 a = *(const __attribute__((address_space(3))) bf16x8 *)(
            ks + r * ROW + swz<D>(r, 4 * c + q4) * 16);
        sacc[st][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[0][c], sacc[st][0], 0, 0, 0);
        sacc[st][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[1][c], sacc[st][1], 0, 0, 0);
      }
    }
    // page validity of each sub-tile's keys (a sub-tile lies in one page)
    bool sub_ok[4] = {true, true, true, true};
    if constexpr (kMasked) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int pj = kt * PPT + (16 * st) / BS;
        sub_ok[st] = pj < npages && (unsigned)bt[pj] < (unsigned)num_blocks;
      }
    }
    // online softmax, then P as bf16 B operands
    i16x4 pb[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float sv[4][4];
      float mx = -INFINITY;
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float x = sacc[st][t][r] * scale_log2;
          if constexpr (kMasked) {
            const int kk = kt * kKeys + 16 * st + 4 * q4 + r;
            if (!(sub_ok[st] && kk <= pos[t])) x = -INFINITY;
          }
          sv[st][r] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mn = fmaxf(m[t], mx);
      const bool none = mn == -INFINITY;  // the row has seen no key yet
      const float alpha = none ? 1.f : fast_exp2(m[t] - mn);
      const float base = none ? 0.f : mn;
      m[t] = mn;
      lsum[t] *= alpha;
#pragma unroll
      for (int nb = 0; nb < NN; ++nb) o[t][nb] *= alpha;
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = fast_exp2(sv[st][r] - base);
          lsum[t] += p;
          pb[t][st][r] = __builtin_bit_cast(short, (__bf16)p);
        }
    }
    // O^T += V^T P^T over key pairs of sub-tiles (32 keys per instruction)
    const int vrow = 4 * q4 + (j16 >> 2);
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
      const i16x8 b0 = __builtin_shufflevector(pb[0][2 * kp], pb[0][2 * kp + 1], 0, 1, 2, 3, 4,
                                               5, 6, 7);
      const i16x8 b1 = __builtin_shufflevector(pb[1][2 * kp], pb[1][2 * kp + 1], 0, 1, 2, 3, 4,
                                               5, 6, 7);
#pragma unroll
      for (int nb = 0; nb < NN; ++nb) {
        const int chunk = 2 * nb + ((j16 >> 1) & 1);
        const int r0 = 32 * kp + vrow, r1 = r0 + 16;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4 *)(vs + r0 * ROW + swz<D>(r0, chunk) * 16 + (j16 & 1) * 8));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4 *)(vs + r1 * ROW + swz<D>(r1, chunk) * 16 + (j16 & 1) * 8));
        const bf16x8 a =
            __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[0][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, b0),
                                                           o[0][nb], 0, 0, 0);
        o[1][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, b1),
                                                           o[1][nb], 0, 0, 0);
      }
    }
  };

  if (ntiles > 0) {
    fetch(0);
    stage(0);
    if (ntiles > 1) fetch(1);
    __syncthreads();
    for (int kt = 0; kt < ntiles; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < ntiles) {
        stage(buf ^ 1);  // its previous contents were used before the last barrier
        if (kt + 2 < ntiles) fetch(kt + 2);
      }
      if (wave_live && kt * kKeys <= wmax) {
        if (kt * kKeys + kKeys - 1 <= wmin && tile_pages_ok(kt))
          compute(std::integral_constant<bool, false>{}, buf, kt);
        else
          compute(std::integral_constant<bool, true>{}, buf, kt);
      }
      __syncthreads();
    }
  }

  // normalise and store: lane (q4, j) writes d = 16n + 4*q4 .. +3 of row j
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int row = 32 * wave + 16 * t + j16;
    const int tk = row / G;
    if (tk >= ntok) continue;
    float L = lsum[t];
    L += __shfl_xor(L, 16);
    L += __shfl_xor(L, 32);
    const float inv = L > 0.f ? 1.f / L : 0.f;
    char *orow = reinterpret_cast<char *>(out) +
                 ((size_t)(qa + t0 + tk) * num_heads + g * G + row % G) * ROW;
#pragma unroll
    for (int nb = 0; nb < NN; ++nb) {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = o[t][nb][r] * inv;
      BF16::store4(orow + (16 * nb + 4 * q4) * 2, v);
    }
  }
}

template <int D, int BS, int G>
__global__ __launch_bounds__(kThreads) void pa_prefill_gqa(
    void *__restrict__ out, const void *__restrict__ q, const void *__restrict__ k_pool,
    const void *__restrict__ v_pool, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ context_lens, const int32_t *__restrict__ query_start,
    const int32_t *__restrict__ plan, int num_tokens, int num_heads, int num_kv_heads,
    int max_blocks, int num_blocks, float scale_log2) {
  const int items = plan[0] * num_kv_heads;
  for (int k = 0;; ++k) {
    const int it = snake_item(k);
    if (it >= items) break;
    const int32_t *u = plan + kPlanHeader + 2 * (it / num_kv_heads);
    prefill_item<D, BS, G>(out, q, k_pool, v_pool, block_tables, context_lens, query_start,
                           num_tokens, num_heads, num_kv_heads, max_blocks, num_blocks,
                           scale_log2, u[0], u[1], it % num_kv_heads);
    __syncthreads();  // the next item reuses the LDS
  }
}

template <int D, int BS, int G>
int launch(const pa_internal::PrefillLaunch &a) {
  hipStream_t st = reinterpret_cast<hipStream_t>(a.stream);
  auto kernel = pa_prefill_gqa<D, BS, G>;
  static const int per_cu =
      pa_internal::blocks_per_cu(reinterpret_cast<const void *>(kernel), kThreads);
  // items <= num_tokens (each holds at least one chunk token)
  const unsigned grid =
      pa_internal::persistent_grid_items((long long)a.num_tokens * a.num_kv_heads, per_cu);
  if (grid == 0) return 6;
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), 0, st, a.out, a.q, a.k_pool, a.v_pool,
                     a.block_tables, a.context_lens, a.query_start, a.plan, a.num_tokens,
                     a.num_heads, a.num_kv_heads, a.max_blocks, a.num_blocks,
                     a.scale * kLog2e);
  return hipGetLastError() == hipSuccess ? 0 : 6;
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

int prefill_tokens_per_item(int group) { return kRows / group; }

int launch_prefill(const PrefillLaunch &a) {
  hipStream_t st = reinterpret_cast<hipStream_t>(a.stream);
  hipLaunchKernelGGL(pa_prefill_plan, dim3(1), dim3(kPlanThreads), 0, st, a.context_lens,
                     a.query_start, a.num_seqs, a.num_tokens, a.max_blocks * a.block_size,
                     prefill_tokens_per_item(a.num_heads / a.num_kv_heads), a.plan);
  if (hipGetLastError() != hipSuccess) return 6;
  if (a.ev_begin) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(a.ev_begin), st);
  int rc;
  if (a.head_dim == 64)
    rc = a.block_size == 16 ? by_group<64, 16>(a) : by_group<64, 32>(a);
  else
    rc = a.block_size == 16 ? by_group<128, 16>(a) : by_group<128, 32>(a);
  if (rc != 0) return rc;
  if (a.ev_end) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(a.ev_end), st);
  return 0;
}

}  // namespace pa_internal
