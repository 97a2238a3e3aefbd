// KV-cache write, whole-page copies, and the read-bandwidth probes.
//
// Each decode step produces the next token together with the updated KV
// cache (tutorial page, section 4.3, step 3 of the iteration): the new
// token's K and V rows go to the page slot its sequence's page table gives.
// Whole pages move when a sequence needs its own copy of a page it shares
// with others before writing into it (tutorial page, section 4.2, shared
// pages) and when a preempted sequence's pages go to a CPU-side pool and
// come back (sections 4.4 and 4.5).
#include "pagedattn_cache_row.h"
#include "pagedattn_device.h"
#include "pagedattn_internal.h"
#include "pagedattn_probe_launch.h"
#include "pagedattn_timed_launch.h"

namespace {

using namespace pa_dev;

// ------------------------------------------------------------ cache write
// Grid (num_tokens), kCacheThreads threads: block t copies token t's K and V
// rows, all kv-heads, 16 bytes per lane (cache_write_token).
__global__ __launch_bounds__(kCacheThreads) void pa_reshape_and_cache(
    const u32x4 *__restrict__ k, const u32x4 *__restrict__ v, u32x4 *__restrict__ k_pool,
    u32x4 *__restrict__ v_pool, const int64_t *__restrict__ slot_mapping, int num_kv_heads,
    int row_chunks, int block_size, int64_t num_slots) {
  cache_write_token(blockIdx.x, threadIdx.x, k, v, k_pool, v_pool, slot_mapping, num_kv_heads,
                    row_chunks, block_size, num_slots);
}

// ------------------------------------------------ cache write with RoPE
// The position encodings the engine serves include RoPE (showapi.com
// article, section 4.1): K is rotated by its token's position before it is
// cached, and q by the same rotation before attention.  This kernel does
// both in the one pass that writes the cache.  Grid (num_tokens), 256
// threads; a thread takes 16-byte chunks of the token's rows (q heads
// first, then kv-heads):
//   rotary chunks   split halves: chunk j and chunk j + half hold the two
//                   members of pairs j*E .. j*E + E-1; interleaved: one
//                   chunk holds E/2 whole pairs.  Rotated in fp32 with the
//                   table row cos_sin[pos] (cosines, then sines), rounded
//                   to the element type.
//   other chunks    K copied as is (q untouched).
// q is rotated in place; K (rotated) and V go to the page slot.  A token
// whose position is outside the table is skipped, and one whose slot is
// negative or past the pool gets its q rotated but writes no K/V.
// n consecutive floats from p, in 16- or 8-byte steps as n and the
// alignment of p (16 bytes when n is a multiple of 4, else 8) allow
template <int N>
__device__ __forceinline__ void load_floats(const float *p, float (&o)[N]) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      const float4 v = *reinterpret_cast<const float4 *>(p + i);
      o[i] = v.x;
      o[i + 1] = v.y;
      o[i + 2] = v.z;
      o[i + 3] = v.w;
    }
  } else {
    static_assert(N % 2 == 0, "pairs of floats");
#pragma unroll
    for (int i = 0; i < N; i += 2) {
      const float2 v = *reinterpret_cast<const float2 *>(p + i);
      o[i] = v.x;
      o[i + 1] = v.y;
    }
  }
}

template <class T>
__global__ __launch_bounds__(256) void pa_reshape_and_cache_rope(
    u32x4 *__restrict__ q, const u32x4 *__restrict__ k, const u32x4 *__restrict__ v,
    u32x4 *__restrict__ k_pool, u32x4 *__restrict__ v_pool,
    const int64_t *__restrict__ slot_mapping, const int64_t *__restrict__ positions,
    const float *__restrict__ cos_sin, int num_heads, int num_kv_heads, int row_chunks,
    int block_size, int64_t num_slots, int rot_dim, int max_position, int neox) {
  constexpr int E = T::kPerChunk;
  const int t = blockIdx.x;
  const int64_t pos = positions[t];
  if (pos < 0 || pos >= max_position) return;
  const int64_t slot = slot_mapping[t];
  const bool write = slot >= 0 && slot < num_slots;
  const int64_t page = write ? slot / block_size : 0;
  const int64_t off = write ? slot - page * block_size : 0;
  // the table row: rot_dim / 2 cosines then as many sines (rot_dim is a
  // multiple of 2 * E and the table 16-byte aligned, so every group of
  // values a unit reads is aligned to its size)
  const float *cs = cos_sin + pos * rot_dim;
  const int half = rot_dim / 2;
  const int rot_chunks = rot_dim / E;
  // units of a row: split halves take chunk pairs (j, j + rot_chunks / 2),
  // interleaved pairs one chunk each; chunks past rot_dim pass through
  const int units = neox ? row_chunks - rot_chunks / 2 : row_chunks;
  const int rows = num_heads + (write ? num_kv_heads : 0);
  for (int u = threadIdx.x; u < rows * units; u += blockDim.x) {
    const int r = u / units;
    const int j = u - r * units;
    const bool is_q = r < num_heads;
    const int g = r - num_heads;
    u32x4 *qrow = q + ((size_t)t * num_heads + r) * row_chunks;
    const u32x4 *krow = k + ((size_t)t * num_kv_heads + g) * row_chunks;
    u32x4 *prow = k_pool + (((size_t)page * num_kv_heads + g) * block_size + off) * row_chunks;
    const u32x4 *src = is_q ? qrow : krow;
    u32x4 *dst = is_q ? qrow : prow;
    if (neox) {
      if (j >= rot_chunks / 2) {  // past rot_dim
        if (!is_q) prow[j + rot_chunks / 2] = krow[j + rot_chunks / 2];
        continue;
      }
      const int c2 = j + rot_chunks / 2;
      float a[E], b[E], co[E], si[E];
      T::unpack(src[j], a);
      T::unpack(src[c2], b);
      load_floats(cs + j * E, co);
      load_floats(cs + half + j * E, si);
      float ra[E], rb[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        ra[e] = a[e] * co[e] - b[e] * si[e];
        rb[e] = b[e] * co[e] + a[e] * si[e];
      }
      dst[j] = T::pack(ra);
      dst[c2] = T::pack(rb);
    } else {
      if (j >= rot_chunks) {
        if (!is_q) prow[j] = krow[j];
        continue;
      }
      // chunk j holds pairs j*E/2 .. j*E/2 + E/2 - 1
      float x[E], y[E], co[E / 2], si[E / 2];
      T::unpack(src[j], x);
      load_floats(cs + j * (E / 2), co);
      load_floats(cs + half + j * (E / 2), si);
#pragma unroll
      for (int e = 0; e < E / 2; ++e) {
        y[2 * e] = x[2 * e] * co[e] - x[2 * e + 1] * si[e];
        y[2 * e + 1] = x[2 * e + 1] * co[e] + x[2 * e] * si[e];
      }
      dst[j] = T::pack(y);
    }
  }
  if (!write) return;
  for (int u = threadIdx.x; u < num_kv_heads * row_chunks; u += blockDim.x) {
    const int g = u / row_chunks;
    const int c = u - g * row_chunks;
    v_pool[(((size_t)page * num_kv_heads + g) * block_size + off) * row_chunks + c] =
        v[((size_t)t * num_kv_heads + g) * row_chunks + c];
  }
}

// ------------------------------------------------------------ page copy
// Grid (num_pairs, chunks per page), 256 threads.  Workgroup (i, c) copies
// chunk c (16 KiB) of page mapping[i][0] of the source pools to page
// mapping[i][1] of the destination pools, K and V, with 16-byte
// non-temporal loads and stores; all eight loads of a thread are issued
// before its stores.  A pair with a page index outside its pool (negative
// included) is skipped.  Source and destination may be device memory or
// pinned host memory mapped into the device's address space.
constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;
constexpr int kCopyChunk16 = kCopyThreads * kCopyUnroll;  // 16-byte units per chunk

__global__ __launch_bounds__(kCopyThreads) void pa_copy_pages(
    const u32x4 *__restrict__ k_src, const u32x4 *__restrict__ v_src, u32x4 *__restrict__ k_dst,
    u32x4 *__restrict__ v_dst, const int64_t *__restrict__ mapping, int64_t page16,
    int64_t src_blocks, int64_t dst_blocks) {
  const int64_t src = mapping[2 * (size_t)blockIdx.x];
  const int64_t dst = mapping[2 * (size_t)blockIdx.x + 1];
  if (src < 0 || dst < 0 || src >= src_blocks || dst >= dst_blocks) return;
  const int64_t base = (int64_t)blockIdx.y * kCopyChunk16 + threadIdx.x;
  u32x4 kv[kCopyUnroll], vv[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t i = base + u * kCopyThreads;
    if (i < page16) {
      kv[u] = __builtin_nontemporal_load(k_src + src * page16 + i);
      vv[u] = __builtin_nontemporal_load(v_src + src * page16 + i);
    }
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t i = base + u * kCopyThreads;
    if (i < page16) {
      __builtin_nontemporal_store(kv[u], k_dst + dst * page16 + i);
      __builtin_nontemporal_store(vv[u], v_dst + dst * page16 + i);
    }
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
// ------------------------------------------ decode access-pattern probe
// Reads the K and V bytes a decode call reads, in the order the partition
// kernels read them: items (unit, kv-head) of the plan's list, largest units
// first, kv-head fastest, in the snake rounds of snake_item.  WPI == NW: one
// workgroup of NW waves per item (8 where the VALU kernel runs bf16 with one
// query head per kv-head, else 4), the unit's pages dealt to the waves in
// turn.  WPI == 1 (what the grouped-query kernel does for long tables of
// short partitions): wave w of the workgroup's k-th step takes item
// NW * snake_item(k) + w whole.  Each (page, kv-head) run is read as 1 KiB
// wave loads (16 bytes per lane), non-temporal, two pages in flight per
// wave where a run is at most 4 KiB.  In place of the attention arithmetic
// the loaded words are XORed, and each item stores its 16-byte XOR in the
// first chunk of its first query head's output row, which keeps every load
// live (out receives no attention result; items of one sequence's different
// partitions overwrite each other's word).  The rate it reaches is the read
// bandwidth of the decode access pattern on the device, the ceiling the
// partition kernels work against.
template <int NLD, int NW, int WPI>
__global__ __launch_bounds__(64 * NW) void pa_decode_read_probe(
    char *__restrict__ out, const char *__restrict__ k_pool, const char *__restrict__ v_pool,
    const int32_t *__restrict__ block_tables, const int32_t *__restrict__ context_lens,
    const int32_t *__restrict__ plan, int num_seqs, int num_heads, int num_kv_heads,
    int max_blocks, int num_blocks, int block_size, int part_pages, int max_parts,
    int head_row_bytes) {
  constexpr int kRun = NLD * 1024;  // bytes of one (page, kv-head) run
  constexpr int PF = NLD <= 4 ? 2 : 1;
  static_assert(WPI == 1 || WPI == NW, "an item takes one wave or the whole workgroup");
  __shared__ u32x4 s_x[NW];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int iw = WPI == 1 ? 0 : wave;  // this wave's place among the item's waves
  const long long bound = (long long)num_seqs * max_parts * num_kv_heads;
  const size_t page_stride = (size_t)num_kv_heads * kRun;

  // this wave's share of item (unit, kv-head g): the XOR over the whole wave
  auto item_xor = [&](int unit, int g) -> u32x4 {
    const int s = unit / max_parts;
    const int part = unit - s * max_parts;
    const int ctx = min(max(context_lens[s], 0), max_blocks * block_size);
    const int npages = (ctx + block_size - 1) / block_size;
    const int p_begin = part * part_pages;
    const int np = max(0, min(npages - p_begin, part_pages));
    const int np_w = iw < np ? (np - iw + WPI - 1) / WPI : 0;  // this wave's pages
    const int col = p_begin + iw + WPI * lane;
    int my_bid = -1;
    if (iw + WPI * lane < part_pages && col < max_blocks)
      my_bid = block_tables[(size_t)s * max_blocks + col];
    const char *kb = k_pool + (size_t)g * kRun + lane * 16;
    const char *vb = v_pool + (size_t)g * kRun + lane * 16;
    u32x4 x = {0u, 0u, 0u, 0u};
    auto fetch = [&](u32x4 (&c)[2 * NLD], int j) {
      const int bid = __builtin_amdgcn_readlane(my_bid, j);
      const size_t off = (size_t)((unsigned)bid < (unsigned)num_blocks ? bid : 0) * page_stride;
#pragma unroll
      for (int i = 0; i < NLD; ++i) c[i] = load_kv16(kb + off + i * 1024);
#pragma unroll
      for (int i = 0; i < NLD; ++i) c[NLD + i] = load_kv16(vb + off + i * 1024);
    };
    auto fold = [&](const u32x4 (&c)[2 * NLD]) {
#pragma unroll
      for (int i = 0; i < 2 * NLD; ++i) x ^= c[i];
    };
    if constexpr (PF == 2) {
      if (np_w > 0) {
        u32x4 a[2 * NLD], b[2 * NLD];
        fetch(a, 0);
        int j = 0;
        for (; j + 2 < np_w; j += 2) {
          fetch(b, j + 1);
          fold(a);
          fetch(a, j + 2);
          fold(b);
        }
        if (j + 1 < np_w) {
          fetch(b, j + 1);
          fold(a);
          fold(b);
        } else {
          fold(a);
        }
      }
    } else {
      for (int j = 0; j < np_w; ++j) {
        u32x4 c[2 * NLD];
        fetch(c, j);
        fold(c);
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
#pragma unroll
      for (int w = 0; w < 4; ++w) x[w] ^= (uint32_t)__shfl_xor((int)x[w], o);
    return x;
  };
  auto word = [&](int unit, int g) {
    const int s = unit / max_parts;
    const int h0 = g * (num_heads / num_kv_heads);
    return reinterpret_cast<u32x4 *>(out + ((size_t)s * num_heads + h0) * head_row_bytes);
  };

  if constexpr (WPI == 1) {
    for (int k = 0;; ++k) {
      const long long it = (long long)snake_item(k) * NW + wave;
      if (it >= bound) break;
      const int unit = plan[pa_internal::kPlanHeader + it / num_kv_heads];
      if (unit < 0) break;
      const int g = (int)(it % num_kv_heads);
      const u32x4 x = item_xor(unit, g);
      if (lane == 0) *word(unit, g) = x;
    }
  } else {
    for (int k = 0;; ++k) {
      const int it = snake_item(k);
      if (it >= bound) break;
      const int unit = plan[pa_internal::kPlanHeader + it / num_kv_heads];
      if (unit < 0) break;
      const int g = it % num_kv_heads;
      const u32x4 x = item_xor(unit, g);
      if (lane == 0) s_x[wave] = x;
      __syncthreads();
      if (threadIdx.x == 0) {
        u32x4 x_all = s_x[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) x_all ^= s_x[w];
        *word(unit, g) = x_all;
      }
      __syncthreads();  // s_x is reused by the next item
    }
  }
}

}  // namespace

namespace pa_internal {

int launch_reshape_and_cache(const CacheLaunch &a) {
  hipStream_t st = reinterpret_cast<hipStream_t>(a.stream);
  const int row_chunks = a.head_dim * a.elem_bytes / 16;
  hipLaunchKernelGGL(pa_reshape_and_cache, dim3(a.num_tokens), dim3(kCacheThreads), 0, st,
                     reinterpret_cast<const u32x4 *>(a.k), reinterpret_cast<const u32x4 *>(a.v),
                     reinterpret_cast<u32x4 *>(a.k_pool), reinterpret_cast<u32x4 *>(a.v_pool),
                     a.slot_mapping, a.num_kv_heads, row_chunks, a.block_size,
                     (int64_t)a.num_blocks * a.block_size);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

int launch_reshape_and_cache_rope(const RopeLaunch &r) {
  const CacheLaunch &a = r.cache;
  hipStream_t st = reinterpret_cast<hipStream_t>(a.stream);
  const int row_chunks = a.head_dim * a.elem_bytes / 16;
  auto kernel = a.elem_bytes == 2 ? pa_reshape_and_cache_rope<BF16> : pa_reshape_and_cache_rope<F32>;
  hipLaunchKernelGGL(kernel, dim3(a.num_tokens), dim3(256), 0, st,
                     reinterpret_cast<u32x4 *>(r.q), reinterpret_cast<const u32x4 *>(a.k),
                     reinterpret_cast<const u32x4 *>(a.v), reinterpret_cast<u32x4 *>(a.k_pool),
                     reinterpret_cast<u32x4 *>(a.v_pool), a.slot_mapping, r.positions, r.cos_sin,
                     r.num_heads, a.num_kv_heads, row_chunks, a.block_size,
                     (int64_t)a.num_blocks * a.block_size, r.rot_dim, r.max_position, r.neox);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

// The address a kernel uses for p: device memory as it is; pinned host
// memory through its mapping into the device's address space.  Anything
// else (pageable host memory) gives nullptr, since a kernel access to it
// would fault.
const void *device_address(const void *p) {
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();  // a failed query must not look like a launch error
    return nullptr;
  }
  switch (at.type) {
    case hipMemoryTypeDevice:
    case hipMemoryTypeManaged:
    case hipMemoryTypeUnified:
      return p;
    case hipMemoryTypeHost: {
      if (!at.devicePointer || !at.hostPointer) return nullptr;
      const ptrdiff_t off = static_cast<const char *>(p) - static_cast<const char *>(at.hostPointer);
      return static_cast<const char *>(at.devicePointer) + off;
    }
    default:
      return nullptr;
  }
}

int launch_copy_pages(const CopyLaunch &a) {
  const void *ks = device_address(a.k_src), *vs = device_address(a.v_src);
  const void *kd = device_address(a.k_dst), *vd = device_address(a.v_dst);
  const void *map = device_address(a.mapping);
  if (!ks || !vs || !kd || !vd || !map) return 3;  // PA_ERR_UNSUPPORTED: not device-accessible
  hipStream_t st = reinterpret_cast<hipStream_t>(a.stream);
  const int64_t page16 = a.page_bytes / 16;
  const unsigned chunks = (unsigned)((page16 + kCopyChunk16 - 1) / kCopyChunk16);
  hipLaunchKernelGGL(pa_copy_pages, dim3(a.num_pairs, chunks), dim3(kCopyThreads), 0, st,
                     static_cast<const u32x4 *>(ks), static_cast<const u32x4 *>(vs),
                     static_cast<u32x4 *>(const_cast<void *>(kd)),
                     static_cast<u32x4 *>(const_cast<void *>(vd)),
                     static_cast<const int64_t *>(map), page16, (int64_t)a.src_blocks,
                     (int64_t)a.dst_blocks);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

size_t hbm_probe_sink_bytes() { return (size_t)kProbeBlocks * kProbeThreads * 4; }

template <int NLD, int NW, int WPI>
int launch_read_probe_wpi(const DecodeLaunch &a) {
  auto kernel = pa_decode_read_probe<NLD, NW, WPI>;
  static const int per_cu = blocks_per_cu(reinterpret_cast<const void *>(kernel), 64 * NW);
  // an item covers a.chain partitions (one unless WPI == 1)
  const int units = (a.max_parts + a.chain - 1) / a.chain;
  const long long items = (long long)a.num_seqs * units * a.num_kv_heads;
  const unsigned grid = WPI == 1 ? persistent_grid_items((items + NW - 1) / NW,
                                                         per_cu * kDecodeGridRounds)
                                 : decode_grid(a, per_cu);
  if (grid == 0) return 6;
  pa_internal::launch_timed(kernel, dim3(grid), dim3(64 * NW),
                            reinterpret_cast<hipStream_t>(a.stream), a.ev_begin, a.ev_end,
                            reinterpret_cast<char *>(a.out), reinterpret_cast<const char *>(a.k_pool),
                     reinterpret_cast<const char *>(a.v_pool), a.block_tables, a.context_lens,
                     a.plan, a.num_seqs, a.num_heads, a.num_kv_heads, a.max_blocks, a.num_blocks,
                     a.block_size, a.part_pages * a.chain, units,
                     a.head_dim * (a.dtype == 0 ? 4 : 2));
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

// the partition kernels' item shape: the grouped-query kernel's one wave
// per item or four waves per item; the VALU kernel's eight waves for bf16
// with one query head per kv-head, else four
template <int NLD>
int launch_read_probe_nld(const DecodeLaunch &a) {
  const int group = a.num_heads / a.num_kv_heads;
  if (a.dtype == 1 && group >= 2)
    return gqa_wave_items(a) ? launch_read_probe_wpi<NLD, 4, 1>(a)
                             : launch_read_probe_wpi<NLD, 4, 4>(a);
  return a.dtype == 1 && group == 1 ? launch_read_probe_wpi<NLD, 8, 8>(a)
                                    : launch_read_probe_wpi<NLD, 4, 4>(a);
}

int launch_decode_read_probe(const DecodeLaunch &call) {
  // items of the partition kernels' shape, runs of partitions included
  DecodeLaunch a = call;
  a.chain = decode_chain(call);
  if (launch_decode_plan(a) != 0) return 6;
  // the probe kernel's launch records the timing events, if any
  const int run_bytes = a.block_size * a.head_dim * (a.dtype == 0 ? 4 : 2);
  int rc = 3;
  switch (run_bytes / 1024) {
    case 2: rc = launch_read_probe_nld<2>(a); break;
    case 4: rc = launch_read_probe_nld<4>(a); break;
    case 8: rc = launch_read_probe_nld<8>(a); break;
    case 16: rc = launch_read_probe_nld<16>(a); break;
  }
  return rc;
}

int launch_hbm_probe(const void *buf, size_t bytes, void *sink, void *stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const size_t n16 = bytes / 16;
  hipLaunchKernelGGL(pa_hbm_probe, dim3(kProbeBlocks), dim3(kProbeThreads), 0, st,
                     reinterpret_cast<const u32x4 *>(buf), n16,
                     (n16 + kProbeBlocks - 1) / kProbeBlocks, reinterpret_cast<uint32_t *>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

}  // namespace pa_internal
