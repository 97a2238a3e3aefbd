// Device-side helpers shared by the HIP kernels of libpagedattn (gfx950):
// element types, wavefront reductions and load wrappers.  Header-only; every
// kernel translation unit includes it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa_dev {

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
  // (a select, not a branch: the compiler would otherwise give every value
  // its own masked block)
  __device__ static uint32_t round_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    const uint32_t quiet = (u >> 16) | 0x40u;
    return (u & 0x7fffffffu) > 0x7f800000u ? quiet : rounded;
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

// Item of the k-th round of a persistent grid walking a list sorted largest
// first: rounds alternate direction (workgroup b takes items b, 2P-1-b,
// 2P+b, 4P-1-b, ... for a grid of P), so the workgroups that start with the
// largest items of one round take the smallest of the next and the totals
// even out.  Beyond the last item a workgroup has nothing left in later
// rounds either.
__device__ __forceinline__ int snake_item(int k) {
  const int b = (k & 1) ? (int)gridDim.x - 1 - (int)blockIdx.x : (int)blockIdx.x;
  const long long it = (long long)k * gridDim.x + b;
  return it > 0x7fffffffLL ? 0x7fffffff : (int)it;
}

// Merge the NW waves' partial softmax states of one work unit (sequence,
// kv-head, partition) and store the result: normalised output rows when the
// unit covers the whole sequence, else the partition's unnormalised
// (max, sum, accumulator) for the reduce kernel.  acc(w, h, d) gives wave
// w's accumulator for head h at d..d+3, mx / sm its running max (log2 units)
// and sum.  Each thread handles 4 consecutive outputs of one head.
//   out_rows     first output row of the unit's G heads ([G][D] of T)
//   ws_acc_rows  the partition's partial accumulators of the unit's G heads
//                ([G][D] floats, consecutive heads adjacent)
//   ws_ml_rows   their partial (max, sum) pairs ([G][2])
template <class T, int D, int G, int NW, class AccF, class MaxF, class SumF>
__device__ __forceinline__ void merge_waves(AccF acc, MaxF mx, SumF sm, bool whole,
                                            char *out_rows, float *ws_acc_rows,
                                            float *ws_ml_rows) {
  for (int idx = threadIdx.x; idx < G * D / 4; idx += 64 * NW) {
    const int h = idx / (D / 4);
    const int d = (idx % (D / 4)) * 4;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, mx(w, h));
    float L = 0.f, o[4] = {0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float sc = fast_exp2(mx(w, h) - M);
        L = fmaf(sm(w, h), sc, L);
        const float4 a = acc(w, h, d);
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
      T::store4(out_rows + ((size_t)h * D + d) * T::kBytes, o);
    } else {
      *reinterpret_cast<float4 *>(ws_acc_rows + (size_t)h * D + d) =
          make_float4(o[0], o[1], o[2], o[3]);
      if (d == 0) {
        ws_ml_rows[h * 2] = M;
        ws_ml_rows[h * 2 + 1] = L;
      }
    }
  }
}

}  // namespace pa_dev
