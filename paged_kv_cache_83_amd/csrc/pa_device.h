// Device pieces shared by the kernel translation units of libpa (gfx950):
// operand vector types, bf16 conversion, 16-byte moves, the cross-lane-group
// reductions the matrix-core kernels use, split partial loads, stores and
// merges. The host side (argument checks, launch timing) is in pa_host.h.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/pa.h"

namespace pa_detail {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest even; NaN stays a quiet NaN of the same sign.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<uint16_t>(uint16_t v) { return bf16_to_f32(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ uint16_t from_f32<uint16_t>(float v) { return f32_to_bf16(v); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Attended length of sequence i, clamped into [0, max_ctx].
__device__ __forceinline__ int clamp_len(const int32_t* lens, int i, int max_ctx) {
  int len = lens[i];
  return len < 0 ? 0 : (len > max_ctx ? max_ctx : len);
}

__device__ __forceinline__ int guard_block(int p, int N) { return (p >= 0 && p < N) ? p : 0; }

// Width of the K dimension chunks: 32 when it divides d, else the whole d.
__host__ __device__ __forceinline__ int k_chunk(int D) { return (D % 32 == 0) ? 32 : D; }

// VEC elements of T as one 16-byte access when they make up exactly 16 bytes
// (the callers guarantee 16-byte alignment then), element by element otherwise.
template <typename T, int VEC>
__device__ __forceinline__ void load_vec(T (&dst)[VEC], const T* src) {
  if constexpr (VEC * sizeof(T) == 16) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(src);
    __builtin_memcpy(&dst[0], &v, 16);
  } else {
#pragma unroll
    for (int u = 0; u < VEC; ++u) dst[u] = src[u];
  }
}
template <typename T, int VEC>
__device__ __forceinline__ void store_vec(T* dst, const T (&src)[VEC]) {
  if constexpr (VEC * sizeof(T) == 16) {
    u32x4 v;
    __builtin_memcpy(&v, &src[0], 16);
    *reinterpret_cast<u32x4*>(dst) = v;
  } else {
#pragma unroll
    for (int u = 0; u < VEC; ++u) dst[u] = src[u];
  }
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 (hardware round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Max / sum over lanes l, l^16, l^32, l^48 (the four lane groups holding one
// query's keys), through the gfx950 cross-row swap instructions.
__device__ __forceinline__ float max_over_groups(float v) {
  uint32_t u = __float_as_uint(v);
  auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  u = __float_as_uint(v);
  auto b = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_groups(float v) {
  uint32_t u = __float_as_uint(v);
  auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  u = __float_as_uint(v);
  auto b = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Loads and stores of split partials. COH = true: agent-scope relaxed atomic
// accesses, which the compiler emits as coherent (sc1) loads and stores, so a
// partial written by a work item on one XCD is read correctly by the work item
// that merges it on another without writing back or invalidating any L2.
template <bool COH>
__device__ __forceinline__ float part_ld(const float* p) {
  if constexpr (COH)
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    return *p;
}
template <bool COH>
__device__ __forceinline__ float4 part_ld4(const float* p) {
  if constexpr (COH)
    return make_float4(part_ld<true>(p), part_ld<true>(p + 1), part_ld<true>(p + 2), part_ld<true>(p + 3));
  else
    return *reinterpret_cast<const float4*>(p);
}
__device__ __forceinline__ void part_st_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Merge the ns split partials of one (sequence, query head) with the
// online-softmax rule of "KV Cache Management", section "Chunked prefill
// mechanics": M = max_s m_s, w_s = 2^(m_s - M), out = sum_s w_s o_s / sum_s w_s l_s
// (m in log2 units: scores were scaled by log2 e). po: the ns rows of D floats,
// ml: their ns (m, l) pairs. One wave, ns >= 1; writes the D outputs. COH picks
// coherent loads (partials written by other work items of the same launch);
// the arithmetic, hence every output bit, is the same either way.
template <typename T, bool COH = false>
__device__ __forceinline__ void merge_split_row(const float* __restrict__ po,
                                                const float* __restrict__ ml, int ns, int D,
                                                T* __restrict__ o, int lane) {
  const int C4 = D >> 2;  // float4 columns of one partial row
  if ((D & 3) == 0 && C4 <= 64 && (64 % C4) == 0 && ns <= 64) {
    // Lane s holds split s's (m, l); lane (grp, col) sums column col of every
    // groups-th split, then the groups are summed across lanes. Every (m, l)
    // and the first kU rows of each lane are requested together, so the merge
    // waits for memory once; a split's weight 2^(m_s - M) is computed by lane s
    // and fetched from it (every lane takes part: callers run the whole wave).
    // The same arithmetic, in the same order, as the general form below.
    constexpr int kU = 8;
    const int groups = 64 / C4;
    const int col = lane % C4;
    const int grp = lane / C4;
    float mv = -INFINITY, lv = 0.f;
    if (lane < ns) {
      mv = part_ld<COH>(ml + 2 * lane);
      lv = part_ld<COH>(ml + 2 * lane + 1);
    }
    float4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int s = grp + u * groups;
      v[u] = s < ns ? part_ld4<COH>(po + (int64_t)s * D + 4 * col) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const float M = wave_max(mv);
    const float w = lane < ns ? exp2f(mv - M) : 0.f;
    const float inv = 1.f / wave_sum(w * lv);
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int s = grp + u * groups;   // < 64
      const float ww = __shfl(w, s);
      if (s < ns) {
        a.x = fmaf(ww, v[u].x, a.x);
        a.y = fmaf(ww, v[u].y, a.y);
        a.z = fmaf(ww, v[u].z, a.z);
        a.w = fmaf(ww, v[u].w, a.w);
      }
    }
    for (int s = grp + kU * groups; s < ns; s += groups) {   // (lanes diverge: no fetch)
      const float4 x = part_ld4<COH>(po + (int64_t)s * D + 4 * col);
      const float ww = exp2f(part_ld<COH>(ml + 2 * s) - M);
      a.x = fmaf(ww, x.x, a.x);
      a.y = fmaf(ww, x.y, a.y);
      a.z = fmaf(ww, x.z, a.z);
      a.w = fmaf(ww, x.w, a.w);
    }
    for (int off = C4; off < 64; off <<= 1) {
      a.x += __shfl_xor(a.x, off);
      a.y += __shfl_xor(a.y, off);
      a.z += __shfl_xor(a.z, off);
      a.w += __shfl_xor(a.w, off);
    }
    if (grp == 0) {
      o[4 * col + 0] = from_f32<T>(a.x * inv);
      o[4 * col + 1] = from_f32<T>(a.y * inv);
      o[4 * col + 2] = from_f32<T>(a.z * inv);
      o[4 * col + 3] = from_f32<T>(a.w * inv);
    }
    return;
  }
  float M = -INFINITY;
  for (int s = lane; s < ns; s += 64) M = fmaxf(M, part_ld<COH>(ml + 2 * s));
  M = wave_max(M);
  float Lsum = 0.f;
  for (int s = lane; s < ns; s += 64)
    Lsum += exp2f(part_ld<COH>(ml + 2 * s) - M) * part_ld<COH>(ml + 2 * s + 1);
  Lsum = wave_sum(Lsum);
  const float inv = 1.f / Lsum;
  if ((D & 3) == 0 && C4 <= 64 && (64 % C4) == 0) {
    // more than 64 splits: the same lanes and order, loads four deep
    const int groups = 64 / C4;
    const int col = lane % C4;
    const int grp = lane / C4;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    int s = grp;
    for (; s + 3 * groups < ns; s += 4 * groups) {
      float4 x[4];
      float wt[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        x[u] = part_ld4<COH>(po + (int64_t)(s + u * groups) * D + 4 * col);
        wt[u] = part_ld<COH>(ml + 2 * (s + u * groups));
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float ww = exp2f(wt[u] - M);
        a.x = fmaf(ww, x[u].x, a.x);
        a.y = fmaf(ww, x[u].y, a.y);
        a.z = fmaf(ww, x[u].z, a.z);
        a.w = fmaf(ww, x[u].w, a.w);
      }
    }
    for (; s < ns; s += groups) {
      const float4 x = part_ld4<COH>(po + (int64_t)s * D + 4 * col);
      const float ww = exp2f(part_ld<COH>(ml + 2 * s) - M);
      a.x = fmaf(ww, x.x, a.x);
      a.y = fmaf(ww, x.y, a.y);
      a.z = fmaf(ww, x.z, a.z);
      a.w = fmaf(ww, x.w, a.w);
    }
    for (int off = C4; off < 64; off <<= 1) {
      a.x += __shfl_xor(a.x, off);
      a.y += __shfl_xor(a.y, off);
      a.z += __shfl_xor(a.z, off);
      a.w += __shfl_xor(a.w, off);
    }
    if (grp == 0) {
      o[4 * col + 0] = from_f32<T>(a.x * inv);
      o[4 * col + 1] = from_f32<T>(a.y * inv);
      o[4 * col + 2] = from_f32<T>(a.z * inv);
      o[4 * col + 3] = from_f32<T>(a.w * inv);
    }
    return;
  }
  for (int d = lane; d < D; d += 64) {
    float a = 0.f;
    for (int s = 0; s < ns; ++s)
      a = fmaf(exp2f(part_ld<COH>(ml + 2 * s) - M), part_ld<COH>(po + (int64_t)s * D + d), a);
    o[d] = from_f32<T>(a * inv);
  }
}

// Split arrival for the merge inside the decode kernel, called by every lane of
// a work item after it has written its partials with part_st_coherent; counter
// belongs to the item's (sequence, KV head) and counts the splits that have
// finished. The item's coherent stores complete before it counts itself, so
// the wave that finds ns - 1 splits counted before it -- the last, for which
// true is returned -- reads every partial with coherent loads (merge_split_row
// with COH), merges, and puts the counter back to 0.
__device__ __forceinline__ bool split_arrive_last(int* counter, int ns, int lane) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  int prev = 0;
  if (lane == 0) prev = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  prev = __shfl(prev, 0);
  asm volatile("" ::: "memory");
  return prev == ns - 1;
}

}  // namespace pa_detail
