// Pieces shared by the kernel translation units of libpa (gfx950): operand
// vector types, bf16 conversion, 16-byte moves, the cross-lane-group
// reductions the matrix-core kernels use, argument checks and launch timing.
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

inline bool geom_ok(const pa_geom* g) {
  return g && g->num_layers > 0 && g->num_kv_heads > 0 && g->head_dim > 0 && g->block_size > 0 &&
         g->num_blocks > 0 && (g->dtype == PA_F32 || g->dtype == PA_BF16 || g->dtype == PA_FP8);
}
inline int64_t esize(const pa_geom* g) {
  return g->dtype == PA_F32 ? 4 : g->dtype == PA_BF16 ? 2 : 1;
}
// Bytes of one (layer, block, head) tile of K or V: B*d elements, and for FP8
// pools the B scale bytes that follow them.
inline int64_t tile_bytes(const pa_geom* g) {
  return (int64_t)g->block_size * g->head_dim * esize(g) + (g->dtype == PA_FP8 ? g->block_size : 0);
}

inline pa_status launch_status() { return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP; }

// Records hipEvents around one launch when timing is on (pa_prof_enable).
struct ProfScope {
  const char* name;
  hipStream_t st;
  hipEvent_t a = nullptr, b = nullptr;
  bool on;
  ProfScope(const char* n, hipStream_t s);
  ~ProfScope();
};

}  // namespace pa_detail
