// Whole-block moves between the paged pool and a staging buffer (or inside the
// pool), shared by the block-copy entry points and the asynchronous swapper.
//
// "KV Cache Management", sections "Zero-copy deliberation via copy-on-write
// branching" (a shared block is copied whole before a write) and "Asynchronous
// paged swapping" (blocks leave and re-enter the pool as whole frames).
//
// A "run" is one (layer, block, K-or-V) stretch of H_kv*B*d elements, contiguous
// in the pool. Staging frame i holds block ids[i] as 2*L runs, run (layer, kv)
// at ((i*L + layer)*2 + kv) * run_bytes. MODE 0: pool -> pool (copy-on-write
// copy, ids_a = source, ids_b = destination). MODE 1: pool -> staging (gather).
// MODE 2: staging -> pool (scatter). Work-group g moves runs g, g + G, g + 2G, ...
// for a grid of G work-groups: one run each when G covers them all (the block
// copies, which want the whole GPU), or a few work-groups paced against the
// host link (the swapper, which must leave the GPU to decode).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pa_detail {

// Block ids read from a device array.
struct PtrIds {
  const int32_t* p;
  __device__ int32_t operator()(int64_t i) const { return p[i]; }
};

// Up to kArgIds block ids carried in the kernel arguments themselves, so a
// launch needs no device-side id buffer (and nothing to keep alive until the
// kernel has run).
constexpr int kArgIds = 256;
struct ArgIds {
  int32_t v[kArgIds];
  __device__ int32_t operator()(int64_t i) const { return v[i]; }
};

// Stand-in for the unused second id list of a gather or scatter.
struct NoIds {
  __device__ int32_t operator()(int64_t) const { return -1; }
};

template <int MODE, typename V, typename IdsA, typename IdsB>
__global__ __launch_bounds__(256) void block_move_kernel(char* __restrict__ kpool,
                                                         char* __restrict__ vpool,
                                                         char* __restrict__ staging, IdsA ids_a,
                                                         IdsB ids_b, int L, int N,
                                                         int64_t run_bytes, int64_t runs) {
  for (int64_t r = blockIdx.x; r < runs; r += gridDim.x) {
    const int kv = (int)(r & 1);
    const int layer = (int)((r >> 1) % L);
    const int64_t i = (r >> 1) / L;
    char* pool = kv ? vpool : kpool;
    const char* src;
    char* dst;
    if (MODE == 0) {
      int a = ids_a(i), b = ids_b(i);
      if (a < 0 || a >= N || b < 0 || b >= N) continue;
      src = pool + ((int64_t)layer * N + a) * run_bytes;
      dst = pool + ((int64_t)layer * N + b) * run_bytes;
    } else {
      int a = ids_a(i);
      if (a < 0 || a >= N) continue;
      char* p = pool + ((int64_t)layer * N + a) * run_bytes;
      char* s = staging + (((i * L) + layer) * 2 + kv) * run_bytes;
      src = (MODE == 1) ? p : s;
      dst = (MODE == 1) ? s : p;
    }
    const V* sv = reinterpret_cast<const V*>(src);
    V* dv = reinterpret_cast<V*>(dst);
    const int64_t n = run_bytes / (int64_t)sizeof(V);
    constexpr int U = 4;
    for (int64_t base = threadIdx.x; base < n; base += (int64_t)blockDim.x * U) {
      V tmp[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        int64_t k = base + (int64_t)u * blockDim.x;
        if (k < n) tmp[u] = __builtin_nontemporal_load(sv + k);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        int64_t k = base + (int64_t)u * blockDim.x;
        if (k < n) __builtin_nontemporal_store(tmp[u], dv + k);
      }
    }
  }
}

}  // namespace pa_detail
