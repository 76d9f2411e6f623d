// Direct-to-register loads of a pair of 16-slot bf16 blocks (32 keys) as MFMA
// operand fragments, shared by the decode kernel and the short-chunk prefill
// kernel. Lane l = (c = l % 16, gq = l / 16) of a wave holds, for each 16x16x32
// product, A[row = c][k = 8*gq .. +8] and B[k = 8*gq .. +8][col = c]; the pool
// layout (K [N][H_kv][d/32][16][32], V [N][H_kv][d][16]) lets every fragment be
// one 16-byte load: a K row chunk of 8 dimensions, or 8 consecutive slots of
// one V dimension.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "pa_device.h"

namespace pa_detail {

constexpr int kMfmaMaxBps = 256;  // table entries of one split, held 64 per register

// Work list of a ragged launch, passed by value in the kernel arguments (so a
// captured graph keeps the list it was captured with): item k is (sequence,
// split) packed as sequence | split << 16, longest items first. A launch with
// more items than fit takes the uniform plan instead.
constexpr int kMaxRaggedItems = 896;
struct RaggedItems {
  int32_t n;
  uint32_t v[kMaxRaggedItems];
};
struct NoRaggedItems {};

#ifndef PA_MFMA_STAGES
#define PA_MFMA_STAGES 2
#endif
#ifndef PA_MFMA_WPE
#define PA_MFMA_WPE 2
#endif
template <int D>
struct MfmaCfg {
  static constexpr int KC = D / 32;  // QK k-steps
  static constexpr int DT = D / 16;  // PV row tiles
  static constexpr int kStages = PA_MFMA_STAGES;  // pairs of blocks in flight per wave
};

template <int D>
struct PairFrags {
  u32x4 k[2][MfmaCfg<D>::KC];
  u32x4 v[MfmaCfg<D>::DT];
};

// K/V tiles read once per step are streamed past the caches (non-temporal loads
// sustain ~12% more HBM read bandwidth on this part); tiles shared by many
// sequences of the batch use ordinary loads so the repeats hit in L2 / MALL.
template <bool NT>
__device__ __forceinline__ u32x4 kv_load16(const uint16_t* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  else return *reinterpret_cast<const u32x4*>(p);
}

// Block id at offset `off` (wave-uniform, < 256) of the split's table chunk:
// register off / 64 of lane off % 64, picked without branches.
__device__ __forceinline__ int table_at(const int (&tb)[4], int off) {
  const int r = off >> 6;
  const int v = r == 0 ? tb[0] : r == 1 ? tb[1] : r == 2 ? tb[2] : tb[3];
  return __builtin_amdgcn_readlane(v, off & 63);
}

// new_key: pair-local index (0..31) of the token appended in this launch, whose
// K row is taken from knew_row (its pool slot may not hold it yet), or -1.
template <int D, bool NT>
__device__ __forceinline__ void issue_pair(PairFrags<D>& f, const uint16_t* __restrict__ kl,
                                           const uint16_t* __restrict__ vl, int p0, int p1, int Hkv,
                                           int g, int k_sel, int k_off0, int v_sel, int v_off,
                                           int gq, int new_key, const uint16_t* knew_row) {
  constexpr int KC = MfmaCfg<D>::KC;
  constexpr int DT = MfmaCfg<D>::DT;
  constexpr int TILE = 16 * D;
  const uint16_t* krow = kl + ((int64_t)(k_sel ? p1 : p0) * Hkv + g) * TILE;
  const uint16_t* vrow = vl + ((int64_t)(v_sel ? p1 : p0) * Hkv + g) * TILE;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
      f.k[t][kc] = kv_load16<NT>(krow + kc * 512 + (k_off0 + 4 * t) * 32 + 8 * gq);
    if (16 * k_sel + k_off0 + 4 * t == new_key) {  // lane-divergent: plain loads
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        f.k[t][kc] = *reinterpret_cast<const u32x4*>(knew_row + 32 * kc + 8 * gq);
    }
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) f.v[dt] = kv_load16<NT>(vrow + dt * 256 + v_off);
}

// How a matrix-core decode launch hands out its results (a template argument
// of the kernels, so that a launch carries only the code of its own mode): the
// outputs themselves (one split covers every sequence), split partials for the
// combine launch, or split partials merged inside the launch by each
// sequence's last split.
enum : int { kOutPartial = 0, kOutDirect = 1, kOutMerge = 2 };

// End of a matrix-core decode work item (sequence i, KV head g, split s). Lane
// (c = lane % 16, gq = lane / 16) holds O^T[d = 16*dt + 4*gq + e][query c] in
// acc[dt][e] for query head h = g*G + c (valid for c < G), and the split's
// (m, l) for that head (l already summed over the lane groups). A split that
// covers the sequence (kOutDirect, or a one-split sequence) writes the
// normalised output; otherwise the split's partial row goes to the workspace --
// with kOutMerge as coherent stores, after which the last split of (i, g) to
// finish (counted in counters) merges every row of the group (the in-kernel
// merge of "KV Cache Management", section "Chunked prefill mechanics"). Called
// by the whole wave.
template <int D, int OUT>
__device__ __forceinline__ void mfma_split_epilogue(const f32x4 (&acc)[D / 16], float m_run,
                                                    float l_run, int lane, int i, int g, int G,
                                                    int Hq, int Hkv, int s, int S_max, int ns,
                                                    uint16_t* __restrict__ out,
                                                    float* __restrict__ part_o,
                                                    float* __restrict__ part_ml,
                                                    int* __restrict__ counters) {
  constexpr int DT = D / 16;
  const int c = lane & 15;
  const int gq = lane >> 4;
  const int h = g * G + c;
  const bool qvalid = c < G;
  if (OUT == kOutDirect || ns == 1) {   // one split covers the sequence: the output itself
    if (!qvalid) return;
    const float inv = 1.f / l_run;
    uint16_t* o = out + ((int64_t)i * Hq + h) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<uint2*>(o + 16 * dt + 4 * gq) =
          make_uint2(pack_bf16x2(acc[dt][0] * inv, acc[dt][1] * inv),
                     pack_bf16x2(acc[dt][2] * inv, acc[dt][3] * inv));
    return;
  }
  const int64_t row = ((int64_t)i * Hq + (qvalid ? h : g * G)) * S_max + s;
  float* po = part_o + row * D;
  if constexpr (OUT == kOutPartial) {
    if (!qvalid) return;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<float4*>(po + 16 * dt + 4 * gq) =
          make_float4(acc[dt][0], acc[dt][1], acc[dt][2], acc[dt][3]);
    if (gq == 0) {
      part_ml[row * 2 + 0] = m_run;
      part_ml[row * 2 + 1] = l_run;
    }
    return;
  } else {
  if (qvalid) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e) part_st_coherent(po + 16 * dt + 4 * gq + e, acc[dt][e]);
    if (gq == 0) {
      part_st_coherent(part_ml + row * 2 + 0, m_run);
      part_st_coherent(part_ml + row * 2 + 1, l_run);
    }
  }
  if (split_arrive_last(counters + (int64_t)i * Hkv + g, ns, lane)) {
#pragma unroll 1
    for (int t = 0; t < G; ++t) {
      const int64_t row0 = ((int64_t)i * Hq + g * G + t) * S_max;
      merge_split_row<uint16_t, true>(part_o + row0 * D, part_ml + row0 * 2, ns, D,
                                      out + ((int64_t)i * Hq + g * G + t) * D, lane);
    }
    if (lane == 0) __hip_atomic_store(counters + (int64_t)i * Hkv + g, 0, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
  }
  }
}

}  // namespace pa_detail
