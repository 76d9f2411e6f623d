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

}  // namespace pa_detail
