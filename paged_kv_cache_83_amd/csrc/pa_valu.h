// Streaming paged decode on the vector ALUs (gfx950, wave64): fp32 or bf16
// pools with 16-slot blocks, head dim 64 or 128, 1, 2 or 4 query heads per KV
// head (and 8 at head dim 128). It is the decode path for pools and shapes the matrix-core kernel
// does not take (fp32 pools above all), and the vector-ALU alternative that
// shows what the matrix cores buy on the grouped shapes.
//
// "KV Cache Management", section "The PagedAttention virtual memory model":
// the kernel takes the block table as an input, loads the physical block ids
// on chip and walks the logical blocks; section "Chunked prefill mechanics":
// the running maximum m and normaliser l, with the accumulator rescaled by
// exp(m_prev - m_new) as each tile of keys arrives.
//
// One wave = one work item (sequence i, KV head g, split s), no barrier other
// than the wave's own LDS ordering. Per iteration it takes KPI keys (BPI = KPI
// / 16 blocks, 8 KB of K and 8 KB of V) in 8 K and 8 V loads per lane, each
// load instruction reading 1 KB of one tile contiguously (lane l: bytes 16 l
// .. 16 l + 15 of that KB), so that a wave's load touches 8 cache lines and
// not 64:
//   scores:  a K tile is rows of (32-dim chunk, slot), 32*b bytes each, PPR
//            16-byte pieces: lane l holds piece l % PPR of KPL keys' rows
//            (every chunk of them) and dots it with the matching pieces of
//            the group's queries, read from LDS; fp32 pools use FMAs, bf16
//            pools v_dot2_f32_bf16 (two products per instruction, fp32
//            accumulation). The PPR lanes of a row group then sum their
//            pieces (DPP lane swaps), and each key's score is taken by one
//            lane of the group (its owner) and its duplicates.
//   softmax: per query head a wave maximum, exp2 of the scaled scores, a
//            rescale of the accumulators only when the head's maximum moved.
//            Probabilities go to LDS (fp32, or bf16 for the bf16 dot).
//   P.V:     a V tile is dimension-major, each dim's 16 slots 16*b contiguous
//            bytes (PPD pieces): lane l holds slots of piece l % PPD of DT
//            dims per block and accumulates their products with those slots'
//            probabilities (LDS). After the last iteration the PPD lanes of a
//            dim sum their accumulators and each lane keeps D/64 dims.
// The K registers of iteration it+1 are loaded as soon as the scores of it are
// formed and the V registers of it+1 as soon as its P.V is done, so one
// iteration of loads is always in flight; the last iteration is peeled so the
// steady loop issues unconditionally (a conditional issue makes the compiler
// wait for every outstanding load).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "pa_device.h"

namespace pa_detail {

template <typename T, int D>
struct ValuCfg {
  static constexpr int ES = (int)sizeof(T);
  // keys per iteration: 8 KB of K rows (and of V), which keeps a wave's K and V
  // registers at 64 VGPRs whatever the element size
  static constexpr int KPI = 8192 / (D * ES);
  static constexpr int BPI = KPI / 16;            // blocks per iteration
  static constexpr int EPL = 16 / ES;             // elements per 16-byte load
  static constexpr int NL = 8;                    // K (and V) loads per lane and iteration
  static constexpr int LPT = 16 * D * ES / 1024;  // loads per (block, head) tile
  // K tile rows (chunk of 32 dims, slot): PPR pieces of 16 bytes; RPL rows per
  // load; SPL loads per chunk (slot ranges of RPL); KPL keys per lane
  static constexpr int PPR = 2 * ES;
  static constexpr int RPL = 64 / PPR;
  static constexpr int SPL = 16 / RPL;
  static constexpr int KPL = KPI * PPR / 64;
  // V tile rows (dim: 16 slots): PPD pieces of EPL slots; DPW dims per load;
  // DT dims per lane and block; DPL dims per lane in the output
  static constexpr int PPD = ES;
  static constexpr int DPW = 64 / PPD;
  static constexpr int DT = LPT;
  static constexpr int DPL = D / 64;
  static_assert(D % 64 == 0 && BPI >= 1 && BPI * LPT == NL && KPL <= PPR && DT == DPL * PPD,
                "head dim 64 or 128");
};

// v + the value of another lane of its group of N consecutive lanes, repeated
// until every lane of the group holds the group's sum (N = 1, 2, 4 or 8): DPP
// lane swaps (lane ^ 1, lane ^ 2, then the other quad of eight lanes). Each
// lane adds the same operands, so the group's lanes hold identical bits.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8, "group of 1, 2, 4 or 8 lanes");
  if constexpr (N >= 2) v += dpp_mov<0xB1>(v);    // quad_perm [1,0,3,2]
  if constexpr (N >= 4) v += dpp_mov<0x4E>(v);    // quad_perm [2,3,0,1]
  if constexpr (N >= 8) v += dpp_mov<0x141>(v);   // row_half_mirror
  return v;
}

template <bool NT>
__device__ __forceinline__ u32x4 ld16(const void* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  else return *reinterpret_cast<const u32x4*>(p);
}

typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));

// a.b over the element pairs of one 32-bit word each (bf16) plus c, in fp32.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, a),
                                         __builtin_bit_cast(bf16x2_v, b), c, false);
}

// acc += sum over the 16 bytes of k . q (4 fp32 products or 8 bf16 products).
template <typename T>
__device__ __forceinline__ float dot16(const u32x4& k, const u32x4& q, float acc) {
  if constexpr (sizeof(T) == 4) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = fmaf(__uint_as_float(k[e]), __uint_as_float(q[e]), acc);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = dot2_bf16(k[e], q[e], acc);
  }
  return acc;
}

// Workgroup shape of the kernel: up to WMAX waves. 16 where one query head per
// KV head and 256-byte K rows (fp32 d = 64, bf16 d = 128) keep the kernel
// within the 128 registers a full CU of waves leaves each; 8 otherwise.
template <typename T, int D, int G>
struct ValuWg {
  static constexpr int WMAX = (G == 1 && D * (int)sizeof(T) == 256) ? 16 : 8;
};

// LDS words of a workgroup of W waves: the group's queries, then per wave its
// probabilities and its (o, m, l) for the merge across waves.
template <typename T, int D, int G>
struct ValuLds {
  static constexpr int ES = (int)sizeof(T);
  static constexpr int QS = G * D * ES / 4;
  static constexpr int PS = G * ValuCfg<T, D>::KPI * (ES == 2 ? 1 : 2) / 2 + 4;
  static constexpr int MG = G * (D + 2);
  static constexpr int PER_WAVE = (PS + MG + 3) / 4 * 4;   // 16-byte aligned regions
};

// Work item = workgroup (sequence i, KV head g, split s) of W waves: wave wv
// takes blocks [s*bps + wv*bpw, +bpw) of the sequence (bps = W*bpw); the waves'
// results are merged through LDS. A split that covers the whole sequence
// writes the output; otherwise it writes its merged partial (o, m, l) to the
// workspace, merged by the combine launch or, with counters (in-kernel merge),
// by the last split of (i, g) to finish.
// APPEND (runtime flag): the step's new token of sequence i (position len-1)
// comes in knew/vnew [n][H_kv][d]; the wave holding that position writes it
// into the pool and reads it from the inputs (K row by address, V element by
// register) while attending.
template <typename T, int D, int G, bool NT>
__global__ __launch_bounds__((64 * ValuWg<T, D, G>::WMAX)) void decode_valu_kernel(
    T* __restrict__ kpool, T* __restrict__ vpool, const T* __restrict__ q,
    const T* __restrict__ knew, const T* __restrict__ vnew, T* __restrict__ out,
    float* __restrict__ part_o, float* __restrict__ part_ml, const int32_t* __restrict__ tables,
    const int32_t* __restrict__ lens, int64_t layer_off, int N, int Hkv, int Hq, int max_blocks,
    int max_ctx, int bpw, int S_max, float qk_scale, int direct, int append,
    int* __restrict__ counters) {
  using C = ValuCfg<T, D>;
  using LW = ValuLds<T, D, G>;
  constexpr int ES = C::ES, KPI = C::KPI, BPI = C::BPI, EPL = C::EPL, NL = C::NL, LPT = C::LPT;
  constexpr int PPR = C::PPR, RPL = C::RPL, SPL = C::SPL, KPL = C::KPL;
  constexpr int PPD = C::PPD, DPW = C::DPW, DT = C::DT, DPL = C::DPL;
  constexpr int TILE = 16 * D;                       // elements of one (block, head) tile
  constexpr bool BF = sizeof(T) == 2;
  extern __shared__ __attribute__((aligned(16))) uint32_t lds_valu[];
  const int W = blockDim.x >> 6;
  const int wv = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  // queries (as stored: fp32 words or bf16 pairs), then per wave: probabilities
  // of one iteration, and (o, m, l) of each head for the merge across waves
  uint32_t* qs = lds_valu;
  uint32_t* ps = lds_valu + LW::QS + wv * LW::PER_WAVE;
  float* mg_base = reinterpret_cast<float*>(lds_valu + LW::QS + LW::PS);   // + wave * PER_WAVE

  const int w = blockIdx.x;
  const int g = w % Hkv;
  const int si = w / Hkv;
  const int s = si % S_max;
  const int i = si / S_max;
  // K: piece of a chunk row and row within a load; the lane's own key (slot
  // pc % KPL of its KPL keys; the lanes with pc < KPL own distinct keys)
  const int pc = lane % PPR, rg = lane / PPR;
  const int q_own = pc % KPL;
  const int k_own = 16 * (q_own / SPL) + RPL * (q_own % SPL) + rg;
  const bool owner = pc < KPL;
  // V: slot piece and dim within a load; the lane's output dims
  const int sg = lane % PPD, dg = lane / PPD;
  auto dim_of = [&](int r) { return (sg * DPL + r) * DPW + dg; };

  const int bps = W * bpw;         // blocks of one split (workgroup)
  const int B0 = s * bps;

  // The wave's block ids (at most 64), one per lane, read once, and the group's
  // G query rows (contiguous in q), loaded into registers and put in LDS once
  // the first K/V loads are on their way: both requested before the sequence's
  // length is known (ids past its blocks are read but never used).
  const int32_t* trow = tables + (int64_t)i * max_blocks;
  const int tb_idx = B0 + wv * bpw + lane;
  const int tb = (lane < bpw && tb_idx < max_blocks) ? guard_block(trow[tb_idx], N) : 0;
  constexpr int QPIECES = G * D * ES / 16;
  constexpr int QPT = (QPIECES + 63) / 64;   // pieces per thread of a one-wave workgroup
  u32x4 qreg[QPT];
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(q + ((int64_t)i * Hq + (int64_t)g * G) * D);
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const int e = threadIdx.x + j * (int)blockDim.x;
      qreg[j] = e < QPIECES ? src[e] : u32x4{0u, 0u, 0u, 0u};
    }
  }

  const int len = clamp_len(lens, i, max_ctx);
  const int nblk = (len + 15) >> 4;
  if (B0 >= nblk) {   // the whole workgroup (uniform)
    // an empty sequence writes zeros (without a combine launch, by its split 0)
    if ((direct || counters) && len == 0 && s == 0) {
      T* o = out + ((int64_t)i * Hq + (int64_t)g * G) * D;
      for (int e = threadIdx.x; e < G * D; e += blockDim.x) o[e] = from_f32<T>(0.f);
    }
    return;
  }
  const int n_act = min(W, (nblk - B0 + bpw - 1) / bpw);   // waves with blocks
  const bool active = wv < n_act;
  const int b0 = B0 + wv * bpw;
  const int b1 = min(b0 + bpw, nblk);
  const int span = active ? b1 - b0 : 1;
  const int lim = min(len, b1 * 16);  // keys at or past lim belong to a later wave / split or past the length

  const T* kl = kpool + layer_off + (int64_t)g * TILE;   // + block * Hkv * TILE
  const T* vl = vpool + layer_off + (int64_t)g * TILE;
  const int64_t bstride = (int64_t)Hkv * TILE;

  // The appended token (position len-1), if this wave's blocks hold it.
  int new_pos = -1;
  const T* knew_row = knew;
  const T* vnew_row = vnew;
  if (append && active && len > 0 && ((len - 1) >> 4) >= b0 && ((len - 1) >> 4) < b1) {
    new_pos = len - 1;
    knew_row = knew + ((int64_t)i * Hkv + g) * D;
    vnew_row = vnew + ((int64_t)i * Hkv + g) * D;
    const int64_t tile = (int64_t)__builtin_amdgcn_readlane(tb, (new_pos >> 4) - b0) * bstride;
    const int on = new_pos & 15;
    T* kt = kpool + layer_off + (int64_t)g * TILE + tile;
    T* vt = vpool + layer_off + (int64_t)g * TILE + tile;
    for (int e = lane; e < D; e += 64) {
      kt[(e >> 5) * 512 + on * 32 + (e & 31)] = knew_row[e];
      vt[e * 16 + on] = vnew_row[e];
    }
  }

  float acc[G][DT];    // the lane's DT dims, over its slot pieces
  float o_own[G][DPL]; // the lane's output dims, summed over the slot pieces
  float m_run[G], l_part[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_part[h] = 0.f;
#pragma unroll
    for (int t = 0; t < DT; ++t) acc[h][t] = 0.f;
#pragma unroll
    for (int r = 0; r < DPL; ++r) o_own[h][r] = 0.f;
  }

  // The queries to LDS. One wave: its own writes, ordered for its reads below
  // by LDS order (no workgroup barrier, which would also wait for the K/V loads
  // just issued); several waves: every thread writes its pieces, then a
  // barrier that waits for LDS only.
  auto store_queries = [&]() {
    u32x4* dst = reinterpret_cast<u32x4*>(qs);
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const int e = threadIdx.x + j * (int)blockDim.x;
      if (e < QPIECES) dst[e] = qreg[j];
    }
    if (W == 1) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    } else {
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
  };
  if (!active) store_queries();   // the barrier is reached by every wave

  if (active) {
    // Block id of the wave's block b (wave-uniform b, clamped into its range:
    // blocks past it are read but fully masked).
    auto blk_id = [&](int b) { return __builtin_amdgcn_readlane(tb, min(b, span - 1)); };
    // A wave-uniform value held in a vector register, so that compares against
    // it are vector compares (no scalar condition registers held across the
    // unrolled selects below).
    auto in_vgpr = [](int x) {
      int v;
      asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "s"(x));
      return v;
    };

    // Load j of an iteration reads KB j % LPT of the tile of block j / LPT.
    // K: it holds rows RPL*(j % LPT) .. of that tile: chunk (j % LPT) / SPL,
    // slots RPL*((j % LPT) % SPL) + rg; the lane's key slot of it is
    // (j / LPT)*SPL + (j % LPT) % SPL.
    u32x4 kr[NL];
    u32x4 vr[NL];
    auto issue_k = [&](int it) {
      // the appended token's key within the iteration (any value if not in it)
      const int kk = new_pos - (b0 + it * BPI) * 16;
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const int jj = j % LPT;
        const int key0 = 16 * (j / LPT) + RPL * (jj % SPL);   // key of row group 0
        const T* pool = kl + (int64_t)blk_id(it * BPI + j / LPT) * bstride + jj * (1024 / ES) + lane * EPL;
        // the new token's lanes read the input row (the pool's copy is being written)
        const T* fresh = knew_row + 32 * (jj / SPL) + pc * EPL;
        kr[j] = ld16<NT>(new_pos >= 0 && rg == kk - key0 ? fresh : pool);
      }
    };
    auto issue_v = [&](int it) {
#pragma unroll
      for (int j = 0; j < NL; ++j)
        vr[j] = ld16<NT>(vl + (int64_t)blk_id(it * BPI + j / LPT) * bstride + (j % LPT) * (1024 / ES) +
                         lane * EPL);
    };

    auto scores_softmax = [&](int it) {
      const int pos0 = (b0 + it * BPI) * 16;
      float sc[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float a[KPL];
#pragma unroll
        for (int q = 0; q < KPL; ++q) a[q] = 0.f;
#pragma unroll
        for (int c = 0; c < D / 32; ++c) {
          const u32x4 qv = *reinterpret_cast<const u32x4*>(qs + (h * D + 32 * c + pc * EPL) * ES / 4);
#pragma unroll
          for (int b = 0; b < BPI; ++b)
#pragma unroll
            for (int u = 0; u < SPL; ++u) {
              const int j = b * LPT + c * SPL + u;
              a[b * SPL + u] = dot16<T>(kr[j], qv, a[b * SPL + u]);
            }
        }
        float own = 0.f;
#pragma unroll
        for (int q = 0; q < KPL; ++q) {
          const float v = group_sum<PPR>(a[q]);
          own = q == 0 || q_own == q ? v : own;
        }
        sc[h] = (pos0 + k_own < lim) ? own * qk_scale : -INFINITY;
        // with 8 heads the scheduler would otherwise read every head's queries
        // ahead (more registers than a wave has)
        if constexpr (G >= 8) __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float m_new = fmaxf(m_run[h], wave_max(sc[h]));  // finite: the first key is attended
        const float p = __builtin_amdgcn_exp2f(sc[h] - m_new);
        if (m_new != m_run[h]) {   // wave-uniform
          const float alpha = __builtin_amdgcn_exp2f(m_run[h] - m_new);
          l_part[h] *= alpha;
#pragma unroll
          for (int t = 0; t < DT; ++t) acc[h][t] *= alpha;
        }
        m_run[h] = m_new;
        if (owner) {
          l_part[h] += p;
          if constexpr (BF) reinterpret_cast<uint16_t*>(ps)[h * KPI + k_own] = f32_to_bf16(p);
          else reinterpret_cast<float*>(ps)[h * KPI + k_own] = p;
        }
      }
    };

    // Only the last iteration of a wave's range can hold masked keys (blocks
    // past the range, slots past the length) or the appended token: both lie
    // in the sequence's last block, the last block of the last range. Its V
    // registers are fixed up here, outside the steady loop, so the loop's V
    // registers carry no conditional updates (which would make the compiler
    // copy them, and wait for every load in flight to do so).
    // V load j: dim (j % LPT)*DPW + dg of block j / LPT, its slots sg*EPL ..
    // sg*EPL + EPL-1; word c holds slots from sg*EPL + c*EPL/4.
    auto fix_last_v = [&](int it) {
      const int pos0 = (b0 + it * BPI) * 16;
      if (new_pos >= pos0 && new_pos < pos0 + KPI) {   // wave-uniform: the appended token's V
        const int kk = in_vgpr(new_pos - pos0);
        const uint32_t keep = BF ? ((kk & 1) ? 0x0000ffffu : 0xffff0000u) : 0u;
#pragma unroll
        for (int j = 0; j < NL; ++j) {
          const int e = (j % LPT) * DPW + dg;
          const uint32_t nv = BF ? (uint32_t)reinterpret_cast<const uint16_t*>(vnew_row)[e]
                                 : reinterpret_cast<const uint32_t*>(vnew_row)[e];
          const uint32_t nw = BF ? ((kk & 1) ? (nv << 16) : nv) : nv;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int key0 = 16 * (j / LPT) + sg * EPL + c * (EPL / 4);
            const uint32_t wd = vr[j][c];
            const bool hit = BF ? ((kk >> 1) == (key0 >> 1)) : (kk == key0);
            vr[j][c] = hit ? ((wd & keep) | nw) : wd;
          }
        }
      }
      if (pos0 + KPI > lim) {   // wave-uniform: zero the V of masked keys (their data may be NaN)
        const int nval = in_vgpr(lim - pos0);   // keys 0 .. nval-1 of the iteration are attended
#pragma unroll
        for (int j = 0; j < NL; ++j)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int key0 = 16 * (j / LPT) + sg * EPL + c * (EPL / 4);
            const uint32_t wd = vr[j][c];
            if constexpr (BF)
              vr[j][c] = key0 + 1 < nval ? wd : (key0 < nval ? (wd & 0x0000ffffu) : 0u);
            else
              vr[j][c] = key0 < nval ? wd : 0u;
          }
      }
    };

    auto pv = [&]() {
      // The probabilities were written by the score phase of this same wave, in
      // its own LDS region: LDS executes one wave's instructions in order, so
      // only the compiler must keep the reads below the writes (a workgroup
      // barrier would also wait for the next iteration's loads in flight).
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int b = 0; b < BPI; ++b) {
          const u32x4 pv4 = *reinterpret_cast<const u32x4*>(ps + (h * KPI + b * 16 + sg * EPL) * ES / 4);
#pragma unroll
          for (int t = 0; t < DT; ++t) acc[h][t] = dot16<T>(vr[b * LPT + t], pv4, acc[h][t]);
        }
        if constexpr (G >= 8) __builtin_amdgcn_sched_barrier(0);   // as in the score phase
      }
    };

    const int n_it = (span + BPI - 1) / BPI;
    issue_k(0);
    issue_v(0);
    store_queries();
    for (int it = 0; it + 1 < n_it; ++it) {
      scores_softmax(it);
      __builtin_amdgcn_sched_barrier(0);   // the K registers are free only after the scores
      issue_k(it + 1);
      pv();
      __builtin_amdgcn_sched_barrier(0);   // likewise the V registers after P.V
      issue_v(it + 1);
    }
    scores_softmax(n_it - 1);
    fix_last_v(n_it - 1);
    pv();

    // l: the sum over the wave of each lane's own keys; o: each dim summed over
    // its PPD slot pieces, the lane keeping dims dim_of(r)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      l_part[h] = wave_sum(l_part[h]);
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const float v = group_sum<PPD>(acc[h][t]);
#pragma unroll
        for (int r = 0; r < DPL; ++r)
          if (t % DPL == r) o_own[h][r] = t / DPL == 0 || sg == t / DPL ? v : o_own[h][r];
      }
    }
  }

  const int ns = (nblk + bps - 1) / bps;   // splits (workgroups) of this sequence
  const bool whole = direct || ns == 1;    // this split covers the sequence
  const bool coherent = counters != nullptr;
  // The workgroup's result for head h -- maximum M, sum L, unnormalised o of
  // the lane's dims -- goes out as the output or as the split's partial.
  auto finish = [&](int h, float M, float L, const float (&o)[DPL]) {
    if (whole) {   // the output, normalised
      const float inv = 1.f / L;
      T* op = out + ((int64_t)i * Hq + (int64_t)g * G + h) * D;
#pragma unroll
      for (int r = 0; r < DPL; ++r) op[dim_of(r)] = from_f32<T>(o[r] * inv);
    } else {   // the split's partial
      const int64_t row = ((int64_t)i * Hq + (int64_t)g * G + h) * S_max + s;
      if (coherent) {
#pragma unroll
        for (int r = 0; r < DPL; ++r) part_st_coherent(part_o + row * D + dim_of(r), o[r]);
        if (lane == 0) {
          part_st_coherent(part_ml + row * 2 + 0, M);
          part_st_coherent(part_ml + row * 2 + 1, L);
        }
      } else {
#pragma unroll
        for (int r = 0; r < DPL; ++r) part_o[row * D + dim_of(r)] = o[r];
        if (lane == 0) {
          part_ml[row * 2 + 0] = M;
          part_ml[row * 2 + 1] = L;
        }
      }
    }
  };

  if (W == 1) {   // one wave: its registers are the workgroup's result
#pragma unroll
    for (int h = 0; h < G; ++h) finish(h, m_run[h], l_part[h], o_own[h]);
  } else {
    if (active) {   // the wave's (o, m, l) to LDS
      float* mg = mg_base + (int64_t)wv * LW::PER_WAVE;
#pragma unroll
      for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int r = 0; r < DPL; ++r) mg[h * (D + 2) + dim_of(r)] = o_own[h][r];
        if (lane == 0) {
          mg[h * (D + 2) + D] = m_run[h];
          mg[h * (D + 2) + D + 1] = l_part[h];
        }
      }
    }
    __syncthreads();   // every active wave's (o, m, l) is in LDS
    // Merge across the workgroup's waves, same rule as across splits; wave wv
    // takes heads wv, wv + W, ...
#pragma unroll 1
    for (int h = wv; h < G; h += W) {
      float M = -INFINITY;
      for (int x = 0; x < n_act; ++x) M = fmaxf(M, mg_base[x * LW::PER_WAVE + h * (D + 2) + D]);
      float L = 0.f;
      float o[DPL];
#pragma unroll
      for (int r = 0; r < DPL; ++r) o[r] = 0.f;
      for (int x = 0; x < n_act; ++x) {
        const float* mgx = mg_base + x * LW::PER_WAVE + h * (D + 2);
        const float wt = exp2f(mgx[D] - M);
        L = fmaf(wt, mgx[D + 1], L);
#pragma unroll
        for (int r = 0; r < DPL; ++r) o[r] = fmaf(wt, mgx[dim_of(r)], o[r]);
      }
      finish(h, M, L, o);
    }
  }
  if (!coherent || whole) return;
  // In-kernel merge across splits: every wave's partial stores complete, then
  // wave 0 counts the split; the last split of (i, g) merges all of them.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (wv == 0 && split_arrive_last(counters + (int64_t)i * Hkv + g, ns, lane)) {
#pragma unroll 1
    for (int h = 0; h < G; ++h) {
      const int64_t row0 = ((int64_t)i * Hq + (int64_t)g * G + h) * S_max;
      merge_split_row<T, true>(part_o + row0 * D, part_ml + row0 * 2, ns, D,
                               out + ((int64_t)i * Hq + (int64_t)g * G + h) * D, lane);
    }
    if (lane == 0) __hip_atomic_store(counters + (int64_t)i * Hkv + g, 0, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace pa_detail
