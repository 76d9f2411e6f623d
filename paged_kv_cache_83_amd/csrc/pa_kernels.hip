// Device side of libpa for gfx950 (CDNA4, wave64): slot-mapped KV append,
// split-K paged decode (MFMA kernel for bf16 with 16-slot blocks, generic VALU
// kernel for every other supported shape), the cross-split combine, and the
// whole-block copy / gather / scatter kernels.
//
// Sources on the pages:
//   "KV Cache Management", section "The PagedAttention virtual memory model":
//     token t of a sequence lives in logical block l = t / B at offset t mod B;
//     the decode kernel takes the block table as an input, loads the physical
//     block ids on chip and walks the logical blocks 0..floor((S-1)/B).
//   Same page, section "Chunked prefill mechanics": the running maximum m and
//     normaliser l, with the accumulator rescaled by exp(m_prev - m_new) as each
//     tile of keys arrives; the same rule merges the split partials.
//   Same page, sections "Zero-copy deliberation via copy-on-write branching"
//     (copy a shared block into a fresh one) and "Asynchronous paged swapping"
//     (move frames of bytes_per_block between the pool and a staging buffer).
//
// Pool layout (the interface fixes it): K [L][N][H_kv][d/W][B][W] with W = 32 when
// 32 divides d (else W = d), V [L][N][H_kv][d][B]. Keeping V dimension-major inside
// a block means a 16-byte load of V gives 8 consecutive slots of one dimension,
// which is exactly the operand fragment the PV matrix-core instruction wants; K
// is slot-major within 32-dimension chunks, which is what QK^T wants, and the
// chunking lets each K load instruction cover whole 128-byte lines (rows of 64 B
// adjacent in memory) so non-temporal streaming keeps its full bandwidth.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <type_traits>
#include <vector>

#include "../../include/pa.h"
#include "pa_device.h"
#include "pa_host.h"
#include "pa_append.h"
#include "pa_move.h"
#include "pa_fp8.h"
#include "pa_pairs.h"
#include "pa_valu.h"

namespace {

using namespace pa_detail;

// =============================================================================
// Append: token j's K/V go to slot slot_mapping[j] of one layer.
// =============================================================================

// =============================================================================
// Decode, MFMA kernel: bf16 pool, B = 16, d in {64, 128, 256}, up to 16 query
// heads per KV head. One wave = one work item (sequence i, KV head g, split s)
// covering logical blocks [s*bps, min((s+1)*bps, nblk)), bps even and <= 256.
//
// Per pair of blocks (32 keys) it issues two 16x16x32 bf16 MFMA chains:
//   S^T[32 keys][16 q] = K[keys][d] . Q^T[d][q]     (d/32 steps, two row tiles)
//   O^T[d][16 q]      += V^T[d][keys] . P^T[keys][q] (d/16 row tiles)
// Lane l = (c = l%16, gq = l/16). MFMA operand layout on gfx950 (checked on
// the device): A[row = c][k = 8*gq + j], B[k = 8*gq + j][col = c],
// C[row = 4*gq + i][col = c]. Rows of the score tiles are assigned to keys so
// that lane l ends up holding the 8 scores of keys 8*gq .. 8*gq+7 (pair-local)
// for query c -- which is exactly the B-operand fragment of the PV product, so
// probabilities never leave registers. K rows and V^T rows are each fetched
// with 16-byte loads straight from the pool into operand registers; the next
// pair's loads are issued before the current pair is computed (two register
// buffers), so every wave keeps one pair of blocks in flight at all times.
// =============================================================================
#ifndef PA_FP8_STAGES
#define PA_FP8_STAGES 2  // pairs of blocks in flight per wave, FP8 kernel
#endif

// new_pos: position of the token appended in this launch, or -1. Its V is
// substituted into the lane's V^T fragments from vnew (dims 16*dt + c: low half
// of vnew[dt/2] for even dt, high half for odd dt).
template <int D>
__device__ __forceinline__ void compute_pair(PairFrags<D>& f, const bf16x8 (&qf)[MfmaCfg<D>::KC],
                                             f32x4 (&acc)[MfmaCfg<D>::DT], float& m_run,
                                             float& l_run, int blk, int len, int gq,
                                             float qk_scale, int new_pos,
                                             const uint32_t (&vnew)[MfmaCfg<D>::DT / 2],
                                             uint16_t* vt_new) {
  constexpr int KC = MfmaCfg<D>::KC;
  constexpr int DT = MfmaCfg<D>::DT;
  if (new_pos >= blk * 16 && new_pos < blk * 16 + 32) {  // wave-uniform
    const int e = new_pos - blk * 16 - 8 * gq;            // the lane holds pair-local keys 8*gq .. +8
    if (e >= 0 && e < 8) {
      const int word = e >> 1;
      const uint32_t keep = (e & 1) ? 0x0000ffffu : 0xffff0000u;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint32_t nv = (dt & 1) ? (vnew[dt >> 1] >> 16) : (vnew[dt >> 1] & 0xffffu);
        const uint32_t ins = (e & 1) ? (nv << 16) : nv;
#pragma unroll
        for (int wv = 0; wv < 4; ++wv)
          f.v[dt][wv] = (wv == word) ? ((f.v[dt][wv] & keep) | ins) : f.v[dt][wv];
      }
    }
    // The new token's V goes into the pool as its whole tile: the lanes holding
    // that block (every dimension, both halves of the slots) write their
    // fragments -- as loaded, with the new slot patched -- as 16-byte
    // non-temporal stores, where storing the one new element per dimension row
    // would touch 128 separate 32-byte pieces of the tile with 2-byte writes.
    if ((gq >> 1) == ((new_pos - blk * 16) >> 4)) {
      const int c = threadIdx.x & 15;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        __builtin_nontemporal_store(f.v[dt],
                                    reinterpret_cast<u32x4*>(vt_new + (16 * dt + c) * 16 + 8 * (gq & 1)));
    }
  }
  f32x4 sc[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    sc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
      sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, f.k[t][kc]),
                                                      qf[kc], sc[t], 0, 0, 0);
  }
  // Lane holds the scores of pair-local keys 8*gq + 4*t + e for query c.
  const int pos0 = blk * 16 + 8 * gq;
  float sv[8];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      sv[4 * t + e] = (pos0 + 4 * t + e < len) ? sc[t][e] * qk_scale : -INFINITY;
  }
  float mb = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                   fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
  mb = max_over_groups(mb);
  const float m_new = fmaxf(m_run, mb);  // finite: the pair's first key is attended
  float psum = 0.f;
  uint32_t pw[4];
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const float pa = __builtin_amdgcn_exp2f(sv[e] - m_new);
    const float pb = __builtin_amdgcn_exp2f(sv[e + 1] - m_new);
    psum += pa + pb;
    pw[e >> 1] = pack_bf16x2(pa, pb);
  }
  // Rescale only when some query's running maximum moved (alpha == 1 otherwise).
  if (__any(m_new != m_run)) {
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = acc[dt] * alpha;
  }
  l_run += psum;
  m_run = m_new;
  const bf16x8 pf = __builtin_bit_cast(bf16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));

  // Slots at or past the length hold unspecified data (possibly NaN): their
  // probability is 0, and their V elements are zeroed so 0 * V stays 0.
  if (blk * 16 + 32 > len) {
    u32x4 keep;
#pragma unroll
    for (int wv = 0; wv < 4; ++wv) {
      const int p = pos0 + 2 * wv;
      keep[wv] = (p < len ? 0x0000ffffu : 0u) | (p + 1 < len ? 0xffff0000u : 0u);
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) f.v[dt] &= keep;
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, f.v[dt]), pf,
                                                      acc[dt], 0, 0, 0);
}

// APPEND: the step's new token of every sequence (position len-1) comes in
// knew/vnew [n][H_kv][d]; the work item holding that position writes it into the
// pool and uses it from registers (K by address, V by element) while attending.
// RAGGED: the work items come from a list in the arguments (ragged batches:
// only long sequences split, longest items first) instead of the uniform grid
// of every sequence's S_max splits. A ragged launch runs one wave per SIMD:
// its items (about two per SIMD) then go out in two waves of work, and the
// short items of the second refill the SIMDs as the long items of the first
// finish, instead of all starting at once and leaving SIMDs idle once the
// short ones end (chat-like batch: 77 us per launch against 81).
template <int D, int OUT, bool NT, bool APPEND, bool RAGGED>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu((D >= 256 || RAGGED) ? 1 : PA_MFMA_WPE))) void decode_mfma_bf16_kernel(
    uint16_t* __restrict__ kpool, uint16_t* __restrict__ vpool,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ knew,
    const uint16_t* __restrict__ vnew, uint16_t* __restrict__ out, float* __restrict__ part_o,
    float* __restrict__ part_ml, const int32_t* __restrict__ tables,
    const int32_t* __restrict__ lens, int64_t layer_off, int N, int Hkv, int Hq, int G,
    int max_blocks, int max_ctx, int bps, int S_max, float qk_scale, int* __restrict__ counters,
    std::conditional_t<RAGGED, RaggedItems, NoRaggedItems> items) {
  constexpr int KC = MfmaCfg<D>::KC;
  constexpr int DT = MfmaCfg<D>::DT;

  // Work-group order: KV head fastest, so the waves reading the H_kv tiles of
  // the same blocks (adjacent in the pool) start together.
  const int w = blockIdx.x;
  const int g = w % Hkv;
  const int si = w / Hkv;
  int s, i;
  if constexpr (RAGGED) {
    const uint32_t e = items.v[si];
    i = (int)(e & 0xffffu);
    s = (int)(e >> 16);
  } else {
    s = si % S_max;
    i = si / S_max;
  }
  const int lane = threadIdx.x;
  const int c = lane & 15;
  const int gq = lane >> 4;

  const int b0 = s * bps;
  const int h = g * G + c;
  const bool qvalid = c < G;

  // The split's block ids, one per lane and register, read once ("load the
  // physical block pointers on chip"); each pair takes its two ids by readlane.
  // They and the queries are requested before the sequence's length is known
  // (ids past its blocks are read but never used), so the three loads overlap.
  const int32_t* trow = tables + (int64_t)i * max_blocks;
  int tb[4];
  {
    const int lim = min(b0 + bps, max_blocks);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int idx = b0 + 64 * k + lane;
      tb[k] = (64 * k < bps && idx < lim) ? guard_block(trow[idx], N) : 0;
    }
  }

  // Q fragments (B operand of QK): Q[h][32*kc + 8*gq .. +8]; zero for padded columns.
  bf16x8 qf[KC];
  {
    const uint16_t* qrow = q + ((int64_t)i * Hq + (qvalid ? h : 0)) * D;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (qvalid) v = *reinterpret_cast<const uint4*>(qrow + 32 * kc + 8 * gq);
      qf[kc] = __builtin_bit_cast(bf16x8, v);
    }
  }

  const int len = clamp_len(lens, i, max_ctx);
  const int nblk = (len + 15) >> 4;
  if (b0 >= nblk) {
    // an empty sequence writes zeros (without a combine launch, by its split 0)
    if (OUT != kOutPartial && len == 0 && s == 0 && qvalid) {
      uint16_t* o = out + ((int64_t)i * Hq + h) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<uint2*>(o + 16 * dt + 4 * gq) = make_uint2(0u, 0u);
    }
    return;
  }
  const int b1 = min(b0 + bps, nblk);

  f32x4 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.f;

  const uint16_t* kl = kpool + layer_off;
  const uint16_t* vl = vpool + layer_off;

  // The appended token: the item whose split holds its block writes it into the
  // pool and, without waiting for those stores, uses it from the inputs (K row
  // by address, V by element) wherever the pair loads would return its slot.
  int new_pos = -1;
  const uint16_t* knew_row = knew;
  uint16_t* vt_new = nullptr;   // V tile of the appended token's block
  uint32_t vnw[DT / 2];
#pragma unroll
  for (int k = 0; k < DT / 2; ++k) vnw[k] = 0;
  if (APPEND && len > 0 && ((len - 1) >> 4) >= b0 && ((len - 1) >> 4) < b1) {
    new_pos = len - 1;
    knew_row = knew + ((int64_t)i * Hkv + g) * D;
    const uint16_t* vnew_row = vnew + ((int64_t)i * Hkv + g) * D;
    const int pn = table_at(tb, (new_pos >> 4) - b0);
    const int on = new_pos & 15;
    uint16_t* kt = kpool + layer_off + ((int64_t)pn * Hkv + g) * (16 * D);
    if (lane < D / 8) {  // K row: lane moves dims 8*lane .. +8 (a 32-dim chunk takes 4 lanes)
      const u32x4 kv8 = *reinterpret_cast<const u32x4*>(knew_row + 8 * lane);
      *reinterpret_cast<u32x4*>(kt + (lane >> 2) * 512 + on * 32 + 8 * (lane & 3)) = kv8;
    }
    // the V tile is written whole by the pair that holds the token (compute_pair)
    vt_new = vpool + layer_off + ((int64_t)pn * Hkv + g) * (16 * D);
#pragma unroll
    for (int k = 0; k < DT / 2; ++k)
      vnw[k] = (uint32_t)vnew_row[32 * k + c] | ((uint32_t)vnew_row[32 * k + 16 + c] << 16);
  }

  // Row r = c of each score tile holds pair-local key 8*(c>>2) + 4*t + (c&3):
  // block (c >> 3) of the pair, offset 8*((c>>2)&1) + 4*t + (c&3).
  const int k_sel = c >> 3;
  const int k_off0 = 8 * ((c >> 2) & 1) + (c & 3);
  // V^T fragment of lane: block (gq >> 1), dims 16*dt + c, slots 8*(gq&1) .. +8.
  const int v_sel = gq >> 1;
  const int v_off = 16 * c + 8 * (gq & 1);

  const int span = b1 - b0;
  const int npairs = (span + 1) >> 1;
  auto blk_of = [&](int pj) { return b0 + 2 * pj; };   // first block of pair pj
  auto ids = [&](int pj, int& p0, int& p1) {
    const int off = 2 * pj;
    p0 = table_at(tb, off);
    p1 = (off + 1 < span) ? table_at(tb, off + 1) : p0;
  };

  // NS pairs in flight: the loads of pair pj + NS - 1 are issued just before
  // pair pj is computed, into the buffer pair pj - 1 has released. The steady
  // loop issues unconditionally, so the wait before each compute covers only
  // the older pair (a conditional issue would make the compiler wait for all
  // outstanding loads, draining the pipeline every iteration); the last pairs
  // are drained by an unrolled tail.
  constexpr int NS = MfmaCfg<D>::kStages;
  PairFrags<D> f[NS];
  auto issue_at = [&](PairFrags<D>& fr, int pj) {
    int p0, p1;
    ids(pj, p0, p1);
    issue_pair<D, NT>(fr, kl, vl, p0, p1, Hkv, g, k_sel, k_off0, v_sel, v_off, gq,
                      new_pos >= 0 ? new_pos - 16 * blk_of(pj) : -1, knew_row);
  };
  int pj = 0;
  if (npairs >= 2 * NS - 1) {
#pragma unroll
    for (int st = 0; st < NS - 1; ++st) issue_at(f[st], st);
    for (; pj + 2 * NS - 1 <= npairs; pj += NS) {
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        issue_at(f[(st + NS - 1) % NS], pj + st + NS - 1);
        compute_pair<D>(f[st], qf, acc, m_run, l_run, blk_of(pj + st), len, gq, qk_scale,
                        new_pos, vnw, vt_new);
      }
    }
  } else {
#pragma unroll
    for (int st = 0; st < NS - 1; ++st)
      if (st < npairs) issue_at(f[st], st);
  }
  // npairs - pj pairs remain (at most 2*NS - 2); pairs pj .. pj+NS-2 are in flight.
#pragma unroll
  for (int k = 0; k < 2 * NS - 2; ++k) {
    if (pj + k >= npairs) break;
    if (pj + k + NS - 1 < npairs) issue_at(f[(k + NS - 1) % NS], pj + k + NS - 1);
    compute_pair<D>(f[k % NS], qf, acc, m_run, l_run, blk_of(pj + k), len, gq, qk_scale, new_pos,
                    vnw, vt_new);
  }

  l_run = sum_over_groups(l_run);
  // acc[dt][e] = O^T[d = 16*dt + 4*gq + e][q = c]
  mfma_split_epilogue<D, OUT>(acc, m_run, l_run, lane, i, g, G, Hq, Hkv, s, S_max, (nblk + bps - 1) / bps,
                         out, part_o, part_ml, counters);
}

// =============================================================================
// Decode, generic kernel (fp32 or bf16; B <= 64, d <= 256, B*d <= 4096,
// G*d <= 4096). One wave per (sequence, KV head, split). Each block's K and V
// tiles are staged in LDS as fp32; scores, the online-softmax update and the
// PV accumulation run on the vector ALUs in fp32.
// =============================================================================
constexpr int kGenMaxAcc = 64;  // largest G*d / 64 the generic kernel accepts

// R = accumulators per lane, ceil(G*d / 64) rounded up to one of 1, 4, 16, 64.
template <typename T, bool DIRECT, int R, bool APPEND>
__global__ __launch_bounds__(64) void decode_generic_kernel(
    T* __restrict__ kpool, T* __restrict__ vpool, const T* __restrict__ q,
    const T* __restrict__ knew, const T* __restrict__ vnew,
    T* __restrict__ out, float* __restrict__ part_o, float* __restrict__ part_ml,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ lens, int64_t layer_off, int N,
    int Hkv, int Hq, int G, int D, int B, int max_blocks, int max_ctx, int bps, int S_max,
    float qk_scale) {
  extern __shared__ float smem[];
  float* Qs = smem;            // [G][D]
  float* Ks = Qs + G * D;      // [B][D]
  float* Vs = Ks + B * D;      // [D][B]
  float* Ps = Vs + B * D;      // [G][B]
  float* As = Ps + G * B;      // [G]

  const int w = blockIdx.x;
  const int s = w % S_max;
  const int gi = w / S_max;
  const int g = gi % Hkv;
  const int i = gi / Hkv;
  const int lane = threadIdx.x;
  const int GD = G * D;

  const int len = clamp_len(lens, i, max_ctx);
  const int nblk = (len + B - 1) / B;
  const int b0 = s * bps;
  if (b0 >= nblk) {
    if (DIRECT && len == 0) {
      T* o = out + ((int64_t)i * Hq + (int64_t)g * G) * D;
      for (int idx = lane; idx < GD; idx += 64) o[idx] = from_f32<T>(0.f);
    }
    return;
  }
  const int b1 = min(b0 + bps, nblk);

  const T* qg = q + ((int64_t)i * Hq + (int64_t)g * G) * D;  // the group's heads are contiguous
  for (int idx = lane; idx < GD; idx += 64) Qs[idx] = to_f32<T>(qg[idx]);

  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;  // lane q < G owns query q's statistics

  const int32_t* trow = tables + (int64_t)i * max_blocks;
  const int BD = B * D;
  const int W = k_chunk(D);
  // APPEND: the item holding position len-1 writes the step's new token there
  // and uses it from the inputs (the pool's copy may not be visible yet).
  const int new_pos = (APPEND && len > 0 && (len - 1) / B >= b0 && (len - 1) / B < b1) ? len - 1 : -1;
  for (int blk = b0; blk < b1; ++blk) {
    const int p = guard_block(trow[blk], N);
    T* kt = kpool + layer_off + ((int64_t)p * Hkv + g) * BD;
    T* vt = vpool + layer_off + ((int64_t)p * Hkv + g) * BD;
    const int valid = min(B, len - blk * B);
    __syncthreads();
    for (int idx = lane; idx < BD; idx += 64) {
      // memory order of K: [d/W][B][W] -> LDS order [B][d]
      const int jc = idx / (B * W), rem = idx - jc * (B * W);
      const int o = rem / W, jj = rem - o * W;
      Ks[o * D + jc * W + jj] = to_f32<T>(kt[idx]);
      Vs[idx] = to_f32<T>(vt[idx]);
    }
    if (APPEND && new_pos >= 0 && new_pos / B == blk) {
      const int o = new_pos % B;
      const T* kr = knew + ((int64_t)i * Hkv + g) * D;
      const T* vr = vnew + ((int64_t)i * Hkv + g) * D;
      __syncthreads();
      for (int j = lane; j < D; j += 64) {
        const T kv = kr[j], vv = vr[j];
        kt[(j / W) * B * W + o * W + (j % W)] = kv;
        vt[j * B + o] = vv;
        Ks[o * D + j] = to_f32<T>(kv);
        Vs[j * B + o] = to_f32<T>(vv);
      }
    }
    __syncthreads();
    for (int idx = lane; idx < G * B; idx += 64) {
      const int qi = idx / B, k = idx % B;
      float sc = -INFINITY;
      if (k < valid) {
        float dot = 0.f;
        for (int dd = 0; dd < D; ++dd) dot = fmaf(Qs[qi * D + dd], Ks[k * D + dd], dot);
        sc = dot * qk_scale;
      }
      Ps[idx] = sc;
    }
    __syncthreads();
    if (lane < G) {
      float mb = -INFINITY;
      for (int k = 0; k < valid; ++k) mb = fmaxf(mb, Ps[lane * B + k]);
      const float m_new = fmaxf(m_run, mb);
      const float alpha = exp2f(m_run - m_new);
      float ps = 0.f;
      for (int k = 0; k < B; ++k) {
        const float pk = (k < valid) ? exp2f(Ps[lane * B + k] - m_new) : 0.f;
        Ps[lane * B + k] = pk;
        ps += pk;
      }
      l_run = l_run * alpha + ps;
      m_run = m_new;
      As[lane] = alpha;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int idx = lane + 64 * r;
      if (idx < GD) {
        const int qi = idx / D, dd = idx % D;
        float a = acc[r] * As[qi];
        for (int k = 0; k < valid; ++k) a = fmaf(Ps[qi * B + k], Vs[dd * B + k], a);
        acc[r] = a;
      }
    }
  }
  __syncthreads();
  if (lane < G) {
    As[lane] = l_run;
    Ps[lane] = m_run;
  }
  __syncthreads();
  if (DIRECT) {
    T* o = out + ((int64_t)i * Hq + (int64_t)g * G) * D;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int idx = lane + 64 * r;
      if (idx < GD) o[idx] = from_f32<T>(acc[r] / As[idx / D]);
    }
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int idx = lane + 64 * r;
      if (idx < GD) {
        const int qi = idx / D, dd = idx % D;
        const int64_t row = ((int64_t)i * Hq + (int64_t)g * G + qi) * S_max + s;
        part_o[row * D + dd] = acc[r];
      }
    }
    if (lane < G) {
      const int64_t row = ((int64_t)i * Hq + (int64_t)g * G + lane) * S_max + s;
      part_ml[row * 2 + 0] = m_run;
      part_ml[row * 2 + 1] = l_run;
    }
  }
}

// =============================================================================
// Combine: merge the splits of one (sequence, query head) with the online-softmax
// rule: M = max_s m_s, w_s = 2^(m_s - M), out = sum_s w_s o_s / sum_s w_s l_s.
// (m is kept in log2 units: scores were scaled by log2(e).)
// =============================================================================
template <typename T>
__global__ __launch_bounds__(64) void decode_combine_kernel(const float* __restrict__ part_o,
                                                            const float* __restrict__ part_ml,
                                                            T* __restrict__ out,
                                                            const int32_t* __restrict__ lens,
                                                            int Hq, int D, int B, int S_max,
                                                            int bps, int max_ctx,
                                                            int single_written) {
  const int w = blockIdx.x;
  const int h = w % Hq;
  const int i = w / Hq;
  const int lane = threadIdx.x;
  const int len = clamp_len(lens, i, max_ctx);
  const int nblk = (len + B - 1) / B;
  const int ns = min(S_max, (nblk + bps - 1) / bps);
  T* o = out + ((int64_t)i * Hq + h) * D;
  if (ns == 0) {
    for (int d = lane; d < D; d += 64) o[d] = from_f32<T>(0.f);
    return;
  }
  if (ns == 1 && single_written) return;   // the decode launch wrote this row
  const int64_t row0 = ((int64_t)i * Hq + h) * S_max;
  merge_split_row<T>(part_o + row0 * D, part_ml + row0 * 2, ns, D, o, lane);
}

// =============================================================================
// Host-side helpers: argument checks, launch timing.
// =============================================================================
struct ProfRec {
  std::string name;
  hipEvent_t a, b;
};
struct ProfAcc {
  std::string name;
  int64_t launches = 0;
  double ms = 0.0;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_prof_pending;
std::vector<ProfAcc> g_prof_acc;


size_t generic_lds_bytes(int G, int D, int B) {
  return sizeof(float) * ((size_t)G * D + 2 * (size_t)B * D + (size_t)G * B + G + 64);
}

// Blocks per iteration of the streaming VALU kernel (its ValuCfg::BPI).
int valu_bpi(const pa_geom* g) {
  const int bytes = g->head_dim * (int)esize(g);
  return 4 / (bytes <= 128 ? 1 : bytes / 128);
}
// LDS bytes of a VALU workgroup of W waves (ValuLds) and its largest W.
size_t valu_lds_bytes(const pa_geom* g, int G, int W) {
  const int es = (int)esize(g), D = g->head_dim;
  const int bytes = D * es;
  const int kpi = 64 / (bytes <= 128 ? 1 : bytes / 128);
  const size_t qs = (size_t)G * D * es / 4;
  const size_t ps = (size_t)G * kpi * (es == 2 ? 1 : 2) / 2 + 4;
  const size_t mg = (size_t)G * (D + 2);
  return 4 * (qs + (size_t)W * ((ps + mg + 3) / 4 * 4));
}
int valu_wmax(const pa_geom* g, int G) {   // ValuWg::WMAX
  return (G == 1 && g->head_dim * esize(g) == 256) ? 16 : 8;
}

struct DecodePlan {
  int kernel;  // 1 generic, 2 mfma (bf16 pool), 3 mfma (fp8 pool), 4 streaming VALU
  bool stream_kv;  // non-temporal K/V loads
  int bps;         // blocks per split (work item; for the VALU kernel a workgroup)
  int bpw;         // VALU kernel: blocks per wave
  int wg_waves;    // VALU kernel: waves per workgroup
  int S_max;
  bool direct;
  bool merge;       // splits merged inside the decode launch (counters after the partials)
  size_t ws;
  size_t counters_off;
  bool ragged;      // MFMA bf16 kernel: work items from `items`
  RaggedItems items;
};

// Ragged plan for the MFMA bf16 kernel from the host copy of the lengths: a
// sequence longer than C blocks is cut into items of C blocks, the others stay
// whole, and items go out longest first, so the long sequences no longer set
// the launch's end while most waves sit idle. C spreads the batch's blocks over
// about two items per SIMD (the ragged kernel runs one wave per SIMD, so the
// second item of a SIMD starts when its first ends), or covers the longest
// sequence when that is at most three such items. Taken only when the lengths are uneven (longest above 1.5x
// the mean) and the list fits the kernel arguments.
bool plan_ragged(const int32_t* host_lens, int32_t n, int32_t max_ctx, int Hkv, int D,
                 int64_t want_bps, DecodePlan* plan) {
  if (n <= 0 || n > 65535) return false;
  std::vector<int32_t> nb(n);
  int64_t total = 0, longest = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t len = std::min(std::max(host_lens[i], 0), max_ctx);
    nb[i] = (len + 15) / 16;
    total += nb[i];
    longest = std::max<int64_t>(longest, nb[i]);
  }
  if (want_bps <= 0 && (total == 0 || 2 * longest * n <= 3 * total)) return false;
  const int64_t slots = D >= 256 ? 1024 : 2048;
  int64_t C = want_bps > 0 ? want_bps : std::max<int64_t>(16, (total * Hkv + slots - 1) / slots);
  // No split at all when the longest sequence is at most three balanced items:
  // its one item then still ends with the rest of the launch (longest first),
  // and the launch writes its outputs directly, with no partials and no combine
  // launch (chat-like batch: longest 64 blocks against items of 24; 2.59 ms per
  // step unsplit against 2.72 split).
  if (want_bps <= 0 && longest <= 3 * C && longest <= kMfmaMaxBps) C = longest;
  C += C & 1;
  C = std::min<int64_t>(C, kMfmaMaxBps);
  auto count = [&](int64_t c) {
    int64_t k = 0;
    for (int32_t i = 0; i < n; ++i) k += std::max<int64_t>(1, (nb[i] + c - 1) / c);
    return k;
  };
  while (count(C) > kMaxRaggedItems && C < kMfmaMaxBps) C = std::min<int64_t>(kMfmaMaxBps, 2 * C);
  if (count(C) > kMaxRaggedItems) return false;
  struct Item { int32_t size, seq, split; };
  std::vector<Item> list;
  int64_t S = 1;
  for (int32_t i = 0; i < n; ++i) {
    const int64_t c = std::max<int64_t>(1, (nb[i] + C - 1) / C);
    S = std::max(S, c);
    for (int64_t sp = 0; sp < c; ++sp)
      list.push_back({(int32_t)std::min<int64_t>(C, nb[i] - sp * C), i, (int32_t)sp});
  }
  if (S > 65535) return false;
  std::stable_sort(list.begin(), list.end(), [](const Item& a, const Item& b) { return a.size > b.size; });
  plan->ragged = true;
  plan->items.n = (int32_t)list.size();
  for (size_t k = 0; k < list.size(); ++k)
    plan->items.v[k] = (uint32_t)list[k].seq | ((uint32_t)list[k].split << 16);
  plan->bps = (int)C;
  plan->S_max = (int)S;
  return true;
}

pa_status make_plan(const pa_geom* g, int32_t n_seqs, int32_t Hq, int32_t max_ctx,
                    const pa_decode_opts* opts, DecodePlan* plan) {
  if (!geom_ok(g) || n_seqs < 0 || Hq <= 0 || max_ctx < 0) return PA_ERR_INVALID_ARG;
  if (Hq % g->num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  const int D = g->head_dim, B = g->block_size, G = Hq / g->num_kv_heads;
  const bool fp8 = g->dtype == PA_FP8;
  const bool mfma_ok = B == 16 && G <= 16 &&
                       (fp8 ? (D == 64 || D == 128) : (g->dtype == PA_BF16 && (D == 64 || D == 128 || D == 256)));
  const size_t gen_lds = generic_lds_bytes(G, D, B);
  const bool gen_ok = !fp8 && B <= 64 && D <= 256 && B * D <= 4096 && G * D <= 64 * kGenMaxAcc &&
                      G <= 64 && gen_lds <= 65536;
  const bool valu_ok = !fp8 && B == 16 && (D == 64 || D == 128) &&
                       (G == 1 || G == 2 || G == 4 || (G == 8 && D == 128));
  const int want = opts ? opts->kernel : 0;
  int k;
  if (want == 1) {
    if (!gen_ok) return PA_ERR_UNSUPPORTED;
    k = 1;
  } else if (want == 2) {
    if (!mfma_ok) return PA_ERR_UNSUPPORTED;
    k = fp8 ? 3 : 2;
  } else if (want == 3) {
    if (!valu_ok) return PA_ERR_UNSUPPORTED;
    k = 4;
  } else if (want == 0) {
    if (mfma_ok) k = fp8 ? 3 : 2;
    else if (valu_ok) k = 4;
    else if (gen_ok) k = 1;
    else return PA_ERR_UNSUPPORTED;
  } else {
    return PA_ERR_INVALID_ARG;
  }
  const int64_t maxb = ((int64_t)max_ctx + B - 1) / B;
  int64_t bps;
  if (opts && opts->blocks_per_split > 0) {
    bps = opts->blocks_per_split;
  } else {
    // Aim for about one work item per SIMD (256 CUs x 4): each item pays two
    // dependent load latencies at start (block ids, then its first blocks), so
    // fewer, longer items beat more, shorter ones once the chip is covered.
    // The generic kernel walks its blocks one at a time with a load latency per
    // block, so it wants many short items instead.
    // The streaming VALU kernel runs two waves per SIMD and takes four blocks
    // per iteration: about two items per SIMD, at least one iteration each.
    const int64_t units = (int64_t)n_seqs * g->num_kv_heads;
    const int64_t target_items = k == 4 ? 2048 : k >= 2 ? 1024 : 4096;
    const int64_t min_bps = k == 4 ? valu_bpi(g) : k >= 2 ? 16 : 2;
    if (units >= target_items || units == 0) {
      bps = maxb;
    } else {
      const int64_t want_splits = (target_items + units - 1) / units;
      bps = std::max<int64_t>(min_bps, (maxb + want_splits - 1) / want_splits);
    }
  }
  bps = std::max<int64_t>(2, bps);
  bps += bps & 1;  // pairs of blocks never straddle two splits
  int64_t bpw = 0, W = 1;
  if (k == 4) {
    // The VALU kernel: bps blocks per wave (whole iterations, at most 64: a
    // wave's block ids sit in one register); a workgroup of W waves covers as
    // much of the longest sequence as W allows, its waves merged in LDS. Two
    // waves by default: pairs of splits merge in LDS instead of through the
    // workspace (GPT-2 fp32 step 0.134 -> 0.129 ms; 3, 4, 8 or 16 waves slower).
    const int64_t bpi = valu_bpi(g);
    bpw = std::min<int64_t>(64, (bps + bpi - 1) / bpi * bpi);
    const int64_t want_w = opts && opts->waves_per_group > 0 ? opts->waves_per_group : 2;
    W = std::max<int64_t>(1, std::min<int64_t>({want_w, (int64_t)valu_wmax(g, G), (maxb + bpw - 1) / bpw}));
    while (W > 1 && valu_lds_bytes(g, G, (int)W) > 65536) --W;
    bps = bpw * W;
  } else if (k >= 2) {
    bps = std::min<int64_t>(bps, kMfmaMaxBps);
  }
  if (bps > INT32_MAX / 2) bps = INT32_MAX / 2;
  int64_t S = maxb == 0 ? 1 : (maxb + bps - 1) / bps;
  if (opts && (opts->kv_reuse < 0 || opts->kv_reuse > 1)) return PA_ERR_INVALID_ARG;
  if (opts && (opts->merge < 0 || opts->merge > 1 || opts->waves_per_group < 0)) return PA_ERR_INVALID_ARG;
  plan->kernel = k;
  plan->stream_kv = !(opts && opts->kv_reuse == 1);
  plan->bps = (int)bps;
  plan->bpw = (int)bpw;
  plan->wg_waves = (int)W;
  plan->S_max = (int)S;
  plan->ragged = false;
  plan->items.n = 0;
  if (k == 2 && opts && opts->host_context_lens)
    plan_ragged(opts->host_context_lens, n_seqs, max_ctx, g->num_kv_heads, D,
                opts->blocks_per_split, plan);
  S = plan->S_max;
  plan->direct = S == 1;
  plan->merge = !plan->direct && opts && opts->merge == 1 && k >= 2;   // not the generic kernel
  const size_t parts = plan->direct ? 0 : (size_t)n_seqs * Hq * S * (D + 2) * sizeof(float);
  plan->counters_off = parts;
  plan->ws = parts + (plan->merge ? ((size_t)n_seqs * g->num_kv_heads * sizeof(int32_t) + 15) / 16 * 16 : 0);
  return PA_OK;
}

}  // namespace

namespace pa_detail {
ProfScope::ProfScope(const char* n, hipStream_t s, bool allowed, bool bind_kernel)
    : name(n), st(s), on(false), bind(bind_kernel) {
  if (!allowed) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_on) return;
  // the start marker carries no data: no system-scope fence when it completes
  if (hipEventCreateWithFlags(&a, hipEventDisableSystemFence) != hipSuccess) return;
  if (hipEventCreate(&b) != hipSuccess) {
    (void)hipEventDestroy(a);
    return;
  }
  on = hipEventRecord(a, st) == hipSuccess;
  if (!on) {
    (void)hipEventDestroy(a);
    (void)hipEventDestroy(b);
  }
}
ProfScope::~ProfScope() {
  if (!on) return;
  if (bind && !bound) {  // the launch never took place (an argument error)
    (void)hipEventDestroy(a);
    (void)hipEventDestroy(b);
    return;
  }
  if (!bind) (void)hipEventRecord(b, st);
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_pending.push_back({name, a, b});
}
}  // namespace pa_detail

// =============================================================================
// C ABI
// =============================================================================
extern "C" {

pa_status pa_append_kv(const pa_geom* g, void* k_pool, void* v_pool, int32_t layer,
                       const void* k_new, const void* v_new, const int64_t* slot_mapping,
                       int32_t n_tokens, void* stream) {
  if (!geom_ok(g) || layer < 0 || layer >= g->num_layers || n_tokens < 0) return PA_ERR_INVALID_ARG;
  if (n_tokens == 0) return PA_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !slot_mapping) return PA_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  const int D = g->head_dim, B = g->block_size, H = g->num_kv_heads;
  const int64_t layer_off = (int64_t)layer * g->num_blocks * H * B * D;
  const int64_t nslots = (int64_t)g->num_blocks * B;
  if (g->dtype == PA_FP8) {
    ProfScope ps("append", st);
    if (!launch_append_fp8(st, (uint8_t*)k_pool, (uint8_t*)v_pool, (const uint16_t*)k_new,
                           (const uint16_t*)v_new, SlotsFromArray{slot_mapping}, (int64_t)n_tokens,
                           H, D, B, nslots, (int64_t)layer * g->num_blocks * H * tile_bytes(g)))
      return PA_ERR_UNSUPPORTED;
    return launch_status();
  }
  const size_t lds = g->dtype == PA_BF16 ? append_lds_bytes<uint16_t>(D) : append_lds_bytes<float>(D);
  if (lds > 65536) return PA_ERR_UNSUPPORTED;
  ProfScope ps("append", st, true, true);
  const int64_t items = ((int64_t)n_tokens + kAppendChunk - 1) / kAppendChunk * H;
  const int64_t wgs = (items + kXcds - 1) / kXcds * kXcds;  // a multiple of the XCD count
  if (wgs > INT32_MAX) return PA_ERR_UNSUPPORTED;
  const dim3 grid((unsigned)wgs);
  if (g->dtype == PA_BF16) {
    if (D % 8 == 0)
      PA_TIMED_LAUNCH(ps, (append_kv_kernel<uint16_t, 8, SlotsFromArray>), grid, dim3(256), lds, st,
                         (uint16_t*)k_pool, (uint16_t*)v_pool, (const uint16_t*)k_new,
                         (const uint16_t*)v_new, SlotsFromArray{slot_mapping}, n_tokens, H, D, B, nslots,
                         layer_off);
    else
      PA_TIMED_LAUNCH(ps, (append_kv_kernel<uint16_t, 1, SlotsFromArray>), grid, dim3(256), lds, st,
                         (uint16_t*)k_pool, (uint16_t*)v_pool, (const uint16_t*)k_new,
                         (const uint16_t*)v_new, SlotsFromArray{slot_mapping}, n_tokens, H, D, B, nslots,
                         layer_off);
  } else {
    if (D % 4 == 0)
      PA_TIMED_LAUNCH(ps, (append_kv_kernel<float, 4, SlotsFromArray>), grid, dim3(256), lds, st,
                         (float*)k_pool, (float*)v_pool, (const float*)k_new, (const float*)v_new,
                         SlotsFromArray{slot_mapping}, n_tokens, H, D, B, nslots, layer_off);
    else
      PA_TIMED_LAUNCH(ps, (append_kv_kernel<float, 1, SlotsFromArray>), grid, dim3(256), lds, st,
                         (float*)k_pool, (float*)v_pool, (const float*)k_new, (const float*)v_new,
                         SlotsFromArray{slot_mapping}, n_tokens, H, D, B, nslots, layer_off);
  }
  return launch_status();
}

size_t pa_decode_workspace_bytes(const pa_geom* g, int32_t n_seqs, int32_t n_q_heads,
                                 int32_t max_context_len, const pa_decode_opts* opts) {
  DecodePlan plan;
  if (make_plan(g, n_seqs, n_q_heads, max_context_len, opts, &plan) != PA_OK) return 0;
  return plan.ws;
}

}  // extern "C"

// pa_decode and pa_decode_append share this: knew/vnew are null for a plain decode.
static pa_status decode_impl(const pa_geom* g, void* k_pool, void* v_pool, int32_t layer,
                             const void* q, const void* knew, const void* vnew, void* out,
                             int32_t n_seqs, int32_t n_q_heads, const int32_t* block_tables,
                             int32_t max_blocks_per_seq, const int32_t* context_lens,
                             int32_t max_context_len, float scale, const pa_decode_opts* opts,
                             void* workspace, size_t workspace_bytes, void* stream,
                             bool timing = true) {
  DecodePlan plan;
  pa_status st0 = make_plan(g, n_seqs, n_q_heads, max_context_len, opts, &plan);
  if (st0 != PA_OK) return st0;
  if (layer < 0 || layer >= g->num_layers || max_blocks_per_seq < 0) return PA_ERR_INVALID_ARG;
  const int B = g->block_size, D = g->head_dim, Hkv = g->num_kv_heads;
  if ((int64_t)max_blocks_per_seq * B < max_context_len) return PA_ERR_INVALID_ARG;
  if (n_seqs == 0) return PA_OK;
  if (!k_pool || !v_pool || !q || !out || !block_tables || !context_lens) return PA_ERR_INVALID_ARG;
  const bool append = knew != nullptr;
  if (append != (vnew != nullptr)) return PA_ERR_INVALID_ARG;
  if (!plan.direct && (!workspace || workspace_bytes < plan.ws)) return PA_ERR_WORKSPACE;
  const int64_t items = (int64_t)(plan.ragged ? plan.items.n : (int64_t)n_seqs * plan.S_max) * Hkv;
  if (items > INT32_MAX) return PA_ERR_UNSUPPORTED;
  hipStream_t st = (hipStream_t)stream;
  if (!(scale > 0.f)) scale = 1.f / std::sqrt((float)D);
  const float qk_scale = scale * kLog2e;
  const int G = n_q_heads / Hkv;
  const int64_t layer_off = (int64_t)layer * g->num_blocks * Hkv * B * D;
  float* part_o = (float*)workspace;
  float* part_ml = plan.direct ? nullptr : part_o + (size_t)n_seqs * n_q_heads * plan.S_max * D;
  int* counters = plan.merge ? (int*)((char*)workspace + plan.counters_off) : nullptr;
  {
    ProfScope ps("decode_partial", st, timing, true);
    const dim3 grid((unsigned)items), block(64);
    // the matrix-core kernels take the output mode as a template argument
#define PA_OUT_MODE(LAUNCH, DD)                                    \
  do {                                                             \
    if (plan.direct) LAUNCH(DD, kOutDirect);                       \
    else if (plan.merge) LAUNCH(DD, kOutMerge);                    \
    else LAUNCH(DD, kOutPartial);                                  \
  } while (0)
    if (plan.kernel == 3) {
      const int64_t off8 = (int64_t)layer * g->num_blocks * Hkv * tile_bytes(g);
#define PA_FP8_LAUNCH_A(DD, DIR, NTV, APP)                                                         \
  PA_TIMED_LAUNCH(ps, (decode_mfma_fp8_kernel<DD, DIR, NTV, PA_FP8_STAGES, APP>), grid, block, 0,    \
                     st, (uint8_t*)k_pool, (uint8_t*)v_pool, (const uint16_t*)q,                    \
                     (const uint16_t*)knew, (const uint16_t*)vnew, (uint16_t*)out, part_o, part_ml, \
                     block_tables, context_lens, off8, g->num_blocks, Hkv, n_q_heads, G,           \
                     max_blocks_per_seq, max_context_len, plan.bps, plan.S_max, qk_scale, counters)
      // the step's tokens (decode_append) are quantized into the pool by the
      // items that hold them, inside the decode launch
#define PA_FP8_LAUNCH_X(DD, DIR, NTV)                            \
  do {                                                           \
    if (append) PA_FP8_LAUNCH_A(DD, DIR, NTV, true);             \
    else PA_FP8_LAUNCH_A(DD, DIR, NTV, false);                   \
  } while (0)
#define PA_FP8_LAUNCH(DD, DIR)                                   \
  do {                                                           \
    if (plan.stream_kv) PA_FP8_LAUNCH_X(DD, DIR, true);          \
    else PA_FP8_LAUNCH_X(DD, DIR, false);                        \
  } while (0)
      if (D == 64) PA_OUT_MODE(PA_FP8_LAUNCH, 64);
      else PA_OUT_MODE(PA_FP8_LAUNCH, 128);
#undef PA_FP8_LAUNCH
#undef PA_FP8_LAUNCH_X
#undef PA_FP8_LAUNCH_A
    } else if (plan.kernel == 2) {
#define PA_MFMA_LAUNCH_RG(DD, DIR, NTV, APP, RG, ITEMS)                                           \
  PA_TIMED_LAUNCH(ps, (decode_mfma_bf16_kernel<DD, DIR, NTV, APP, RG>), grid, block, 0, st,        \
                     (uint16_t*)k_pool, (uint16_t*)v_pool, (const uint16_t*)q,                     \
                     (const uint16_t*)knew, (const uint16_t*)vnew, (uint16_t*)out, part_o,         \
                     part_ml, block_tables, context_lens, layer_off, g->num_blocks, Hkv,          \
                     n_q_heads, G, max_blocks_per_seq, max_context_len, plan.bps, plan.S_max,      \
                     qk_scale, counters, ITEMS)
#define PA_MFMA_LAUNCH_X(DD, DIR, NTV, APP)                                                       \
  do {                                                                                           \
    if (plan.ragged) PA_MFMA_LAUNCH_RG(DD, DIR, NTV, APP, true, plan.items);                      \
    else PA_MFMA_LAUNCH_RG(DD, DIR, NTV, APP, false, NoRaggedItems{});                            \
  } while (0)
#define PA_MFMA_LAUNCH_NT(DD, DIR, NTV)                     \
  do {                                                      \
    if (append) PA_MFMA_LAUNCH_X(DD, DIR, NTV, true);       \
    else PA_MFMA_LAUNCH_X(DD, DIR, NTV, false);             \
  } while (0)
#define PA_MFMA_LAUNCH(DD, DIR)                                          \
  do {                                                                   \
    if (plan.stream_kv) PA_MFMA_LAUNCH_NT(DD, DIR, true);                \
    else PA_MFMA_LAUNCH_NT(DD, DIR, false);                              \
  } while (0)
      if (D == 64) PA_OUT_MODE(PA_MFMA_LAUNCH, 64);
      else if (D == 128) PA_OUT_MODE(PA_MFMA_LAUNCH, 128);
      else PA_OUT_MODE(PA_MFMA_LAUNCH, 256);
#undef PA_MFMA_LAUNCH
#undef PA_MFMA_LAUNCH_NT
#undef PA_MFMA_LAUNCH_X
#undef PA_MFMA_LAUNCH_RG
#undef PA_OUT_MODE
    } else if (plan.kernel == 4) {
#define PA_VALU_LAUNCH_X(T, DD, GG, NTV)                                                          \
  PA_TIMED_LAUNCH(ps, (decode_valu_kernel<T, DD, GG, NTV>), grid, dim3(64 * plan.wg_waves),         \
                     valu_lds_bytes(g, G, plan.wg_waves), st, (T*)k_pool,                          \
                     (T*)v_pool, (const T*)q, (const T*)knew, (const T*)vnew, (T*)out, part_o,     \
                     part_ml, block_tables, context_lens, layer_off, g->num_blocks, Hkv,          \
                     n_q_heads, max_blocks_per_seq, max_context_len, plan.bpw, plan.S_max,         \
                     qk_scale, plan.direct ? 1 : 0, append ? 1 : 0, counters)
#define PA_VALU_LAUNCH_G(T, DD, NTV)                  \
  do {                                                \
    if (G == 1) PA_VALU_LAUNCH_X(T, DD, 1, NTV);      \
    else if (G == 2) PA_VALU_LAUNCH_X(T, DD, 2, NTV); \
    else PA_VALU_LAUNCH_X(T, DD, 4, NTV);             \
  } while (0)
#define PA_VALU_LAUNCH(T, NTV)                                          \
  do {                                                                  \
    if (D == 64) PA_VALU_LAUNCH_G(T, 64, NTV);                          \
    else if (G == 8) PA_VALU_LAUNCH_X(T, 128, 8, NTV);                  \
    else PA_VALU_LAUNCH_G(T, 128, NTV);                                 \
  } while (0)
      if (g->dtype == PA_F32) {
        if (plan.stream_kv) PA_VALU_LAUNCH(float, true); else PA_VALU_LAUNCH(float, false);
      } else {
        if (plan.stream_kv) PA_VALU_LAUNCH(uint16_t, true); else PA_VALU_LAUNCH(uint16_t, false);
      }
#undef PA_VALU_LAUNCH
#undef PA_VALU_LAUNCH_G
#undef PA_VALU_LAUNCH_X
    } else {
      const size_t lds = generic_lds_bytes(G, D, B);
#define PA_GEN_LAUNCH_X(T, DIR, RR, APP)                                                          \
  PA_TIMED_LAUNCH(ps, (decode_generic_kernel<T, DIR, RR, APP>), grid, block, lds, st, (T*)k_pool,  \
                     (T*)v_pool, (const T*)q, (const T*)knew, (const T*)vnew, (T*)out, part_o,     \
                     part_ml, block_tables, context_lens, layer_off, g->num_blocks, Hkv,          \
                     n_q_heads, G, D, B, max_blocks_per_seq, max_context_len, plan.bps,            \
                     plan.S_max, qk_scale)
#define PA_GEN_LAUNCH_R(T, DIR, RR)                      \
  do {                                                   \
    if (append) PA_GEN_LAUNCH_X(T, DIR, RR, true);       \
    else PA_GEN_LAUNCH_X(T, DIR, RR, false);             \
  } while (0)
#define PA_GEN_LAUNCH(T, DIR)                         \
  do {                                                \
    const int need = (G * D + 63) / 64;               \
    if (need <= 1) PA_GEN_LAUNCH_R(T, DIR, 1);        \
    else if (need <= 4) PA_GEN_LAUNCH_R(T, DIR, 4);   \
    else if (need <= 16) PA_GEN_LAUNCH_R(T, DIR, 16); \
    else PA_GEN_LAUNCH_R(T, DIR, 64);                 \
  } while (0)
      if (g->dtype == PA_F32) {
        if (plan.direct) PA_GEN_LAUNCH(float, true); else PA_GEN_LAUNCH(float, false);
      } else {
        if (plan.direct) PA_GEN_LAUNCH(uint16_t, true); else PA_GEN_LAUNCH(uint16_t, false);
      }
#undef PA_GEN_LAUNCH_X
#undef PA_GEN_LAUNCH_R
#undef PA_GEN_LAUNCH
    }
    if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  }
  if (!plan.direct && !plan.merge) {
    ProfScope ps("decode_combine", st, timing, true);
    const dim3 grid((unsigned)((int64_t)n_seqs * n_q_heads)), block(64);
    // the MFMA and streaming VALU kernels write a one-split sequence's output
    // themselves; the generic kernel leaves every split to the combine
    const int single_written = plan.kernel != 1;
    if (g->dtype == PA_F32)  // bf16 output for bf16 and fp8 pools
      PA_TIMED_LAUNCH(ps, (decode_combine_kernel<float>), grid, block, 0, st, part_o, part_ml,
                         (float*)out, context_lens, n_q_heads, D, B, plan.S_max, plan.bps,
                         max_context_len, single_written);
    else
      PA_TIMED_LAUNCH(ps, (decode_combine_kernel<uint16_t>), grid, block, 0, st, part_o, part_ml,
                         (uint16_t*)out, context_lens, n_q_heads, D, B, plan.S_max, plan.bps,
                         max_context_len, single_written);
    if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  }
  return PA_OK;
}

// Split partials of the allocation-free decode entry point: a file-scope
// device array (one copy per GPU, kept until the process ends). Host code uses
// the address hipGetSymbolAddress gives on each device, never the name.
constexpr size_t kDecodeScratchBytes = 16u << 20;
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {
std::mutex g_scratch_mu;
std::vector<void*> g_scratch_dev;   // device id -> address of `scratch` there

// Address of this device's copy of `scratch`, looked up on the first call made
// with the device current.
pa_status decode_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return PA_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if ((size_t)dev >= g_scratch_dev.size()) g_scratch_dev.resize(dev + 1, nullptr);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return PA_ERR_HIP;
    }
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return PA_OK;
}
}  // namespace

extern "C" {

pa_status pa_decode(const pa_geom* g, const void* k_pool, const void* v_pool, int32_t layer,
                    const void* q, void* out, int32_t n_seqs, int32_t n_q_heads,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t max_context_len, float scale,
                    const pa_decode_opts* opts, void* workspace, size_t workspace_bytes,
                    void* stream) {
  return decode_impl(g, const_cast<void*>(k_pool), const_cast<void*>(v_pool), layer, q, nullptr,
                     nullptr, out, n_seqs, n_q_heads, block_tables, max_blocks_per_seq, context_lens,
                     max_context_len, scale, opts, workspace, workspace_bytes, stream);
}

pa_status pa_decode_append(const pa_geom* g, void* k_pool, void* v_pool, int32_t layer,
                           const void* q, const void* k_new, const void* v_new, void* out,
                           int32_t n_seqs, int32_t n_q_heads, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t max_context_len, float scale, const pa_decode_opts* opts,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (n_seqs > 0 && (!k_new || !v_new)) return PA_ERR_INVALID_ARG;
  return decode_impl(g, k_pool, v_pool, layer, q, k_new, v_new, out, n_seqs, n_q_heads,
                     block_tables, max_blocks_per_seq, context_lens, max_context_len, scale, opts,
                     workspace, workspace_bytes, stream);
}

pa_status pa_decode_append_noalloc(const pa_geom* g, void* k_pool, void* v_pool, int32_t layer,
                                   const void* q, const void* k_new, const void* v_new, void* out,
                                   int32_t n_seqs, int32_t n_q_heads, const int32_t* block_tables,
                                   int32_t max_blocks_per_seq, const int32_t* context_lens,
                                   int32_t max_context_len, float scale,
                                   const pa_decode_opts* opts, void* stream) {
  if (n_seqs > 0 && (!k_new || !v_new)) return PA_ERR_INVALID_ARG;
  // the combine launch merges the splits (the in-kernel merge's counters would
  // have to start at zero), and no timing events are created
  pa_decode_opts o = opts ? *opts : pa_decode_opts{};
  o.merge = 0;
  DecodePlan plan;
  const pa_status st0 = make_plan(g, n_seqs, n_q_heads, max_context_len, &o, &plan);
  if (st0 != PA_OK) return st0;
  if (plan.ws > kDecodeScratchBytes) return PA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (plan.ws > 0) {
    const pa_status st1 = decode_scratch(&ws);
    if (st1 != PA_OK) return st1;
  }
  return decode_impl(g, k_pool, v_pool, layer, q, k_new, v_new, out, n_seqs, n_q_heads,
                     block_tables, max_blocks_per_seq, context_lens, max_context_len, scale, &o, ws,
                     plan.ws > 0 ? kDecodeScratchBytes : 0, stream, /*timing=*/false);
}

static pa_status block_move(int mode, const char* name, const pa_geom* g, void* k_pool,
                            void* v_pool, void* staging, const int32_t* ids_a,
                            const int32_t* ids_b, int32_t n, void* stream) {
  if (!geom_ok(g) || n < 0) return PA_ERR_INVALID_ARG;
  if (n == 0) return PA_OK;
  if (!k_pool || !v_pool || !ids_a || (mode == 0 && !ids_b) || (mode != 0 && !staging))
    return PA_ERR_INVALID_ARG;
  const int64_t run = (int64_t)g->num_kv_heads * tile_bytes(g);
  const int64_t runs = (int64_t)n * g->num_layers * 2;
  if (runs > INT32_MAX) return PA_ERR_UNSUPPORTED;
  hipStream_t st = (hipStream_t)stream;
  ProfScope ps(name, st);
  const dim3 grid((unsigned)runs), block(256);
#define PA_MOVE(M, V)                                                                  \
  hipLaunchKernelGGL((block_move_kernel<M, V, PtrIds, PtrIds>), grid, block, 0, st,        \
                     (char*)k_pool,                                                         \
                     (char*)v_pool, (char*)staging, PtrIds{ids_a},                          \
                     PtrIds{mode == 0 ? ids_b : ids_a},                                     \
                     g->num_layers, g->num_blocks, run, runs)
#define PA_MOVE_MODE(M)                                            \
  do {                                                             \
    if (run % 16 == 0) PA_MOVE(M, u32x4);                          \
    else if (run % 4 == 0) PA_MOVE(M, uint32_t);                   \
    else if (run % 2 == 0) PA_MOVE(M, uint16_t);                   \
    else PA_MOVE(M, uint8_t);                                      \
  } while (0)
  if (mode == 0) PA_MOVE_MODE(0);
  else if (mode == 1) PA_MOVE_MODE(1);
  else PA_MOVE_MODE(2);
#undef PA_MOVE_MODE
#undef PA_MOVE
  return launch_status();
}

pa_status pa_copy_blocks(const pa_geom* g, void* k_pool, void* v_pool, const int32_t* src,
                         const int32_t* dst, int32_t n_pairs, void* stream) {
  return block_move(0, "copy_blocks", g, k_pool, v_pool, nullptr, src, dst, n_pairs, stream);
}

pa_status pa_gather_blocks(const pa_geom* g, const void* k_pool, const void* v_pool,
                           const int32_t* block_ids, int32_t n, void* staging, void* stream) {
  return block_move(1, "gather", g, const_cast<void*>(k_pool), const_cast<void*>(v_pool), staging,
                    block_ids, nullptr, n, stream);
}

pa_status pa_scatter_blocks(const pa_geom* g, void* k_pool, void* v_pool, const void* staging,
                            const int32_t* block_ids, int32_t n, void* stream) {
  return block_move(2, "scatter", g, k_pool, v_pool, const_cast<void*>(staging), block_ids, nullptr,
                    n, stream);
}

pa_status pa_copy_to_host(void* host_dst, const void* device_src, size_t bytes, void* stream) {
  if (bytes == 0) return PA_OK;
  if (!host_dst || !device_src) return PA_ERR_INVALID_ARG;
  return hipMemcpyAsync(host_dst, device_src, bytes, hipMemcpyDeviceToHost, (hipStream_t)stream) ==
                 hipSuccess
             ? PA_OK
             : PA_ERR_HIP;
}

pa_status pa_copy_to_device(void* device_dst, const void* host_src, size_t bytes, void* stream) {
  if (bytes == 0) return PA_OK;
  if (!device_dst || !host_src) return PA_ERR_INVALID_ARG;
  return hipMemcpyAsync(device_dst, host_src, bytes, hipMemcpyHostToDevice, (hipStream_t)stream) ==
                 hipSuccess
             ? PA_OK
             : PA_ERR_HIP;
}

pa_status pa_prof_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = on != 0;
  return PA_OK;
}

static void prof_drain_locked() {
  for (auto& r : g_prof_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) == hipSuccess && hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) {
      ProfAcc* acc = nullptr;
      for (auto& x : g_prof_acc)
        if (x.name == r.name) acc = &x;
      if (!acc) {
        g_prof_acc.push_back({r.name, 0, 0.0});
        acc = &g_prof_acc.back();
      }
      acc->launches += 1;
      acc->ms += ms;
    }
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_prof_pending.clear();
}

pa_status pa_prof_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  prof_drain_locked();
  g_prof_acc.clear();
  return PA_OK;
}

pa_status pa_prof_read(const char* kernel, int64_t* launches, double* total_ms) {
  if (!kernel || !launches || !total_ms) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  prof_drain_locked();
  *launches = 0;
  *total_ms = 0.0;
  for (auto& x : g_prof_acc)
    if (x.name == kernel) {
      *launches = x.launches;
      *total_ms = x.ms;
    }
  return PA_OK;
}

}  // extern "C"
