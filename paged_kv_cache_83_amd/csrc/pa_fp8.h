// One-byte KV storage (PA_FP8): the quantizing append and the decode kernel.
//
// Format (the pages give b_elem = 1 and no scale, "KV Cache Management",
// section "From Context Tokens to KV State", Eq. (1)): OCP FP8 E4M3 codes and,
// per (token, KV head), one power-of-two scale 2^e stored as the byte e + 127,
// with e the smallest integer such that max|x| <= 448 * 2^e. A (layer, block,
// head) tile is the B*d codes followed by the B scale bytes of its slots; with
// B = 16 the codes are ordered so that each lane of the decode kernel reads 16
// contiguous bytes and each load instruction 512 bytes of a block
// (fp8_k_index, fp8_v_index; other geometries keep the bf16 element order).
//
// Decode keeps the bf16 matrix-core path: E4M3 converts to bf16 exactly
// (v_cvt_scalef32_pk_bf16_fp8 with scale 1), the K scale of each key multiplies
// its score and the V scale of each key its probability before the PV product,
// both as exact power-of-two scalings in fp32 (v_ldexp_f32). The bytes read per
// key and head fall from 2*d*2 to 2*(d+1).
#pragma once

#include "pa_device.h"
#include "pa_pairs.h"

namespace pa_detail {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kFp8ScaleBias = 127;

// Smallest e with amax <= 448 * 2^e, clamped to [-127, 127]; 0 for amax == 0.
// amax = f * 2^x with f in [0.5, 1) and x = E - 126 for a normal float with
// exponent field E; 448 = 0.875 * 2^9, so e = x - 9 when f <= 0.875 (the
// significand 1.m <= 1.75, i.e. m <= 0x600000) and x - 8 otherwise. Integer
// logic only, so every caller takes the same decision. amax must be finite.
__device__ __forceinline__ int fp8_scale_exp(float amax) {
  const uint32_t b = __float_as_uint(amax);
  if (b == 0u) return 0;
  const int E = (int)(b >> 23);
  if (E == 0) return -127;  // below 2^-126: 448 * 2^-127 already covers it
  const int x = E - 126;
  const int e = (b & 0x7fffffu) <= 0x600000u ? x - 9 : x - 8;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Eight E4M3 codes (bytes of w, lowest first) as bf16, exactly.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(u32x2 w) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, true);
  const u32x4 u = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                   __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)};
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ int byte_of(u32x2 w, int k) {  // k compile-time after unrolling
  return (int)((w[k >> 2] >> (8 * (k & 3))) & 0xffu);
}

// Byte of slot o's dimension j among a tile's codes. K, B = 16 and 64 | D:
// rows of 64 codes, one chunk of 16 rows per 64 dimensions, the slots in row
// order 0-3, 8-11, 4-7, 12-15 (o with bits 2 and 3 swapped), so the 8 keys that
// one score tile's lanes read from a block are 512 contiguous bytes; a row's
// 8-dimension groups in the order 0, 4, 1, 5, 2, 6, 3, 7, so the 16 bytes of
// lane group gq are its fragments of two consecutive 32-dimension k-steps.
// V, B = 16 and 32 | D: per 32 dimensions 512 bytes [slot half][dim % 16]
// [(dim / 16) % 2][slot % 8], so a lane's 8 slots of two dimension tiles are 16
// contiguous bytes. Other geometries: the bf16 orders (K [D/W][B][W], V [D][B]).
__device__ __forceinline__ int fp8_k_index(int o, int j, int B, int D) {
  if (B == 16 && (D & 63) == 0)
    return 1024 * (j >> 6) + 64 * (o ^ ((((o >> 2) ^ (o >> 3)) & 1) * 12)) + 16 * ((j >> 3) & 3) +
           8 * ((j >> 5) & 1) + (j & 7);
  const int W = k_chunk(D);
  return (j / W) * B * W + o * W + j % W;
}
__device__ __forceinline__ int fp8_v_index(int o, int j, int B, int D) {
  if (B == 16 && (D & 31) == 0)
    return 512 * (j >> 5) + 256 * (o >> 3) + 16 * (j & 15) + 8 * ((j >> 4) & 1) + (o & 7);
  return j * B + o;
}

// ---------------------------------------------------------------------------
// Quantizing append: one wave per (token, KV head). The wave reduces max|x|
// over the head's d values, derives e, and writes the d codes and the scale
// byte of K and of V into the token's slot. k_new / v_new: bf16 [n][H][d].
// ---------------------------------------------------------------------------

template <typename SlotSrc>
__global__ __launch_bounds__(256) void append_fp8_kernel(uint8_t* __restrict__ kpool,
                                                        uint8_t* __restrict__ vpool,
                                                        const uint16_t* __restrict__ knew,
                                                        const uint16_t* __restrict__ vnew,
                                                        SlotSrc slots, int64_t n_tok, int H, int D,
                                                        int B, int64_t nslots, int64_t layer_off) {
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (item >= n_tok * H) return;
  const int64_t j = item / H;
  const int h = (int)(item % H);
  const int64_t slot = slots(j);
  if (slot < 0 || slot >= nslots) return;
  const int64_t p = slot / B;
  const int o = (int)(slot % B);
  const int64_t TB = (int64_t)B * D + B;
#pragma unroll
  for (int kv = 0; kv < 2; ++kv) {
    const uint16_t* row = (kv ? vnew : knew) + (j * H + h) * D;
    uint8_t* t = (kv ? vpool : kpool) + layer_off + (p * H + h) * TB;
    float amax = 0.f;
    for (int d = lane; d < D; d += 64) amax = fmaxf(amax, fabsf(bf16_to_f32(row[d])));
    amax = wave_max(amax);
    const int e = fp8_scale_exp(amax);
    for (int d = lane; d < D; d += 64) {
      const float x = __builtin_amdgcn_ldexpf(bf16_to_f32(row[d]), -e);
      const uint8_t code = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(x, 0.0f, 0, false) & 0xff);
      t[kv ? fp8_v_index(o, d, B, D) : fp8_k_index(o, d, B, D)] = code;
    }
    if (lane == 0) t[(int64_t)B * D + o] = (uint8_t)(e + kFp8ScaleBias);
  }
}

// Bulk form for d = 128, B = 16: a work group quantizes 16 consecutive rows of
// one head. Thread t handles piece t % 16 (8 dimensions) of row t / 16, for K
// and for V; the row's maximum comes from its 16 lanes. K pieces leave as
// 8-byte stores into their row. V goes through LDS: when 8 rows land in 8
// consecutive slots of one block starting at a multiple of 8 (a chunk of a
// prompt), each dimension's 8 codes leave as one 8-byte store; otherwise as
// single bytes. The codes are those of the general kernel (same scale rule,
// same conversion instruction).
template <typename SlotSrc>
__global__ __launch_bounds__(256) void append_fp8_rows16_kernel(uint8_t* __restrict__ kpool,
                                                               uint8_t* __restrict__ vpool,
                                                               const uint16_t* __restrict__ knew,
                                                               const uint16_t* __restrict__ vnew,
                                                               SlotSrc slots, int64_t n_tok, int H,
                                                               int64_t nslots, int64_t layer_off) {
  constexpr int D = 128, B = 16;
  constexpr int64_t TB = (int64_t)B * D + B;
  __shared__ uint8_t vcodes[16][D];  // [row][dimension]
  __shared__ int64_t rslot[16];
  const int h = (int)(blockIdx.x % H);
  const int64_t grp = blockIdx.x / H;
  const int t = threadIdx.x, r = t >> 4, piece = t & 15;
  const int64_t j = grp * 16 + r;
  int64_t slot = -1;
  if (j < n_tok) {
    slot = slots(j);
    if (slot < 0 || slot >= nslots) slot = -1;
  }
  if (piece == 0) rslot[r] = slot;
  const int64_t p = slot >= 0 ? slot / B : 0;
  const int o = slot >= 0 ? (int)(slot % B) : 0;
#pragma unroll
  for (int kv = 0; kv < 2; ++kv) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (j < n_tok) raw = *reinterpret_cast<const u32x4*>((kv ? vnew : knew) + (j * H + h) * D + 8 * piece);
    float x[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = __uint_as_float(raw[k] << 16);
      x[2 * k + 1] = __uint_as_float(raw[k] & 0xffff0000u);
    }
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(x[k]));
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 16));
    const int e = fp8_scale_exp(amax);
    uint32_t c[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(x[4 * k], -e),
                                              __builtin_amdgcn_ldexpf(x[4 * k + 1], -e), 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(x[4 * k + 2], -e),
                                          __builtin_amdgcn_ldexpf(x[4 * k + 3], -e), w, true);
      c[k] = (uint32_t)w;
    }
    uint8_t* tile = (kv ? vpool : kpool) + layer_off + (p * H + h) * TB;
    if (kv == 0) {
      if (slot >= 0) {
        const int d0 = 8 * piece;
        *reinterpret_cast<u32x2*>(tile + fp8_k_index(o, d0, B, D)) = u32x2{c[0], c[1]};
      }
    } else {
      *reinterpret_cast<u32x2*>(&vcodes[r][8 * piece]) = u32x2{c[0], c[1]};
    }
    if (piece == 0 && slot >= 0) tile[(int64_t)B * D + o] = (uint8_t)(e + kFp8ScaleBias);
  }
  __syncthreads();
  // V: thread t writes dimension t % 128 of rows 8 * (t / 128) .. + 7
  const int d = t & (D - 1), hf = t >> 7;
  const int64_t s0 = rslot[8 * hf];
  bool contig = s0 >= 0 && (s0 % 8) == 0;
#pragma unroll
  for (int k = 1; k < 8; ++k) contig = contig && rslot[8 * hf + k] == s0 + k;
  if (contig) {
    uint32_t lo = 0u, hi = 0u;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      lo |= (uint32_t)vcodes[8 * hf + k][d] << (8 * k);
      hi |= (uint32_t)vcodes[8 * hf + 4 + k][d] << (8 * k);
    }
    uint8_t* tile = vpool + layer_off + ((s0 / B) * H + h) * TB;
    *reinterpret_cast<u32x2*>(tile + fp8_v_index((int)(s0 % B), d, B, D)) = u32x2{lo, hi};
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t sk = rslot[8 * hf + k];
      if (sk < 0) continue;
      uint8_t* tile = vpool + layer_off + ((sk / B) * H + h) * TB;
      tile[fp8_v_index((int)(sk % B), d, B, D)] = vcodes[8 * hf + k][d];
    }
  }
}

// The quantizing append for n_tok rows: the bulk form when the geometry allows,
// the general one otherwise. Returns false if the grid would be too large.
template <typename SlotSrc>
inline bool launch_append_fp8(hipStream_t st, uint8_t* kpool, uint8_t* vpool, const uint16_t* knew,
                              const uint16_t* vnew, SlotSrc slots, int64_t n_tok, int H, int D,
                              int B, int64_t nslots, int64_t layer_off) {
  if (D == 128 && B == 16) {
    const int64_t wgs = (n_tok + 15) / 16 * H;
    if (wgs > INT32_MAX) return false;
    hipLaunchKernelGGL((append_fp8_rows16_kernel<SlotSrc>), dim3((unsigned)wgs), dim3(256), 0, st,
                       kpool, vpool, knew, vnew, slots, n_tok, H, nslots, layer_off);
    return true;
  }
  const int64_t wgs = (n_tok * H + 3) / 4;  // one wave per (row, head)
  if (wgs > INT32_MAX) return false;
  hipLaunchKernelGGL((append_fp8_kernel<SlotSrc>), dim3((unsigned)wgs), dim3(256), 0, st, kpool,
                     vpool, knew, vnew, slots, n_tok, H, D, B, nslots, layer_off);
  return true;
}

// ---------------------------------------------------------------------------
// Decode, FP8 pool, matrix cores: B = 16, d in {64, 128}, up to 16 query heads
// per KV head. The work decomposition, the score-row / key assignment, the
// split-K partials and the pipelining are those of the bf16 kernel; per pair
// of blocks a lane loads 16-byte code pieces (K: 16 dims of one key; V: 8 keys
// of two dims, from the tile orders of fp8_k_index / fp8_v_index) and the 8 K
// and 8 V scale bytes of its 8 keys.
// ---------------------------------------------------------------------------
template <int D>
struct Fp8Frags {
  u32x4 k[2][D / 64];  // score tile t: dims 64 j + 8 gq .. + 8, then 64 j + 32 + 8 gq .. + 8
  u32x4 v[D / 32];     // slots 8 (gq & 1) .. + 8 of dims 16 (2 u) + c, then 16 (2 u + 1) + c
  u32x2 ks, vs;
};

// The 8 codes that form K fragment kc of score tile t: dims 32 kc + 8 gq .. + 8.
template <int D>
__device__ __forceinline__ u32x2 fp8_k_frag(const Fp8Frags<D>& f, int t, int kc) {
  const u32x4 w = f.k[t][kc >> 1];
  return (kc & 1) ? u32x2{w[2], w[3]} : u32x2{w[0], w[1]};
}
// The 8 codes of the V^T fragment of dimension tile dt.
template <int D>
__device__ __forceinline__ u32x2 fp8_v_frag(const Fp8Frags<D>& f, int dt) {
  const u32x4 w = f.v[dt >> 1];
  return (dt & 1) ? u32x2{w[2], w[3]} : u32x2{w[0], w[1]};
}
template <bool NT>
__device__ __forceinline__ u32x2 kv_load8(const uint8_t* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  else return *reinterpret_cast<const u32x2*>(p);
}
template <bool NT>
__device__ __forceinline__ u32x4 fp8_load16(const uint8_t* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  else return *reinterpret_cast<const u32x4*>(p);
}

// Lane (c, gq): k_lane = 64 * (c & 7) + 16 * gq (row 8 t + (c & 7) of the key's
// block holds its key of score tile t), v_lane = 256 * (gq & 1) + 16 * c, s_off =
// 8 * (gq & 1).
template <int D, bool NT>
__device__ __forceinline__ void fp8_issue_pair(Fp8Frags<D>& f, const uint8_t* __restrict__ kl,
                                               const uint8_t* __restrict__ vl, int p0, int p1,
                                               int Hkv, int g, int k_sel, int k_lane, int v_sel,
                                               int v_lane, int s_off) {
  constexpr int TB = 16 * D + 16;
  const uint8_t* kt = kl + ((int64_t)(k_sel ? p1 : p0) * Hkv + g) * TB;
  const uint8_t* ks = kl + ((int64_t)(v_sel ? p1 : p0) * Hkv + g) * TB;
  const uint8_t* vt = vl + ((int64_t)(v_sel ? p1 : p0) * Hkv + g) * TB;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int j = 0; j < D / 64; ++j) f.k[t][j] = fp8_load16<NT>(kt + 1024 * j + 512 * t + k_lane);
#pragma unroll
  for (int u = 0; u < D / 32; ++u) f.v[u] = fp8_load16<NT>(vt + 512 * u + v_lane);
  f.ks = kv_load8<NT>(ks + 16 * D + s_off);
  f.vs = kv_load8<NT>(vt + 16 * D + s_off);
}

// Zeroes the V codes of the lane's slots whose bit is clear in keep (8 slots,
// one byte mask each).
template <int D>
__device__ __forceinline__ void fp8_mask_v(Fp8Frags<D>& f, u32x2 keep) {
  const u32x4 k4 = {keep[0], keep[1], keep[0], keep[1]};
#pragma unroll
  for (int u = 0; u < D / 32; ++u) f.v[u] &= k4;
}

template <int D>
__device__ __forceinline__ void fp8_compute_pair(Fp8Frags<D>& f, const bf16x8 (&qf)[D / 32],
                                                 f32x4 (&acc)[D / 16], float& m_run, float& l_run,
                                                 int blk, int len, int gq, float qk_scale) {
  constexpr int KC = D / 32;
  constexpr int DT = D / 16;
  f32x4 sc[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    sc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
      sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(fp8_k_frag(f, t, kc)), qf[kc],
                                                      sc[t], 0, 0, 0);
  }
  // Lane holds the scores of pair-local keys 8*gq + 4*t + e for query c; byte
  // 4*t + e of f.ks is that key's K scale.
  const int pos0 = blk * 16 + 8 * gq;
  float sv[8];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      sv[4 * t + e] = (pos0 + 4 * t + e < len)
                          ? __builtin_amdgcn_ldexpf(sc[t][e] * qk_scale,
                                                    byte_of(f.ks, 4 * t + e) - kFp8ScaleBias)
                          : -INFINITY;
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
    // The PV operand carries each key's V scale (an exact power of two).
    pw[e >> 1] = pack_bf16x2(__builtin_amdgcn_ldexpf(pa, byte_of(f.vs, e) - kFp8ScaleBias),
                             __builtin_amdgcn_ldexpf(pb, byte_of(f.vs, e + 1) - kFp8ScaleBias));
  }
  if (__any(m_new != m_run)) {
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = acc[dt] * alpha;
  }
  l_run += psum;
  m_run = m_new;
  const bf16x8 pf = __builtin_bit_cast(bf16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));

  // Slots at or past the length hold unspecified bytes (possibly NaN codes):
  // their codes become 0 so that 0 * V stays 0.
  if (blk * 16 + 32 > len) {
    u32x2 keep = {0u, 0u};
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (pos0 + k < len) keep[k >> 2] |= 0xffu << (8 * (k & 3));
    fp8_mask_v(f, keep);
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(fp8_v_frag(f, dt)), pf, acc[dt],
                                                      0, 0, 0);
}

// One token's K and V rows (bf16, d values each) quantized into slot o of
// their block's tiles by one wave, with the append kernels' rule and
// instructions (one power-of-two scale per row from its largest magnitude,
// E4M3 codes by the same pair conversion), so the pool bytes are theirs: lane
// l < D/8 takes K dims 8 l .. + 7, lane D/8 + l the same V dims.
template <int D>
__device__ __forceinline__ void fp8_put_token(uint8_t* __restrict__ kt, uint8_t* __restrict__ vt,
                                              const uint16_t* __restrict__ krow,
                                              const uint16_t* __restrict__ vrow, int o, int lane) {
  constexpr int P = D / 8;  // pieces of a row
  const bool is_v = lane >= P;
  const int piece = lane & (P - 1);
  u32x4 raw = {0u, 0u, 0u, 0u};
  if (lane < 2 * P) raw = *reinterpret_cast<const u32x4*>((is_v ? vrow : krow) + 8 * piece);
  float x[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = __uint_as_float(raw[k] << 16);
    x[2 * k + 1] = __uint_as_float(raw[k] & 0xffff0000u);
  }
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(x[k]));
#pragma unroll
  for (int m = P / 2; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, P));
  const int e = fp8_scale_exp(amax);
  uint32_t c[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(x[4 * k], -e),
                                            __builtin_amdgcn_ldexpf(x[4 * k + 1], -e), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(x[4 * k + 2], -e),
                                        __builtin_amdgcn_ldexpf(x[4 * k + 3], -e), w, true);
    c[k] = (uint32_t)w;
  }
  if (lane < P) {
    *reinterpret_cast<u32x2*>(kt + fp8_k_index(o, 8 * piece, 16, D)) = u32x2{c[0], c[1]};
    if (piece == 0) kt[16 * D + o] = (uint8_t)(e + kFp8ScaleBias);
  } else if (lane < 2 * P) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      vt[fp8_v_index(o, 8 * piece + k, 16, D)] = (uint8_t)(c[k >> 2] >> (8 * (k & 3)));
    if (piece == 0) vt[16 * D + o] = (uint8_t)(e + kFp8ScaleBias);
  }
}

// APPEND: the step's new token of every sequence (position len-1) comes in
// knew/vnew [n][H_kv][d] (bf16); the item whose range holds that position
// quantizes it into the pool (fp8_put_token) and waits for those stores
// before it loads any pair, so its loads of the block read the new codes.
template <int D, int OUT, bool NT, int NS, bool APPEND>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void decode_mfma_fp8_kernel(
    uint8_t* __restrict__ kpool, uint8_t* __restrict__ vpool,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ knew,
    const uint16_t* __restrict__ vnew, uint16_t* __restrict__ out, float* __restrict__ part_o,
    float* __restrict__ part_ml, const int32_t* __restrict__ tables,
    const int32_t* __restrict__ lens, int64_t layer_off, int N, int Hkv, int Hq, int G,
    int max_blocks, int max_ctx, int bps, int S_max, float qk_scale, int* __restrict__ counters) {
  constexpr int KC = D / 32;
  constexpr int DT = D / 16;

  const int w = blockIdx.x;
  const int g = w % Hkv;
  const int si = w / Hkv;
  const int s = si % S_max;
  const int i = si / S_max;
  const int lane = threadIdx.x;
  const int c = lane & 15;
  const int gq = lane >> 4;

  const int len = clamp_len(lens, i, max_ctx);
  const int nblk = (len + 15) >> 4;
  const int b0 = s * bps;
  const int h = g * G + c;
  const bool qvalid = c < G;
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

  const int32_t* trow = tables + (int64_t)i * max_blocks;
  int tb[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int idx = b0 + 64 * k + lane;
    tb[k] = (64 * k < b1 - b0 && idx < b1) ? guard_block(trow[idx], N) : 0;
  }

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

  f32x4 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.f;

  const uint8_t* kl = kpool + layer_off;
  const uint8_t* vl = vpool + layer_off;
  if constexpr (APPEND) {
    if (len > 0 && b1 == nblk) {   // wave-uniform: the last block of the sequence is this item's
      constexpr int TB = 16 * D + 16;
      const int64_t tile = ((int64_t)table_at(tb, nblk - 1 - b0) * Hkv + g) * TB;
      const int64_t row = ((int64_t)i * Hkv + g) * D;
      fp8_put_token<D>(kpool + layer_off + tile, vpool + layer_off + tile, knew + row, vnew + row,
                       (len - 1) & 15, lane);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the codes are in L2 before any pair load
    }
  }
  // Score row c of each tile holds pair-local key 8*(c>>2) + 4*t + (c&3): block
  // c >> 3, tile row 8*t + (c&7).
  const int k_sel = c >> 3;
  const int k_lane = 64 * (c & 7) + 16 * gq;
  // V^T fragment: block (gq >> 1), dims 16*dt + c, slots 8*(gq&1) .. +8; the
  // lane's 8 keys are the same slots of the same block, whose scales it reads.
  const int v_sel = gq >> 1;
  const int v_lane = 256 * (gq & 1) + 16 * c;
  const int s_off = 8 * (gq & 1);

  const int span = b1 - b0;
  const int npairs = (span + 1) >> 1;
  auto issue_at = [&](Fp8Frags<D>& fr, int pj) {
    const int off = 2 * pj;
    const int p0 = table_at(tb, off);
    const int p1 = (off + 1 < span) ? table_at(tb, off + 1) : p0;
    fp8_issue_pair<D, NT>(fr, kl, vl, p0, p1, Hkv, g, k_sel, k_lane, v_sel, v_lane, s_off);
  };
  // NS pairs in flight; steady loop issues unconditionally, the tail drains
  // (the structure of the bf16 kernel).
  Fp8Frags<D> f[NS];
  int pj = 0;
  if (npairs >= 2 * NS - 1) {
#pragma unroll
    for (int st = 0; st < NS - 1; ++st) issue_at(f[st], st);
    for (; pj + 2 * NS - 1 <= npairs; pj += NS) {
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        issue_at(f[(st + NS - 1) % NS], pj + st + NS - 1);
        fp8_compute_pair<D>(f[st], qf, acc, m_run, l_run, b0 + 2 * (pj + st), len, gq, qk_scale);
      }
    }
  } else {
#pragma unroll
    for (int st = 0; st < NS - 1; ++st)
      if (st < npairs) issue_at(f[st], st);
  }
#pragma unroll
  for (int k = 0; k < 2 * NS - 2; ++k) {
    if (pj + k >= npairs) break;
    if (pj + k + NS - 1 < npairs) issue_at(f[(k + NS - 1) % NS], pj + k + NS - 1);
    fp8_compute_pair<D>(f[k % NS], qf, acc, m_run, l_run, b0 + 2 * (pj + k), len, gq, qk_scale);
  }

  l_run = sum_over_groups(l_run);
  mfma_split_epilogue<D, OUT>(acc, m_run, l_run, lane, i, g, G, Hq, Hkv, s, S_max, (nblk + bps - 1) / bps,
                         out, part_o, part_ml, counters);
}

}  // namespace pa_detail
