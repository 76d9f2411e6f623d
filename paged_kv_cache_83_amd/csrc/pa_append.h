// The tile append kernel, shared by the slot-mapped append and by chunked
// prefill (which derives each token's slot from its chunk's block table).
#pragma once

#include "pa_device.h"

namespace pa_detail {

// Slot of token j given explicitly (negative = skip).
struct SlotsFromArray {
  const int64_t* slots;
  __device__ int64_t operator()(int64_t j) const { return slots[j]; }
};

// Batch of chunks: chunk i owns rows [q_start[i], q_start[i+1]) of the token
// arrays; its row r is position ctx_lens[i] + r - q_start[i] of sequence i, which
// lives in block tables[i][pos / B] at offset pos mod B. Returns the chunk of row
// j (or -1) with its position. Values are clamped the same way everywhere they
// are read: q_start into [0, n_tok] and non-decreasing, chunk lengths to
// max_q_len, cached lengths so that cached + chunk <= max_ctx.
struct ChunkBatch {
  const int32_t* q_start;
  const int32_t* ctx_lens;
  int n_seqs;
  int n_tok;
  int max_q_len;
  int max_ctx;
  __device__ int start(int i) const {
    const int v = q_start[i];
    return v < 0 ? 0 : (v > n_tok ? n_tok : v);
  }
  // first row, number of rows and cached tokens of chunk i
  __device__ void chunk(int i, int& a, int& q_len, int& ctx) const {
    a = start(i);
    int b = start(i + 1);
    b = b < a ? a : b;
    q_len = b - a > max_q_len ? max_q_len : b - a;
    ctx = ctx_lens[i];
    ctx = ctx < 0 ? 0 : ctx;
    ctx = ctx > max_ctx - q_len ? max_ctx - q_len : ctx;
    ctx = ctx < 0 ? 0 : ctx;
  }
  __device__ int find(int64_t j) const {  // largest i with start(i) <= j, or -1
    int lo = 0, hi = n_seqs - 1, ans = -1;
    while (lo <= hi) {
      const int mid = (lo + hi) >> 1;
      if (start(mid) <= j) { ans = mid; lo = mid + 1; }
      else hi = mid - 1;
    }
    return ans;
  }
};

struct SlotsFromTables {
  ChunkBatch cb;
  const int32_t* tables;
  int max_blocks;
  int B;
  int N;
  __device__ int64_t operator()(int64_t j) const {
    const int i = cb.find(j);
    if (i < 0) return -1;
    int a, q_len, ctx;
    cb.chunk(i, a, q_len, ctx);
    if (j - a >= q_len) return -1;
    const int pos = ctx + (int)(j - a);
    const int lb = pos / B;
    if (lb >= max_blocks) return -1;
    const int p = tables[(int64_t)i * max_blocks + lb];
    if (p < 0 || p >= N) return -1;
    return (int64_t)p * B + pos % B;
  }
};

// One work group per (16 consecutive tokens, KV head). The chunk's K and V rows
// are read with 16-byte loads into LDS while the slots load (the source addresses
// do not depend on them); then each K piece goes to its place in the K tile, and
// V, whose tile keeps one row of B slots per dimension, is written from its
// transposed LDS copy with the lanes along the slots: tokens in consecutive
// slots of one block give contiguous stores. Every token carries its own
// destination, so any slot mapping is handled.
constexpr int kAppendChunk = 16;
constexpr int kXcds = 8;  // accelerator complex dies of the part, which take work groups in turn

template <typename T>
constexpr size_t append_lds_bytes(int D) {
  return kAppendChunk * sizeof(int64_t) + (size_t)kAppendChunk * D * sizeof(T) +
         (size_t)D * (kAppendChunk + 1) * sizeof(T);
}

template <typename T, int VEC, typename SlotSrc>
__global__ __launch_bounds__(256) void append_kv_kernel(T* __restrict__ kpool, T* __restrict__ vpool,
                                                        const T* __restrict__ knew,
                                                        const T* __restrict__ vnew, SlotSrc slots,
                                                        int n_tok, int Hkv, int D, int B,
                                                        int64_t nslots, int64_t layer_off) {
  extern __shared__ __align__(16) unsigned char append_smem[];
  constexpr int LD = kAppendChunk + 1;  // padded row of the transposed V chunk
  int64_t* s_slot = reinterpret_cast<int64_t*>(append_smem);
  T* s_k = reinterpret_cast<T*>(append_smem + kAppendChunk * sizeof(int64_t));  // [token][D]
  T* s_v = s_k + kAppendChunk * D;                                                // [D][LD]
  // Work groups go to the 8 XCDs round-robin; give each XCD a contiguous range of
  // (head, chunk) items so that neighbouring chunks, which share the V rows of a
  // block they straddle, are written through the same L2 one after the other.
  const int64_t nchunks = ((int64_t)n_tok + kAppendChunk - 1) / kAppendChunk;
  const int64_t per_xcd = (int64_t)gridDim.x / kXcds;
  const int64_t item = (int64_t)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (item >= nchunks * Hkv) return;
  const int h = (int)(item / nchunks);
  const int64_t j0 = (item - (int64_t)h * nchunks) * kAppendChunk;
  const int tid = threadIdx.x;
  const int nk = (int)min<int64_t>(kAppendChunk, n_tok - j0);  // tokens in this chunk
  if (tid < kAppendChunk) {
    int64_t sl = -1;
    if (tid < nk) {
      sl = slots(j0 + tid);
      if (sl < 0 || sl >= nslots) sl = -1;  // negative: skip; out of range: ignored
    }
    s_slot[tid] = sl;
  }
  const int pieces = D / VEC;
  for (int idx = tid; idx < nk * pieces; idx += blockDim.x) {
    const int k = idx / pieces, d0 = (idx - k * pieces) * VEC;
    const int64_t row = ((j0 + k) * Hkv + h) * D + d0;
    T kv[VEC], vv[VEC];
    load_vec<T, VEC>(kv, knew + row);
    load_vec<T, VEC>(vv, vnew + row);
    store_vec<T, VEC>(s_k + k * D + d0, kv);
#pragma unroll
    for (int u = 0; u < VEC; ++u) s_v[(d0 + u) * LD + k] = vv[u];
  }
  __syncthreads();
  const int W = k_chunk(D);  // VEC divides W: a piece stays in one K chunk
  for (int idx = tid; idx < nk * pieces; idx += blockDim.x) {
    const int k = idx / pieces, d0 = (idx - k * pieces) * VEC;
    const int64_t sl = s_slot[k];
    if (sl < 0) continue;
    const int64_t p = sl / B;
    const int o = (int)(sl - p * B);
    T kv[VEC];
    load_vec<T, VEC>(kv, s_k + k * D + d0);
    store_vec<T, VEC>(kpool + layer_off + (p * Hkv + h) * (int64_t)B * D + (int64_t)(d0 / W) * B * W +
                          (int64_t)o * W + (d0 % W),
                      kv);
  }
  if constexpr (sizeof(T) == 2) {
    // The usual bulk case: the chunk's 16 tokens fill one whole block in order.
    // Each V row of the tile is then 16 consecutive slots, written as two
    // 16-byte stores (8 slots each) instead of 16 element stores.
    bool whole = B == kAppendChunk && nk == kAppendChunk && s_slot[0] >= 0 && s_slot[0] % B == 0;
#pragma unroll
    for (int k = 1; k < kAppendChunk; ++k) whole = whole && s_slot[k] == s_slot[0] + k;
    if (whole) {  // uniform: every thread read the same slots
      const int64_t p = s_slot[0] / B;
      T* tile = vpool + layer_off + (p * Hkv + h) * (int64_t)B * D;
      for (int idx = tid; idx < 2 * D; idx += blockDim.x) {
        const int d = idx >> 1, half = idx & 1;
        const T* src = s_v + d * LD + 8 * half;
        uint32_t w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          w[u] = (uint32_t)src[2 * u] | ((uint32_t)src[2 * u + 1] << 16);
        *reinterpret_cast<uint4*>(tile + (int64_t)d * B + 8 * half) = make_uint4(w[0], w[1], w[2], w[3]);
      }
      return;
    }
  }
  for (int idx = tid; idx < kAppendChunk * D; idx += blockDim.x) {
    const int k = idx % kAppendChunk, d = idx / kAppendChunk;
    const int64_t sl = s_slot[k];
    if (sl < 0) continue;
    const int64_t p = sl / B;
    const int o = (int)(sl - p * B);
    vpool[layer_off + (p * Hkv + h) * (int64_t)B * D + (int64_t)d * B + o] = s_v[d * LD + k];
  }
}

}  // namespace pa_detail
