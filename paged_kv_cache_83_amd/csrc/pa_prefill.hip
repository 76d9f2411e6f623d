// Chunked-prefill (multi-query) paged attention for gfx950.
//
// Source: "KV Cache Management", section "Chunked prefill mechanics". A prompt is
// processed in chunks; the queries of chunk k attend over the keys and values of
// every earlier chunk, already in paged blocks, and over the chunk's own tokens
// with a lower-triangular causal mask; the chunk's keys and values are written
// into the sequence's paged blocks. Writing them first and then attending over
// the pool with the causal mask gives the same outputs (every query sees exactly
// the positions at or before its own) and lets one kernel read every key through
// the block table ("The PagedAttention virtual memory model").
//
// Kernel shape. A work group (4 waves) owns one tile of 128 query rows of one
// (chunk, KV head): the G query heads of the group times 128/G consecutive chunk
// tokens, 32 rows per wave, as two 16-column MFMA tiles. It walks the visible
// keys in pairs of blocks (32 keys). Each pair's K and V tiles (4 per pair) are
// loaded once for the 128 rows straight from global memory into LDS (16 bytes
// per lane), two pairs ahead of use in three rotating images, then read as MFMA
// operand fragments at the offsets the decode kernel uses on the pool (the LDS
// image has the pool's tile layout, but for a swap of 16-byte columns in the
// K rows of slots 8-15 that keeps the fragment reads free of bank conflicts):
//   S^T[32 keys][16 rows] = K[keys][d] . Q^T[d][rows]     (two tiles of rows)
//   O^T[d][16 rows]      += V^T[d][keys] . P^T[keys][rows]
// with the online-softmax update of the same section between them. The QK^T
// products of the next pair are issued before the softmax of the current one,
// so the matrix cores and the vector ALUs work at the same time. The vector
// work per pair is kept small: the causal mask only on pairs that cross some
// row's position, the softmax scale folded into the exponent's FMA, and the
// accumulators rescaled only when a row's maximum has grown by more than 2^8
// over the reference it exponentiates against (the result is the same; the
// reference is only a bound on the size of the probabilities). Work-group
// order is XCD-aware: the tiles of one (chunk, KV head) run one after another on
// one XCD, so its history is read from HBM once and from that XCD's L2 after.
// Chunks of at most 32 query rows per KV head take a second kernel,
// prefill_short_kernel: one wave holds all of them and streams the history
// through registers like the decode kernel.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "../../include/pa.h"
#include "pa_append.h"
#include "pa_addr.h"
#include "pa_device.h"
#include "pa_host.h"
#include "pa_fp8.h"
#include "pa_pairs.h"

namespace {

using namespace pa_detail;

constexpr int kPfWaves = 4;
constexpr int kPfRowsPerWave = 32;                  // two 16-column MFMA tiles
constexpr int kPfRows = kPfWaves * kPfRowsPerWave;  // query rows per work group

// Wait until at most N of this wave's global-to-LDS loads are in flight and its
// LDS reads have completed, then synchronise the work group. Written out because
// the barrier intrinsic with a fence waits for every outstanding load.
template <int N>
__device__ __forceinline__ void lds_wait_sync() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Splitting the visible keys of a tile across work groups (for batches too small
// to fill the chip): each split writes its unnormalised output, its reference
// maximum (log2 units) and its sum, and a second kernel merges them with the
// online-softmax rule ("Chunked prefill mechanics": the m, l, O recurrence).
constexpr int kPfMaxSplits = 64;
constexpr int kPfAutoMaxSplits = 4;
constexpr int kPfTargetWgs = 512;       // two resident work groups per CU
constexpr int kPfMinPairsPerSplit = 8;

struct PfSplit {
  int n;           // splits per tile; 1: outputs are written directly
  float* part_o;   // [n_tokens][Hq][n][D], when n > 1
  float* part_ml;  // [n_tokens][Hq][n][2]: reference maximum (log2 units), sum
};

// Pairs of blocks in flight per wave in the short-chunk kernel (bf16 and FP8
// pools).
#ifndef PA_SHORT_STAGES
#define PA_SHORT_STAGES 2
#endif
#ifndef PA_FP8_SHORT_STAGES
#define PA_FP8_SHORT_STAGES 2
#endif

// Growth of a row's maximum (log2 units) tolerated before the accumulators are
// rescaled to a new reference.
constexpr float kLazyLog2 = 8.0f;

// Vector ALU instructions placed after each QK^T product of the next pair in a
// steady step (the softmax of the current pair is spread over them). Measured
// with conflict-free K fragment reads: 10 (and 12, 14) beat 4, 5, 8, 16 and 20
// by 2% on the chunked-prefill workload and 5% on the prefix-reuse one.
#ifndef PA_PF_VALU_PER_MFMA
#define PA_PF_VALU_PER_MFMA 10
#endif
constexpr int kPfValuPerMfma = PA_PF_VALU_PER_MFMA;
// ... and before the first of them, after the fragment reads.
#ifndef PA_PF_LEAD_VALU
#define PA_PF_LEAD_VALU 0
#endif
constexpr int kPfLeadValu = PA_PF_LEAD_VALU;

// Maximum of three scores in one instruction. The scores reaching it are finite
// or -inf (masked), so the quieting of signalling NaNs that fmaxf must do on the
// products of the matrix cores (an extra instruction per operand) is not needed.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float d;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}

// acc + lo + hi of a packed pair of bf16 values, in one dot-product instruction
// (against the pair (1, 1)).
typedef __bf16 pf_bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float add_bf16x2(uint32_t pair, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(pf_bf16x2, pair),
                                         __builtin_bit_cast(pf_bf16x2, 0x3f803f80u), acc, false);
}

// This wave's LDS accesses have completed; then synchronise the work group
// (no wait for global loads still in flight into registers).
__device__ __forceinline__ void lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int D>
struct PfCfg {
  static constexpr int KC = D / 32;                        // QK k-steps
  static constexpr int DT = D / 16;                        // PV row tiles
  static constexpr int TILE_BYTES = 16 * D * 2;            // one (block, head) K or V tile
  static constexpr int PAIR_BYTES = 4 * TILE_BYTES;        // K0, K1, V0, V1
  static constexpr int LOADS = PAIR_BYTES / (16 * 64 * kPfWaves);  // 16-byte loads per thread
};

// The same kernel serves bf16 pools (FP8 = false: tiles go straight from HBM
// into LDS) and one-byte pools (FP8 = true: each thread loads its share of the
// pair's E4M3 codes and scale bytes a step ahead into registers and converts
// them to bf16 with the power-of-two scale of their key in the conversion
// instruction (round to nearest even of code x 2^e, exact unless below bf16's
// normal range, 2^-126), writing into the same LDS image the bf16 path builds,
// so everything after the staging is shared).
template <int D, int G, bool FP8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void prefill_mfma_kernel(
    const char* __restrict__ kpool, const char* __restrict__ vpool,
    const uint16_t* __restrict__ q, uint16_t* __restrict__ out, ChunkBatch cb,
    const int32_t* __restrict__ tables, int64_t layer_off, int N, int Hkv, int Hq, int max_blocks,
    int n_tiles, float qk_scale, PfSplit sp) {
  constexpr int KC = PfCfg<D>::KC;
  constexpr int DT = PfCfg<D>::DT;
  constexpr int TILE = PfCfg<D>::TILE_BYTES;  // one bf16 tile in the LDS image
  constexpr int PAIR = PfCfg<D>::PAIR_BYTES;
  constexpr int LOADS = PfCfg<D>::LOADS;
  constexpr int PTILE = FP8 ? 16 * D + 16 : TILE;  // one tile in the pool (codes + scales)
  constexpr int TQ = kPfRows / G;        // chunk tokens per work group
  constexpr int TW = kPfRowsPerWave / G;  // chunk tokens per wave
  extern __shared__ __align__(16) unsigned char pf_smem[];  // three pair images

  // Work groups are dealt to the XCDs in turn (group b runs on XCD b % 8). XCD x
  // takes the (chunk, KV head) groups x, x + 8, x + 16, ... (group = chunk * H_kv
  // + head), each group's splits and tiles one after another, the last (longest)
  // tiles first: a group's history is read into one L2, and every XCD gets the
  // same mix of short and long chunks (with H_kv = 8, one head of every chunk).
  const int64_t per_group = (int64_t)n_tiles * sp.n;
  const int64_t u = blockIdx.x / kXcds;
  const int64_t ig = (int64_t)(blockIdx.x % kXcds) + kXcds * (u / per_group);
  if (ig >= (int64_t)cb.n_seqs * Hkv) return;  // whole work group
  const int64_t rem = u % per_group;
  const int split = (int)(rem % sp.n);
  const int tile = n_tiles - 1 - (int)(rem / sp.n);
  const int g = (int)(ig % Hkv);
  const int i = (int)(ig / Hkv);
  int a, q_len, ctx;
  cb.chunk(i, a, q_len, ctx);
  const int t0 = tile * TQ;
  if (t0 >= q_len) return;  // whole work group
  const int kmax = ctx + min(t0 + TQ, q_len);  // keys [0, kmax) are visible to some row
  const int nblk = (kmax + 15) >> 4;
  const int npairs = (nblk + 1) >> 1;
  // this split's pairs [pbeg, pend); the causal diagonal falls in the last split
  const int pbeg = (int)((int64_t)split * npairs / sp.n);
  const int pend = (int)((int64_t)(split + 1) * npairs / sp.n);

  const int tid = threadIdx.x;
  // the wave index is uniform; readfirstlane lets the compiler keep what derives
  // from it (tile choice, load bases) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, c = lane & 15, gq = lane >> 4;

  // Query rows of this wave: row r = 16*ct + c is token t0 + TW*wave + r/G,
  // query head g*G + r%G. Rows past the chunk end get zero queries (finite
  // scores) and are not written.
  bf16x8 qf[2][KC];
  int qpos[2];
  bool rvalid[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int r = 16 * ct + c;
    const int tok = t0 + TW * wave + r / G;
    rvalid[ct] = tok < q_len;
    qpos[ct] = rvalid[ct] ? ctx + tok : kmax - 1;
    const uint16_t* qrow = q + ((int64_t)(a + (rvalid[ct] ? tok : 0)) * Hq + g * G + r % G) * D;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (rvalid[ct]) v = *reinterpret_cast<const u32x4*>(qrow + 32 * kc + 8 * gq);
      qf[ct][kc] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // Smallest query position of the wave (its first row, or every row past the
  // chunk end): pairs wholly at or below it need no causal mask.
  const int qmin = (t0 + TW * wave < q_len) ? ctx + t0 + TW * wave : kmax - 1;

  f32x4 acc[2][DT];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[ct][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};
  float ms[2] = {0.f, 0.f};                // -m_run * c (0 while m_run = -inf)
  float thr[2] = {-INFINITY, -INFINITY};   // m_run + kLazyLog2 / c
  const float lazy_gap = kLazyLog2 / qk_scale;

  const int32_t* trow = tables + (int64_t)i * max_blocks;
  const char* kl = kpool + layer_off;  // layer_off in bytes
  const char* vl = vpool + layer_off;

  // Pair image in LDS: [K blk0][K blk1][V blk0][V blk1], each tile as in the
  // pool except that in the K tiles' rows of slots 8-15 the 16-byte columns
  // trade places in pairs (column j at j ^ 2): a K fragment read takes slots s
  // and s + 8 of a chunk in one instruction, 512 bytes apart, which would
  // otherwise fall in the same LDS banks (measured: 4 conflict cycles per read,
  // none with the swap). The unit at 16-byte index x of a K chunk holds the
  // pool's unit x ^ ((x >> 4) & 2).
  // Three images rotate: the pair whose softmax and PV are being done, the next
  // pair (its keys are read for QK^T one step early) and the pair after that
  // (its loads in flight). Loads go from global memory straight into LDS: lane
  // l of wave w puts its 16 bytes at image offset 16 * (256 u + 64 w + l), the
  // same place the thread's own store would. The compiler does not order these
  // loads against LDS reads, so each step waits for them itself (vmcnt) before
  // its one barrier.
  const char* kg = kl + (int64_t)g * PTILE;  // head g's tile in block 0
  const char* vg = vl + (int64_t)g * PTILE;
  const int64_t blk_stride = (int64_t)Hkv * PTILE;

  // The split's block ids, one per lane and register: a window of 256 blocks
  // from wbase, read by readlane when a pair's loads are issued (no memory
  // round trip per pair). Pairs are issued in increasing order; the window moves
  // on when one falls past it (a wait for that load, once every 128 pairs).
  int tb[4];
  int wbase = 2 * pbeg;
  auto load_window = [&]() {
#pragma unroll
    for (int k = 0; k < 4; ++k)  // (lanes past the split's blocks repeat its last id)
      tb[k] = guard_block(trow[min(wbase + 64 * k + lane, nblk - 1)], N);
  };
  load_window();
  auto pair_ids = [&](int pj, int& p0, int& p1) {
    const int b0 = 2 * pj;
    if (b0 - wbase >= 256) {  // uniform
      wbase = b0;
      load_window();
    }
    p0 = table_at(tb, b0 - wbase);
    p1 = (b0 + 1 < nblk) ? table_at(tb, b0 + 1 - wbase) : p0;
  };
  // Load u of a thread fills the same tile (K or V of the pair's first or
  // second block) at the same offset on every pair: fixed per wave, so only
  // the two block products change from pair to pair.
  const char* ld_base[LOADS];
  bool ld_second[LOADS];
#pragma unroll
  for (int u = 0; u < LOADS; ++u) {
    const int woff = (u * 256 + wave * 64) * 16;  // the wave's first byte in the image
    const int tl = woff / TILE;                   // tile of the whole wave
    ld_second[u] = (tl & 1) != 0;
    ld_base[u] = (tl < 2 ? kg : vg) + (woff - tl * TILE);
  }
  // (d = 128: one load instruction of the work group fills exactly one tile,
  // load u tile u, so the choice of block and array is known at compile time)
  constexpr bool kLoadIsTile = TILE == 16 * 64 * kPfWaves;
  constexpr int KP = LOADS / 2;  // loads (pieces) of K tiles: the first half; the rest V
  const int k_src = (lane ^ ((lane >> 4) & 2)) * 16;   // K: the pool unit of the lane's LDS unit
  auto issue = [&](int pj, int buf) {
    int p0, p1;
    pair_ids(pj, p0, p1);
    // block ids are in [0, N) and a block's stride fits 32 bits: unsigned products
    const uint64_t off0 = (uint64_t)(uint32_t)p0 * (uint32_t)blk_stride;
    const uint64_t off1 = (uint64_t)(uint32_t)p1 * (uint32_t)blk_stride;
    unsigned char* img = pf_smem + buf;
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int woff = (u * 256 + wave * 64) * 16;
      const char* base;
      if constexpr (kLoadIsTile)
        base = (u < 2 ? kg : vg) + ((u & 1) ? off1 : off0) + wave * 64 * 16;
      else
        base = ld_base[u] + (ld_second[u] ? off1 : off0);
      // The base is uniform; pinning it to scalar registers lets the load take
      // it as its scalar base with the lane's 16-byte offset, instead of a
      // 64-bit vector address computed per load.
      // (readfirstlane returns a signed int: join_address_words widens both
      // halves as unsigned 32-bit words, so the low word is not sign-extended.)
      const uint64_t bu = reinterpret_cast<uint64_t>(base);
      const uint32_t bhi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(bu >> 32));
      const uint32_t blo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)bu);
      const uint64_t bs = join_address_words(bhi, blo);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(bs) + (u < KP ? k_src : lane * 16),
                                       (__attribute__((address_space(3))) void*)(img + woff), 16,
                                       0, 0);
    }
  };

  // FP8 staging. Piece u of a thread is the 8 elements whose bf16 form sits at
  // image offset 16 * (256 u + tid), element el of tile tl in the bf16 order
  // (K: slot (el / 32) % 16, dims 32 (el / 512) + el % 32 .. + 8; V: dim el / 16,
  // slots el % 16 .. + 8): in the pool, 8 contiguous code bytes of the one-byte
  // tile order, plus the scale bytes of their keys (K: one key; V: 8 slots).
  struct Raw {
    u32x2 code[LOADS];
    uint32_t ks;       // K: the scale byte of piece u in byte u
    u32x2 vs[KP];      // V: 8 bytes each, one per slot
  };
  auto load_raw = [&](int pj, Raw& r) {
    int p0, p1;
    pair_ids(pj, p0, p1);
    r.ks = 0u;
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int woff = (u * 256 + wave * 64) * 16;
      const int tl = woff / TILE;                      // the same for all lanes of a wave
      const int el = (woff - tl * TILE) / 2 + lane * 8;  // first element of the piece
      const int p = (tl & 1) ? p1 : p0;
      const char* t = (tl < 2 ? kg : vg) + p * blk_stride;
      const int code_off = u < KP ? fp8_k_index((el >> 5) & 15, 32 * (el >> 9) + (el & 31), 16, D)
                                  : fp8_v_index(el & 15, el >> 4, 16, D);
      r.code[u] = *reinterpret_cast<const u32x2*>(t + code_off);
      if (u < KP)  // K: one key, the slot of the W-chunk row
        r.ks |= (uint32_t)(uint8_t)t[16 * D + ((el >> 5) & 15)] << (8 * u);
      else         // V: slots el % 16 .. + 7 of one dimension
        r.vs[u - KP] = *reinterpret_cast<const u32x2*>(t + 16 * D + (el & 15));
    }
  };
  // The conversion takes the scale as an fp32 operand: 2^(b - 127) is the float
  // whose bits are b << 23 (a scale byte of 0 gives 0: rows with max |x| <=
  // 448 * 2^-127 become 0). Its bf16 pair result is used as a whole 32-bit word.
  auto cvt2 = [](uint32_t word, float scale, auto hi_half) -> uint32_t {
    if constexpr (decltype(hi_half)::value)
      return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, scale, true));
    else
      return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, scale, false));
  };
  using lo_t = std::integral_constant<bool, false>;
  using hi_t = std::integral_constant<bool, true>;
  auto stash_raw = [&](const Raw& r, int buf) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int woff = (u * 256 + wave * 64) * 16;
      u32x4 w;
      if (u < KP) {  // K: the 8 codes of one key, one scale
        const float sk = __uint_as_float(((r.ks >> (8 * u)) & 0xffu) << 23);
        w = u32x4{cvt2(r.code[u][0], sk, lo_t{}), cvt2(r.code[u][0], sk, hi_t{}),
                  cvt2(r.code[u][1], sk, lo_t{}), cvt2(r.code[u][1], sk, hi_t{})};
      } else {  // V: 8 keys; each code pair converted with both keys' scales, halves merged
        float sv[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
          sv[k] = __uint_as_float(((r.vs[u - KP][k >> 2] >> (8 * (k & 3))) & 0xffu) << 23);
        const uint32_t m = 0x0000ffffu;
        w = u32x4{(cvt2(r.code[u][0], sv[0], lo_t{}) & m) | (cvt2(r.code[u][0], sv[1], lo_t{}) & ~m),
                  (cvt2(r.code[u][0], sv[2], hi_t{}) & m) | (cvt2(r.code[u][0], sv[3], hi_t{}) & ~m),
                  (cvt2(r.code[u][1], sv[4], lo_t{}) & m) | (cvt2(r.code[u][1], sv[5], lo_t{}) & ~m),
                  (cvt2(r.code[u][1], sv[6], hi_t{}) & m) | (cvt2(r.code[u][1], sv[7], hi_t{}) & ~m)};
      }
      // K pieces go to their swapped column (the LDS unit that holds this pool unit)
      *reinterpret_cast<u32x4*>(pf_smem + buf + woff + (u < KP ? k_src : lane * 16)) = w;
    }
  };

  // Score row c of each tile holds pair-local key 8*(c>>2) + 4*t + (c&3): block
  // (c >> 3) of the pair, offset 8*((c>>2)&1) + 4*t + (c&3). V^T fragment of a
  // lane: block (gq >> 1), dims 16*dt + c, slots 8*(gq&1) .. +8.
  const int k_sel = c >> 3;
  const int k_off0 = 8 * ((c >> 2) & 1) + (c & 3);
  const int k_col = 16 * (gq ^ (2 * ((c >> 2) & 1)));   // slot k_off0 + 4t >= 8 iff (c >> 2) & 1
  const int v_sel = gq >> 1;
  const int v_off = 32 * c + 16 * (gq & 1);  // bytes

  // S^T of one pair for both row tiles: K fragments from the pair's image, then
  // the QK^T products (their results are consumed one step later).
  auto scores = [&](int buf, f32x4 (&sc)[2][2]) {
    const unsigned char* img = pf_smem + buf;
    u32x4 kf[2][KC];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        kf[t][kc] = *reinterpret_cast<const u32x4*>(img + k_sel * TILE + kc * 1024 +
                                                    (k_off0 + 4 * t) * 64 + k_col);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        sc[ct][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
          sc[ct][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, kf[t][kc]), qf[ct][kc], sc[ct][t], 0, 0, 0);
      }
  };

  // Softmax update and PV of pair pj from its scores and its V image. EDGE:
  // the pair may hold keys above some row's position or past the valid data
  // (else it is known to hold neither, and the products of the next pair,
  // issued just before, are interleaved with the softmax).
  //
  // Scores stay unscaled through the mask and the maximum (the scale is
  // positive); the scale enters in the exponent: p = 2^(s * c + ms), ms = -m * c
  // for the row's reference maximum m. The reference moves only when a score
  // passes it by more than kLazyLog2 (log2 units), i.e. exceeds thr = m +
  // kLazyLog2 / c: until then p stays below 2^kLazyLog2, which bf16 and the fp32
  // sums hold as exactly as p <= 1, and the accumulators need no rescaling. The
  // test is per lane (its 8 scores against thr); only when some lane of the wave
  // passes is the exact row maximum formed across the row's four lane groups,
  // the references of the rows that passed moved to it, their accumulators
  // rescaled and the probabilities recomputed. The first pair always moves it
  // (m = -inf; key 0 is visible to every row). A row may see no key of a split
  // at all (a later split than its position): m stays -inf, ms 0, p 0.
  auto finish = [&](int pj, const u32x4 (&vin)[DT], const f32x4 (&sc)[2][2], auto edge) {
    constexpr bool EDGE = decltype(edge)::value;
    u32x4 vf[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vf[dt] = vin[dt];
    const int key0 = 32 * pj + 8 * gq;  // this lane's keys: key0 + 4*t + e (scores), key0 + e (V)
    if (EDGE && 32 * pj + 32 > kmax) {  // slots past the valid data: V zeroed (0 * NaN guard)
      u32x4 keep;
#pragma unroll
      for (int wv = 0; wv < 4; ++wv) {
        const int p = key0 + 2 * wv;
        keep[wv] = (p < kmax ? 0x0000ffffu : 0u) | (p + 1 < kmax ? 0xffff0000u : 0u);
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) vf[dt] &= keep;
    }
    const bool diag = EDGE && 32 * pj + 31 > qmin;  // uniform: some key of the pair is above some row
    float sv[2][8], lmax[2], psum[2];
    uint32_t pw[2][4];
    bool pass = false;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[ct][4 * t + e] = sc[ct][t][e];
      if (diag) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (key0 + 4 * t + e > qpos[ct]) sv[ct][4 * t + e] = -INFINITY;
      }
      lmax[ct] = max3f(max3f(sv[ct][0], sv[ct][1], sv[ct][2]), max3f(sv[ct][3], sv[ct][4], sv[ct][5]),
                       max3f(sv[ct][6], sv[ct][7], sv[ct][7]));
      pass = pass || lmax[ct] > thr[ct];
    }
    auto probs = [&]() {
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        psum[ct] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float pa = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[ct][e], qk_scale, ms[ct]));
          const float pb = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[ct][e + 1], qk_scale, ms[ct]));
          pw[ct][e >> 1] = pack_bf16x2(pa, pb);
          // the row sum takes the probabilities as the P.V products do (bf16)
          psum[ct] = add_bf16x2(pw[ct][e >> 1], psum[ct]);
        }
      }
    };
    probs();
    if constexpr (!EDGE) {
      // One scheduling region holds the K fragment reads and QK^T products of
      // the next pair and this softmax: spread the vector work between the
      // products, so the matrix core and the vector ALU work at the same time
      // within the wave (by default the products would all issue first). The
      // empty asm keeps the probabilities in this region (the compiler would
      // otherwise sink them past the reference test, next to their use).
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
        asm volatile("" : "+v"(psum[ct]), "+v"(pw[ct][0]), "+v"(pw[ct][1]), "+v"(pw[ct][2]),
                     "+v"(pw[ct][3]));
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * KC, 0);  // LDS reads
      if constexpr (kPfLeadValu > 0)  // vector work while the reads are in flight
        __builtin_amdgcn_sched_group_barrier(0x002, kPfLeadValu, 0);
#pragma unroll
      for (int k = 0; k < 4 * KC; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, kPfValuPerMfma, 0);  // vector ALU
      }
    }
    if (__any(pass)) {  // uniform, rare
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const float mb = max_over_groups(lmax[ct]);
        const float m_new = mb > thr[ct] ? mb : m_run[ct];
        const float alpha =
            m_new == m_run[ct] ? 1.f : __builtin_amdgcn_exp2f((m_run[ct] - m_new) * qk_scale);
        l_run[ct] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[ct][dt] = acc[ct][dt] * alpha;
        m_run[ct] = m_new;
        ms[ct] = m_new == -INFINITY ? 0.f : -m_new * qk_scale;
        thr[ct] = m_new + lazy_gap;
      }
      probs();
    }
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      l_run[ct] += psum[ct];
      const bf16x8 pf =
          __builtin_bit_cast(bf16x8, make_uint4(pw[ct][0], pw[ct][1], pw[ct][2], pw[ct][3]));
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        acc[ct][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vf[dt]),
                                                              pf, acc[ct][dt], 0, 0, 0);
    }
  };

  // Step pj: loads of pair pj+2 go out; V of pair pj is read; once pair pj+1
  // has landed (every wave waited for its own loads, then the barrier), its
  // QK^T products are issued, and the softmax and PV of pair pj run while the
  // matrix cores work on them. Steady steps (edge = false): the pairs the step
  // loads exist and pair pj needs no mask, so the step has no branch before its
  // reference test.
  // b_cur, b_next, b_new: byte offsets of the images of pairs pj, pj+1, pj+2.
  int b_cur = 0, b_next = PAIR, b_new = 2 * PAIR;
  Raw raw;  // FP8: the pair after next, in registers
  using edge_t = std::integral_constant<bool, true>;
  using steady_t = std::integral_constant<bool, false>;
  auto step = [&](int pj, const f32x4 (&sc_cur)[2][2], f32x4 (&sc_next)[2][2], auto edge) {
    constexpr bool EDGE = decltype(edge)::value;
    if constexpr (!FP8) {
      if (!EDGE || pj + 2 < pend) issue(pj + 2, b_new);
    }
    u32x4 vf[DT];
    const unsigned char* img = pf_smem + b_cur;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      vf[dt] = *reinterpret_cast<const u32x4*>(img + (2 + v_sel) * TILE + dt * 512 + v_off);
    if (!EDGE || pj + 1 < pend) {
      if constexpr (FP8)
        lds_sync();  // this wave's stores of pair pj+1 (last step) are done; then all waves'
      else if (!EDGE || pj + 2 < pend)
        lds_wait_sync<LOADS>();  // pair pj+1 landed; pair pj+2 may still be in flight
      else
        lds_wait_sync<0>();
      scores(b_next, sc_next);
    }
    if constexpr (FP8) {
      // pair pj+2 into the free image (every wave finished reading it before the
      // last barrier; the next barrier waits for these stores), converted while
      // the products of pair pj+1 run; then the codes of pair pj+3 are loaded
      if (!EDGE || pj + 2 < pend) stash_raw(raw, b_new);
      if (!EDGE || pj + 3 < pend) load_raw(pj + 3, raw);
    }
    finish(pj, vf, sc_cur, edge);
    const int b_old = b_cur;
    b_cur = b_next;
    b_next = b_new;
    b_new = b_old;
  };
  if (pbeg < pend) {
  if constexpr (FP8) {
    load_raw(pbeg, raw);
    stash_raw(raw, 0);
    if (pend - pbeg > 1) {
      load_raw(pbeg + 1, raw);
      stash_raw(raw, PAIR);
    }
    if (pend - pbeg > 2) load_raw(pbeg + 2, raw);
    lds_sync();
  } else {
    issue(pbeg, 0);
    if (pend - pbeg > 1) {
      issue(pbeg + 1, PAIR);
      lds_wait_sync<LOADS>();
    } else {
      lds_wait_sync<0>();
    }
  }
  f32x4 sa[2][2], sb[2][2];
  scores(0, sa);
  int pj = pbeg;  // the ranges below are uniform across the work group
  {
    // pairs wholly at or below the tile's first position whose step needs no
    // test of the pairs after it (bf16: pair pj+2 exists; FP8: pj+3 as well)
    const int psteady = min((ctx + t0 + 1) >> 5, pend - (FP8 ? 3 : 2));
    for (; pj + 1 < psteady; pj += 2) {
      step(pj, sa, sb, steady_t{});
      step(pj + 1, sb, sa, steady_t{});
    }
  }
  for (; pj + 1 < pend; pj += 2) {
    step(pj, sa, sb, edge_t{});
    step(pj + 1, sb, sa, edge_t{});
  }
  if (pj < pend) step(pj, sa, sb, edge_t{});
  }  // pbeg < pend (uniform); an empty split writes m = -inf, l = 0, O = 0

  // acc[ct][dt][e] = O^T[d = 16*dt + 4*gq + e][row 16*ct + c]
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const float l = sum_over_groups(l_run[ct]);
    if (!rvalid[ct]) continue;
    const int r = 16 * ct + c;
    const int tok = t0 + TW * wave + r / G;
    const int64_t row = (int64_t)(a + tok) * Hq + g * G + r % G;
    if (sp.n == 1) {
      const float inv = 1.f / l;
      uint16_t* o = out + row * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<uint2*>(o + 16 * dt + 4 * gq) =
            make_uint2(pack_bf16x2(acc[ct][dt][0] * inv, acc[ct][dt][1] * inv),
                       pack_bf16x2(acc[ct][dt][2] * inv, acc[ct][dt][3] * inv));
    } else {
      const int64_t slot = row * sp.n + split;
      float* po = sp.part_o + slot * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<f32x4*>(po + 16 * dt + 4 * gq) = acc[ct][dt];
      if (gq == 0)
        *reinterpret_cast<float2*>(sp.part_ml + slot * 2) =
            make_float2(m_run[ct] == -INFINITY ? -INFINITY : m_run[ct] * qk_scale, l);
    }
  }
}

// Merges the splits of every output row: weights 2^(m_s - M), normalised by
// the weighted sums. D/4 lanes per row (16-byte loads of four dimensions), so a
// 256-thread work group merges 1024/D rows.
template <int D>
__global__ __launch_bounds__(256) void prefill_combine_kernel(const float* __restrict__ part_o,
                                                              const float* __restrict__ part_ml,
                                                              uint16_t* __restrict__ out,
                                                              int64_t rows, int S) {
  constexpr int LPR = D / 4;  // lanes per row
  const int64_t row = (int64_t)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  if (row >= rows) return;
  const int col = 4 * (threadIdx.x % LPR);
  const float* ml = part_ml + row * S * 2;
  // finite: the split holding pair 0 gives every row key 0
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, ml[2 * s]);
  float L = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < S; ++s) {
    const float w = __builtin_amdgcn_exp2f(ml[2 * s] - M);  // 0 for an empty split
    L = fmaf(w, ml[2 * s + 1], L);
    const f32x4 v = *reinterpret_cast<const f32x4*>(part_o + (row * S + s) * D + col);
    o += w * v;
  }
  const float inv = 1.f / L;
  *reinterpret_cast<uint2*>(out + row * D + col) =
      make_uint2(pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv));
}

// Short chunks: at most 32 query rows per KV head (G x chunk length <= 32, a
// few tokens per sequence, as when a draft's tokens are verified against a long
// history). A 128-row tile would leave most of its waves on padding, so one wave
// per (chunk, KV head, split of the keys) holds every row of the chunk as CT
// 16-column MFMA tiles and takes each pair of blocks from the pool straight into
// operand registers, the way the decode kernel does (two pairs in flight, no
// LDS); the pair's K and V fragments serve all CT tiles, so the history is read
// once. Row r = 16*ct + c is chunk token r / G, query head g*G + r % G; its keys
// stop at its own position, so pairs reaching past the chunk's first position
// are masked per column, and slots at or past the chunk's end get zero
// probability and zeroed V. Splits cover bps blocks each (even, at most 256: the
// table entries of a split sit in four registers of the wave); with more than
// one, each writes its partial result in the layout prefill_combine_kernel
// merges. With CT = 2 and d = 128 on bf16 pools the wave holds 64 accumulator,
// 32 query and 128 fragment registers per lane, beyond the 256 of two waves per
// SIMD: it runs alone on its SIMD, which the launch sizes for (about one wave
// per SIMD). FP8 fragments are half as large, so that variant keeps the
// two-wave budget (with two registers spilled), which measured faster than one
// wave per SIMD with three pairs in flight.
//
// FP8 pools (E4M3 codes with a power-of-two scale per token and head): the
// pair's codes and scale bytes come in as the FP8 decode kernel loads them
// (16-byte pieces of the one-byte tile order), the codes are converted to bf16
// exactly in registers,
// each key's K scale multiplies its score (ldexp, exact) and its V scale is
// folded into its probability in the PV operand, as in the FP8 decode kernel.
template <int D, int CT, bool FP8>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu((CT * D > 128 && !FP8) ? 1 : PA_MFMA_WPE))) void prefill_short_kernel(
    const char* __restrict__ kpool, const char* __restrict__ vpool,
    const uint16_t* __restrict__ q, uint16_t* __restrict__ out, ChunkBatch cb,
    const int32_t* __restrict__ tables, int64_t layer_off, int N, int Hkv, int Hq, int G,
    int max_blocks, int bps, float qk_scale, PfSplit sp) {
  constexpr int KC = MfmaCfg<D>::KC;
  constexpr int DT = MfmaCfg<D>::DT;
  constexpr int NS = FP8 ? PA_FP8_SHORT_STAGES : PA_SHORT_STAGES;
  using Frags = std::conditional_t<FP8, Fp8Frags<D>, PairFrags<D>>;

  // KV head fastest, then split: the waves reading one sequence's blocks start together.
  const int w = blockIdx.x;
  const int g = w % Hkv;
  const int si = w / Hkv;
  const int s = si % sp.n;
  const int i = si / sp.n;
  if (i >= cb.n_seqs) return;
  const int lane = threadIdx.x;
  const int c = lane & 15;
  const int gq = lane >> 4;
  int a, q_len, ctx;
  cb.chunk(i, a, q_len, ctx);
  if (q_len == 0) return;
  const int total = ctx + q_len;  // keys [0, total) exist; row t sees [0, ctx + t]
  const int nblk = (total + 15) >> 4;
  const int b0 = s * bps;
  const int b1 = min(b0 + bps, nblk);

  bf16x8 qf[CT][KC];
  int lim[CT];
  bool rvalid[CT];
  int64_t orow[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int r = 16 * ct + c;
    const int t = r / G;
    rvalid[ct] = t < q_len;
    lim[ct] = rvalid[ct] ? ctx + t + 1 : total;  // padding columns: zero queries, any limit
    orow[ct] = (int64_t)(a + (rvalid[ct] ? t : 0)) * Hq + g * G + r % G;
    const uint16_t* qrow = q + orow[ct] * D;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (rvalid[ct]) v = *reinterpret_cast<const u32x4*>(qrow + 32 * kc + 8 * gq);
      qf[ct][kc] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x4 acc[CT][DT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[ct][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[CT], l_run[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    m_run[ct] = -INFINITY;
    l_run[ct] = 0.f;
  }

  if (b0 < b1) {  // uniform; an empty split (past the chunk's end) writes m = -inf, l = 0, O = 0
    const int32_t* trow = tables + (int64_t)i * max_blocks;
    int tb[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int idx = b0 + 64 * k + lane;
      tb[k] = (64 * k < b1 - b0 && idx < b1) ? guard_block(trow[idx], N) : 0;
    }
    const char* kl = kpool + layer_off;  // layer_off in bytes
    const char* vl = vpool + layer_off;
    // Score row c of each tile holds pair-local key 8*(c>>2) + 4*t + (c&3); the
    // lane's V^T fragment is block (gq >> 1), dims 16*dt + c, slots 8*(gq&1) .. +8
    // (FP8: the lane's 8 keys are those slots, whose scale bytes it loads).
    const int k_sel = c >> 3;
    const int k_off0 = 8 * ((c >> 2) & 1) + (c & 3);
    const int v_sel = gq >> 1;
    const int v_off = 16 * c + 8 * (gq & 1);
    const int span = b1 - b0;
    const int npairs = (span + 1) >> 1;
    auto issue_at = [&](Frags& fr, int pj) {
      const int off = 2 * pj;
      const int p0 = table_at(tb, off);
      const int p1 = (off + 1 < span) ? table_at(tb, off + 1) : p0;
      if constexpr (FP8)
        fp8_issue_pair<D, true>(fr, reinterpret_cast<const uint8_t*>(kl),
                                reinterpret_cast<const uint8_t*>(vl), p0, p1, Hkv, g, k_sel,
                                64 * (c & 7) + 16 * gq, v_sel, 256 * (gq & 1) + 16 * c, 8 * (gq & 1));
      else
        issue_pair<D, true>(fr, reinterpret_cast<const uint16_t*>(kl),
                            reinterpret_cast<const uint16_t*>(vl), p0, p1, Hkv, g, k_sel, k_off0,
                            v_sel, v_off, gq, -1, nullptr);
      // Keep the loads ahead of the products of the pair before them: moved
      // below its first product they would start only after that pair's wait.
      __builtin_amdgcn_sched_barrier(0);
    };

    // One pair: S^T for every tile, the masked online-softmax update (the scale
    // enters in the exponent, p = 2^(s*c - m*c); the reference maximum moves
    // only when passed by more than kLazyLog2), then O^T += V^T P^T per tile.
    auto compute = [&](Frags& f, int pj) {
      const int k0 = 16 * (b0 + 2 * pj);  // first key of the pair
      bf16x8 kb[2][KC];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          if constexpr (FP8) kb[t][kc] = fp8x8_to_bf16(fp8_k_frag(f, t, kc));
          else kb[t][kc] = __builtin_bit_cast(bf16x8, f.k[t][kc]);
        }
      f32x4 sc[CT][2];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          sc[ct][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kc = 0; kc < KC; ++kc)
            sc[ct][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[t][kc], qf[ct][kc], sc[ct][t],
                                                                0, 0, 0);
        }
      const int key0 = k0 + 8 * gq;  // the lane's keys: key0 + 4*t + e (scores), key0 + e (V)
      if (k0 + 32 > total) {  // uniform: slots past the data hold anything (0 * NaN guard)
        if constexpr (FP8) {
          u32x2 keep = {0u, 0u};
#pragma unroll
          for (int k = 0; k < 8; ++k)
            if (key0 + k < total) keep[k >> 2] |= 0xffu << (8 * (k & 3));
          fp8_mask_v(f, keep);
        } else {
          u32x4 keep;
#pragma unroll
          for (int wv = 0; wv < 4; ++wv) {
            const int p = key0 + 2 * wv;
            keep[wv] = (p < total ? 0x0000ffffu : 0u) | (p + 1 < total ? 0xffff0000u : 0u);
          }
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) f.v[dt] &= keep;
        }
      }
      const bool masked = k0 + 32 > ctx + 1;  // uniform: some key past the first row's position
      float m_new[CT], psum[CT];
      uint32_t pw[CT][4];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        float sv[8];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if constexpr (FP8)  // the key's K scale, exactly
              sv[4 * t + e] = __builtin_amdgcn_ldexpf(sc[ct][t][e],
                                                      byte_of(f.ks, 4 * t + e) - kFp8ScaleBias);
            else
              sv[4 * t + e] = sc[ct][t][e];
          }
        if (masked) {
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (key0 + 4 * t + e >= lim[ct]) sv[4 * t + e] = -INFINITY;
        }
        float mb = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                         fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
        mb = max_over_groups(mb);
        // A column may see no key of this split yet (its maximum stays -inf and
        // its probabilities 0).
        const float m_cand = fmaxf(m_run[ct], mb);
        m_new[ct] = ((m_cand - m_run[ct]) * qk_scale > kLazyLog2) ? m_cand : m_run[ct];
        const float ms = (m_new[ct] == -INFINITY) ? 0.f : -m_new[ct] * qk_scale;
        psum[ct] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float pa = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[e], qk_scale, ms));
          const float pb = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[e + 1], qk_scale, ms));
          psum[ct] += pa + pb;
          if constexpr (FP8)  // the PV operand carries each key's V scale
            pw[ct][e >> 1] =
                pack_bf16x2(__builtin_amdgcn_ldexpf(pa, byte_of(f.vs, e) - kFp8ScaleBias),
                            __builtin_amdgcn_ldexpf(pb, byte_of(f.vs, e + 1) - kFp8ScaleBias));
          else
            pw[ct][e >> 1] = pack_bf16x2(pa, pb);
        }
      }
      bool moved = false;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) moved = moved || m_new[ct] != m_run[ct];
      if (__any(moved)) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const float alpha = (m_new[ct] == m_run[ct])
                                  ? 1.f
                                  : __builtin_amdgcn_exp2f((m_run[ct] - m_new[ct]) * qk_scale);
          l_run[ct] *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) acc[ct][dt] = acc[ct][dt] * alpha;
        }
      }
      bf16x8 vb[DT];  // the V^T fragments as bf16, shared by the tiles
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        if constexpr (FP8) vb[dt] = fp8x8_to_bf16(fp8_v_frag(f, dt));
        else vb[dt] = __builtin_bit_cast(bf16x8, f.v[dt]);
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        l_run[ct] += psum[ct];
        m_run[ct] = m_new[ct];
        const bf16x8 pf =
            __builtin_bit_cast(bf16x8, make_uint4(pw[ct][0], pw[ct][1], pw[ct][2], pw[ct][3]));
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          acc[ct][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb[dt], pf, acc[ct][dt], 0, 0, 0);
      }
    };

    // NS pairs in flight, as in the decode kernel: the steady loop issues
    // unconditionally, an unrolled tail drains the last pairs.
    Frags f[NS];
    int pj = 0;
    if (npairs >= 2 * NS - 1) {
#pragma unroll
      for (int st = 0; st < NS - 1; ++st) issue_at(f[st], st);
      for (; pj + 2 * NS - 1 <= npairs; pj += NS) {
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          issue_at(f[(st + NS - 1) % NS], pj + st + NS - 1);
          compute(f[st], pj + st);
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
      compute(f[k % NS], pj + k);
    }
  }

  // acc[ct][dt][e] = O^T[d = 16*dt + 4*gq + e][row 16*ct + c]
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const float l = sum_over_groups(l_run[ct]);
    if (!rvalid[ct]) continue;
    if (sp.n == 1) {
      const float inv = 1.f / l;
      uint16_t* o = out + orow[ct] * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<uint2*>(o + 16 * dt + 4 * gq) =
            make_uint2(pack_bf16x2(acc[ct][dt][0] * inv, acc[ct][dt][1] * inv),
                       pack_bf16x2(acc[ct][dt][2] * inv, acc[ct][dt][3] * inv));
    } else {
      const int64_t slot = orow[ct] * sp.n + s;
      float* po = sp.part_o + slot * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<f32x4*>(po + 16 * dt + 4 * gq) = acc[ct][dt];
      if (gq == 0)
        *reinterpret_cast<float2*>(sp.part_ml + slot * 2) =
            make_float2(m_run[ct] == -INFINITY ? -INFINITY : m_run[ct] * qk_scale, l);
    }
  }
}

template <int D, int G, bool FP8>
void launch_prefill(dim3 grid, size_t lds, ProfScope& ps, const char* kp, const char* vp,
                    const uint16_t* q, uint16_t* out, ChunkBatch cb, const int32_t* tables,
                    int64_t layer_off, int N, int Hkv, int Hq, int max_blocks, int n_tiles,
                    float qk_scale, PfSplit sp) {
  PA_TIMED_LAUNCH(ps, (prefill_mfma_kernel<D, G, FP8>), grid, dim3(256), lds, ps.st, kp, vp, q, out,
                  cb, tables, layer_off, N, Hkv, Hq, max_blocks, n_tiles, qk_scale, sp);
}

template <int D, bool FP8>
bool launch_prefill_g(int G, dim3 grid, size_t lds, ProfScope& ps, const char* kp,
                      const char* vp, const uint16_t* q, uint16_t* out, ChunkBatch cb,
                      const int32_t* tables, int64_t layer_off, int N, int Hkv, int Hq,
                      int max_blocks, int n_tiles, float qk_scale, PfSplit sp) {
#define PA_PF_CASE(GG)                                                                     \
  case GG:                                                                                \
    launch_prefill<D, GG, FP8>(grid, lds, ps, kp, vp, q, out, cb, tables, layer_off, N, Hkv,  \
                               Hq, max_blocks, n_tiles, qk_scale, sp);                     \
    return true;
  switch (G) {
    PA_PF_CASE(1)
    PA_PF_CASE(2)
    PA_PF_CASE(4)
    PA_PF_CASE(8)
    PA_PF_CASE(16)
    PA_PF_CASE(32)
    default:
      return false;
  }
#undef PA_PF_CASE
}

// Splits for a launch of `items` tiles whose longest walk is max_pairs pairs: as
// many as bring the grid to two resident work groups per CU, at least
// kPfMinPairsPerSplit pairs each.
int auto_splits(int64_t items, int max_pairs) {
  if (items >= kPfTargetWgs) return 1;
  int s = (int)((kPfTargetWgs + items - 1) / items);
  s = std::min(s, std::max(1, max_pairs / kPfMinPairsPerSplit));
  return std::max(1, std::min(s, kPfAutoMaxSplits));
}

size_t split_bytes(int64_t n_tokens, int Hq, int D, int S) {
  return S > 1 ? (size_t)S * n_tokens * Hq * (D + 2) * sizeof(float) : 0;
}

// Short-chunk kernel: about one wave per SIMD once the batch is split (each
// wave pays two dependent load latencies at start, block ids then its first
// pair, so fewer, longer waves beat more, shorter ones), at least 16 blocks each.
constexpr int64_t kPfShortTargetWaves = 1024;
constexpr int64_t kPfShortMinBps = 16;

struct PfPlan {
  bool short_path;  // prefill_short_kernel, else prefill_mfma_kernel
  int CT;           // short: 16-column tiles of query rows (1 or 2)
  int S;            // splits of the keys
  int bps;          // short: blocks per split
  int n_tiles;      // tile kernel: 128-row tiles per (chunk, KV head)
};

// Launch shape of pa_prefill (arguments already checked). Chunks of at most 32
// query rows per KV head take the short kernel when their keys fit in at most
// kPfMaxSplits splits of kMfmaMaxBps blocks (with n_splits > 0: exactly that many
// splits); everything else takes the tile kernel.
PfPlan pf_plan(int n_seqs, int Hkv, int G, int max_q_len, int max_ctx, int n_splits, bool fp8) {
  PfPlan p{};
  const int64_t maxb = ((int64_t)max_ctx + 15) / 16;
  if ((int64_t)G * max_q_len <= 32 && maxb > 0) {
    int64_t S, bps;
    if (n_splits > 0) {
      S = n_splits;
      bps = (maxb + S - 1) / S;
    } else {
      const int64_t units = (int64_t)n_seqs * Hkv;
      const int64_t want = units >= kPfShortTargetWaves ? 1 : (kPfShortTargetWaves + units - 1) / units;
      bps = std::max(kPfShortMinBps, (maxb + want - 1) / want);
      bps = std::min<int64_t>(bps + (bps & 1), kMfmaMaxBps);
      S = (maxb + bps - 1) / bps;
    }
    bps = std::max<int64_t>(2, bps + (bps & 1));  // pairs never straddle two splits
    if (bps <= kMfmaMaxBps && S <= kPfMaxSplits) {
      p.short_path = true;
      p.CT = G * max_q_len <= 16 ? 1 : 2;
      p.S = (int)S;
      p.bps = (int)bps;
      return p;
    }
  }
  const int TQ = kPfRows / G;
  p.n_tiles = (max_q_len + TQ - 1) / TQ;
  const int64_t tiles = (int64_t)n_seqs * Hkv * p.n_tiles;
  const int max_pairs = (int)((maxb + 1) / 2);
  p.S = n_splits == 0 ? auto_splits(tiles, max_pairs) : n_splits;
  return p;
}

// The tile kernel without splits: what an automatic choice falls back to when
// the caller's workspace cannot hold the partials.
PfPlan pf_plan_unsplit(int G, int max_q_len) {
  PfPlan p{};
  const int TQ = kPfRows / G;
  p.n_tiles = (max_q_len + TQ - 1) / TQ;
  p.S = 1;
  return p;
}

// Argument checks shared by pa_prefill and pa_prefill_workspace_bytes.
pa_status pf_check(const pa_geom* g, int32_t n_seqs, int32_t n_tokens, int32_t n_q_heads,
                   int32_t max_q_len, int32_t max_context_len, int32_t n_splits) {
  if (!geom_ok(g) || n_seqs < 0 || n_tokens < 0 || n_q_heads <= 0 || max_q_len < 0 ||
      max_context_len < 0 || n_splits < 0 || n_splits > kPfMaxSplits)
    return PA_ERR_INVALID_ARG;
  const int B = g->block_size, D = g->head_dim, Hkv = g->num_kv_heads;
  if (n_q_heads % Hkv != 0 || max_q_len > max_context_len) return PA_ERR_INVALID_ARG;
  const int G = n_q_heads / Hkv;
  if ((g->dtype != PA_BF16 && g->dtype != PA_FP8) || B != 16 || (D != 64 && D != 128) || G > 32 ||
      32 % G != 0)
    return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

}  // namespace

extern "C" {

size_t pa_prefill_workspace_bytes(const pa_geom* g, int32_t n_seqs, int32_t n_tokens,
                                  int32_t n_q_heads, int32_t max_q_len, int32_t max_context_len,
                                  int32_t n_splits) {
  if (pf_check(g, n_seqs, n_tokens, n_q_heads, max_q_len, max_context_len, n_splits) != PA_OK)
    return 0;
  if (n_seqs == 0 || n_tokens == 0 || max_q_len == 0) return 0;
  const PfPlan p = pf_plan(n_seqs, g->num_kv_heads, n_q_heads / g->num_kv_heads, max_q_len,
                           max_context_len, n_splits, g->dtype == PA_FP8);
  return split_bytes(n_tokens, n_q_heads, g->head_dim, p.S);
}

pa_status pa_prefill(const pa_geom* g, void* k_pool, void* v_pool, int32_t layer, const void* q,
                     const void* k_new, const void* v_new, void* out, int32_t n_seqs,
                     int32_t n_tokens, int32_t n_q_heads, const int32_t* q_start,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* ctx_lens, int32_t max_q_len, int32_t max_context_len,
                     float scale, int32_t n_splits, void* workspace, size_t workspace_bytes,
                     void* stream) {
  {
    const pa_status st =
        pf_check(g, n_seqs, n_tokens, n_q_heads, max_q_len, max_context_len, n_splits);
    if (st == PA_ERR_INVALID_ARG) return st;
    if (layer < 0 || layer >= g->num_layers || max_blocks_per_seq < 0) return PA_ERR_INVALID_ARG;
    if ((int64_t)max_blocks_per_seq * g->block_size < max_context_len) return PA_ERR_INVALID_ARG;
    if (st != PA_OK) return st;
  }
  const int B = g->block_size, D = g->head_dim, Hkv = g->num_kv_heads;
  const int G = n_q_heads / Hkv;
  const bool fp8 = g->dtype == PA_FP8;
  if (n_seqs == 0 || n_tokens == 0 || max_q_len == 0) return PA_OK;
  if (!k_pool || !v_pool || !q || !k_new || !v_new || !out || !q_start || !block_tables || !ctx_lens)
    return PA_ERR_INVALID_ARG;
  PfPlan plan = pf_plan(n_seqs, Hkv, G, max_q_len, max_context_len, n_splits, fp8);
  if (plan.S > 1 && (!workspace || workspace_bytes < split_bytes(n_tokens, n_q_heads, D, plan.S))) {
    if (n_splits != 0) return PA_ERR_WORKSPACE;
    plan = pf_plan_unsplit(G, max_q_len);  // automatic choice without room for partials
  }
  const int S = plan.S;
  hipStream_t st = (hipStream_t)stream;
  const int64_t tile_b = fp8 ? (int64_t)B * D + B : (int64_t)B * D * 2;  // bytes per pool tile
  const int64_t layer_off = (int64_t)layer * g->num_blocks * Hkv * tile_b;   // bytes
  if (Hkv * tile_b > UINT32_MAX) return PA_ERR_UNSUPPORTED;  // a block's stride: 32-bit products
  const ChunkBatch cb{q_start, ctx_lens, n_seqs, n_tokens, max_q_len, max_context_len};

  if (fp8) {  // the chunks' rows are quantized into their positions (one wave per row and head)
    ProfScope ps("prefill_append", st);
    const SlotsFromTables src{cb, block_tables, max_blocks_per_seq, B, g->num_blocks};
    if (!launch_append_fp8(st, (uint8_t*)k_pool, (uint8_t*)v_pool, (const uint16_t*)k_new,
                           (const uint16_t*)v_new, src, (int64_t)n_tokens, Hkv, D, B,
                           (int64_t)g->num_blocks * B, layer_off))
      return PA_ERR_UNSUPPORTED;
    if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  } else {  // the chunks' keys and values go to their positions through the block tables
    ProfScope ps("prefill_append", st, true, true);
    const int64_t items = ((int64_t)n_tokens + kAppendChunk - 1) / kAppendChunk * Hkv;
    const int64_t wgs = (items + kXcds - 1) / kXcds * kXcds;
    if (wgs > INT32_MAX) return PA_ERR_UNSUPPORTED;
    const SlotsFromTables src{cb, block_tables, max_blocks_per_seq, B, g->num_blocks};
    PA_TIMED_LAUNCH(ps, (append_kv_kernel<uint16_t, 8, SlotsFromTables>), dim3((unsigned)wgs),
                    dim3(256), append_lds_bytes<uint16_t>(D), st, (uint16_t*)k_pool,
                    (uint16_t*)v_pool, (const uint16_t*)k_new, (const uint16_t*)v_new, src,
                    n_tokens, Hkv, D, B, (int64_t)g->num_blocks * B, layer_off / 2);
    if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  }
  PfSplit sp{S, nullptr, nullptr};
  if (S > 1) {
    sp.part_o = static_cast<float*>(workspace);
    sp.part_ml = sp.part_o + (int64_t)n_tokens * n_q_heads * S * D;
  }
  {
    ProfScope ps(plan.short_path ? "prefill_short" : "prefill_attention", st, true, true);
    if (!(scale > 0.f)) scale = 1.f / std::sqrt((float)D);
    const float qk_scale = scale * kLog2e;
    const char* kp = static_cast<const char*>(k_pool);
    const char* vp = static_cast<const char*>(v_pool);
    const uint16_t* qq = static_cast<const uint16_t*>(q);
    uint16_t* oo = static_cast<uint16_t*>(out);
    if (plan.short_path) {
      const int64_t waves = (int64_t)n_seqs * Hkv * S;
      if (waves > INT32_MAX) return PA_ERR_UNSUPPORTED;
      const dim3 grid((unsigned)waves);
#define PA_PF_SHORT(DD, CC, F8)                                                                  \
  PA_TIMED_LAUNCH(ps, (prefill_short_kernel<DD, CC, F8>), grid, dim3(64), 0, st, kp, vp, qq, oo,  \
                     cb, block_tables, layer_off, g->num_blocks, Hkv, n_q_heads, G,              \
                     max_blocks_per_seq, plan.bps, qk_scale, sp)
#define PA_PF_SHORT_D(DD, F8)          \
  if (plan.CT == 1) PA_PF_SHORT(DD, 1, F8); \
  else PA_PF_SHORT(DD, 2, F8);
      if (fp8) {
        if (D == 64) { PA_PF_SHORT_D(64, true) } else { PA_PF_SHORT_D(128, true) }
      } else {
        if (D == 64) { PA_PF_SHORT_D(64, false) } else { PA_PF_SHORT_D(128, false) }
      }
#undef PA_PF_SHORT_D
#undef PA_PF_SHORT
    } else {
      // each XCD gets ceil(groups / 8) (chunk, KV head) groups of n_tiles x S items
      const int64_t groups = (int64_t)n_seqs * Hkv;
      const int64_t wgs = kXcds * ((groups + kXcds - 1) / kXcds) * plan.n_tiles * S;
      if (wgs > INT32_MAX) return PA_ERR_UNSUPPORTED;
      const dim3 grid((unsigned)wgs);
      const size_t lds = 3 * (size_t)(D == 64 ? PfCfg<64>::PAIR_BYTES : PfCfg<128>::PAIR_BYTES);
#define PA_PF_LAUNCH(DD, F8)                                                                  \
  launch_prefill_g<DD, F8>(G, grid, lds, ps, kp, vp, qq, oo, cb, block_tables, layer_off,     \
                           g->num_blocks, Hkv, n_q_heads, max_blocks_per_seq, plan.n_tiles,   \
                           qk_scale, sp)
      const bool ok = D == 64 ? (fp8 ? PA_PF_LAUNCH(64, true) : PA_PF_LAUNCH(64, false))
                              : (fp8 ? PA_PF_LAUNCH(128, true) : PA_PF_LAUNCH(128, false));
#undef PA_PF_LAUNCH
      if (!ok) return PA_ERR_UNSUPPORTED;
    }
    if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  }
  if (S > 1) {
    ProfScope ps("prefill_combine", st, true, true);
    const int64_t rows = (int64_t)n_tokens * n_q_heads;
    const int rows_per_wg = 1024 / D;
    const int64_t wgs = (rows + rows_per_wg - 1) / rows_per_wg;
    if (wgs > INT32_MAX) return PA_ERR_UNSUPPORTED;
    if (D == 64)
      PA_TIMED_LAUNCH(ps, (prefill_combine_kernel<64>), dim3((unsigned)wgs), dim3(256), 0, st,
                         sp.part_o, sp.part_ml, (uint16_t*)out, rows, S);
    else
      PA_TIMED_LAUNCH(ps, (prefill_combine_kernel<128>), dim3((unsigned)wgs), dim3(256), 0, st,
                         sp.part_o, sp.part_ml, (uint16_t*)out, rows, S);
    if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  }
  return PA_OK;
}

}  // extern "C"
