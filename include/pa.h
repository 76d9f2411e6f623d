/*
 * pa.h -- C interface of libpa, paged-KV attention decode for AMD MI355X (gfx950).
 *
 * What the library computes, and where the pages define it:
 *   - KV footprint: "KV Cache Management", section "From Context Tokens to KV
 *     State", Eq. (1), and section "The PagedAttention virtual memory model"
 *     (block bytes, blocks per prompt); per-rank form with tensor parallelism:
 *     "EfficientAgent: What Makes KV Cache Offloading Work for Concurrent
 *     Agents?", section "KV footprint and hardware balance", Eq. (1).
 *   - Block tables and slot-mapped writes: "KV Cache Management", section "The
 *     PagedAttention virtual memory model" (l = floor(t/B), o = t mod B, T[l] = p).
 *   - Paged decode attention: same page, same section (the kernel takes the
 *     block table as an input and walks logical blocks 0..floor((S-1)/B)), with
 *     the online softmax of section "Chunked prefill mechanics".
 *   - Reference counts, fork, copy-on-write, release: same page, section
 *     "Zero-copy deliberation via copy-on-write branching"; error behaviour from
 *     "PagedAttention" (Inference book, ch. 14), sections "It is the same
 *     function" and "Inference Lab increment".
 *   - Block gather/scatter and the host copy: "KV Cache Management", section
 *     "Asynchronous paged swapping".
 *   - One-byte (FP8) storage: b_elem = 1 in Eq. (1) of "KV Cache Management",
 *     section "From Context Tokens to KV State". The pages name no format or
 *     scale; the library uses OCP FP8 E4M3 elements with one power-of-two scale
 *     per (token, KV head) for K and for V (see PA_FP8 below).
 *
 * ---------------------------------------------------------------------------
 * Memory layout (fixed by this interface)
 * ---------------------------------------------------------------------------
 * A pool is two device arrays of the geometry's element type (fp32 or bf16):
 *   K pool [L][N][H_kv][d/W][B][W]  element (layer, block, head, slot o, dim j) at
 *                                   chunk j/W, slot o, position j%W; W = 32 when 32
 *                                   divides d, else W = d (i.e. [L][N][H_kv][B][d])
 *   V pool [L][N][H_kv][d][B]        element (layer, block, head, dim, slot offset)
 * Each (layer, block, head) is one contiguous run of B*d elements in both. The
 * 32-wide dimension chunks of K make every K load of the decode kernel cover
 * whole 128-byte lines; V's dimension-major runs give 8 consecutive slots of one
 * dimension per 16-byte load.
 * A slot is block * B + offset. A block table is int32 [n_seqs][max_blocks]
 * (row-major); entry j of row i is the physical block of sequence i's logical
 * block j. context_lens[i] is the number of tokens sequence i attends to.
 * Staging (gather/scatter): for the i-th listed block, bytes_per_block bytes
 * laid out [L][2][run]: that layer's K run of the block, then its V run, each
 * exactly as stored in the pool.
 * FP8 pools (PA_FP8) are bytes [L][N][H_kv][B*d + B]: each (layer, block, head)
 * tile holds the B*d element codes followed by B scale bytes, one per slot in
 * slot order. Code of slot o, dimension j: K, when B = 16 and 64 divides d, at
 * 1024*(j/64) + 64*r(o) + 16*((j/8)%4) + 8*((j/32)%2) + j%8 with r(o) = o with
 * bits 2 and 3 swapped (rows of 64 codes, slots 0-3, 8-11, 4-7, 12-15, a row's
 * 8-dimension groups in the order 0, 4, 1, 5, 2, 6, 3, 7), else in the bf16 order above
 * ((j/W)*B*W + o*W + j%W); V, when B = 16 and 32 divides d, at 512*(j/32) +
 * 256*(o/8) + 16*(j%16) + 8*((j/16)%2) + o%8, else at j*B + o. (The decode
 * kernel's lanes then read 16 contiguous bytes each, 512 per block and
 * instruction.) A slot's d values x
 * (one token of one head) are stored as codes c_j = E4M3(x_j * 2^-e), rounded
 * to nearest with ties to the even code, and the byte e + 127, where e is the
 * smallest integer with max_j |x_j| <= 448 * 2^e (clamped to [-127, 127]; e = 0
 * when all x_j are 0); the stored values are E4M3(c_j) * 2^e. Queries, outputs
 * and new K/V rows of an FP8 pool are bf16.
 *
 * ---------------------------------------------------------------------------
 * Conventions
 * ---------------------------------------------------------------------------
 * Ownership: the caller allocates and owns every device and host buffer; no
 *   entry point allocates device or pinned memory. Decode split partials live
 *   in a caller-provided workspace (size from pa_decode_workspace_bytes); the
 *   swapper works in caller buffers sized by pa_swapper_buffer_bytes.
 * Streams: `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   Device entry points only enqueue work and return; results are visible after
 *   the caller synchronises the stream.
 * Errors: every entry point returns pa_status. Arguments and geometry are
 *   checked on the host before anything is launched; a launch failure returns
 *   PA_ERR_HIP. Block manager calls that fail leave the manager unchanged.
 * Device-side preconditions (not checked on the host): block ids in tables and
 *   id lists lie in [0, N); slots lie in [0, N*B) or are negative (skip);
 *   context_lens[i] <= max_context_len <= max_blocks_per_seq * B. Kernels guard
 *   their own memory accesses against out-of-range ids and lengths (an
 *   out-of-range slot is skipped, an out-of-range block id is read as block 0,
 *   a length is clamped), so bad indices give wrong numbers, never a fault.
 * Dtypes: q, out and both pools share one dtype (bf16 for q, out and new rows
 *   of an FP8 pool); arithmetic is fp32.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1,   /* bad pointer, size, index or geometry           */
  PA_ERR_OUT_OF_BLOCKS = -2, /* the free list cannot satisfy the request        */
  PA_ERR_DOUBLE_FREE = -3,   /* dropping a reference that does not exist        */
  PA_ERR_NOT_FOUND = -4,     /* unknown sequence id                             */
  PA_ERR_HIP = -5,           /* a HIP runtime call or launch failed             */
  PA_ERR_WORKSPACE = -6,     /* decode workspace too small                      */
  PA_ERR_UNSUPPORTED = -7,   /* geometry outside what the kernels implement     */
  PA_ERR_OUT_OF_FRAMES = -8  /* the host frame pool has no free run long enough  */
} pa_status;

/* PA_FP8: E4M3 codes with per-(token, head) power-of-two scales (layout above). */
typedef enum { PA_F32 = 0, PA_BF16 = 1, PA_FP8 = 2 } pa_dtype;

/* Pool geometry: L layers, H_kv KV heads of dimension d, blocks of B slots,
 * N physical blocks, element type dtype (a pa_dtype value). */
typedef struct {
  int32_t num_layers;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t num_blocks;
  int32_t dtype;
} pa_geom;

const char* pa_status_str(int32_t status);
int32_t pa_version(void);

/* ---------------------------------------------------------------- footprint */

/* Bytes of K and V one token occupies on one rank: 2*L*d*b*max(1, ceil(H_kv/tp)).
 * tp == 1 gives Eq. (1) of "KV Cache Management". Returns -1 on bad input. */
int64_t pa_bytes_per_token(int32_t num_layers, int32_t num_kv_heads, int32_t head_dim,
                           int32_t elem_bytes, int32_t tp);
/* M_block = 2*L*H_kv*B*d*b ("The PagedAttention virtual memory model"), plus for
 * FP8 pools the 2*L*H_kv*B scale bytes; -1 on bad geometry. */
int64_t pa_bytes_per_block(const pa_geom* g);
/* ceil(tokens / block_size); -1 on bad input. */
int64_t pa_blocks_for_tokens(int64_t tokens, int32_t block_size);
/* Bytes of one pool array (K or V): L*N*H_kv*B*d*b (+ L*N*H_kv*B scale bytes
 * for FP8); -1 on bad geometry. */
int64_t pa_pool_bytes(const pa_geom* g);

/* ------------------------------------------------------------ device entry points */

/* Slot-mapped write of new keys and values into one layer.
 * k_new, v_new: [n_tokens][H_kv][d] device arrays. slot_mapping: int64 [n_tokens]
 * device array; token j goes to block slot/B, offset slot%B; a negative slot
 * skips the token; slots must be distinct. Source: "KV Cache Management", "The PagedAttention virtual
 * memory model" (write into T[l] at offset o); "PagedAttention", "The real cache". */
pa_status pa_append_kv(const pa_geom* g, void* k_pool, void* v_pool, int32_t layer,
                       const void* k_new, const void* v_new, const int64_t* slot_mapping,
                       int32_t n_tokens, void* stream);

/* Decode tuning; pass NULL for the defaults. */
typedef struct {
  int32_t blocks_per_split; /* logical blocks per split-K work item (0 = choose; rounded up to even) */
  int32_t kernel;           /* 0 = choose, 1 = generic kernel (LDS-staged, any B <= 64, d <= 256),
                               2 = MFMA kernel (bf16 or FP8 pools, B = 16), 3 = streaming VALU
                               kernel (fp32 or bf16 pools, B = 16, d in {64, 128}, 1, 2 or 4
                               query heads per KV head, or 8 with d = 128); the choice takes
                               MFMA, then the streaming VALU kernel, then the generic one */
  int32_t kv_reuse;         /* 0: each K/V block is read once per step -> stream it past the
                               caches (non-temporal loads); 1: blocks are shared by many
                               sequences of the batch (forks, common prefixes) -> ordinary
                               loads so repeats hit in L2 / Infinity Cache (MFMA kernel) */
  int32_t merge;            /* 0: split partials are merged by a second launch; 1: merged inside
                               the decode launch by the last split of each (sequence, KV head) to
                               finish (MFMA and streaming VALU kernels; the generic kernel keeps
                               the second launch). The workspace then ends with one int32 counter per
                               (sequence, KV head), which must be zero before the workspace's
                               first such call (allocate it zeroed); every call leaves them zero.
                               Two calls sharing a workspace must not overlap. */
  const int32_t* host_context_lens; /* optional host copy of context_lens ([n_seqs], equal to
                               the device array; NULL = not given). With it the MFMA bf16
                               kernel takes a ragged plan when the lengths are uneven (the
                               longest above 1.5x the mean): only sequences longer than an item
                               size cut into items, the items listed longest first (with
                               blocks_per_split > 0, that item size and the list always). A host
                               copy shorter than the device lengths leaves outputs incomplete. */
  int32_t waves_per_group;  /* streaming VALU kernel: waves per workgroup, which split the
                               workgroup's blocks and merge in LDS (0 = choose: 2; capped at 16
                               for one query head per KV head with 256-byte rows, else 8) */
} pa_decode_opts;

/* Workspace bytes pa_decode needs for these sizes and options (0 when the
 * chosen plan writes the output directly). Returns 0 also for invalid input;
 * pa_decode reports the error. */
size_t pa_decode_workspace_bytes(const pa_geom* g, int32_t n_seqs, int32_t n_q_heads,
                                 int32_t max_context_len, const pa_decode_opts* opts);

/* Ragged-batch GQA decode over block tables, one layer.
 * q, out: [n_seqs][n_q_heads][d] device arrays (pool dtype). Query head h reads
 * KV head h / (n_q_heads / H_kv). For sequence i, out[i][h] =
 * sum_t softmax_t(scale * q[i][h] . K_t) V_t over its first context_lens[i]
 * tokens, read through block_tables row i. scale <= 0 means 1/sqrt(d).
 * context_lens[i] == 0 writes zeros. max_context_len bounds every
 * context_lens[i] (lengths above it are clamped) and sizes the launch. Splits
 * the keys into runs of blocks_per_split blocks processed in parallel and merges
 * them with the online-softmax rule of "Chunked prefill mechanics". Results do
 * not depend on which physical blocks hold the data. */
pa_status pa_decode(const pa_geom* g, const void* k_pool, const void* v_pool, int32_t layer,
                    const void* q, void* out, int32_t n_seqs, int32_t n_q_heads,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t max_context_len, float scale,
                    const pa_decode_opts* opts, void* workspace, size_t workspace_bytes,
                    void* stream);

/* One decode step's append and decode, fused: for each sequence i, the new
 * token's key and value (k_new[i], v_new[i], [n_seqs][H_kv][d] device arrays)
 * are written at position context_lens[i] - 1, i.e. into block
 * block_tables[i][(len-1)/B] at offset (len-1)%B, and then out is computed as
 * pa_decode computes it over the first context_lens[i] tokens, that one
 * included. The pool afterwards holds exactly what pa_append_kv with
 * slot = table[(len-1)/B]*B + (len-1)%B followed by pa_decode leaves. The
 * block holding position len-1 must be owned by sequence i alone (a shared tail
 * block is copied first, by copy-on-write) and context_lens[i] == 0 writes
 * nothing. Source: "KV Cache Management", "The PagedAttention virtual memory
 * model" (a step writes its token at offset o of its current block, then
 * attends over the table); "PagedAttention", "The real cache". */
pa_status pa_decode_append(const pa_geom* g, void* k_pool, void* v_pool, int32_t layer,
                           const void* q, const void* k_new, const void* v_new, void* out,
                           int32_t n_seqs, int32_t n_q_heads, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t max_context_len, float scale, const pa_decode_opts* opts,
                           void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation: the same
 * decode step as pa_decode_append, with the split partials in a file-scope
 * device array of the library (16 MiB = 16777216 bytes per GPU, held until the
 * process ends) instead of a caller workspace. It allocates nothing and records
 * no timing events; the partials are merged by the combine launch (opts->merge
 * is ignored). A launch plan whose partials need more than 16 MiB (see
 * pa_decode_workspace_bytes with merge = 0) returns PA_ERR_WORKSPACE before
 * anything is launched. Every call on one GPU shares that GPU's array: calls
 * that overlap on one GPU (other streams, other threads) race and must not be
 * issued. */
pa_status pa_decode_append_noalloc(const pa_geom* g, void* k_pool, void* v_pool, int32_t layer,
                                   const void* q, const void* k_new, const void* v_new, void* out,
                                   int32_t n_seqs, int32_t n_q_heads, const int32_t* block_tables,
                                   int32_t max_blocks_per_seq, const int32_t* context_lens,
                                   int32_t max_context_len, float scale,
                                   const pa_decode_opts* opts, void* stream);

/* Chunked-prefill (multi-query) paged attention, one layer. Source: "KV Cache
 * Management", section "Chunked prefill mechanics": the queries of a chunk
 * attend over every cached token of their sequence and, inside the chunk, over
 * the tokens at or before their own position; the chunk's keys and values are
 * written into the sequence's paged blocks.
 * Batch of n_seqs chunks packed by rows: chunk i owns rows q_start[i] ..
 * q_start[i+1]-1 (q_start: int32 [n_seqs+1] device array, non-decreasing, last
 * entry n_tokens) of q, out [n_tokens][n_q_heads][d] and k_new, v_new
 * [n_tokens][H_kv][d] (pool dtype). ctx_lens[i] (int32 device) tokens of sequence
 * i are already cached; the chunk's row r is position ctx_lens[i] + r - q_start[i].
 * block_tables row i ([n_seqs][max_blocks_per_seq] int32 device) must already
 * cover ctx_lens[i] + chunk length tokens (the blocks the chunk is written into
 * must be owned by sequence i alone). The call first writes each row's K/V at
 * its position, then out[row][h] = sum over visible positions t of
 * softmax_t(scale * q . K_t) V_t, KV head h / (n_q_heads / H_kv), visible = 0 ..
 * the row's own position. max_q_len bounds every chunk length and sizes the
 * launch; max_context_len bounds ctx_lens[i] + chunk length (values are clamped
 * to these bounds, never read past them). scale <= 0 means 1/sqrt(d).
 * Implemented for bf16 and FP8 (E4M3, per-token scales) pools with B = 16,
 * d in {64, 128} and n_q_heads / H_kv dividing 32; other geometries return
 * PA_ERR_UNSUPPORTED.
 * Splits: the visible keys of each group of query rows may be cut into n_splits
 * ranges processed in parallel, whose partial results (unnormalised output,
 * maximum, sum) go to the caller's workspace and are merged by the same
 * online-softmax rule (section "Chunked prefill mechanics"). n_splits = 1: no
 * split, no workspace; 2..64: that many (PA_ERR_WORKSPACE if workspace_bytes is
 * below pa_prefill_workspace_bytes for the same arguments); 0: chosen from the
 * launch shape, falling back to no split when the workspace is missing or too
 * small. Short chunks on bf16 pools (n_q_heads / H_kv x max_q_len <= 32, e.g. a
 * few draft tokens per sequence) are computed one wave per (chunk, KV head,
 * split), the automatic choice splitting long histories into up to 64 ranges of
 * at most 256 blocks; longer chunks in 128-row tiles with up to 4 splits. */
pa_status pa_prefill(const pa_geom* g, void* k_pool, void* v_pool, int32_t layer, const void* q,
                     const void* k_new, const void* v_new, void* out, int32_t n_seqs,
                     int32_t n_tokens, int32_t n_q_heads, const int32_t* q_start,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* ctx_lens, int32_t max_q_len, int32_t max_context_len,
                     float scale, int32_t n_splits, void* workspace, size_t workspace_bytes,
                     void* stream);
/* Device workspace bytes pa_prefill needs when called with these arguments (0:
 * none; also 0 for bad or unsupported arguments). The automatic choice
 * (n_splits 0) uses exactly this much when given it. */
size_t pa_prefill_workspace_bytes(const pa_geom* g, int32_t n_seqs, int32_t n_tokens,
                                  int32_t n_q_heads, int32_t max_q_len, int32_t max_context_len,
                                  int32_t n_splits);

/* Copy-on-write block copy: for each k, block dst[k] <- block src[k] in every
 * layer, K and V, all B slots. src, dst: int32 [n_pairs] device arrays; no dst
 * may appear as a src or twice. Source: "KV Cache Management", "Zero-copy
 * deliberation via copy-on-write branching". */
pa_status pa_copy_blocks(const pa_geom* g, void* k_pool, void* v_pool, const int32_t* src,
                         const int32_t* dst, int32_t n_pairs, void* stream);

/* staging[i] <- block block_ids[i] (the staging layout above; n * bytes_per_block
 * bytes). block_ids: int32 [n] device array. Source: "Asynchronous paged swapping". */
pa_status pa_gather_blocks(const pa_geom* g, const void* k_pool, const void* v_pool,
                           const int32_t* block_ids, int32_t n, void* staging, void* stream);

/* block block_ids[i] <- staging[i]; the inverse of pa_gather_blocks. Ids must be distinct. */
pa_status pa_scatter_blocks(const pa_geom* g, void* k_pool, void* v_pool, const void* staging,
                            const int32_t* block_ids, int32_t n, void* stream);

/* Asynchronous copies over the host link (hipMemcpyAsync). host buffers should
 * be pinned (page-locked) for the copy to be asynchronous and run at link speed. */
pa_status pa_copy_to_host(void* host_dst, const void* device_src, size_t bytes, void* stream);
pa_status pa_copy_to_device(void* device_dst, const void* host_src, size_t bytes, void* stream);

/* ---------------------------------------------------------------- timing */

/* When enabled, the library records a hipEvent pair on the launch stream around
 * each kernel it launches and accumulates per-kernel durations. Kernel names:
 * "append", "decode_partial", "decode_combine", "copy_blocks", "gather", "scatter".
 * pa_prof_read synchronises the recorded events. */
pa_status pa_prof_enable(int32_t on);
pa_status pa_prof_reset(void);
pa_status pa_prof_read(const char* kernel, int64_t* launches, double* total_ms);

/* ---------------------------------------------------------------- block manager */
/* Host-only state: a FIFO free list of block ids (initial order given by the
 * caller, NULL = 0..N-1), a reference count per block and a block table and
 * length per sequence. Appends allocate at block boundaries; a write into a
 * partly filled block whose count is above 1 first takes a fresh block and
 * reports a (src, dst) copy for pa_copy_blocks. Every call checks its
 * preconditions before changing anything. Every call takes the manager's
 * mutex, so calls from several threads (e.g. the completion steps of
 * asynchronous migrations, run on a HIP host-function thread) are serialised. */
typedef struct pa_bm pa_bm;

pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                       pa_bm** out);
void pa_bm_destroy(pa_bm* bm);
int32_t pa_bm_num_free(const pa_bm* bm);
/* Tokens per block, -1 for NULL. */
int32_t pa_bm_block_size(const pa_bm* bm);
/* Reference count of a block, -1 if the id is out of range. */
int32_t pa_bm_refcount(const pa_bm* bm, int32_t block);

/* Raw allocator: take n blocks (count 1), all or none. */
pa_status pa_bm_alloc(pa_bm* bm, int32_t n, int32_t* ids_out);
/* The free queue front to back: the first min(cap, size) ids go to ids_out,
 * *n_out gets the queue length. */
pa_status pa_bm_free_list(const pa_bm* bm, int32_t* ids_out, int32_t cap, int32_t* n_out);
/* One more reference to each listed (allocated) block. */
pa_status pa_bm_incref(pa_bm* bm, const int32_t* ids, int32_t n);
/* Drop one reference from each listed block; a block reaching 0 returns to the
 * back of the free list. PA_ERR_DOUBLE_FREE if a block has no reference left. */
pa_status pa_bm_free_blocks(pa_bm* bm, const int32_t* ids, int32_t n);

pa_status pa_bm_seq_new(pa_bm* bm, int32_t* seq_out);
/* New sequence whose table is the n listed (allocated) blocks, each gaining a
 * reference, and whose length is n * block_size: a request that hit a cached
 * prefix starts from its full blocks ("KV Cache Management", section "Prefix
 * Caching Across Turns", block-aligned truncation). n may be 0. */
pa_status pa_bm_seq_from_blocks(pa_bm* bm, const int32_t* ids, int32_t n, int32_t* seq_out);
/* Child gets a copy of the parent's table and length; every block gains a reference. */
pa_status pa_bm_seq_fork(pa_bm* bm, int32_t parent, int32_t* child_out);
/* Reserve n_tokens more positions. slots_out (may be NULL) receives n_tokens
 * int64 slots; *n_cow_out is 0 or 1 and, when 1, cow_src_out[0]/cow_dst_out[0]
 * name the block copy that must precede the write. */
pa_status pa_bm_seq_append(pa_bm* bm, int32_t seq, int32_t n_tokens, int64_t* slots_out,
                           int32_t* cow_src_out, int32_t* cow_dst_out, int32_t* n_cow_out);
/* Append counts[k] tokens to seqs[k] for every k, all or nothing. slots_out
 * receives sum(counts) slots in order; cow arrays need room for n entries. */
pa_status pa_bm_append_batch(pa_bm* bm, const int32_t* seqs, const int32_t* counts, int32_t n,
                             int64_t* slots_out, int32_t* cow_src_out, int32_t* cow_dst_out,
                             int32_t* n_cow_out);
/* Drop a reference to every block of the table; blocks reaching 0 are freed. */
pa_status pa_bm_seq_release(pa_bm* bm, int32_t seq);
/* Swap-out: drop the sequence's reference to the listed logical blocks and mark
 * them not resident (-1 in the table); phys_out receives their physical ids. */
pa_status pa_bm_seq_swap_out(pa_bm* bm, int32_t seq, const int32_t* logical, int32_t n,
                             int32_t* phys_out);
/* Swap-in: give the listed non-resident logical blocks fresh physical blocks. */
pa_status pa_bm_seq_swap_in(pa_bm* bm, int32_t seq, const int32_t* logical, int32_t n,
                            int32_t* phys_out);
/* Reorder the free list: entry k becomes the current entry perm[k]. perm must be
 * a permutation of 0..n-1 with n == pa_bm_num_free(bm). Lets a caller hand out
 * freed frames in a fresh order (e.g. a seeded shuffle before a swap-in). */
pa_status pa_bm_permute_free(pa_bm* bm, const int32_t* perm, int32_t n);
pa_status pa_bm_seq_info(const pa_bm* bm, int32_t seq, int64_t* n_tokens, int32_t* n_blocks);
/* Copy the table (up to cap entries) into table_out; *n_blocks gets its length. */
pa_status pa_bm_seq_table(const pa_bm* bm, int32_t seq, int32_t* table_out, int32_t cap,
                          int32_t* n_blocks);
/* Decode-step tables for a batch: row k of tables_out ([n][max_blocks]) holds
 * seqs[k]'s table padded with `pad`; lens_out[k] its length. */
pa_status pa_bm_build_tables(const pa_bm* bm, const int32_t* seqs, int32_t n, int32_t max_blocks,
                             int32_t pad, int32_t* tables_out, int32_t* lens_out);
/* Check internal invariants: every count covers the table references to its
 * block (and the blocks reserved by swap-ins in flight), the free list holds
 * each zero-count block exactly once and nothing else, every table has
 * ceil(length / B) entries, and every used host frame is held by exactly one
 * host-tier or in-flight entry. PA_OK if consistent. */
pa_status pa_bm_validate(const pa_bm* bm);

/* ---------------------------------------------------------------- tiered residency */
/* Source: "KV Cache Management", section "Asynchronous paged swapping". Each
 * table entry carries a residency tag. A migration to the host takes a
 * contiguous run of frames from a pinned host pool at its start (step 1) while
 * the blocks stay allocated and readable; the copy runs in the background
 * (step 2); its completion retags the entries as host-resident with their frame
 * indices and pushes the vacated blocks to the back of the free queue (step 3).
 * The return path reserves fresh blocks at its start and, on completion, points
 * the entries at them and returns the frames to the pool. A sequence with a
 * migration in flight cannot be forked or released, and an append cannot write
 * into a tail block that is host-resident or in flight. Host-resident entries
 * read -1 in pa_bm_seq_table / pa_bm_build_tables. The manager holds only the
 * frame bookkeeping; the bytes live in the pinned buffer a pa_swapper moves them into. */
typedef enum {
  PA_TIER_HBM = 0,         /* resident in the device pool; index = block id           */
  PA_TIER_HOST = 1,        /* in host memory; index = host frame (-1: swapped out by
                              pa_bm_seq_swap_out, no frame of the pool)                */
  PA_TIER_PENDING_OUT = 2, /* copy to the host in flight; index = block id (still valid) */
  PA_TIER_PENDING_IN = 3   /* copy back in flight; index = host frame                  */
} pa_tier;

/* Give the manager a host pool of num_frames frames (frames 0..num_frames-1).
 * Runs are handed out first fit from the lowest frame; a freed run merges with
 * free neighbours. One pool per manager (PA_ERR_INVALID_ARG if one is attached). */
pa_status pa_bm_attach_host_pool(pa_bm* bm, int32_t num_frames);
/* Remove the host pool; PA_ERR_INVALID_ARG if none is attached or a frame is in
 * use (an entry is host-resident or in flight). */
pa_status pa_bm_detach_host_pool(pa_bm* bm);
/* Free frames of the attached pool, -1 without one. */
int32_t pa_bm_host_frames_free(const pa_bm* bm);
/* Free runs of the host pool in increasing start order (first min(cap, count)
 * into starts/lengths); *n_out gets the number of runs. */
pa_status pa_bm_host_free_runs(const pa_bm* bm, int32_t* starts, int32_t* lengths, int32_t cap,
                               int32_t* n_out);
/* Residency tag (a pa_tier value) and index of logical block `logical` of seq. */
pa_status pa_bm_block_tier(const pa_bm* bm, int32_t seq, int32_t logical, int32_t* tier,
                           int32_t* index);
/* Step 1 for the n listed logical blocks (distinct, all PA_TIER_HBM, n >= 1):
 * reserve frames first .. first+n-1 (logical[k] goes to frame first + k) and
 * mark the entries PA_TIER_PENDING_OUT. phys_out[k] receives the block to copy
 * from. PA_ERR_OUT_OF_FRAMES if no free run of n frames exists. */
pa_status pa_bm_swap_out_begin(pa_bm* bm, int32_t seq, const int32_t* logical, int32_t n,
                               int32_t* phys_out, int32_t* first_frame_out);
/* Step 3, after the copy has completed: the entries become PA_TIER_HOST and the
 * sequence's references to their blocks are dropped (a block reaching count 0
 * goes to the back of the free queue). Every entry must be PENDING_OUT. */
pa_status pa_bm_swap_out_finish(pa_bm* bm, int32_t seq, const int32_t* logical, int32_t n);
/* Return path: for PA_TIER_HOST entries holding a frame, take n fresh blocks
 * from the free queue (all or none: PA_ERR_OUT_OF_BLOCKS) and mark the entries
 * PA_TIER_PENDING_IN. phys_out[k] / frames_out[k]: destination block and
 * source frame of logical[k]. The table keeps -1 until the finish step. */
pa_status pa_bm_swap_in_begin(pa_bm* bm, int32_t seq, const int32_t* logical, int32_t n,
                              int32_t* phys_out, int32_t* frames_out);
/* After the copy back has completed: entries point at their new blocks
 * (PA_TIER_HBM) and their frames return to the pool. Every entry must be
 * PENDING_IN. */
pa_status pa_bm_swap_in_finish(pa_bm* bm, int32_t seq, const int32_t* logical, int32_t n);

/* ---------------------------------------------------------------- asynchronous swapper */
/* Moves blocks between the device pool and a pinned host frame pool in the
 * background, following "KV Cache Management", section "Asynchronous paged
 * swapping" (copy stream, pinned frames, completion callback that retags the
 * table) and its paragraph on the pipelined chunked reload. The caller owns the
 * memory: a page-locked host buffer of num_frames frames (frame f at byte
 * f * frame_bytes, one block in the staging layout of pa_gather_blocks) and a
 * device staging buffer split into two halves of chunk_blocks blocks. The
 * swapper creates only two streams of its own (default priority), one for the
 * gather / scatter kernels and one for the DMA copies, so that packing chunk
 * k+1 overlaps the copy of chunk k, and the events that hand the halves between
 * them. The kernels use a few work-groups only, paced to the host link. Chunks
 * of all migrations alternate between the two halves in issue order; the
 * completion step of each migration (pa_bm_swap_out_finish /
 * pa_bm_swap_in_finish) runs on the HIP runtime's host-function thread when its
 * last copy or kernel has finished. The block manager and both buffers must
 * outlive the swapper; one swapper per manager at a time. */
typedef struct pa_swapper pa_swapper;

/* Swapper tuning; pass NULL for the defaults. */
typedef struct {
  int32_t chunk_blocks; /* blocks per staging half (0 = about 64 MiB)                          */
  int32_t move_wgs;     /* work-groups per gather / scatter launch (0 = 512)                  */
  int32_t direct;       /* 1: no staging and no kernels; each block moves as two strided DMA
                           copies (K and V: L rows of one run each, the pool's layer pitch)
                           straight between the pool and its frame, on the DMA stream */
} pa_swap_opts;

/* Buffer sizes a swapper of num_frames frames with these options needs (either
 * output may be NULL): *host_bytes = num_frames * bytes_per_block of pinned host
 * memory, *staging_bytes = 2 * chunk_blocks * bytes_per_block of device memory
 * (0 in direct mode). PA_ERR_INVALID_ARG for bad input. */
pa_status pa_swapper_buffer_bytes(const pa_geom* g, int32_t num_frames, const pa_swap_opts* opts,
                                  size_t* host_bytes, size_t* staging_bytes);

/* k_pool, v_pool: the device pools of geometry g. host_frames: page-locked host
 * memory (hipHostMalloc, or a pinned torch tensor) of host_bytes bytes; staging:
 * device memory of staging_bytes bytes (may be NULL in direct mode). Attaches a
 * host pool of num_frames frames to bm (see pa_bm_attach_host_pool). Allocates
 * no memory. PA_ERR_WORKSPACE if a buffer is smaller than
 * pa_swapper_buffer_bytes says, PA_ERR_INVALID_ARG if host_frames is not
 * page-locked, PA_ERR_HIP if a stream or event cannot be created. */
pa_status pa_swapper_create(const pa_geom* g, pa_bm* bm, void* k_pool, void* v_pool,
                            int32_t num_frames, const pa_swap_opts* opts, void* host_frames,
                            size_t host_bytes, void* staging, size_t staging_bytes,
                            pa_swapper** out);
/* Waits for every migration (pa_swapper_sync), detaches the host pool from the
 * manager and frees the swapper's streams and events; the caller may then free
 * its two buffers. Refuses, changing nothing, while a frame is in use (an entry
 * is host-resident or in flight: bring it back or release its sequence first;
 * PA_ERR_INVALID_ARG) or while a completion step has not run after the wait
 * (PA_ERR_HIP); the swapper then stays usable. */
pa_status pa_swapper_destroy(pa_swapper* s);
/* Move the n listed logical blocks of seq to the host: pa_bm_swap_out_begin
 * now (errors from it are returned and nothing is queued), then per chunk a
 * gather kernel and one device-to-host copy into the reserved run of frames,
 * then the completion step. The copies are ordered after all work queued on
 * after_stream before this call (NULL: no ordering), so the kernels that wrote
 * these blocks must be queued there. The blocks stay readable by decode until
 * the completion step frees them; nothing may write them meanwhile. Returns
 * once the work is queued. A HIP failure after the reservation leaves the
 * entries in flight and makes every later call return PA_ERR_HIP. */
pa_status pa_swap_out_async(pa_swapper* s, int32_t seq, const int32_t* logical, int32_t n,
                            void* after_stream);
/* Bring the n listed host-tier blocks of seq back: pa_bm_swap_in_begin now
 * (fresh blocks from the front of the free queue), then per chunk one
 * host-to-device copy per run of consecutive frames and a scatter kernel into
 * the fresh blocks, then the completion step (table remapped, frames freed).
 * Ordered after after_stream as above: blocks freed before this call may still
 * be in use by kernels queued there. */
pa_status pa_swap_in_async(pa_swapper* s, int32_t seq, const int32_t* logical, int32_t n,
                           void* after_stream);
/* Make `stream` wait (on the device) for every copy and kernel queued so far. */
pa_status pa_swapper_fence(pa_swapper* s, void* stream);
/* Block the calling thread until every queued migration, completion step
 * included, has finished. Returns the first error a completion step reported. */
pa_status pa_swapper_sync(pa_swapper* s);
/* Migrations whose completion step has not run yet; -1 for NULL. */
int32_t pa_swapper_pending(const pa_swapper* s);
/* Any of the outputs may be NULL: the caller's pinned frame buffer, the kernel
 * and DMA streams (hipStream_t), bytes per frame, blocks per staging half, and
 * the bytes moved by completed swap-outs and swap-ins. */
pa_status pa_swapper_info(const pa_swapper* s, void** host_frames, void** kernel_stream,
                          void** dma_stream, int64_t* frame_bytes, int32_t* chunk_blocks,
                          int64_t* bytes_out, int64_t* bytes_in);

/* ---------------------------------------------------------------- radix prefix cache */
/* Source: "KV Cache Management", section "Prefix Caching Across Turns" (Table 4,
 * Definition 0.2, "Longest prefix matching", "Dynamic radix eviction",
 * Figure 6). A host-side index of cached KV blocks over a block manager. Each
 * node binds a run of token ids to the physical blocks that hold them, with a
 * parent, children, a reference count (requests currently using it) and a last
 * access time; non-branching runs share one node. Only whole blocks are indexed:
 * edges split at block boundaries, and a node's children are keyed by the
 * block_size tokens of their first block. The tree holds one block-manager
 * reference per block it indexes and drops it on eviction; the block manager must
 * outlive the tree. Node ids are assigned 1, 2, ... in creation order (0 is the
 * root) and never reused. A logical clock ticks once per match and per insert.
 * Every call takes the tree's mutex. */
typedef struct pa_radix pa_radix;

pa_status pa_radix_create(pa_bm* bm, pa_radix** out);
/* Drops the tree's reference on every indexed block, then frees the tree. */
pa_status pa_radix_destroy(pa_radix* r);
/* Longest prefix match of tokens[0..n_tokens): *s_match gets the number of
 * leading tokens found in the tree (token level, into a partly matching block),
 * *s_usable = floor(s_match / block_size) * block_size, and blocks_out the
 * s_usable / block_size block ids that hold them, in order. Every node on the
 * matched path (including one used only in part) gains a pin and gets the new
 * clock value as its last access; *handle names the deepest such node (0 when
 * nothing was matched) and pa_radix_unpin(handle) removes exactly these pins.
 * PA_ERR_INVALID_ARG, with nothing changed, if cap < s_usable / block_size. */
pa_status pa_radix_match(pa_radix* r, const int32_t* tokens, int64_t n_tokens, int64_t* s_match,
                         int64_t* s_usable, int32_t* blocks_out, int32_t cap, int32_t* n_blocks,
                         int64_t* handle);
/* Remove one pin from the node and each of its ancestors. PA_ERR_NOT_FOUND for
 * an unknown (or evicted) node, PA_ERR_INVALID_ARG if some node on the path has
 * no pin; handle 0 is a no-op. */
pa_status pa_radix_unpin(pa_radix* r, int64_t handle);
/* Index a finished request: blocks[k] holds tokens[k*B .. (k+1)*B). Only the
 * first min(n_blocks, n_tokens / B) whole blocks count. Blocks already indexed
 * under the same tokens stay as they are (the caller's copies are not taken);
 * the rest form one new node below the longest matched path (a node matched in
 * part is split at the block boundary first) and gain one reference each.
 * *adopted (may be NULL) gets the number of blocks taken. PA_ERR_INVALID_ARG,
 * with nothing changed, if a block to be taken is not allocated. */
pa_status pa_radix_insert(pa_radix* r, const int32_t* tokens, int64_t n_tokens,
                          const int32_t* blocks, int32_t n_blocks, int32_t* adopted);
/* Leaf-first LRU eviction: while the block manager has fewer than target_free
 * free blocks, remove the dormant leaf (no pin, no children) with the oldest
 * last access (ties: lower id), dropping the tree's reference on its blocks;
 * a parent left without children and pins becomes a candidate in turn. The
 * first min(cap, count) evicted ids go to ids_out in order; *n_evicted (may be
 * NULL) gets the count. Stops early when no candidate is left. If the block
 * manager refuses to drop a leaf's references (PA_ERR_DOUBLE_FREE: a block the
 * tree indexes was freed behind its back), that leaf is left untouched, still a
 * candidate, and the call returns the error; leaves evicted before it stay
 * evicted and are reported as above. */
pa_status pa_radix_evict(pa_radix* r, int32_t target_free, int64_t* ids_out, int32_t cap,
                         int32_t* n_evicted);
/* Counts (any output may be NULL): nodes (root excluded), indexed blocks,
 * dormant leaves (eviction candidates), pinned nodes. */
pa_status pa_radix_info(const pa_radix* r, int64_t* nodes, int64_t* blocks, int64_t* dormant,
                        int64_t* pinned);
/* Ids of all nodes (root excluded) in increasing order: the first min(cap, n)
 * to ids_out, *n_out gets n. */
pa_status pa_radix_node_ids(const pa_radix* r, int64_t* ids_out, int64_t cap, int64_t* n_out);
/* One node: meta_out[0..3] = parent id, pin count, last access, number of
 * blocks; its tokens (up to tok_cap) and blocks (up to blk_cap) are copied out.
 * PA_ERR_NOT_FOUND for an unknown id. */
pa_status pa_radix_node(const pa_radix* r, int64_t id, int64_t* meta_out, int32_t* tokens_out,
                        int64_t tok_cap, int32_t* blocks_out, int32_t blk_cap);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
