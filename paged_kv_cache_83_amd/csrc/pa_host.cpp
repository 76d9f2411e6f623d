// Host side of libpa: status strings, KV footprint arithmetic and the block manager.
//
// Footprint: "KV Cache Management", section "From Context Tokens to KV State",
// Eq. (1), and section "The PagedAttention virtual memory model" (M_block,
// N_blocks); per-rank heads from "EfficientAgent ...", Eq. (1).
//
// Block manager: "KV Cache Management", sections "The PagedAttention virtual
// memory model" (allocate at o == 0, write in place otherwise; FIFO free list),
// "Prefix Caching Across Turns" (a request starts from cached full blocks),
// "Zero-copy deliberation via copy-on-write branching" (fork, copy-on-write,
// release) and "Asynchronous paged swapping" (frames leave and re-enter the
// pool); "PagedAttention" (Inference book, ch. 14) for the error contract
// (out-of-blocks, double free, failed reservations leak nothing).
//
// Tiered residency: "KV Cache Management", section "Asynchronous paged
// swapping". A migration to the host takes a contiguous run of frames from a
// pinned host pool (step 1); the copy runs in the background (step 2); only
// when it has completed are the entries retagged as host-resident with their
// frame indices and the vacated HBM blocks pushed to the back of the free queue
// (step 3). The return path reserves fresh blocks first and remaps the entries
// and frees the frames when the copy back has completed. Completion steps are
// called from a HIP host-function thread, so every entry point takes the
// manager's mutex.

#include <algorithm>
#include <climits>
#include <cstdint>
#include <cstring>
#include <deque>
#include <map>
#include <mutex>
#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/pa.h"

namespace {

constexpr int32_t kNotResident = -1;

bool geom_ok(const pa_geom* g) {
  return g && g->num_layers > 0 && g->num_kv_heads > 0 && g->head_dim > 0 && g->block_size > 0 &&
         g->num_blocks > 0 && (g->dtype == PA_F32 || g->dtype == PA_BF16 || g->dtype == PA_FP8);
}

int64_t elem_bytes(int32_t dtype) { return dtype == PA_F32 ? 4 : dtype == PA_BF16 ? 2 : 1; }

// One (layer, block, head) tile: B*d elements, then B scale bytes for FP8.
int64_t tile_bytes(const pa_geom* g) {
  return (int64_t)g->block_size * g->head_dim * elem_bytes(g->dtype) +
         (g->dtype == PA_FP8 ? g->block_size : 0);
}

// One entry of a migration in flight: the HBM block and the host frame it
// moves between; out = true for HBM -> host.
struct Pend {
  bool out;
  int32_t phys;
  int32_t frame;
};

struct Seq {
  std::vector<int32_t> table;
  int64_t len = 0;
  std::map<int32_t, int32_t> host;   // logical -> frame, entries in the host tier
  std::map<int32_t, Pend> pending;   // logical -> migration in flight
};

// Frames 0..F-1 of the pinned host buffer. Runs of consecutive frames are
// handed out first fit (lowest start); a freed run merges with free neighbours.
struct HostPool {
  int32_t num_frames = 0;
  std::vector<char> used;
  std::map<int32_t, int32_t> runs;   // start -> length, free runs, never adjacent

  explicit HostPool(int32_t f) : num_frames(f), used(f, 0) { runs[0] = f; }
  int32_t num_free() const {
    int64_t n = 0;
    for (const auto& r : runs) n += r.second;
    return (int32_t)n;
  }
  // First frame of a run of n, or -1 if no free run is long enough.
  int32_t alloc_run(int32_t n) {
    for (auto it = runs.begin(); it != runs.end(); ++it) {
      if (it->second < n) continue;
      int32_t start = it->first, len = it->second;
      runs.erase(it);
      if (len > n) runs[start + n] = len - n;
      for (int32_t f = start; f < start + n; ++f) used[f] = 1;
      return start;
    }
    return -1;
  }
  // Frames must be allocated and distinct (checked by the caller).
  void free(const std::vector<int32_t>& frames) {
    for (int32_t f : frames) used[f] = 0;
    std::vector<int32_t> fs(frames);
    std::sort(fs.begin(), fs.end());
    for (size_t k = 0; k < fs.size();) {
      size_t e = k + 1;
      while (e < fs.size() && fs[e] == fs[e - 1] + 1) ++e;
      int32_t start = fs[k], len = (int32_t)(e - k);
      auto nx = runs.lower_bound(start);
      if (nx != runs.end() && nx->first == start + len) {   // merge with the run after
        len += nx->second;
        runs.erase(nx);
      }
      auto pv = runs.lower_bound(start);
      if (pv != runs.begin()) {
        --pv;
        if (pv->first + pv->second == start) {              // merge with the run before
          pv->second += len;
          k = e;
          continue;
        }
      }
      runs[start] = len;
      k = e;
    }
  }
};

}  // namespace

struct pa_bm {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::deque<int32_t> free_list;      // pop front, push back
  std::vector<int32_t> ref;
  std::unordered_map<int32_t, Seq> seqs;
  int32_t next_seq = 0;
  HostPool* host_pool = nullptr;
  mutable std::mutex mu;

  ~pa_bm() { delete host_pool; }

  void decref(int32_t b) {
    if (--ref[b] == 0) free_list.push_back(b);
  }
  int32_t take() {
    int32_t b = free_list.front();
    free_list.pop_front();
    ref[b] = 1;
    return b;
  }
  Seq* find(int32_t s) {
    auto it = seqs.find(s);
    return it == seqs.end() ? nullptr : &it->second;
  }
  const Seq* find(int32_t s) const {
    auto it = seqs.find(s);
    return it == seqs.end() ? nullptr : &it->second;
  }
  // Blocks an append of n tokens needs: {copy-on-write, fresh}; -1 if the tail
  // block it would write into is not resident.
  int need(const Seq& q, int64_t n, int64_t* cow, int64_t* fresh) const {
    *cow = 0;
    *fresh = 0;
    if (n <= 0) return 0;
    const int64_t B = block_size;
    if (q.len % B != 0) {
      int32_t tail = q.table[q.len / B];
      if (tail == kNotResident || q.pending.count((int32_t)(q.len / B))) return -1;
      if (ref[tail] > 1) *cow = 1;
    }
    // positions t in [len, len + n) with t % B == 0
    *fresh = (q.len + n + B - 1) / B - (q.len + B - 1) / B;
    return 0;
  }
  // Performs an append already known to fit.
  void do_append(Seq& q, int64_t n, int64_t* slots, int32_t* cow_src, int32_t* cow_dst,
                 int32_t* n_cow) {
    const int64_t B = block_size;
    *n_cow = 0;
    if (n > 0 && q.len % B != 0) {
      int64_t lb = q.len / B;
      int32_t old = q.table[lb];
      if (ref[old] > 1) {
        int32_t nb = take();
        --ref[old];  // another owner still holds it
        q.table[lb] = nb;
        if (cow_src) cow_src[0] = old;
        if (cow_dst) cow_dst[0] = nb;
        *n_cow = 1;
      }
    }
    for (int64_t k = 0; k < n; ++k) {
      int64_t t = q.len + k;
      int64_t lb = t / B, off = t % B;
      if (off == 0) q.table.push_back(take());
      if (slots) slots[k] = (int64_t)q.table[lb] * B + off;
    }
    q.len += n;
  }
};

extern "C" {

const char* pa_status_str(int32_t s) {
  switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_OUT_OF_BLOCKS: return "out of blocks";
    case PA_ERR_DOUBLE_FREE: return "double free";
    case PA_ERR_NOT_FOUND: return "unknown sequence";
    case PA_ERR_HIP: return "HIP runtime error";
    case PA_ERR_WORKSPACE: return "workspace too small";
    case PA_ERR_UNSUPPORTED: return "unsupported geometry";
    case PA_ERR_OUT_OF_FRAMES: return "no run of free host frames";
    default: return "unknown status";
  }
}

int32_t pa_version(void) { return 1; }

int64_t pa_bytes_per_token(int32_t L, int32_t H_kv, int32_t d, int32_t b, int32_t tp) {
  if (L <= 0 || H_kv <= 0 || d <= 0 || b <= 0 || tp <= 0) return -1;
  int64_t heads = std::max<int64_t>(1, (H_kv + tp - 1) / tp);
  return 2 * (int64_t)L * heads * d * b;
}

int64_t pa_bytes_per_block(const pa_geom* g) {
  if (!geom_ok(g)) return -1;
  return 2 * (int64_t)g->num_layers * g->num_kv_heads * tile_bytes(g);
}

int64_t pa_blocks_for_tokens(int64_t tokens, int32_t B) {
  if (tokens < 0 || B <= 0) return -1;
  return (tokens + B - 1) / B;
}

int64_t pa_pool_bytes(const pa_geom* g) {
  if (!geom_ok(g)) return -1;
  return (int64_t)g->num_layers * g->num_blocks * g->num_kv_heads * tile_bytes(g);
}

// ------------------------------------------------------------------ block manager

pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                       pa_bm** out) {
  if (!out || num_blocks <= 0 || block_size <= 0) return PA_ERR_INVALID_ARG;
  *out = nullptr;
  pa_bm* bm = new (std::nothrow) pa_bm();
  if (!bm) return PA_ERR_INVALID_ARG;
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->ref.assign(num_blocks, 0);
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete bm;
        return PA_ERR_INVALID_ARG;
      }
      seen[b] = 1;
      bm->free_list.push_back(b);
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) bm->free_list.push_back(i);
  }
  *out = bm;
  return PA_OK;
}

void pa_bm_destroy(pa_bm* bm) { delete bm; }

int32_t pa_bm_num_free(const pa_bm* bm) {
  if (!bm) return -1;
  std::lock_guard<std::mutex> lk(bm->mu);
  return (int32_t)bm->free_list.size();
}

int32_t pa_bm_block_size(const pa_bm* bm) { return bm ? bm->block_size : -1; }

int32_t pa_bm_refcount(const pa_bm* bm, int32_t b) {
  if (!bm || b < 0 || b >= bm->num_blocks) return -1;
  std::lock_guard<std::mutex> lk(bm->mu);
  return bm->ref[b];
}

pa_status pa_bm_free_list(const pa_bm* bm, int32_t* ids_out, int32_t cap, int32_t* n_out) {
  if (!bm || cap < 0 || (cap > 0 && !ids_out) || !n_out) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(bm->mu);
  int32_t k = 0;
  for (int32_t b : bm->free_list) {
    if (k >= cap) break;
    ids_out[k++] = b;
  }
  *n_out = (int32_t)bm->free_list.size();
  return PA_OK;
}

pa_status pa_bm_alloc(pa_bm* bm, int32_t n, int32_t* ids_out) {
  if (!bm || n < 0 || (n > 0 && !ids_out)) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(bm->mu);
  if ((size_t)n > bm->free_list.size()) return PA_ERR_OUT_OF_BLOCKS;
  for (int32_t i = 0; i < n; ++i) ids_out[i] = bm->take();
  return PA_OK;
}

pa_status pa_bm_incref(pa_bm* bm, const int32_t* ids, int32_t n) {
  if (!bm || n < 0 || (n > 0 && !ids)) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(bm->mu);
  for (int32_t i = 0; i < n; ++i)
    if (ids[i] < 0 || ids[i] >= bm->num_blocks || bm->ref[ids[i]] == 0) return PA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i) ++bm->ref[ids[i]];
  return PA_OK;
}

pa_status pa_bm_free_blocks(pa_bm* bm, const int32_t* ids, int32_t n) {
  if (!bm || n < 0 || (n > 0 && !ids)) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(bm->mu);
  std::unordered_map<int32_t, int32_t> drops;
  for (int32_t i = 0; i < n; ++i) {
    int32_t b = ids[i];
    if (b < 0 || b >= bm->num_blocks) return PA_ERR_INVALID_ARG;
    if (++drops[b] > bm->ref[b]) return PA_ERR_DOUBLE_FREE;
  }
  for (int32_t i = 0; i < n; ++i) bm->decref(ids[i]);
  return PA_OK;
}

pa_status pa_bm_seq_new(pa_bm* bm, int32_t* seq_out) {
  if (!bm || !seq_out) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(bm->mu);
  int32_t s = bm->next_seq++;
  bm->seqs.emplace(s, Seq());
  *seq_out = s;
  return PA_OK;
}

pa_status pa_bm_seq_from_blocks(pa_bm* bm, const int32_t* ids, int32_t n, int32_t* seq_out) {
  if (!bm || !seq_out || n < 0 || (n > 0 && !ids)) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(bm->mu);
  for (int32_t i = 0; i < n; ++i)
    if (ids[i] < 0 || ids[i] >= bm->num_blocks || bm->ref[ids[i]] == 0) return PA_ERR_INVALID_ARG;
  Seq q;
  q.table.assign(ids, ids + n);
  q.len = (int64_t)n * bm->block_size;
  for (int32_t b : q.table) ++bm->ref[b];
  int32_t s = bm->next_seq++;
  bm->seqs.emplace(s, std::move(q));
  *seq_out = s;
  return PA_OK;
}

pa_status pa_bm_seq_fork(pa_bm* bm, int32_t parent, int32_t* child_out) {
  if (!bm || !child_out) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(bm->mu);
  const Seq* p = bm->find(parent);
  if (!p) return PA_ERR_NOT_FOUND;
  if (!p->pending.empty()) return PA_ERR_INVALID_ARG;
  for (int32_t b : p->table)
    if (b == kNotResident) return PA_ERR_INVALID_ARG;
  Seq child;
  child.table = p->table;   // 1. duplicate the table
  child.len = p->len;       // 3. same starting length
  for (int32_t b : child.table) ++bm->ref[b];   // 2. one more reference per block
  int32_t c = bm->next_seq++;
  bm->seqs.emplace(c, std::move(child));
  *child_out = c;
  return PA_OK;
}

pa_status pa_bm_seq_append(pa_bm* bm, int32_t seq, int32_t n, int64_t* slots_out,
                           int32_t* cow_src, int32_t* cow_dst, int32_t* n_cow) {
  if (!bm || n < 0 || !n_cow) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(bm->mu);
  Seq* q = bm->find(seq);
  if (!q) return PA_ERR_NOT_FOUND;
  int64_t cow = 0, fresh = 0;
  if (bm->need(*q, n, &cow, &fresh) != 0) return PA_ERR_INVALID_ARG;
  if (cow && (!cow_src || !cow_dst)) return PA_ERR_INVALID_ARG;
  if ((size_t)(cow + fresh) > bm->free_list.size()) return PA_ERR_OUT_OF_BLOCKS;
  bm->do_append(*q, n, slots_out, cow_src, cow_dst, n_cow);
  return PA_OK;
}

pa_status pa_bm_append_batch(pa_bm* bm, const int32_t* seqs, const int32_t* counts, int32_t n,
                             int64_t* slots_out, int32_t* cow_src, int32_t* cow_dst,
                             int32_t* n_cow_out) {
  if (!bm || n < 0 || !n_cow_out || (n > 0 && (!seqs || !counts))) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(bm->mu);
  for (int32_t k = 0; k < n; ++k) {
    if (counts[k] < 0) return PA_ERR_INVALID_ARG;
    const Seq* q = bm->find(seqs[k]);
    if (!q) return PA_ERR_NOT_FOUND;
    if (counts[k] > 0 && q->len % bm->block_size != 0 &&
        (q->table[q->len / bm->block_size] == kNotResident ||
         q->pending.count((int32_t)(q->len / bm->block_size))))
      return PA_ERR_INVALID_ARG;
  }
  // Sequences in one batch may share a tail block (so whether a later one must
  // copy depends on the earlier ones): run the appends in order on the real
  // state and restore a snapshot if the pool runs dry part-way.
  std::deque<int32_t> free_snap = bm->free_list;
  std::vector<int32_t> ref_snap = bm->ref;
  std::unordered_map<int32_t, Seq> touched;
  for (int32_t k = 0; k < n; ++k)
    if (!touched.count(seqs[k])) touched.emplace(seqs[k], *bm->find(seqs[k]));
  int64_t off = 0;
  int32_t ncow = 0;
  for (int32_t k = 0; k < n; ++k) {
    Seq* q = bm->find(seqs[k]);
    int64_t cow = 0, fresh = 0;
    bm->need(*q, counts[k], &cow, &fresh);
    bool room = (size_t)(cow + fresh) <= bm->free_list.size();
    bool cow_room = !cow || (cow_src && cow_dst);
    if (!room || !cow_room) {
      bm->free_list = std::move(free_snap);
      bm->ref = std::move(ref_snap);
      for (auto& kv : touched) *bm->find(kv.first) = std::move(kv.second);
      return room ? PA_ERR_INVALID_ARG : PA_ERR_OUT_OF_BLOCKS;
    }
    int32_t c = 0;
    bm->do_append(*q, counts[k], slots_out ? slots_out + off : nullptr,
                  cow_src ? cow_src + ncow : nullptr, cow_dst ? cow_dst + ncow : nullptr, &c);
    ncow += c;
    off += counts[k];
  }
  *n_cow_out = ncow;
  return PA_OK;
}

pa_status pa_bm_seq_release(pa_bm* bm, int32_t seq) {
  if (!bm) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(bm->mu);
  Seq* q = bm->find(seq);
  if (!q) return PA_ERR_NOT_FOUND;
  if (!q->pending.empty()) return PA_ERR_INVALID_ARG;   // a migration is in flight
  for (int32_t b : q->table)
    if (b != kNotResident) bm->decref(b);
  if (!q->host.empty()) {
    std::vector<int32_t> frames;
    for (const auto& kv : q->host) frames.push_back(kv.second);
    bm->host_pool->free(frames);
  }
  bm->seqs.erase(seq);
  return PA_OK;
}

static pa_status check_logical(const Seq& q, const int32_t* logical, int32_t n, bool want_resident) {
  std::vector<char> seen(q.table.size(), 0);
  for (int32_t i = 0; i < n; ++i) {
    int32_t lb = logical[i];
    if (lb < 0 || (size_t)lb >= q.table.size() || seen[lb]) return PA_ERR_INVALID_ARG;
    seen[lb] = 1;
    bool resident = q.table[lb] != kNotResident;
    if (resident != want_resident || q.pending.count(lb)) return PA_ERR_INVALID_ARG;
    if (!want_resident && q.host.count(lb)) return PA_ERR_INVALID_ARG;   // held by the host pool
  }
  return PA_OK;
}

pa_status pa_bm_seq_swap_out(pa_bm* bm, int32_t seq, const int32_t* logical, int32_t n,
                             int32_t* phys_out) {
  if (!bm || n < 0 || (n > 0 && (!logical || !phys_out))) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(bm->mu);
  Seq* q = bm->find(seq);
  if (!q) return PA_ERR_NOT_FOUND;
  pa_status st = check_logical(*q, logical, n, true);
  if (st != PA_OK) return st;
  for (int32_t i = 0; i < n; ++i) {
    int32_t& e = q->table[logical[i]];
    phys_out[i] = e;
    bm->decref(e);
    e = kNotResident;
  }
  return PA_OK;
}

pa_status pa_bm_seq_swap_in(pa_bm* bm, int32_t seq, const int32_t* logical, int32_t n,
                            int32_t* phys_out) {
  if (!bm || n < 0 || (n > 0 && (!logical || !phys_out))) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(bm->mu);
  Seq* q = bm->find(seq);
  if (!q) return PA_ERR_NOT_FOUND;
  pa_status st = check_logical(*q, logical, n, false);
  if (st != PA_OK) return st;
  if ((size_t)n > bm->free_list.size()) return PA_ERR_OUT_OF_BLOCKS;
  for (int32_t i = 0; i < n; ++i) {
    int32_t b = bm->take();
    q->table[logical[i]] = b;
    phys_out[i] = b;
  }
  return PA_OK;
}

pa_status pa_bm_permute_free(pa_bm* bm, const int32_t* perm, int32_t n) {
  if (!bm || n < 0 || (n > 0 && !perm)) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(bm->mu);
  if ((size_t)n != bm->free_list.size()) return PA_ERR_INVALID_ARG;
  std::vector<char> seen(n, 0);
  for (int32_t k = 0; k < n; ++k) {
    if (perm[k] < 0 || perm[k] >= n || seen[perm[k]]) return PA_ERR_INVALID_ARG;
    seen[perm[k]] = 1;
  }
  std::vector<int32_t> cur(bm->free_list.begin(), bm->free_list.end());
  std::deque<int32_t> next;
  for (int32_t k = 0; k < n; ++k) next.push_back(cur[perm[k]]);
  bm->free_list.swap(next);
  return PA_OK;
}

pa_status pa_bm_seq_info(const pa_bm* bm, int32_t seq, int64_t* n_tokens, int32_t* n_blocks) {
  if (!bm) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(bm->mu);
  const Seq* q = bm->find(seq);
  if (!q) return PA_ERR_NOT_FOUND;
  if (n_tokens) *n_tokens = q->len;
  if (n_blocks) *n_blocks = (int32_t)q->table.size();
  return PA_OK;
}

pa_status pa_bm_seq_table(const pa_bm* bm, int32_t seq, int32_t* table_out, int32_t cap,
                          int32_t* n_blocks) {
  if (!bm || cap < 0 || (cap > 0 && !table_out)) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(bm->mu);
  const Seq* q = bm->find(seq);
  if (!q) return PA_ERR_NOT_FOUND;
  int32_t m = (int32_t)std::min<size_t>(q->table.size(), (size_t)cap);
  if (m) std::memcpy(table_out, q->table.data(), sizeof(int32_t) * m);
  if (n_blocks) *n_blocks = (int32_t)q->table.size();
  return PA_OK;
}

pa_status pa_bm_build_tables(const pa_bm* bm, const int32_t* seqs, int32_t n, int32_t max_blocks,
                             int32_t pad, int32_t* tables_out, int32_t* lens_out) {
  if (!bm || n < 0 || max_blocks < 0 || (n > 0 && (!seqs || !tables_out || !lens_out)))
    return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(bm->mu);
  for (int32_t k = 0; k < n; ++k) {
    const Seq* q = bm->find(seqs[k]);
    if (!q) return PA_ERR_NOT_FOUND;
    if (q->table.size() > (size_t)max_blocks || q->len > INT32_MAX) return PA_ERR_INVALID_ARG;
  }
  for (int32_t k = 0; k < n; ++k) {
    const Seq* q = bm->find(seqs[k]);
    int32_t* row = tables_out + (int64_t)k * max_blocks;
    size_t m = q->table.size();
    if (m) std::memcpy(row, q->table.data(), sizeof(int32_t) * m);
    for (size_t j = m; j < (size_t)max_blocks; ++j) row[j] = pad;
    lens_out[k] = (int32_t)q->len;
  }
  return PA_OK;
}

// ------------------------------------------------------------------ tiered residency

pa_status pa_bm_attach_host_pool(pa_bm* bm, int32_t num_frames) {
  if (!bm || num_frames <= 0) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(bm->mu);
  if (bm->host_pool) return PA_ERR_INVALID_ARG;
  bm->host_pool = new (std::nothrow) HostPool(num_frames);
  return bm->host_pool ? PA_OK : PA_ERR_INVALID_ARG;
}

pa_status pa_bm_detach_host_pool(pa_bm* bm) {
  if (!bm) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(bm->mu);
  if (!bm->host_pool || bm->host_pool->num_free() != bm->host_pool->num_frames)
    return PA_ERR_INVALID_ARG;
  delete bm->host_pool;
  bm->host_pool = nullptr;
  return PA_OK;
}

int32_t pa_bm_host_frames_free(const pa_bm* bm) {
  if (!bm) return -1;
  std::lock_guard<std::mutex> lk(bm->mu);
  return bm->host_pool ? bm->host_pool->num_free() : -1;
}

pa_status pa_bm_host_free_runs(const pa_bm* bm, int32_t* starts, int32_t* lengths, int32_t cap,
                               int32_t* n_out) {
  if (!bm || cap < 0 || (cap > 0 && (!starts || !lengths)) || !n_out) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(bm->mu);
  if (!bm->host_pool) return PA_ERR_INVALID_ARG;
  int32_t k = 0;
  for (const auto& r : bm->host_pool->runs) {
    if (k >= cap) break;
    starts[k] = r.first;
    lengths[k] = r.second;
    ++k;
  }
  *n_out = (int32_t)bm->host_pool->runs.size();
  return PA_OK;
}

// (tag, index) of one entry; index is the HBM block for PA_TIER_HBM and
// PA_TIER_PENDING_OUT, the host frame for PA_TIER_HOST and PA_TIER_PENDING_IN
// (-1 for an entry swapped out by pa_bm_seq_swap_out, which holds no frame).
static void tier_of(const Seq& q, int32_t lb, int32_t* tier, int32_t* index) {
  auto pe = q.pending.find(lb);
  if (pe != q.pending.end()) {
    *tier = pe->second.out ? PA_TIER_PENDING_OUT : PA_TIER_PENDING_IN;
    *index = pe->second.out ? pe->second.phys : pe->second.frame;
    return;
  }
  auto he = q.host.find(lb);
  if (he != q.host.end()) {
    *tier = PA_TIER_HOST;
    *index = he->second;
    return;
  }
  if (q.table[lb] == kNotResident) {
    *tier = PA_TIER_HOST;
    *index = -1;
    return;
  }
  *tier = PA_TIER_HBM;
  *index = q.table[lb];
}

pa_status pa_bm_block_tier(const pa_bm* bm, int32_t seq, int32_t logical, int32_t* tier,
                           int32_t* index) {
  if (!bm || !tier || !index) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(bm->mu);
  const Seq* q = bm->find(seq);
  if (!q) return PA_ERR_NOT_FOUND;
  if (logical < 0 || (size_t)logical >= q->table.size()) return PA_ERR_INVALID_ARG;
  tier_of(*q, logical, tier, index);
  return PA_OK;
}

// A non-empty list of distinct in-range logical blocks of a known sequence.
static pa_status migration_list(pa_bm* bm, int32_t seq, const int32_t* logical, int32_t n,
                                Seq** out) {
  if (n <= 0 || !logical) return PA_ERR_INVALID_ARG;
  Seq* q = bm->find(seq);
  if (!q) return PA_ERR_NOT_FOUND;
  std::vector<char> seen(q->table.size(), 0);
  for (int32_t i = 0; i < n; ++i) {
    int32_t lb = logical[i];
    if (lb < 0 || (size_t)lb >= q->table.size() || seen[lb]) return PA_ERR_INVALID_ARG;
    seen[lb] = 1;
  }
  *out = q;
  return PA_OK;
}

pa_status pa_bm_swap_out_begin(pa_bm* bm, int32_t seq, const int32_t* logical, int32_t n,
                               int32_t* phys_out, int32_t* first_frame_out) {
  if (!bm || !phys_out || !first_frame_out) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(bm->mu);
  if (!bm->host_pool) return PA_ERR_INVALID_ARG;
  Seq* q = nullptr;
  pa_status st = migration_list(bm, seq, logical, n, &q);
  if (st != PA_OK) return st;
  for (int32_t i = 0; i < n; ++i) {
    int32_t t, idx;
    tier_of(*q, logical[i], &t, &idx);
    if (t != PA_TIER_HBM) return PA_ERR_INVALID_ARG;
  }
  int32_t first = bm->host_pool->alloc_run(n);      // step 1: one contiguous run
  if (first < 0) return PA_ERR_OUT_OF_FRAMES;
  for (int32_t i = 0; i < n; ++i) {
    int32_t p = q->table[logical[i]];
    q->pending[logical[i]] = Pend{true, p, first + i};
    phys_out[i] = p;
  }
  *first_frame_out = first;
  return PA_OK;
}

pa_status pa_bm_swap_out_finish(pa_bm* bm, int32_t seq, const int32_t* logical, int32_t n) {
  if (!bm) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(bm->mu);
  Seq* q = nullptr;
  pa_status st = migration_list(bm, seq, logical, n, &q);
  if (st != PA_OK) return st;
  for (int32_t i = 0; i < n; ++i) {
    auto it = q->pending.find(logical[i]);
    if (it == q->pending.end() || !it->second.out) return PA_ERR_INVALID_ARG;
  }
  for (int32_t i = 0; i < n; ++i) {                  // step 3: retag, free the HBM blocks
    auto it = q->pending.find(logical[i]);
    Pend e = it->second;
    q->pending.erase(it);
    bm->decref(e.phys);
    q->table[logical[i]] = kNotResident;
    q->host[logical[i]] = e.frame;
  }
  return PA_OK;
}

pa_status pa_bm_swap_in_begin(pa_bm* bm, int32_t seq, const int32_t* logical, int32_t n,
                              int32_t* phys_out, int32_t* frames_out) {
  if (!bm || !phys_out || !frames_out) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(bm->mu);
  Seq* q = nullptr;
  pa_status st = migration_list(bm, seq, logical, n, &q);
  if (st != PA_OK) return st;
  for (int32_t i = 0; i < n; ++i) {
    int32_t t, idx;
    tier_of(*q, logical[i], &t, &idx);
    if (t != PA_TIER_HOST || idx < 0) return PA_ERR_INVALID_ARG;
  }
  if ((size_t)n > bm->free_list.size()) return PA_ERR_OUT_OF_BLOCKS;
  for (int32_t i = 0; i < n; ++i) {
    int32_t p = bm->take();
    int32_t frame = q->host[logical[i]];
    q->pending[logical[i]] = Pend{false, p, frame};
    phys_out[i] = p;
    frames_out[i] = frame;
  }
  return PA_OK;
}

pa_status pa_bm_swap_in_finish(pa_bm* bm, int32_t seq, const int32_t* logical, int32_t n) {
  if (!bm) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(bm->mu);
  Seq* q = nullptr;
  pa_status st = migration_list(bm, seq, logical, n, &q);
  if (st != PA_OK) return st;
  for (int32_t i = 0; i < n; ++i) {
    auto it = q->pending.find(logical[i]);
    if (it == q->pending.end() || it->second.out) return PA_ERR_INVALID_ARG;
  }
  std::vector<int32_t> frames;
  for (int32_t i = 0; i < n; ++i) {
    auto it = q->pending.find(logical[i]);
    Pend e = it->second;
    q->pending.erase(it);
    q->table[logical[i]] = e.phys;
    q->host.erase(logical[i]);
    frames.push_back(e.frame);
  }
  bm->host_pool->free(frames);
  return PA_OK;
}

pa_status pa_bm_validate(const pa_bm* bm) {
  if (!bm) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(bm->mu);
  std::vector<int64_t> uses(bm->num_blocks, 0);
  for (const auto& kv : bm->seqs) {
    const Seq& q = kv.second;
    int64_t want = (q.len + bm->block_size - 1) / bm->block_size;
    if ((int64_t)q.table.size() != want) return PA_ERR_INVALID_ARG;
    for (int32_t b : q.table) {
      if (b == kNotResident) continue;
      if (b < 0 || b >= bm->num_blocks) return PA_ERR_INVALID_ARG;
      ++uses[b];
    }
    for (const auto& kv : q.pending) {
      const Pend& e = kv.second;
      if (e.phys < 0 || e.phys >= bm->num_blocks) return PA_ERR_INVALID_ARG;
      if (e.out ? q.table[kv.first] != e.phys : q.table[kv.first] != kNotResident)
        return PA_ERR_INVALID_ARG;
      if (!e.out) ++uses[e.phys];    // reserved for the copy back, not yet in the table
    }
    for (const auto& kv : q.host)
      if (q.table[kv.first] != kNotResident) return PA_ERR_INVALID_ARG;
  }
  if (bm->host_pool) {   // every used frame is held by exactly one host or in-flight entry
    const HostPool& hp = *bm->host_pool;
    std::vector<int32_t> holders(hp.num_frames, 0);
    for (const auto& sq : bm->seqs) {
      for (const auto& kv : sq.second.host) ++holders[kv.second];
      for (const auto& kv : sq.second.pending)
        if (kv.second.out) ++holders[kv.second.frame];
    }
    int64_t free_frames = 0;
    for (int32_t f = 0; f < hp.num_frames; ++f) {
      if (holders[f] > 1 || (holders[f] == 1) != (hp.used[f] != 0)) return PA_ERR_INVALID_ARG;
      free_frames += !hp.used[f];
    }
    if (free_frames != hp.num_free()) return PA_ERR_INVALID_ARG;
  }
  std::vector<char> in_free(bm->num_blocks, 0);
  for (int32_t b : bm->free_list) {
    if (b < 0 || b >= bm->num_blocks || in_free[b]) return PA_ERR_INVALID_ARG;
    in_free[b] = 1;
  }
  for (int32_t b = 0; b < bm->num_blocks; ++b) {
    if (bm->ref[b] < uses[b]) return PA_ERR_INVALID_ARG;
    if ((bm->ref[b] == 0) != (in_free[b] != 0)) return PA_ERR_INVALID_ARG;
  }
  return PA_OK;
}

}  // extern "C"
