// Radix prefix cache: a host-side index of cached KV blocks over the block
// manager, after "KV Cache Management", section "Prefix Caching Across Turns":
// Table 4 (node fields), Definition 0.2, "Longest prefix matching" (walk from the
// root, block-aligned truncation S_usable = floor(S_match / B) * B) and "Dynamic
// radix eviction" (pinned vs dormant nodes, LRU order over dormant leaves,
// iterative pruning until the free pool reaches a target, cascading eligibility
// of a parent left without children), with Figure 6.
//
// Only whole blocks are shared, so a node always holds a whole number of blocks
// and edges split at block boundaries. Children are found by the hash of the B
// tokens of their first block (a full-block comparison confirms a hit); a second
// index by first token serves the token-level S_match into a block that matches
// only in part. Dormant leaves sit in an ordered set keyed by (last access, id),
// so the least recently used one is its first element and a parent that becomes
// a dormant leaf joins at its own timestamp. The tree talks to the block manager
// only through its C interface (one reference per indexed block).

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <set>
#include <unordered_map>
#include <utility>
#include <vector>

#include "../../include/pa.h"

namespace {

struct Node {
  int64_t id = 0;
  Node* parent = nullptr;
  std::vector<int32_t> tokens;   // prefix_tokens: a whole number of blocks
  std::vector<int32_t> blocks;   // block_ids: tokens.size() / B entries
  std::unordered_multimap<uint64_t, Node*> kids;       // hash of the first block
  std::unordered_multimap<int32_t, Node*> kids_by_tok; // first token
  int64_t ref = 0;               // pins held by requests
  uint64_t last = 0;             // last access (logical clock)
  bool in_lru = false;
  uint64_t lru_key = 0;          // `last` when it entered the dormant-leaf set
};

uint64_t block_hash(const int32_t* t, int32_t B) {
  uint64_t h = 0xcbf29ce484222325ull;   // FNV-1a over 32-bit words, then a final mix
  for (int32_t i = 0; i < B; ++i) {
    h ^= (uint32_t)t[i];
    h *= 0x100000001b3ull;
  }
  h ^= h >> 31;
  h *= 0x9e3779b97f4a7c15ull;
  h ^= h >> 29;
  return h;
}

struct Walk {
  std::vector<Node*> path;   // nodes matched in full
  Node* partial = nullptr;   // node matched in part (whole blocks pb, then a mismatch)
  int64_t pb = 0;
  int64_t s_match = 0;
};

}  // namespace

struct pa_radix {
  pa_bm* bm = nullptr;
  int32_t B = 0;
  Node root;
  std::unordered_map<int64_t, Node*> nodes;            // root excluded
  std::set<std::pair<uint64_t, int64_t>> lru;          // dormant leaves
  uint64_t clock = 0;
  int64_t next_id = 1;
  int64_t n_blocks = 0;
  int64_t n_pinned = 0;
  mutable std::mutex mu;
  Walk w;                                              // reused between calls

  Node* child_with_block(Node* n, const int32_t* t) const {
    auto range = n->kids.equal_range(block_hash(t, B));
    for (auto it = range.first; it != range.second; ++it)
      if (std::memcmp(it->second->tokens.data(), t, sizeof(int32_t) * B) == 0) return it->second;
    return nullptr;
  }

  // Tokens of t[0..len) (len <= B) that agree with the first block of some child.
  int64_t best_first_block(Node* n, const int32_t* t, int64_t len) const {
    if (len <= 0) return 0;
    int64_t best = 0;
    auto range = n->kids_by_tok.equal_range(t[0]);
    for (auto it = range.first; it != range.second; ++it) {
      const int32_t* c = it->second->tokens.data();
      int64_t lim = std::min<int64_t>(len, B), k = 0;
      while (k < lim && c[k] == t[k]) ++k;
      best = std::max(best, k);
    }
    return best;
  }

  void walk(const int32_t* t, int64_t n) {
    w.path.clear();
    w.partial = nullptr;
    w.pb = 0;
    Node* node = &root;
    int64_t pos = 0;
    for (;;) {
      Node* c = pos + B <= n ? child_with_block(node, t + pos) : nullptr;
      if (!c) {
        w.s_match = pos + best_first_block(node, t + pos, n - pos);
        return;
      }
      const int64_t nb = (int64_t)c->blocks.size();
      int64_t j = 1;   // the first block matched through the lookup
      while (j < nb && pos + (j + 1) * B <= n &&
             std::memcmp(c->tokens.data() + j * B, t + pos + j * B, sizeof(int32_t) * B) == 0)
        ++j;
      if (j == nb) {
        w.path.push_back(c);
        node = c;
        pos += nb * B;
        continue;
      }
      w.partial = c;
      w.pb = j;
      int64_t k = 0;
      const int32_t* ct = c->tokens.data() + j * B;
      const int32_t* pt = t + pos + j * B;
      while (k < B && pos + j * B + k < n && ct[k] == pt[k]) ++k;
      w.s_match = pos + j * B + k;
      return;
    }
  }

  // Keep the dormant-leaf set in step with a node's pins, children and time.
  void refresh(Node* n) {
    if (n == &root) return;
    bool want = n->ref == 0 && n->kids.empty();
    if (n->in_lru && (!want || n->lru_key != n->last)) {
      lru.erase({n->lru_key, n->id});
      n->in_lru = false;
    }
    if (want && !n->in_lru) {
      lru.insert({n->last, n->id});
      n->in_lru = true;
      n->lru_key = n->last;
    }
  }

  void pin(Node* n) {
    if (n->ref++ == 0) ++n_pinned;
  }

  static void erase_kid(Node* parent, Node* kid, uint64_t h, int32_t tok) {
    auto r1 = parent->kids.equal_range(h);
    for (auto it = r1.first; it != r1.second; ++it)
      if (it->second == kid) {
        parent->kids.erase(it);
        break;
      }
    auto r2 = parent->kids_by_tok.equal_range(tok);
    for (auto it = r2.first; it != r2.second; ++it)
      if (it->second == kid) {
        parent->kids_by_tok.erase(it);
        break;
      }
  }

  void add_kid(Node* parent, Node* kid) {
    parent->kids.emplace(block_hash(kid->tokens.data(), B), kid);
    parent->kids_by_tok.emplace(kid->tokens[0], kid);
  }

  Node* new_node(Node* parent) {
    Node* n = new Node();
    n->id = next_id++;
    n->parent = parent;
    nodes.emplace(n->id, n);
    return n;
  }
};

extern "C" {

pa_status pa_radix_create(pa_bm* bm, pa_radix** out) {
  if (!bm || !out) return PA_ERR_INVALID_ARG;
  *out = nullptr;
  const int32_t B = pa_bm_block_size(bm);
  if (B <= 0) return PA_ERR_INVALID_ARG;
  pa_radix* r = new (std::nothrow) pa_radix();
  if (!r) return PA_ERR_INVALID_ARG;
  r->bm = bm;
  r->B = B;
  *out = r;
  return PA_OK;
}

pa_status pa_radix_destroy(pa_radix* r) {
  if (!r) return PA_ERR_INVALID_ARG;
  {
    std::lock_guard<std::mutex> lk(r->mu);
    for (auto& kv : r->nodes) {
      Node* n = kv.second;
      if (!n->blocks.empty()) pa_bm_free_blocks(r->bm, n->blocks.data(), (int32_t)n->blocks.size());
      delete n;
    }
    r->nodes.clear();
  }
  delete r;
  return PA_OK;
}

pa_status pa_radix_match(pa_radix* r, const int32_t* tokens, int64_t n_tokens, int64_t* s_match,
                         int64_t* s_usable, int32_t* blocks_out, int32_t cap, int32_t* n_blocks,
                         int64_t* handle) {
  if (!r || n_tokens < 0 || (n_tokens > 0 && !tokens) || cap < 0 || (cap > 0 && !blocks_out))
    return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(r->mu);
  r->walk(tokens, n_tokens);
  Walk& w = r->w;
  int64_t nb = w.pb;
  for (Node* n : w.path) nb += (int64_t)n->blocks.size();
  if (nb > cap) return PA_ERR_INVALID_ARG;
  int64_t k = 0;
  for (Node* n : w.path)
    for (int32_t b : n->blocks) blocks_out[k++] = b;
  for (int64_t j = 0; j < w.pb; ++j) blocks_out[k++] = w.partial->blocks[j];
  const uint64_t t = ++r->clock;
  Node* deepest = nullptr;
  for (Node* n : w.path) {
    r->pin(n);
    n->last = t;
    r->refresh(n);
    deepest = n;
  }
  if (w.partial && w.pb > 0) {
    r->pin(w.partial);
    w.partial->last = t;
    r->refresh(w.partial);
    deepest = w.partial;
  }
  if (s_match) *s_match = w.s_match;
  if (s_usable) *s_usable = nb * r->B;
  if (n_blocks) *n_blocks = (int32_t)nb;
  if (handle) *handle = deepest ? deepest->id : 0;
  return PA_OK;
}

pa_status pa_radix_unpin(pa_radix* r, int64_t handle) {
  if (!r) return PA_ERR_INVALID_ARG;
  if (handle == 0) return PA_OK;
  std::lock_guard<std::mutex> lk(r->mu);
  auto it = r->nodes.find(handle);
  if (it == r->nodes.end()) return PA_ERR_NOT_FOUND;
  for (Node* n = it->second; n != &r->root; n = n->parent)
    if (n->ref == 0) return PA_ERR_INVALID_ARG;
  for (Node* n = it->second; n != &r->root; n = n->parent) {
    if (--n->ref == 0) --r->n_pinned;
    r->refresh(n);
  }
  return PA_OK;
}

pa_status pa_radix_insert(pa_radix* r, const int32_t* tokens, int64_t n_tokens,
                          const int32_t* blocks, int32_t n_blocks, int32_t* adopted) {
  if (!r || n_tokens < 0 || n_blocks < 0 || (n_tokens > 0 && !tokens) || (n_blocks > 0 && !blocks))
    return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(r->mu);
  const int64_t B = r->B;
  const int64_t nb = std::min<int64_t>(n_blocks, n_tokens / B);
  r->walk(tokens, nb * B);
  Walk& w = r->w;
  int64_t done = 0;
  for (Node* n : w.path) done += (int64_t)n->blocks.size();
  const bool split = w.partial && w.pb > 0;
  const int64_t start = done + (split ? w.pb : 0);   // first block the tree lacks
  if (start < nb) {
    pa_status rc = pa_bm_incref(r->bm, blocks + start, (int32_t)(nb - start));
    if (rc != PA_OK) return rc;
  }
  const uint64_t t = ++r->clock;
  for (Node* n : w.path) {
    n->last = t;
    r->refresh(n);
  }
  if (split) {
    w.partial->last = t;
    r->refresh(w.partial);
  }
  if (adopted) *adopted = 0;
  if (start >= nb) return PA_OK;
  Node* node = w.path.empty() ? &r->root : w.path.back();
  if (split) {   // the partly matched node splits after its first pb blocks
    Node* p = w.partial;
    Node* up = r->new_node(p->parent);
    up->tokens.assign(p->tokens.begin(), p->tokens.begin() + w.pb * B);
    up->blocks.assign(p->blocks.begin(), p->blocks.begin() + w.pb);
    up->ref = p->ref;
    if (up->ref > 0) ++r->n_pinned;
    up->last = t;
    const uint64_t h = block_hash(p->tokens.data(), r->B);
    pa_radix::erase_kid(p->parent, p, h, p->tokens[0]);
    r->add_kid(p->parent, up);
    p->tokens.erase(p->tokens.begin(), p->tokens.begin() + w.pb * B);
    p->blocks.erase(p->blocks.begin(), p->blocks.begin() + w.pb);
    p->parent = up;
    r->add_kid(up, p);
    r->refresh(up);
    node = up;
  }
  Node* c = r->new_node(node);
  c->tokens.assign(tokens + start * B, tokens + nb * B);
  c->blocks.assign(blocks + start, blocks + nb);
  c->last = t;
  r->add_kid(node, c);
  r->refresh(c);
  r->refresh(node);
  r->n_blocks += nb - start;
  if (adopted) *adopted = (int32_t)(nb - start);
  return PA_OK;
}

pa_status pa_radix_evict(pa_radix* r, int32_t target_free, int64_t* ids_out, int32_t cap,
                         int32_t* n_evicted) {
  if (!r || cap < 0 || (cap > 0 && !ids_out)) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(r->mu);
  int32_t count = 0;
  pa_status rc = PA_OK;
  while (!r->lru.empty() && pa_bm_num_free(r->bm) < target_free) {
    auto first = r->lru.begin();
    Node* leaf = r->nodes.at(first->second);
    // The block manager's call is all or nothing: when it refuses (a block lost
    // the tree's reference behind its back) the leaf stays as it is, still a
    // candidate, and the call stops with the leaves evicted so far.
    rc = pa_bm_free_blocks(r->bm, leaf->blocks.data(), (int32_t)leaf->blocks.size());
    if (rc != PA_OK) break;
    r->lru.erase(first);
    leaf->in_lru = false;
    Node* p = leaf->parent;
    pa_radix::erase_kid(p, leaf, block_hash(leaf->tokens.data(), r->B), leaf->tokens[0]);
    r->n_blocks -= (int64_t)leaf->blocks.size();
    if (count < cap) ids_out[count] = leaf->id;
    ++count;
    r->nodes.erase(leaf->id);
    delete leaf;
    r->refresh(p);   // cascading eligibility
  }
  if (n_evicted) *n_evicted = count;
  return rc;
}

pa_status pa_radix_info(const pa_radix* r, int64_t* nodes, int64_t* blocks, int64_t* dormant,
                        int64_t* pinned) {
  if (!r) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(r->mu);
  if (nodes) *nodes = (int64_t)r->nodes.size();
  if (blocks) *blocks = r->n_blocks;
  if (dormant) *dormant = (int64_t)r->lru.size();
  if (pinned) *pinned = r->n_pinned;
  return PA_OK;
}

pa_status pa_radix_node_ids(const pa_radix* r, int64_t* ids_out, int64_t cap, int64_t* n_out) {
  if (!r || cap < 0 || (cap > 0 && !ids_out) || !n_out) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(r->mu);
  std::vector<int64_t> ids;
  ids.reserve(r->nodes.size());
  for (auto& kv : r->nodes) ids.push_back(kv.first);
  std::sort(ids.begin(), ids.end());
  for (int64_t i = 0; i < (int64_t)ids.size() && i < cap; ++i) ids_out[i] = ids[i];
  *n_out = (int64_t)ids.size();
  return PA_OK;
}

pa_status pa_radix_node(const pa_radix* r, int64_t id, int64_t* meta_out, int32_t* tokens_out,
                        int64_t tok_cap, int32_t* blocks_out, int32_t blk_cap) {
  if (!r || !meta_out || tok_cap < 0 || blk_cap < 0 || (tok_cap > 0 && !tokens_out) ||
      (blk_cap > 0 && !blocks_out))
    return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(r->mu);
  auto it = r->nodes.find(id);
  if (it == r->nodes.end()) return PA_ERR_NOT_FOUND;
  const Node* n = it->second;
  meta_out[0] = n->parent->id;
  meta_out[1] = n->ref;
  meta_out[2] = (int64_t)n->last;
  meta_out[3] = (int64_t)n->blocks.size();
  int64_t nt = std::min<int64_t>(tok_cap, (int64_t)n->tokens.size());
  std::copy(n->tokens.begin(), n->tokens.begin() + nt, tokens_out);
  int64_t nbk = std::min<int64_t>(blk_cap, (int64_t)n->blocks.size());
  std::copy(n->blocks.begin(), n->blocks.begin() + nbk, blocks_out);
  return PA_OK;
}

}  // extern "C"
