"""Prefix-cache scenarios shared by the oracle's pins (test_oracle_radix.py) and the
library's tests (test_radix.py). Each takes an `impl` adapter:

  impl.make(num_blocks, block_size, free_order=None) -> (bm, tree)
  impl.free_list(bm) -> free block ids, front first
  impl.nodes(tree) -> {id: (parent, ref_count, last_access, tokens, blocks)}, root excluded

and checks what the pages fix ("KV Cache Management", section "Prefix Caching
Across Turns") through behaviour a caller sees: the longest cached prefix, the
block-aligned usable part, which blocks come back, which blocks eviction frees
and in what order, and the reference counts of the block manager.
"""
import json
import os

import numpy as np

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "radix.json")))


def order(n, head):
    return list(head) + [b for b in range(n) if b not in head]


def run_request(bm, tree, tokens, keep_pinned=False):
    """Serve one request the way the pages describe: resolve the longest cached
    prefix, start the sequence from its full blocks, fill the rest with fresh
    blocks, then hand the finished request's blocks to the tree and release the
    sequence. Returns (s_match, s_usable, matched blocks, handle, table)."""
    s_match, s_usable, blocks, handle = tree.match(tokens)
    sid = bm.seq_from_blocks(blocks)
    bm.append(sid, len(tokens) - s_usable)
    table = bm.table(sid)
    tree.insert(tokens, table)
    if not keep_pinned:
        tree.unpin(handle)
    bm.release(sid)
    return s_match, s_usable, blocks, handle, table


def lcp(a, b):
    k = 0
    while k < len(a) and k < len(b) and a[k] == b[k]:
        k += 1
    return k


# ---- the pages' worked examples -------------------------------------------------
def truncation_example(impl):
    c = GOLD["truncation_example"]
    B = c["block_size"]
    bm, tree = impl.make(c["num_blocks"], B)
    rng = np.random.default_rng(1)
    cached = [int(x) for x in rng.integers(1000, 2000, c["cached_tokens"])]
    run_request(bm, tree, cached)
    shared = c["shared_tokens"]
    prompt = cached[:shared] + [int(x) for x in rng.integers(5000, 6000, c["prompt_tokens"] - shared)]
    s_match, s_usable, blocks, handle = tree.match(prompt)
    assert s_match == c["expect_s_match"]
    assert s_usable == c["expect_s_usable"]
    assert len(blocks) == c["expect_full_blocks"]
    assert s_match - s_usable == c["expect_tail_tokens"]
    # the reused blocks are the cached request's first blocks, in order
    assert blocks == _cached_table(bm, tree, cached)[:len(blocks)]
    tree.unpin(handle)


def _cached_table(bm, tree, tokens):
    _, _, blocks, handle = tree.match(tokens)
    tree.unpin(handle)
    return blocks


def napkin_prefix_hit(impl):
    c = GOLD["napkin_0_4"]
    B = c["block_size"]
    n_blocks = c["expect_blocks"] + 8
    bm, tree = impl.make(n_blocks, B)
    rng = np.random.default_rng(2)
    system = [int(x) for x in rng.integers(0, 32000, c["prefix_tokens"])]
    run_request(bm, tree, system + [7] * 5)
    query = [int(x) for x in rng.integers(0, 32000, c["novel_tokens"])]
    s_match, s_usable, blocks, handle = tree.match(system + query)
    assert s_usable == c["expect_s_usable"] and len(blocks) == c["expect_blocks"]
    assert len(system + query) - s_usable == c["expect_prefill_tokens"]
    tree.unpin(handle)


def figure7_worker(impl):
    c = GOLD["figure7_worker"]
    B = c["block_size"]
    bm, tree = impl.make(c["prompt_tokens"] // B + 16, B)
    rng = np.random.default_rng(3)
    prompt = [int(x) for x in rng.integers(0, 50000, c["prompt_tokens"])]
    run_request(bm, tree, prompt[:c["cached_tokens"]])
    s_match, s_usable, blocks, handle = tree.match(prompt)
    assert s_usable == c["expect_s_usable"]
    assert len(blocks) == c["expect_blocks_skipped"]
    assert len(prompt) - s_usable == c["expect_prefill_tokens"]
    assert s_usable / len(prompt) == c["expect_hit_fraction"]
    tree.unpin(handle)


def figure6_eviction(impl):
    """Figure 6: two pinned nodes (system prompt, Python scratchpad) and a dormant
    chain (Bash shell, then Git status below it); eviction takes Git status first
    (block 31), then Bash shell, and never a pinned node."""
    c = GOLD["figure6_eviction"]
    B = c["block_size"]
    nb = c["node_blocks"]
    head = nb["system"] + nb["python"] + nb["bash"] + nb["git"]
    bm, tree = impl.make(64, B, order(64, head))
    tok = {}
    base = 100
    for name in ("system", "python", "bash", "git"):
        tok[name] = list(range(base, base + len(nb[name]) * B))
        base += 1000
    # earlier traffic: a Python turn, a Bash turn, then the Git turn that extends it
    run_request(bm, tree, tok["system"] + tok["python"])
    run_request(bm, tree, tok["system"] + tok["bash"])
    run_request(bm, tree, tok["system"] + tok["bash"] + tok["git"])
    got = {name: _cached_table(bm, tree, _path(tok, name))[-len(nb[name]):]
           for name in ("system", "python", "bash", "git")}
    assert got == nb
    # a Python request is running: system prompt and scratchpad are pinned
    _, _, _, running = tree.match(tok["system"] + tok["python"] + [9, 9, 9])
    first = tree.evict(bm.num_free() + 1)
    assert len(first) == 1
    assert impl.free_list(bm)[-len(c["expect_first_freed"]):] == c["expect_first_freed"]
    assert _cached_table(bm, tree, _path(tok, "git")) == nb["system"] + nb["bash"]
    second = tree.evict(bm.num_free() + 1)
    assert len(second) == 1
    assert impl.free_list(bm)[-len(nb["bash"]):] == nb["bash"]
    assert tree.evict(10 ** 6) == []                       # only pinned nodes are left
    assert _cached_table(bm, tree, _path(tok, "python")) == nb["system"] + nb["python"]
    tree.unpin(running)
    assert len(tree.evict(10 ** 6)) == 2                   # both dormant now: scratchpad, then system
    assert impl.free_list(bm)[-3:] == nb["python"] + nb["system"]
    assert bm.num_free() == 64


def _path(tok, name):
    if name == "system":
        return tok["system"]
    if name == "python":
        return tok["system"] + tok["python"]
    if name == "bash":
        return tok["system"] + tok["bash"]
    return tok["system"] + tok["bash"] + tok["git"]


# ---- brute force: the longest prefix over everything inserted ------------------------
def conversations(seed, n_conv, B, vocab=4):
    """Multi-turn traffic: a few system prompts, conversations that append turns
    (history grows), and tokens from a tiny vocabulary so that sequences often
    agree for part of a block."""
    rng = np.random.default_rng(seed)
    systems = [[int(x) for x in rng.integers(0, vocab, int(rng.integers(0, 4 * B)))]
               for _ in range(3)]
    reqs = []
    for _ in range(n_conv):
        hist = list(systems[int(rng.integers(0, 3))])
        for _ in range(int(rng.integers(1, 4))):
            hist = hist + [int(x) for x in rng.integers(0, vocab, int(rng.integers(1, 2 * B + 3)))]
            reqs.append(list(hist))
    order_ = rng.permutation(len(reqs))
    return [reqs[i] for i in order_]


def brute_force_prefixes(impl, seed, B):
    reqs = conversations(seed, 14, B)
    need = sum(len(r) // B + 2 for r in reqs) + 8
    bm, tree = impl.make(need, B)
    flat = {}                         # prefix of k full blocks -> block id (first inserter)
    stored = []                       # token lists truncated to full blocks
    for r in reqs:
        s_match, s_usable, blocks, handle, table = run_request(bm, tree, r)
        exp = max([lcp(r, s) for s in stored], default=0)
        assert s_match == exp, (s_match, exp)
        assert s_usable == (exp // B) * B
        assert blocks == [flat[tuple(r[:(k + 1) * B])] for k in range(s_usable // B)]
        for k in range(len(r) // B):
            flat.setdefault(tuple(r[:(k + 1) * B]), table[k])
        stored.append(r[:(len(r) // B) * B])
    # probes that diverge inside a block, run past the end, or are empty
    rng = np.random.default_rng(seed + 100)
    for _ in range(40):
        base = stored[int(rng.integers(0, len(stored)))]
        cut = int(rng.integers(0, len(base) + 1))
        probe = base[:cut] + [int(x) for x in rng.integers(0, 5, int(rng.integers(0, 2 * B)))]
        s_match, s_usable, blocks, handle = tree.match(probe)
        exp = max(lcp(probe, s) for s in stored)
        assert s_match == exp and s_usable == (exp // B) * B
        assert blocks == [flat[tuple(probe[:(k + 1) * B])] for k in range(s_usable // B)]
        tree.unpin(handle)
    # the tree holds exactly one reference on each indexed block and nothing else
    held = set(flat.values())
    for b in range(need):
        assert bm.refcount(b) == (1 if b in held else 0)
    assert bm.num_free() == need - len(held)
    return tree, flat


def pin_counts(impl, seed, B):
    """A node's ref_count is the number of outstanding matches that use any of its
    blocks; unpinning every handle brings all counts back to zero."""
    reqs = conversations(seed, 10, B)
    bm, tree = impl.make(sum(len(r) // B + 2 for r in reqs) + 8, B)
    for r in reqs:
        run_request(bm, tree, r)
    rng = np.random.default_rng(seed + 7)
    live = []
    for _ in range(25):
        r = reqs[int(rng.integers(0, len(reqs)))]
        probe = r[:int(rng.integers(0, len(r) + 1))] + [99]
        _, _, blocks, handle = tree.match(probe)
        live.append((set(blocks), handle))
        if rng.random() < 0.3 and live:
            _, h = live.pop(int(rng.integers(0, len(live))))
            tree.unpin(h)
        for nid, (_, ref, _, _, nblocks) in impl.nodes(tree).items():
            assert ref == sum(1 for bs, _ in live if bs & set(nblocks)), nid
    for _, h in live:
        tree.unpin(h)
    assert all(v[1] == 0 for v in impl.nodes(tree).values())


# ---- eviction ------------------------------------------------------------------------
def lru_order(impl, seed, B):
    """Disjoint conversations (one node each) touched in a random order: single
    evictions free them least recently used first."""
    rng = np.random.default_rng(seed)
    K = 9
    bm, tree = impl.make(K * 4 + 4, B)
    convs = [[1000 * (i + 1) + t for t in range(int(rng.integers(1, 4)) * B)] for i in range(K)]
    for c in convs:
        run_request(bm, tree, c)
    tables = [_cached_table(bm, tree, c) for c in convs]
    touch = [int(i) for i in rng.permutation(K)]
    for i in touch:
        _, _, _, h = tree.match(convs[i][:B] + [7])
        tree.unpin(h)
    freed = []
    for _ in range(K):
        before = bm.num_free()
        ev = tree.evict(before + 1)
        assert len(ev) == 1
        got = impl.free_list(bm)[before:]
        freed.append(next(i for i in range(K) if sorted(tables[i]) == sorted(got)))
    assert freed == touch
    assert tree.evict(10 ** 6) == []


def child_first(impl, B):
    """A chain of turns (A, then A+B', then A+B'+C'): touching only the oldest
    part does not let it go before its descendants."""
    bm, tree = impl.make(32, B)
    a = list(range(100, 100 + 2 * B))
    b = list(range(300, 300 + B))
    c = list(range(500, 500 + B))
    run_request(bm, tree, a)
    run_request(bm, tree, a + b)
    run_request(bm, tree, a + b + c)
    ta, tb, tc = (_cached_table(bm, tree, x) for x in (a, a + b, a + b + c))
    _, _, _, h = tree.match(a + [1, 2, 3])                 # most recent access: the root chunk
    tree.unpin(h)
    got = []
    for _ in range(3):
        before = bm.num_free()
        assert len(tree.evict(before + 1)) == 1
        got.append(impl.free_list(bm)[before:])
    assert got == [tc[-1:], tb[-1:], ta]


def eviction_stops_at_target(impl, seed, B):
    """evict(target) stops as soon as the free pool reaches the target: it takes
    exactly the leaves that single evictions, each asking for one more free block,
    take until the target is met."""
    reqs = conversations(seed, 12, B)
    n = sum(len(r) // B + 2 for r in reqs) + 8
    pair = []
    for _ in range(2):
        bm, tree = impl.make(n, B)
        for r in reqs:
            run_request(bm, tree, r)
        pair.append((bm, tree))
    (bm1, t1), (bm2, t2) = pair
    target = bm1.num_free() + 3
    assert t1.evict(bm1.num_free()) == []                  # already met: nothing to do
    ev = t1.evict(target)
    assert bm1.num_free() >= target
    steps = []
    while bm2.num_free() < target:
        one = t2.evict(bm2.num_free() + 1)
        assert len(one) == 1
        steps += one
    assert len(ev) == len(steps)
    assert impl.free_list(bm1) == impl.free_list(bm2)


def shared_with_live_sequence(impl, B):
    """Evicting a node whose blocks a live sequence still uses drops only the
    tree's reference; the blocks stay allocated for that sequence."""
    bm, tree = impl.make(16, B)
    a = list(range(10, 10 + 2 * B))
    run_request(bm, tree, a)
    _, _, blocks, h = tree.match(a)
    sid = bm.seq_from_blocks(blocks)
    tree.unpin(h)
    free0 = bm.num_free()
    assert len(tree.evict(10 ** 6)) == 1
    assert bm.num_free() == free0
    assert all(bm.refcount(b) == 1 for b in blocks)
    assert tree.match(a)[1] == 0
    bm.release(sid)
    assert bm.num_free() == 16


def random_with_eviction(impl, seed, B):
    """Traffic under memory pressure. After every request: the index is
    prefix-closed, holds one reference per indexed block and the block manager's
    counts are exactly those references; the request just served matches in full
    with its own table; every surviving block is one that a request which had that
    prefix held; blocks of running (pinned) requests are never freed."""
    rng = np.random.default_rng(seed)
    reqs = conversations(seed, 24, B)
    N = 40
    bm, tree = impl.make(N, B)
    history = {}                                # prefix of k full blocks -> block ids seen
    live = []                                   # (blocks, handle) of running requests
    evictions = 0
    for r in reqs:
        r = r[:(N // 3 - 2) * B]
        need = len(r) // B + 2
        if bm.num_free() < need:
            evictions += len(tree.evict(need))
            for bs, _ in live:
                assert all(bm.refcount(b) >= 1 for b in bs)
        if bm.num_free() < need:
            for _, h in live:
                tree.unpin(h)
            live = []
            evictions += len(tree.evict(need))
        assert bm.num_free() >= need
        _, _, blocks, handle, table = run_request(bm, tree, r, keep_pinned=True)
        if rng.random() < 0.5:
            live.append((blocks, handle))
        else:
            tree.unpin(handle)
        full = len(r) // B
        for k in range(full):
            history.setdefault(tuple(r[:(k + 1) * B]), set()).add(table[k])
        got = _cached_table(bm, tree, r)
        assert got == table[:full]
        nodes = impl.nodes(tree)
        held = {}
        for nid, (parent, ref, _, tokens, nblocks) in nodes.items():
            assert parent == 0 or parent in nodes
            assert len(tokens) == len(nblocks) * B and len(nblocks) > 0
            for blk in nblocks:
                held[blk] = held.get(blk, 0) + 1
        assert all(v == 1 for v in held.values())
        for b in range(N):
            assert bm.refcount(b) == held.get(b, 0)
        for nid, toks in _paths(nodes).items():
            blks = _path_blocks(nodes, nid)
            for k in range(len(blks)):
                assert blks[k] in history[tuple(toks[:(k + 1) * B])]
    assert evictions > 0
    for _, h in live:
        tree.unpin(h)
    tree.evict(10 ** 6)
    assert bm.num_free() == N and impl.nodes(tree) == {}


def _paths(nodes):
    out = {}
    for nid in nodes:
        toks, cur = [], nid
        while cur != 0:
            toks = list(nodes[cur][3]) + toks
            cur = nodes[cur][0]
        out[nid] = toks
    return out


def _path_blocks(nodes, nid):
    blks, cur = [], nid
    while cur != 0:
        blks = list(nodes[cur][4]) + blks
        cur = nodes[cur][0]
    return blks
