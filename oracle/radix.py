"""Radix prefix cache over the block manager (oracle; test infrastructure).

Passages followed ("KV Cache Management", section "Prefix Caching Across
Turns"):

* Table 4 and Definition 0.2: a node binds a slice of token ids (prefix_tokens)
  to the ordered physical block ids backing it (block_ids), with a children map,
  a parent, a ref_count (requests currently using the node) and a last_access
  timestamp; non-branching stretches are one node (radix compaction).
* "Longest prefix matching": walk from the root matching slices of the prompt;
  S_match is the longest matched prefix; only fully packed blocks are shared,
  so the usable hit is S_usable = floor(S_match / B) * B (block-aligned
  truncation) and the tail is recomputed.
* "Dynamic radix eviction": nodes with ref_count >= 1 are pinned; dormant
  (ref_count == 0) leaves are eviction candidates, least recently used first;
  evicting a leaf releases its blocks and removes it from its parent; a parent
  left without children and with ref_count == 0 becomes a candidate in turn;
  eviction stops once the free pool holds the target number of blocks.

Readings taken (the pages leave them open):

* Because only full blocks are shared, every node holds a whole number of
  blocks and edges split only at block boundaries; children are keyed by the B
  tokens of their first block (the "next branch token" of a token-level tree,
  at block granularity).
* The tree owns one block-manager reference per block it indexes; eviction
  drops that reference (a block still used by a live sequence stays allocated
  until the sequence releases it).
* A match pins every node on the matched path, including a node only partly
  used; last_access is a logical clock that ticks once per match or insert.
* Inserting tokens that the tree already holds keeps the tree's blocks; the
  caller's duplicate blocks are not adopted. A node split keeps the deeper part
  (with the children, ref_count and last_access) as the original node object so
  that handles to it stay valid; the new upper node copies ref_count and
  last_access.
"""

from __future__ import annotations

from .block_manager import BlockManager, InvalidArgument


class Node:
    def __init__(self, node_id, tokens, blocks, parent):
        self.id = node_id
        self.prefix_tokens = list(tokens)
        self.block_ids = list(blocks)
        self.children = {}                  # tuple(first B tokens) -> Node
        self.parent = parent
        self.ref_count = 0
        self.last_access = 0


class RadixCache:
    def __init__(self, bm: BlockManager):
        self.bm = bm
        self.B = bm.block_size
        self.root = Node(0, [], [], None)
        self.clock = 0
        self._next_id = 1
        self.nodes = {0: self.root}

    # ---- helpers -------------------------------------------------------------
    def _tick(self):
        self.clock += 1
        return self.clock

    def _key(self, tokens, pos):
        return tuple(tokens[pos:pos + self.B])

    def _walk(self, tokens):
        """Nodes fully matched, the partly matched node (or None) with the number of
        its blocks matched, and the token-level match length S_match."""
        B = self.B
        path, node, pos = [], self.root, 0
        partial, partial_blocks = None, 0
        s_match = 0
        while True:
            child = node.children.get(self._key(tokens, pos)) if pos + B <= len(tokens) else None
            if child is None:
                # token-level match into the first block of any child (S_match only)
                best = 0
                for c in node.children.values():
                    k = 0
                    while (k < B and pos + k < len(tokens) and k < len(c.prefix_tokens)
                           and c.prefix_tokens[k] == tokens[pos + k]):
                        k += 1
                    best = max(best, k)
                s_match = pos + best
                break
            j = 0                                      # whole blocks of child matched
            nb = len(child.block_ids)
            while j < nb and pos + (j + 1) * B <= len(tokens) and \
                    child.prefix_tokens[j * B:(j + 1) * B] == tokens[pos + j * B:pos + (j + 1) * B]:
                j += 1
            if j == nb:
                path.append(child)
                node, pos = child, pos + nb * B
                continue
            partial, partial_blocks = child, j
            k = 0                                      # tokens of the next block that still match
            while (k < B and pos + j * B + k < len(tokens) and
                   child.prefix_tokens[j * B + k] == tokens[pos + j * B + k]):
                k += 1
            s_match = pos + j * B + k
            break
        return path, partial, partial_blocks, s_match

    # ---- lookups -------------------------------------------------------------
    def match(self, tokens):
        """(S_match, S_usable, block ids of the usable prefix, handle). Pins the
        matched path; the handle (a node id) unpins it."""
        tokens = [int(t) for t in tokens]
        path, partial, pb, s_match = self._walk(tokens)
        blocks = [b for n in path for b in n.block_ids]
        pinned = list(path)
        if partial is not None and pb > 0:
            blocks += partial.block_ids[:pb]
            pinned.append(partial)
        s_usable = len(blocks) * self.B
        assert s_usable == (s_match // self.B) * self.B
        t = self._tick()
        for n in pinned:
            n.ref_count += 1
            n.last_access = t
        handle = pinned[-1].id if pinned else 0
        return s_match, s_usable, blocks, handle

    def unpin(self, handle):
        if handle not in self.nodes:
            raise InvalidArgument(f"unknown node {handle}")
        n = self.nodes[handle]
        chain = []
        while n is not self.root:
            if n.ref_count == 0:
                raise InvalidArgument("node is not pinned")
            chain.append(n)
            n = n.parent
        for n in chain:
            n.ref_count -= 1

    def insert(self, tokens, blocks):
        """Index the whole blocks of a sequence: blocks[k] holds tokens[kB:(k+1)B].
        Returns how many of the caller's blocks the tree adopted (took a
        reference on)."""
        B = self.B
        tokens = [int(t) for t in tokens]
        nb = min(len(blocks), len(tokens) // B)
        tokens, blocks = tokens[:nb * B], [int(b) for b in blocks[:nb]]
        path, partial, pb, _ = self._walk(tokens)
        done = sum(len(n.block_ids) for n in path)
        split = partial is not None and pb > 0
        start = done + (pb if split else 0)           # first block the tree lacks
        if start < nb:
            self.bm.incref(blocks[start:])            # checks every id before any change
        t = self._tick()
        for n in path + ([partial] if split else []):
            n.last_access = t
        if start >= nb:                               # every block already indexed
            return 0
        node = path[-1] if path else self.root
        if split:                                     # the partly matched node splits after pb blocks
            upper = Node(self._next_id, partial.prefix_tokens[:pb * B], partial.block_ids[:pb],
                         partial.parent)
            self._next_id += 1
            self.nodes[upper.id] = upper
            upper.ref_count = partial.ref_count
            upper.last_access = t
            partial.parent.children[self._key(upper.prefix_tokens, 0)] = upper
            partial.prefix_tokens = partial.prefix_tokens[pb * B:]
            partial.block_ids = partial.block_ids[pb:]
            partial.parent = upper
            upper.children[self._key(partial.prefix_tokens, 0)] = partial
            node = upper
        new = Node(self._next_id, tokens[start * B:], blocks[start:], node)
        self._next_id += 1
        self.nodes[new.id] = new
        new.last_access = t
        node.children[self._key(new.prefix_tokens, 0)] = new
        return len(new.block_ids)

    # ---- eviction ------------------------------------------------------------
    def dormant_leaves(self):
        return [n for n in self.nodes.values()
                if n is not self.root and not n.children and n.ref_count == 0]

    def evict(self, target_free):
        """Evict least recently used dormant leaves (ties: lower node id) until
        the block manager has target_free free blocks or none is left. Returns
        the evicted node ids in order."""
        out = []
        while self.bm.num_free() < target_free:
            cand = self.dormant_leaves()
            if not cand:
                break
            leaf = min(cand, key=lambda n: (n.last_access, n.id))
            self.bm.free_blocks(leaf.block_ids)
            del leaf.parent.children[self._key(leaf.prefix_tokens, 0)]
            del self.nodes[leaf.id]
            out.append(leaf.id)
        return out

    def cached_blocks(self):
        return sum(len(n.block_ids) for n in self.nodes.values())
