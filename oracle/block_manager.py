"""Reference block manager (oracle): free list, reference counts, block tables.

Passages followed:

* "KV Cache Management", section "The PagedAttention virtual memory model": a
  token at offset o != 0 goes into the already allocated block T[l]; at o == 0
  a free block id is popped and appended to the table.
* Same page, Table 3 / section "Asynchronous paged swapping": free ids are kept
  in a FIFO queue. The reading taken: pop from the front, return freed ids at
  the back, and start from an order the caller gives.
* Same page, section "Zero-copy deliberation via copy-on-write branching":
  fork = duplicate the table, increment every listed block's count, give the
  child the parent's length; a write into a block whose count is above one
  first takes a new block, copies the shared one into it, decrements the old
  count and remaps the table entry; release decrements every block of the table
  and returns those reaching zero to the free list.
* "PagedAttention" (Inference book), sections "Paging", "It is the same
  function" and "Inference Lab increment": out-of-blocks and double-free are
  errors, and a reservation that cannot be met leaks nothing.
* "KV Cache Management", section "Asynchronous paged swapping": swapping out
  releases a sequence's frames to the free queue and marks the table entries as
  not resident; swapping in takes fresh frames and remaps the entries.
  The asynchronous form of the same section (steps 1-3 of the migration):
  a contiguous run of frames is taken from a pre-allocated pinned host pool,
  the copy runs in the background, and only when it completes are the entries
  retagged from the accelerator tier to the host tier (with their host frame
  indices) and the vacated accelerator blocks pushed to the free queue. The
  return path mirrors it: fresh blocks are reserved first, the entries point at
  them once the copy back completes, and the host frames are released.
* "KV Cache Management", section "Prefix Caching Across Turns" (block-aligned
  truncation): a request that hits a cached prefix starts with the cached full
  blocks as the first entries of its table, one more reference each, and a
  length of that many whole blocks; its own tokens go into fresh blocks.

Every operation checks all of its preconditions before it changes anything, so a
failed call leaves the manager exactly as it was.
"""

from __future__ import annotations

from collections import deque


class BlockManagerError(Exception):
    pass


class OutOfBlocks(BlockManagerError):
    pass


class DoubleFree(BlockManagerError):
    pass


class InvalidArgument(BlockManagerError):
    pass


NOT_RESIDENT = -1

# Residency tags of a table entry ("KV Cache Management", "Asynchronous paged
# swapping": the extended block table's TIER_HBM / TIER_HOST tags, plus the two
# in-flight states of the asynchronous migration).
TIER_HBM, TIER_HOST, TIER_PENDING_OUT, TIER_PENDING_IN = 0, 1, 2, 3


class OutOfFrames(BlockManagerError):
    pass


class HostPool:
    """Frames 0..F-1 of a pinned host buffer; runs of consecutive frames are
    handed out first-fit (lowest start) and freed runs merge with neighbours."""

    def __init__(self, num_frames):
        if num_frames < 1:
            raise InvalidArgument("num_frames must be positive")
        self.num_frames = num_frames
        self.free_runs = [(0, num_frames)]      # sorted, non-adjacent (start, length)
        self.used = [False] * num_frames

    def num_free(self):
        return sum(n for _, n in self.free_runs)

    def alloc_run(self, n):
        if n < 1:
            raise InvalidArgument("run length must be positive")
        for k, (start, length) in enumerate(self.free_runs):
            if length >= n:
                if length == n:
                    del self.free_runs[k]
                else:
                    self.free_runs[k] = (start + n, length - n)
                for f in range(start, start + n):
                    self.used[f] = True
                return start
        raise OutOfFrames(f"no run of {n} free frames")

    def free(self, frames):
        frames = [int(f) for f in frames]
        if len(set(frames)) != len(frames):
            raise DoubleFree("frame listed twice")
        for f in frames:
            if not 0 <= f < self.num_frames:
                raise InvalidArgument(f"frame {f} out of range")
            if not self.used[f]:
                raise DoubleFree(f"frame {f} is not allocated")
        for f in frames:
            self.used[f] = False
        # rebuild the run list from the used map (plain and obviously correct)
        runs, f = [], 0
        while f < self.num_frames:
            if self.used[f]:
                f += 1
                continue
            g = f
            while g < self.num_frames and not self.used[g]:
                g += 1
            runs.append((f, g - f))
            f = g
        self.free_runs = runs


class BlockManager:
    def __init__(self, num_blocks, block_size, free_order=None):
        if num_blocks < 1 or block_size < 1:
            raise InvalidArgument("num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if free_order is None else [int(x) for x in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise InvalidArgument("free_order must be a permutation of 0..N-1")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = deque(order)
        self.ref = [0] * num_blocks
        self.tables = {}
        self.lengths = {}
        self._next_seq = 0
        self.host_pool = None
        self.host = {}       # sid -> {logical: host frame} (entries in the host tier)
        self.pending = {}    # sid -> {logical: ("out", phys, frame) | ("in", phys, frame)}

    # ---- raw allocator -------------------------------------------------------
    def num_free(self):
        return len(self.free)

    def refcount(self, block):
        return self.ref[block]

    def alloc(self, n):
        """Take n blocks (count 1 each), all or none."""
        if n < 0:
            raise InvalidArgument("negative count")
        if n > len(self.free):
            raise OutOfBlocks(f"need {n}, have {len(self.free)}")
        out = [self.free.popleft() for _ in range(n)]
        for b in out:
            self.ref[b] = 1
        return out

    def incref(self, ids):
        for b in ids:
            if not 0 <= b < self.num_blocks or self.ref[b] == 0:
                raise InvalidArgument(f"block {b} is not allocated")
        for b in ids:
            self.ref[b] += 1

    def free_blocks(self, ids):
        """Drop one reference from each id; ids reaching zero go back to the queue."""
        pending = {}
        for b in ids:
            if not 0 <= b < self.num_blocks:
                raise InvalidArgument(f"block {b} out of range")
            pending[b] = pending.get(b, 0) + 1
            if pending[b] > self.ref[b]:
                raise DoubleFree(f"block {b} has no reference left to drop")
        for b in ids:
            self._decref(b)

    def _decref(self, b):
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free.append(b)

    # ---- sequences -----------------------------------------------------------
    def _check_seq(self, sid):
        if sid not in self.tables:
            raise InvalidArgument(f"unknown sequence {sid}")

    def seq_new(self):
        sid = self._next_seq
        self._next_seq += 1
        self.tables[sid] = []
        self.lengths[sid] = 0
        return sid

    def seq_from_blocks(self, ids):
        """New sequence whose table is `ids` (allocated blocks, one more reference
        each) and whose length is len(ids) * B."""
        ids = [int(b) for b in ids]
        for b in ids:
            if not 0 <= b < self.num_blocks or self.ref[b] == 0:
                raise InvalidArgument(f"block {b} is not allocated")
        sid = self.seq_new()
        for b in ids:
            self.ref[b] += 1
        self.tables[sid] = ids
        self.lengths[sid] = len(ids) * self.block_size
        return sid

    def fork(self, parent):
        self._check_seq(parent)
        table = self.tables[parent]
        if any(p == NOT_RESIDENT for p in table) or self.pending.get(parent):
            raise InvalidArgument("cannot fork a sequence with blocks swapped out or in flight")
        child = self._next_seq
        self._next_seq += 1
        self.tables[child] = list(table)            # 1. duplicate the table
        for p in table:                             # 2. one more reference each
            self.ref[p] += 1
        self.lengths[child] = self.lengths[parent]  # 3. same starting length
        return child

    def blocks_needed(self, sid, n):
        """(copy-on-write blocks, fresh blocks) an append of n tokens would take."""
        table, S, B = self.tables[sid], self.lengths[sid], self.block_size
        cow = 0
        if n > 0 and S % B != 0:
            tail = table[S // B]
            if tail == NOT_RESIDENT or (S // B) in self.pending.get(sid, {}):
                raise InvalidArgument("tail block is swapped out or in flight")
            if self.ref[tail] > 1:
                cow = 1
        fresh = sum(1 for t in range(S, S + n) if t % B == 0)
        return cow, fresh

    def append(self, sid, n):
        """Reserve room for n more tokens; returns (slots, copy_pairs).

        slots[k] is the flat slot (block * B + offset) of token S + k, and
        copy_pairs lists (src, dst) block copies that must run before the write.
        """
        self._check_seq(sid)
        if n < 0:
            raise InvalidArgument("negative token count")
        cow, fresh = self.blocks_needed(sid, n)
        if cow + fresh > len(self.free):
            raise OutOfBlocks(f"need {cow + fresh}, have {len(self.free)}")
        table, S, B = self.tables[sid], self.lengths[sid], self.block_size
        pairs = []
        if cow:
            lb = S // B
            old = table[lb]
            new = self.free.popleft()
            self.ref[new] = 1
            self.ref[old] -= 1          # still >= 1: another owner keeps it
            table[lb] = new
            pairs.append((old, new))
        slots = []
        for t in range(S, S + n):
            lb, off = t // B, t % B
            if off == 0:
                new = self.free.popleft()
                self.ref[new] = 1
                table.append(new)
            slots.append(table[lb] * B + off)
        self.lengths[sid] = S + n
        return slots, pairs

    def release(self, sid):
        """Decrement every block of the table; blocks reaching zero are freed.
        Host frames the sequence holds go back to the host pool; a sequence with
        a migration in flight cannot be released."""
        self._check_seq(sid)
        if self.pending.get(sid):
            raise InvalidArgument("migration in flight")
        for p in self.tables[sid]:
            if p != NOT_RESIDENT:
                self._decref(p)
        frames = list(self.host.pop(sid, {}).values())
        if frames:
            self.host_pool.free(frames)
        self.pending.pop(sid, None)
        del self.tables[sid]
        del self.lengths[sid]

    def swap_out(self, sid, logical):
        """Drop the sequence's reference to the listed logical blocks; returns
        the physical ids they had (in list order)."""
        self._check_seq(sid)
        table = self.tables[sid]
        if len(set(logical)) != len(logical):
            raise InvalidArgument("repeated logical block")
        for lb in logical:
            if not 0 <= lb < len(table) or table[lb] == NOT_RESIDENT or lb in self.pending.get(sid, {}):
                raise InvalidArgument(f"logical block {lb} is not resident or is in flight")
        phys = [table[lb] for lb in logical]
        for lb in logical:
            self._decref(table[lb])
            table[lb] = NOT_RESIDENT
        return phys

    def swap_in(self, sid, logical):
        """Give the listed non-resident logical blocks fresh physical blocks."""
        self._check_seq(sid)
        table = self.tables[sid]
        if len(set(logical)) != len(logical):
            raise InvalidArgument("repeated logical block")
        for lb in logical:
            if (not 0 <= lb < len(table) or table[lb] != NOT_RESIDENT or lb in self.host.get(sid, {})
                    or lb in self.pending.get(sid, {})):
                raise InvalidArgument(f"logical block {lb} is resident, pool-held or in flight")
        if len(logical) > len(self.free):
            raise OutOfBlocks(f"need {len(logical)}, have {len(self.free)}")
        out = []
        for lb in logical:
            p = self.free.popleft()
            self.ref[p] = 1
            table[lb] = p
            out.append(p)
        return out

    # ---- asynchronous migration between tiers -------------------------------
    def attach_host_pool(self, pool):
        self.host_pool = pool

    def _check_logical(self, sid, logical):
        self._check_seq(sid)
        if len(logical) == 0 or len(set(logical)) != len(logical):
            raise InvalidArgument("empty or repeated logical block list")
        for lb in logical:
            if not 0 <= lb < len(self.tables[sid]):
                raise InvalidArgument(f"logical block {lb} out of range")

    def tier(self, sid, lb):
        """(tag, index): index is the physical block for TIER_HBM / TIER_PENDING_OUT
        and the host frame for TIER_HOST / TIER_PENDING_IN."""
        self._check_seq(sid)
        if not 0 <= lb < len(self.tables[sid]):
            raise InvalidArgument(f"logical block {lb} out of range")
        pend = self.pending.get(sid, {}).get(lb)
        if pend is not None:
            kind, phys, frame = pend
            return (TIER_PENDING_OUT, phys) if kind == "out" else (TIER_PENDING_IN, frame)
        if lb in self.host.get(sid, {}):
            return TIER_HOST, self.host[sid][lb]
        if self.tables[sid][lb] == NOT_RESIDENT:
            return TIER_HOST, -1        # swapped out by the caller-managed path: no pool frame
        return TIER_HBM, self.tables[sid][lb]

    def swap_out_begin(self, sid, logical):
        """Step 1: take a contiguous run of host frames for the listed resident
        blocks (frame first + k for logical[k]); the blocks stay allocated and
        readable until swap_out_finish. Returns (physical ids, first frame)."""
        if self.host_pool is None:
            raise InvalidArgument("no host pool attached")
        self._check_logical(sid, logical)
        for lb in logical:
            if self.tier(sid, lb)[0] != TIER_HBM:
                raise InvalidArgument(f"logical block {lb} is not resident in HBM")
        first = self.host_pool.alloc_run(len(logical))
        pend = self.pending.setdefault(sid, {})
        phys = []
        for k, lb in enumerate(logical):
            p = self.tables[sid][lb]
            pend[lb] = ("out", p, first + k)
            phys.append(p)
        return phys, first

    def swap_out_finish(self, sid, logical):
        """Step 3 (the copy completed): retag the entries as host-resident with
        their frames and drop the sequence's references to the HBM blocks."""
        self._check_logical(sid, logical)
        pend = self.pending.get(sid, {})
        for lb in logical:
            if pend.get(lb, ("",))[0] != "out":
                raise InvalidArgument(f"logical block {lb} has no swap-out in flight")
        host = self.host.setdefault(sid, {})
        for lb in logical:
            _, p, frame = pend.pop(lb)
            self._decref(p)
            self.tables[sid][lb] = NOT_RESIDENT
            host[lb] = frame

    def swap_in_begin(self, sid, logical):
        """Reserve fresh HBM blocks (all or none) for host-resident entries; the
        entries stay non-resident until swap_in_finish. Returns (new physical
        ids, host frames) in list order."""
        self._check_logical(sid, logical)
        for lb in logical:
            tag, frame = self.tier(sid, lb)
            if tag != TIER_HOST or frame < 0:
                raise InvalidArgument(f"logical block {lb} is not in the host pool tier")
        if len(logical) > len(self.free):
            raise OutOfBlocks(f"need {len(logical)}, have {len(self.free)}")
        pend = self.pending.setdefault(sid, {})
        phys, frames = [], []
        for lb in logical:
            p = self.free.popleft()
            self.ref[p] = 1
            frame = self.host[sid][lb]
            pend[lb] = ("in", p, frame)
            phys.append(p)
            frames.append(frame)
        return phys, frames

    def swap_in_finish(self, sid, logical):
        """The copy back completed: entries point at their new blocks and the
        host frames return to the pool."""
        self._check_logical(sid, logical)
        pend = self.pending.get(sid, {})
        for lb in logical:
            if pend.get(lb, ("",))[0] != "in":
                raise InvalidArgument(f"logical block {lb} has no swap-in in flight")
        frames = []
        for lb in logical:
            _, p, frame = pend.pop(lb)
            self.tables[sid][lb] = p
            del self.host[sid][lb]
            frames.append(frame)
        self.host_pool.free(frames)

    def permute_free(self, perm):
        """Reorder the free queue: entry k becomes the current entry perm[k]."""
        perm = [int(x) for x in perm]
        if sorted(perm) != list(range(len(self.free))):
            raise InvalidArgument("perm must be a permutation of the free positions")
        cur = list(self.free)
        self.free = deque(cur[k] for k in perm)

    def table(self, sid):
        self._check_seq(sid)
        return list(self.tables[sid])

    def length(self, sid):
        self._check_seq(sid)
        return self.lengths[sid]

    def blocks_in_use(self):
        return self.num_blocks - len(self.free)
