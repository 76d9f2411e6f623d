"""Pins of the oracle's tiered residency ("KV Cache Management", section
"Asynchronous paged swapping", steps 1-3 of the migration and the return path):
hand-worked host-pool runs, the order of events the page gives (frames taken at
the start, blocks freed to the back of the FIFO only when the copy completes),
all-or-nothing failures, and conservation of blocks and frames."""
import random

import pytest

from oracle import block_manager as obm
from oracle.block_manager import (TIER_HBM, TIER_HOST, TIER_PENDING_IN, TIER_PENDING_OUT,
                                  BlockManager, HostPool)


def test_host_pool_exact_sequence():
    """Hand-worked: runs are taken first fit from the lowest frame, and a freed
    run merges with free neighbours."""
    hp = HostPool(10)
    assert hp.alloc_run(3) == 0            # frames 0-2
    assert hp.alloc_run(4) == 3            # frames 3-6
    hp.free([0, 1, 2])
    assert hp.free_runs == [(0, 3), (7, 3)]
    assert hp.alloc_run(3) == 0            # the lowest run that fits
    with pytest.raises(obm.OutOfFrames):   # 3 frames free (7-9) but not 4 in a row
        hp.alloc_run(4)
    hp.free([3, 4, 5, 6])
    assert hp.free_runs == [(3, 7)]         # merged with the tail run 7-9
    assert hp.alloc_run(7) == 3
    assert hp.num_free() == 0
    hp.free([9])
    with pytest.raises(obm.DoubleFree):
        hp.free([9])


def test_host_pool_errors_change_nothing():
    hp = HostPool(4)
    hp.alloc_run(2)
    before = (list(hp.free_runs), list(hp.used))
    with pytest.raises(obm.DoubleFree):
        hp.free([2])                        # not allocated
    with pytest.raises(obm.DoubleFree):
        hp.free([0, 0])
    with pytest.raises(obm.InvalidArgument):
        hp.free([7])
    with pytest.raises(obm.OutOfFrames):
        hp.alloc_run(3)
    assert (list(hp.free_runs), list(hp.used)) == before


def _mgr(N=12, F=8, B=4):
    bm = BlockManager(N, B, list(range(N)))
    bm.attach_host_pool(HostPool(F))
    return bm


def test_migration_follows_the_pages_steps():
    bm = _mgr()
    s = bm.seq_new()
    bm.append(s, 14)                         # 4 blocks: 0, 1, 2, 3
    assert bm.table(s) == [0, 1, 2, 3]
    free_before = list(bm.free)
    # step 1: a contiguous run of host frames; the blocks stay allocated and readable
    phys, first = bm.swap_out_begin(s, [1, 2])
    assert phys == [1, 2] and first == 0
    assert list(bm.free) == free_before
    assert bm.table(s) == [0, 1, 2, 3]
    assert bm.tier(s, 1) == (TIER_PENDING_OUT, 1) and bm.tier(s, 2) == (TIER_PENDING_OUT, 2)
    assert bm.host_pool.num_free() == 6
    # step 3: copy completed: host tier with frame indices, blocks to the back of the FIFO
    bm.swap_out_finish(s, [1, 2])
    assert bm.tier(s, 1) == (TIER_HOST, 0) and bm.tier(s, 2) == (TIER_HOST, 1)
    assert bm.table(s) == [0, -1, -1, 3]
    assert list(bm.free) == free_before + [1, 2]
    # return path: fresh blocks from the front, entries stay non-resident until done
    new, frames = bm.swap_in_begin(s, [2, 1])
    assert new == free_before[:2] and frames == [1, 0]
    assert bm.table(s) == [0, -1, -1, 3]
    assert bm.tier(s, 2) == (TIER_PENDING_IN, 1)
    bm.swap_in_finish(s, [2, 1])
    assert bm.table(s) == [0, new[1], new[0], 3]
    assert bm.tier(s, 1) == (TIER_HBM, new[1])
    assert bm.host_pool.num_free() == 8


def test_shared_block_survives_swap_out_of_one_owner():
    bm = _mgr()
    a = bm.seq_new()
    bm.append(a, 8)                          # blocks 0, 1
    b = bm.fork(a)
    bm.swap_out_begin(a, [0])
    bm.swap_out_finish(a, [0])
    assert bm.refcount(0) == 1 and 0 not in bm.free     # b still holds it
    assert bm.table(b) == [0, 1]


def test_errors_leave_state_unchanged():
    bm = _mgr(N=6, F=3)
    s = bm.seq_new()
    bm.append(s, 16)                         # blocks 0-3
    snap = lambda: (list(bm.free), list(bm.ref), bm.table(s), dict(bm.pending.get(s, {})),
                    dict(bm.host.get(s, {})), list(bm.host_pool.free_runs))
    before = snap()
    for bad in (lambda: bm.swap_out_begin(s, [0, 1, 2, 3]),   # 4 frames wanted, 3 exist
                lambda: bm.swap_out_finish(s, [0]),           # nothing in flight
                lambda: bm.swap_in_begin(s, [0]),             # resident
                lambda: bm.swap_out_begin(s, [0, 0]),
                lambda: bm.swap_out_begin(s, [9])):
        with pytest.raises(obm.BlockManagerError):
            bad()
        assert snap() == before
    bm.swap_out_begin(s, [0, 1])
    mid = snap()
    for bad in (lambda: bm.swap_out_begin(s, [1]),            # already in flight
                lambda: bm.release(s),                        # migration in flight
                lambda: bm.fork(s),
                lambda: bm.swap_in_finish(s, [0])):
        with pytest.raises(obm.BlockManagerError):
            bad()
        assert snap() == mid
    bm.swap_out_finish(s, [0, 1])
    # swap-in needs 2 fresh blocks; take every free block first so it cannot get them
    other = bm.seq_new()
    bm.append(other, 4 * bm.num_free())
    full = snap()
    with pytest.raises(obm.OutOfBlocks):
        bm.swap_in_begin(s, [0, 1])
    assert snap() == full


def test_release_returns_host_frames():
    bm = _mgr()
    s = bm.seq_new()
    bm.append(s, 12)
    bm.swap_out_begin(s, [0, 2])
    bm.swap_out_finish(s, [0, 2])
    assert bm.host_pool.num_free() == 6
    bm.release(s)
    assert bm.host_pool.num_free() == 8 and bm.num_free() == 12


def test_random_migrations_conserve_blocks_and_frames():
    rng = random.Random(83)
    N, F, B = 40, 24, 4
    bm = BlockManager(N, B, rng.sample(range(N), N))
    bm.attach_host_pool(HostPool(F))
    seqs = []
    for _ in range(400):
        op = rng.random()
        try:
            if op < 0.2 or not seqs:
                s = bm.seq_new()
                bm.append(s, rng.randint(1, 20))
                seqs.append(s)
            elif op < 0.45:
                s = rng.choice(seqs)
                res = [lb for lb in range(len(bm.table(s))) if bm.tier(s, lb)[0] == TIER_HBM]
                if res:
                    pick = rng.sample(res, rng.randint(1, len(res)))
                    bm.swap_out_begin(s, pick)
                    if rng.random() < 0.8:
                        bm.swap_out_finish(s, pick)
            elif op < 0.7:
                s = rng.choice(seqs)
                for lb, (kind, _, _) in list(bm.pending.get(s, {}).items()):
                    (bm.swap_out_finish if kind == "out" else bm.swap_in_finish)(s, [lb])
                hosted = [lb for lb in range(len(bm.table(s))) if bm.tier(s, lb)[0] == TIER_HOST]
                if hosted:
                    pick = rng.sample(hosted, rng.randint(1, len(hosted)))
                    bm.swap_in_begin(s, pick)
                    if rng.random() < 0.8:
                        bm.swap_in_finish(s, pick)
            elif op < 0.85:
                s = rng.choice(seqs)
                if not bm.pending.get(s):
                    bm.release(s)
                    seqs.remove(s)
            else:
                s = rng.choice(seqs)
                bm.append(s, rng.randint(0, 6))
        except obm.BlockManagerError:
            pass
        # conservation: every block is free or referenced; every frame free or held
        held = set()
        for s in seqs:
            held |= set(bm.host.get(s, {}).values())
            held |= {f for (_, _, f) in bm.pending.get(s, {}).values()}
        assert bm.host_pool.num_free() + len(held) == F
        assert sorted(f for f in range(F) if bm.host_pool.used[f]) == sorted(held)
        refs = [0] * N
        for s in seqs:
            for lb, p in enumerate(bm.table(s)):
                if p >= 0:
                    refs[p] += 1
            for lb, (kind, p, _) in bm.pending.get(s, {}).items():
                if kind == "in":
                    refs[p] += 1
        assert refs == bm.ref
        assert sorted(bm.free) == [b for b in range(N) if bm.ref[b] == 0]
