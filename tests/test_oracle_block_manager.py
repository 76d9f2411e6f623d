"""Pins of oracle.block_manager against the pages' worked scenarios and invariants."""
import copy
import json
import os

import numpy as np
import pytest

from oracle.block_manager import (BlockManager, DoubleFree, InvalidArgument, NOT_RESIDENT,
                                  OutOfBlocks)
from oracle import footprint as fp

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "block_manager.json")))


def _free_order(num_blocks, head):
    rest = [b for b in range(num_blocks) if b not in head]
    return list(head) + rest


def _run(case):
    bm = BlockManager(case["num_blocks"], case["block_size"],
                      _free_order(case["num_blocks"], case["free_order_head"]))
    names, copies = {}, []
    for op in case["ops"]:
        if op[0] == "new":
            names[op[1]] = bm.seq_new()
        elif op[0] == "append":
            _, pairs = bm.append(names[op[1]], op[2])
            copies += [list(p) for p in pairs]
        elif op[0] == "fork":
            names[op[2]] = bm.fork(names[op[1]])
    return bm, names, copies


@pytest.mark.parametrize("key", ["figure5_boundary", "figure5_cow"])
def test_figure5(key):
    case = GOLD[key]
    bm, names, copies = _run(case)
    for name, table in case["expect_tables"].items():
        assert bm.table(names[name]) == table
    for b, r in case["expect_refcounts"].items():
        assert bm.refcount(int(b)) == r
    assert copies == case["expect_copies"]


def test_p3_fork_example():
    c = GOLD["p3_fork"]
    bm = BlockManager(c["num_blocks"], c["block_size"])
    a = bm.seq_new()
    bm.append(a, c["prefix_tokens"])
    assert bm.blocks_in_use() == c["expect_blocks_after_prefix"]
    b = bm.fork(a)
    assert bm.blocks_in_use() == c["expect_blocks_after_fork"]
    assert all(bm.refcount(p) == c["expect_refcount_after_fork"] for p in bm.table(a))
    _, pairs1 = bm.append(a, 1)
    assert len(pairs1) == c["expect_copies_first_writer"]
    _, pairs2 = bm.append(b, 1)
    assert len(pairs2) == c["expect_copies_second_writer"]
    assert bm.blocks_in_use() == c["expect_blocks_final"]
    assert c["independent_caches_blocks"] == 2 * fp.blocks_for_tokens(c["prefix_tokens"] + 1, c["block_size"])
    # the two full prefix blocks stay shared; the tails are private
    ta, tb = bm.table(a), bm.table(b)
    assert ta[:2] == tb[:2] and ta[2] != tb[2]
    assert [bm.refcount(p) for p in ta] == [2, 2, 1] and bm.refcount(tb[2]) == 1


def test_release_after_figure5():
    r = GOLD["release"]
    bm, names, _ = _run(GOLD[r["after"]])
    free_before = list(bm.free)
    bm.release(names[r["release"]])
    for b, cnt in r["expect_refcounts"].items():
        assert bm.refcount(int(b)) == cnt
    assert list(bm.free) == free_before + r["expect_freed"]
    assert bm.table(names["A"]) == r["expect_table_A"]


def test_allocate_on_boundary_rule():
    # o != 0 writes into T[l]; o == 0 pops a fresh block (KV Cache Management,
    # The PagedAttention virtual memory model). One token at a time and one
    # multi-token call give the same table and slots.
    for B in (1, 4, 16):
        order = list(np.random.default_rng(B).permutation(64))
        bm1, bm2 = BlockManager(64, B, order), BlockManager(64, B, order)
        s1, s2 = bm1.seq_new(), bm2.seq_new()
        slots1 = []
        for _ in range(50):
            slots1 += bm1.append(s1, 1)[0]
        slots2, _ = bm2.append(s2, 50)
        assert slots1 == slots2
        t = bm1.table(s1)
        assert len(t) == fp.blocks_for_tokens(50, B) and t == order[:len(t)]
        for pos, slot in enumerate(slots1):
            assert slot == t[pos // B] * B + pos % B


def test_out_of_blocks_leaks_nothing():
    bm = BlockManager(4, 16)
    a = bm.seq_new()
    bm.append(a, 40)                       # 3 blocks
    b = bm.seq_new()
    before = copy.deepcopy(bm.__dict__)
    with pytest.raises(OutOfBlocks):
        bm.append(b, 17)                   # would need 2, only 1 left
    assert bm.__dict__ == before
    with pytest.raises(OutOfBlocks):
        bm.alloc(2)
    assert bm.__dict__ == before


def test_cow_without_free_block_fails_cleanly():
    bm = BlockManager(3, 16)
    a = bm.seq_new()
    bm.append(a, 40)                       # all 3 blocks, tail holds 8
    b = bm.fork(a)
    before = copy.deepcopy(bm.__dict__)
    with pytest.raises(OutOfBlocks):
        bm.append(b, 1)                    # copy-on-write needs a block
    assert bm.__dict__ == before


def test_double_free():
    bm = BlockManager(8, 16)
    ids = bm.alloc(2)
    bm.free_blocks(ids)
    with pytest.raises(DoubleFree):
        bm.free_blocks([ids[0]])
    ids2 = bm.alloc(1)
    before = copy.deepcopy(bm.__dict__)
    with pytest.raises(DoubleFree):
        bm.free_blocks([ids2[0], ids2[0]])  # second drop has no reference left
    assert bm.__dict__ == before


def test_swap_out_in_roundtrip_state():
    bm = BlockManager(16, 4, list(range(16)))
    a = bm.seq_new()
    bm.append(a, 14)                        # 4 blocks: 0,1,2,3
    phys = bm.swap_out(a, [1, 3])
    assert phys == [1, 3]
    assert bm.table(a) == [0, NOT_RESIDENT, 2, NOT_RESIDENT]
    assert list(bm.free)[-2:] == [1, 3]
    with pytest.raises(InvalidArgument):
        bm.append(a, 1)                     # tail is not resident
    new = bm.swap_in(a, [1, 3])
    assert new == [4, 5] and bm.table(a) == [0, 4, 2, 5]
    with pytest.raises(InvalidArgument):
        bm.swap_in(a, [1])


def _check_invariants(bm):
    count = [0] * bm.num_blocks
    for t in bm.tables.values():
        for p in t:
            if p != NOT_RESIDENT:
                count[p] += 1
    free = set(bm.free)
    assert len(free) == len(bm.free)
    for p in range(bm.num_blocks):
        assert bm.ref[p] >= count[p]
        assert (bm.ref[p] == 0) == (p in free)
    for sid, t in bm.tables.items():
        assert len(t) == fp.blocks_for_tokens(bm.lengths[sid], bm.block_size)


def test_random_ops_keep_invariants():
    rng = np.random.default_rng(83)
    for trial in range(20):
        bm = BlockManager(48, int(rng.choice([1, 2, 4, 16])), list(rng.permutation(48)))
        live = []
        for _ in range(150):
            op = rng.integers(0, 7)
            before = copy.deepcopy(bm.__dict__)
            try:
                if op == 0 or not live:
                    live.append(bm.seq_new())
                elif op == 1:
                    bm.append(int(rng.choice(live)), int(rng.integers(0, 40)))
                elif op == 2:
                    live.append(bm.fork(int(rng.choice(live))))
                elif op == 3:
                    s = int(rng.choice(live))
                    bm.release(s)
                    live.remove(s)
                elif op == 4:
                    s = int(rng.choice(live))
                    t = bm.table(s)
                    res = [i for i, p in enumerate(t) if p != NOT_RESIDENT]
                    if res:
                        pick = sorted(rng.choice(res, size=min(len(res), 2), replace=False).tolist())
                        bm.swap_out(s, pick)
                elif op == 5:
                    s = int(rng.choice(live))
                    out = [i for i, p in enumerate(bm.table(s)) if p == NOT_RESIDENT]
                    bm.swap_in(s, out)
                else:
                    bm.append(int(rng.choice(live)), 1)
            except (OutOfBlocks, InvalidArgument):
                assert bm.__dict__ == before
            _check_invariants(bm)
