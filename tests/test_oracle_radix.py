"""Pins of the prefix-cache oracle (oracle/radix.py) to what fixes it from outside:
the pages' worked examples (tests/golden/radix.json: the S_match = 100, B = 16
truncation, the 4,096-token prefix of Napkin Math 0.4, the 32,000-of-40,000
worker of Figure 7, and the leaf-first eviction of Figure 6), brute force over
everything inserted (longest common prefix, block-aligned truncation, the block
ids of a flat map keyed by whole-block prefixes), and eviction properties stated
through caller-visible actions (least recently touched goes first, descendants
before ancestors, pinned requests keep their blocks, the block manager's counts
add up)."""
import pytest

from oracle import block_manager as obm
from oracle import radix as orx
from tests import radix_scenarios as sc


class OracleImpl:
    @staticmethod
    def make(num_blocks, block_size, free_order=None):
        bm = obm.BlockManager(num_blocks, block_size, free_order)
        return bm, orx.RadixCache(bm)

    @staticmethod
    def free_list(bm):
        return list(bm.free)

    @staticmethod
    def nodes(tree):
        return {n.id: (n.parent.id, n.ref_count, n.last_access, list(n.prefix_tokens),
                       list(n.block_ids))
                for n in tree.nodes.values() if n is not tree.root}


IMPL = OracleImpl()


def test_truncation_example():
    sc.truncation_example(IMPL)


def test_napkin_prefix_hit():
    sc.napkin_prefix_hit(IMPL)


def test_figure7_worker():
    sc.figure7_worker(IMPL)


def test_figure6_eviction():
    sc.figure6_eviction(IMPL)


@pytest.mark.parametrize("seed,B", [(0, 4), (1, 4), (2, 2), (3, 8), (4, 1)])
def test_brute_force_prefixes(seed, B):
    sc.brute_force_prefixes(IMPL, seed, B)


@pytest.mark.parametrize("seed", [0, 1])
def test_pin_counts(seed):
    sc.pin_counts(IMPL, seed, 4)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_lru_order(seed):
    sc.lru_order(IMPL, seed, 4)


def test_child_first():
    sc.child_first(IMPL, 4)


@pytest.mark.parametrize("seed", [0, 5])
def test_eviction_stops_at_target(seed):
    sc.eviction_stops_at_target(IMPL, seed, 4)


def test_shared_with_live_sequence():
    sc.shared_with_live_sequence(IMPL, 4)


@pytest.mark.parametrize("seed,B", [(0, 4), (1, 2), (2, 4)])
def test_random_with_eviction(seed, B):
    sc.random_with_eviction(IMPL, seed, B)


def test_seq_from_blocks():
    bm = obm.BlockManager(8, 4)
    a = bm.seq_new()
    bm.append(a, 9)
    t = bm.table(a)
    s = bm.seq_from_blocks(t[:2])
    assert bm.table(s) == t[:2] and bm.length(s) == 8
    assert [bm.refcount(b) for b in t] == [2, 2, 1]
    slots, pairs = bm.append(s, 1)                 # a fresh block: the shared ones are full
    assert pairs == [] and slots[0] // 4 not in t
    with pytest.raises(obm.InvalidArgument):
        bm.seq_from_blocks([7])                    # not allocated
    bm.release(a)
    bm.release(s)
    assert bm.num_free() == 8


def test_unpin_errors():
    bm, tree = IMPL.make(8, 2)
    with pytest.raises(obm.InvalidArgument):
        tree.unpin(5)
    sc.run_request(bm, tree, [1, 2, 3, 4])
    _, _, _, h = tree.match([1, 2, 3, 4])
    tree.unpin(h)
    with pytest.raises(obm.InvalidArgument):
        tree.unpin(h)
    tree.unpin(0)                                  # an empty match pins nothing
