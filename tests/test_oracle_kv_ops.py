"""Pins of oracle.kv_ops and oracle.layout: hand-worked tiny placements
(tests/golden/layout_tiny.json), read-back of appended tokens, copy and
gather/scatter round trips."""
import json
import os

import numpy as np

from oracle import attention as att
from oracle import kv_ops, layout
from oracle import layout as olayout
from oracle.block_manager import BlockManager
from synth import gen

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "layout_tiny.json")))
KCHUNK = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "layout_kchunk.json")))


def test_k_chunk_offsets():
    B, d = KCHUNK["block_size"], KCHUNK["head_dim"]
    kp = np.zeros(olayout.k_pool_shape(1, 1, 1, B, d), np.float32)
    for case in KCHUNK["cases"]:
        vals = np.zeros(d, np.float32)
        vals[case["j"]] = 1.0
        k2 = kp.copy()
        layout.write_k(k2, 0, 0, 0, case["o"], vals)
        assert np.flatnonzero(k2.reshape(-1)).tolist() == [case["offset"]]
        assert layout.read_k(k2, 0, 0, 0, case["o"])[case["j"]] == 1.0
        assert layout.read_k_tile(k2, 0, 0, 0)[case["o"], case["j"]] == 1.0


def _tiny_pools():
    g = GOLD["geometry"]
    L, N, H, B, d = g["layers"], g["blocks"], g["kv_heads"], g["block_size"], g["head_dim"]
    kp = np.zeros(layout.k_pool_shape(L, N, H, B, d), np.float32)
    vp = np.zeros(layout.v_pool_shape(L, N, H, B, d), np.float32)
    kf, vf = kp.reshape(-1), vp.reshape(-1)
    for p in range(N):
        for o in range(B):
            for j in range(d):
                kf[p * B * d + o * d + j] = 100 * p + 10 * o + j           # K[0][p][0][o][j]
                vf[p * d * B + j * B + o] = 1000 + 100 * p + 10 * o + j    # V[0][p][0][j][o]
    return kp, vp, B


def test_tiny_rebuild():
    kp, vp, B = _tiny_pools()
    K, V = att.rebuild_sequence(kp, vp, 0, GOLD["table"], GOLD["length"], B, "f32")
    assert K[:, 0, :].tolist() == GOLD["expect_K"]
    assert V[:, 0, :].tolist() == GOLD["expect_V"]


def test_tiny_append():
    kp, vp, B = _tiny_pools()
    a = GOLD["append"]
    k_new = np.array(a["k_new"], np.float32)[:, None, :]
    v_new = np.array(a["v_new"], np.float32)[:, None, :]
    k2, v2 = kv_ops.append_kv(kp, vp, 0, k_new, v_new, a["slots"], B)
    kdiff = {str(i): float(x) for i, (x, y) in enumerate(zip(k2.reshape(-1), kp.reshape(-1))) if x != y}
    vdiff = {str(i): float(x) for i, (x, y) in enumerate(zip(v2.reshape(-1), vp.reshape(-1))) if x != y}
    assert kdiff == {k: float(v) for k, v in a["expect_k_flat_changes"].items()}
    assert vdiff == {k: float(v) for k, v in a["expect_v_flat_changes"].items()}


def test_tiny_gather():
    kp, vp, _ = _tiny_pools()
    st = kv_ops.gather_blocks(kp, vp, GOLD["gather"]["ids"])
    assert st.tolist() == GOLD["gather"]["expect_staging"]


def _random_pools(L, N, H, B, d, dtype, seed):
    kp = gen.normal_values(seed, layout.k_pool_shape(L, N, H, B, d), dtype)
    vp = gen.normal_values(seed + 1, layout.v_pool_shape(L, N, H, B, d), dtype)
    return kp, vp


def test_appended_history_reads_back_exactly():
    L, N, H, B, d = 3, 32, 2, 4, 8
    for dtype in ("f32", "bf16"):
        kp, vp = _random_pools(L, N, H, B, d, dtype, 1)
        bm = BlockManager(N, B, gen.permutation(2, N))
        lengths = [1, 9, 30]
        hist = []
        for i, S in enumerate(lengths):
            s = bm.seq_new()
            slots, _ = bm.append(s, S)
            kn = gen.normal_values(10 + i, (S, H, d), dtype)
            vn = gen.normal_values(20 + i, (S, H, d), dtype)
            kp, vp = kv_ops.append_kv(kp, vp, 2, kn, vn, slots, B)
            hist.append((s, kn, vn))
        for s, kn, vn in hist:
            K, V = att.rebuild_sequence(kp, vp, 2, bm.table(s), bm.length(s), B, dtype)
            assert np.array_equal(K, layout.widen(kn, dtype))
            assert np.array_equal(V, layout.widen(vn, dtype))


def test_slot_mapping_matches_manager_slots():
    bm = BlockManager(64, 16, gen.permutation(9, 64))
    s = bm.seq_new()
    slots, _ = bm.append(s, 100)
    got = kv_ops.slot_mapping([bm.table(s)] * 100, list(range(100)), 16)
    assert got.tolist() == slots


def test_copy_blocks_is_a_copy():
    L, N, H, B, d = 2, 8, 2, 4, 4
    kp, vp = _random_pools(L, N, H, B, d, "bf16", 3)
    k2, v2 = kv_ops.copy_blocks(kp, vp, [1, 5], [6, 2])
    assert np.array_equal(k2[:, 6], kp[:, 1]) and np.array_equal(v2[:, 6], vp[:, 1])
    assert np.array_equal(k2[:, 2], kp[:, 5]) and np.array_equal(v2[:, 2], vp[:, 5])
    untouched = [0, 1, 3, 4, 5, 7]
    assert np.array_equal(k2[:, untouched], kp[:, untouched])
    assert np.array_equal(v2[:, untouched], vp[:, untouched])


def test_gather_scatter_round_trip_keeps_logical_content():
    L, N, H, B, d = 2, 40, 2, 4, 8
    for dtype in ("f32", "bf16"):
        kp, vp = _random_pools(L, N, H, B, d, dtype, 4)
        bm = BlockManager(N, B, gen.permutation(5, N))
        s = bm.seq_new()
        bm.append(s, 37)                       # 10 blocks
        before = [att.rebuild_sequence(kp, vp, layer, bm.table(s), 37, B, dtype) for layer in range(L)]
        logical = [0, 3, 4, 9]
        phys = bm.swap_out(s, logical)
        staging = kv_ops.gather_blocks(kp, vp, phys)
        assert staging.shape == (4, L, 2, H * B * d)
        assert staging.nbytes == 4 * 2 * L * H * B * d * kp.itemsize   # bytes_per_block per frame
        # clobber the freed frames, then bring the data back into fresh blocks
        for p in phys:
            kp[:, p] = 0
            vp[:, p] = 0
        new = bm.swap_in(s, logical)
        assert set(new).isdisjoint(set(phys))
        kp, vp = kv_ops.scatter_blocks(kp, vp, staging, new)
        for layer in range(L):
            K, V = att.rebuild_sequence(kp, vp, layer, bm.table(s), 37, B, dtype)
            assert np.array_equal(K, before[layer][0]) and np.array_equal(V, before[layer][1])
        # scatter(gather(x)) at the same ids is the identity
        k3, v3 = kv_ops.scatter_blocks(kp, vp, kv_ops.gather_blocks(kp, vp, new), new)
        assert np.array_equal(k3.view(np.uint8), kp.view(np.uint8))
        assert np.array_equal(v3.view(np.uint8), vp.view(np.uint8))
