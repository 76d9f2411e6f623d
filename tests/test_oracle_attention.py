"""Pins of oracle.attention: brute force on tiny inputs, closed forms, an independent
library routine, invariants (block placement, poisoned unused slots) and the
online-softmax split form against the direct one."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as att
from oracle import layout
from oracle.block_manager import BlockManager
from synth import gen


# ---------------------------------------------------------------------------
# Test-side placement: writes contiguous per-sequence K/V into flat pool arrays
# using the documented flat index formulas directly (a different route from the
# oracle's shaped numpy indexing).
def place_flat(Ks, Vs, tables, L, N, H, B, d, layer=0, fill=np.nan, dtype=np.float32):
    kflat = np.full(L * N * H * B * d, fill, dtype=dtype)
    vflat = np.full(L * N * H * B * d, fill, dtype=dtype)
    W = 32 if d % 32 == 0 else d          # K dimension-chunk width
    for K, V, table in zip(Ks, Vs, tables):
        for t in range(K.shape[0]):
            p, o = table[t // B], t % B
            for h in range(H):
                run = ((layer * N + p) * H + h) * B * d
                for j in range(d):
                    kflat[run + (j // W) * B * W + o * W + j % W] = K[t, h, j]
                    vflat[run + j * B + o] = V[t, h, j]
    return (kflat.reshape(layout.k_pool_shape(L, N, H, B, d)),
            vflat.reshape(layout.v_pool_shape(L, N, H, B, d)))


def brute(q, K, V, scale):
    """exp(s_t) / sum exp(s), straight from the definition, in Python floats."""
    Hq, d = len(q), len(q[0])
    S, Hkv = len(K), len(K[0])
    G = Hq // Hkv
    out = []
    for h in range(Hq):
        g = h // G
        w = [math.exp(scale * sum(q[h][j] * K[t][g][j] for j in range(d))) for t in range(S)]
        Z = sum(w)
        out.append([sum(w[t] * V[t][g][j] for t in range(S)) / Z for j in range(d)])
    return np.array(out)


def _tables_from_manager(lengths, N, B, seed):
    bm = BlockManager(N, B, gen.permutation(seed, N))
    tables = []
    for S in lengths:
        s = bm.seq_new()
        bm.append(s, int(S))
        tables.append(bm.table(s))
    return tables


@pytest.mark.parametrize("B", [1, 4, 16])
def test_brute_force_tiny(B):
    rng = np.random.default_rng(7 + B)
    L, N, Hq, Hkv, d = 2, 64, 4, 2, (64 if B == 4 else 8)
    lengths = [1, 17, 40]
    tables = _tables_from_manager(lengths, N, B, 11)
    Ks = [rng.standard_normal((S, Hkv, d)).astype(np.float32) for S in lengths]
    Vs = [rng.standard_normal((S, Hkv, d)).astype(np.float32) for S in lengths]
    q = rng.standard_normal((len(lengths), Hq, d)).astype(np.float32)
    kp, vp = place_flat(Ks, Vs, tables, L, N, Hkv, B, d, layer=1)
    got = att.paged_decode(q, kp, vp, 1, tables, lengths, B, "f32")
    scale = 1 / math.sqrt(d)
    for i in range(len(lengths)):
        ref = brute(q[i].astype(np.float64).tolist(), Ks[i].astype(np.float64).tolist(),
                    Vs[i].astype(np.float64).tolist(), scale)
        np.testing.assert_allclose(got[i], ref, rtol=1e-9, atol=1e-12)


def test_against_torch_sdpa():
    rng = np.random.default_rng(3)
    L, N, Hq, Hkv, d, B = 1, 128, 8, 2, 16, 16
    lengths = [5, 33, 200, 16]
    tables = _tables_from_manager(lengths, N, B, 5)
    Ks = [rng.standard_normal((S, Hkv, d)).astype(np.float32) for S in lengths]
    Vs = [rng.standard_normal((S, Hkv, d)).astype(np.float32) for S in lengths]
    q = rng.standard_normal((len(lengths), Hq, d)).astype(np.float32)
    kp, vp = place_flat(Ks, Vs, tables, L, N, Hkv, B, d)
    got = att.paged_decode(q, kp, vp, 0, tables, lengths, B, "f32")
    G = Hq // Hkv
    for i, S in enumerate(lengths):
        qt = torch.from_numpy(q[i].astype(np.float64))[None, :, None, :]          # [1, Hq, 1, d]
        kt = torch.from_numpy(Ks[i].astype(np.float64)).permute(1, 0, 2)          # [Hkv, S, d]
        vt = torch.from_numpy(Vs[i].astype(np.float64)).permute(1, 0, 2)
        kt = kt.repeat_interleave(G, dim=0)[None].contiguous()
        vt = vt.repeat_interleave(G, dim=0)[None].contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0, :, 0, :].numpy()
        np.testing.assert_allclose(got[i], ref, rtol=1e-10, atol=1e-12)


def _single(q, K, V, scale=None):
    """paged_decode of one sequence whose blocks are placed in order."""
    S, Hkv, d = K.shape
    B = 4
    table = list(range(-(-S // B)))
    kp, vp = place_flat([K], [V], [table], 1, max(1, len(table)), Hkv, B, d)
    return att.paged_decode(q[None], kp, vp, 0, [table], [S], B, "f32", scale=scale)[0]


def test_single_token_returns_its_value():
    rng = np.random.default_rng(1)
    K = rng.standard_normal((1, 2, 8)).astype(np.float32)
    V = rng.standard_normal((1, 2, 8)).astype(np.float32)
    q = rng.standard_normal((4, 8)).astype(np.float32)
    out = _single(q, K, V)
    for h in range(4):
        assert np.array_equal(out[h], V[0, h // 2].astype(np.float64))


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(2)
    K = rng.standard_normal((13, 2, 8)).astype(np.float32)
    V = rng.standard_normal((13, 2, 8)).astype(np.float32)
    out = _single(np.zeros((4, 8), np.float32), K, V)
    for h in range(4):
        np.testing.assert_allclose(out[h], V[:, h // 2].astype(np.float64).mean(axis=0), rtol=1e-12, atol=1e-14)


def test_equal_keys_give_mean_of_values():
    rng = np.random.default_rng(4)
    K = np.tile(rng.standard_normal((1, 2, 8)).astype(np.float32), (9, 1, 1))
    V = rng.standard_normal((9, 2, 8)).astype(np.float32)
    out = _single(rng.standard_normal((4, 8)).astype(np.float32), K, V)
    for h in range(4):
        np.testing.assert_allclose(out[h], V[:, h // 2].astype(np.float64).mean(axis=0), rtol=1e-12, atol=1e-14)


def test_two_keys_weights_one_to_three_pin_the_scale():
    # d = 4, default scale 1/2: s_0 = 0, s_1 = ln 3  ->  o = (v_0 + 3 v_1) / 4.
    d = 4
    K = np.zeros((2, 1, d), np.float64)
    K[1, 0, 0] = 2 * math.log(3)
    V = np.array([[[1.0, 2.0, -3.0, 0.5]], [[5.0, -1.0, 7.0, 0.25]]])
    q = np.array([[1.0, 0.0, 0.0, 0.0]])
    B, table = 2, [0]
    kp, vp = place_flat([K], [V], [table], 1, 1, 1, B, d, dtype=np.float64)
    kp = kp.astype(np.float32)   # K[1,0,0] is not exact in f32; recompute the expected weight from it
    vp = vp.astype(np.float32)
    out = att.paged_decode(q.astype(np.float32)[None], kp, vp, 0, [table], [2], B, "f32")[0, 0]
    w1 = math.exp(0.5 * float(np.float32(2 * math.log(3))))
    expect = (V[0, 0] + w1 * V[1, 0]) / (1 + w1)
    np.testing.assert_allclose(out, expect, rtol=1e-12)
    np.testing.assert_allclose(out, (V[0, 0] + 3 * V[1, 0]) / 4, rtol=1e-6)
    # an explicit scale of 1 gives weights 1 : 9
    out1 = att.paged_decode(q.astype(np.float32)[None], kp, vp, 0, [table], [2], B, "f32", scale=1.0)[0, 0]
    w = math.exp(float(np.float32(2 * math.log(3))))
    np.testing.assert_allclose(out1, (V[0, 0] + w * V[1, 0]) / (1 + w), rtol=1e-12)


def test_gqa_groups_are_contiguous():
    # H_q = 4, H_kv = 2: heads 0,1 read KV head 0 and heads 2,3 read KV head 1.
    rng = np.random.default_rng(5)
    K = rng.standard_normal((6, 2, 8)).astype(np.float32)
    V = np.zeros((6, 2, 8), np.float32)
    V[:, 0, :] = 1.5
    V[:, 1, :] = -2.5
    out = _single(rng.standard_normal((4, 8)).astype(np.float32), K, V)
    np.testing.assert_allclose(out[:2], 1.5, rtol=1e-12)
    np.testing.assert_allclose(out[2:], -2.5, rtol=1e-12)


def test_dominant_key():
    rng = np.random.default_rng(6)
    d = 16
    K = rng.standard_normal((20, 1, d)).astype(np.float32) * 0.1
    q = np.zeros((1, d), np.float32)
    q[0, 0] = 1.0
    K[7, 0, 0] = 80.0 * math.sqrt(d)       # score +80 above the rest (scale 1/sqrt(d))
    V = rng.standard_normal((20, 1, d)).astype(np.float32)
    out = _single(q, K, V)
    np.testing.assert_allclose(out[0], V[7, 0].astype(np.float64), rtol=0, atol=1e-30 + 1e-25)


def test_block_placement_invariance_and_poisoned_slots():
    rng = np.random.default_rng(8)
    L, N, Hq, Hkv, d, B = 1, 64, 4, 2, 8, 4
    lengths = [3, 25, 31]
    Ks = [rng.standard_normal((S, Hkv, d)).astype(np.float32) for S in lengths]
    Vs = [rng.standard_normal((S, Hkv, d)).astype(np.float32) for S in lengths]
    q = rng.standard_normal((3, Hq, d)).astype(np.float32)
    outs = []
    for seed in (1, 2, 3):
        tables = _tables_from_manager(lengths, N, B, seed)
        kp, vp = place_flat(Ks, Vs, tables, L, N, Hkv, B, d, fill=np.nan)
        outs.append(att.paged_decode(q, kp, vp, 0, tables, lengths, B, "f32"))
    assert np.isfinite(outs[0]).all()
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    # and equal to the same data in a fully finite pool
    tables = _tables_from_manager(lengths, N, B, 1)
    kp, vp = place_flat(Ks, Vs, tables, L, N, Hkv, B, d, fill=0.0)
    assert np.array_equal(att.paged_decode(q, kp, vp, 0, tables, lengths, B, "f32"), outs[0])


def test_bf16_inputs_are_widened_exactly():
    bits = np.array([0x3F80, 0xC000, 0x3E80, 0x0001], dtype=np.uint16)   # 1, -2, 0.25, tiny subnormal
    vals = layout.widen(bits, "bf16")
    assert vals[0] == 1.0 and vals[1] == -2.0 and vals[2] == 0.25
    assert vals[3] == np.float64(np.frombuffer(np.uint32(0x00010000).tobytes(), np.float32)[0])
    assert gen.f32_to_bf16_bits(np.array([1.0, -2.0, 0.25], np.float32)).tolist() == [0x3F80, 0xC000, 0x3E80]


def test_zero_length_gives_zeros():
    q = np.ones((1, 2, 4), np.float32)
    kp = np.full(layout.k_pool_shape(1, 1, 1, 4, 4), np.nan, np.float32)
    vp = np.full(layout.v_pool_shape(1, 1, 1, 4, 4), np.nan, np.float32)
    out = att.paged_decode(q, kp, vp, 0, [[0]], [0], 4, "f32")
    assert np.array_equal(out, np.zeros((1, 2, 4)))


@pytest.mark.parametrize("S", [1, 2, 15, 16, 17, 100, 257])
def test_online_split_equals_direct(S):
    rng = np.random.default_rng(S)
    Hq, Hkv, d = 4, 2, 8
    q = rng.standard_normal((Hq, d)) * 3
    K = rng.standard_normal((S, Hkv, d))
    V = rng.standard_normal((S, Hkv, d))
    ref = att.attend(q, K, V, 0.35)
    for split in (1, 7, 16, 64, 1024):
        for tile in (1, 5, 16):
            got = att.attend_split(q, K, V, 0.35, split, tile)
            np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)
