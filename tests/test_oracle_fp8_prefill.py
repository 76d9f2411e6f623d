"""Pins of the FP8 chunked-prefill oracle (oracle/fp8.paged_prefill), each by a
route other than its own arithmetic:

* on values that E4M3 x 2**e represents exactly (and bf16 too), it equals the
  separately pinned bf16 prefill oracle on the same values, outputs and the
  stored cache alike;
* a chunk of one token is a decode step over the pool after the append: the
  separately pinned FP8 decode oracle (values not representable, so the chunk's
  own key and value enter quantized);
* "Chunked prefill mechanics": a prompt cut into chunks gives exactly the
  monolithic result;
* the chunk's rows are stored at the positions the block table gives, read back
  through the documented byte offsets.
"""
import numpy as np
import pytest

from oracle import fp8
from oracle import layout as olayout
from oracle import prefill as opf
from oracle.block_manager import BlockManager
from synth import gen


def _tables(ctx, qlens, N, B, seed):
    bm = BlockManager(N, B, gen.permutation(seed, N))
    out = []
    for c, ql in zip(ctx, qlens):
        s = bm.seq_new()
        bm.append(s, int(c))
        bm.append(s, int(ql))
        out.append(bm.table(s))
    return out


def _fill_history(kp, vp, tables, ctx, Hkv, d, B, rng, values=None):
    for t, c in zip(tables, ctx):
        for pos in range(int(c)):
            for h in range(Hkv):
                kv = rng.standard_normal(d) * 3 if values is None else values(rng)
                vv = rng.standard_normal(d) / 2 if values is None else values(rng)
                fp8.write_token(kp, vp, 0, t[pos // B], h, pos % B, kv, vv, B, d)


def _bits(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_representable_values_equal_bf16_prefill():
    B, d, Hkv, Hq = 16, 64, 2, 8
    ctx, qlens = [37, 0, 16], [21, 40, 1]
    N = 24
    tables = _tables(ctx, qlens, N, B, 3)
    rng = np.random.default_rng(5)
    finite = fp8.TABLE[(~np.isnan(fp8.TABLE)) & (np.abs(fp8.TABLE) <= 448)]

    def rep(rng_):
        e = int(rng_.integers(-6, 3))
        v = rng_.choice(finite, d) * 2.0 ** e
        v[0] = 448.0 * 2.0 ** e              # pins the row's scale at e
        return v
    kp8 = np.zeros(fp8.pool_shape(1, N, Hkv, B, d), np.uint8)
    vp8 = np.zeros_like(kp8)
    kb = np.zeros(olayout.k_pool_shape(1, N, Hkv, B, d), np.uint16)
    vb = np.zeros(olayout.v_pool_shape(1, N, Hkv, B, d), np.uint16)
    for t, c in zip(tables, ctx):
        for pos in range(c):
            for h in range(Hkv):
                kv, vv = rep(rng), rep(rng)
                fp8.write_token(kp8, vp8, 0, t[pos // B], h, pos % B, kv, vv, B, d)
                olayout.write_k(kb, 0, t[pos // B], h, pos % B, _bits(kv))
                olayout.write_v(vb, 0, t[pos // B], h, pos % B, _bits(vv))
    n_tok = sum(qlens)
    kn = np.stack([np.stack([_bits(rep(rng)) for _ in range(Hkv)]) for _ in range(n_tok)])
    vn = np.stack([np.stack([_bits(rep(rng)) for _ in range(Hkv)]) for _ in range(n_tok)])
    q = gen.normal_values(7, (n_tok, Hq, d), "bf16")
    qs = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    kp2, vp2, got = fp8.paged_prefill(q, kn, vn, kp8, vp8, 0, tables, qs, ctx, B)
    kb2, vb2, ref = opf.paged_prefill(q, kn, vn, kb, vb, 0, tables, qs, ctx, B, "bf16")
    assert np.array_equal(got, ref)
    for t, c, ql in zip(tables, ctx, qlens):                      # the stored chunk rows agree
        for pos in range(c, c + ql):
            for h in range(Hkv):
                assert np.array_equal(fp8.read_k(kp2, 0, t[pos // B], h, pos % B, B, d),
                                      olayout.widen(olayout.read_k(kb2, 0, t[pos // B], h, pos % B), "bf16"))
                assert np.array_equal(fp8.read_v(vp2, 0, t[pos // B], h, pos % B, B, d),
                                      olayout.widen(olayout.read_v(vb2, 0, t[pos // B], h, pos % B), "bf16"))


def test_one_token_chunks_are_decode_steps():
    B, d, Hkv, Hq = 16, 128, 2, 16
    ctx = [0, 15, 16, 70]
    qlens = [1] * len(ctx)
    N = 16
    tables = _tables(ctx, qlens, N, B, 11)
    rng = np.random.default_rng(13)
    kp = np.zeros(fp8.pool_shape(1, N, Hkv, B, d), np.uint8)
    vp = np.zeros_like(kp)
    _fill_history(kp, vp, tables, ctx, Hkv, d, B, rng)
    n = len(ctx)
    q = gen.normal_values(17, (n, Hq, d), "bf16")
    kn = gen.normal_values(18, (n, Hkv, d), "bf16")
    vn = gen.normal_values(19, (n, Hkv, d), "bf16")
    qs = np.arange(n + 1, dtype=np.int32)
    kp2, vp2, got = fp8.paged_prefill(q, kn, vn, kp, vp, 0, tables, qs, ctx, B)
    slots = [t[c // B] * B + c % B for t, c in zip(tables, ctx)]
    ka, va = fp8.append_kv(kp, vp, 0, kn, vn, slots, B)
    assert np.array_equal(ka, kp2) and np.array_equal(va, vp2)
    ref = fp8.paged_decode(q, ka, va, 0, tables, [c + 1 for c in ctx], B)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("chunk", [1, 7, 32, 100])
def test_chunked_equals_monolithic(chunk):
    B, d, Hkv, Hq, S = 16, 64, 2, 4, 150
    N = 16
    tables = _tables([0], [S], N, B, 23)
    kp = np.zeros(fp8.pool_shape(1, N, Hkv, B, d), np.uint8)
    vp = np.zeros_like(kp)
    q = gen.normal_values(29, (S, Hq, d), "bf16")
    kn = gen.normal_values(30, (S, Hkv, d), "bf16")
    vn = gen.normal_values(31, (S, Hkv, d), "bf16")
    km, vm, mono = fp8.paged_prefill(q, kn, vn, kp, vp, 0, tables, np.array([0, S], np.int32), [0], B)
    outs, kc, vc = [], kp, vp
    for c in range(0, S, chunk):
        ql = min(chunk, S - c)
        kc, vc, o = fp8.paged_prefill(q[c:c + ql], kn[c:c + ql], vn[c:c + ql], kc, vc, 0, tables,
                                      np.array([0, ql], np.int32), [c], B)
        outs.append(o)
    assert np.array_equal(np.concatenate(outs), mono)
    assert np.array_equal(kc, km) and np.array_equal(vc, vm)
