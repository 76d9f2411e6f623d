"""Pins of the chunked-prefill oracle (oracle/prefill.py) against what the pages
and the mathematics fix, each by a route other than the oracle's own:

* one query token per chunk is a decode step: the decode oracle (pinned on its
  own) over the pool after the append;
* an empty history is ordinary causal self-attention: torch's scaled dot-product
  attention with is_causal=True, float64 on the CPU;
* with a history, torch's attention with an explicit mask (every cached token
  visible, lower-triangular inside the chunk), on K/V concatenated by the test;
* "Chunked prefill mechanics": slicing a prompt into chunks gives exactly the
  monolithic result;
* brute force in Python floats on a tiny case;
* the chunk's keys and values land in the pool at the positions the block table
  gives, read back through the documented flat index formulas.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as att
from oracle import prefill as opf
from oracle.block_manager import BlockManager
from synth import gen
from tests.test_oracle_attention import brute, place_flat


def make_case(ctx, qlens, Hq, Hkv, d, B, N, seed, L=1, layer=0):
    """History K/V placed in a NaN-filled pool through block tables that cover the
    history and the chunk; chunk rows q, k_new, v_new packed by chunk."""
    rng = np.random.default_rng(seed)
    bm = BlockManager(N, B, gen.permutation(seed, N))
    tables = []
    for c, ql in zip(ctx, qlens):
        s = bm.seq_new()
        bm.append(s, int(c))
        bm.append(s, int(ql))
        tables.append(bm.table(s))
    Ks = [rng.standard_normal((c, Hkv, d)).astype(np.float32) for c in ctx]
    Vs = [rng.standard_normal((c, Hkv, d)).astype(np.float32) for c in ctx]
    kp, vp = place_flat(Ks, Vs, tables, L, N, Hkv, B, d, layer=layer)
    n_tok = int(sum(qlens))
    q_start = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int64)
    q = rng.standard_normal((n_tok, Hq, d)).astype(np.float32)
    kn = rng.standard_normal((n_tok, Hkv, d)).astype(np.float32)
    vn = rng.standard_normal((n_tok, Hkv, d)).astype(np.float32)
    return dict(tables=tables, Ks=Ks, Vs=Vs, kp=kp, vp=vp, q=q, kn=kn, vn=vn, q_start=q_start,
                ctx=np.asarray(ctx), qlens=np.asarray(qlens))


def run(case, B, layer=0, scale=None):
    return opf.paged_prefill(case["q"], case["kn"], case["vn"], case["kp"], case["vp"], layer,
                             case["tables"], case["q_start"], case["ctx"], B, "f32", scale=scale)


def test_one_token_chunks_equal_decode():
    B, Hq, Hkv, d = 16, 8, 2, 32
    ctx = [0, 5, 16, 31, 100]
    case = make_case(ctx, [1] * len(ctx), Hq, Hkv, d, B, 64, seed=3)
    kp2, vp2, out = run(case, B)
    dec = att.paged_decode(case["q"], kp2, vp2, 0, case["tables"], [c + 1 for c in ctx], B, "f32")
    np.testing.assert_allclose(out, dec, rtol=1e-12, atol=1e-13)


def _sdpa(q, K, V, mask=None, causal=False):
    """torch scaled_dot_product_attention, float64, GQA by repeating K/V heads."""
    Hq, Hkv = q.shape[1], K.shape[1]
    G = Hq // Hkv
    qt = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)[None]            # [1, Hq, T, d]
    kt = torch.from_numpy(K.astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    vt = torch.from_numpy(V.astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt.contiguous(), vt.contiguous(),
                                                         attn_mask=m, is_causal=causal)
    return o[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("B", [4, 16])
def test_empty_history_is_causal_self_attention(B):
    Hq, Hkv, d = 8, 2, 16
    qlens = [1, 7, 33, 64]
    case = make_case([0] * len(qlens), qlens, Hq, Hkv, d, B, 128, seed=5)
    _, _, out = run(case, B)
    for i, ql in enumerate(qlens):
        a, b = case["q_start"][i], case["q_start"][i + 1]
        ref = _sdpa(case["q"][a:b], case["kn"][a:b], case["vn"][a:b], causal=True)
        np.testing.assert_allclose(out[a:b], ref, rtol=1e-10, atol=1e-12)


def test_history_visible_and_chunk_causal():
    B, Hq, Hkv, d = 16, 4, 4, 16
    ctx, qlens = [3, 40, 16, 77], [5, 1, 20, 16]
    case = make_case(ctx, qlens, Hq, Hkv, d, B, 128, seed=7)
    _, _, out = run(case, B)
    for i, (c, ql) in enumerate(zip(ctx, qlens)):
        a, b = case["q_start"][i], case["q_start"][i + 1]
        K = np.concatenate([case["Ks"][i], case["kn"][a:b]])
        V = np.concatenate([case["Vs"][i], case["vn"][a:b]])
        mask = np.array([[j <= c + t for j in range(c + ql)] for t in range(ql)])
        ref = _sdpa(case["q"][a:b], K, V, mask=mask)
        np.testing.assert_allclose(out[a:b], ref, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("chunk", [1, 5, 16, 24])
def test_chunked_equals_monolithic(chunk):
    """"Chunked prefill mechanics": chunks attend over the cached earlier chunks and
    give exactly the monolithic pass (here to float64 rounding)."""
    B, Hq, Hkv, d, S = 16, 8, 2, 16, 70
    mono = make_case([0], [S], Hq, Hkv, d, B, 64, seed=9)
    _, _, ref = run(mono, B)
    kp, vp = mono["kp"], mono["vp"]
    table = mono["tables"][0]
    outs = []
    for c in range(0, S, chunk):
        ql = min(chunk, S - c)
        qs = np.array([0, ql], dtype=np.int64)
        kp, vp, o = opf.paged_prefill(mono["q"][c:c + ql], mono["kn"][c:c + ql],
                                      mono["vn"][c:c + ql], kp, vp, 0, [table], qs, [c], B, "f32")
        outs.append(o)
    np.testing.assert_allclose(np.concatenate(outs), ref, rtol=1e-12, atol=1e-13)


def test_brute_force_tiny():
    B, Hq, Hkv, d = 4, 4, 2, 4
    ctx, qlens = [2, 6], [3, 4]
    case = make_case(ctx, qlens, Hq, Hkv, d, B, 16, seed=13)
    _, _, out = run(case, B)
    scale = 1 / math.sqrt(d)
    for i, (c, ql) in enumerate(zip(ctx, qlens)):
        a = int(case["q_start"][i])
        K = np.concatenate([case["Ks"][i], case["kn"][a:a + ql]]).astype(np.float64)
        V = np.concatenate([case["Vs"][i], case["vn"][a:a + ql]]).astype(np.float64)
        for t in range(ql):
            ref = brute(case["q"][a + t].astype(np.float64).tolist(), K[:c + t + 1].tolist(),
                        V[:c + t + 1].tolist(), scale)
            np.testing.assert_allclose(out[a + t], ref, rtol=1e-9, atol=1e-12)


def test_chunk_written_at_table_positions():
    B, Hq, Hkv, d, L, N = 4, 2, 2, 32, 2, 32
    ctx, qlens = [3, 0, 8], [6, 4, 1]
    case = make_case(ctx, qlens, Hq, Hkv, d, B, N, seed=17, L=L, layer=1)
    kp2, vp2, _ = opf.paged_prefill(case["q"], case["kn"], case["vn"], case["kp"], case["vp"], 1,
                                    case["tables"], case["q_start"], case["ctx"], B, "f32")
    kflat, vflat = kp2.reshape(-1), vp2.reshape(-1)
    W = 32
    for i, (c, ql) in enumerate(zip(ctx, qlens)):
        a = int(case["q_start"][i])
        for t in range(ql):
            pos = c + t
            p, o = case["tables"][i][pos // B], pos % B
            for h in range(Hkv):
                run_ = ((1 * N + p) * Hkv + h) * B * d
                for j in range(d):
                    assert kflat[run_ + (j // W) * B * W + o * W + j % W] == case["kn"][a + t, h, j]
                    assert vflat[run_ + j * B + o] == case["vn"][a + t, h, j]
    # nothing else changed: the layer-0 pools and untouched slots are as before
    assert np.array_equal(kp2[0], case["kp"][0], equal_nan=True)
    assert np.array_equal(vp2[0], case["vp"][0], equal_nan=True)
