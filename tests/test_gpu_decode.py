"""GPU parity of paged decode (append + pa_decode) against the oracle.

Attention outputs must match the float64 oracle to max-abs-error <= 2e-2 with bf16
inputs/outputs and <= 1e-5 with fp32; the append must be bit-exact; outputs must
be bitwise identical under any permutation of physical blocks; unused slots are
NaN-poisoned throughout."""
import zlib

import numpy as np
import pytest
import torch

import paged_kv_cache_83_amd as pk
from oracle import attention as oatt
from tests.gpu_helpers import (BF16_TOL, F32_TOL, make_batch, max_abs_err, need_gpu,
                               oracle_step, padded_tables, print_case, to_dev, to_host)

pytestmark = pytest.mark.gpu

RAGGED = [1, 2, 15, 16, 17, 31, 32, 33, 47, 64, 100, 257]


def run_library(batch, layer, kernel="auto", bps=0, scale=0.0, tables=None, lengths=None,
                max_ctx=None, merge=False, ws=None, waves=0, host_lens=None):
    """Upload the batch, run the library's append + decode on one layer; returns
    (out, k_pool, v_pool) in storage form. merge=True merges the splits inside
    the decode launch (zeroed workspace, or the one passed in)."""
    geom = pk.Geometry(batch.L, batch.Hkv, batch.d, batch.B, batch.N, batch.dtype)
    K, V = to_dev(batch.k_pool, batch.dtype), to_dev(batch.v_pool, batch.dtype)
    slots = torch.from_numpy(batch.slots_new).cuda()
    pk.append_kv(geom, K, V, layer, to_dev(batch.k_new, batch.dtype),
                 to_dev(batch.v_new, batch.dtype), slots)
    tabs = padded_tables(batch.tables if tables is None else tables, batch.max_blocks)
    lens = batch.lengths if lengths is None else lengths
    max_ctx = int(max(lens)) if max_ctx is None else max_ctx
    q = to_dev(batch.q, batch.dtype)
    out = torch.empty_like(q)
    if ws is None:
        ws_bytes = pk.decode_workspace_bytes(geom, q.shape[0], q.shape[1], max_ctx, bps, kernel,
                                             merge, waves, host_lens)
        ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    pk.decode(geom, K, V, layer, q, out, torch.from_numpy(tabs).cuda(),
              torch.from_numpy(np.asarray(lens, np.int32)).cuda(), max_ctx, scale=scale,
              workspace=ws, blocks_per_split=bps, kernel=kernel, merge=merge, waves_per_group=waves,
              host_lens=host_lens)
    torch.cuda.synchronize()
    return to_host(out, batch.dtype), to_host(K, batch.dtype), to_host(V, batch.dtype)


CASES = [
    # name, dtype, L, N, Hq, Hkv, d, B, kernel, bps
    ("mfma_d128_g8", "bf16", 2, 160, 64, 8, 128, 16, "mfma", 0),
    ("mfma_d128_g8_split2", "bf16", 2, 160, 64, 8, 128, 16, "mfma", 2),
    ("mfma_d128_g4", "bf16", 1, 160, 32, 8, 128, 16, "mfma", 4),
    ("mfma_d64_g16", "bf16", 1, 160, 32, 2, 64, 16, "mfma", 0),
    ("mfma_d256_g2", "bf16", 1, 160, 4, 2, 256, 16, "mfma", 6),
    ("mfma_d128_mha", "bf16", 1, 160, 4, 4, 128, 16, "mfma", 0),
    ("generic_bf16_d128_g8", "bf16", 1, 160, 16, 2, 128, 16, "generic", 4),
    ("generic_bf16_b4", "bf16", 1, 700, 8, 2, 32, 4, "generic", 0),
    ("generic_f32_d64_mha", "f32", 2, 160, 12, 12, 64, 16, "generic", 0),
    ("generic_f32_d64_split", "f32", 1, 160, 6, 3, 64, 16, "generic", 2),
    ("generic_f32_b32_g4", "f32", 1, 100, 8, 2, 128, 32, "generic", 0),
    ("generic_f32_b1", "f32", 1, 1200, 2, 1, 16, 1, "generic", 64),
    ("valu_f32_d64_mha", "f32", 2, 160, 12, 12, 64, 16, "valu", 0),
    ("valu_f32_d64_g2_split2", "f32", 1, 160, 6, 3, 64, 16, "valu", 2),
    ("valu_f32_d128_g4", "f32", 1, 160, 8, 2, 128, 16, "valu", 0),
    ("valu_f32_d128_g8_split3", "f32", 1, 160, 16, 2, 128, 16, "valu", 3),
    ("valu_bf16_d128_g8", "bf16", 1, 160, 64, 8, 128, 16, "valu", 0),
    ("valu_bf16_d128_g8_split2", "bf16", 1, 160, 16, 2, 128, 16, "valu", 2),
    ("valu_bf16_d64_g2_split6", "bf16", 1, 160, 8, 4, 64, 16, "valu", 6),
    ("valu_bf16_d128_mha", "bf16", 1, 160, 4, 4, 128, 16, "valu", 64),
    ("valu_bf16_d64_g4", "bf16", 2, 160, 16, 4, 64, 16, "valu", 0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decode_parity(case):
    need_gpu()
    name, dtype, L, N, Hq, Hkv, d, B, kernel, bps = case
    print_case(test="decode_parity", case=name)
    batch = make_batch(dtype, L, N, Hq, Hkv, d, B, RAGGED, seed=zlib.crc32(name.encode()) % 10000)
    tol = BF16_TOL if dtype == "bf16" else F32_TOL
    for layer in range(L):
        out, K, V = run_library(batch, layer, kernel=kernel, bps=bps)
        ek, ev, expect = oracle_step(batch, layer)
        assert np.array_equal(K.view(np.uint8), ek.view(np.uint8)), "append mismatch"
        assert np.array_equal(V.view(np.uint8), ev.view(np.uint8)), "append mismatch"
        assert np.isfinite(out.astype(np.float32) if dtype == "f32" else out).all()
        err = max_abs_err(out, expect, dtype)
        assert err <= tol, (name, layer, err)


def test_single_token_returns_its_value_bitwise():
    need_gpu()
    print_case(test="single_token")
    for kernel, dtype, d in (("mfma", "bf16", 128), ("generic", "f32", 64), ("generic", "bf16", 64),
                             ("valu", "f32", 64), ("valu", "bf16", 128), ("valu", "f32", 128)):
        batch = make_batch(dtype, 1, 8, 8, 2, d, 16, [1, 1, 1], seed=5)
        out, _, _ = run_library(batch, 0, kernel=kernel)
        for i in range(3):
            for h in range(8):
                assert np.array_equal(out[i, h], batch.v_new[i, h // 4]), (kernel, dtype)


def test_zero_length_writes_zeros():
    need_gpu()
    print_case(test="zero_length")
    for kernel, dtype, bps in (("mfma", "bf16", 0), ("mfma", "bf16", 2), ("generic", "f32", 2),
                               ("valu", "f32", 2), ("valu", "f32", 0), ("valu", "bf16", 2)):
        batch = make_batch(dtype, 1, 64, 8, 2, 64 if dtype == "f32" else 128, 16, [0, 40, 0, 70],
                           seed=9)
        out, _, _ = run_library(batch, 0, kernel=kernel, bps=bps)
        _, _, expect = oracle_step(batch, 0)
        assert not np.any(out[0].view(np.uint8)) and not np.any(out[2].view(np.uint8))
        assert max_abs_err(out, expect, dtype) <= (BF16_TOL if dtype == "bf16" else F32_TOL)


@pytest.mark.parametrize("kernel,dtype,d,Hq", [("mfma", "bf16", 128, 16), ("generic", "f32", 64, 16),
                                                ("valu", "f32", 64, 8), ("valu", "bf16", 128, 16)])
def test_block_placement_invariance_bitwise(kernel, dtype, d, Hq):
    """Same logical content under a different physical permutation: identical bits."""
    need_gpu()
    print_case(test="placement", kernel=kernel)
    L, N, Hkv, B = 1, 200, 2, 16
    lengths = [33, 250, 7, 129]
    a = make_batch(dtype, L, N, Hq, Hkv, d, B, lengths, seed=21)
    b = make_batch(dtype, L, N, Hq, Hkv, d, B, lengths, seed=22)
    # give b the same logical content as a: copy each token's K/V to b's placement
    from oracle import layout as ol
    for ta, tb, S in zip(a.tables, b.tables, lengths):
        for lb in range(len(ta)):
            b.k_pool[:, tb[lb]] = a.k_pool[:, ta[lb]]
            b.v_pool[:, tb[lb]] = a.v_pool[:, ta[lb]]
    b.q, b.k_new, b.v_new = a.q, a.k_new, a.v_new
    assert b.tables != a.tables
    out_a, _, _ = run_library(a, 0, kernel=kernel, bps=4)
    out_b, _, _ = run_library(b, 0, kernel=kernel, bps=4)
    assert np.array_equal(out_a.view(np.uint8), out_b.view(np.uint8))
    del ol


def test_split_count_invariance():
    """One split against many: fp32 within 1e-6; bf16 MFMA within the bf16 tolerance."""
    need_gpu()
    print_case(test="splits")
    lengths = [700, 1, 333, 1024]
    f = make_batch("f32", 1, 300, 8, 4, 64, 16, lengths, seed=31)
    one, _, _ = run_library(f, 0, kernel="generic", bps=1024)
    many, _, _ = run_library(f, 0, kernel="generic", bps=2)
    assert np.max(np.abs(one.astype(np.float64) - many.astype(np.float64))) <= 1e-6
    one, _, _ = run_library(f, 0, kernel="valu", bps=64)     # 16 splits at most (1024 tokens)
    many, _, _ = run_library(f, 0, kernel="valu", bps=2)
    assert np.max(np.abs(one.astype(np.float64) - many.astype(np.float64))) <= 1e-6
    _, _, expect = oracle_step(f, 0)
    assert max_abs_err(many, expect, "f32") <= F32_TOL
    b = make_batch("bf16", 1, 300, 64, 8, 128, 16, lengths, seed=32)
    one, _, _ = run_library(b, 0, kernel="mfma", bps=1024)
    many, _, _ = run_library(b, 0, kernel="mfma", bps=2)
    _, _, expect = oracle_step(b, 0)
    assert max_abs_err(one, expect, "bf16") <= BF16_TOL
    assert max_abs_err(many, expect, "bf16") <= BF16_TOL


def test_explicit_scale():
    need_gpu()
    print_case(test="scale")
    batch = make_batch("f32", 1, 100, 4, 2, 64, 16, [50, 90], seed=41)
    out, _, _ = run_library(batch, 0, kernel="generic", scale=0.3)
    _, _, expect = oracle_step(batch, 0, scale=0.3)
    assert max_abs_err(out, expect, "f32") <= F32_TOL
    batch = make_batch("bf16", 1, 100, 16, 2, 128, 16, [50, 90], seed=42)
    out, _, _ = run_library(batch, 0, kernel="mfma", scale=0.02)
    _, _, expect = oracle_step(batch, 0, scale=0.02)
    assert max_abs_err(out, expect, "bf16") <= BF16_TOL


def test_auto_kernel_choice_matches_oracle():
    need_gpu()
    print_case(test="auto")
    for dtype, d, B in (("bf16", 128, 16), ("f32", 64, 16), ("bf16", 64, 8)):
        batch = make_batch(dtype, 1, 200, 16, 4, d, B, [5, 77, 300], seed=51)
        out, _, _ = run_library(batch, 0)
        _, _, expect = oracle_step(batch, 0)
        assert max_abs_err(out, expect, dtype) <= (BF16_TOL if dtype == "bf16" else F32_TOL)


def test_unsupported_and_bad_arguments():
    need_gpu()
    print_case(test="bad_args")
    geom = pk.Geometry(1, 2, 128, 16, 8, "f32")
    K, V = pk.alloc_pools(geom)
    q = torch.zeros(1, 4, 128, device="cuda")
    out = torch.empty_like(q)
    tabs = torch.zeros(1, 1, dtype=torch.int32, device="cuda")
    lens = torch.ones(1, dtype=torch.int32, device="cuda")
    with pytest.raises(pk.PagedKVError):
        pk.decode(geom, K, V, 0, q, out, tabs, lens, 16, kernel="mfma")    # fp32 has no MFMA path
    with pytest.raises(pk.PagedKVError):
        pk.decode(geom, K, V, 0, q, out, tabs, lens, 17)                    # table too short
    g64 = pk.Geometry(1, 1, 64, 16, 8, "f32")                               # 8 heads at d = 64:
    K64, V64 = pk.alloc_pools(g64)                                          # not a VALU shape
    q64 = torch.zeros(1, 8, 64, device="cuda")
    with pytest.raises(pk.PagedKVError):
        pk.decode(g64, K64, V64, 0, q64, torch.empty_like(q64), tabs, lens, 16, kernel="valu")
    with pytest.raises(ValueError):
        pk.decode(geom, K, V, 0, q.to(torch.bfloat16), out, tabs, lens, 16)  # dtype mismatch


def test_kv_reuse_policy_same_result():
    """Cached (kv_reuse) and streamed K/V loads compute the same bits."""
    need_gpu()
    print_case(test="kv_reuse")
    batch = make_batch("bf16", 1, 200, 32, 4, 128, 16, [1, 40, 300, 777], seed=61)
    geom = pk.Geometry(1, 4, 128, 16, 200, "bf16")
    outs = []
    for reuse in (False, True):
        K, V = to_dev(batch.k_pool, "bf16"), to_dev(batch.v_pool, "bf16")
        pk.append_kv(geom, K, V, 0, to_dev(batch.k_new, "bf16"), to_dev(batch.v_new, "bf16"),
                     torch.from_numpy(batch.slots_new).cuda())
        q = to_dev(batch.q, "bf16")
        out = torch.empty_like(q)
        ws = torch.empty(max(1, pk.decode_workspace_bytes(geom, 4, 32, 777)), dtype=torch.uint8,
                         device="cuda")
        pk.decode(geom, K, V, 0, q, out, torch.from_numpy(padded_tables(batch.tables, batch.max_blocks)).cuda(),
                  torch.from_numpy(batch.lengths.astype(np.int32)).cuda(), 777, workspace=ws,
                  kv_reuse=reuse)
        torch.cuda.synchronize()
        outs.append(to_host(out, "bf16"))
    assert np.array_equal(outs[0], outs[1])
    _, _, expect = oracle_step(batch, 0)
    assert max_abs_err(outs[0], expect, "bf16") <= BF16_TOL


MERGE_CASES = [
    # name, dtype, Hq, Hkv, d, bps, lengths, kernel
    ("f32_d64_mha_bps2", "f32", 12, 12, 64, 2, RAGGED, "valu"),
    ("f32_d128_g4_bps4", "f32", 8, 2, 128, 4, RAGGED + [1000], "valu"),
    ("bf16_d128_g8_bps2", "bf16", 64, 8, 128, 2, RAGGED, "valu"),
    ("bf16_d64_g2_auto", "bf16", 8, 4, 64, 0, RAGGED + [3000, 16 * 64 * 3 + 5], "valu"),
    ("f32_d64_g2_empty", "f32", 6, 3, 64, 2, [0, 40, 0, 300, 1], "valu"),
    ("mfma_d128_g4_empty", "bf16", 16, 4, 128, 2, [0, 40, 0, 300, 1], "mfma"),
    ("mfma_d128_g8_bps2", "bf16", 64, 8, 128, 2, RAGGED, "mfma"),
    ("mfma_d128_g4_auto", "bf16", 32, 8, 128, 0, RAGGED + [3000, 16 * 64 * 3 + 5], "mfma"),
    ("mfma_d64_g16_bps4", "bf16", 32, 2, 64, 4, RAGGED + [1000], "mfma"),
    ("mfma_d256_g2_bps6", "bf16", 4, 2, 256, 6, RAGGED, "mfma"),
]


@pytest.mark.parametrize("case", MERGE_CASES, ids=[c[0] for c in MERGE_CASES])
def test_in_kernel_merge(case):
    """Splits merged inside the decode launch (the last split of each sequence and
    KV head to finish merges, through a counter it resets) give the bits of the
    separate combine launch; the same zeroed workspace serves later calls, so the
    counters are back at zero after each one; one-split sequences are written
    directly."""
    need_gpu()
    name, dtype, Hq, Hkv, d, bps, lengths, kernel = case
    print_case(test="in_kernel_merge", case=name)
    batch = make_batch(dtype, 1, 700, Hq, Hkv, d, 16, lengths, seed=zlib.crc32(name.encode()) % 10000)
    sep, _, _ = run_library(batch, 0, kernel=kernel, bps=bps)
    geom = pk.Geometry(1, Hkv, d, 16, 700, dtype)
    need = pk.decode_workspace_bytes(geom, len(lengths), Hq, int(max(lengths)), bps, kernel, True)
    assert need >= pk.decode_workspace_bytes(geom, len(lengths), Hq, int(max(lengths)), bps, kernel)
    ws = torch.zeros(max(1, need), dtype=torch.uint8, device="cuda")
    for rep in range(3):
        got, _, _ = run_library(batch, 0, kernel=kernel, bps=bps, merge=True, ws=ws)
        assert np.array_equal(got.view(np.uint8), sep.view(np.uint8)), (name, rep)
    counters = ws[-((len(lengths) * Hkv * 4 + 15) // 16 * 16):].cpu().numpy()
    assert not counters.any(), "counters not back at zero"
    _, _, expect = oracle_step(batch, 0)
    assert max_abs_err(got, expect, dtype) <= (BF16_TOL if dtype == "bf16" else F32_TOL)


WG_CASES = [
    # name, dtype, Hq, Hkv, d, bps (per wave), waves per workgroup, merge
    ("f32_d64_mha_w16", "f32", 12, 12, 64, 2, 16, False),
    ("f32_d64_mha_w4_merge", "f32", 12, 12, 64, 2, 4, True),
    ("f32_d128_g4_w8", "f32", 8, 2, 128, 1, 8, True),
    ("bf16_d128_g8_w8_merge", "bf16", 64, 8, 128, 2, 8, True),
    ("bf16_d128_mha_w16", "bf16", 4, 4, 128, 2, 16, False),
    ("bf16_d64_g2_w2", "bf16", 8, 4, 64, 4, 2, False),
]


@pytest.mark.parametrize("case", WG_CASES, ids=[c[0] for c in WG_CASES])
def test_valu_workgroup_waves(case):
    """Several waves per workgroup split its blocks and merge through LDS; the
    workgroup's merged partial then goes to the combine launch or the in-kernel
    merge. Against the oracle, and (fp32) within 1e-6 of one wave per item."""
    need_gpu()
    name, dtype, Hq, Hkv, d, bps, waves, merge = case
    print_case(test="valu_workgroup_waves", case=name)
    lengths = RAGGED + [1000, 16 * 40]
    batch = make_batch(dtype, 1, 700, Hq, Hkv, d, 16, lengths, seed=zlib.crc32(name.encode()) % 10000)
    got, _, _ = run_library(batch, 0, kernel="valu", bps=bps, merge=merge, waves=waves)
    _, _, expect = oracle_step(batch, 0)
    assert max_abs_err(got, expect, dtype) <= (BF16_TOL if dtype == "bf16" else F32_TOL), name
    one, _, _ = run_library(batch, 0, kernel="valu", bps=bps, merge=merge)
    if dtype == "f32":
        assert np.max(np.abs(got.astype(np.float64) - one.astype(np.float64))) <= 1e-6, name
    again, _, _ = run_library(batch, 0, kernel="valu", bps=bps, merge=merge, waves=waves)
    assert np.array_equal(got.view(np.uint8), again.view(np.uint8)), name


RAGGED_PLAN_CASES = [
    # name, Hq, Hkv, d, lengths, bps, merge
    ("uneven_auto", 32, 8, 128, [1, 2000, 17, 300, 0, 1024, 64, 5000, 33], 0, False),
    ("uneven_auto_merge", 32, 8, 128, [1, 2000, 17, 300, 0, 1024, 64, 5000, 33], 0, True),
    ("items_of_6", 64, 8, 128, [300, 1, 900, 40, 0], 6, False),
    ("items_of_4_merge_d64", 32, 2, 64, [129, 3000, 7, 640], 4, True),
    ("items_of_2_g16_d64", 32, 2, 64, RAGGED, 2, False),
    # longest sequence within three balanced items: one item each, outputs direct
    ("unsplit_auto", 32, 8, 128, [1, 40, 300, 700, 17, 100, 0], 0, False),
    ("unsplit_auto_merge", 32, 8, 128, [1, 40, 300, 700, 17, 100, 0], 0, True),
]


@pytest.mark.parametrize("case", RAGGED_PLAN_CASES, ids=[c[0] for c in RAGGED_PLAN_CASES])
def test_ragged_plan(case):
    """With the host copy of the lengths the MFMA kernel takes a list of work
    items -- long sequences cut into items, longest first -- from its arguments:
    outputs within the bf16 tolerance of the oracle (and of the uniform plan),
    empty sequences zero, and the same bits on a second call."""
    need_gpu()
    name, Hq, Hkv, d, lengths, bps, merge = case
    print_case(test="ragged_plan", case=name)
    batch = make_batch("bf16", 1, 900, Hq, Hkv, d, 16, lengths, seed=zlib.crc32(name.encode()) % 10000)
    hl = np.asarray(lengths, np.int32)
    got, _, _ = run_library(batch, 0, kernel="mfma", bps=bps, merge=merge, host_lens=hl)
    _, _, expect = oracle_step(batch, 0)
    assert max_abs_err(got, expect, "bf16") <= BF16_TOL, name
    for i, S in enumerate(lengths):
        if S == 0:
            assert not np.any(got[i].view(np.uint8)), (name, i)
    uniform, _, _ = run_library(batch, 0, kernel="mfma", bps=bps, merge=merge)
    assert np.max(np.abs(olayout_widen(got) - olayout_widen(uniform))) <= BF16_TOL
    again, _, _ = run_library(batch, 0, kernel="mfma", bps=bps, merge=merge, host_lens=hl)
    assert np.array_equal(got.view(np.uint8), again.view(np.uint8)), name


def olayout_widen(a):
    from oracle import layout
    return layout.widen(a, "bf16")


def test_uniform_lengths_keep_the_uniform_plan():
    """Even lengths: the host copy changes nothing (same bits as without it)."""
    need_gpu()
    print_case(test="ragged_uniform")
    lengths = [700] * 6
    batch = make_batch("bf16", 1, 400, 32, 8, 128, 16, lengths, seed=808)
    a, _, _ = run_library(batch, 0, kernel="mfma")
    b, _, _ = run_library(batch, 0, kernel="mfma", host_lens=np.asarray(lengths, np.int32))
    assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
