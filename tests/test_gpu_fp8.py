"""GPU parity of one-byte (FP8) KV storage against the FP8 oracle.

The reading of the pages ("KV Cache Management": b_elem = 1 byte for FP8, no
format or scale given) is the one oracle/fp8.py states: OCP E4M3 codes with one
power-of-two scale per (token, KV head), the smallest 2**e with max|x| <=
448 * 2**e. Quantization is integer / rounding work, so pools must match the
oracle bit for bit; decode outputs (bf16) are within 2e-2 * max(1, max |o|) of
the oracle's exact attention over the dequantized cache, per (sequence, query
head): rows here carry magnitudes 10**U(-1, 1) (one case 10**U(-4, 4)), and a
bf16 output keeps about 2**-9 of its magnitude. Unused slots hold NaN codes and scale
byte 0xFF, which the kernels must never let into a result.
"""
import zlib

import numpy as np
import pytest
import torch

import paged_kv_cache_83_amd as pk
from oracle import block_manager as obm
from oracle import fp8
from oracle import kv_ops as okv
from oracle import layout as olayout
from synth import gen
from tests.gpu_helpers import (BF16_TOL, max_abs_err, need_gpu, padded_tables, print_case, to_dev,
                               to_host)

pytestmark = pytest.mark.gpu


def scaled_rows(seed, n, H, d, decades=4.0):
    """bf16 rows of N(0,1) values times a per-row magnitude 10**U(-decades, decades)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, H, d)) * 10.0 ** rng.uniform(-decades, decades, (n, H, 1))
    return gen.f32_to_bf16_bits(x.astype(np.float32))


def place_rows(kp, vp, layer, N, H, B, d, slots, K, V):
    """Quantize rows K, V [n, H, d] (float64) with the oracle into the listed slots
    of byte pools [L, N, H, B*d + B], through the documented offsets."""
    TB = B * d + B
    n = len(slots)
    kc, ks = fp8.quantize_rows(K.reshape(n * H, d))
    vc, vs = fp8.quantize_rows(V.reshape(n * H, d))
    p = np.repeat(np.asarray(slots) // B, H)
    o = np.repeat(np.asarray(slots) % B, H)
    h = np.tile(np.arange(H), n)
    base = ((layer * N + p) * H + h) * TB
    j = np.arange(d)
    kidx = base[:, None] + fp8.k_code_index(o[:, None], j[None], B, d)
    vidx = base[:, None] + fp8.v_code_index(o[:, None], j[None], B, d)
    kf, vf = kp.reshape(-1), vp.reshape(-1)
    kf[kidx] = kc
    vf[vidx] = vc
    kf[base + B * d + o] = ks
    vf[base + B * d + o] = vs


def poisoned_pools(L, N, H, B, d):
    kp = np.full(fp8.pool_shape(L, N, H, B, d), 0x7F, np.uint8)
    vp = np.full_like(kp, 0x7F)
    for t in (kp, vp):
        t[..., B * d:] = 0xFF
    return kp, vp


APPEND_CASES = [
    # name, L, N, H, d, B, n_tokens
    ("d128_b16", 2, 40, 8, 128, 16, 70),
    ("d64_b16", 1, 33, 2, 64, 16, 200),
    ("d96_b16", 1, 20, 2, 96, 16, 50),      # K in the bf16 order (64 does not divide 96), V reordered
    ("d32_b16", 1, 20, 2, 32, 16, 50),      # the same with one 32-dimension V group
    ("d40_b4", 2, 20, 3, 40, 4, 50),        # W = d = 40
    ("d5_b3", 1, 17, 1, 5, 3, 40),
]


@pytest.mark.parametrize("case", APPEND_CASES, ids=[c[0] for c in APPEND_CASES])
def test_fp8_append_bit_exact(case):
    need_gpu()
    name, L, N, H, d, B, n = case
    print_case(test="fp8_append", case=name)
    rng = np.random.default_rng(len(name) * 7)
    kp = rng.integers(0, 256, fp8.pool_shape(L, N, H, B, d), dtype=np.uint8)
    vp = rng.integers(0, 256, fp8.pool_shape(L, N, H, B, d), dtype=np.uint8)
    n = min(n, N * B)
    slots = rng.permutation(N * B)[:n].astype(np.int64)
    slots[::9] = -1
    kn, vn = scaled_rows(1, n, H, d), scaled_rows(2, n, H, d)
    kn[0] = 0                                                     # all-zero rows: e = 0
    vn[1] = gen.f32_to_bf16_bits(np.full((H, d), 448.0 * 2.0 ** -5, np.float32))
    vn[2] = gen.f32_to_bf16_bits(np.full((H, d), 3.0e38, np.float32))
    kn[3] = gen.f32_to_bf16_bits(np.full((H, d), 2.0 ** -120, np.float32))
    layer = L - 1
    geom = pk.Geometry(L, H, d, B, N, "fp8")
    K, V = to_dev(kp, "fp8"), to_dev(vp, "fp8")
    pk.append_kv(geom, K, V, layer, to_dev(kn, "bf16"), to_dev(vn, "bf16"),
                 torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    ek, ev = fp8.append_kv(kp, vp, layer, kn, vn, slots, B)
    assert np.array_equal(to_host(K, "fp8"), ek), "K pool"
    assert np.array_equal(to_host(V, "fp8"), ev), "V pool"


def make_decode_case(Hq, Hkv, d, lengths, seed, N=None, L=2, decades=1.0):
    B = 16
    need = sum(-(-int(S) // B) for S in lengths)
    N = N or need + 7
    order = gen.permutation(seed, N)
    bm = obm.BlockManager(N, B, order)
    tables = []
    for S in lengths:
        s = bm.seq_new()
        bm.append(s, int(S))
        tables.append(bm.table(s))
    kp, vp = poisoned_pools(L, N, Hkv, B, d)
    for layer in range(L):
        for i, S in enumerate(lengths):
            slots = np.array([tables[i][t // B] * B + t % B for t in range(int(S))], np.int64)
            K = olayout.widen(scaled_rows(seed + 10 * i + layer, int(S), Hkv, d, decades), "bf16")
            V = olayout.widen(scaled_rows(seed + 10 * i + layer + 5, int(S), Hkv, d, decades), "bf16")
            place_rows(kp, vp, layer, N, Hkv, B, d, slots, K, V)
    q = gen.normal_values(seed + 3, (len(lengths), Hq, d), "bf16")
    return dict(N=N, L=L, B=B, Hq=Hq, Hkv=Hkv, d=d, tables=tables, lengths=np.asarray(lengths),
                kp=kp, vp=vp, q=q)


def run_decode(c, layer, bps=0, kv_reuse=False, K=None, V=None, tables=None, merge=False, ws=None):
    geom = pk.Geometry(c["L"], c["Hkv"], c["d"], c["B"], c["N"], "fp8")
    K = to_dev(c["kp"], "fp8") if K is None else K
    V = to_dev(c["vp"], "fp8") if V is None else V
    tabs = c["tables"] if tables is None else tables
    mb = max(1, max(len(t) for t in tabs))
    n = len(c["lengths"])
    max_ctx = int(max(c["lengths"].max(), 1))
    q = to_dev(c["q"], "bf16")
    out = torch.full_like(q, float("nan"))
    if ws is None:
        ws_bytes = pk.decode_workspace_bytes(geom, n, c["Hq"], max_ctx, bps, merge=merge)
        ws = torch.zeros(max(1, ws_bytes), dtype=torch.uint8, device="cuda")
    pk.decode(geom, K, V, layer, q, out, torch.from_numpy(padded_tables(tabs, mb)).cuda(),
              torch.from_numpy(c["lengths"].astype(np.int32)).cuda(), max_ctx, workspace=ws,
              blocks_per_split=bps, kv_reuse=kv_reuse, merge=merge)
    torch.cuda.synchronize()
    return to_host(out, "bf16")


def rel_err(got, expect):
    """max |got - expect| over each (sequence, query head), divided by
    max(1, max |expect|) of that head: bf16 output keeps ~2**-9 of the value."""
    g = olayout.widen(got, "bf16")
    scale = np.maximum(1.0, np.max(np.abs(expect), axis=-1, keepdims=True))
    return float(np.max(np.abs(g - expect) / scale))


DECODE_CASES = [
    # name, Hq, Hkv, d, lengths, blocks per split, decades of per-row magnitude
    ("d128_g8_direct", 64, 8, 128, [1, 17, 300, 1000, 31], 0, 1.0),
    ("d128_g8_splits", 32, 4, 128, [700, 1, 33, 2048], 4, 1.0),
    ("d64_g4", 16, 4, 64, [5, 129, 400], 0, 1.0),
    ("d64_g16_splits", 32, 2, 64, [250, 16, 600], 2, 1.0),
    ("d128_mha", 4, 4, 128, [90, 1, 64], 0, 1.0),
    ("with_empty", 16, 2, 128, [0, 45, 0, 300], 2, 1.0),
    ("d128_wide_range", 32, 4, 128, [400, 129], 4, 4.0),   # magnitudes 1e-4 .. 1e4: relative bound
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_fp8_decode_parity(case):
    need_gpu()
    name, Hq, Hkv, d, lengths, bps, decades = case
    print_case(test="fp8_decode", case=name)
    c = make_decode_case(Hq, Hkv, d, lengths, seed=len(name) * 13, decades=decades)
    for layer in (0, 1):
        got = run_decode(c, layer, bps)
        expect = fp8.paged_decode(c["q"], c["kp"], c["vp"], layer, c["tables"], c["lengths"], c["B"])
        assert np.isfinite(olayout.widen(got, "bf16")).all(), name
        err = rel_err(got, expect)
        assert err <= BF16_TOL, (name, layer, err, max_abs_err(got, expect, "bf16"))
    cached = run_decode(c, 1, bps, kv_reuse=True)
    assert np.array_equal(cached, run_decode(c, 1, bps))           # load kind changes no bit


def test_fp8_placement_invariance_bitwise():
    need_gpu()
    print_case(test="fp8_placement")
    a = make_decode_case(16, 2, 128, [300, 77], seed=61)
    b = make_decode_case(16, 2, 128, [300, 77], seed=62, N=a["N"])
    for ta, tb in zip(a["tables"], b["tables"]):
        for lb in range(len(ta)):
            b["kp"][:, tb[lb]] = a["kp"][:, ta[lb]]
            b["vp"][:, tb[lb]] = a["vp"][:, ta[lb]]
    b["q"] = a["q"]
    assert a["tables"] != b["tables"]
    assert np.array_equal(run_decode(a, 0), run_decode(b, 0))


FUSED_CASES = [
    # name, d, lengths, blocks per split, merge inside the launch
    ("d128", 128, [1, 40, 257, 16], 0, False),
    ("d128_split2", 128, [1, 40, 257, 16, 0, 100], 2, False),
    ("d128_split4_merge", 128, [300, 17, 64, 1], 4, True),
    ("d64_split2", 64, [1, 40, 257, 16, 0, 33], 2, False),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_fp8_decode_append_fused_api(case):
    """pa_decode_append on an FP8 pool: the item holding each sequence's last
    block quantizes the step's token into slot len-1 inside the decode launch
    (pool bytes equal the oracle's append) and attends over it."""
    need_gpu()
    name, d, lengths, bps, merge = case
    print_case(test="fp8_decode_append", case=name)
    c = make_decode_case(32, 4, d, lengths, seed=71 + len(name))
    B, layer = c["B"], 1
    n = len(lengths)
    kn, vn = scaled_rows(81, n, c["Hkv"], d, 1.0), scaled_rows(82, n, c["Hkv"], d, 1.0)
    slots = [c["tables"][i][(S - 1) // B] * B + (S - 1) % B if S > 0 else -1
             for i, S in enumerate(lengths)]
    ek, ev = fp8.append_kv(c["kp"], c["vp"], layer, kn, vn, slots, B)
    geom = pk.Geometry(c["L"], c["Hkv"], d, B, c["N"], "fp8")
    K, V = to_dev(c["kp"], "fp8"), to_dev(c["vp"], "fp8")
    mb = max(len(t) for t in c["tables"])
    q = to_dev(c["q"], "bf16")
    out = torch.full_like(q, float("nan"))
    max_ctx = max(lengths)
    ws = torch.zeros(max(1, pk.decode_workspace_bytes(geom, n, 32, max_ctx, bps, "auto", merge)),
                     dtype=torch.uint8, device="cuda")
    pk.decode_append(geom, K, V, layer, q, to_dev(kn, "bf16"), to_dev(vn, "bf16"), out,
                     torch.from_numpy(padded_tables(c["tables"], mb)).cuda(),
                     torch.tensor(lengths, dtype=torch.int32, device="cuda"), max_ctx, workspace=ws,
                     blocks_per_split=bps, merge=merge)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(K, "fp8"), ek) and np.array_equal(to_host(V, "fp8"), ev)
    expect = fp8.paged_decode(c["q"], ek, ev, layer, c["tables"], lengths, B)
    assert rel_err(to_host(out, "bf16"), expect) <= BF16_TOL


@pytest.mark.parametrize("geo", [(2, 30, 8, 128, 16), (1, 20, 1, 4, 3)], ids=["d128", "odd_run"])
def test_fp8_block_moves_bit_exact(geo):
    need_gpu()
    L, N, H, d, B = geo
    print_case(test="fp8_block_moves", geo=geo)
    rng = np.random.default_rng(5)
    kp = rng.integers(0, 256, fp8.pool_shape(L, N, H, B, d), dtype=np.uint8)
    vp = rng.integers(0, 256, fp8.pool_shape(L, N, H, B, d), dtype=np.uint8)
    geom = pk.Geometry(L, H, d, B, N, "fp8")
    assert pk.bytes_per_block(geom) == 2 * L * H * (B * d + B)
    K, V = to_dev(kp, "fp8"), to_dev(vp, "fp8")
    src, dst = np.array([3, 7, 1], np.int32), np.array([10, 2, 15], np.int32)
    pk.copy_blocks(geom, K, V, torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda())
    ek, ev = okv.copy_blocks(kp, vp, src, dst)
    assert np.array_equal(to_host(K, "fp8"), ek) and np.array_equal(to_host(V, "fp8"), ev)
    ids = np.array([4, 0, 19, 8], np.int32)
    staging = torch.empty(len(ids) * pk.bytes_per_block(geom), dtype=torch.uint8, device="cuda")
    pk.gather_blocks(geom, K, V, torch.from_numpy(ids).cuda(), staging)
    expect = okv.gather_blocks(ek, ev, ids)
    assert np.array_equal(staging.cpu().numpy(), np.ascontiguousarray(expect).view(np.uint8).ravel())
    back = np.array([12, 13, 5, 6], np.int32)
    pk.scatter_blocks(geom, K, V, staging, torch.from_numpy(back).cuda())
    sk, sv = okv.scatter_blocks(ek, ev, expect, back)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(K, "fp8"), sk) and np.array_equal(to_host(V, "fp8"), sv)


def test_fp8_swap_round_trip():
    need_gpu()
    print_case(test="fp8_swap")
    L, N, H, d, B = 2, 48, 2, 128, 16
    rng = np.random.default_rng(9)
    kp = rng.integers(0, 256, fp8.pool_shape(L, N, H, B, d), dtype=np.uint8)
    vp = rng.integers(0, 256, fp8.pool_shape(L, N, H, B, d), dtype=np.uint8)
    geom = pk.Geometry(L, H, d, B, N, "fp8")
    bm = pk.BlockManager(N, B, gen.permutation(3, N))
    s = bm.seq_new()
    bm.append(s, 16 * 20)
    K, V = to_dev(kp, "fp8"), to_dev(vp, "fp8")
    before = [(kp[:, p].copy(), vp[:, p].copy()) for p in bm.table(s)]
    sw = pk.Swapper(geom, bm, K, V, 24, chunk_blocks=7)
    sw.swap_out(s, list(range(20)))
    sw.sync()
    free = torch.as_tensor(bm.free_list(), dtype=torch.long, device="cuda")
    K.index_fill_(1, free, 0x7F)
    V.index_fill_(1, free, 0x7F)
    bm.permute_free(gen.permutation(4, bm.num_free()))
    sw.swap_in(s, list(range(19, -1, -1)))
    sw.sync()
    Kh, Vh = to_host(K, "fp8"), to_host(V, "fp8")
    for lb, p in enumerate(bm.table(s)):
        assert np.array_equal(Kh[:, p], before[lb][0]) and np.array_equal(Vh[:, p], before[lb][1])
    sw.close()


def test_fp8_unsupported_geometries():
    need_gpu()
    print_case(test="fp8_unsupported")
    geom = pk.Geometry(1, 2, 64, 8, 8, "fp8")                      # B = 8: no FP8 decode kernel
    K, V = pk.alloc_pools(geom)
    q = torch.zeros(1, 4, 64, dtype=torch.bfloat16, device="cuda")
    tab = torch.zeros(1, 2, dtype=torch.int32, device="cuda")
    ln = torch.ones(1, dtype=torch.int32, device="cuda")
    with pytest.raises(pk.PagedKVError):
        pk.decode(geom, K, V, 0, q, torch.empty_like(q), tab, ln, 1)
    geom = pk.Geometry(1, 2, 64, 16, 8, "fp8")
    K, V = pk.alloc_pools(geom)
    with pytest.raises(pk.PagedKVError):                            # generic kernel: bf16 / fp32 only
        pk.decode(geom, K, V, 0, q, torch.empty_like(q), tab, ln, 1, kernel="generic")
    kn = torch.zeros(1, 2, 64, dtype=torch.bfloat16, device="cuda")
    geom8 = pk.Geometry(1, 2, 64, 8, 8, "fp8")
    K8, V8 = pk.alloc_pools(geom8)
    with pytest.raises(pk.PagedKVError):                            # chunked prefill: B = 16 only
        pk.prefill(geom8, K8, V8, 0, q, kn, kn, torch.empty_like(q),
                   torch.tensor([0, 1], dtype=torch.int32, device="cuda"), tab,
                   torch.zeros(1, dtype=torch.int32, device="cuda"), 1, 1)


def test_fp8_in_kernel_merge_same_bits():
    """FP8 decode with the splits merged inside the launch gives the bits of the
    separate combine launch, call after call on one zeroed workspace."""
    need_gpu()
    print_case(test="fp8_in_kernel_merge")
    for name, Hq, Hkv, d, lengths, bps, dec in DECODE_CASES:
        if bps == 0:
            continue
        c = make_decode_case(Hq, Hkv, d, lengths, seed=zlib.crc32(name.encode()) % 10000, decades=dec)
        sep = run_decode(c, 0, bps=bps)
        geom = pk.Geometry(c["L"], Hkv, d, c["B"], c["N"], "fp8")
        need = pk.decode_workspace_bytes(geom, len(lengths), Hq, int(max(max(lengths), 1)), bps,
                                         merge=True)
        ws = torch.zeros(max(1, need), dtype=torch.uint8, device="cuda")
        for rep in range(2):
            got = run_decode(c, 0, bps=bps, merge=True, ws=ws)
            assert np.array_equal(got.view(np.uint8), sep.view(np.uint8)), (name, rep)


def test_fp8_gqa70b_32k_full_size_sampled():
    """The 70B decode batch on one-byte pools at its full per-layer size (16 x
    32,768 tokens, a 32,768-block pool of 8 heads, head dim 128), two layers, in
    the launch plan the benchmark times (8 splits of 256 blocks and the combine):
    sampled (sequence, layer) outputs against the oracle. The pools hold random
    finite E4M3 codes with scale bytes 2^-3 .. 2^3 in seeded random placement."""
    need_gpu()
    print_case(test="fp8_full_size")
    L, N, H, Hq, B, d, n, S = 2, 32768, 8, 64, 16, 128, 16, 32768
    tb = fp8.tile_bytes(B, d)
    g = torch.Generator(device="cuda").manual_seed(8311)
    pools = []
    for _ in range(2):
        t = torch.randint(0, 0x7F, (L, N, H, tb), generator=g, device="cuda", dtype=torch.int32)
        sign = torch.randint(0, 2, (L, N, H, tb), generator=g, device="cuda", dtype=torch.int32) << 7
        t = (t | sign).to(torch.uint8)                     # codes 0x7F / 0xFF (NaN) never occur
        t[..., B * d:] = torch.randint(124, 131, (L, N, H, B), generator=g, device="cuda",
                                       dtype=torch.int32).to(torch.uint8)
        pools.append(t)
    K, V = pools
    order = gen.permutation(8312, N)
    nb = S // B
    tables = [[int(x) for x in order[i * nb:(i + 1) * nb]] for i in range(n)]
    q = gen.normal_values(8313, (n, Hq, d), "bf16")
    c = dict(N=N, L=L, B=B, Hq=Hq, Hkv=H, d=d, tables=tables, lengths=np.full(n, S), q=q)
    rng = np.random.default_rng(8314)
    samples = [(int(rng.integers(0, n)), int(rng.integers(0, L))) for _ in range(3)]
    kh, vh = K.cpu().numpy(), V.cpu().numpy()
    for layer in sorted({s[1] for s in samples}):
        got = run_decode(c, layer, K=K, V=V)
        assert np.isfinite(olayout.widen(got, "bf16")).all()
        for (i, lyr) in samples:
            if lyr != layer:
                continue
            expect = fp8.paged_decode(q, kh, vh, layer, tables, c["lengths"], B, seqs=[i])
            err = rel_err(got[i:i + 1], expect[i:i + 1])
            assert err <= BF16_TOL, (i, layer, err)
    del K, V, pools
    torch.cuda.empty_cache()
