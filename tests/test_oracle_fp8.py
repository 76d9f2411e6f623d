"""Pins of the FP8 oracle (oracle/fp8.py) to what fixes it from outside:

* the OFP8 E4M3 definition: torch's float8_e4m3fn type decodes all 256 codes to
  the same values, and encodes values in range (codes, midpoints between
  adjacent codes, random values) to the same codes (round to nearest, ties to
  even);
* closed forms of the format (largest finite 448, smallest normal 2**-6,
  smallest subnormal 2**-9, NaN codes, signed zero);
* the scale rule by brute force with exact arithmetic: 448 * 2**e covers the
  largest magnitude and 448 * 2**(e - 1) does not;
* the rounding error of a quantized vector: at most half a unit in the last
  place of the E4M3 value (2**-4 relative for normal codes, 2**(e-10) absolute
  below the normal range);
* the pool layout: bytes read back through the documented flat offsets;
* decode over a pool whose values E4M3 represents exactly equals the (separately
  pinned) bf16 oracle on the same values.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from oracle import fp8
from oracle import layout as olayout
from synth import gen


def test_table_matches_torch_e4m3fn():
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn)
    ref = codes.to(torch.float32).numpy().astype(np.float64)
    assert np.array_equal(np.isnan(ref), np.isnan(fp8.TABLE))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], fp8.TABLE[ok])


def test_closed_forms():
    assert fp8.decode_code(0x7E) == 448.0 and fp8.decode_code(0xFE) == -448.0
    assert fp8.decode_code(0x08) == 2.0 ** -6                  # smallest normal
    assert fp8.decode_code(0x01) == 2.0 ** -9                  # smallest subnormal
    assert fp8.decode_code(0x07) == 7 * 2.0 ** -9              # largest subnormal
    assert math.isnan(fp8.decode_code(0x7F)) and math.isnan(fp8.decode_code(0xFF))
    assert fp8.decode_code(0x38) == 1.0                        # exponent field 7 = bias
    assert fp8.decode_code(0x80) == 0.0 and math.copysign(1, fp8.decode_code(0x80)) == -1
    finite = fp8.TABLE[~np.isnan(fp8.TABLE)]
    assert len(finite) == 254 and np.max(finite) == 448.0


def test_round_trip_every_finite_code():
    finite = [c for c in range(256) if c not in (0x7F, 0xFF)]
    assert fp8.encode(fp8.decode(finite)).tolist() == finite


def _torch_codes(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_matches_torch_including_ties():
    pos = fp8.TABLE[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2                          # every midpoint: ties
    quarter = pos[:-1] + (pos[1:] - pos[:-1]) / 4
    rng = np.random.default_rng(5)
    rand = rng.uniform(-448, 448, 20000)
    small = rng.uniform(-2 ** -5, 2 ** -5, 5000)
    for x in (pos, mids, quarter, -mids, rand.astype(np.float32).astype(np.float64),
              small.astype(np.float32).astype(np.float64)):
        assert np.array_equal(fp8.encode(x), _torch_codes(x))


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        fp8.encode([449.0])
    with pytest.raises(ValueError):
        fp8.encode([math.nan])


def test_scale_rule_brute_force():
    rng = np.random.default_rng(9)
    cases = list(rng.lognormal(0, 12, 4000)) + [448.0 * 2.0 ** k for k in range(-40, 40)]
    cases += [math.nextafter(448.0 * 2.0 ** k, math.inf) for k in range(-40, 40)]
    cases += [math.nextafter(448.0 * 2.0 ** k, 0) for k in range(-40, 40)]
    cases += [2.0 ** k for k in range(-60, 60)] + [1e-300, 5e-45, 3.4e38]
    for a in cases:
        e = fp8.scale_exponent(a)
        assert -127 <= e <= 127
        if -127 < e < 127:
            assert a <= math.ldexp(448.0, e), a
            assert a > math.ldexp(448.0, e - 1), a
        elif e == -127:
            assert a <= math.ldexp(448.0, -127)
    assert fp8.scale_exponent(0.0) == 0
    assert fp8.scale_exponent(448.0) == 0 and fp8.scale_exponent(448.5) == 1
    assert fp8.scale_exponent(224.0) == -1 and fp8.scale_exponent(224.01) == 0


def test_quantize_error_within_half_ulp():
    rng = np.random.default_rng(11)
    for trial in range(200):
        d = int(rng.choice([5, 64, 128]))
        x = rng.standard_normal(d) * 10.0 ** rng.uniform(-6, 6)
        if trial % 7 == 0:
            x[rng.integers(0, d)] *= 1e4                          # one outlier channel
        codes, sb = fp8.quantize_vector(x)
        e = sb - fp8.SCALE_BIAS
        y = fp8.dequantize_vector(codes, sb)
        amax = np.max(np.abs(x))
        assert np.max(np.abs(y)) <= 448.0 * 2.0 ** e
        assert amax > 448.0 * 2.0 ** (e - 1)
        err = np.abs(y - x)
        bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** (e - 10))
        assert np.all(err <= bound * (1 + 1e-12)), trial
    codes, sb = fp8.quantize_vector(np.zeros(8))
    assert sb == fp8.SCALE_BIAS and not codes.any()


def test_pool_layout_flat_offsets():
    L, N, H, B, d = 2, 5, 3, 4, 64
    W = olayout.k_chunk(d)
    kp = np.zeros(fp8.pool_shape(L, N, H, B, d), np.uint8)
    vp = np.zeros_like(kp)
    rng = np.random.default_rng(3)
    kv, vv = rng.standard_normal(d) * 3, rng.standard_normal(d) / 7
    layer, p, h, o = 1, 3, 2, 2
    fp8.write_token(kp, vp, layer, p, h, o, kv, vv, B, d)
    kc, ks = fp8.quantize_vector(kv)
    vc, vs = fp8.quantize_vector(vv)
    tile = B * d + B
    base = ((layer * N + p) * H + h) * tile
    kf, vf = kp.reshape(-1), vp.reshape(-1)
    for j in range(d):
        assert kf[base + (j // W) * B * W + o * W + j % W] == kc[j]
        assert vf[base + j * B + o] == vc[j]
    assert kf[base + B * d + o] == ks and vf[base + B * d + o] == vs
    assert np.count_nonzero(kp) <= d + 1 and np.count_nonzero(vp) <= d + 1
    assert np.array_equal(fp8.read_k(kp, layer, p, h, o, B, d), fp8.dequantize_vector(kc, ks))
    assert np.array_equal(fp8.read_v(vp, layer, p, h, o, B, d), fp8.dequantize_vector(vc, vs))


@pytest.mark.parametrize("d", [128, 64])
def test_pool_layout_flat_offsets_b16(d):
    """B = 16 with 64 | d: K rows of 64 codes in slot order 0-3, 8-11, 4-7, 12-15
    per 64-dimension chunk, a row's dimensions in 8-wide groups 0, 4, 1, 5, 2, 6,
    3, 7; V as [d/32][slot half][dim % 16][(dim / 16) % 2][slot % 8]. The
    expected tiles are built row by row from that description."""
    L, N, H, B = 1, 3, 2, 16
    row_slots = [0, 1, 2, 3, 8, 9, 10, 11, 4, 5, 6, 7, 12, 13, 14, 15]
    rng = np.random.default_rng(11)
    kp = np.zeros(fp8.pool_shape(L, N, H, B, d), np.uint8)
    vp = np.zeros_like(kp)
    KC = np.zeros((B, d), np.uint8)
    VC = np.zeros((B, d), np.uint8)
    KS = np.zeros(B, np.uint8)
    VS = np.zeros(B, np.uint8)
    p, h = 2, 1
    for o in range(B):
        kv, vv = rng.standard_normal(d) * (o + 1), rng.standard_normal(d) / (o + 1)
        fp8.write_token(kp, vp, 0, p, h, o, kv, vv, B, d)
        KC[o], KS[o] = fp8.quantize_vector(kv)
        VC[o], VS[o] = fp8.quantize_vector(vv)
    group_order = [0, 4, 1, 5, 2, 6, 3, 7]
    k_expect = b"".join(bytes(KC[row_slots[r], 64 * c + 8 * gr:64 * c + 8 * gr + 8])
                        for c in range(d // 64) for r in range(16) for gr in group_order)
    v_parts = []
    for u in range(d // 32):
        for half in range(2):
            for dm in range(16):
                for hi in range(2):
                    dim = 32 * u + 16 * hi + dm
                    v_parts.append(bytes(VC[8 * half:8 * half + 8, dim]))
    v_expect = b"".join(v_parts)
    assert bytes(kp[0, p, h, :B * d]) == k_expect
    assert bytes(vp[0, p, h, :B * d]) == v_expect
    assert bytes(kp[0, p, h, B * d:]) == bytes(KS) and bytes(vp[0, p, h, B * d:]) == bytes(VS)
    assert np.array_equal(fp8.read_k_tile(kp, 0, p, h, B, d),
                          np.stack([fp8.dequantize_vector(KC[o], KS[o]) for o in range(B)]))
    assert np.array_equal(fp8.read_v_tile(vp, 0, p, h, B, d),
                          np.stack([fp8.dequantize_vector(VC[o], VS[o]) for o in range(B)]))


@pytest.mark.parametrize("B,d", [(16, 128), (16, 64), (16, 96), (16, 40), (4, 64), (3, 5), (8, 128)])
def test_pool_layout_is_a_bijection(B, d):
    """Every (slot, dimension) has its own byte of the tile's B*d code bytes."""
    o = np.arange(B)[:, None]
    j = np.arange(d)[None, :]
    for index in (fp8.k_code_index, fp8.v_code_index):
        offs = np.broadcast_to(index(o, j, B, d), (B, d)).reshape(-1)
        assert np.array_equal(np.sort(offs), np.arange(B * d)), (index.__name__, B, d)


def test_decode_equals_bf16_oracle_on_representable_values():
    """Values that E4M3 x 2**e represents exactly (and bf16 too): the FP8 pool
    decodes to exactly what the bf16 oracle gives for the same values."""
    L, N, H, Hq, B, d = 1, 24, 2, 8, 16, 64
    rng = np.random.default_rng(17)
    lengths = [37, 16, 70]
    order = gen.permutation(4, N)
    tables, k = [], 0
    for S in lengths:
        nb = -(-S // B)
        tables.append([int(x) for x in order[k:k + nb]])
        k += nb
    finite = fp8.TABLE[(~np.isnan(fp8.TABLE)) & (np.abs(fp8.TABLE) <= 448)]
    kp8 = np.zeros(fp8.pool_shape(L, N, H, B, d), np.uint8)
    vp8 = np.zeros_like(kp8)
    kb = np.zeros(olayout.k_pool_shape(L, N, H, B, d), np.uint16)
    vb = np.zeros(olayout.v_pool_shape(L, N, H, B, d), np.uint16)

    def bf16_bits(x):
        return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)

    for i, S in enumerate(lengths):
        for t in range(S):
            p, o = tables[i][t // B], t % B
            for h in range(H):
                e = int(rng.integers(-8, 4))
                kv = rng.choice(finite, d) * 2.0 ** e
                vv = rng.choice(finite, d) * 2.0 ** e
                kv[0], vv[0] = 448.0 * 2.0 ** e, -448.0 * 2.0 ** e      # pins the scale at e
                fp8.write_token(kp8, vp8, 0, p, h, o, kv, vv, B, d)
                olayout.write_k(kb, 0, p, h, o, bf16_bits(kv))
                olayout.write_v(vb, 0, p, h, o, bf16_bits(vv))
    q = gen.normal_values(21, (len(lengths), Hq, d), "bf16")
    got = fp8.paged_decode(q, kp8, vp8, 0, tables, lengths, B)
    ref = oatt.paged_decode(q, kb, vb, 0, tables, lengths, B, "bf16")
    assert np.array_equal(got, ref)


def test_append_quantizes_at_table_slots():
    L, N, H, B, d = 2, 6, 2, 4, 32
    kp = np.zeros(fp8.pool_shape(L, N, H, B, d), np.uint8)
    vp = np.zeros_like(kp)
    kn = gen.normal_values(1, (3, H, d), "bf16")
    vn = gen.normal_values(2, (3, H, d), "bf16")
    slots = [9, -1, 22]
    kp2, vp2 = fp8.append_kv(kp, vp, 1, kn, vn, slots, B)
    assert not kp2[0].any() and not vp2[0].any()             # other layer untouched
    for j, s in enumerate(slots):
        for h in range(H):
            if s < 0:
                continue
            kx = olayout.widen(kn[j, h], "bf16")
            vx = olayout.widen(vn[j, h], "bf16")
            assert np.array_equal(fp8.read_k(kp2, 1, s // B, h, s % B, B, d),
                                  fp8.dequantize_vector(*fp8.quantize_vector(kx)))
            assert np.array_equal(fp8.read_v(vp2, 1, s // B, h, s % B, B, d),
                                  fp8.dequantize_vector(*fp8.quantize_vector(vx)))


def test_quantize_rows_equals_per_vector():
    rng = np.random.default_rng(23)
    X = rng.standard_normal((40, 64)) * 10.0 ** rng.uniform(-5, 5, (40, 1))
    X[3] = 0.0
    codes, sb = fp8.quantize_rows(X)
    for r in range(40):
        c, b = fp8.quantize_vector(X[r])
        assert np.array_equal(codes[r], c) and sb[r] == b


def test_tile_reads_equal_slot_reads():
    L, N, H, B, d = 2, 4, 2, 4, 64
    rng = np.random.default_rng(29)
    kp = np.zeros(fp8.pool_shape(L, N, H, B, d), np.uint8)
    vp = np.zeros_like(kp)
    for p in range(N):
        for h in range(H):
            for o in range(B):
                fp8.write_token(kp, vp, 1, p, h, o, rng.standard_normal(d) * 5,
                                rng.standard_normal(d) / 3, B, d)
    for p in range(N):
        for h in range(H):
            kt = fp8.read_k_tile(kp, 1, p, h, B, d)
            vt = fp8.read_v_tile(vp, 1, p, h, B, d)
            for o in range(B):
                assert np.array_equal(kt[o], fp8.read_k(kp, 1, p, h, o, B, d))
                assert np.array_equal(vt[o], fp8.read_v(vp, 1, p, h, o, B, d))
