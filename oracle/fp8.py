"""One-byte (FP8) KV storage, oracle side (test infrastructure).

Passages followed:

* "KV Cache Management", section "From Context Tokens to KV State", Eq. (1), and
  section "Retain, Evict, Recompute, or Offload": the per-token footprint is
  2 * L * H_kv * d * b_elem with b_elem = 1 byte for FP8. The pages name no
  element format and no scale, so the reading taken here (stated once, used by
  both sides) is:

  - element format: OCP 8-bit floating point E4M3 ("E4M3FN": 1 sign bit, 4
    exponent bits with bias 7, 3 mantissa bits, no infinities, the all-ones
    magnitude 0x7F is NaN, largest finite value 448), as defined by the OCP
    8-bit Floating Point Specification (OFP8);
  - one scale per (token, KV head) for K and one for V: a power of two 2**e,
    with e the smallest integer such that max|x| <= 448 * 2**e over the d
    values of that token's head (so no element overflows), clamped to
    [-127, 127], and e = 0 for an all-zero vector; stored as one byte e + 127
    (the E8M0 encoding of the OCP Microscaling Formats specification);
  - elements: x * 2**-e rounded to the nearest E4M3 value, ties to the even
    code (round-to-nearest-even of OFP8); the stored value is code * 2**e.

* Pool layout (a property of the library's interface, restated; the pages give
  no byte layout for a one-byte cache): every (layer, block, head) tile holds
  the B * d element codes followed by the B scale bytes of its slots, one per
  slot in slot order; a pool is uint8 [L][N][H_kv][B*d + B]. Code of slot o,
  dimension j:

  - K, when B = 16 and 64 divides d: at 1024 * (j // 64) + 64 * r(o)
    + 16 * ((j // 8) % 4) + 8 * ((j // 32) % 2) + j % 8, where r(o) swaps bits 2
    and 3 of o: rows of 64 codes, slots in row order 0-3, 8-11, 4-7, 12-15, a
    row holding its 64 dimensions as 8-dimension groups 0, 4, 1, 5, 2, 6, 3, 7;
    otherwise at (j // W) * B * W + o * W + j % W with W = 32 when 32 divides d,
    else W = d (the bf16 K layout);
  - V, when B = 16 and 32 divides d: at 512 * (j // 32) + 256 * (o // 8)
    + 16 * (j % 16) + 8 * ((j // 16) % 2) + o % 8; otherwise at j * B + o (the
    bf16 V layout).

Everything here is plain and slow on purpose: the code table is the spec's
formula evaluated for all 256 codes and encoding is a nearest-value search in it.
"""

from __future__ import annotations

import math

import numpy as np

from . import attention
from . import layout

E4M3_MAX = 448.0
SCALE_BIAS = 127


def decode_code(c: int) -> float:
    """Value of one E4M3 code (OFP8: bias 7, subnormals at exponent field 0,
    S.1111.111 is NaN)."""
    s = -1.0 if c & 0x80 else 1.0
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * m * 2.0 ** -9                 # (m / 8) * 2**(1 - 7)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


TABLE = np.array([decode_code(c) for c in range(256)], dtype=np.float64)
# finite non-negative codes in increasing value order: 0x00 .. 0x7E
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALS = TABLE[:0x7F]


def encode(values) -> np.ndarray:
    """Nearest E4M3 code of each value, ties to the even code. |v| must not
    exceed 448 (the scale rule guarantees it); zero keeps its sign."""
    v = np.asarray(values, dtype=np.float64)
    if not np.all(np.isfinite(v)) or np.any(np.abs(v) > E4M3_MAX):
        raise ValueError("E4M3 encode: value out of range")
    a = np.abs(v).ravel()
    hi = np.searchsorted(_POS_VALS, a, side="left")          # first code with value >= a
    hi = np.minimum(hi, len(_POS_VALS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALS[lo]
    d_hi = _POS_VALS[hi] - a
    pick = np.where(d_lo < d_hi, lo, hi)
    tie = (d_lo == d_hi) & (lo != hi)
    pick = np.where(tie, np.where(_POS_CODES[lo] % 2 == 0, lo, hi), pick)
    codes = _POS_CODES[pick].astype(np.uint8)
    neg = np.signbit(v.ravel())
    codes = np.where(neg, codes | np.uint8(0x80), codes).astype(np.uint8)
    return codes.reshape(v.shape)


def decode(codes) -> np.ndarray:
    return TABLE[np.asarray(codes, dtype=np.uint8)]


def scale_exponent(amax: float) -> int:
    """Smallest integer e with amax <= 448 * 2**e, clamped to [-127, 127];
    0 for amax == 0. Exact: 448 = 0.875 * 2**9 and frexp gives amax = m * 2**x
    with m in [0.5, 1), so the condition is m <= 0.875 * 2**(9 + e - x)."""
    amax = float(amax)
    if amax == 0.0:
        return 0
    m, x = math.frexp(amax)
    e = x - 9 if m <= 0.875 else x - 8
    return max(-127, min(127, e))


def quantize_vector(x):
    """(codes uint8 [d], scale byte) of one token's head vector (float64 values)."""
    x = np.asarray(x, dtype=np.float64)
    e = scale_exponent(np.max(np.abs(x)) if x.size else 0.0)
    return encode(x * 2.0 ** -e), e + SCALE_BIAS


def quantize_rows(X):
    """quantize_vector applied to every row of X [n, d]: (codes [n, d], bytes [n])."""
    X = np.asarray(X, dtype=np.float64)
    e = np.array([scale_exponent(a) for a in np.max(np.abs(X), axis=1)], dtype=np.int64)
    codes = encode(X * np.ldexp(1.0, -e)[:, None])
    return codes, (e + SCALE_BIAS).astype(np.uint8)


def dequantize_vector(codes, scale_byte) -> np.ndarray:
    return decode(codes) * 2.0 ** (int(scale_byte) - SCALE_BIAS)


# ---- pool layout ------------------------------------------------------------
def tile_bytes(block_size: int, head_dim: int) -> int:
    return block_size * head_dim + block_size


def pool_shape(num_layers, num_blocks, num_kv_heads, block_size, head_dim):
    return (num_layers, num_blocks, num_kv_heads, tile_bytes(block_size, head_dim))


def _swap_bits_2_3(o):
    return (o & ~12) | ((o >> 1) & 4) | ((o << 1) & 8)


def k_code_index(offset, j, block_size, head_dim):
    """Byte of slot `offset`'s dimension j in a K tile (ints or integer arrays)."""
    if block_size == 16 and head_dim % 64 == 0:
        return (1024 * (j // 64) + 64 * _swap_bits_2_3(offset) + 16 * ((j // 8) % 4)
                + 8 * ((j // 32) % 2) + j % 8)
    W = layout.k_chunk(head_dim)
    return (j // W) * block_size * W + offset * W + (j % W)


def v_code_index(offset, j, block_size, head_dim):
    """Byte of slot `offset`'s dimension j in a V tile (ints or integer arrays)."""
    if block_size == 16 and head_dim % 32 == 0:
        return 512 * (j // 32) + 256 * (offset // 8) + 16 * (j % 16) + 8 * ((j // 16) % 2) + offset % 8
    return j * block_size + offset


def write_token(k_pool, v_pool, layer, phys, head, offset, k_vals, v_vals, block_size, head_dim):
    """Quantize one token's K and V (float64 [d] each) into slot `offset`."""
    kc, ks = quantize_vector(k_vals)
    vc, vs = quantize_vector(v_vals)
    kt = k_pool[layer, phys, head]
    vt = v_pool[layer, phys, head]
    for j in range(head_dim):
        kt[k_code_index(offset, j, block_size, head_dim)] = kc[j]
        vt[v_code_index(offset, j, block_size, head_dim)] = vc[j]
    kt[block_size * head_dim + offset] = ks
    vt[block_size * head_dim + offset] = vs


def read_k(k_pool, layer, phys, head, offset, block_size, head_dim) -> np.ndarray:
    """Dequantized K (float64 [d]) of one slot."""
    kt = k_pool[layer, phys, head]
    codes = [kt[k_code_index(offset, j, block_size, head_dim)] for j in range(head_dim)]
    return dequantize_vector(codes, kt[block_size * head_dim + offset])


def read_v(v_pool, layer, phys, head, offset, block_size, head_dim) -> np.ndarray:
    vt = v_pool[layer, phys, head]
    codes = [vt[v_code_index(offset, j, block_size, head_dim)] for j in range(head_dim)]
    return dequantize_vector(codes, vt[block_size * head_dim + offset])


def append_kv(k_pool, v_pool, layer, k_new, v_new, slots, block_size, dtype="bf16"):
    """Copies of the pools with token j's K/V (storage form [n, H_kv, d]) quantized
    into slot slots[j] of one layer; a negative slot skips the token."""
    kp, vp = k_pool.copy(), v_pool.copy()
    kf, vf = layout.widen(k_new, dtype), layout.widen(v_new, dtype)
    num_kv_heads, head_dim = kf.shape[1], kf.shape[2]
    for j, s in enumerate(np.asarray(slots).tolist()):
        if s < 0:
            continue
        phys, off = s // block_size, s % block_size
        for h in range(num_kv_heads):
            write_token(kp, vp, layer, phys, h, off, kf[j, h], vf[j, h], block_size, head_dim)
    return kp, vp


def _tile_offsets(index, block_size, head_dim):
    o = np.arange(block_size)[:, None]
    j = np.arange(head_dim)[None, :]
    return index(o, j, block_size, head_dim)                                    # [B, d]


def read_k_tile(k_pool, layer, phys, head, block_size, head_dim) -> np.ndarray:
    """Dequantized K of all B slots of one (layer, block, head), as [B, d]."""
    kt = k_pool[layer, phys, head]
    codes = kt[_tile_offsets(k_code_index, block_size, head_dim)]
    scales = kt[block_size * head_dim:].astype(np.int64) - SCALE_BIAS
    return decode(codes) * np.ldexp(1.0, scales)[:, None]


def read_v_tile(v_pool, layer, phys, head, block_size, head_dim) -> np.ndarray:
    """Dequantized V of all B slots of one (layer, block, head), as [B, d]."""
    vt = v_pool[layer, phys, head]
    codes = vt[_tile_offsets(v_code_index, block_size, head_dim)]
    scales = vt[block_size * head_dim:].astype(np.int64) - SCALE_BIAS
    return decode(codes) * np.ldexp(1.0, scales)[:, None]


def rebuild_sequence(k_pool, v_pool, layer, table, length, block_size, head_dim):
    """Dequantized contiguous K, V ([S, H_kv, d] float64) of one sequence."""
    num_kv_heads = k_pool.shape[2]
    K = np.zeros((length, num_kv_heads, head_dim), dtype=np.float64)
    V = np.zeros((length, num_kv_heads, head_dim), dtype=np.float64)
    for lb in range(-(-length // block_size)):
        phys, first = int(table[lb]), lb * block_size
        valid = min(block_size, length - first)      # the last block may be partly filled
        for h in range(num_kv_heads):
            K[first:first + valid, h] = read_k_tile(k_pool, layer, phys, h, block_size, head_dim)[:valid]
            V[first:first + valid, h] = read_v_tile(v_pool, layer, phys, h, block_size, head_dim)[:valid]
    return K, V


def paged_decode(q, k_pool, v_pool, layer, tables, lengths, block_size, q_dtype="bf16",
                 scale=None, seqs=None):
    """Decode output [n, H_q, d] (float64) over FP8 pools: the exact attention of
    the dequantized cache (the stored values code * 2**e)."""
    head_dim = q.shape[2]
    if scale is None or scale == 0.0:
        scale = attention.default_scale(head_dim)
    qf = layout.widen(q, q_dtype)
    out = np.zeros(qf.shape, dtype=np.float64)
    idx = range(q.shape[0]) if seqs is None else seqs
    for i in idx:
        K, V = rebuild_sequence(k_pool, v_pool, layer, tables[i], int(lengths[i]), block_size,
                                head_dim)
        out[i] = attention.attend(qf[i], K, V, scale)
    return out


def paged_prefill(q, k_new, v_new, k_pool, v_pool, layer, tables, q_start, ctx_lens, block_size,
                  q_dtype="bf16", scale=None, chunks=None):
    """Chunked prefill over FP8 pools: (pools after the chunks are written, float64
    outputs [n_tok, H_q, d]).

    "KV Cache Management", section "Chunked prefill mechanics": chunk i's row t
    attends over the cached positions and the chunk's positions 0 .. t. Reading
    taken for one-byte storage (the page names no order for a quantized cache):
    the chunk is written first and every key and value is then read back as
    stored, so the chunk's own rows enter quantized, as the cached ones do (the
    same order the decode step follows: the new token is appended, then attended).
    """
    from . import prefill as _prefill
    head_dim = q.shape[2]
    if scale is None or scale == 0.0:
        scale = attention.default_scale(head_dim)
    slots = _prefill.chunk_slots(tables, q_start, ctx_lens, block_size)
    kp, vp = append_kv(k_pool, v_pool, layer, k_new, v_new, slots, block_size, q_dtype)
    qf = layout.widen(q, q_dtype)
    out = np.zeros(qf.shape, dtype=np.float64)
    idx = range(len(ctx_lens)) if chunks is None else chunks
    for i in idx:
        a, b = _prefill.chunk_bounds(q_start, i)
        c = int(ctx_lens[i])
        K, V = rebuild_sequence(kp, vp, layer, tables[i], c + (b - a), block_size, head_dim)
        out[a:b] = _prefill.chunk_attention(qf[a:b], K[c:], V[c:], K[:c], V[:c], scale)
    return kp, vp, out
