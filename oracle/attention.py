"""Decode attention over a paged pool, computed the plain way (oracle).

Definition followed: "KV Cache Management", section "Chunked prefill mechanics":
O = Softmax(Q K^T / sqrt(d_head) + M) V. For one decode query the mask M only
removes positions at or beyond the sequence's attended length, so for query head
h with KV head g = h // G (G = H_q / H_kv, contiguous groups of query heads share
one KV head, "KV Cache Management", section "From Context Tokens to KV State"):

    s_t = scale * <q_h, K[t, g]>            for t < S
    o_h = sum_t exp(s_t) V[t, g] / sum_t exp(s_t)

The keys and values are first rebuilt as contiguous [S, H_kv, d] tensors by
walking the block table (section "The PagedAttention virtual memory model":
logical block l = t // B is physical block T[l], offset t mod B), exactly as a
non-paged cache would hold them. All arithmetic is float64 on exactly widened
inputs. Subtracting the row maximum before exp is the usual overflow guard; it
does not change the value.

``attend_online`` / ``attend_split`` restate the same result by the running
statistics of the section's FlashDecoding-style recurrence (m, l and O rescaled
block by block, then partial results merged the same way). They are an
independent route to the same number and are checked against ``attend``.
"""

from __future__ import annotations

import math

import numpy as np

from . import layout


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


def rebuild_sequence(k_pool, v_pool, layer, table, length, block_size, dtype):
    """Contiguous K, V ([S, H_kv, d], float64) of one sequence from its block table."""
    num_kv_heads = k_pool.shape[2]
    head_dim = v_pool.shape[3]              # V pool is [L, N, H_kv, d, B]
    K = np.zeros((length, num_kv_heads, head_dim), dtype=np.float64)
    V = np.zeros((length, num_kv_heads, head_dim), dtype=np.float64)
    num_blocks = -(-length // block_size)
    for lb in range(num_blocks):
        phys = int(table[lb])
        first = lb * block_size
        valid = min(block_size, length - first)   # the last block may be partly filled
        for h in range(num_kv_heads):
            k_tile = layout.widen(layout.read_k_tile(k_pool, layer, phys, h), dtype)
            v_tile = layout.widen(layout.read_v_tile(v_pool, layer, phys, h), dtype)
            K[first:first + valid, h] = k_tile[:valid]
            V[first:first + valid, h] = v_tile[:valid]
    return K, V


def attend(q, K, V, scale):
    """Softmax attention of every query head over contiguous K, V.

    q: [H_q, d] float64; K, V: [S, H_kv, d] float64. Returns [H_q, d] float64.
    With S == 0 there is nothing to attend and the result is zero.
    """
    num_q_heads, head_dim = q.shape
    S, num_kv_heads, _ = K.shape
    group = num_q_heads // num_kv_heads
    out = np.zeros((num_q_heads, head_dim), dtype=np.float64)
    if S == 0:
        return out
    for h in range(num_q_heads):
        g = h // group
        s = scale * (K[:, g, :] @ q[h])
        p = np.exp(s - s.max())
        out[h] = (p @ V[:, g, :]) / p.sum()
    return out


def paged_decode(q, k_pool, v_pool, layer, tables, lengths, block_size, dtype, scale=None,
                 seqs=None):
    """Decode output [n, H_q, d] (float64) for every sequence (or the listed ones).

    q is in storage form [n, H_q, d]; tables[i] is sequence i's block table and
    lengths[i] its attended length.
    """
    head_dim = q.shape[2]
    if scale is None or scale == 0.0:
        scale = default_scale(head_dim)
    qf = layout.widen(q, dtype)
    out = np.zeros(qf.shape, dtype=np.float64)
    idx = range(q.shape[0]) if seqs is None else seqs
    for i in idx:
        K, V = rebuild_sequence(k_pool, v_pool, layer, tables[i], int(lengths[i]), block_size,
                                dtype)
        out[i] = attend(qf[i], K, V, scale)
    return out


def _block_stats(q_h, K_blk, V_blk, scale):
    """m_block, l_block, O_block of one tile of keys (unnormalised)."""
    s = scale * (K_blk @ q_h)
    m_blk = s.max()
    p = np.exp(s - m_blk)
    return m_blk, p.sum(), p @ V_blk


def _merge(m_prev, l_prev, O_prev, m_blk, l_blk, O_blk):
    """m_new = max(m_prev, m_block); l and O rescaled by exp(m_prev - m_new) and
    exp(m_block - m_new) and added ("KV Cache Management", online softmax)."""
    m_new = max(m_prev, m_blk)
    a = math.exp(m_prev - m_new) if m_prev != -math.inf else 0.0
    b = math.exp(m_blk - m_new) if m_blk != -math.inf else 0.0
    return m_new, l_prev * a + l_blk * b, O_prev * a + O_blk * b


def attend_online(q_h, K_g, V_g, scale, tile):
    """One head by the online recurrence over key tiles of `tile` positions.

    Returns the unnormalised state (m, l, O); the output is O / l.
    """
    m, l, O = -math.inf, 0.0, np.zeros(V_g.shape[1], dtype=np.float64)
    for start in range(0, K_g.shape[0], tile):
        stats = _block_stats(q_h, K_g[start:start + tile], V_g[start:start + tile], scale)
        m, l, O = _merge(m, l, O, *stats)
    return m, l, O


def attend_split(q, K, V, scale, split_tokens, tile):
    """All heads: split the keys into runs of `split_tokens`, run the online
    recurrence in each, then merge the runs' (m, l, O) with the same rule."""
    num_q_heads, head_dim = q.shape
    S, num_kv_heads, _ = K.shape
    group = num_q_heads // num_kv_heads
    out = np.zeros((num_q_heads, head_dim), dtype=np.float64)
    if S == 0:
        return out
    for h in range(num_q_heads):
        g = h // group
        m, l, O = -math.inf, 0.0, np.zeros(head_dim, dtype=np.float64)
        for start in range(0, S, split_tokens):
            part = attend_online(q[h], K[start:start + split_tokens, g],
                                 V[start:start + split_tokens, g], scale, tile)
            m, l, O = _merge(m, l, O, *part)
        out[h] = O / l
    return out
