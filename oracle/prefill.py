"""Chunked-prefill attention over a paged pool, computed the plain way (oracle).

Test infrastructure: only the tests, the smoke check and the benchmark's
CPU-baseline / parity leg use this module; the library never does.

Definition followed: "KV Cache Management", section "Chunked prefill mechanics".
A prompt is cut into chunks; chunk k's queries Q_k attend over the keys and
values of all earlier chunks, already held in paged blocks, concatenated with
the chunk's own projections:

    K_<=k = [K_cached || K_k],   V_<=k = [V_cached || V_k]
    O_k   = Softmax(Q_k K_<=k^T / sqrt(d_head) + M_k) V_<=k

M_k lets every query see every cached token and, inside the chunk, only tokens
at or before its own position (lower-triangular causal mask). Afterwards K_k and
V_k are written into the sequence's paged blocks.

Batch convention (the library's): chunk i has ctx_lens[i] tokens already cached
(positions 0 .. c_i - 1, read through its block table) and q_len_i new tokens at
positions c_i .. c_i + q_len_i - 1, stored as rows q_start[i] .. q_start[i+1] - 1
of the packed arrays q [n_tok, H_q, d], k_new / v_new [n_tok, H_kv, d]. Its block
table must already cover c_i + q_len_i tokens (the blocks the chunk is written
into). Query heads map to KV heads in contiguous groups, as for decode.

Everything is float64 on exactly widened inputs; the history comes from the pool
as it is before the chunk is written, the chunk's own keys and values from the
inputs, exactly as the equations concatenate them.
"""

from __future__ import annotations

import numpy as np

from . import attention, kv_ops, layout


def chunk_bounds(q_start, i):
    return int(q_start[i]), int(q_start[i + 1])


def chunk_slots(tables, q_start, ctx_lens, block_size):
    """Slot (block * B + offset) of every new token: position p of chunk i lives in
    physical block tables[i][p // B] at offset p mod B ("The PagedAttention virtual
    memory model")."""
    n_tok = int(q_start[-1])
    slots = np.full(n_tok, -1, dtype=np.int64)
    for i in range(len(ctx_lens)):
        a, b = chunk_bounds(q_start, i)
        for j in range(a, b):
            p = int(ctx_lens[i]) + (j - a)
            slots[j] = int(tables[i][p // block_size]) * block_size + p % block_size
    return slots


def chunk_attention(q_rows, k_rows, v_rows, K_hist, V_hist, scale):
    """Outputs [q_len, H_q, d] of one chunk: token t (0-based inside the chunk)
    attends over the c cached tokens and chunk tokens 0 .. t."""
    K_all = np.concatenate([K_hist, k_rows], axis=0)
    V_all = np.concatenate([V_hist, v_rows], axis=0)
    c = K_hist.shape[0]
    out = np.zeros(q_rows.shape, dtype=np.float64)
    for t in range(q_rows.shape[0]):
        visible = c + t + 1
        out[t] = attention.attend(q_rows[t], K_all[:visible], V_all[:visible], scale)
    return out


def paged_prefill(q, k_new, v_new, k_pool, v_pool, layer, tables, q_start, ctx_lens, block_size,
                  dtype, scale=None, chunks=None):
    """Pools after the chunks are written, and the float64 outputs [n_tok, H_q, d]
    (rows of chunks not listed in `chunks` stay zero)."""
    head_dim = q.shape[2]
    if scale is None or scale == 0.0:
        scale = attention.default_scale(head_dim)
    qf = layout.widen(q, dtype)
    kf = layout.widen(k_new, dtype)
    vf = layout.widen(v_new, dtype)
    out = np.zeros(qf.shape, dtype=np.float64)
    idx = range(len(ctx_lens)) if chunks is None else chunks
    for i in idx:
        a, b = chunk_bounds(q_start, i)
        K_hist, V_hist = attention.rebuild_sequence(k_pool, v_pool, layer, tables[i],
                                                    int(ctx_lens[i]), block_size, dtype)
        out[a:b] = chunk_attention(qf[a:b], kf[a:b], vf[a:b], K_hist, V_hist, scale)
    slots = chunk_slots(tables, q_start, ctx_lens, block_size)
    k_after, v_after = kv_ops.append_kv(k_pool, v_pool, layer, k_new, v_new, slots, block_size)
    return k_after, v_after, out
