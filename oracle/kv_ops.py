"""Block-level data movement on numpy pools (oracle).

Every operation is a plain element-by-element loop over what it moves, written
from these passages:

* append -- "KV Cache Management", section "The PagedAttention virtual memory
  model": the new token's key and value go to physical block T[l] at offset o;
  "PagedAttention" (Inference book), section "The real cache": each new key and
  value is written to the sequence's block and offset.
* copy   -- "KV Cache Management", section "Zero-copy deliberation via
  copy-on-write branching": copy the B tokens of the shared block into the new
  one (the whole block: every layer, K and V, all B slots).
* gather / scatter -- "KV Cache Management", section "Asynchronous paged
  swapping": a list of frames of bytes_per_block each is moved as a unit.

Slots follow the library's convention: a negative slot means "skip this token".
All functions mutate copies and return them (inputs are left untouched).
"""

from __future__ import annotations

import numpy as np

from . import layout


def append_kv(k_pool, v_pool, layer, k_new, v_new, slots, block_size):
    """Write k_new[j], v_new[j] (each [H_kv, d]) at slot slots[j] of one layer."""
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    num_kv_heads = k_new.shape[1]
    for j, s in enumerate(np.asarray(slots, dtype=np.int64)):
        if s < 0:
            continue
        phys, off = int(s) // block_size, int(s) % block_size
        for h in range(num_kv_heads):
            layout.write_k(k_out, layer, phys, h, off, k_new[j, h])
            layout.write_v(v_out, layer, phys, h, off, v_new[j, h])
    return k_out, v_out


def copy_blocks(k_pool, v_pool, src, dst):
    """pool[:, dst[k]] <- pool[:, src[k]] for every pair, every layer, K and V."""
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    for s, d in zip(np.asarray(src).tolist(), np.asarray(dst).tolist()):
        for layer in range(k_pool.shape[0]):
            k_out[layer, d] = k_pool[layer, s]
            v_out[layer, d] = v_pool[layer, s]
    return k_out, v_out


def gather_blocks(k_pool, v_pool, block_ids):
    """Staging [n, L, 2, run]: block i's K run then V run for every layer."""
    num_layers = k_pool.shape[0]
    run = int(np.prod(k_pool.shape[2:]))
    staging = np.empty((len(block_ids), num_layers, 2, run), dtype=k_pool.dtype)
    for i, p in enumerate(np.asarray(block_ids).tolist()):
        for layer in range(num_layers):
            staging[i, layer, 0] = k_pool[layer, p].reshape(-1)
            staging[i, layer, 1] = v_pool[layer, p].reshape(-1)
    return staging


def scatter_blocks(k_pool, v_pool, staging, block_ids):
    """Inverse of gather_blocks: pool[:, ids[i]] <- staging[i]."""
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    kshape = k_pool.shape[2:]
    vshape = v_pool.shape[2:]
    for i, p in enumerate(np.asarray(block_ids).tolist()):
        for layer in range(k_pool.shape[0]):
            k_out[layer, p] = staging[i, layer, 0].reshape(kshape)
            v_out[layer, p] = staging[i, layer, 1].reshape(vshape)
    return k_out, v_out


def slot_mapping(tables, positions, block_size):
    """Slot of each (sequence, position) pair: T[t // B] * B + t mod B."""
    return np.array([layout.slot_of(tables[i], int(t), block_size)
                     for i, t in enumerate(positions)], dtype=np.int64)
