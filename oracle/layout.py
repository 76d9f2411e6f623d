"""How the oracle reads and writes a paged KV pool (oracle).

Address translation follows "KV Cache Management", section "The PagedAttention
virtual memory model": token t of a sequence lives in logical block l = t // B at
offset o = t mod B, and the sequence's block table T maps l to a physical block
id p = T[l] in [0, N).

The in-memory arrangement of a pool is a documented property of the library's
interface, restated here independently (this module shares no code with the
library):

* K pool, shape [L, N, H_kv, d/W, B, W] with W = 32 when 32 divides d and
  W = d otherwise: element (layer, p, head, o, j) sits at chunk j // W, slot o,
  position j % W (for W = d this is simply [L, N, H_kv, B, d]).
* V pool, shape [L, N, H_kv, d, B]: element (layer, p, head, j, o).
  Within one (layer, block, head) both are one contiguous run of B*d elements;
  K keeps each token's values together within 32-wide dimension chunks, V keeps
  each dimension's B values together.
* Staging buffer for gather/scatter: for the i-th listed block, M_block bytes
  laid out as [L][2][run], where index 0 holds the block's K run of that layer
  and index 1 its V run, each run copied as stored in the pool. This is the
  "bytes_per_block" frame of "KV Cache Management", section "Asynchronous paged
  swapping".

Pools are numpy arrays in storage form: float32, or uint16 holding bf16 bits.
"""

from __future__ import annotations

import numpy as np


def k_chunk(head_dim: int) -> int:
    """Width W of the K dimension chunks."""
    return 32 if head_dim % 32 == 0 else head_dim


def k_pool_shape(num_layers, num_blocks, num_kv_heads, block_size, head_dim):
    W = k_chunk(head_dim)
    return (num_layers, num_blocks, num_kv_heads, head_dim // W, block_size, W)


def v_pool_shape(num_layers, num_blocks, num_kv_heads, block_size, head_dim):
    return (num_layers, num_blocks, num_kv_heads, head_dim, block_size)


def logical_block(t: int, block_size: int) -> int:
    """l = floor(t / B)."""
    return t // block_size


def block_offset(t: int, block_size: int) -> int:
    """o = t mod B."""
    return t % block_size


def slot_of(table, t: int, block_size: int) -> int:
    """Flat write address of token t: T[l] * B + o."""
    return int(table[logical_block(t, block_size)]) * block_size + block_offset(t, block_size)


def read_k(k_pool: np.ndarray, layer: int, phys: int, head: int, offset: int) -> np.ndarray:
    """The d values of K stored for (layer, block phys, head, slot offset)."""
    return k_pool[layer, phys, head, :, offset, :].reshape(-1)


def read_v(v_pool: np.ndarray, layer: int, phys: int, head: int, offset: int) -> np.ndarray:
    """The d values of V stored for (layer, block phys, head, slot offset)."""
    return v_pool[layer, phys, head, :, offset]


def read_k_tile(k_pool: np.ndarray, layer: int, phys: int, head: int) -> np.ndarray:
    """K of all B slots of one (layer, block, head), as [B, d] (slot-major)."""
    chunks = k_pool[layer, phys, head]                 # [d/W, B, W]
    return np.concatenate([chunks[c] for c in range(chunks.shape[0])], axis=1)


def read_v_tile(v_pool: np.ndarray, layer: int, phys: int, head: int) -> np.ndarray:
    """V of all B slots of one (layer, block, head), as [B, d] (slot-major)."""
    return v_pool[layer, phys, head, :, :].T


def write_k(k_pool: np.ndarray, layer: int, phys: int, head: int, offset: int, values) -> None:
    nchunk, W = k_pool.shape[3], k_pool.shape[5]
    k_pool[layer, phys, head, :, offset, :] = np.asarray(values).reshape(nchunk, W)


def write_v(v_pool: np.ndarray, layer: int, phys: int, head: int, offset: int, values) -> None:
    v_pool[layer, phys, head, :, offset] = values


def widen(storage: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored elements (bf16 bits become the float32 with
    those top 16 bits, which float64 represents exactly)."""
    if dtype == "f32":
        return np.asarray(storage, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(storage, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)
