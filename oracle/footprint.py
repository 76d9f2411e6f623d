"""KV footprint arithmetic (oracle).

Sources:
* "KV Cache Management", section "From Context Tokens to KV State", Eq. (1):
  bytes per token = 2 * layers * kv_heads * head_dim * bytes_per_element.
* "KV Cache Management", section "The PagedAttention virtual memory model":
  block bytes = 2 * L * H_kv * B * d * b, and blocks for a prompt = ceil(S / B).
* "KV Cache Management", section "Quantitative trade-offs in block sizing":
  unused tail slots (B - S mod B) mod B, expected value (B - 1) / 2.
* "EfficientAgent ...", section "KV footprint and hardware balance", Eq. (1):
  per-rank bytes per token = 2 * L * d * s * max(1, ceil(H_kv / TP)).
"""

from __future__ import annotations

import math


def bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, elem_bytes: int,
                    tp: int = 1) -> int:
    """m_token on one rank. With tp == 1 this is Eq. (1) of "KV Cache Management".

    With tp > 1 each rank holds ceil(H_kv / TP) heads, and at least one (heads are
    replicated when there are fewer KV heads than ranks), per the EfficientAgent
    per-rank footprint equation.
    """
    if tp < 1:
        raise ValueError("tp must be >= 1")
    heads_on_rank = max(1, -(-num_kv_heads // tp))
    return 2 * num_layers * heads_on_rank * head_dim * elem_bytes


def bytes_per_block(num_layers: int, num_kv_heads: int, head_dim: int, elem_bytes: int,
                    block_size: int) -> int:
    """M_block = 2 * L * H_kv * B * d * b: one block holds B tokens of every layer and head."""
    return 2 * num_layers * num_kv_heads * block_size * head_dim * elem_bytes


def blocks_for_tokens(num_tokens: int, block_size: int) -> int:
    """N_blocks = ceil(S / B)."""
    if num_tokens < 0 or block_size < 1:
        raise ValueError("bad arguments")
    return math.ceil(num_tokens / block_size) if num_tokens else 0


def tail_slots(num_tokens: int, block_size: int) -> int:
    """Delta_tail = (B - (S mod B)) mod B: unused slots in the last block."""
    return (block_size - (num_tokens % block_size)) % block_size


def expected_tail_slots(block_size: int) -> float:
    """E[Delta_tail] = (B - 1) / 2 when S mod B is uniform over {0, ..., B-1}."""
    return (block_size - 1) / 2.0


def tail_waste_fraction(block_size: int, mean_length: float) -> float:
    """Expected waste fraction ~ (b - 1) / (2 * mean length) ("PagedAttention",
    section "What it costs in the last block")."""
    return (block_size - 1) / (2.0 * mean_length)
