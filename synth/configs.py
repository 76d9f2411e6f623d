"""The workloads, as geometry plus a recipe for their random parts.

Shapes follow the workloads the pages describe:

* ``gpt2_fp32``   -- the GPT-2 paged cache of "PagedAttention" (Inference book,
  ch. 14, section "The real cache"): 12 layers, 12 heads, head dim 64, fp32.
* ``chat_ragged`` -- the chat-like log-normal length mix of the same chapter
  (section "Where contiguous allocation wastes memory", workload table: median
  lengths, maximum context 1,024, 16-token blocks) on a 32-layer GQA model.
* ``gqa70b_32k``  -- the 70B grouped-query model of "KV Cache Management"
  (section "From Context Tokens to KV State", Napkin Math 0.1): 80 layers,
  8 KV heads of dim 128, 16-bit storage, 64 query heads (Napkin Math 0.3),
  at a 32,768-token context.
* ``fork_cow``    -- branches forked from one shared prefix whose last block is
  partly filled ("KV Cache Management", section "Zero-copy deliberation via
  copy-on-write branching"; "PagedAttention", section "Sharing and copy-on-write").
* ``offload``     -- the 70B geometry at 131,072 tokens with half of each
  trajectory's blocks moved to a host tier and back ("KV Cache Management",
  section "Asynchronous paged swapping").
* ``prefill_chunks`` -- the 70B geometry prefilling 2,048-token prompts in
  512-token chunks ("KV Cache Management", section "Chunked prefill
  mechanics", Figure 8): the batch holds chunk k = 1..4 of different prompts,
  i.e. histories of 0, 512, 1,024 and 1,536 cached tokens.
* ``gqa70b_32k_fp8`` -- ``gqa70b_32k`` with b_elem = 1 ("KV Cache Management",
  section "From Context Tokens to KV State", Eq. (1): one byte for FP8).
* ``offload_overlap`` -- the ``gqa70b_32k`` decode batch keeps stepping while one
  more 16,384-token trajectory (the 70B example of "KV Cache Management",
  section "Retain, Evict, Recompute, or Offload", Figure 10) moves to pinned
  host memory and back on a copy stream of its own (same page, section
  "Asynchronous paged swapping").
* ``prefix_reuse`` -- requests to the 70B geometry that share a 4,096-token
  system prompt and bring 32 novel tokens each ("KV Cache Management", section
  "Prefix Caching Across Turns", Napkin Math 0.4): the radix prefix cache
  resolves the prompt, only the novel tokens are prefilled over the cached
  history, and the finished requests' blocks are indexed and evicted leaf-first
  (LRU) under a 384-block budget (the 256-block prompt plus room for four
  batches), so that every step from the fourth on evicts.
* ``prefill_chunks_fp8`` -- ``prefill_chunks`` on one-byte E4M3 pools.
* ``spec_verify`` -- the ``gqa70b_32k`` batch taking 4 new tokens per sequence in
  one multi-query pass (a short chunk over a 32,764-token history: "Chunked
  prefill mechanics" with a chunk of 4), as when draft tokens are checked.
* ``spec_verify_fp8`` -- ``spec_verify`` on one-byte E4M3 pools.

Seeds: workload k (1-based, in the order above) uses master seed 8300 + k.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional


@dataclass(frozen=True)
class Workload:
    name: str
    index: int                 # 1-based position in CONFIGS
    num_layers: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str                 # "f32", "bf16" or "fp8" (one-byte pool, bf16 queries)
    num_blocks: int            # physical blocks in the pool
    num_seqs: int
    # length recipe (interpreted by synth.gen.context_lengths)
    length_kind: str           # "uniform", "lognormal", "fixed", "fork"
    length_min: int = 1
    length_max: int = 1
    length_median: float = 0.0
    length_sigma: float = 0.0
    # fork workload
    prefix_len: int = 0
    suffix_min: int = 0
    suffix_max: int = 0
    # offload workload
    offload_fraction: float = 0.0
    offload_chunk_blocks: int = 0
    # chunked-prefill workload: prompt length (length_max) cut into chunks
    chunk_len: int = 0
    # overlapped-offload workload: tokens of the trajectory that migrates
    mover_len: int = 0
    notes: str = ""
    extra: Dict[str, float] = field(default_factory=dict)

    @property
    def seed(self) -> int:
        return 8300 + self.index

    @property
    def elem_bytes(self) -> int:
        return {"f32": 4, "bf16": 2, "fp8": 1}[self.dtype]

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


CONFIGS = [
    Workload(
        name="gpt2_fp32", index=1, num_layers=12, num_q_heads=12, num_kv_heads=12,
        head_dim=64, block_size=16, dtype="f32", num_blocks=1024, num_seqs=8,
        length_kind="uniform", length_min=1, length_max=1024,
        notes="GPT-2-small geometry, MHA, fp32; attended lengths uniform in [1, 1024]",
    ),
    Workload(
        name="chat_ragged", index=2, num_layers=32, num_q_heads=32, num_kv_heads=8,
        head_dim=128, block_size=16, dtype="bf16", num_blocks=8192, num_seqs=256,
        # sigma = sqrt(2 ln(371/300)) makes the uncapped log-normal mean equal the
        # chat-like mean final length (371) for the stated median (300).
        length_kind="lognormal", length_min=1, length_max=1024, length_median=300.0,
        length_sigma=0.6520,
        notes="chat-like ragged batch; log-normal lengths, median 300, capped at 1024",
    ),
    Workload(
        name="gqa70b_32k", index=3, num_layers=80, num_q_heads=64, num_kv_heads=8,
        head_dim=128, block_size=16, dtype="bf16", num_blocks=32768, num_seqs=16,
        length_kind="fixed", length_min=32768, length_max=32768,
        notes="70B GQA geometry (327,680 B/token), 16 x 32,768-token trajectories",
    ),
    Workload(
        name="fork_cow", index=4, num_layers=32, num_q_heads=32, num_kv_heads=8,
        head_dim=128, block_size=16, dtype="bf16", num_blocks=8192, num_seqs=64,
        length_kind="fork", prefix_len=16392, suffix_min=256, suffix_max=2048,
        notes="64 branches of one 16,392-token prefix (tail block holds 8 tokens)",
    ),
    Workload(
        name="offload", index=5, num_layers=80, num_q_heads=64, num_kv_heads=8,
        head_dim=128, block_size=16, dtype="bf16", num_blocks=32768, num_seqs=4,
        length_kind="fixed", length_min=131072, length_max=131072,
        offload_fraction=0.5, offload_chunk_blocks=512,
        notes="4 x 131,072-token trajectories; half of each one's blocks offloaded",
    ),
    Workload(
        name="prefill_chunks", index=6, num_layers=80, num_q_heads=64, num_kv_heads=8,
        head_dim=128, block_size=16, dtype="bf16", num_blocks=4096, num_seqs=16,
        length_kind="prefill", length_min=2048, length_max=2048, chunk_len=512,
        notes="16 prompts of 2,048 tokens in 512-token chunks; sequence i runs chunk (i mod 4) + 1",
    ),
    Workload(
        name="offload_overlap", index=7, num_layers=80, num_q_heads=64, num_kv_heads=8,
        head_dim=128, block_size=16, dtype="bf16", num_blocks=32768 + 1024, num_seqs=16,
        length_kind="fixed", length_min=32768, length_max=32768, mover_len=16384,
        offload_chunk_blocks=64,
        notes="gqa70b_32k decode batch + one 16,384-token trajectory swapped out and back",
    ),
    Workload(
        name="gqa70b_32k_fp8", index=8, num_layers=80, num_q_heads=64, num_kv_heads=8,
        head_dim=128, block_size=16, dtype="fp8", num_blocks=32768, num_seqs=16,
        length_kind="fixed", length_min=32768, length_max=32768,
        notes="gqa70b_32k with one-byte E4M3 storage (per-token, per-head scales)",
    ),
    Workload(
        name="prefix_reuse", index=9, num_layers=80, num_q_heads=64, num_kv_heads=8,
        head_dim=128, block_size=16, dtype="bf16", num_blocks=384 + 16 * 258 + 32, num_seqs=16,
        length_kind="prefix", prefix_len=4096, chunk_len=32,
        notes="16 requests per step: 4,096 cached system tokens + 32 novel tokens each; the "
              "prefix cache runs in the first 384 blocks, the no-reuse comparison in the rest",
        extra={"budget_blocks": 384, "watermark_blocks": 32},
    ),
    Workload(
        name="prefill_chunks_fp8", index=10, num_layers=80, num_q_heads=64, num_kv_heads=8,
        head_dim=128, block_size=16, dtype="fp8", num_blocks=4096, num_seqs=16,
        length_kind="prefill", length_min=2048, length_max=2048, chunk_len=512,
        notes="prefill_chunks on one-byte E4M3 pools (the chunks are quantized as they are written)",
    ),
    Workload(
        name="spec_verify", index=11, num_layers=80, num_q_heads=64, num_kv_heads=8,
        head_dim=128, block_size=16, dtype="bf16", num_blocks=32768, num_seqs=16,
        length_kind="verify", length_min=32768, length_max=32768, chunk_len=4,
        notes="the gqa70b_32k batch checking 4 new tokens per sequence in one pass (32,764 cached)",
    ),
    Workload(
        name="spec_verify_fp8", index=12, num_layers=80, num_q_heads=64, num_kv_heads=8,
        head_dim=128, block_size=16, dtype="fp8", num_blocks=32768, num_seqs=16,
        length_kind="verify", length_min=32768, length_max=32768, chunk_len=4,
        notes="spec_verify on one-byte E4M3 pools",
    ),
]

_BY_NAME = {c.name: c for c in CONFIGS}


def get_config(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        return CONFIGS[name_or_index - 1]
    return _BY_NAME[name_or_index]


def scaled(cfg: Workload, *, num_layers: Optional[int] = None, num_seqs: Optional[int] = None,
           num_blocks: Optional[int] = None, length_max: Optional[int] = None,
           prefix_len: Optional[int] = None, suffix_max: Optional[int] = None,
           suffix_min: Optional[int] = None) -> Workload:
    """A smaller copy of a workload with the same structure (for CPU-sized tests)."""
    d = dict(cfg.__dict__)
    if num_layers is not None:
        d["num_layers"] = num_layers
    if num_seqs is not None:
        d["num_seqs"] = num_seqs
    if num_blocks is not None:
        d["num_blocks"] = num_blocks
    if length_max is not None:
        d["length_max"] = length_max
        if cfg.length_kind == "fixed":
            d["length_min"] = length_max
    if prefix_len is not None:
        d["prefix_len"] = prefix_len
    if suffix_max is not None:
        d["suffix_max"] = suffix_max
    if suffix_min is not None:
        d["suffix_min"] = suffix_min
    return Workload(**d)
