"""Seeded random draws for the decode workloads.

Every function takes a Workload (or a seed) and returns plain numpy arrays. Named
sub-streams come from ``numpy.random.SeedSequence(cfg.seed).spawn``, one per
purpose, so adding a draw for one purpose never shifts another.

Floating values are standard normal. bf16 values are produced as raw 16-bit
patterns (the top half of a float32 normal draw, rounded to nearest even), so
both sides of a comparison receive identical bits.
"""

from __future__ import annotations

import numpy as np

from .configs import Workload

# Sub-stream indices (fixed forever: changing one changes every input).
_LENGTHS, _FREE_ORDER, _SUFFIX, _OFFLOAD, _VALUES, _REALLOC, _TOKENS = range(7)


def _stream(seed: int, which: int) -> np.random.Generator:
    children = np.random.SeedSequence(seed).spawn(8)
    return np.random.default_rng(children[which])


def context_lengths(cfg: Workload) -> np.ndarray:
    """Attended length of every sequence in the decode step (int64, >= 1).

    The attended length counts the token appended in the same step.
    """
    rng = _stream(cfg.seed, _LENGTHS)
    n = cfg.num_seqs
    if cfg.length_kind == "uniform":
        return rng.integers(cfg.length_min, cfg.length_max + 1, size=n).astype(np.int64)
    if cfg.length_kind == "lognormal":
        raw = rng.lognormal(mean=np.log(cfg.length_median), sigma=cfg.length_sigma, size=n)
        return np.clip(np.rint(raw), cfg.length_min, cfg.length_max).astype(np.int64)
    if cfg.length_kind == "fixed":
        return np.full(n, cfg.length_min, dtype=np.int64)
    if cfg.length_kind == "fork":
        return cfg.prefix_len + suffix_lengths(cfg)
    if cfg.length_kind in ("prefill", "verify"):
        return prefill_histories(cfg) + cfg.chunk_len
    if cfg.length_kind == "prefix":
        return np.full(n, cfg.prefix_len + cfg.chunk_len, dtype=np.int64)
    raise ValueError(cfg.length_kind)


def prefill_histories(cfg: Workload) -> np.ndarray:
    """Cached tokens before each sequence's chunk: sequence i runs chunk
    (i mod K) + 1 of a prompt of length_max tokens cut into K chunks; for the
    verify workload every sequence holds length_max - chunk_len tokens."""
    if cfg.length_kind == "verify":
        return np.full(cfg.num_seqs, cfg.length_max - cfg.chunk_len, dtype=np.int64)
    k = cfg.length_max // cfg.chunk_len
    return (np.arange(cfg.num_seqs) % k * cfg.chunk_len).astype(np.int64)


def suffix_lengths(cfg: Workload) -> np.ndarray:
    """Private suffix length of each forked branch, uniform in [suffix_min, suffix_max]."""
    rng = _stream(cfg.seed, _SUFFIX)
    return rng.integers(cfg.suffix_min, cfg.suffix_max + 1, size=cfg.num_seqs).astype(np.int64)


def free_order(cfg: Workload) -> np.ndarray:
    """Order in which the pool's physical block ids are handed out (a permutation)."""
    rng = _stream(cfg.seed, _FREE_ORDER)
    return rng.permutation(cfg.num_blocks).astype(np.int32)


def realloc_shuffle(cfg: Workload, n: int, round_index: int = 0) -> np.ndarray:
    """A permutation of n items, used to reshuffle free blocks before a swap-in.
    Round k > 0 (e.g. the k-th pass of a multi-pass round trip) draws from its
    own child of the same sub-stream; round 0 is the sub-stream itself."""
    if round_index == 0:
        rng = _stream(cfg.seed, _REALLOC)
    else:
        child = np.random.SeedSequence(cfg.seed).spawn(8)[_REALLOC].spawn(round_index + 1)[round_index]
        rng = np.random.default_rng(child)
    return rng.permutation(n).astype(np.int64)


def offload_choice(cfg: Workload, blocks_per_seq: int) -> np.ndarray:
    """For each sequence, the sorted logical block indices picked for offload.

    Returns an int64 array [num_seqs, k] with k = round(fraction * blocks_per_seq).
    """
    rng = _stream(cfg.seed, _OFFLOAD)
    k = int(round(cfg.offload_fraction * blocks_per_seq))
    out = np.empty((cfg.num_seqs, k), dtype=np.int64)
    for i in range(cfg.num_seqs):
        out[i] = np.sort(rng.choice(blocks_per_seq, size=k, replace=False))
    return out


def permutation(seed: int, n: int) -> np.ndarray:
    return np.random.default_rng(seed).permutation(n).astype(np.int32)


def normal_f32(seed: int, shape) -> np.ndarray:
    """Standard-normal float32 array."""
    return np.random.default_rng(seed).standard_normal(size=shape, dtype=np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def normal_values(seed: int, shape, dtype: str) -> np.ndarray:
    """Standard-normal values in storage form: float32 array, or uint16 bf16 bits."""
    x = normal_f32(seed, shape)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def value_seed(cfg: Workload, tag: int) -> int:
    """A derived integer seed for one named value tensor of a workload."""
    ss = np.random.SeedSequence([cfg.seed, _VALUES, int(tag)])
    return int(ss.generate_state(1, dtype=np.uint32)[0])


# Tags for value tensors (stable).
TAG_Q, TAG_KNEW, TAG_VNEW, TAG_KPOOL, TAG_VPOOL, TAG_KHIST, TAG_VHIST = range(7)


def prefix_reuse_tokens(cfg: Workload, n_steps: int, vocab: int = 32000):
    """Token ids of the prefix-reuse workload: one shared system prompt of
    cfg.prefix_len tokens and, for each of n_steps steps, cfg.num_seqs requests of
    cfg.chunk_len novel tokens (int32 arrays; the prompt of a request is the
    system prompt followed by its novel tokens)."""
    rng = _stream(cfg.seed, _TOKENS)
    system = rng.integers(0, vocab, cfg.prefix_len).astype(np.int32)
    novel = rng.integers(0, vocab, (n_steps, cfg.num_seqs, cfg.chunk_len)).astype(np.int32)
    return system, novel
