"""Whole-step drivers over the library's entry points (orchestration only).

Each function issues the library calls one step of a paged-KV workload makes, in
the order the pages give, on one stream:

* decode_step    -- per layer: write the batch's new K/V into their slots, then
                    decode every sequence through its block table ("KV Cache
                    Management", "The PagedAttention virtual memory model";
                    "PagedAttention", "The real cache"); by default both in
                    one fused launch.
* cow_copy       -- the block copies copy-on-write asks for before a write into a
                    shared block ("Zero-copy deliberation via copy-on-write
                    branching").
* offload / restore -- frames moved out to pinned host memory through a staging
                    buffer and back into other blocks ("Asynchronous paged
                    swapping").

No arithmetic of the method happens here: every byte is moved or computed by
libpa's kernels.
"""

from __future__ import annotations

from typing import Callable, Optional, Sequence

import torch

from . import api
from .api import Geometry


def decode_step(geom: Geometry, k_pool, v_pool, q_all, k_new_all, v_new_all, slots, tables, lens,
                max_context_len: int, out_all, workspace, layers: Optional[Sequence[int]] = None,
                blocks_per_split: int = 0, kernel: str = "auto", stream=None,
                around_decode: Optional[Callable[[int, bool], None]] = None, kv_reuse: bool = False,
                fused: bool = True, merge: bool = False, waves_per_group: int = 0,
                host_lens=None):
    """One decode step: for each layer, append the new tokens, then decode.

    q_all [L, n, H_q, d]; k_new_all / v_new_all [L, n_tok, H_kv, d]; slots int64
    [n_tok]; tables int32 [n, max_blocks]; lens int32 [n]; out_all [L, n, H_q, d].
    fused=True (one new token per sequence, at position lens[i] - 1 of its table,
    n_tok == n) does both in one launch per layer and ignores `slots`;
    fused=False issues the slot-mapped append and the decode separately.
    merge=True merges the splits inside the decode launch (zeroed workspace);
    host_lens (host copy of lens) lets the library plan ragged batches.
    around_decode(layer, before) is called just before and after each layer's
    decode call (host side, e.g. to switch per-kernel timing on and off).
    """
    for layer in (range(geom.num_layers) if layers is None else layers):
        if not fused:
            api.append_kv(geom, k_pool, v_pool, layer, k_new_all[layer], v_new_all[layer], slots,
                          stream=stream)
        if around_decode is not None:
            around_decode(layer, True)
        if fused:
            api.decode_append(geom, k_pool, v_pool, layer, q_all[layer], k_new_all[layer],
                              v_new_all[layer], out_all[layer], tables, lens, max_context_len,
                              workspace=workspace, blocks_per_split=blocks_per_split,
                              kernel=kernel, stream=stream, kv_reuse=kv_reuse, merge=merge,
                              waves_per_group=waves_per_group, host_lens=host_lens)
        else:
            api.decode(geom, k_pool, v_pool, layer, q_all[layer], out_all[layer], tables, lens,
                       max_context_len, workspace=workspace, blocks_per_split=blocks_per_split,
                       kernel=kernel, stream=stream, kv_reuse=kv_reuse, merge=merge,
                              waves_per_group=waves_per_group, host_lens=host_lens)
        if around_decode is not None:
            around_decode(layer, False)


def prepare_decode_step(geom: Geometry, k_pool, v_pool, q_all, k_new_all, v_new_all, tables, lens,
                        max_context_len: int, out_all, workspace,
                        layers: Optional[Sequence[int]] = None, blocks_per_split: int = 0,
                        kernel: str = "auto", stream=None,
                        around_decode: Optional[Callable[[int, bool], None]] = None,
                        kv_reuse: bool = False, merge: bool = False, waves_per_group: int = 0,
                        host_lens=None) -> Callable[[], None]:
    """The fused decode step of decode_step (one new token per sequence, at
    position lens[i] - 1) with each layer's call checked and marshalled once:
    returns step(), which runs every layer's decode_append on the same buffers."""
    calls = [(layer, api.DecodeAppendCall(geom, k_pool, v_pool, layer, q_all[layer],
                                          k_new_all[layer], v_new_all[layer], out_all[layer],
                                          tables, lens, max_context_len, workspace=workspace,
                                          blocks_per_split=blocks_per_split, kernel=kernel,
                                          stream=stream, kv_reuse=kv_reuse, merge=merge,
                                          waves_per_group=waves_per_group, host_lens=host_lens))
             for layer in (range(geom.num_layers) if layers is None else layers)]

    def step():
        for layer, call in calls:
            if around_decode is not None:
                around_decode(layer, True)
            call()
            if around_decode is not None:
                around_decode(layer, False)
    return step


def cow_copy(geom: Geometry, k_pool, v_pool, pairs, device, stream=None):
    """Run the (src, dst) block copies a copy-on-write reservation returned."""
    if not pairs:
        return
    src = torch.tensor([p[0] for p in pairs], dtype=torch.int32, device=device)
    dst = torch.tensor([p[1] for p in pairs], dtype=torch.int32, device=device)
    api.copy_blocks(geom, k_pool, v_pool, src, dst, stream=stream)


def offload(geom: Geometry, k_pool, v_pool, block_ids: torch.Tensor, host_frames: torch.Tensor,
            staging: torch.Tensor, chunk_blocks: int, stream=None, on_chunk=None):
    """Gather the listed blocks chunk by chunk into `staging` and copy each chunk
    to `host_frames` (pinned, len(block_ids) * bytes_per_block bytes, uint8).
    The caller synchronises the stream before reusing the blocks."""
    per = api.bytes_per_block(geom)
    n = block_ids.numel()
    for start in range(0, n, chunk_blocks):
        m = min(chunk_blocks, n - start)
        api.gather_blocks(geom, k_pool, v_pool, block_ids[start:start + m], staging, stream=stream)
        if on_chunk is not None:
            on_chunk("gather", start, m)
        api.copy_to_host(host_frames[start * per:(start + m) * per], staging, m * per, stream=stream)
        if on_chunk is not None:
            on_chunk("d2h", start, m)


def restore(geom: Geometry, k_pool, v_pool, block_ids: torch.Tensor, host_frames: torch.Tensor,
            staging: torch.Tensor, chunk_blocks: int, stream=None, on_chunk=None):
    """Inverse of offload: copy each chunk of frames back to `staging` and scatter
    it into the listed (new) blocks."""
    per = api.bytes_per_block(geom)
    n = block_ids.numel()
    for start in range(0, n, chunk_blocks):
        m = min(chunk_blocks, n - start)
        api.copy_to_device(staging, host_frames[start * per:(start + m) * per], m * per, stream=stream)
        if on_chunk is not None:
            on_chunk("h2d", start, m)
        api.scatter_blocks(geom, k_pool, v_pool, staging, block_ids[start:start + m], stream=stream)
        if on_chunk is not None:
            on_chunk("scatter", start, m)
