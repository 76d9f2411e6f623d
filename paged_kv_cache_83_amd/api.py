"""Python binding of libpa: argument marshalling only.

Every function here checks that tensors are where and what the C interface
expects (device, dtype, contiguity, size) -- the C side only sees raw pointers
and cannot -- and then calls the library. No arithmetic of the method happens
here; torch is used for device memory and streams only.
"""

from __future__ import annotations

import ctypes as C
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np
import torch

from . import _lib
from ._lib import check

_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}
_CODE = {"f32": _lib.PA_F32, "bf16": _lib.PA_BF16, "fp8": _lib.PA_FP8}


@dataclass(frozen=True)
class Geometry:
    num_layers: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    dtype: str  # "f32", "bf16" or "fp8" (E4M3 codes with per-(token, head) scales)

    def c(self) -> _lib.pa_geom:
        return _lib.pa_geom(self.num_layers, self.num_kv_heads, self.head_dim, self.block_size,
                            self.num_blocks, _CODE[self.dtype])

    @property
    def torch_dtype(self) -> torch.dtype:
        """Storage type of the pools (uint8 bytes for fp8)."""
        return _TORCH[self.dtype]

    @property
    def io_dtype(self) -> torch.dtype:
        """Type of queries, outputs and new K/V rows: bf16 for fp8 pools."""
        return torch.bfloat16 if self.dtype == "fp8" else _TORCH[self.dtype]

    @property
    def elem_bytes(self) -> int:
        return {"f32": 4, "bf16": 2, "fp8": 1}[self.dtype]

    @property
    def tile_bytes(self) -> int:
        """Bytes of one (layer, block, head) tile of K (or V): B*d elements, and
        for fp8 the B scale bytes after them."""
        extra = self.block_size if self.dtype == "fp8" else 0
        return self.block_size * self.head_dim * self.elem_bytes + extra

    @property
    def k_chunk(self) -> int:
        """Width W of K's dimension chunks (32 when it divides head_dim, else head_dim)."""
        return 32 if self.head_dim % 32 == 0 else self.head_dim

    @property
    def k_pool_shape(self):
        """[L, N, H_kv, d/W, B, W], the K layout include/pa.h documents; fp8 pools
        are bytes [L, N, H_kv, tile_bytes]."""
        if self.dtype == "fp8":
            return (self.num_layers, self.num_blocks, self.num_kv_heads, self.tile_bytes)
        W = self.k_chunk
        return (self.num_layers, self.num_blocks, self.num_kv_heads, self.head_dim // W,
                self.block_size, W)

    @property
    def v_pool_shape(self):
        if self.dtype == "fp8":
            return (self.num_layers, self.num_blocks, self.num_kv_heads, self.tile_bytes)
        return (self.num_layers, self.num_blocks, self.num_kv_heads, self.head_dim, self.block_size)

    @property
    def pool_numel(self) -> int:
        per_tile = self.tile_bytes if self.dtype == "fp8" else self.block_size * self.head_dim
        return self.num_layers * self.num_blocks * self.num_kv_heads * per_tile


def _L():
    return _lib.load()


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream, device) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dev(t: torch.Tensor, what: str, dtype=None, numel=None) -> None:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{what} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{what} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{what} must have {numel} elements, got {t.numel()}")


# --------------------------------------------------------------------- footprint
def bytes_per_token(num_layers, num_kv_heads, head_dim, elem_bytes, tp=1) -> int:
    return int(_L().pa_bytes_per_token(num_layers, num_kv_heads, head_dim, elem_bytes, tp))


def bytes_per_block(geom: Geometry) -> int:
    g = geom.c()
    return int(_L().pa_bytes_per_block(C.byref(g)))


def blocks_for_tokens(tokens: int, block_size: int) -> int:
    return int(_L().pa_blocks_for_tokens(tokens, block_size))


def pool_bytes(geom: Geometry) -> int:
    g = geom.c()
    return int(_L().pa_pool_bytes(C.byref(g)))


def alloc_pools(geom: Geometry, device="cuda"):
    """Uninitialised K and V pools of the documented shapes (torch owns them)."""
    k = torch.empty(geom.k_pool_shape, dtype=geom.torch_dtype, device=device)
    v = torch.empty(geom.v_pool_shape, dtype=geom.torch_dtype, device=device)
    return k, v


# --------------------------------------------------------------------- device ops
def append_kv(geom: Geometry, k_pool, v_pool, layer: int, k_new, v_new, slot_mapping, stream=None):
    n = slot_mapping.numel()
    _dev(k_pool, "k_pool", geom.torch_dtype, geom.pool_numel)
    _dev(v_pool, "v_pool", geom.torch_dtype, geom.pool_numel)
    per = geom.num_kv_heads * geom.head_dim
    _dev(k_new, "k_new", geom.io_dtype, n * per)
    _dev(v_new, "v_new", geom.io_dtype, n * per)
    _dev(slot_mapping, "slot_mapping", torch.int64)
    g = geom.c()
    check(_L().pa_append_kv(C.byref(g), _ptr(k_pool), _ptr(v_pool), layer, _ptr(k_new),
                            _ptr(v_new), _ptr(slot_mapping), n, _stream(stream, k_pool.device)),
          "pa_append_kv")


def _opts(blocks_per_split: int, kernel: int, kv_reuse: bool = False,
          merge: bool = False, waves_per_group: int = 0, host_lens=None) -> _lib.pa_decode_opts:
    """pa_decode_opts; host_lens (a C-contiguous int32 numpy array, kept alive by
    the caller for the call) is the host copy of context_lens."""
    return _lib.pa_decode_opts(int(blocks_per_split), int(kernel), 1 if kv_reuse else 0,
                               1 if merge else 0,
                               None if host_lens is None else host_lens.ctypes.data,
                               int(waves_per_group))


def _host_lens(host_lens, n=None):
    if host_lens is None:
        return None
    a = np.ascontiguousarray(np.asarray(host_lens), dtype=np.int32)
    if a.ndim != 1 or (n is not None and a.size != n):
        raise ValueError("host_lens must be [n_seqs] lengths")
    return a


KERNELS = {"auto": 0, "generic": 1, "mfma": 2, "valu": 3}


def decode_workspace_bytes(geom: Geometry, n_seqs: int, n_q_heads: int, max_context_len: int,
                           blocks_per_split: int = 0, kernel: str = "auto",
                           merge: bool = False, waves_per_group: int = 0, host_lens=None) -> int:
    """Bytes of decode workspace for these sizes and options. With merge=True the
    workspace must be allocated zeroed (torch.zeros) before its first use."""
    g = geom.c()
    hl = _host_lens(host_lens, n_seqs)
    o = _opts(blocks_per_split, KERNELS[kernel], False, merge, waves_per_group, hl)
    return int(_L().pa_decode_workspace_bytes(C.byref(g), n_seqs, n_q_heads, max_context_len,
                                              C.byref(o)))


def _decode_args(geom: Geometry, k_pool, v_pool, q, out, block_tables, context_lens,
                 max_context_len, workspace, o, need_workspace: bool = True):
    _dev(k_pool, "k_pool", geom.torch_dtype, geom.pool_numel)
    _dev(v_pool, "v_pool", geom.torch_dtype, geom.pool_numel)
    if q.dim() != 3 or q.shape[2] != geom.head_dim:
        raise ValueError("q must be [n_seqs, n_q_heads, head_dim]")
    n, hq = int(q.shape[0]), int(q.shape[1])
    _dev(q, "q", geom.io_dtype)
    _dev(out, "out", geom.io_dtype, q.numel())
    if block_tables.dim() != 2 or block_tables.shape[0] != n:
        raise ValueError("block_tables must be [n_seqs, max_blocks]")
    _dev(block_tables, "block_tables", torch.int32)
    _dev(context_lens, "context_lens", torch.int32, n)
    g = geom.c()
    if not need_workspace:
        return g, n, hq, None, 0
    need = int(_L().pa_decode_workspace_bytes(C.byref(g), n, hq, max_context_len, C.byref(o)))
    ws_ptr, ws_bytes = None, 0
    if need:
        if workspace is None:
            raise ValueError(f"decode needs a workspace of {need} bytes")
        _dev(workspace, "workspace")
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    return g, n, hq, ws_ptr, ws_bytes


def decode(geom: Geometry, k_pool, v_pool, layer: int, q, out, block_tables, context_lens,
           max_context_len: int, scale: float = 0.0, workspace=None, blocks_per_split: int = 0,
           kernel: str = "auto", stream=None, kv_reuse: bool = False, merge: bool = False,
           waves_per_group: int = 0, host_lens=None):
    """out[i, h] = softmax attention of q[i, h] over sequence i's first
    context_lens[i] tokens, read through block_tables[i]. kv_reuse=True when many
    sequences of the batch share blocks (keeps them cacheable). merge=True merges
    the splits inside the decode launch (the workspace must start zeroed)."""
    hl = _host_lens(host_lens, q.shape[0])
    o = _opts(blocks_per_split, KERNELS[kernel], kv_reuse, merge, waves_per_group, hl)
    g, n, hq, ws_ptr, ws_bytes = _decode_args(geom, k_pool, v_pool, q, out, block_tables,
                                              context_lens, max_context_len, workspace, o)
    check(_L().pa_decode(C.byref(g), _ptr(k_pool), _ptr(v_pool), layer, _ptr(q), _ptr(out), n, hq,
                         _ptr(block_tables), int(block_tables.shape[1]), _ptr(context_lens),
                         int(max_context_len), float(scale), C.byref(o), ws_ptr, ws_bytes,
                         _stream(stream, q.device)),
          "pa_decode")


def decode_append(geom: Geometry, k_pool, v_pool, layer: int, q, k_new, v_new, out, block_tables,
                  context_lens, max_context_len: int, scale: float = 0.0, workspace=None,
                  blocks_per_split: int = 0, kernel: str = "auto", stream=None,
                  kv_reuse: bool = False, merge: bool = False, waves_per_group: int = 0,
                  host_lens=None):
    """Write each sequence's new token (k_new[i], v_new[i]: [n_seqs, H_kv, d]) at
    position context_lens[i] - 1 through its block table, then decode as
    `decode` does, in one launch."""
    hl = _host_lens(host_lens, q.shape[0])
    o = _opts(blocks_per_split, KERNELS[kernel], kv_reuse, merge, waves_per_group, hl)
    g, n, hq, ws_ptr, ws_bytes = _decode_args(geom, k_pool, v_pool, q, out, block_tables,
                                              context_lens, max_context_len, workspace, o)
    per = geom.num_kv_heads * geom.head_dim
    _dev(k_new, "k_new", geom.io_dtype, n * per)
    _dev(v_new, "v_new", geom.io_dtype, n * per)
    check(_L().pa_decode_append(C.byref(g), _ptr(k_pool), _ptr(v_pool), layer, _ptr(q),
                                _ptr(k_new), _ptr(v_new), _ptr(out), n, hq, _ptr(block_tables),
                                int(block_tables.shape[1]), _ptr(context_lens),
                                int(max_context_len), float(scale), C.byref(o), ws_ptr, ws_bytes,
                                _stream(stream, q.device)),
          "pa_decode_append")


class DecodeAppendCall:
    """decode_append with its arguments checked and marshalled once: each call
    is then one C call with the stored arguments. For a decode loop that reuses
    the same buffers (static q / k_new / v_new / out / table / length tensors
    whose contents change between calls), where the per-call checks would cost
    more host time than a short launch runs. The tensors (and host_lens, which
    may be updated in place) must stay alive and in place; max_context_len may
    change per call."""

    def __init__(self, geom: Geometry, k_pool, v_pool, layer: int, q, k_new, v_new, out,
                 block_tables, context_lens, max_context_len: int, scale: float = 0.0,
                 workspace=None, blocks_per_split: int = 0, kernel: str = "auto", stream=None,
                 kv_reuse: bool = False, merge: bool = False, waves_per_group: int = 0,
                 host_lens=None):
        hl = _host_lens(host_lens, q.shape[0])
        o = _opts(blocks_per_split, KERNELS[kernel], kv_reuse, merge, waves_per_group, hl)
        g, n, hq, ws_ptr, ws_bytes = _decode_args(geom, k_pool, v_pool, q, out, block_tables,
                                                  context_lens, max_context_len, workspace, o)
        per = geom.num_kv_heads * geom.head_dim
        _dev(k_new, "k_new", geom.io_dtype, n * per)
        _dev(v_new, "v_new", geom.io_dtype, n * per)
        self._keep = (hl, o, g, k_pool, v_pool, q, k_new, v_new, out, block_tables, context_lens,
                      workspace)
        self._fn = _L().pa_decode_append
        self._n, self._hq, self._g, self._o, self._ws_bytes = n, hq, g, o, ws_bytes
        self._head = (C.byref(g), _ptr(k_pool), _ptr(v_pool), int(layer), _ptr(q), _ptr(k_new),
                      _ptr(v_new), _ptr(out), n, hq, _ptr(block_tables), int(block_tables.shape[1]),
                      _ptr(context_lens))
        self._tail = (float(scale), C.byref(o), ws_ptr, ws_bytes, _stream(stream, q.device))
        self._max_ctx = int(max_context_len)

    def __call__(self, max_context_len: Optional[int] = None) -> None:
        if max_context_len is not None and int(max_context_len) != self._max_ctx:
            m = int(max_context_len)
            need = int(_L().pa_decode_workspace_bytes(C.byref(self._g), self._n, self._hq, m,
                                                       C.byref(self._o)))
            if need > self._ws_bytes:
                raise ValueError(f"decode needs a workspace of {need} bytes")
            self._max_ctx = m
        check(self._fn(*self._head, self._max_ctx, *self._tail), "pa_decode_append")


# Bytes of the library's own partials array behind decode_append_noalloc.
NOALLOC_SCRATCH_BYTES = 16 << 20


def decode_append_noalloc(geom: Geometry, k_pool, v_pool, layer: int, q, k_new, v_new, out,
                          block_tables, context_lens, max_context_len: int, scale: float = 0.0,
                          blocks_per_split: int = 0, kernel: str = "auto", stream=None,
                          kv_reuse: bool = False):
    """decode_append with the split partials in the library's own device array
    (NOALLOC_SCRATCH_BYTES per GPU) instead of a workspace: no allocation, for
    callers that cannot allocate. Calls that overlap on one GPU race."""
    o = _opts(blocks_per_split, KERNELS[kernel], kv_reuse)
    g, n, hq, _, _ = _decode_args(geom, k_pool, v_pool, q, out, block_tables, context_lens,
                                  max_context_len, None, o, need_workspace=False)
    per = geom.num_kv_heads * geom.head_dim
    _dev(k_new, "k_new", geom.io_dtype, n * per)
    _dev(v_new, "v_new", geom.io_dtype, n * per)
    check(_L().pa_decode_append_noalloc(C.byref(g), _ptr(k_pool), _ptr(v_pool), layer, _ptr(q),
                                        _ptr(k_new), _ptr(v_new), _ptr(out), n, hq,
                                        _ptr(block_tables), int(block_tables.shape[1]),
                                        _ptr(context_lens), int(max_context_len), float(scale),
                                        C.byref(o), _stream(stream, q.device)),
          "pa_decode_append_noalloc")


def prefill_workspace_bytes(geom: Geometry, n_seqs: int, n_tokens: int, n_q_heads: int,
                            max_q_len: int, max_context_len: int, splits: int = 0) -> int:
    """Workspace bytes prefill needs for these arguments (splits 0: what the
    automatic choice uses)."""
    g = geom.c()
    return int(_L().pa_prefill_workspace_bytes(C.byref(g), n_seqs, n_tokens, n_q_heads, max_q_len,
                                                max_context_len, splits))


def prefill(geom: Geometry, k_pool, v_pool, layer: int, q, k_new, v_new, out, q_start, block_tables,
            ctx_lens, max_q_len: int, max_context_len: int, scale: float = 0.0, stream=None,
            splits: int = 0, workspace=None):
    """Chunked prefill of one layer: chunk i = rows q_start[i]..q_start[i+1]-1 of q
    [n_tok, H_q, d] / k_new, v_new [n_tok, H_kv, d], at positions ctx_lens[i] + r.
    Writes the chunks' K/V through block_tables, then attends causally; out gets
    [n_tok, H_q, d]. splits: 0 = automatic (uses `workspace` when given and large
    enough), 1 = none, k = k splits (needs `workspace`, a device tensor of at least
    prefill_workspace_bytes bytes)."""
    _dev(k_pool, "k_pool", geom.torch_dtype, geom.pool_numel)
    _dev(v_pool, "v_pool", geom.torch_dtype, geom.pool_numel)
    if q.dim() != 3 or q.shape[2] != geom.head_dim:
        raise ValueError("q must be [n_tokens, n_q_heads, head_dim]")
    n_tok, hq = int(q.shape[0]), int(q.shape[1])
    _dev(q, "q", geom.io_dtype)
    _dev(out, "out", geom.io_dtype, q.numel())
    per = geom.num_kv_heads * geom.head_dim
    _dev(k_new, "k_new", geom.io_dtype, n_tok * per)
    _dev(v_new, "v_new", geom.io_dtype, n_tok * per)
    if block_tables.dim() != 2:
        raise ValueError("block_tables must be [n_seqs, max_blocks]")
    n = int(block_tables.shape[0])
    _dev(block_tables, "block_tables", torch.int32)
    _dev(q_start, "q_start", torch.int32, n + 1)
    _dev(ctx_lens, "ctx_lens", torch.int32, n)
    if workspace is not None and (not workspace.is_cuda or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous device tensor")
    g = geom.c()
    check(_L().pa_prefill(C.byref(g), _ptr(k_pool), _ptr(v_pool), layer, _ptr(q), _ptr(k_new),
                          _ptr(v_new), _ptr(out), n, n_tok, hq, _ptr(q_start), _ptr(block_tables),
                          int(block_tables.shape[1]), _ptr(ctx_lens), int(max_q_len),
                          int(max_context_len), float(scale), int(splits), _ptr(workspace),
                          0 if workspace is None else workspace.numel() * workspace.element_size(),
                          _stream(stream, q.device)),
          "pa_prefill")


def _ids(t, what, n=None):
    _dev(t, what, torch.int32, n)


def copy_blocks(geom: Geometry, k_pool, v_pool, src, dst, stream=None):
    _dev(k_pool, "k_pool", geom.torch_dtype, geom.pool_numel)
    _dev(v_pool, "v_pool", geom.torch_dtype, geom.pool_numel)
    n = src.numel()
    _ids(src, "src")
    _ids(dst, "dst", n)
    g = geom.c()
    check(_L().pa_copy_blocks(C.byref(g), _ptr(k_pool), _ptr(v_pool), _ptr(src), _ptr(dst), n,
                              _stream(stream, k_pool.device)), "pa_copy_blocks")


def gather_blocks(geom: Geometry, k_pool, v_pool, block_ids, staging, stream=None):
    _dev(k_pool, "k_pool", geom.torch_dtype, geom.pool_numel)
    _dev(v_pool, "v_pool", geom.torch_dtype, geom.pool_numel)
    n = block_ids.numel()
    _ids(block_ids, "block_ids")
    _dev(staging, "staging")
    if staging.numel() * staging.element_size() < n * bytes_per_block(geom):
        raise ValueError("staging buffer too small")
    g = geom.c()
    check(_L().pa_gather_blocks(C.byref(g), _ptr(k_pool), _ptr(v_pool), _ptr(block_ids), n,
                                _ptr(staging), _stream(stream, k_pool.device)), "pa_gather_blocks")


def scatter_blocks(geom: Geometry, k_pool, v_pool, staging, block_ids, stream=None):
    _dev(k_pool, "k_pool", geom.torch_dtype, geom.pool_numel)
    _dev(v_pool, "v_pool", geom.torch_dtype, geom.pool_numel)
    n = block_ids.numel()
    _ids(block_ids, "block_ids")
    _dev(staging, "staging")
    if staging.numel() * staging.element_size() < n * bytes_per_block(geom):
        raise ValueError("staging buffer too small")
    g = geom.c()
    check(_L().pa_scatter_blocks(C.byref(g), _ptr(k_pool), _ptr(v_pool), _ptr(staging),
                                 _ptr(block_ids), n, _stream(stream, k_pool.device)),
          "pa_scatter_blocks")


def copy_to_host(host_dst: torch.Tensor, device_src: torch.Tensor, nbytes: Optional[int] = None,
                 stream=None):
    if host_dst.is_cuda or not device_src.is_cuda:
        raise ValueError("copy_to_host: host_dst on the host, device_src on the device")
    if not host_dst.is_contiguous() or not device_src.is_contiguous():
        raise ValueError("copy_to_host: contiguous tensors only")
    cap = min(host_dst.numel() * host_dst.element_size(), device_src.numel() * device_src.element_size())
    nbytes = cap if nbytes is None else int(nbytes)
    if nbytes > cap:
        raise ValueError("copy_to_host: nbytes exceeds a buffer")
    check(_L().pa_copy_to_host(_ptr(host_dst), _ptr(device_src), nbytes,
                               _stream(stream, device_src.device)), "pa_copy_to_host")


def copy_to_device(device_dst: torch.Tensor, host_src: torch.Tensor, nbytes: Optional[int] = None,
                   stream=None):
    if host_src.is_cuda or not device_dst.is_cuda:
        raise ValueError("copy_to_device: host_src on the host, device_dst on the device")
    if not host_src.is_contiguous() or not device_dst.is_contiguous():
        raise ValueError("copy_to_device: contiguous tensors only")
    cap = min(host_src.numel() * host_src.element_size(), device_dst.numel() * device_dst.element_size())
    nbytes = cap if nbytes is None else int(nbytes)
    if nbytes > cap:
        raise ValueError("copy_to_device: nbytes exceeds a buffer")
    check(_L().pa_copy_to_device(_ptr(device_dst), _ptr(host_src), nbytes,
                                 _stream(stream, device_dst.device)), "pa_copy_to_device")


# --------------------------------------------------------------------- timing
class Profiler:
    """Per-kernel launch timing recorded by the library with hipEvents."""

    @staticmethod
    def enable(on: bool = True):
        check(_L().pa_prof_enable(1 if on else 0), "pa_prof_enable")

    @staticmethod
    def reset():
        check(_L().pa_prof_reset(), "pa_prof_reset")

    @staticmethod
    def read(kernel: str):
        n, ms = C.c_int64(0), C.c_double(0.0)
        check(_L().pa_prof_read(kernel.encode(), C.byref(n), C.byref(ms)), "pa_prof_read")
        return int(n.value), float(ms.value)


# --------------------------------------------------------------------- block manager
def _i32arr(values) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(values, dtype=np.int32))


def _p32(a: np.ndarray):
    return a.ctypes.data_as(C.POINTER(C.c_int32))


def _p64(a: np.ndarray):
    return a.ctypes.data_as(C.POINTER(C.c_int64))


class BlockManager:
    """Host block manager of libpa (free list, reference counts, block tables)."""

    def __init__(self, num_blocks: int, block_size: int, free_order: Optional[Sequence[int]] = None):
        self._lib = _L()
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)
        h = C.c_void_p()
        fo = None if free_order is None else _i32arr(free_order)
        if fo is not None and fo.size != num_blocks:
            raise ValueError("free_order must list every block once")
        check(self._lib.pa_bm_create(num_blocks, block_size, None if fo is None else _p32(fo),
                                     C.byref(h)), "pa_bm_create")
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            self._lib.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def num_free(self) -> int:
        return int(self._lib.pa_bm_num_free(self._h))

    def refcount(self, block: int) -> int:
        return int(self._lib.pa_bm_refcount(self._h, block))

    def alloc(self, n: int):
        out = np.empty(max(n, 1), np.int32)
        check(self._lib.pa_bm_alloc(self._h, n, _p32(out)), "pa_bm_alloc")
        return out[:n].tolist()

    def incref(self, ids):
        a = _i32arr(ids)
        check(self._lib.pa_bm_incref(self._h, _p32(a), a.size), "pa_bm_incref")

    def free_blocks(self, ids):
        a = _i32arr(ids)
        check(self._lib.pa_bm_free_blocks(self._h, _p32(a), a.size), "pa_bm_free_blocks")

    def seq_new(self) -> int:
        s = C.c_int32()
        check(self._lib.pa_bm_seq_new(self._h, C.byref(s)), "pa_bm_seq_new")
        return s.value

    def seq_from_blocks(self, ids) -> int:
        """New sequence starting from the listed cached full blocks (one more
        reference each), length len(ids) * block_size."""
        a = _i32arr(ids)
        s = C.c_int32()
        check(self._lib.pa_bm_seq_from_blocks(self._h, _p32(a), a.size, C.byref(s)),
              "pa_bm_seq_from_blocks")
        return s.value

    def fork(self, parent: int) -> int:
        s = C.c_int32()
        check(self._lib.pa_bm_seq_fork(self._h, parent, C.byref(s)), "pa_bm_seq_fork")
        return s.value

    def append(self, seq: int, n_tokens: int):
        """Returns (slots as int64 numpy array, list of (src, dst) copy pairs)."""
        slots = np.empty(max(n_tokens, 1), np.int64)
        src, dst, nc = C.c_int32(), C.c_int32(), C.c_int32()
        check(self._lib.pa_bm_seq_append(self._h, seq, n_tokens, _p64(slots), C.byref(src),
                                         C.byref(dst), C.byref(nc)), "pa_bm_seq_append")
        pairs = [(src.value, dst.value)] if nc.value else []
        return slots[:n_tokens], pairs

    def append_batch(self, seqs, counts):
        s, c = _i32arr(seqs), _i32arr(counts)
        total = int(c.sum()) if c.size else 0
        slots = np.empty(max(total, 1), np.int64)
        cs, cd = np.empty(max(s.size, 1), np.int32), np.empty(max(s.size, 1), np.int32)
        nc = C.c_int32()
        check(self._lib.pa_bm_append_batch(self._h, _p32(s), _p32(c), s.size, _p64(slots),
                                           _p32(cs), _p32(cd), C.byref(nc)), "pa_bm_append_batch")
        return slots[:total], list(zip(cs[:nc.value].tolist(), cd[:nc.value].tolist()))

    def release(self, seq: int):
        check(self._lib.pa_bm_seq_release(self._h, seq), "pa_bm_seq_release")

    def swap_out(self, seq: int, logical):
        a = _i32arr(logical)
        out = np.empty(max(a.size, 1), np.int32)
        check(self._lib.pa_bm_seq_swap_out(self._h, seq, _p32(a), a.size, _p32(out)),
              "pa_bm_seq_swap_out")
        return out[:a.size].tolist()

    def swap_in(self, seq: int, logical):
        a = _i32arr(logical)
        out = np.empty(max(a.size, 1), np.int32)
        check(self._lib.pa_bm_seq_swap_in(self._h, seq, _p32(a), a.size, _p32(out)),
              "pa_bm_seq_swap_in")
        return out[:a.size].tolist()

    def permute_free(self, perm):
        """Free-list entry k becomes the current entry perm[k]."""
        a = _i32arr(perm)
        check(self._lib.pa_bm_permute_free(self._h, _p32(a), a.size), "pa_bm_permute_free")

    def info(self, seq: int):
        n, b = C.c_int64(), C.c_int32()
        check(self._lib.pa_bm_seq_info(self._h, seq, C.byref(n), C.byref(b)), "pa_bm_seq_info")
        return n.value, b.value

    def length(self, seq: int) -> int:
        return self.info(seq)[0]

    def table(self, seq: int):
        _, nb = self.info(seq)
        out = np.empty(max(nb, 1), np.int32)
        m = C.c_int32()
        check(self._lib.pa_bm_seq_table(self._h, seq, _p32(out), nb, C.byref(m)), "pa_bm_seq_table")
        return out[:nb].tolist()

    def build_tables(self, seqs, max_blocks: int, pad: int = 0):
        """(tables int32 [n, max_blocks], lens int32 [n]) as numpy arrays."""
        s = _i32arr(seqs)
        tables = np.empty((max(s.size, 1), max(max_blocks, 1)), np.int32)
        lens = np.empty(max(s.size, 1), np.int32)
        check(self._lib.pa_bm_build_tables(self._h, _p32(s), s.size, max_blocks, pad, _p32(tables),
                                           _p32(lens)), "pa_bm_build_tables")
        return tables[:s.size, :max_blocks], lens[:s.size]

    def validate(self):
        check(self._lib.pa_bm_validate(self._h), "pa_bm_validate")

    def free_list(self):
        """The free queue, front to back."""
        n = C.c_int32()
        out = np.empty(max(self.num_blocks, 1), np.int32)
        check(self._lib.pa_bm_free_list(self._h, _p32(out), out.size, C.byref(n)), "pa_bm_free_list")
        return out[:n.value].tolist()

    # ---- tiered residency ("Asynchronous paged swapping") -------------------
    def attach_host_pool(self, num_frames: int):
        check(self._lib.pa_bm_attach_host_pool(self._h, int(num_frames)), "pa_bm_attach_host_pool")

    def detach_host_pool(self):
        check(self._lib.pa_bm_detach_host_pool(self._h), "pa_bm_detach_host_pool")

    def host_frames_free(self) -> int:
        return int(self._lib.pa_bm_host_frames_free(self._h))

    def host_free_runs(self):
        """Free runs of the host frame pool as [(start, length)], by start."""
        n = C.c_int32()
        check(self._lib.pa_bm_host_free_runs(self._h, None, None, 0, C.byref(n)), "pa_bm_host_free_runs")
        st, ln = np.empty(max(n.value, 1), np.int32), np.empty(max(n.value, 1), np.int32)
        check(self._lib.pa_bm_host_free_runs(self._h, _p32(st), _p32(ln), n.value, C.byref(n)),
              "pa_bm_host_free_runs")
        return list(zip(st[:n.value].tolist(), ln[:n.value].tolist()))

    def tier(self, seq: int, logical: int):
        """(tag, index) of one table entry; tags are the PA_TIER_* values."""
        t, i = C.c_int32(), C.c_int32()
        check(self._lib.pa_bm_block_tier(self._h, seq, logical, C.byref(t), C.byref(i)),
              "pa_bm_block_tier")
        return t.value, i.value

    def swap_out_begin(self, seq: int, logical):
        """Returns (physical blocks, first host frame)."""
        a = _i32arr(logical)
        phys, first = np.empty(max(a.size, 1), np.int32), C.c_int32()
        check(self._lib.pa_bm_swap_out_begin(self._h, seq, _p32(a), a.size, _p32(phys),
                                             C.byref(first)), "pa_bm_swap_out_begin")
        return phys[:a.size].tolist(), first.value

    def swap_out_finish(self, seq: int, logical):
        a = _i32arr(logical)
        check(self._lib.pa_bm_swap_out_finish(self._h, seq, _p32(a), a.size), "pa_bm_swap_out_finish")

    def swap_in_begin(self, seq: int, logical):
        """Returns (new physical blocks, host frames)."""
        a = _i32arr(logical)
        phys, frames = np.empty(max(a.size, 1), np.int32), np.empty(max(a.size, 1), np.int32)
        check(self._lib.pa_bm_swap_in_begin(self._h, seq, _p32(a), a.size, _p32(phys),
                                            _p32(frames)), "pa_bm_swap_in_begin")
        return phys[:a.size].tolist(), frames[:a.size].tolist()

    def swap_in_finish(self, seq: int, logical):
        a = _i32arr(logical)
        check(self._lib.pa_bm_swap_in_finish(self._h, seq, _p32(a), a.size), "pa_bm_swap_in_finish")


class RadixCache:
    """Radix prefix cache of libpa over a BlockManager (host only): longest
    prefix match with block-aligned truncation, insertion of finished requests,
    leaf-first LRU eviction. Keeps the BlockManager alive."""

    def __init__(self, bm: BlockManager):
        self._lib = _L()
        self.bm = bm
        self.block_size = bm.block_size
        h = C.c_void_p()
        check(self._lib.pa_radix_create(bm._h, C.byref(h)), "pa_radix_create")
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            self._lib.pa_radix_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def match(self, tokens):
        """(s_match, s_usable, block ids of the usable prefix, handle); pins the path."""
        t = _i32arr(tokens)
        out = np.empty(t.size // self.block_size + 1, np.int32)
        sm, su, h = C.c_int64(), C.c_int64(), C.c_int64()
        nb = C.c_int32()
        check(self._lib.pa_radix_match(self._h, _p32(t), t.size, C.byref(sm), C.byref(su), _p32(out),
                                       out.size, C.byref(nb), C.byref(h)), "pa_radix_match")
        return int(sm.value), int(su.value), out[:nb.value].tolist(), int(h.value)

    def unpin(self, handle: int):
        check(self._lib.pa_radix_unpin(self._h, int(handle)), "pa_radix_unpin")

    def insert(self, tokens, blocks) -> int:
        """Index a finished request's whole blocks; returns how many were adopted."""
        t, b = _i32arr(tokens), _i32arr(blocks)
        n = C.c_int32()
        check(self._lib.pa_radix_insert(self._h, _p32(t), t.size, _p32(b), b.size, C.byref(n)),
              "pa_radix_insert")
        return int(n.value)

    def evict(self, target_free: int):
        """Evict dormant leaves, LRU first, until target_free blocks are free;
        returns the evicted node ids in order."""
        cap = max(1, self.info()["nodes"])
        out = np.empty(cap, np.int64)
        n = C.c_int32()
        check(self._lib.pa_radix_evict(self._h, int(target_free), _p64(out), cap, C.byref(n)),
              "pa_radix_evict")
        return out[:n.value].tolist()

    def info(self):
        v = [C.c_int64() for _ in range(4)]
        check(self._lib.pa_radix_info(self._h, *[C.byref(x) for x in v]), "pa_radix_info")
        return dict(zip(("nodes", "blocks", "dormant", "pinned"), (int(x.value) for x in v)))

    def node_ids(self):
        n = C.c_int64()
        check(self._lib.pa_radix_node_ids(self._h, None, 0, C.byref(n)), "pa_radix_node_ids")
        out = np.empty(max(1, n.value), np.int64)
        check(self._lib.pa_radix_node_ids(self._h, _p64(out), out.size, C.byref(n)),
              "pa_radix_node_ids")
        return out[:n.value].tolist()

    def node(self, node_id: int):
        """(parent, pins, last access, tokens, blocks) of one node."""
        meta = np.zeros(4, np.int64)
        check(self._lib.pa_radix_node(self._h, node_id, _p64(meta), None, 0, None, 0),
              "pa_radix_node")
        nb = int(meta[3])
        toks = np.empty(max(1, nb * self.block_size), np.int32)
        blks = np.empty(max(1, nb), np.int32)
        check(self._lib.pa_radix_node(self._h, node_id, _p64(meta), _p32(toks), toks.size,
                                      _p32(blks), blks.size), "pa_radix_node")
        return (int(meta[0]), int(meta[1]), int(meta[2]), toks[:nb * self.block_size].tolist(),
                blks[:nb].tolist())

    def nodes(self):
        return {i: self.node(i) for i in self.node_ids()}


# Buffers of swappers whose destroy call was refused while the object was being
# collected: the library still addresses them, so they are kept for the process.
_HELD_BY_LIBRARY = []


class Swapper:
    """Asynchronous block migration between the device pool and pinned host frames
    (pa_swapper_*). Copies run on the swapper's own streams; each migration's
    completion step retags the block manager's table when its copies are done.
    The pinned frame buffer and the device staging buffer are allocated here
    with torch (sizes from pa_swapper_buffer_bytes) and handed to the library,
    which allocates no memory of its own.

    `after` (swap_out / swap_in): the stream whose earlier work the copies must
    follow; None means the current stream of the pools' device, 0 means none."""

    def __init__(self, geom: Geometry, bm: BlockManager, k_pool: torch.Tensor, v_pool: torch.Tensor,
                 num_frames: int, chunk_blocks: int = 0, move_wgs: int = 0, direct: bool = False):
        _dev(k_pool, "k_pool")
        _dev(v_pool, "v_pool")
        self._lib = _L()
        self._bm, self._k, self._v = bm, k_pool, v_pool     # kept alive with the swapper
        self.device = k_pool.device
        h = C.c_void_p()
        g = geom.c()
        opts = _lib.pa_swap_opts(int(chunk_blocks), int(move_wgs), 1 if direct else 0)
        hb, sb = C.c_size_t(), C.c_size_t()
        check(self._lib.pa_swapper_buffer_bytes(C.byref(g), int(num_frames), C.byref(opts),
                                                C.byref(hb), C.byref(sb)), "pa_swapper_buffer_bytes")
        self._host = torch.empty(max(1, hb.value), dtype=torch.uint8, pin_memory=True)
        self._staging = (torch.empty(sb.value, dtype=torch.uint8, device=self.device)
                         if sb.value else None)
        check(self._lib.pa_swapper_create(C.byref(g), bm._h, _ptr(k_pool), _ptr(v_pool),
                                          int(num_frames), C.byref(opts), self._host.data_ptr(),
                                          hb.value, _ptr(self._staging) if sb.value else None,
                                          sb.value, C.byref(h)),
              "pa_swapper_create")
        self._h = h
        self.num_frames = int(num_frames)
        host, ks, ds = C.c_void_p(), C.c_void_p(), C.c_void_p()
        fb, cb = C.c_int64(), C.c_int32()
        check(self._lib.pa_swapper_info(h, C.byref(host), C.byref(ks), C.byref(ds), C.byref(fb),
                                        C.byref(cb), None, None), "pa_swapper_info")
        self.frame_bytes, self.chunk_blocks = fb.value, cb.value
        self._host_ptr = host.value
        # (kernel stream, DMA stream), e.g. for a profiler; use fence() to order work after them
        self.streams = (torch.cuda.ExternalStream(ks.value, device=self.device),
                        torch.cuda.ExternalStream(ds.value, device=self.device))

    def _after(self, after):
        if after is None:
            return torch.cuda.current_stream(self.device).cuda_stream
        return _stream(after, self.device)

    def swap_out(self, seq: int, logical, after=None):
        a = _i32arr(logical)
        check(self._lib.pa_swap_out_async(self._h, seq, _p32(a), a.size, self._after(after)),
              "pa_swap_out_async")

    def swap_in(self, seq: int, logical, after=None):
        a = _i32arr(logical)
        check(self._lib.pa_swap_in_async(self._h, seq, _p32(a), a.size, self._after(after)),
              "pa_swap_in_async")

    def fence(self, stream=None):
        """Make `stream` (default: current) wait on the device for the work queued so far."""
        check(self._lib.pa_swapper_fence(self._h, _stream(stream, self.device)), "pa_swapper_fence")

    def sync(self):
        check(self._lib.pa_swapper_sync(self._h), "pa_swapper_sync")

    def pending(self) -> int:
        return int(self._lib.pa_swapper_pending(self._h))

    def bytes_moved(self):
        """(bytes of completed swap-outs, bytes of completed swap-ins)."""
        o, i = C.c_int64(), C.c_int64()
        check(self._lib.pa_swapper_info(self._h, None, None, None, None, None, C.byref(o),
                                        C.byref(i)), "pa_swapper_info")
        return o.value, i.value

    def host_frames(self) -> np.ndarray:
        """The pinned frame buffer as uint8 [num_frames, frame_bytes] (no copy)."""
        buf = (C.c_uint8 * (self.num_frames * self.frame_bytes)).from_address(self._host_ptr)
        return np.ctypeslib.as_array(buf).reshape(self.num_frames, self.frame_bytes)

    def close(self):
        """Destroy the swapper. Raises (and leaves the swapper usable) while an
        entry still holds a frame or a migration has not completed."""
        if getattr(self, "_h", None):
            check(self._lib.pa_swapper_destroy(self._h), "pa_swapper_destroy")
            self._h = None
            self._host = self._staging = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            # refused: the library still uses both buffers, so they must outlive it
            _HELD_BY_LIBRARY.append((getattr(self, "_host", None), getattr(self, "_staging", None)))
