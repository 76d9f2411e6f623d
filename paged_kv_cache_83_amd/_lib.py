"""ctypes declarations for libpa.so (the C interface in include/pa.h).

Loading fails loudly: there is no fallback implementation anywhere in this
package, so a missing or stale library is an error, never a silent CPU path.
"""

from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("PA_LIB", os.path.join(_HERE, "libpa.so"))

PA_OK = 0
STATUS_NAMES = {
    0: "PA_OK", -1: "PA_ERR_INVALID_ARG", -2: "PA_ERR_OUT_OF_BLOCKS", -3: "PA_ERR_DOUBLE_FREE",
    -4: "PA_ERR_NOT_FOUND", -5: "PA_ERR_HIP", -6: "PA_ERR_WORKSPACE", -7: "PA_ERR_UNSUPPORTED",
    -8: "PA_ERR_OUT_OF_FRAMES",
}
PA_TIER_HBM, PA_TIER_HOST, PA_TIER_PENDING_OUT, PA_TIER_PENDING_IN = 0, 1, 2, 3
PA_F32, PA_BF16, PA_FP8 = 0, 1, 2


class pa_geom(C.Structure):
    _fields_ = [("num_layers", C.c_int32), ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("block_size", C.c_int32), ("num_blocks", C.c_int32), ("dtype", C.c_int32)]


class pa_swap_opts(C.Structure):
    _fields_ = [("chunk_blocks", C.c_int32), ("move_wgs", C.c_int32), ("direct", C.c_int32)]


class pa_decode_opts(C.Structure):
    _fields_ = [("blocks_per_split", C.c_int32), ("kernel", C.c_int32), ("kv_reuse", C.c_int32),
                ("merge", C.c_int32), ("host_context_lens", C.c_void_p),
                ("waves_per_group", C.c_int32)]


_i32, _i64, _f32, _f64 = C.c_int32, C.c_int64, C.c_float, C.c_double
_vp, _sz = C.c_void_p, C.c_size_t
_pg = C.POINTER(pa_geom)
_popts = C.POINTER(pa_decode_opts)
_pi32, _pi64, _pf64 = C.POINTER(_i32), C.POINTER(_i64), C.POINTER(_f64)

# name -> (restype, argtypes); every symbol include/pa.h declares.
SIGNATURES = {
    "pa_status_str": (C.c_char_p, [_i32]),
    "pa_version": (_i32, []),
    "pa_bytes_per_token": (_i64, [_i32, _i32, _i32, _i32, _i32]),
    "pa_bytes_per_block": (_i64, [_pg]),
    "pa_blocks_for_tokens": (_i64, [_i64, _i32]),
    "pa_pool_bytes": (_i64, [_pg]),
    "pa_append_kv": (_i32, [_pg, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _vp]),
    "pa_decode_workspace_bytes": (_sz, [_pg, _i32, _i32, _i32, _popts]),
    "pa_decode": (_i32, [_pg, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _vp, _i32, _vp, _i32, _f32,
                         _popts, _vp, _sz, _vp]),
    "pa_decode_append": (_i32, [_pg, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _i32, _i32, _vp, _i32,
                                _vp, _i32, _f32, _popts, _vp, _sz, _vp]),
    "pa_decode_append_noalloc": (_i32, [_pg, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _i32, _i32, _vp,
                                        _i32, _vp, _i32, _f32, _popts, _vp]),
    "pa_prefill": (_i32, [_pg, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp,
                          _i32, _vp, _i32, _i32, _f32, _i32, _vp, _sz, _vp]),
    "pa_prefill_workspace_bytes": (_sz, [_pg, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_copy_blocks": (_i32, [_pg, _vp, _vp, _vp, _vp, _i32, _vp]),
    "pa_gather_blocks": (_i32, [_pg, _vp, _vp, _vp, _i32, _vp, _vp]),
    "pa_scatter_blocks": (_i32, [_pg, _vp, _vp, _vp, _vp, _i32, _vp]),
    "pa_copy_to_host": (_i32, [_vp, _vp, _sz, _vp]),
    "pa_copy_to_device": (_i32, [_vp, _vp, _sz, _vp]),
    "pa_prof_enable": (_i32, [_i32]),
    "pa_prof_reset": (_i32, []),
    "pa_prof_read": (_i32, [C.c_char_p, _pi64, _pf64]),
    "pa_bm_create": (_i32, [_i32, _i32, _pi32, C.POINTER(_vp)]),
    "pa_bm_destroy": (None, [_vp]),
    "pa_bm_num_free": (_i32, [_vp]),
    "pa_bm_block_size": (_i32, [_vp]),
    "pa_bm_refcount": (_i32, [_vp, _i32]),
    "pa_bm_alloc": (_i32, [_vp, _i32, _pi32]),
    "pa_bm_incref": (_i32, [_vp, _pi32, _i32]),
    "pa_bm_free_blocks": (_i32, [_vp, _pi32, _i32]),
    "pa_bm_seq_new": (_i32, [_vp, _pi32]),
    "pa_bm_seq_from_blocks": (_i32, [_vp, _pi32, _i32, _pi32]),
    "pa_bm_seq_fork": (_i32, [_vp, _i32, _pi32]),
    "pa_bm_seq_append": (_i32, [_vp, _i32, _i32, _pi64, _pi32, _pi32, _pi32]),
    "pa_bm_append_batch": (_i32, [_vp, _pi32, _pi32, _i32, _pi64, _pi32, _pi32, _pi32]),
    "pa_bm_seq_release": (_i32, [_vp, _i32]),
    "pa_bm_seq_swap_out": (_i32, [_vp, _i32, _pi32, _i32, _pi32]),
    "pa_bm_seq_swap_in": (_i32, [_vp, _i32, _pi32, _i32, _pi32]),
    "pa_bm_permute_free": (_i32, [_vp, _pi32, _i32]),
    "pa_bm_seq_info": (_i32, [_vp, _i32, _pi64, _pi32]),
    "pa_bm_seq_table": (_i32, [_vp, _i32, _pi32, _i32, _pi32]),
    "pa_bm_build_tables": (_i32, [_vp, _pi32, _i32, _i32, _i32, _pi32, _pi32]),
    "pa_bm_validate": (_i32, [_vp]),
    "pa_bm_free_list": (_i32, [_vp, _pi32, _i32, _pi32]),
    "pa_bm_attach_host_pool": (_i32, [_vp, _i32]),
    "pa_bm_detach_host_pool": (_i32, [_vp]),
    "pa_bm_host_frames_free": (_i32, [_vp]),
    "pa_bm_host_free_runs": (_i32, [_vp, _pi32, _pi32, _i32, _pi32]),
    "pa_bm_block_tier": (_i32, [_vp, _i32, _i32, _pi32, _pi32]),
    "pa_bm_swap_out_begin": (_i32, [_vp, _i32, _pi32, _i32, _pi32, _pi32]),
    "pa_bm_swap_out_finish": (_i32, [_vp, _i32, _pi32, _i32]),
    "pa_bm_swap_in_begin": (_i32, [_vp, _i32, _pi32, _i32, _pi32, _pi32]),
    "pa_bm_swap_in_finish": (_i32, [_vp, _i32, _pi32, _i32]),
    "pa_swapper_buffer_bytes": (_i32, [_pg, _i32, C.POINTER(pa_swap_opts), C.POINTER(_sz),
                                       C.POINTER(_sz)]),
    "pa_swapper_create": (_i32, [_pg, _vp, _vp, _vp, _i32, C.POINTER(pa_swap_opts), _vp, _sz, _vp,
                                 _sz, C.POINTER(_vp)]),
    "pa_swapper_destroy": (_i32, [_vp]),
    "pa_swap_out_async": (_i32, [_vp, _i32, _pi32, _i32, _vp]),
    "pa_swap_in_async": (_i32, [_vp, _i32, _pi32, _i32, _vp]),
    "pa_swapper_fence": (_i32, [_vp, _vp]),
    "pa_swapper_sync": (_i32, [_vp]),
    "pa_swapper_pending": (_i32, [_vp]),
    "pa_swapper_info": (_i32, [_vp, C.POINTER(_vp), C.POINTER(_vp), C.POINTER(_vp), _pi64, _pi32,
                               _pi64, _pi64]),
    "pa_radix_create": (_i32, [_vp, C.POINTER(_vp)]),
    "pa_radix_destroy": (_i32, [_vp]),
    "pa_radix_match": (_i32, [_vp, _pi32, _i64, _pi64, _pi64, _pi32, _i32, _pi32, _pi64]),
    "pa_radix_unpin": (_i32, [_vp, _i64]),
    "pa_radix_insert": (_i32, [_vp, _pi32, _i64, _pi32, _i32, _pi32]),
    "pa_radix_evict": (_i32, [_vp, _i32, _pi64, _i32, _pi32]),
    "pa_radix_info": (_i32, [_vp, _pi64, _pi64, _pi64, _pi64]),
    "pa_radix_node_ids": (_i32, [_vp, _pi64, _i64, _pi64]),
    "pa_radix_node": (_i32, [_vp, _i64, _pi64, _pi32, _i64, _pi32, _i32]),
}

_lib = None


def load() -> C.CDLL:
    """Load libpa.so once and declare every function; raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libpa.so not found at {LIB_PATH}; build it with "
            "`python paged_kv_cache_83_amd/build.py` (there is no fallback path)")
    lib = C.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class PagedKVError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        name = STATUS_NAMES.get(status, str(status))
        super().__init__(f"{what}: {name}")


class OutOfBlocksError(PagedKVError):
    pass


class DoubleFreeError(PagedKVError):
    pass


class OutOfFramesError(PagedKVError):
    pass


def check(status: int, what: str) -> None:
    if status == PA_OK:
        return
    if status == -2:
        raise OutOfBlocksError(status, what)
    if status == -3:
        raise DoubleFreeError(status, what)
    if status == -8:
        raise OutOfFramesError(status, what)
    raise PagedKVError(status, what)
