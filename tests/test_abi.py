"""The C-ABI library loads on the host and exports every symbol include/pa.h declares."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")
LIB = os.path.join(ROOT, "paged_kv_cache_83_amd", "libpa.so")


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared()
    for must in ("pa_append_kv", "pa_decode", "pa_copy_blocks", "pa_gather_blocks",
                 "pa_scatter_blocks", "pa_bytes_per_token", "pa_decode_workspace_bytes",
                 "pa_bm_create", "pa_bm_seq_append", "pa_bm_seq_fork", "pa_bm_seq_release"):
        assert must in names


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(LIB)
    missing = [n for n in declared() if not hasattr(lib, n)]
    assert not missing, missing
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (pa_[a-z0-9_]+)$", out, flags=re.M))
    assert set(declared()) <= exported


def test_binding_declares_every_symbol():
    from paged_kv_cache_83_amd import _lib
    assert set(declared()) == set(_lib.SIGNATURES)


def test_library_is_for_gfx950():
    # the device code object embedded in the library targets gfx950
    blob = open(LIB, "rb").read()
    assert b"gfx950" in blob


def test_host_entry_points_reject_bad_arguments():
    import paged_kv_cache_83_amd as pk
    from paged_kv_cache_83_amd import _lib
    L = _lib.load()
    assert L.pa_bytes_per_token(0, 8, 128, 2, 1) == -1
    assert L.pa_blocks_for_tokens(-1, 16) == -1
    g = _lib.pa_geom(80, 8, 128, 16, 32768, 1)
    assert L.pa_bytes_per_block(ctypes.byref(g)) == 5242880
    bad = _lib.pa_geom(80, 8, 128, 16, 32768, 7)
    assert L.pa_bytes_per_block(ctypes.byref(bad)) == -1
    # device entry points validate before touching any pointer (no GPU needed)
    assert L.pa_decode(ctypes.byref(bad), None, None, 0, None, None, 1, 64, None, 1, None, 16, 0.0,
                       None, None, 0, None) == -1
    assert L.pa_append_kv(ctypes.byref(g), None, None, 99, None, None, None, 1, None) == -1
    assert L.pa_copy_blocks(ctypes.byref(g), None, None, None, None, 3, None) == -1
    # 65 query heads cannot be grouped over 8 KV heads
    assert L.pa_decode(ctypes.byref(g), None, None, 0, None, None, 1, 65, None, 1, None, 16, 0.0,
                       None, None, 0, None) == -1
    # table too short for max_context_len
    assert L.pa_decode(ctypes.byref(g), None, None, 0, None, None, 1, 64, None, 1, None, 17, 0.0,
                       None, None, 0, None) == -1
    # zero sequences is a no-op
    assert L.pa_decode(ctypes.byref(g), None, None, 0, None, None, 0, 64, None, 1, None, 16, 0.0,
                       None, None, 0, None) == 0
    assert pk.bytes_per_token(80, 8, 128, 2) == 327680


def test_workspace_sizing():
    import paged_kv_cache_83_amd as pk
    g = pk.Geometry(80, 8, 128, 16, 32768, "bf16")
    ws = pk.decode_workspace_bytes(g, 16, 64, 32768)
    # 16 seqs x 64 heads x splits x (128 + 2) floats
    assert ws > 0 and ws % (16 * 64 * 130 * 4) == 0
    # one split per sequence writes the output directly (generic kernel) ...
    assert pk.decode_workspace_bytes(g, 16, 64, 32768, blocks_per_split=4096, kernel="generic") == 0
    # ... while the MFMA kernel caps a split at 256 blocks: 2048 blocks -> 8 splits
    assert pk.decode_workspace_bytes(g, 16, 64, 32768, blocks_per_split=4096) == 16 * 64 * 8 * 130 * 4
    g1 = pk.Geometry(12, 12, 64, 16, 1024, "f32")
    assert pk.decode_workspace_bytes(g1, 8, 12, 1024, kernel="generic") >= 0
    with pytest.raises(Exception):
        pk.decode_workspace_bytes(g1, 8, 12, 1024, kernel="bogus")


def test_prefill_workspace_sizing():
    """The prefill launch plan as the workspace query reports it (host only)."""
    import paged_kv_cache_83_amd as pk
    g = pk.Geometry(80, 8, 128, 16, 32768, "bf16")
    row = 64 * 130 * 4                                  # one token: 64 heads x (128 + 2) floats
    # 16 sequences x 4 draft tokens over 32,764 cached: short chunks (8 x 4 = 32 rows
    # per KV head), 128 waves before splitting -> 8 splits of 256 blocks
    assert pk.prefill_workspace_bytes(g, 16, 64, 64, 4, 32768) == 8 * 64 * row
    assert pk.prefill_workspace_bytes(g, 16, 64, 64, 4, 32768, 3) == 3 * 64 * row
    # one sequence, short history: 63 blocks in splits of at least 16 -> 4
    assert pk.prefill_workspace_bytes(g, 1, 4, 64, 4, 1000) == 4 * 4 * row
    # long chunks (8 x 33 > 32 rows): 128-row tiles, at most 4 automatic splits
    assert pk.prefill_workspace_bytes(g, 16, 16 * 2048, 64, 2048, 4096) == 0
    assert pk.prefill_workspace_bytes(g, 1, 33, 64, 33, 32768) == 4 * 33 * row
    # explicit counts are honoured; 1 needs nothing; out of range and bad shapes give 0
    assert pk.prefill_workspace_bytes(g, 16, 64, 64, 4, 32768, 1) == 0
    assert pk.prefill_workspace_bytes(g, 16, 64, 64, 4, 32768, 64) == 64 * 64 * row
    assert pk.prefill_workspace_bytes(g, 16, 64, 64, 4, 32768, 65) == 0
    assert pk.prefill_workspace_bytes(g, 16, 64, 60, 4, 32768) == 0       # 60 heads over 8
    assert pk.prefill_workspace_bytes(g, 16, 64, 64, 5, 4) == 0           # chunk past the bound


def test_prepared_decode_call_checks_its_buffers_once_on_the_host():
    """DecodeAppendCall checks every buffer when it is built (the per-call path
    then only passes the stored arguments): host tensors are refused before any
    device call is made."""
    import torch
    import paged_kv_cache_83_amd as pk
    geom = pk.Geometry(1, 2, 64, 16, 8, "f32")
    k_pool = torch.zeros(geom.pool_numel, dtype=torch.float32)
    v_pool = torch.zeros_like(k_pool)
    q = torch.zeros(2, 2, 64)
    new = torch.zeros(2, 2, 64)
    tables = torch.zeros(2, 2, dtype=torch.int32)
    lens = torch.ones(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="CUDA"):
        pk.DecodeAppendCall(geom, k_pool, v_pool, 0, q, new, new, torch.empty_like(q), tables, lens, 1)
