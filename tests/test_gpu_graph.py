"""A whole decode step (every layer's fused append + decode, and the combine
launches of split plans, or the merge inside the decode launch with its
counters) captured in a HIP graph and replayed must give the same bits as the
eager launches, on every replay; likewise one chunked-prefill
call (append through the tables, tile or short-chunk attention, split merge).

Between replays the program does its own eager work on the same stream (an
eager decode into another buffer, a NaN refill of the graph's output) and
synchronises, so a replay that skipped a node or reused stale memory would
show up as a mismatch."""
import numpy as np
import pytest
import torch

import paged_kv_cache_83_amd as pk
from paged_kv_cache_83_amd import steps
from tests.gpu_helpers import make_batch, need_gpu, padded_tables, print_case, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # name, dtype, L, N, Hq, Hkv, d, B, lengths, bps, kernel, merge
    ("mfma_direct", "bf16", 3, 300, 32, 8, 128, 16, [1, 17, 300, 1024, 77], 0, "auto", False),
    ("mfma_split", "bf16", 2, 300, 32, 8, 128, 16, [1, 17, 300, 1024, 77], 4, "mfma", False),
    ("generic_f32_split", "f32", 2, 300, 12, 12, 64, 16, [5, 250, 900, 33], 2, "generic", False),
    ("valu_f32_split", "f32", 2, 300, 12, 12, 64, 16, [5, 250, 900, 33], 2, "valu", False),
    ("valu_f32_merge", "f32", 2, 300, 12, 12, 64, 16, [5, 250, 900, 33], 2, "valu", True),
    ("valu_bf16_merge", "bf16", 2, 300, 32, 8, 128, 16, [1, 17, 300, 1024, 77], 4, "valu", True),
    ("mfma_merge", "bf16", 2, 300, 32, 8, 128, 16, [1, 17, 300, 1024, 77], 4, "mfma", True),
    ("mfma_ragged", "bf16", 2, 400, 32, 8, 128, 16, [1, 17, 3000, 1024, 77, 0], 0, "mfma", "ragged"),
]


def _bits(t):
    return t.contiguous().view(torch.uint8).cpu().numpy()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_graph_replay_matches_eager(case):
    need_gpu()
    name, dtype, L, N, Hq, Hkv, d, B, lengths, bps, kernel, merge = case
    print_case(test="graph_replay", case=name)
    batch = make_batch(dtype, L, N, Hq, Hkv, d, B, lengths, seed=71, poison=False)
    geom = pk.Geometry(L, Hkv, d, B, N, dtype)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        K, V = to_dev(batch.k_pool, dtype), to_dev(batch.v_pool, dtype)
        n = len(lengths)
        q_all = torch.stack([to_dev(batch.q, dtype)] * L)
        kn = torch.stack([to_dev(batch.k_new, dtype)] * L)
        vn = torch.stack([to_dev(batch.v_new, dtype)] * L)
        tabs = torch.from_numpy(padded_tables(batch.tables, batch.max_blocks)).cuda()
        lens = torch.from_numpy(np.asarray(lengths, np.int32)).cuda()
        max_ctx = max(lengths)
        host_lens = np.asarray(lengths, np.int32) if merge == "ragged" else None
        merge = merge is True
        ws = torch.zeros(max(1, pk.decode_workspace_bytes(geom, n, Hq, max_ctx, bps, kernel, merge,
                                                          0, host_lens)),
                         dtype=torch.uint8, device="cuda")
        out_eager = torch.empty_like(q_all)
        out_graph = torch.full_like(q_all, float("nan"))
        other = torch.empty_like(q_all)

    def step(out):
        steps.decode_step(geom, K, V, q_all, kn, vn, None, tabs, lens, max_ctx, out, ws,
                          blocks_per_split=bps, kernel=kernel, stream=s, merge=merge,
                          host_lens=host_lens)

    step(out_eager)
    torch.cuda.synchronize()
    ref, k_ref, v_ref = _bits(out_eager), _bits(K), _bits(V)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step(out_graph)
    torch.cuda.synchronize()
    for rep in range(4):
        with torch.cuda.stream(s):
            out_graph.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out_graph), ref), (name, rep)
        assert np.array_equal(_bits(K), k_ref) and np.array_equal(_bits(V), v_ref), (name, rep)
        step(other)                      # eager work between replays, same workspace
        torch.cuda.synchronize()
        assert np.array_equal(_bits(other), ref), (name, rep)


PREFILL_CASES = [
    # name, dtype, Hq, Hkv, d, ctx, qlens, splits
    ("prefill_tiles", "bf16", 16, 2, 128, [0, 300, 700], [40, 33, 130], 1),
    ("prefill_tiles_split", "bf16", 16, 2, 128, [0, 300, 700], [40, 33, 130], 3),
    ("prefill_short_auto", "bf16", 64, 8, 128, [2000, 700, 3], [4, 4, 4], 0),
    ("prefill_short_fp8_auto", "fp8", 64, 8, 128, [2000, 700, 3], [4, 4, 4], 0),
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_prefill_graph_replay_matches_eager(case):
    """pa_prefill (append through the tables, attention, and the merge of split
    partials) captured in a HIP graph: every replay gives the eager bits, with
    eager prefills into another buffer, sharing the workspace, between replays."""
    need_gpu()
    from tests.test_gpu_prefill import make_prefill_batch
    from tests.test_gpu_prefill_fp8 import make_fp8_prefill
    name, dtype, Hq, Hkv, d, ctx, qlens, splits = case
    print_case(test="prefill_graph_replay", case=name)
    if dtype == "fp8":
        b = make_fp8_prefill(Hq, Hkv, d, ctx, qlens, seed=73)
        b["L"] = 1
    else:
        b = make_prefill_batch(Hq, Hkv, d, ctx, qlens, seed=73)
    geom = pk.Geometry(1, Hkv, d, 16, b["N"], dtype)
    n, n_tok = len(qlens), int(sum(qlens))
    max_q, max_ctx = int(max(qlens)), int(max(c + q for c, q in zip(ctx, qlens)))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        if dtype == "fp8":
            K = torch.from_numpy(np.ascontiguousarray(b["kp"])).cuda()
            V = torch.from_numpy(np.ascontiguousarray(b["vp"])).cuda()
        else:
            K, V = to_dev(b["kp"], "bf16"), to_dev(b["vp"], "bf16")
        q = to_dev(b["q"], "bf16")
        kn, vn = to_dev(b["kn"], "bf16"), to_dev(b["vn"], "bf16")
        qs = torch.from_numpy(b["q_start"]).cuda()
        tabs = torch.from_numpy(padded_tables(b["tables"], max(len(t) for t in b["tables"]))).cuda()
        cl = torch.from_numpy(b["ctx"]).cuda()
        need = pk.prefill_workspace_bytes(geom, n, n_tok, Hq, max_q, max_ctx, splits)
        ws = torch.empty(max(1, need), dtype=torch.uint8, device="cuda")
        out_eager = torch.empty_like(q)
        out_graph = torch.full_like(q, float("nan"))
        other = torch.empty_like(q)

    def call(out):
        pk.prefill(geom, K, V, 0, q, kn, vn, out, qs, tabs, cl, max_q, max_ctx, stream=s,
                   splits=splits, workspace=ws)

    call(out_eager)
    torch.cuda.synchronize()
    ref, k_ref, v_ref = _bits(out_eager), _bits(K), _bits(V)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(out_graph)
    torch.cuda.synchronize()
    for rep in range(4):
        with torch.cuda.stream(s):
            out_graph.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out_graph), ref), (name, rep)
        assert np.array_equal(_bits(K), k_ref) and np.array_equal(_bits(V), v_ref), (name, rep)
        call(other)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(other), ref), (name, rep)
