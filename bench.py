#!/usr/bin/env python3
"""Paged-KV decode benchmark on one MI355X.

Default workload (the headline): the 70B grouped-query geometry at 32K context
(80 layers, 64 query / 8 KV heads, head dim 128, bf16, 16-slot blocks), 16
sequences of 32,768 attended tokens in a 32,768-block pool (171.8 GB) with a
seeded random physical block order. A step = for every layer, pa_append_kv of
the batch's new keys/values, then pa_decode (split-K partial + combine). Inputs
are resident in HBM before the timed region starts. Prints one JSON line whose
`value` is KV bytes read per second (sum over sequences of attended tokens x
bytes per token, all layers).

Other workloads (--config): gpt2_fp32 and chat_ragged run the same decode step;
fork_cow times copy-on-write copies + bulk suffix append + decode; offload
times the gather -> host -> scatter round trip of half of each trajectory and
checks that decode is bitwise identical before and after; offload_overlap runs
the headline decode batch while one more trajectory goes to pinned host memory
and back through the asynchronous swapper; prefill_chunks times chunked
prefill; prefix_reuse serves requests that share a cached system prompt through
the radix prefix cache and prefills only their novel tokens.
"""

from __future__ import annotations

import argparse
import contextlib
import gc
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

PEAK_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0   # dense bf16 matrix-core peak of the part
METRIC = "paged-decode KV GB/s (% of HBM peak) + decode tokens/s, 70B-GQA 32K ctx"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="gqa70b_32k")
    ap.add_argument("--bps", type=int, default=0, help="blocks per split (0 = library default)")
    ap.add_argument("--kernel", default="auto", choices=["auto", "generic", "mfma", "valu"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=48,
                    help="(sequence, layer) pairs the oracle times for the CPU baseline")
    ap.add_argument("--no-prof", action="store_true", help="do not record per-kernel events")
    ap.add_argument("--prof-every", type=int, default=8,
                    help="record kernel events around the decode of every k-th layer")
    ap.add_argument("--cold", action="store_true",
                    help="also time steps after writing a 1 GiB buffer (flushes L2 and MALL)")
    ap.add_argument("--cold-only", action="store_true",
                    help="decode / fork workloads: run only the cold steps (for counter passes)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a 1 GiB device copy (for scaling HBM byte counters)")
    ap.add_argument("--parity-samples", type=int, default=4)
    ap.add_argument("--pf-splits", type=int, default=0,
                    help="prefill key splits (0 = library's choice, 1 = none)")
    ap.add_argument("--no-baseline-leg", action="store_true",
                    help="prefix_reuse: skip the no-reuse comparison leg")
    ap.add_argument("--checked-calls", action="store_true",
                    help="decode: check and marshal every layer's call (decode_step) instead of "
                         "preparing each layer's call once (prepare_decode_step)")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step in a HIP graph and time its replays")
    ap.add_argument("--unfused", action="store_true",
                    help="append the step's tokens with a separate launch before each decode")
    ap.add_argument("--wg-waves", type=int, default=0,
                    help="streaming VALU kernel: waves per workgroup (0 = library default)")
    ap.add_argument("--merge", default="auto", choices=["auto", "on", "off"],
                    help="merge decode splits inside the decode launch (auto: for the streaming "
                         "VALU kernel, where it is faster; the MFMA kernels' last split would "
                         "merge all eight heads serially, slower than the combine launch)")
    ap.add_argument("--no-merge", action="store_true", help="same as --merge off")
    ap.add_argument("--kv-reuse", action="store_true",
                    help="decode workloads: cached instead of non-temporal K/V loads")
    ap.add_argument("--no-ragged", action="store_true",
                    help="do not give the library the host copy of the lengths (no ragged plan)")
    ap.add_argument("--chunk-blocks", type=int, default=-1,
                    help="offload_overlap: blocks per staging chunk (-1 = the workload's, 0 = library default)")
    ap.add_argument("--move-wgs", type=int, default=0,
                    help="offload_overlap: work-groups per swap gather/scatter launch (0 = library default)")
    ap.add_argument("--offload-fraction", type=float, default=1.0,
                    help="offload workload: fraction of the chosen blocks moved (host RAM bound)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_sha(kernel: str) -> str:
    """sha256 prefix of a kernel's source: for the bf16 matrix-core decode kernel
    its section of pa_kernels.hip (from its banner to the generic kernel's), for
    the streaming VALU and FP8 decode kernels their headers, for the prefill tile
    kernel pa_prefill.hip, each with the device and pair-load helpers. Edits
    elsewhere leave it unchanged."""
    here = os.path.dirname(os.path.abspath(__file__))
    csrc = os.path.join(here, "paged_kv_cache_83_amd", "csrc")
    h = hashlib.sha256()
    if kernel == "decode_mfma_bf16_kernel":
        text = open(os.path.join(csrc, "pa_kernels.hip"), "rb").read()
        h.update(text[text.index(b"// Decode, MFMA kernel:"):text.index(b"// Decode, generic kernel")])
    elif kernel == "decode_valu_kernel":
        h.update(open(os.path.join(csrc, "pa_valu.h"), "rb").read())
    elif kernel == "decode_mfma_fp8_kernel":
        h.update(open(os.path.join(csrc, "pa_fp8.h"), "rb").read())
    elif kernel == "prefill_mfma_kernel":
        h.update(open(os.path.join(csrc, "pa_prefill.hip"), "rb").read())
    else:
        raise ValueError(kernel)
    h.update(open(os.path.join(csrc, "pa_device.h"), "rb").read())
    h.update(open(os.path.join(csrc, "pa_pairs.h"), "rb").read())
    return h.hexdigest()[:16]


def profiled_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary of this
    kernel on this workload (FETCH_SIZE and WRITE_SIZE, scaled by a 1 GiB copy),
    or None when there is none or the kernel source has changed since."""
    here = os.path.dirname(os.path.abspath(__file__))
    stem = kernel[:-len("_kernel")]
    path = next((p for p in (os.path.join(here, "profiles", f"{stem}_{workload}_{kind}.md")
                             for kind in ("hbm_counters", "counters")) if os.path.exists(p)), None)
    if path is None:
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.split(":", 1)[0].strip() in ("source_sha256_prefix", "traffic_bytes_per_launch"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("source_sha256_prefix") != kernel_source_sha(kernel) or \
            "traffic_bytes_per_launch" not in fields:
        return None
    return int(fields["traffic_bytes_per_launch"])


def calibrate_copy():
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    dst.copy_(src)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n,
                      "seconds": dt, "GB_per_s_rw": 2 * n / dt / 1e9}), flush=True)


class Timer:
    """Times a region on one stream with hipEvents (torch.cuda.Event records on
    the stream passed in, which is the stream every library call uses)."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def __enter__(self):
        self.torch.cuda.synchronize()
        self.t0 = time.perf_counter()
        self.a = self.torch.cuda.Event(enable_timing=True)
        self.b = self.torch.cuda.Event(enable_timing=True)
        self.a.record(self.stream)
        return self

    def __exit__(self, *exc):
        self.b.record(self.stream)
        self.torch.cuda.synchronize()
        self.wall_ms = (time.perf_counter() - self.t0) * 1e3
        self.ms = max(self.a.elapsed_time(self.b), 0.0)
        return False


class StepTimes:
    """hipEvents between consecutive steps on one stream: per-step median, min, max."""

    def __init__(self, torch, stream, n):
        self.stream = stream
        self.ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        self.i = 0

    def mark(self):
        self.ev[self.i].record(self.stream)
        self.i += 1

    def summary(self):
        ms = sorted(self.ev[k].elapsed_time(self.ev[k + 1]) for k in range(self.i - 1))
        if not ms:
            return None
        return {"median": round(ms[len(ms) // 2], 4), "min": round(ms[0], 4), "max": round(ms[-1], 4)}


def make_runner(torch, stream, step, use_graph):
    """Returns a callable running one step: `step` itself, or the replay of a
    HIP graph holding one captured step (captured after the eager warm-up)."""
    if not use_graph:
        return step
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        step()
    torch.cuda.synchronize()
    log("captured one step in a HIP graph")
    return g.replay


def timed_steps(torch, stream, run, steps):
    st = StepTimes(torch, stream, steps)
    with Timer(torch, stream) as t:
        for _ in range(steps):
            st.mark()
            run()
        st.mark()
    return t, st.summary()


def setup(args):
    import torch
    import paged_kv_cache_83_amd as pk
    from synth import get_config
    cfg = get_config(args.config)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    # one ordinary (default-priority) stream for all work: graph capture needs a
    # stream other than the legacy default one
    stream = torch.cuda.Stream(dev)
    torch.cuda.set_stream(stream)
    geom = pk.Geometry(cfg.num_layers, cfg.num_kv_heads, cfg.head_dim, cfg.block_size,
                       cfg.num_blocks, cfg.dtype)
    log(f"config={cfg.name} L={cfg.num_layers} n={cfg.num_seqs} Hq={cfg.num_q_heads} "
        f"Hkv={cfg.num_kv_heads} d={cfg.head_dim} B={cfg.block_size} N={cfg.num_blocks} "
        f"dtype={cfg.dtype} pool={2 * pk.pool_bytes(geom) / 1e9:.1f} GB")
    gen_ = torch.Generator(device=dev)
    gen_.manual_seed(cfg.seed)
    k_pool, v_pool = pk.alloc_pools(geom, dev)
    if cfg.dtype == "fp8":
        fill_fp8_pools(torch, pk, geom, gen_, k_pool, v_pool, dev)
    else:
        k_pool.normal_(generator=gen_)
        v_pool.normal_(generator=gen_)
    return torch, pk, cfg, dev, stream, geom, gen_, k_pool, v_pool


def fp8_tile_order(B: int, d: int, is_k: bool) -> np.ndarray:
    """For each code byte of a one-byte tile, the (slot * d + dim) it holds: the
    tile order include/pa.h documents (B = 16: K rows of 64 codes in slot order
    0-3, 8-11, 4-7, 12-15, a row's 8-dim groups in the order 0, 4, 1, 5, 2, 6, 3,
    7; V [d/32][slot/8][dim%16][(dim/16)%2][slot%8]; else the bf16 orders)."""
    o = np.arange(B)[:, None]
    j = np.arange(d)[None, :]
    if is_k and B == 16 and d % 64 == 0:
        r = (o & ~12) | ((o >> 1) & 4) | ((o << 1) & 8)
        pos = 1024 * (j // 64) + 64 * r + 16 * ((j // 8) % 4) + 8 * ((j // 32) % 2) + j % 8
    elif is_k:
        W = 32 if d % 32 == 0 else d
        pos = (j // W) * B * W + o * W + j % W
    elif B == 16 and d % 32 == 0:
        pos = 512 * (j // 32) + 256 * (o // 8) + 16 * (j % 16) + 8 * ((j // 16) % 2) + o % 8
    else:
        pos = j * B + o
    order = np.empty(B * d, np.int64)
    order[np.broadcast_to(pos, (B, d)).reshape(-1)] = (o * d + j).reshape(-1)
    return order


def fill_fp8_pools(torch, pk, geom, gen_, k_pool, v_pool, dev, chunk_blocks=8192):
    """Every slot of an FP8 pool gets seeded N(0,1) K/V rows (rounded to bf16),
    quantized with plain torch operations on the device: per (token, head) the
    power-of-two scale 2^e with e the smallest integer such that max|x| <= 448 * 2^e,
    torch's float8_e4m3fn cast of x * 2^-e, the byte e + 127, laid out in the pool's
    documented tile format (the codes in the order of fp8_tile_order, then the B
    scale bytes). The pools are input data: neither the library nor the oracle
    writes them."""
    L, N, H, B, d = (geom.num_layers, geom.num_blocks, geom.num_kv_heads, geom.block_size,
                     geom.head_dim)
    order = {is_k: torch.from_numpy(fp8_tile_order(B, d, is_k)).to(dev) for is_k in (True, False)}
    for layer in range(L):
        for b0 in range(0, N, chunk_blocks):
            nb = min(chunk_blocks, N - b0)
            for pool, is_k in ((k_pool, True), (v_pool, False)):
                x = torch.randn((nb, B, H, d), generator=gen_, device=dev).to(torch.bfloat16).float()
                amax = x.abs().amax(-1)
                m, ex = torch.frexp(amax)
                e = torch.where(m <= 0.875, ex - 9, ex - 8).clamp(-127, 127)
                e = torch.where(amax == 0, torch.zeros_like(e), e)
                codes = (x * torch.exp2(-e.float()).unsqueeze(-1)).to(torch.float8_e4m3fn)
                codes = codes.view(torch.uint8).permute(0, 2, 1, 3).reshape(nb, H, B * d)
                pool[layer, b0:b0 + nb, :, :B * d] = codes.index_select(2, order[is_k])
                pool[layer, b0:b0 + nb, :, B * d:] = (e + 127).to(torch.uint8).permute(0, 2, 1)
    if k_pool.is_cuda:
        torch.cuda.synchronize()


def to_np(torch, t, dtype):
    t = t.contiguous().cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if dtype == "bf16" else t.numpy()


# =============================================================================
# Decode workloads (gqa70b_32k, gpt2_fp32, chat_ragged)
# =============================================================================
def run_decode(args):
    torch, pk, cfg, dev, stream, geom, gen_, k_pool, v_pool = setup(args)
    from paged_kv_cache_83_amd import steps
    from synth import gen
    L, n, Hq, Hkv, d, B = (cfg.num_layers, cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads,
                           cfg.head_dim, cfg.block_size)
    lengths = gen.context_lengths(cfg)
    fp8 = cfg.dtype == "fp8"
    # bytes of K and V per token over all layers (FP8: plus one scale byte per head, K and V)
    m_token = pk.bytes_per_block(geom) // B
    io = geom.io_dtype
    q_all = torch.randn((L, n, Hq, d), generator=gen_, device=dev).to(io)
    k_new = torch.randn((L, n, Hkv, d), generator=gen_, device=dev).to(io)
    v_new = torch.randn((L, n, Hkv, d), generator=gen_, device=dev).to(io)

    # host block bookkeeping: history, then the decode step's one new token each
    bm = pk.BlockManager(cfg.num_blocks, B, gen.free_order(cfg))
    seqs = [bm.seq_new() for _ in range(n)]
    for s, S in zip(seqs, lengths):
        bm.append(s, int(S) - 1)
    slots_np, cow = bm.append_batch(seqs, [1] * n)
    assert not cow
    max_blocks = max(bm.info(s)[1] for s in seqs)
    tables_np, lens_np = bm.build_tables(seqs, max_blocks)
    assert np.array_equal(lens_np, lengths)
    slots = torch.from_numpy(slots_np).to(dev)
    tables = torch.from_numpy(np.ascontiguousarray(tables_np)).to(dev)
    lens = torch.from_numpy(np.ascontiguousarray(lens_np)).to(dev)
    max_ctx = int(lengths.max())
    out = torch.empty((L, n, Hq, d), dtype=io, device=dev)
    valu_path = args.kernel == "valu" or (args.kernel == "auto" and cfg.dtype == "f32")
    merge = (not args.no_merge and args.merge != "off") and (args.merge == "on" or valu_path)
    host_lens = None if args.no_ragged else np.asarray(lens_np, np.int32)
    ws_bytes = pk.decode_workspace_bytes(geom, n, Hq, max_ctx, args.bps, args.kernel, merge,
                                         args.wg_waves, host_lens)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)   # merge counters start at 0
    torch.cuda.synchronize()

    # host copies of the sampled sequences' blocks, before any library kernel writes the pool
    rng = np.random.default_rng(cfg.seed)
    samples = [(int(rng.integers(0, n)), int(rng.integers(0, L))) for _ in range(args.parity_samples)]
    snap = {}

    def take_snapshot(i, layer):
        ids = torch.from_numpy(np.asarray(tables_np[i, :math.ceil(lengths[i] / B)], np.int64)).to(dev)
        snap[(i, layer)] = (k_pool[layer].index_select(0, ids).cpu(),
                            v_pool[layer].index_select(0, ids).cpu(), ids.cpu().numpy())

    for key in samples:
        take_snapshot(*key)

    profiling = [False]

    def around(layer, before):
        if profiling[0] and layer % args.prof_every == 0:
            pk.Profiler.enable(before)

    def step():
        steps.decode_step(geom, k_pool, v_pool, q_all, k_new, v_new, slots, tables, lens, max_ctx, out,
                          ws, blocks_per_split=args.bps, kernel=args.kernel, stream=stream,
                          around_decode=around, fused=not args.unfused, merge=merge,
                          waves_per_group=args.wg_waves, host_lens=host_lens,
                          kv_reuse=args.kv_reuse)

    if not args.unfused and not args.checked_calls:
        # the same fused step with each layer's call checked and marshalled once
        step = steps.prepare_decode_step(geom, k_pool, v_pool, q_all, k_new, v_new, tables, lens,
                                         max_ctx, out, ws, blocks_per_split=args.bps,
                                         kernel=args.kernel, stream=stream, around_decode=around,
                                         kv_reuse=args.kv_reuse, merge=merge,
                                         waves_per_group=args.wg_waves, host_lens=host_lens)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")
    run = make_runner(torch, stream, step, args.graph)
    if args.graph:
        run()

    if not args.no_prof and not args.graph:
        pk.Profiler.reset()
        profiling[0] = True
    if args.cold_only:
        args.cold = True
    else:
        t, step_ms = timed_steps(torch, stream, run, args.steps)
        profiling[0] = False
        ms_per_step = max(t.ms, t.wall_ms) / args.steps
        log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step {step_ms}")

    cold = None
    if args.cold:
        flush = torch.zeros(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        tot = 0.0
        for _ in range(args.steps):
            flush.add_(1.0)
            with Timer(torch, stream) as tc:
                run()
            tot += tc.ms
        cold = tot / args.steps
        log(f"cold (1 GiB written before each step): {cold:.3f} ms/step")
        if args.cold_only:
            profiling[0] = False
            ms_per_step, step_ms = cold, None

    kv_bytes_step = int(lengths.sum()) * m_token
    value = kv_bytes_step / (ms_per_step * 1e-3) / 1e9

    # ---- roofline of the dominant kernel (decode partial), timed live ----------
    roofline, kernel_ms = None, {}
    if not args.no_prof and not args.graph:
        for name in ("decode_partial", "decode_combine", "append"):
            cnt, tot = pk.Profiler.read(name)
            if cnt:
                kernel_ms[name] = {"launches": cnt, "avg_us": 1e3 * tot / cnt}
        cnt, tot = pk.Profiler.read("decode_partial")
        if cnt:
            eb = geom.elem_bytes
            ib = 2 if fp8 else eb                                                # q / out element bytes
            # what the step must move; split partials (the launch plan's choice)
            # are left out, so they show up only in the measured traffic
            per_launch = (int(lengths.sum()) * 2 * Hkv * (d * eb + (1 if fp8 else 0))  # K and V (+ scales)
                          + 2 * n * Hq * d * ib                                  # queries, outputs
                          + 4 * int(sum(math.ceil(S / B) for S in lengths))       # block-table entries
                          + (0 if args.unfused                                   # fused new K/V:
                             else 2 * n * Hkv * (2 * d + d + 1) if fp8           # bf16 rows in, codes + scale out
                             else 4 * n * Hkv * d * eb))                          # rows in, rows out
            avg_s = tot / cnt * 1e-3
            achieved = per_launch / avg_s / 1e9
            mfma = cfg.dtype in ("bf16", "fp8") and B == 16 and args.kernel in ("auto", "mfma")
            valu = not mfma and B == 16 and d in (64, 128) and Hq // Hkv in (1, 2, 4, 8) \
                and args.kernel in ("auto", "valu")
            kname = (("decode_mfma_fp8_kernel" if fp8 else "decode_mfma_bf16_kernel") if mfma
                     else "decode_valu_kernel" if valu else "decode_generic_kernel")
            roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / PEAK_GBS, 4),
                        "traffic": profiled_traffic(kname, cfg.name) if (args.bps == 0 and args.kernel == "auto"
                                                                        and not args.unfused) else None,
                        "kernel": kname,
                        "bytes_per_launch": per_launch, "avg_launch_us": round(avg_s * 1e6, 2)}

    # ---- parity on sampled (sequence, layer) outputs against the oracle ---------
    parity, cpu_baseline = None, None
    if args.parity_samples or not args.no_cpu_baseline:
        from oracle import attention as oatt
        from oracle import block_manager as obm
        from oracle import kv_ops as okv
        om = obm.BlockManager(cfg.num_blocks, B, gen.free_order(cfg))
        oseqs = []
        for S in lengths:
            s = om.seq_new()
            om.append(s, int(S) - 1)
            oseqs.append(s)
        oslots = [om.append(s, 1)[0][0] for s in oseqs]
        otables = [om.table(s) for s in oseqs]

        from oracle import fp8 as ofp8
        io_name = "bf16" if fp8 else cfg.dtype

        def oracle_one(i, layer):
            kb, vb, ids = snap[(i, layer)]
            kloc, vloc = to_np(torch, kb, cfg.dtype)[None], to_np(torch, vb, cfg.dtype)[None]
            remap = {int(p): j for j, p in enumerate(ids)}
            table = [remap[p] for p in otables[i]]
            slot = remap[oslots[i] // B] * B + oslots[i] % B
            kn = to_np(torch, k_new[layer, i:i + 1], io_name)
            vn = to_np(torch, v_new[layer, i:i + 1], io_name)
            q = to_np(torch, q_all[layer, i:i + 1], io_name)
            if fp8:
                kloc, vloc = ofp8.append_kv(kloc, vloc, 0, kn, vn, [slot], B)
                return ofp8.paged_decode(q, kloc, vloc, 0, [table], [int(lengths[i])], B)[0]
            kloc, vloc = okv.append_kv(kloc, vloc, 0, kn, vn, [slot], B)
            return oatt.paged_decode(q, kloc, vloc, 0, [table], [int(lengths[i])], B, cfg.dtype)[0]

        errs = []
        for (i, layer) in samples:
            expect = oracle_one(i, layer)
            got = out[layer, i].float().cpu().numpy().astype(np.float64)
            errs.append(float(np.max(np.abs(got - expect))))
        tol = 1e-5 if cfg.dtype == "f32" else 2e-2
        if errs:
            parity = {"samples": len(errs), "max_abs_err": max(errs), "tol": tol, "ok": max(errs) <= tol}
            log(f"parity {parity}")

        if not args.no_cpu_baseline:
            try:
                from threadpoolctl import threadpool_limits
            except Exception:  # pragma: no cover
                threadpool_limits = None
            cores = len(os.sched_getaffinity(0))
            # the FP8 oracle dequantizes every tile in numpy (~4.5 s per 32K-token pair)
            n_pairs = max(2, args.cpu_sample // 12) if fp8 else args.cpu_sample
            pairs = [(int(rng.integers(0, n)), int(rng.integers(0, L))) for _ in range(n_pairs)]
            for key in pairs:
                if key not in snap:
                    take_snapshot(*key)
            limiter = threadpool_limits(limits=cores) if threadpool_limits else contextlib.nullcontext()
            with limiter:
                t0 = time.perf_counter()
                for (i, layer) in pairs:
                    oracle_one(i, layer)
                cpu_s = time.perf_counter() - t0
            step_s = cpu_s / len(pairs) * n * L
            cpu_baseline = {"value": round(kv_bytes_step / step_s / 1e9, 4), "unit": "GB/s", "cores": cores,
                            "kind": "oracle", "tokens_per_s": round(n / step_s, 4),
                            "sample": f"{len(pairs)} (sequence, layer) decodes of this workload timed in "
                                      f"{cpu_s:.1f} s, scaled to the {n}-sequence x {L}-layer step"}

    result = {
        "metric": METRIC if cfg.name == "gqa70b_32k" else f"paged-decode KV GB/s + tokens/s, {cfg.name}",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) Q/K/V, seeded random block placement)",
        "config": {"workload": cfg.name, "num_layers": L, "num_q_heads": Hq, "num_kv_heads": Hkv,
                   "head_dim": d, "block_size": B, "num_seqs": n, "context_len": int(lengths.max()),
                   "pool_blocks": cfg.num_blocks, "kv_bytes_per_step": kv_bytes_step,
                   "global_batch": n, "seq_len": int(lengths.max()), "parallelism": "none (1 GPU)",
                   "append": "separate launch" if args.unfused else "fused into decode",
                   "split_merge": ("none (every sequence in one split)" if ws_bytes == 0
                                   else "inside the decode launch (where splits exist)" if merge
                                   else "separate launch"),
                   "launch": ("hip graph replay" if args.graph
                              else "eager, calls checked per call" if args.unfused or args.checked_calls
                              else "eager, calls prepared once")},
        "step_ms": step_ms,
        "tokens_per_s": round(n / (ms_per_step * 1e-3), 2),
        "pct_hbm_peak": round(100 * value / PEAK_GBS, 2),
        "roofline": roofline,
        "cpu_baseline": cpu_baseline,
        "kernels": kernel_ms,
        "kernels_timing": ("every {}th layer's launches, from a start event the library records "
                           "on the launch stream before the kernel to a stop event the kernel's "
                           "own launch takes at its end (hipExtLaunchKernelGGL)"
                           .format(args.prof_every)) if kernel_ms else None,
        "parity": parity,
    }
    if cold is not None:
        result["cold_ms_per_step"] = round(cold, 4)
        result["cold_value"] = round(kv_bytes_step / (cold * 1e-3) / 1e9, 2)
    print(json.dumps(result), flush=True)


# =============================================================================
# Fork + copy-on-write workload
# =============================================================================
def run_fork(args):
    torch, pk, cfg, dev, stream, geom, gen_, k_pool, v_pool = setup(args)
    from paged_kv_cache_83_amd import steps
    from synth import gen
    L, Hq, Hkv, d, B = cfg.num_layers, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size
    n = cfg.num_seqs
    suffix = gen.suffix_lengths(cfg)
    lengths = gen.context_lengths(cfg)
    bm = pk.BlockManager(cfg.num_blocks, B, gen.free_order(cfg))
    parent = bm.seq_new()
    bm.append(parent, cfg.prefix_len)
    branches = [bm.fork(parent) for _ in range(n)]
    bulk_slots, pairs = [], []
    for b, m in zip(branches, suffix):
        s, p = bm.append(b, int(m) - 1)
        bulk_slots.append(s)
        pairs += p
    dec_slots, cow = bm.append_batch(branches, [1] * n)
    assert len(pairs) == n and not cow
    bulk = torch.from_numpy(np.concatenate(bulk_slots)).to(dev)
    n_bulk = bulk.numel()
    max_blocks = max(bm.info(b)[1] for b in branches)
    tables_np, lens_np = bm.build_tables(branches, max_blocks)
    assert np.array_equal(lens_np, lengths)
    tables = torch.from_numpy(np.ascontiguousarray(tables_np)).to(dev)
    lens = torch.from_numpy(np.ascontiguousarray(lens_np)).to(dev)
    dec = torch.from_numpy(dec_slots).to(dev)
    kb = torch.randn((L, n_bulk, Hkv, d), generator=gen_, device=dev).to(geom.torch_dtype)
    vb = torch.randn((L, n_bulk, Hkv, d), generator=gen_, device=dev).to(geom.torch_dtype)
    q_all = torch.randn((L, n, Hq, d), generator=gen_, device=dev).to(geom.torch_dtype)
    kn = torch.randn((L, n, Hkv, d), generator=gen_, device=dev).to(geom.torch_dtype)
    vn = torch.randn((L, n, Hkv, d), generator=gen_, device=dev).to(geom.torch_dtype)
    out = torch.empty((L, n, Hq, d), dtype=geom.torch_dtype, device=dev)
    max_ctx = int(lengths.max())
    ws = torch.empty(max(1, pk.decode_workspace_bytes(geom, n, Hq, max_ctx)), dtype=torch.uint8, device=dev)
    src = torch.tensor([p[0] for p in pairs], dtype=torch.int32, device=dev)
    dst = torch.tensor([p[1] for p in pairs], dtype=torch.int32, device=dev)

    def step():
        pk.copy_blocks(geom, k_pool, v_pool, src, dst, stream=stream)
        for layer in range(L):
            pk.append_kv(geom, k_pool, v_pool, layer, kb[layer], vb[layer], bulk, stream=stream)
        # the 64 branches share the prefix blocks: keep them cacheable
        steps.decode_step(geom, k_pool, v_pool, q_all, kn, vn, dec, tables, lens, max_ctx, out, ws,
                          stream=stream, kv_reuse=True, fused=not args.unfused)

    for _ in range(args.warmup):
        step()
    run = make_runner(torch, stream, step, args.graph)
    if args.graph:
        run()
    pk.Profiler.reset()
    pk.Profiler.enable(not args.graph and not args.no_prof)
    if not args.cold_only:
        t, step_ms = timed_steps(torch, stream, run, args.steps)
        ms = max(t.ms, t.wall_ms) / args.steps
    cold = None
    if args.cold or args.cold_only:
        flush = torch.zeros(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        tot = 0.0
        for _ in range(args.steps):
            flush.add_(1.0)
            with Timer(torch, stream) as tc:
                run()
            tot += tc.ms
        cold = tot / args.steps
        log(f"cold (1 GiB written before each step): {cold:.3f} ms/step")
        if args.cold_only:
            ms, step_ms = cold, None
    pk.Profiler.enable(False)
    m_token = pk.bytes_per_token(L, Hkv, d, geom.elem_bytes)
    logical = int(lengths.sum()) * m_token
    unique = (cfg.prefix_len + int(suffix.sum())) * m_token
    kern = {}
    for name in ("copy_blocks", "append", "decode_partial", "decode_combine"):
        cnt, tot = pk.Profiler.read(name)
        if cnt:
            kern[name] = {"launches": cnt, "avg_us": round(1e3 * tot / cnt, 2)}
    blk = pk.bytes_per_block(geom)
    copy_gbs = (2 * n * blk) / (kern["copy_blocks"]["avg_us"] * 1e-6) / 1e9 if kern else None
    result = {
        "metric": "fork/copy-on-write step: decode tokens/s and logical KV GB/s, fork_cow",
        "value": round(n / (ms * 1e-3), 2), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "branches": n, "prefix_len": cfg.prefix_len,
                   "suffix_tokens": int(suffix.sum()), "cow_pairs": len(pairs), "num_layers": L},
        "logical_kv_GBps": round(logical / (ms * 1e-3) / 1e9, 1),
        "unique_kv_GBps": round(unique / (ms * 1e-3) / 1e9, 1),
        "copy_blocks_GBps_rw": round(copy_gbs, 1) if copy_gbs else None,
        "step_ms": step_ms,
        "launch": "hip graph replay" if args.graph else "eager",
        "kernels": kern,
    }
    if cold is not None:
        result["cold_ms_per_step"] = round(cold, 4)
        result["cold_logical_kv_GBps"] = round(logical / (cold * 1e-3) / 1e9, 1)
        result["cold_unique_kv_GBps"] = round(unique / (cold * 1e-3) / 1e9, 1)
    print(json.dumps(result), flush=True)


# =============================================================================
# Chunked prefill
# =============================================================================
def run_prefill(args):
    torch, pk, cfg, dev, stream, geom, gen_, k_pool, v_pool = setup(args)
    from synth import gen
    L, n, Hq, Hkv, d, B = (cfg.num_layers, cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads,
                           cfg.head_dim, cfg.block_size)
    C = cfg.chunk_len
    hist = gen.prefill_histories(cfg)
    bm = pk.BlockManager(cfg.num_blocks, B, gen.free_order(cfg))
    seqs = [bm.seq_new() for _ in range(n)]
    for s_, c in zip(seqs, hist):
        if c:
            bm.append(s_, int(c))
        bm.append(s_, C)
    max_blocks = max(bm.info(s_)[1] for s_ in seqs)
    tables_np, lens_np = bm.build_tables(seqs, max_blocks)
    assert np.array_equal(lens_np, hist + C)
    n_tok = n * C
    fp8 = cfg.dtype == "fp8"
    io_name = "bf16" if fp8 else cfg.dtype
    q_all = torch.randn((L, n_tok, Hq, d), generator=gen_, device=dev).to(geom.io_dtype)
    k_all = torch.randn((L, n_tok, Hkv, d), generator=gen_, device=dev).to(geom.io_dtype)
    v_all = torch.randn((L, n_tok, Hkv, d), generator=gen_, device=dev).to(geom.io_dtype)
    out = torch.empty_like(q_all)
    q_start = torch.arange(0, n_tok + 1, C, dtype=torch.int32, device=dev)
    tables = torch.from_numpy(np.ascontiguousarray(tables_np)).to(dev)
    ctx = torch.from_numpy(hist.astype(np.int32)).to(dev)
    max_ctx = int((hist + C).max())
    pf_ws = torch.empty(max(1, pk.prefill_workspace_bytes(geom, n, n_tok, Hq, C, max_ctx,
                                                           args.pf_splits)),
                        dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    profiling = [False]

    def step():
        for layer in range(L):
            prof = profiling[0] and layer % args.prof_every == 0
            if prof:
                pk.Profiler.enable(True)
            pk.prefill(geom, k_pool, v_pool, layer, q_all[layer], k_all[layer], v_all[layer],
                       out[layer], q_start, tables, ctx, C, max_ctx, stream=stream,
                       splits=args.pf_splits, workspace=pf_ws)
            if prof:
                pk.Profiler.enable(False)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    run = make_runner(torch, stream, step, args.graph)
    if args.graph:
        run()
    if not args.no_prof and not args.graph:
        pk.Profiler.reset()
        profiling[0] = True
    t, step_ms = timed_steps(torch, stream, run, args.steps)
    profiling[0] = False
    ms = max(t.ms, t.wall_ms) / args.steps
    # causal attention FLOPs: 2 per multiply-add, QK^T and PV, over the visible keys
    macs_layer = sum(2 * Hq * d * (C * int(c) + C * (C + 1) // 2) for c in hist)
    flops_step = 2 * macs_layer * L
    value = flops_step / (ms * 1e-3) / 1e12
    log(f"timed {args.steps} steps: {ms:.3f} ms/step, {value:.1f} TFLOP/s")

    kern, roofline = {}, None
    if not args.no_prof and not args.graph:
        for name in ("prefill_append", "prefill_attention", "prefill_short", "prefill_combine"):
            cnt, tot = pk.Profiler.read(name)
            if cnt:
                kern[name] = {"launches": cnt, "avg_us": round(1e3 * tot / cnt, 2)}
        # the attention kernel the library chose: 128-row tiles, or one wave per
        # (chunk, KV head, split) for chunks of at most 32 query rows per KV head
        attn = next((k for k in ("prefill_short", "prefill_attention") if k in kern), None)
        kname = {"prefill_short": "prefill_short_kernel",
                 "prefill_attention": "prefill_mfma_kernel"}.get(attn)
        if attn:
            avg_s = kern[attn]["avg_us"] * 1e-6
            # algorithmic bytes of one launch: the visible K/V (history and chunk,
            # pool bytes per token and head), the queries and outputs (bf16)
            kv_tok = 2 * d * (1 if fp8 else geom.elem_bytes) + (2 if fp8 else 0)
            bytes_layer = int(sum(int(c) + C for c in hist)) * Hkv * kv_tok + 2 * n_tok * Hq * d * 2
            flops_layer = 2 * macs_layer
            if flops_layer / bytes_layer >= PEAK_BF16_TFLOPS * 1e12 / (PEAK_GBS * 1e9):
                ach = flops_layer / avg_s / 1e12
                roofline = {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
                            "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                            "traffic": profiled_traffic(kname, cfg.name) if args.pf_splits == 0
                            else None, "kernel": kname,
                            "flops_per_launch": flops_layer, "avg_launch_us": round(avg_s * 1e6, 2)}
            else:
                ach = bytes_layer / avg_s / 1e9
                roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_GBS,
                            "unit": "GB/s", "frac": round(ach / PEAK_GBS, 4), "traffic": None,
                            "kernel": kname, "bytes_per_launch": bytes_layer,
                            "avg_launch_us": round(avg_s * 1e6, 2)}
            if "prefill_combine" in kern:
                roofline["combine_avg_us"] = kern["prefill_combine"]["avg_us"]

    # parity on sampled (chunk, layer) outputs; cpu baseline = the oracle on a sample
    parity, cpu_baseline = None, None
    if args.parity_samples or not args.no_cpu_baseline:
        from oracle import prefill as opf
        from oracle import fp8 as ofp8
        from oracle import block_manager as obm
        om = obm.BlockManager(cfg.num_blocks, B, gen.free_order(cfg))
        otables = []
        for c in hist:
            s_ = om.seq_new()
            if c:
                om.append(s_, int(c))
            om.append(s_, C)
            otables.append(om.table(s_))
        rng = np.random.default_rng(cfg.seed)

        def oracle_one(i, layer):
            # the chunk's history is untouched by the step (it writes positions
            # hist[i] .. hist[i]+C-1 only), so the pool after the run serves
            ids = otables[i]
            idx = torch.as_tensor(ids, dtype=torch.long, device=dev)
            rows = slice(i * C, (i + 1) * C)
            qs = np.array([0, C], dtype=np.int64)
            qr, kr, vr = (to_np(torch, x[layer, rows], io_name) for x in (q_all, k_all, v_all))
            if fp8:   # pool bytes as filled (torch), the chunk quantized by the oracle itself
                kb = k_pool[layer].index_select(0, idx).cpu().numpy()[None]
                vb = v_pool[layer].index_select(0, idx).cpu().numpy()[None]
                _, _, o = ofp8.paged_prefill(qr, kr, vr, kb, vb, 0, [list(range(len(ids)))], qs,
                                             [int(hist[i])], B)
                return o
            kb = to_np(torch, k_pool[layer].index_select(0, idx), cfg.dtype)[None]
            vb = to_np(torch, v_pool[layer].index_select(0, idx), cfg.dtype)[None]
            _, _, o = opf.paged_prefill(qr, kr, vr, kb, vb, 0, [list(range(len(ids)))], qs,
                                        [int(hist[i])], B, cfg.dtype)
            return o

        errs = []
        for _ in range(args.parity_samples):
            i, layer = int(rng.integers(0, n)), int(rng.integers(0, L))
            expect = oracle_one(i, layer)
            got = out[layer, i * C:(i + 1) * C].float().cpu().numpy().astype(np.float64)
            scale_ = np.maximum(1.0, np.max(np.abs(expect), axis=-1, keepdims=True)) if fp8 else 1.0
            errs.append(float(np.max(np.abs(got - expect) / scale_)))
        if errs:
            parity = {"samples": len(errs), ("max_rel_err" if fp8 else "max_abs_err"): max(errs),
                      "tol": 2e-2, "ok": max(errs) <= 2e-2}
            log(f"parity {parity}")
        if not args.no_cpu_baseline:
            try:
                from threadpoolctl import threadpool_limits
            except Exception:  # pragma: no cover
                threadpool_limits = None
            cores = len(os.sched_getaffinity(0))
            pairs = [(int(rng.integers(0, n)), int(rng.integers(0, L))) for _ in range(args.cpu_sample // 8)]
            limiter = threadpool_limits(limits=cores) if threadpool_limits else contextlib.nullcontext()
            with limiter:
                t0 = time.perf_counter()
                flops = 0
                for (i, layer) in pairs:
                    oracle_one(i, layer)
                    flops += 4 * Hq * d * (C * int(hist[i]) + C * (C + 1) // 2)
                cpu_s = time.perf_counter() - t0
            cpu_baseline = {"value": round(flops / cpu_s / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
                            "kind": "oracle", "tokens_per_s": round(len(pairs) * C / cpu_s / L, 4),
                            "sample": f"{len(pairs)} (chunk, layer) prefills of this workload timed in "
                                      f"{cpu_s:.1f} s; rate in causal attention FLOP/s"}

    result = {
        "metric": f"chunked-prefill attention TFLOP/s (causal) + prefill tokens/s, {cfg.name}",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) Q/K/V, seeded random block placement"
                + (", history quantized to E4M3 by torch)" if fp8 else ")"),
        "config": {"workload": cfg.name, "num_layers": L, "num_q_heads": Hq, "num_kv_heads": Hkv,
                   "head_dim": d, "block_size": B, "num_seqs": n, "chunk_len": C,
                   "histories": sorted(set(int(c) for c in hist)), "prompt_len": cfg.length_max,
                   "splits": args.pf_splits,
                   "launch": "hip graph replay" if args.graph else "eager"},
        "step_ms": step_ms,
        "tokens_per_s": round(n_tok / (ms * 1e-3), 1),
        "roofline": roofline,
        "cpu_baseline": cpu_baseline,
        "kernels": kern,
        "parity": parity,
    }
    print(json.dumps(result), flush=True)


# =============================================================================
# Offload round trip
# =============================================================================
def alloc_pinned_passes(torch, n_seqs, cols, per, max_passes=16):
    """The largest pinned host buffer that allocates for a round trip of
    n_seqs x cols blocks of `per` bytes: all of them in one pass, else the
    blocks of ceil(cols / P) columns per sequence for P = 2, 3, ... Returns
    (buffer, passes, columns per pass, the refused requests in bytes). torch
    rounds a pinned request up to a power of two, so the bytes pinned are that
    rounding of the request."""
    refused = []
    for passes in range(1, max_passes + 1):
        cpp = -(-cols // passes)
        want = n_seqs * cpp * per
        t0 = time.perf_counter()
        try:
            host = torch.empty(want, dtype=torch.uint8, pin_memory=True)
        except RuntimeError:
            refused.append(want)
            log(f"pinned request of {want / 2**30:.1f} GiB refused")
            continue
        log(f"pinned {want / 2**30:.1f} GiB in {time.perf_counter() - t0:.1f} s: {passes} pass(es)")
        return host, passes, cpp, refused
    raise RuntimeError("no pinned host buffer allocates for the round trip")


def run_offload(args):
    """Config-5 round trip at its stated size: a seeded 50% of each of the four
    131,072-token trajectories' blocks (16,384 blocks, 80 GiB) goes through
    gather -> device-to-host -> release -> re-allocation from a reshuffled free
    list -> host-to-device -> scatter, in as many passes as the largest pinned
    buffer the machine grants requires; then all 80 layers are decoded again."""
    torch, pk, cfg, dev, stream, geom, gen_, k_pool, v_pool = setup(args)
    from paged_kv_cache_83_amd import steps
    from synth import gen
    from oracle import attention as oatt
    from oracle import kv_ops as okv
    L, Hq, Hkv, d, B, n = (cfg.num_layers, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                           cfg.block_size, cfg.num_seqs)
    lengths = gen.context_lengths(cfg)
    bm = pk.BlockManager(cfg.num_blocks, B, gen.free_order(cfg))
    seqs = [bm.seq_new() for _ in range(n)]
    for s, S in zip(seqs, lengths):
        bm.append(s, int(S) - 1)
    bm.append_batch(seqs, [1] * n)
    q_all = torch.randn((L, n, Hq, d), generator=gen_, device=dev).to(geom.torch_dtype)
    kn = torch.randn((L, n, Hkv, d), generator=gen_, device=dev).to(geom.torch_dtype)
    vn = torch.randn((L, n, Hkv, d), generator=gen_, device=dev).to(geom.torch_dtype)
    max_ctx = int(lengths.max())
    lens = torch.from_numpy(lengths.astype(np.int32)).to(dev)
    ws = torch.empty(max(1, pk.decode_workspace_bytes(geom, n, Hq, max_ctx)), dtype=torch.uint8, device=dev)
    rng = np.random.default_rng(cfg.seed)

    # decode of the step's token (fused append) before the round trip; the append
    # rewrites the same slot with the same values when the step runs again after it
    def decode():
        tabs = [bm.table(s) for s in seqs]
        slots = torch.tensor([t[(int(S) - 1) // B] * B + (int(S) - 1) % B for t, S in zip(tabs, lengths)],
                             dtype=torch.int64, device=dev)
        tables_np, _ = bm.build_tables(seqs, max(len(t) for t in tabs))
        out = torch.empty((L, n, Hq, d), dtype=geom.torch_dtype, device=dev)
        steps.decode_step(geom, k_pool, v_pool, q_all, kn, vn, slots,
                          torch.from_numpy(np.ascontiguousarray(tables_np)).to(dev), lens, max_ctx, out, ws,
                          stream=stream, fused=not args.unfused)
        torch.cuda.synchronize()
        return out

    before = decode()
    log("decode before the round trip done (80 layers)")
    # oracle inputs for sampled (sequence, layer) outputs: the blocks as they are now
    dec_samples = [(int(rng.integers(0, n)), int(rng.integers(0, L))) for _ in range(args.parity_samples)]
    dec_snap = {}
    for (i, layer) in dec_samples:
        tab = bm.table(seqs[i])
        ids = torch.tensor(tab, dtype=torch.int64, device=dev)
        dec_snap[(i, layer)] = (to_np(torch, k_pool[layer].index_select(0, ids), "bf16")[None],
                                to_np(torch, v_pool[layer].index_select(0, ids), "bf16")[None])

    blocks_per_seq = bm.info(seqs[0])[1]
    choice = gen.offload_choice(cfg, blocks_per_seq)
    keep = max(1, int(round(args.offload_fraction * choice.shape[1])))
    choice = choice[:, :keep]
    per = pk.bytes_per_block(geom)
    total = n * keep * per
    log(f"round trip of {n * keep} blocks = {total / 2**30:.1f} GiB")
    host, passes, cpp, refused = alloc_pinned_passes(torch, n, keep, per)
    chunk = cfg.offload_chunk_blocks
    staging = torch.empty(chunk * per, dtype=torch.uint8, device=dev)

    legs = {"gather": [], "d2h": [], "h2d": [], "scatter": []}
    marks = []

    def mark(kind, start, m):
        ev = torch.cuda.Event(enable_timing=True)
        ev.record(stream)
        marks.append((kind, m, ev))

    def leg_times(start_ev):
        prev = start_ev
        for kind, m, ev in marks:
            legs[kind].append((m, prev.elapsed_time(ev)))
            prev = ev
        marks.clear()

    t_out_ms = t_in_ms = 0.0
    frames_checked, frames_equal = 0, True
    moved = 0
    for p in range(passes):
        part = choice[:, p * cpp:(p + 1) * cpp]
        if part.shape[1] == 0:
            continue
        phys = [bm.swap_out(s, part[k].tolist()) for k, s in enumerate(seqs)]
        ids_np = np.concatenate(phys).astype(np.int32)
        ids = torch.from_numpy(ids_np).to(dev)
        m_pass = ids.numel()
        # sampled frames: the oracle's gather of the same blocks, taken now
        pos = np.sort(rng.choice(m_pass, size=min(8, m_pass), replace=False))
        sel = torch.from_numpy(ids_np[pos].astype(np.int64)).to(dev)
        ks = to_np(torch, k_pool.index_select(1, sel), "bf16")
        vs = to_np(torch, v_pool.index_select(1, sel), "bf16")
        expect = np.ascontiguousarray(okv.gather_blocks(ks, vs, list(range(len(pos))))).view(np.uint8)
        expect = expect.reshape(len(pos), per)
        with Timer(torch, stream) as t_out:
            steps.offload(geom, k_pool, v_pool, ids, host, staging, chunk, stream=stream, on_chunk=mark)
        leg_times(t_out.a)
        t_out_ms += t_out.ms
        hv = host.numpy()
        for r, q in enumerate(pos):
            frames_checked += 1
            frames_equal &= bool(np.array_equal(hv[q * per:(q + 1) * per], expect[r]))
        # the released blocks may now be handed out again: scribble over them,
        # reshuffle the free list, bring the pass back into fresh blocks
        k_pool[:, ids.long()] = float("nan")
        v_pool[:, ids.long()] = float("nan")
        torch.cuda.synchronize()
        bm.permute_free(gen.realloc_shuffle(cfg, bm.num_free(), p))
        new_phys = [bm.swap_in(s, part[k].tolist()) for k, s in enumerate(seqs)]
        new_ids = torch.from_numpy(np.concatenate(new_phys).astype(np.int32)).to(dev)
        moved_away = float(np.mean(np.concatenate(new_phys) != ids_np))
        with Timer(torch, stream) as t_in:
            steps.restore(geom, k_pool, v_pool, new_ids, host, staging, chunk, stream=stream, on_chunk=mark)
        leg_times(t_in.a)
        t_in_ms += t_in.ms
        moved += m_pass
        log(f"pass {p + 1}/{passes}: {m_pass} blocks out {t_out.ms:.1f} ms, back {t_in.ms:.1f} ms; "
            f"{100 * moved_away:.1f}% of them in a different block; sampled frames equal so far: {frames_equal}")
    bm.validate()
    after = decode()
    bit_exact = bool(torch.equal(before.view(torch.int16), after.view(torch.int16)))
    log(f"decode after the round trip bitwise equal: {bit_exact}")
    errs = []
    for (i, layer), (kl, vl) in dec_snap.items():
        got = after[layer, i:i + 1].float().cpu().numpy().astype(np.float64)
        # the snapshot holds the table's blocks in order: logical block j at local id j
        tab = list(range(kl.shape[1]))
        slot = (int(lengths[i]) - 1)
        kk, vv = okv.append_kv(kl, vl, 0, to_np(torch, kn[layer, i:i + 1], "bf16"),
                               to_np(torch, vn[layer, i:i + 1], "bf16"), [slot], B)
        expect = oatt.paged_decode(to_np(torch, q_all[layer, i:i + 1], "bf16"), kk, vv, 0, [tab],
                                   [int(lengths[i])], B, "bf16")
        errs.append(float(np.max(np.abs(got - expect))))
    parity = {"samples": len(errs), "max_abs_err": max(errs) if errs else None, "tol": 2e-2,
              "ok": (max(errs) <= 2e-2) if errs else None}
    log(f"parity after the round trip {parity}")

    def rate(kind, factor):
        m = sum(x[0] for x in legs[kind])
        ms = sum(x[1] for x in legs[kind])
        return round(factor * m * per / (ms * 1e-3) / 1e9, 1), round(ms, 2)

    g_gbs, g_ms = rate("gather", 2)
    s_gbs, s_ms = rate("scatter", 2)
    d_gbs, d_ms = rate("d2h", 1)
    h_gbs, h_ms = rate("h2d", 1)
    result = {
        "metric": "offload round trip: gather/scatter GB/s (read+write), host link GB/s, offload",
        "value": round(2 * moved * per / ((t_out_ms + t_in_ms) * 1e-3) / 1e9, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": 1, "warmup": 0, "ms_per_step": round(t_out_ms + t_in_ms, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "num_seqs": n, "context_len": int(lengths.max()),
                   "blocks_moved": int(moved), "bytes_moved": int(moved * per), "chunk_blocks": chunk,
                   "offload_fraction": args.offload_fraction, "passes": passes,
                   "blocks_per_pass": n * cpp, "pinned_request_bytes": int(host.numel()),
                   "pinned_requests_refused": refused},
        "gather_GBps_rw": g_gbs, "gather_ms": g_ms, "scatter_GBps_rw": s_gbs, "scatter_ms": s_ms,
        "d2h_GBps": d_gbs, "d2h_ms": d_ms, "h2d_GBps": h_gbs, "h2d_ms": h_ms,
        "roofline": {"bound": "hbm", "kernel": "block_move_kernel (gather)", "achieved": g_gbs,
                     "peak": PEAK_GBS, "unit": "GB/s", "frac": round(g_gbs / PEAK_GBS, 4), "traffic": None},
        "sampled_frames": {"checked": frames_checked, "equal_to_oracle_gather": frames_equal},
        "decode_bitwise_equal_after_round_trip": bit_exact,
        "parity": parity,
    }
    print(json.dumps(result), flush=True)
    if not (bit_exact and frames_equal and (parity["ok"] in (None, True))):
        sys.exit(1)


# =============================================================================
# Overlapped asynchronous offload
# =============================================================================
PEAK_HOST_LINK_GBS = 64.0   # PCIe Gen5 x16, one direction
# "KV Cache Management", section "Retain, Evict, Recompute, or Offload", Figure 10:
# the 5.0 GiB state of a 70B trajectory at S = 16,384 streams out and back over
# PCIe Gen5 x16 in 215 ms.
PAGES_ROUND_TRIP_MS = 215.0


def run_overlap(args):
    """The gqa70b_32k decode batch steps on the compute stream while one more
    trajectory goes to pinned host memory and back through pa_swapper.

    Phase A: decode alone. Phase B: the round trip alone (freed blocks poisoned
    and the free queue reshuffled before the way back, decode of the trajectory
    compared bit for bit). Phase C: the swap-out is queued, then enough decode
    steps to cover it; once its completion step has run the free queue is
    reshuffled again and the swap-in is queued, followed by more decode steps.
    Reports the host-link rates alone and overlapped, the decode slowdown and
    the fraction of the migration's time hidden behind decode."""
    torch, pk, cfg, dev, stream, geom, gen_, k_pool, v_pool = setup(args)
    from paged_kv_cache_83_amd import steps
    from synth import gen
    L, n, Hq, Hkv, d, B = (cfg.num_layers, cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads,
                           cfg.head_dim, cfg.block_size)
    lengths = gen.context_lengths(cfg)
    bm = pk.BlockManager(cfg.num_blocks, B, gen.free_order(cfg))
    seqs = [bm.seq_new() for _ in range(n)]
    for s, S in zip(seqs, lengths):
        bm.append(s, int(S) - 1)
    slots_np, cow = bm.append_batch(seqs, [1] * n)
    assert not cow
    mover = bm.seq_new()
    bm.append(mover, cfg.mover_len)
    nblk = bm.info(mover)[1]
    lbs = list(range(nblk))
    max_blocks = max(bm.info(s)[1] for s in seqs)
    tables_np, lens_np = bm.build_tables(seqs, max_blocks)
    slots = torch.from_numpy(slots_np).to(dev)
    tables = torch.from_numpy(np.ascontiguousarray(tables_np)).to(dev)
    lens = torch.from_numpy(np.ascontiguousarray(lens_np)).to(dev)
    max_ctx = int(lengths.max())
    dt = geom.torch_dtype
    q_all = torch.randn((L, n, Hq, d), generator=gen_, device=dev).to(dt)
    k_new = torch.randn((L, n, Hkv, d), generator=gen_, device=dev).to(dt)
    v_new = torch.randn((L, n, Hkv, d), generator=gen_, device=dev).to(dt)
    out = torch.empty((L, n, Hq, d), dtype=dt, device=dev)
    ws = torch.empty(max(1, pk.decode_workspace_bytes(geom, n, Hq, max_ctx)), dtype=torch.uint8,
                     device=dev)
    q_m = torch.randn((L, 1, Hq, d), generator=gen_, device=dev).to(dt)
    ws_m = torch.empty(max(1, pk.decode_workspace_bytes(geom, 1, Hq, cfg.mover_len)),
                       dtype=torch.uint8, device=dev)

    def step():
        steps.decode_step(geom, k_pool, v_pool, q_all, k_new, v_new, slots, tables, lens, max_ctx,
                          out, ws, stream=stream, fused=not args.unfused)

    def decode_mover():
        t = torch.from_numpy(np.asarray([bm.table(mover)], np.int32)).to(dev)
        ln = torch.tensor([cfg.mover_len], dtype=torch.int32, device=dev)
        o = torch.empty((L, 1, Hq, d), dtype=dt, device=dev)
        for layer in range(L):
            pk.decode(geom, k_pool, v_pool, layer, q_m[layer], o[layer], t, ln, cfg.mover_len,
                      workspace=ws_m, stream=stream)
        torch.cuda.synchronize()
        return o

    # ---- phase A: decode alone ----------------------------------------------
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_a, st_a = timed_steps(torch, stream, step, args.steps)
    dec_ms = st_a["median"]
    out_ref = out.clone()
    mover_ref = decode_mover()
    log(f"decode alone: {dec_ms:.3f} ms/step (median of {args.steps})")

    chunk = cfg.offload_chunk_blocks if args.chunk_blocks < 0 else args.chunk_blocks
    sw = pk.Swapper(geom, bm, k_pool, v_pool, nblk, chunk, args.move_wgs)
    moved = nblk * sw.frame_bytes
    log(f"trajectory: {cfg.mover_len} tokens = {nblk} blocks = {moved / 2**30:.2f} GiB, "
        f"chunks of {sw.chunk_blocks} blocks")
    ev = lambda: torch.cuda.Event(enable_timing=True)    # noqa: E731

    side = torch.cuda.Stream(dev)      # idle stream: marks issue and completion times

    def migrate(kind, after):
        a, b = ev(), ev()
        a.record(side)
        (sw.swap_out if kind == "out" else sw.swap_in)(mover, lbs, after=after)
        sw.fence(side)
        b.record(side)
        return a, b

    def poison_and_shuffle(poison):
        if poison:
            free = torch.as_tensor(bm.free_list(), dtype=torch.long, device=dev)
            k_pool.index_fill_(1, free, float("nan"))
            v_pool.index_fill_(1, free, float("nan"))
        bm.permute_free(gen.realloc_shuffle(cfg, bm.num_free()))

    # ---- phase B: round trip alone ------------------------------------------
    torch.cuda.synchronize()
    if not args.no_prof:
        pk.Profiler.reset()
        pk.Profiler.enable(True)
    o_a, o_b = migrate("out", stream)
    sw.sync()
    assert all(bm.tier(mover, lb)[0] == pk.PA_TIER_HOST for lb in lbs)
    poison_and_shuffle(True)
    i_a, i_b = migrate("in", stream)       # ordered after the poisoning on the compute stream
    sw.sync()
    side.synchronize()
    pk.Profiler.enable(False)
    out_ms_alone, in_ms_alone = o_a.elapsed_time(o_b), i_a.elapsed_time(i_b)
    mig_alone = out_ms_alone + in_ms_alone
    alone_ok = bool(torch.equal(decode_mover().view(torch.int16), mover_ref.view(torch.int16)))
    log(f"round trip alone: out {out_ms_alone:.1f} ms, in {in_ms_alone:.1f} ms, bitwise {alone_ok}")
    kern = {}
    if not args.no_prof:
        for name in ("swap_gather", "swap_scatter"):
            cnt, tot = pk.Profiler.read(name)
            if cnt:
                kern[name] = {"launches": cnt, "avg_us": round(1e3 * tot / cnt, 2),
                              "GBps_rw": round(2 * moved / (tot * 1e-3) / 1e9, 1)}

    # ---- phase C: round trip behind decode -----------------------------------
    k1 = int(math.ceil(out_ms_alone / dec_ms)) + 2
    k2 = int(math.ceil(in_ms_alone / dec_ms)) + 2
    torch.cuda.synchronize()
    times = StepTimes(torch, stream, k1 + k2)
    c_a = ev()
    c_a.record(stream)
    o_a, o_b = migrate("out", stream)
    for _ in range(k1):
        times.mark()
        step()
    sw.sync()                                # host waits for the completion step only
    poison_and_shuffle(False)                # host-side: fresh blocks differ from the old ones
    # No kernel queued on the compute stream touches the trajectory's blocks (the
    # batch never frees a block), so the way back needs no ordering after it.
    i_a, i_b = migrate("in", 0)
    for _ in range(k2):
        times.mark()
        step()
    times.mark()
    c_b = ev()
    c_b.record(stream)
    sw.sync()
    torch.cuda.synchronize()
    out_ms_ov, in_ms_ov = o_a.elapsed_time(o_b), i_a.elapsed_time(i_b)
    compute_ms = c_a.elapsed_time(c_b)
    total_ms = max(compute_ms, c_a.elapsed_time(i_b))
    serial_ms = (k1 + k2) * dec_ms + mig_alone
    hidden = (serial_ms - total_ms) / mig_alone
    st_c = times.summary()
    batch_ok = bool(torch.equal(out.view(torch.int16), out_ref.view(torch.int16)))
    mover_ok = bool(torch.equal(decode_mover().view(torch.int16), mover_ref.view(torch.int16)))
    log(f"overlapped: {k1}+{k2} steps in {compute_ms:.1f} ms (alone {(k1 + k2) * dec_ms:.1f}), "
        f"out {out_ms_ov:.1f} ms, in {in_ms_ov:.1f} ms, hidden {hidden:.3f}")

    # ---- CPU baseline: the oracle's gather + scatter on a sample of blocks -----
    cpu_baseline = None
    if not args.no_cpu_baseline:
        from oracle import kv_ops as okv
        sample = bm.table(mover)[:16]
        idx = torch.as_tensor(sample, dtype=torch.long, device=dev)
        kb = to_np(torch, k_pool.index_select(1, idx), cfg.dtype)
        vb = to_np(torch, v_pool.index_select(1, idx), cfg.dtype)
        ids = list(range(len(sample)))
        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 10.0:
            st = okv.gather_blocks(kb, vb, ids)
            okv.scatter_blocks(kb, vb, st, ids[::-1])
            reps += 1
        cpu_s = time.perf_counter() - t0
        cpu_baseline = {"value": round(2 * reps * len(sample) * sw.frame_bytes / cpu_s / 1e9, 3),
                        "unit": "GB/s", "cores": 1, "kind": "oracle",
                        "sample": f"{reps} gather + scatter passes of {len(sample)} blocks of this "
                                  f"workload through the oracle's kv_ops in {cpu_s:.1f} s"}

    link_ov = 2 * moved / ((out_ms_ov + in_ms_ov) * 1e-3) / 1e9
    pages_gbs = 2 * moved / (PAGES_ROUND_TRIP_MS * 1e-3) / 1e9
    result = {
        "metric": "host-link GB/s of a 16K-token 70B trajectory round trip overlapped with "
                  "70B-GQA 32K decode",
        "value": round(link_ov, 2), "unit": "GB/s", "n_gpus": 1, "steps": k1 + k2,
        "warmup": args.warmup, "ms_per_step": round(compute_ms / (k1 + k2), 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": round(link_ov / pages_gbs, 4),
        "baseline": {"round_trip_ms": PAGES_ROUND_TRIP_MS, "GBps": round(pages_gbs, 2),
                     "source": "KVM 'Retain, Evict, Recompute, or Offload', Figure 10: 5.0 GiB "
                               "(70B, S = 16,384) out and back over PCIe Gen5 x16, napkin figure"},
        "round_trip_ms": {"alone": round(mig_alone, 2), "overlapped": round(out_ms_ov + in_ms_ov, 2)},
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) pools, seeded block placement)",
        "config": {"workload": cfg.name, "num_seqs": n, "context_len": int(lengths.max()),
                   "mover_tokens": cfg.mover_len, "mover_blocks": nblk, "bytes_each_way": moved,
                   "chunk_blocks": sw.chunk_blocks, "pool_blocks": cfg.num_blocks},
        "decode_ms_alone": dec_ms, "decode_step_ms_overlapped": st_c,
        "decode_slowdown": round(compute_ms / ((k1 + k2) * dec_ms), 4),
        "swap_out_ms": {"alone": round(out_ms_alone, 2), "overlapped": round(out_ms_ov, 2)},
        "swap_in_ms": {"alone": round(in_ms_alone, 2), "overlapped": round(in_ms_ov, 2)},
        "d2h_GBps": {"alone": round(moved / out_ms_alone / 1e6, 2),
                     "overlapped": round(moved / out_ms_ov / 1e6, 2)},
        "h2d_GBps": {"alone": round(moved / in_ms_alone / 1e6, 2),
                     "overlapped": round(moved / in_ms_ov / 1e6, 2)},
        "overlap": {"serial_ms": round(serial_ms, 2), "overlapped_ms": round(total_ms, 2),
                    "hidden_fraction_of_migration": round(hidden, 4)},
        "roofline": {"bound": "host link", "achieved": round(link_ov, 2), "peak": PEAK_HOST_LINK_GBS,
                     "unit": "GB/s", "frac": round(link_ov / PEAK_HOST_LINK_GBS, 4), "traffic": None,
                     "note": "DMA copies, one direction at a time; peak = PCIe Gen5 x16 per direction"},
        "cpu_baseline": cpu_baseline,
        "kernels": kern,
        "parity": {"round_trip_alone_bitwise": alone_ok, "batch_decode_during_overlap_bitwise": batch_ok,
                   "round_trip_overlapped_bitwise": mover_ok},
    }
    sw.close()
    print(json.dumps(result), flush=True)
    if not (alone_ok and batch_ok and mover_ok):
        sys.exit(1)


# =============================================================================
# Prefix reuse through the radix cache
# =============================================================================
def admit(bm, tree, prompts, block_size, watermark, clock=None):
    """Admit a batch through the prefix cache: match every prompt (pinning the
    cached path), evict dormant leaves if the free pool would fall below the
    watermark, then start each sequence from its cached full blocks and reserve
    blocks for the rest. Works on the library's or the oracle's objects.
    `clock` (optional list of 3 floats) accumulates seconds spent matching,
    evicting and reserving."""
    c0 = time.perf_counter()
    matches = [tree.match(p) for p in prompts]
    need = sum(-(-(len(p) - m[1]) // block_size) for p, m in zip(prompts, matches))
    c1 = time.perf_counter()
    evicted = []
    if bm.num_free() < need + watermark:
        evicted = tree.evict(need + watermark)
    c2 = time.perf_counter()
    seqs = []
    for p, m in zip(prompts, matches):
        sid = bm.seq_from_blocks(m[2])
        bm.append(sid, len(p) - m[1])
        seqs.append(sid)
    if clock is not None:
        clock[0] += c1 - c0
        clock[1] += c2 - c1
        clock[2] += time.perf_counter() - c2
    return seqs, [m[3] for m in matches], [m[1] for m in matches], evicted


def retire(bm, tree, prompts, seqs, handles):
    """Index the finished requests' blocks, drop their pins, release them."""
    adopted = []
    for p, sid, h in zip(prompts, seqs, handles):
        adopted.append(tree.insert(p, bm.table(sid)))
        tree.unpin(h)
        bm.release(sid)
    return adopted


def run_prefix_reuse(args):
    torch, pk, cfg, dev, stream, geom, gen_, k_pool, v_pool = setup(args)
    from synth import gen
    L, n, Hq, Hkv, d, B = (cfg.num_layers, cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads,
                           cfg.head_dim, cfg.block_size)
    P, C = cfg.prefix_len, cfg.chunk_len
    budget, watermark = int(cfg.extra["budget_blocks"]), int(cfg.extra["watermark_blocks"])
    n_steps = args.warmup + args.steps + 1      # the last batch measures latency alone
    system, novel = gen.prefix_reuse_tokens(cfg, n_steps)
    prompts_of = [[np.concatenate([system, novel[k, i]]) for i in range(n)] for k in range(n_steps)]
    S = P + C
    maxb = -(-S // B)
    bm = pk.BlockManager(budget, B)
    tree = pk.RadixCache(bm)

    # the system prompt's K/V per layer (inputs), written once by a cold prefill
    k_sys = torch.randn((L, P, Hkv, d), generator=gen_, device=dev).to(geom.torch_dtype)
    v_sys = torch.randn((L, P, Hkv, d), generator=gen_, device=dev).to(geom.torch_dtype)
    q_all = torch.randn((L, n * C, Hq, d), generator=gen_, device=dev).to(geom.torch_dtype)
    k_all = torch.randn((L, n * C, Hkv, d), generator=gen_, device=dev).to(geom.torch_dtype)
    v_all = torch.randn((L, n * C, Hkv, d), generator=gen_, device=dev).to(geom.torch_dtype)
    out = torch.empty_like(q_all)

    sid0 = bm.seq_new()
    bm.append(sid0, P)
    t0 = torch.tensor([bm.table(sid0)], dtype=torch.int32, device=dev)
    zero1 = torch.zeros(1, dtype=torch.int32, device=dev)
    qs0 = torch.tensor([0, P], dtype=torch.int32, device=dev)
    q_sys = torch.empty((P, Hq, d), dtype=geom.torch_dtype, device=dev)
    o_sys = torch.empty_like(q_sys)
    with Timer(torch, stream) as tc:
        for layer in range(L):
            q_sys.normal_(generator=gen_)
            pk.prefill(geom, k_pool, v_pool, layer, q_sys, k_sys[layer], v_sys[layer], o_sys, qs0, t0,
                       zero1, P, P, stream=stream)
    cold_ms = tc.ms
    tree.insert(system, bm.table(sid0))
    bm.release(sid0)
    log(f"cold prefill of the {P}-token system prompt: {cold_ms:.2f} ms (80 layers, q drawn per layer)")

    q_start = torch.arange(0, n * C + 1, C, dtype=torch.int32, device=dev)
    pf_ws = torch.empty(max(1, pk.prefill_workspace_bytes(geom, n, n * C, Hq, C, S, args.pf_splits)),
                        dtype=torch.uint8, device=dev)
    # two sets of tables: the host fills one while kernels of the previous batch
    # still read the other; an event per set says when its upload has run
    tables_h = [torch.empty((n, maxb), dtype=torch.int32).pin_memory() for _ in range(2)]
    ctx_h = [torch.empty(n, dtype=torch.int32).pin_memory() for _ in range(2)]
    tables_d = [torch.empty((n, maxb), dtype=torch.int32, device=dev) for _ in range(2)]
    ctx_d = [torch.empty(n, dtype=torch.int32, device=dev) for _ in range(2)]
    uploaded = [torch.cuda.Event() for _ in range(2)]
    for e in uploaded:
        e.record(stream)
    torch.cuda.synchronize()

    profiling = [False]
    record = []          # per step: usable lengths, evicted ids, adopted counts
    host_s = [0.0, 0.0]  # admission (including tables and their copy), retirement
    parts = [0.0] * 6    # match, evict, reserve, build tables, queue table copies, wait

    def step(k):
        """Admit batch k, queue its 80 layers, retire it. No wait for the device:
        the host admits batch k+1 while the kernels of batch k run. Blocks that
        eviction or release hands out again are only written by kernels queued
        later on the same stream."""
        prompts = prompts_of[k]
        buf = k % 2
        h0 = time.perf_counter()
        seqs, handles, usable, evicted = admit(bm, tree, prompts, B, watermark, parts)
        if any(u != P for u in usable):
            raise RuntimeError(f"step {k}: cached prefix lost ({usable}); the budget is too small")
        ha = time.perf_counter()
        tabs, lens = bm.build_tables(seqs, maxb)
        hw0 = time.perf_counter()
        uploaded[buf].synchronize()   # the upload two batches ago has left this pinned set
        hw1 = time.perf_counter()
        tables_h[buf].numpy()[:] = tabs
        ctx_h[buf].numpy()[:] = np.asarray(usable, np.int32)
        hb = time.perf_counter()
        tables_d[buf].copy_(tables_h[buf], non_blocking=True)
        ctx_d[buf].copy_(ctx_h[buf], non_blocking=True)
        uploaded[buf].record(stream)
        h1 = time.perf_counter()
        parts[3] += (hb - ha) - (hw1 - hw0)
        parts[4] += h1 - hb
        parts[5] += hw1 - hw0  # the host is ahead of the device: not host work
        for layer in range(L):
            prof = profiling[0] and layer % args.prof_every == 0
            if prof:
                pk.Profiler.enable(True)
            pk.prefill(geom, k_pool, v_pool, layer, q_all[layer], k_all[layer], v_all[layer],
                       out[layer], q_start, tables_d[buf], ctx_d[buf], C, S, stream=stream,
                       splits=args.pf_splits, workspace=pf_ws)
            if prof:
                pk.Profiler.enable(False)
        h2 = time.perf_counter()
        adopted = retire(bm, tree, prompts, seqs, handles)
        h3 = time.perf_counter()
        host_s[0] += (h1 - h0) - (hw1 - hw0)
        host_s[1] += h3 - h2
        record.append((list(usable), list(evicted), adopted))

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    # the host loop allocates small Python objects (block id lists): move what
    # exists now out of the collector's view, so a full collection over
    # everything torch allocated does not land inside the timed steps
    gc.collect()
    gc.freeze()
    host_s[:] = [0.0, 0.0]
    parts[:] = [0.0] * 6
    if not args.no_prof:
        pk.Profiler.reset()
        profiling[0] = True
    with Timer(torch, stream) as t:
        for k in range(args.warmup, args.warmup + args.steps):
            step(k)
    profiling[0] = False
    ms = max(t.ms, t.wall_ms) / args.steps
    evicted_timed = sum(len(r[1]) for r in record[args.warmup:])
    host_timed, parts_timed = list(host_s), list(parts)
    # one more batch on its own: admission to outputs ready (time to first token of the batch)
    with Timer(torch, stream) as tl:
        step(n_steps - 1)
    latency_ms = max(tl.ms, tl.wall_ms)
    value = n / (ms * 1e-3)
    info = tree.info()
    log(f"timed {args.steps} steps: {ms:.3f} ms/step, {value:.1f} requests/s; evicted "
        f"{evicted_timed} nodes; tree {info}")

    kern, roofline = {}, None
    macs_layer = sum(2 * Hq * d * (C * P + C * (C + 1) // 2) for _ in range(n))
    if not args.no_prof:
        for name in ("prefill_append", "prefill_attention", "prefill_combine"):
            cnt, tot = pk.Profiler.read(name)
            if cnt:
                kern[name] = {"launches": cnt, "avg_us": round(1e3 * tot / cnt, 2)}
        if "prefill_attention" in kern:
            avg_s = kern["prefill_attention"]["avg_us"] * 1e-6
            ach = 2 * macs_layer / avg_s / 1e12
            roofline = {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": None,
                        "kernel": "prefill_mfma_kernel", "flops_per_launch": 2 * macs_layer,
                        "avg_launch_us": round(avg_s * 1e6, 2)}
            if "prefill_combine" in kern:
                roofline["combine_avg_us"] = kern["prefill_combine"]["avg_us"]

    # host cost of one lookup of a full prompt (cached path of 4,096 tokens), through the binding
    probe = prompts_of[-1][0]
    reps = 2000
    h0 = time.perf_counter()
    for _ in range(reps):
        _, _, _, h = tree.match(probe)
        tree.unpin(h)
    match_us = (time.perf_counter() - h0) / reps * 1e6

    # parity: sampled (request, layer) outputs of the last step against the oracle,
    # which takes the history from the inputs (the system prompt's K/V), not the pool
    parity, cpu_baseline, radix_parity = None, None, None
    if args.parity_samples or not args.no_cpu_baseline:
        from oracle import attention as oatt
        from oracle import layout as olayout
        from oracle import prefill as opf
        rng = np.random.default_rng(cfg.seed)
        scale = oatt.default_scale(d)

        def oracle_one(i, layer):
            rows = slice(i * C, (i + 1) * C)
            w = lambda x: olayout.widen(to_np(torch, x, cfg.dtype), cfg.dtype)  # noqa: E731
            return opf.chunk_attention(w(q_all[layer, rows]), w(k_all[layer, rows]), w(v_all[layer, rows]),
                                       w(k_sys[layer]), w(v_sys[layer]), scale)

        errs = []
        for _ in range(args.parity_samples):
            i, layer = int(rng.integers(0, n)), int(rng.integers(0, L))
            expect = oracle_one(i, layer)
            got = out[layer, i * C:(i + 1) * C].float().cpu().numpy().astype(np.float64)
            errs.append(float(np.max(np.abs(got - expect))))
        if errs:
            parity = {"samples": len(errs), "max_abs_err": max(errs), "tol": 2e-2,
                      "ok": max(errs) <= 2e-2}
            log(f"parity {parity}")

        # the same admission / retirement sequence on the oracle block manager and tree
        from oracle import block_manager as obm
        from oracle import radix as orx
        om = obm.BlockManager(budget, B)
        ot = orx.RadixCache(om)
        s0 = om.seq_new()
        om.append(s0, P)
        ot.insert(system, om.table(s0))
        om.release(s0)
        same = True
        for k in range(n_steps):
            prompts = prompts_of[k]
            seqs, handles, usable, evicted = admit(om, ot, prompts, B, watermark)
            adopted = retire(om, ot, prompts, seqs, handles)
            same &= (list(usable), list(evicted), adopted) == record[k]
        for _ in range(reps):                          # the timed lookups touched the tree too
            _, _, _, h = ot.match(probe)
            ot.unpin(h)
        onodes = {x.id: (x.parent.id, x.ref_count, x.last_access, list(x.prefix_tokens),
                         list(x.block_ids)) for x in ot.nodes.values() if x is not ot.root}
        same &= onodes == tree.nodes() and list(om.free) == bm.free_list()
        radix_parity = {"steps": n_steps, "requests": n * n_steps, "identical": bool(same)}
        log(f"radix parity {radix_parity}")

        if not args.no_cpu_baseline:
            cores = len(os.sched_getaffinity(0))
            pairs = [(int(rng.integers(0, n)), int(rng.integers(0, L))) for _ in range(max(1, args.cpu_sample // 12))]
            c0 = time.perf_counter()
            for (i, layer) in pairs:
                oracle_one(i, layer)
            per_pair = (time.perf_counter() - c0) / len(pairs)
            c1 = time.perf_counter()
            _, _, _, h = ot.match(probe)
            ot.unpin(h)
            radix_s = time.perf_counter() - c1
            per_req = per_pair * L + radix_s
            cpu_baseline = {"value": round(1.0 / per_req, 6), "unit": "requests/s", "cores": cores,
                            "kind": "oracle",
                            "sample": f"{len(pairs)} (request, layer) chunk attentions of this workload "
                                      f"({per_pair:.2f} s each) x {L} layers + one oracle prefix match "
                                      f"({radix_s * 1e3:.1f} ms)"}

    # no reuse: the same requests prefilled from scratch (4,128 tokens each) in the rest of the pool
    nr = None
    if not args.no_baseline_leg:
        tables_nr = (budget + torch.arange(n * maxb, dtype=torch.int32, device=dev)).view(n, maxb)
        q_nr = torch.randn((n * S, Hq, d), generator=gen_, device=dev).to(geom.torch_dtype)
        k_nr = torch.randn((n * S, Hkv, d), generator=gen_, device=dev).to(geom.torch_dtype)
        v_nr = torch.randn((n * S, Hkv, d), generator=gen_, device=dev).to(geom.torch_dtype)
        o_nr = torch.empty_like(q_nr)
        qs_nr = torch.arange(0, n * S + 1, S, dtype=torch.int32, device=dev)
        z_nr = torch.zeros(n, dtype=torch.int32, device=dev)
        pk.prefill(geom, k_pool, v_pool, 0, q_nr, k_nr, v_nr, o_nr, qs_nr, tables_nr, z_nr, S, S,
                   stream=stream)
        with Timer(torch, stream) as tn:
            for layer in range(L):
                pk.prefill(geom, k_pool, v_pool, layer, q_nr, k_nr, v_nr, o_nr, qs_nr, tables_nr, z_nr,
                           S, S, stream=stream)
        nr_ms = max(tn.ms, tn.wall_ms)
        nr = {"ms_per_step": round(nr_ms, 3), "requests_per_s": round(n / (nr_ms * 1e-3), 2),
              "prefill_tokens": n * S, "speedup_with_reuse": round(nr_ms / ms, 1),
              "note": "same 16 prompts prefilled from token 0 (attention + K/V write, 80 layers); "
                      "one step, inputs reused across layers"}
        log(f"no reuse: {nr}")

    result = {
        "metric": "prefix-hit prefill requests/s (radix prefix cache + paged prefill attention), "
                  "70B-GQA, 4,096 cached + 32 novel tokens",
        "value": round(value, 2), "unit": "requests/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded token ids and N(0,1) Q/K/V)",
        "config": {"workload": cfg.name, "num_layers": L, "num_q_heads": Hq, "num_kv_heads": Hkv,
                   "head_dim": d, "block_size": B, "requests_per_step": n, "prefix_tokens": P,
                   "novel_tokens": C, "cache_budget_blocks": budget, "watermark_blocks": watermark,
                   "launch": "eager"},
        "host": {"admit_us_per_request": round(host_timed[0] / (args.steps * n) * 1e6, 2),
                 "retire_us_per_request": round(host_timed[1] / (args.steps * n) * 1e6, 2),
                 "admit_parts_us_per_request": {
                     k_: round(v_ / (args.steps * n) * 1e6, 2) for k_, v_ in
                     zip(("match", "evict", "reserve", "build_tables", "queue_copies"), parts_timed)},
                 "wait_for_free_table_set_us_per_request": round(parts_timed[5] / (args.steps * n) * 1e6,
                                                                 2),
                 "match_unpin_us_4128_tokens": round(match_us, 2),
                 "evicted_nodes_timed": evicted_timed, "tree": info},
        "batch_latency_ms": round(latency_ms, 3),
        "cold_system_prefill_ms": round(cold_ms, 3),
        "no_reuse": nr,
        "roofline": roofline,
        "cpu_baseline": cpu_baseline,
        "kernels": kern,
        "parity": parity,
        "radix_parity": radix_parity,
    }
    print(json.dumps(result), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the decode path here runs on exactly one GPU; --gpus {args.gpus} is not "
              "supported (across GPUs the path would shard by KV head or by sequence, with "
              "no exchange inside it)", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    from synth import get_config
    cfg = get_config(args.config)
    if cfg.name == "offload":
        run_offload(args)
    elif cfg.name == "offload_overlap":
        run_overlap(args)
    elif cfg.length_kind in ("prefill", "verify"):
        run_prefill(args)
    elif cfg.length_kind == "prefix":
        run_prefix_reuse(args)
    elif cfg.length_kind == "fork":
        run_fork(args)
    else:
        run_decode(args)


if __name__ == "__main__":
    main()
