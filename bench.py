#!/usr/bin/env python3
"""Paged-KV decode benchmark on one MI355X.

A step is one decode step of the whole batch across every layer: for each layer,
pa_append_kv writes the batch's new keys and values into their slots, then
pa_decode attends every query head over its sequence's paged cache (split-K
partial kernel + combine). Inputs (pool, tables, queries) are resident in HBM
before the timed region starts.

Default workload: the 70B grouped-query geometry at 32K context (80 layers,
64 query / 8 KV heads, head dim 128, bf16, 16-slot blocks), 16 sequences of
32,768 attended tokens, 32,768-block pool (171.8 GB) in a seeded random
physical order.

Prints one JSON line. `value` is KV bytes read per second for the step
(sum over sequences of attended tokens x bytes per token, all layers).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="gqa70b_32k")
    ap.add_argument("--bps", type=int, default=0, help="blocks per split (0 = library default)")
    ap.add_argument("--kernel", default="auto", choices=["auto", "generic", "mfma"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=48,
                    help="(sequence, layer) pairs the oracle times for the CPU baseline")
    ap.add_argument("--no-prof", action="store_true", help="do not record per-kernel events")
    ap.add_argument("--prof-every", type=int, default=8,
                    help="record kernel events around the decode of every k-th layer")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a 1 GiB device copy (for scaling HBM byte counters)")
    ap.add_argument("--parity-samples", type=int, default=4)
    return ap.parse_args()


def profiled_traffic(workload: str):
    """HBM bytes per decode launch from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, scaled by a 1 GiB copy), or None when the kernel
    source has changed since those counters were taken."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "profiles", f"decode_mfma_bf16_{workload}_hbm_counters.md")
    src = os.path.join(here, "paged_kv_cache_83_amd", "csrc", "pa_kernels.hip")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.split(":", 1)[0].strip() in ("source_sha256_prefix", "traffic_bytes_per_launch"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    if fields.get("source_sha256_prefix") != sha or "traffic_bytes_per_launch" not in fields:
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
    del src, dst
    big = torch.ones(8 << 30, dtype=torch.bfloat16, device="cuda")   # 16 GiB, read once per sum
    for _ in range(2):
        big.sum(dtype=torch.float32)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    reps = 5
    for _ in range(reps):
        big.sum(dtype=torch.float32)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    print(json.dumps({"calibration": "device read (sum)", "bytes_read": big.numel() * 2,
                      "seconds": dt, "GB_per_s_read": big.numel() * 2 / dt / 1e9}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on exactly one GPU; --gpus {args.gpus} is not "
              "supported (see the sharding note in DESIGN.md)", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return

    import torch
    import paged_kv_cache_83_amd as pk
    from synth import gen, get_config

    cfg = get_config(args.config)
    if cfg.length_kind not in ("fixed", "uniform", "lognormal"):
        print(f"bench.py: config {cfg.name} is not a plain decode batch", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    geom = pk.Geometry(cfg.num_layers, cfg.num_kv_heads, cfg.head_dim, cfg.block_size,
                       cfg.num_blocks, cfg.dtype)
    L, n, Hq, Hkv, d, B = (cfg.num_layers, cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads,
                           cfg.head_dim, cfg.block_size)
    lengths = gen.context_lengths(cfg)
    m_token = pk.bytes_per_token(L, Hkv, d, geom.elem_bytes)
    print(f"[bench] config={cfg.name} L={L} n={n} Hq={Hq} Hkv={Hkv} d={d} B={B} N={cfg.num_blocks} "
          f"dtype={cfg.dtype} pool={2 * pk.pool_bytes(geom) / 1e9:.1f} GB", file=sys.stderr, flush=True)

    # ---- inputs resident in HBM -------------------------------------------------
    gpu_gen = torch.Generator(device=dev)
    gpu_gen.manual_seed(cfg.seed)
    k_pool, v_pool = pk.alloc_pools(geom, dev)
    k_pool.normal_(generator=gpu_gen)
    v_pool.normal_(generator=gpu_gen)
    q_all = torch.randn((L, n, Hq, d), generator=gpu_gen, device=dev).to(geom.torch_dtype)
    k_new = torch.randn((L, n, Hkv, d), generator=gpu_gen, device=dev).to(geom.torch_dtype)
    v_new = torch.randn((L, n, Hkv, d), generator=gpu_gen, device=dev).to(geom.torch_dtype)

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
    out = torch.empty((L, n, Hq, d), dtype=geom.torch_dtype, device=dev)
    ws_bytes = pk.decode_workspace_bytes(geom, n, Hq, max_ctx, args.bps, args.kernel)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    # snapshot of the sampled sequences' blocks, before any library kernel writes the pool
    rng = np.random.default_rng(cfg.seed)
    samples = [(int(rng.integers(0, n)), int(rng.integers(0, L))) for _ in range(args.parity_samples)]
    snap = {}
    for (i, layer) in samples:
        ids = torch.from_numpy(np.asarray(tables_np[i, :math.ceil(lengths[i] / B)], np.int64)).to(dev)
        snap[(i, layer)] = (k_pool[layer].index_select(0, ids).cpu(), v_pool[layer].index_select(0, ids).cpu(),
                            ids.cpu().numpy())

    profiling = [False]

    def step():
        for layer in range(L):
            pk.append_kv(geom, k_pool, v_pool, layer, k_new[layer], v_new[layer], slots, stream=stream)
            # per-kernel events are recorded around the decode of every prof_every-th layer
            sample = profiling[0] and layer % args.prof_every == 0
            if sample:
                pk.Profiler.enable(True)
            pk.decode(geom, k_pool, v_pool, layer, q_all[layer], out[layer], tables, lens, max_ctx,
                      workspace=ws, blocks_per_split=args.bps, kernel=args.kernel, stream=stream)
            if sample:
                pk.Profiler.enable(False)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    if not args.no_prof:
        pk.Profiler.reset()
        profiling[0] = True
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    profiling[0] = False
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = max(gpu_ms, wall * 1e3) / args.steps
    print(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step", file=sys.stderr, flush=True)

    kv_bytes_step = int(lengths.sum()) * m_token
    value = kv_bytes_step / (ms_per_step * 1e-3) / 1e9
    tokens_per_s = n / (ms_per_step * 1e-3)

    # ---- roofline of the dominant kernel (decode partial), timed live ----------
    roofline = None
    kernel_ms = {}
    if not args.no_prof:
        for name in ("decode_partial", "decode_combine"):
            cnt, tot = pk.Profiler.read(name)
            if cnt:
                kernel_ms[name] = {"launches": cnt, "avg_us": 1e3 * tot / cnt}
        cnt, tot = pk.Profiler.read("decode_partial")
        if cnt:
            eb = geom.elem_bytes
            splits = max(1, ws_bytes // (n * Hq * (d + 2) * 4)) if ws_bytes else 1
            per_launch = (int(lengths.sum()) * 2 * Hkv * d * eb          # K and V of attended tokens
                          + n * Hq * d * eb                               # queries
                          + 4 * int(sum(math.ceil(S / B) for S in lengths))  # block-table entries
                          + (n * Hq * splits * (d + 2) * 4 if ws_bytes else n * Hq * d * eb))
            avg_s = tot / cnt * 1e-3
            achieved = per_launch / avg_s / 1e9
            roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": 8000.0, "unit": "GB/s",
                        "frac": round(achieved / 8000.0, 4),
                        "traffic": profiled_traffic(cfg.name) if args.bps == 0 and args.kernel == "auto" else None,
                        "kernel": "decode_mfma_bf16_kernel" if cfg.dtype == "bf16" else "decode_generic_kernel",
                        "bytes_per_launch": per_launch, "avg_launch_us": round(avg_s * 1e6, 2)}

    # ---- parity on sampled (sequence, layer) outputs against the oracle ---------
    parity = None
    cpu_baseline = None
    if args.parity_samples or not args.no_cpu_baseline:
        from oracle import attention as oatt
        from oracle import kv_ops as okv
        from oracle import block_manager as obm
        obm_ = obm.BlockManager(cfg.num_blocks, B, gen.free_order(cfg))
        oseqs = []
        for S in lengths:
            s = obm_.seq_new()
            obm_.append(s, int(S) - 1)
            oseqs.append(s)
        oslots = [obm_.append(s, 1)[0][0] for s in oseqs]
        otables = [obm_.table(s) for s in oseqs]

        def to_np(t):
            return t.view(torch.int16).numpy().view(np.uint16) if cfg.dtype == "bf16" else t.numpy()

        def oracle_one(i, layer):
            kb, vb, ids = snap[(i, layer)]
            # a local pool holding only this sequence's blocks, renumbered 0..nb-1
            kloc = to_np(kb)[None]
            vloc = to_np(vb)[None]
            remap = {int(p): j for j, p in enumerate(ids)}
            table = [remap[p] for p in otables[i]]
            slot = remap[oslots[i] // B] * B + oslots[i] % B
            kn = to_np(k_new[layer, i:i + 1].cpu())
            vn = to_np(v_new[layer, i:i + 1].cpu())
            kloc, vloc = okv.append_kv(kloc, vloc, 0, kn, vn, [slot], B)
            q = to_np(q_all[layer, i:i + 1].cpu())
            return oatt.paged_decode(q, kloc, vloc, 0, [table], [int(lengths[i])], B, cfg.dtype)[0]

        errs = []
        for (i, layer) in samples[:args.parity_samples]:
            expect = oracle_one(i, layer)
            got = out[layer, i].float().cpu().numpy().astype(np.float64)
            errs.append(float(np.max(np.abs(got - expect))))
        tol = 2e-2 if cfg.dtype == "bf16" else 1e-5
        parity = {"samples": len(errs), "max_abs_err": max(errs) if errs else None, "tol": tol,
                  "ok": bool(errs) and max(errs) <= tol}
        print(f"[bench] parity {parity}", file=sys.stderr, flush=True)

        if not args.no_cpu_baseline:
            try:
                from threadpoolctl import threadpool_limits
            except Exception:  # pragma: no cover
                threadpool_limits = None
            cores = len(os.sched_getaffinity(0))
            pairs = [(int(rng.integers(0, n)), int(rng.integers(0, L))) for _ in range(args.cpu_sample)]
            for (i, layer) in pairs:
                if (i, layer) not in snap:
                    ids = torch.from_numpy(np.asarray(tables_np[i, :math.ceil(lengths[i] / B)], np.int64)).to(dev)
                    snap[(i, layer)] = (k_pool[layer].index_select(0, ids).cpu(),
                                        v_pool[layer].index_select(0, ids).cpu(), ids.cpu().numpy())
            import contextlib
            limiter = threadpool_limits(limits=cores) if threadpool_limits else contextlib.nullcontext()
            with limiter:
                t0 = time.perf_counter()
                for (i, layer) in pairs:
                    oracle_one(i, layer)
                cpu_s = time.perf_counter() - t0
            per_pair = cpu_s / len(pairs)
            step_s = per_pair * n * L
            cpu_tok = n / step_s
            cpu_gbs = kv_bytes_step / step_s / 1e9
            cpu_baseline = {"value": round(cpu_gbs, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
                            "tokens_per_s": round(cpu_tok, 4),
                            "sample": f"{len(pairs)} (sequence, layer) decodes of the same workload "
                                      f"(each {int(lengths[0])} tokens x {Hq} heads) timed in "
                                      f"{cpu_s:.1f} s, scaled to the {n}-sequence x {L}-layer step"}

    result = {
        "metric": "paged-decode KV GB/s (% of HBM peak) + decode tokens/s, 70B-GQA 32K ctx",
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
                   "global_batch": n, "seq_len": int(lengths.max()), "parallelism": "none (1 GPU)"},
        "tokens_per_s": round(tokens_per_s, 2),
        "pct_hbm_peak": round(100 * value / 8000.0, 2),
        "roofline": roofline,
        "cpu_baseline": cpu_baseline,
        "kernels": kernel_ms,
        "parity": parity,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
