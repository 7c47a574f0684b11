#!/usr/bin/env python3
"""Throughput of one decode step of paged-KV attention on one MI355X.

A step is the whole hot path over one batch: each request's new K/V token is
appended to its block and slot and its query attends over the whole paged
history (one fused attention launch through the C ABI, plus the log-sum-exp
merge when the context is split).  Inputs are synthetic, seeded, and resident
in HBM before timing starts.  Successive steps rotate over R copies of the
inputs so that no step finds its K/V in the 256 MB Infinity Cache.

Prints ONE JSON line.  `value` is algorithmic HBM bytes per step (history K/V
read once, new K/V read and written once, q, f32 out, block-table entries and
positions) times steps, divided by the wall time of the timed region.
`roofline.achieved` divides the same bytes by the GPU time per step, from HIP
events recorded on the launch stream around the replayed region.  `cpu_baseline` times
the fp64 oracle on the host cores on the same workload.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c2|c3|c4|c5]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np

METRIC = "paged decode attention HBM GB/s (% of MI355X peak) and KV-tokens/s"
PEAK_HBM_GBPS = 8000.0           # MI355X HBM3E, decimal GB/s
INFINITY_CACHE_BYTES = 256 << 20
DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}


def kernel_source_digest() -> str:
    """sha256 over the HIP sources and headers: ties committed counter data to this kernel build."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_decode_blocks_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h", ".cpp")):
            h.update(name.encode())
            h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()[:16]


def workload_label(cfg, step_desc):
    lens = cfg.lengths
    if lens[0] == "const":
        ctx = f"ctx {lens[1]}"
    elif lens[0] == "fixed":
        ctx = "ctx {" + ",".join(map(str, lens[1])) + "}"
    else:
        ctx = f"ctx {lens[0]}[{lens[1]},{lens[2]}]"
    return (f"{cfg.name}: B{cfg.B} Hq{cfg.H_q}/Hkv{cfg.H_kv} D{cfg.D} {cfg.dtype} bs{cfg.block_size} {ctx}, "
            f"{step_desc}")


def traffic_from_profile(workload: str, digest: str):
    """HBM bytes per launch from a committed counter summary, if it was taken on this exact kernel build."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None
    if d.get("kernel_src_digest") != digest:
        return None
    return d.get("hbm_bytes_per_launch")


def read_ceiling(pkv, torch, dev, nbytes: int = 4 << 30, reps: int = 6) -> float:
    """HBM read bandwidth (GB/s) of the library's plain streaming-read probe on this device.

    One 4 GiB read per launch (16x the Infinity Cache), best of a few grid sizes.
    """
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    best = 0.0
    for grid in (16384, 32768):
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            pkv.probe_stream_read(buf, sink, grid)
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / 1e3)
        best = max(best, nbytes / float(np.median(times[1:])) / 1e9)
    del buf
    return best


def cpu_baseline(w, step_bytes_total: float, kv_tokens: int, budget_s: float = 10.0):
    """Time the fp64 oracle (as it stands) on the host cores on the same step; bounded to ~budget_s."""
    import oracle
    threads = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        threads = min(threads, int(os.environ["OMP_NUM_THREADS"]))
    used = oracle.threads(threads)
    kp, vp = w.k_pool.copy(), w.v_pool.copy()
    times = []
    t_end = time.perf_counter() + budget_s
    while True:
        t0 = time.perf_counter()
        if w.positions is not None:
            oracle.kv_append(w.cfg.dtype, w.k_new, w.v_new, kp, vp, w.block_tables, w.positions, w.cfg.block_size)
        oracle.paged_decode_attention(w.cfg.dtype, w.q, kp, vp, w.block_tables, w.context_lens, w.scale,
                                      nthreads=used)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() >= t_end or len(times) >= 1000:
            break
    med = float(np.median(times))
    return {
        "value": round(step_bytes_total / med / 1e9, 3),
        "unit": "GB/s",
        "kv_tokens_per_s": round(kv_tokens / med, 1),
        "s_per_step": med,
        "cores": used,
        "kind": "oracle",
        "sample": f"the whole step of the same workload (seed {w.seed}), repeated {len(times)}x within "
                  f"~{budget_s:.0f} s; median per step; fp64 C + OpenMP over (request, head)",
    }


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="c2", choices=["c1", "c2", "c3", "c4", "c5"])
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--partition", type=int, default=None, help="split-KV partition size (default: the workload's)")
    ap.add_argument("--no-append", action="store_true", help="attention only (no kv_append in the step)")
    ap.add_argument("--rotate", type=int, default=0, help="input copies to rotate over (0 = enough to defeat MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--no-graph", action="store_true", help="launch every step eagerly (for counter runs)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes 5 times (scales HBM byte counters)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "this build runs on one GPU only: the step has no cross-GPU exchange; "
                                   "run with --gpus 1 (sharding is described in DESIGN.md)",
                          "n_gpus": args.gpus}))
        return 2

    import torch
    import paged_kv_decode_blocks_amd as pkv
    from workloads import get_config, make_workload, step_bytes
    from workloads.device import upload

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        return 3
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        n = args.copy_calibration // 4 * 4
        src = torch.ones(n // 4, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "dispatches": 5}))
        return 0
    lib = pkv.load_library()

    cfg = get_config(args.config)
    append = not args.no_append
    P = cfg.partition_size if args.partition is None else args.partition
    w = make_workload(cfg, args.seed, append=append)
    B, H_q, H_kv, D, bs = cfg.B, cfg.H_q, cfg.H_kv, cfg.D, cfg.block_size
    max_ctx = int(w.context_lens.max())
    sb = step_bytes(cfg, w.context_lens, append)
    bytes_per_step = sb["total"] if append else sb["attention_only"]
    kv_tokens = int(w.context_lens.sum())
    read_per_step = sb["kv_history"]

    R = args.rotate or max(2, math.ceil(4 * INFINITY_CACHE_BYTES / max(read_per_step, 1)))
    base = upload(w, dev)
    sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(R - 1)]
    ws_bytes = pkv.decode_workspace_bytes(B, H_q, D, max_ctx, P)
    calls = []
    P_ = ctypes.c_void_p
    dt = DTYPE_CODE[cfg.dtype]
    for s in sets:
        s["out"] = torch.empty((B, H_q, D), dtype=torch.float32, device=dev)
        s["ws"] = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
        if append:
            a = (dt, P_(s["out"].data_ptr()), P_(s["q"].data_ptr()), H_q * D, P_(s["k_new"].data_ptr()),
                 P_(s["v_new"].data_ptr()), H_kv * D, P_(s["k_pool"].data_ptr()), P_(s["v_pool"].data_ptr()),
                 P_(s["block_tables"].data_ptr()), w.block_tables.shape[1], P_(s["positions"].data_ptr()),
                 B, H_q, H_kv, D, bs, w.n_blocks, max_ctx, ctypes.c_float(float(w.scale)), P,
                 P_(s["ws"].data_ptr()), ws_bytes)
            calls.append((lib.pkv_append_decode_attention, a))
        else:
            a = (dt, P_(s["out"].data_ptr()), P_(s["q"].data_ptr()), H_q * D, P_(s["k_pool"].data_ptr()),
                 P_(s["v_pool"].data_ptr()), P_(s["block_tables"].data_ptr()), w.block_tables.shape[1],
                 P_(s["context_lens"].data_ptr()), B, H_q, H_kv, D, bs, w.n_blocks, max_ctx,
                 ctypes.c_float(float(w.scale)), P, P_(s["ws"].data_ptr()), ws_bytes)
            calls.append((lib.pkv_paged_decode_attention, a))

    def step(k):
        """One decode step on input set k % R, enqueued on torch's current stream."""
        fn, a = calls[k % R]
        rc = fn(*a, P_(torch.cuda.current_stream().cuda_stream))
        if rc:
            raise RuntimeError(f"step failed: {lib.pkv_status_string(rc).decode()}: {lib.pkv_last_error().decode()}")

    for k in range(args.warmup):
        step(k)
    launch = pkv.last_launch()
    torch.cuda.synchronize()

    # The step is launch-bound on the host for small batches, so the throughput
    # region replays a HIP graph holding one step per input set (the library
    # makes no allocation, memset or synchronisation, so it captures as is).
    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for k in range(R):
                step(k)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    reps, rem = divmod(args.steps, R) if graph is not None else (0, args.steps)
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g0.record(stream)
    for _ in range(reps):
        graph.replay()
    for k in range(rem):
        step(k)
    g1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gpu_region_s = g0.elapsed_time(g1) / 1e3

    # For reference: the same steps launched one by one, an event pair around
    # each launch (this adds the dispatch latency of every launch).
    n_ev = min(args.steps, 200)
    ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    torch.cuda.synchronize()
    for k in range(n_ev):
        ev0[k].record(stream)
        step(k)
        ev1[k].record(stream)
    torch.cuda.synchronize()

    launch_ms = np.array([a.elapsed_time(b) for a, b in zip(ev0, ev1)])
    value = bytes_per_step * args.steps / elapsed / 1e9
    # Per-step GPU time from the events around the replayed region: the step's
    # launches back to back, without the host's dispatch latency that an event
    # pair around a single eager launch also catches.
    gpu_step_s = gpu_region_s / args.steps
    achieved = bytes_per_step / gpu_step_s / 1e9
    ceiling = read_ceiling(pkv, torch, dev)
    digest = kernel_source_digest()
    traffic = traffic_from_profile(cfg.name + ("" if append else "_attn"), digest)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {
            "workload": workload_label(cfg, "kv_append + paged decode attention (fused)" if append
                                       else "paged decode attention"),
            "batch": B, "heads_q": H_q, "heads_kv": H_kv, "head_dim": D, "block_size": bs,
            "kv_tokens_per_step": kv_tokens, "max_context_len": max_ctx, "partition_size": P,
            "accumulate": "f32", "output": "f32", "seed": w.seed, "input_rotation_sets": R,
            "algorithmic_bytes_per_step": int(bytes_per_step), "launch": launch,
            "timed_loop": (f"{reps} replays of a HIP graph of {R} steps + {rem} eager steps" if graph is not None
                           else f"{rem} eager steps"),
        },
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBPS, 2),
        "kv_tokens_per_s": round(kv_tokens * args.steps / elapsed, 1),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
            "kernel": "decode attention launch(es) of one step (fused append; + LSE merge when split)",
            "gpu_us_per_step": round(gpu_step_s * 1e6, 2),
            "stream_read_probe_GBps": round(ceiling, 1),
            "frac_of_stream_read_probe": round(achieved / ceiling, 4),
            "eager_launch_us": {"mean": round(float(launch_ms.mean()) * 1e3, 2),
                          "p10": round(float(np.percentile(launch_ms, 10)) * 1e3, 2),
                          "p50": round(float(np.median(launch_ms)) * 1e3, 2),
                          "p90": round(float(np.percentile(launch_ms, 90)) * 1e3, 2)},
            "kernel_src_digest": digest,
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, bytes_per_step, kv_tokens, args.cpu_budget)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
