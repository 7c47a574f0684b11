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
GRAPH_MIN_STEPS = 32      # steps per replayed graph (cycling over the input sets): fewer graph launches
DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}


def _code_only(text: str) -> str:
    """C/C++ source with comments removed and whitespace runs collapsed (the digest ignores
    edits that cannot change the build; the sources hold no string with a comment marker)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_digest() -> str:
    """sha256 over the HIP sources and headers, comments excluded: ties committed counter
    data to the kernel sources it was taken with."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_decode_blocks_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h", ".cpp")):
            h.update(name.encode())
            h.update(_code_only(open(os.path.join(csrc, name), encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def workload_label(cfg, step_desc):
    lens = cfg.lengths
    if lens[0] == "const":
        ctx = f"ctx {lens[1]}"
    elif lens[0] == "fixed":
        ctx = "ctx {" + ",".join(map(str, lens[1])) + "}"
    else:
        ctx = f"ctx {lens[0]}[{lens[1]},{lens[2]}]"
    if getattr(cfg, "fp8", False):
        kv = f"{cfg.dtype} q, fp8 e4m3 K/V (per-row scales)"
    elif getattr(cfg, "mxfp4", False):
        kv = f"{cfg.dtype} q, mxfp4 e2m1 K/V (e8m0 scale per 32)"
    else:
        kv = cfg.dtype
    return (f"{cfg.name}: B{cfg.B} Hq{cfg.H_q}/Hkv{cfg.H_kv} D{cfg.D} {kv} bs{cfg.block_size} {ctx}, "
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


def host_cpu_model() -> str:
    """The host CPU's model string (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(w, step_bytes_total: float, kv_tokens: int, budget_s: float = 10.0):
    """Time the fp64 oracle (as it stands) on the host's cores on the same step, bounded to about
    budget_s, and on one thread on the batch's first requests (a sample of about 2 s)."""
    import oracle
    from workloads import step_bytes

    threads = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        threads = min(threads, int(os.environ["OMP_NUM_THREADS"]))
    used = oracle.threads(threads)
    kp, vp = w.k_pool.copy(), w.v_pool.copy()
    fp8 = getattr(w.cfg, "fp8", False)
    mx4 = getattr(w.cfg, "mxfp4", False)
    ks = vs = None
    if fp8 or mx4:
        ks, vs = w.k_scale.copy(), w.v_scale.copy()
    append = w.positions is not None

    def step(nthreads, k):
        """The oracle's append + attention for requests 0 .. k-1."""
        q, bt, cl = w.q[:k], w.block_tables[:k], w.context_lens[:k]
        if append:
            args = (w.cfg.dtype, w.k_new[:k], w.v_new[:k], kp, vp) + ((ks, vs) if ks is not None else ()) + \
                   (bt, w.positions[:k], w.cfg.block_size)
            (oracle.kv_append_mxfp4 if mx4 else oracle.kv_append_fp8 if fp8 else oracle.kv_append)(*args)
        if mx4:
            oracle.paged_decode_attention_mxfp4(w.cfg.dtype, q, kp, vp, ks, vs, bt, cl, w.scale, nthreads=nthreads)
        elif fp8:
            oracle.paged_decode_attention_fp8(w.cfg.dtype, q, kp, vp, ks, vs, bt, cl, w.scale, nthreads=nthreads)
        else:
            oracle.paged_decode_attention(w.cfg.dtype, q, kp, vp, bt, cl, w.scale, nthreads=nthreads)

    B = int(w.context_lens.size)
    times = []
    t_end = time.perf_counter() + budget_s
    while True:
        t0 = time.perf_counter()
        step(used, B)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() >= t_end or len(times) >= 1000:
            break
    med = float(np.median(times))
    # one thread: the first k requests, covering about 2 s of one-thread work (median of 3)
    frac = min(1.0, 2.0 / max(med * used, 1e-9))
    cum = np.cumsum(w.context_lens.astype(np.int64))
    k = int(min(max(int(np.searchsorted(cum, frac * cum[-1])) + 1, 1), B))
    t1 = []
    for _ in range(3):
        t0 = time.perf_counter()
        step(1, k)
        t1.append(time.perf_counter() - t0)
    med1 = float(np.median(t1))
    sb1 = step_bytes(w.cfg, w.context_lens[:k], append)["total"]
    return {
        "value": round(step_bytes_total / med / 1e9, 3),
        "unit": "GB/s",
        "kv_tokens_per_s": round(kv_tokens / med, 1),
        "s_per_step": med,
        "cores": used,
        "kind": "oracle",
        "cpu_model": host_cpu_model(),
        "host_logical_cpus": os.cpu_count(),
        "sample": f"the whole step of the same workload (seed {w.seed}), repeated {len(times)}x within "
                  f"~{budget_s:.0f} s on {used} threads; median per step; fp64 C + OpenMP over (request, head)",
        "one_thread": {
            "value": round(sb1 / med1 / 1e9, 4),
            "unit": "GB/s",
            "kv_tokens_per_s": round(float(cum[k - 1]) / med1, 1),
            "s_per_sample": med1,
            "sample": f"requests 0..{k - 1} of the batch ({int(cum[k - 1])} of {int(cum[-1])} context tokens, "
                      f"{int(sb1)} algorithmic bytes), append + attention on one thread, median of 3",
        },
    }


def resident_steps(lib, torch, pkv, dev, w, append: bool, P: int, R: int):
    """R device-resident copies of the workload's inputs and, for each, the C-ABI
    call (function, arguments without the trailing stream) of one decode step."""
    from workloads.device import upload

    cfg = w.cfg
    B, H_q, H_kv, D, bs = cfg.B, cfg.H_q, cfg.H_kv, cfg.D, cfg.block_size
    max_ctx = int(w.context_lens.max())
    base = upload(w, dev)
    sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(R - 1)]
    ws_bytes = pkv.decode_workspace_bytes(B, H_q, D, max_ctx, P)
    calls = []
    P_ = ctypes.c_void_p
    dt = DTYPE_CODE[cfg.dtype]
    for s in sets:
        s["out"] = torch.empty((B, H_q, D), dtype=torch.float32, device=dev)
        s["ws"] = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
        if cfg.fp8 or cfg.mxfp4:
            scales = (P_(s["k_scale"].data_ptr()), P_(s["v_scale"].data_ptr()))
            fa = lib.pkv_append_decode_attention_mxfp4 if cfg.mxfp4 else lib.pkv_append_decode_attention_fp8
            fd = lib.pkv_paged_decode_attention_mxfp4 if cfg.mxfp4 else lib.pkv_paged_decode_attention_fp8
            if append:
                a = (dt, P_(s["out"].data_ptr()), P_(s["q"].data_ptr()), H_q * D, P_(s["k_new"].data_ptr()),
                     P_(s["v_new"].data_ptr()), H_kv * D, P_(s["k_pool"].data_ptr()), P_(s["v_pool"].data_ptr()),
                     *scales, P_(s["block_tables"].data_ptr()), w.block_tables.shape[1],
                     P_(s["positions"].data_ptr()), B, H_q, H_kv, D, bs, w.n_blocks, max_ctx,
                     ctypes.c_float(float(w.scale)), P, P_(s["ws"].data_ptr()), ws_bytes)
                calls.append((fa, a))
            else:
                a = (dt, P_(s["out"].data_ptr()), P_(s["q"].data_ptr()), H_q * D, P_(s["k_pool"].data_ptr()),
                     P_(s["v_pool"].data_ptr()), *scales, P_(s["block_tables"].data_ptr()),
                     w.block_tables.shape[1], P_(s["context_lens"].data_ptr()), B, H_q, H_kv, D, bs, w.n_blocks,
                     max_ctx, ctypes.c_float(float(w.scale)), P, P_(s["ws"].data_ptr()), ws_bytes)
                calls.append((fd, a))
            continue
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
    return calls, sets


# (pattern, tile bytes, scale tiles, paths, teams, depths): the per-(block, KV head) reads of the
# grouped kernels at D = 128 -- MXFP4 codes 1 KiB per tile, FP8 codes 2 KiB, bf16 4 KiB; scale
# tiles 64 bytes per pool; paths bit 1 / 2 / 4 moves K / V / scales by DMA into LDS; depth =
# items in flight per wave.  The grouped MXFP4 kernel moves all three by DMA, one head per wave
# or a team of neighbouring heads (K, or K and V, into registers beside it for comparison); the
# FP8 kernel moves K by DMA and V and the scales into registers (all into registers beside it for
# comparison); the bf16 kernel has both.
TILE_PATTERNS = (
    ("mxfp4_registers", 1024, True, 0, (1, 4), (2, 4, 8)),
    ("mxfp4_dma", 1024, True, 7, (1, 4), (2, 4, 8)),
    ("mxfp4_k_registers", 1024, True, 6, (1, 4), (2, 4, 8)),
    ("mxfp4_kv_registers", 1024, True, 4, (1, 4), (2, 4, 8)),
    ("fp8_k_dma", 2048, True, 1, (1, 2, 4), (4,)),
    ("fp8_registers", 2048, True, 0, (1, 4), (4,)),
    ("bf16_registers", 4096, False, 0, (1,), (4,)),
    ("bf16_k_dma", 4096, False, 1, (1,), (4,)),
)


def tile_probe_ids(rng, n_blocks: int, heads: int, team: int, n: int):
    """Block ids for one launch of the tile-read probe: about n items (rounded down to whole
    rounds of the heads / team head groups), item t reading head group t mod (heads / team), and
    within each head group every block at most once, so that no tile is read twice."""
    groups = heads // team
    per_group = min(n // groups, n_blocks)
    per = rng.permuted(np.tile(np.arange(n_blocks, dtype=np.int32), (groups, 1)), axis=1)[:, :per_group]
    return np.ascontiguousarray(per.T).reshape(-1)


def tileprobe_bench(args, torch, pkv, dev) -> int:
    """The read rate of the grouped kernels' access patterns without their arithmetic
    (pkv_probe_tile_read), beside the plain streaming read: K/V pools of 512 Ki blocks x 8 KV
    heads (4, 8 or 16 GiB each, by tile size), about 1 GiB read per launch, item t reading block
    ids[t] for head group t mod (8 / team) with no tile read twice in one launch; four id sets
    rotate.  Each (pattern, team, depth, grid) point: four untimed launches, then 16 timed with events
    on the launch stream.  Grids of 512 .. 2048 four-wave workgroups put 8 .. 32 waves on each
    of the 256 CUs where the probe's registers and LDS let them be resident."""
    heads, n_blocks, reps, target = 8, 512 << 10, 16, 1 << 30
    big = n_blocks * heads * 4096
    kp = torch.zeros(big // 4, dtype=torch.int32, device=dev)
    vp = torch.zeros(big // 4, dtype=torch.int32, device=dev)
    ks = torch.zeros(n_blocks * heads * 64 // 4, dtype=torch.int32, device=dev)
    vs = torch.zeros_like(ks)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    rng = np.random.default_rng(args.seed or 7)
    ceiling = read_ceiling(pkv, torch, dev)
    grids = (512, 768, 1024, 2048)
    results = []

    def id_sets(tile, scales, team):
        n = target // (team * (2 * tile + (128 if scales else 0)))
        return [torch.from_numpy(tile_probe_ids(rng, n_blocks, heads, team, n)).to(dev) for _ in range(4)]

    def launch(sets, k, tile, scales, team, paths, depth, grid):
        return pkv.probe_tile_read(kp, vp, sets[k % 4], sink, heads=heads, tile_bytes=tile, team=team, paths=paths,
                                   depth=depth, k_scale=ks if scales else None, v_scale=vs if scales else None,
                                   grid=grid, stream=stream)

    first = True
    cached = {}
    for name, tile, scales, paths, teams, depths in TILE_PATTERNS:
        for team in teams:
            if (tile, scales, team) not in cached:
                cached[(tile, scales, team)] = id_sets(tile, scales, team)
            sets = cached[(tile, scales, team)]
            for depth in depths:
                for grid in grids:
                    for k in range(8 if first else 4):      # the first point of a process runs slow: warm up longer
                        launch(sets, k, tile, scales, team, paths, depth, grid)
                    first = False
                    torch.cuda.synchronize()
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    nbytes = 0
                    for k in range(reps):
                        nbytes += launch(sets, k, tile, scales, team, paths, depth, grid)
                    e1.record(stream)
                    torch.cuda.synchronize()
                    sec = e0.elapsed_time(e1) / 1e3
                    results.append({"pattern": name, "tile_bytes": tile, "scales": scales, "paths": paths,
                                    "team": team, "depth": depth, "grid": grid,
                                    "us_per_launch": round(sec / reps * 1e6, 2), "GBps": round(nbytes / sec / 1e9, 1)})
                    print(json.dumps(results[-1]), file=sys.stderr, flush=True)
    print(json.dumps({"mode": "tileprobe", "unit": "GB/s", "stream_read_GBps": round(ceiling, 1),
                      "heads": heads, "n_blocks": n_blocks, "bytes_per_launch_approx": target, "timed_launches": reps,
                      "results": results}))
    return 0


def cumask_bench(args) -> int:
    """Decode-step bandwidth on CU-limited streams, alone and beside a GEMM.

    Runs the library's standalone program pkv_cumask (a child process on the
    system ROCm runtime; PyTorch's bundled HIP runtime cannot create CU-masked
    queues here) on the workload's shape and lengths, and prints its result as
    one JSON line.  The parent never initialises the GPU.
    """
    if not os.environ.get("PKV_CUMASK_ENABLE"):
        # Switched off: the program ended with SIGSEGV and no output when started from a
        # Python process; it stays off until the cause is found.
        print(json.dumps({"mode": "cumask", "error": "disabled: pkv_cumask crashed (SIGSEGV, no output) when "
                                                     "started from Python; cause not found"}))
        return 4
    import subprocess
    from workloads import draw_lengths, get_config

    cfg = get_config(args.config)
    append = not args.no_append
    P = cfg.partition_size if args.partition is None else args.partition
    seed = args.seed if args.seed is not None else int(cfg.name[1:])
    lens = draw_lengths(cfg, np.random.default_rng(seed))
    factor = cfg.pool[1] if cfg.pool[0] == "factor" else 1.0
    prog = os.path.join(ROOT, "paged_kv_decode_blocks_amd", "pkv_cumask")
    if not os.path.exists(prog):
        print(json.dumps({"error": f"{prog} not built (paged_kv_decode_blocks_amd.build)"}))
        return 3
    cmd = [prog, "sweep", cfg.dtype, str(cfg.B), str(cfg.H_q), str(cfg.H_kv), str(cfg.D), str(P),
           "1" if append else "0", repr(float(factor)), str(seed), str(max(args.steps // 4, 20)),
           ",".join(str(int(x)) for x in lens)]
    # the program's own RUNPATH ($ORIGIN, /opt/rocm/lib) picks its libraries, not an inherited search path
    env = {k: v for k, v in os.environ.items() if k != "LD_LIBRARY_PATH"}
    r = subprocess.run(cmd, stdout=subprocess.PIPE, text=True, timeout=900, env=env)
    if r.returncode != 0:
        print(json.dumps({"error": f"pkv_cumask exited with {r.returncode}"}))
        return r.returncode
    res = json.loads(r.stdout.strip().splitlines()[-1])
    print(json.dumps({
        "mode": "cumask",
        "metric": "decode-step HBM bandwidth on CU-limited streams",
        "unit": "GB/s",
        "n_gpus": 1,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded finite values; lengths drawn as the workload's; resident, rotated past "
                "the Infinity Cache)",
        "config": {"workload": workload_label(cfg, ("fused append + attention" if append else "attention")
                                              + (f" (split {P})" if P else ""))},
        **res,
    }))
    return 0


def cufrac_bench(args, torch, pkv, dev, lib) -> int:
    """The decode step on a share of the CUs ([P2] section 3.3.1: a fraction of the
    GPU already draws most of the HBM bandwidth for decode attention), alone and
    beside a compute-bound neighbour on the other CUs.

    The step runs as n persistent 16-wave workgroups (pkv_append_decode_attention_persistent),
    each filling one CU's register file, so it occupies n CUs; the neighbour is the
    library's MFMA-bound probe (pkv_probe_mfma_burn), one 100 KiB-LDS workgroup per
    CU, launched first on N - n CUs so that exactly n stay free for the step.  This
    bounds the step's share of the GPU by occupancy instead of a CU-masked queue."""
    from workloads import get_config, make_workload, step_bytes

    cfg = get_config(args.config)
    if cfg.fp8 or cfg.mxfp4 or cfg.H_q != cfg.H_kv or cfg.dtype == "f32":
        print(json.dumps({"mode": "cufrac", "error": f"{args.config}: the persistent step takes f16/bf16 with "
                                                     "one query head per KV head (c2, c3, c4)"}))
        return 2
    P = cfg.partition_size if args.partition is None else args.partition
    w = make_workload(cfg, args.seed, append=True)
    sb = step_bytes(cfg, w.context_lens, True)
    bytes_per_step = sb["total"]
    R = args.rotate or max(2, math.ceil(4 * INFINITY_CACHE_BYTES / max(sb["kv_history"], 1)))
    calls, sets = resident_steps(lib, torch, pkv, dev, w, True, P, R)
    n_cus = int(lib.pkv_device_cu_count())
    P_ = ctypes.c_void_p
    sa = torch.cuda.Stream(device=dev)
    sg = torch.cuda.Stream(device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    K = max(args.steps // 10, 2 * R)

    def step(k, n_wg, stream):
        fn, a = calls[k % R]
        sp = P_(stream.cuda_stream)
        rc = lib.pkv_append_decode_attention_persistent(*a, n_wg, sp) if n_wg else fn(*a, sp)
        if rc:
            raise RuntimeError(f"step failed: {lib.pkv_status_string(rc).decode()}: {lib.pkv_last_error().decode()}")

    gemm = args.neighbour == "gemm"
    GM = GN = GK = 8192                        # the GEMM neighbour: 2 x 8192^3 flops per launch
    if gemm:
        gen = torch.Generator(device=dev)
        gen.manual_seed(11)
        ga = (torch.rand((GM, GK), generator=gen, device=dev) - 0.5).to(torch.bfloat16)
        gb = (torch.rand((GN, GK), generator=gen, device=dev) - 0.5).to(torch.bfloat16)
        gc = torch.empty((GM, GN), dtype=torch.float32, device=dev)

    def burn(n_wg, iters, stream):
        """The neighbour on n_wg CUs: `iters` GEMM launches, or an MFMA chain of `iters` rounds."""
        if gemm:
            for _ in range(iters):
                rc = lib.pkv_probe_gemm_bf16(n_wg, P_(ga.data_ptr()), P_(gb.data_ptr()), P_(gc.data_ptr()), GM, GN, GK,
                                             P_(stream.cuda_stream))
                if rc:
                    break
        else:
            rc = lib.pkv_probe_mfma_burn(n_wg, iters, P_(sink.data_ptr()), P_(stream.cuda_stream))
        if rc:
            raise RuntimeError(f"burn failed: {lib.pkv_status_string(rc).decode()}: {lib.pkv_last_error().decode()}")

    def time_steps(n_wg):
        for k in range(R):
            step(k, n_wg, sa)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(sa)
        for k in range(K):
            step(k, n_wg, sa)
        e1.record(sa)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / K

    def burn_flops(n_wg, iters):
        return iters * 2.0 * GM * GN * GK if gemm else n_wg * 16.0 * iters * 8 * 16384

    def time_burn(n_wg, iters):
        burn(n_wg, 1 if gemm else max(1, iters // 10), sg)
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(sg)
        burn(n_wg, iters, sg)
        g1.record(sg)
        torch.cuda.synchronize()
        return g0.elapsed_time(g1) * 1e-3

    t_full = time_steps(0)
    sweep = []
    for n in (8, 16, 32, 52, 64, 96, 128, 192, 256):
        if n > n_cus:
            continue
        t = time_steps(n)
        sweep.append({"cus": n, "cu_fraction": round(n / n_cus, 3), "us_per_step": round(t * 1e6, 2),
                      "GBps": round(bytes_per_step / t / 1e9, 1)})
    ref = max(r["GBps"] for r in sweep)
    for r in sweep:
        r["frac_of_best"] = round(r["GBps"] / ref, 3)
    print(json.dumps({"sweep_done": len(sweep)}), file=sys.stderr, flush=True)

    # neighbour shares in multiples of 32 CUs: workgroups are dealt over the shader engines,
    # so an uneven neighbour grid leaves some engines one free CU short and a step
    # workgroup waits for one (a 204-CU neighbour cut the 52-CU step to the 32-CU rate)
    corun = []
    iters0 = 2 if gemm else 20000
    for n in (32, 64, 96, 128, 192):
        if n >= n_cus:
            continue
        ta = time_steps(n)
        tb = time_burn(n_cus - n, iters0)
        # the neighbour outlasts the K steps
        iters = max(2 if gemm else 1000, math.ceil(iters0 * (K * ta * 1.3) / tb))
        tb_alone = time_burn(n_cus - n, iters)
        for k in range(R):
            step(k, n, sa)
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(sg)
        burn(n_cus - n, iters, sg)          # first: it takes N - n CUs, the step gets the rest
        g1.record(sg)
        e0.record(sa)
        for k in range(K):
            step(k, n, sa)
        e1.record(sa)
        torch.cuda.synchronize()
        ta2 = e0.elapsed_time(e1) * 1e-3 / K
        tb2 = g0.elapsed_time(g1) * 1e-3
        corun.append({"attention_cus": n, "neighbour_cus": n_cus - n,
                      "attention_alone_GBps": round(bytes_per_step / ta / 1e9, 1),
                      "attention_beside_neighbour_GBps": round(bytes_per_step / ta2 / 1e9, 1),
                      "neighbour_alone_TFLOPs": round(burn_flops(n_cus - n, iters) / tb_alone / 1e12, 1),
                      "neighbour_beside_attention_TFLOPs": round(burn_flops(n_cus - n, iters) / tb2 / 1e12, 1),
                      "neighbour_outlasts_steps": bool(tb2 >= K * ta2)})
    print(json.dumps({
        "mode": "cufrac", "metric": "decode step HBM GB/s on a share of the CUs", "unit": "GB/s",
        "config": {"workload": workload_label(cfg, "kv_append + paged decode attention (fused), persistent "
                                                   "16-wave workgroups"), "partition_size": P,
                   "algorithmic_bytes_per_step": int(bytes_per_step), "input_rotation_sets": R,
                   "steps_per_point": K, "n_cus": n_cus},
        "full_step_default_launch_GBps": round(bytes_per_step / t_full / 1e9, 1),
        "sweep": sweep, ("corun_gemm_neighbour" if gemm else "corun_mfma_neighbour"): corun,
        "neighbour": ("bf16 GEMM c[8192][8192] = a[8192][8192] b_t[8192][8192]^T streaming its operands through "
                      "LDS (pkv_probe_gemm_bf16), one 8-wave workgroup per CU" if gemm else
                      "bf16 MFMA chains on register operands (pkv_probe_mfma_burn), touching no memory"),
        "note": "share bounded by occupancy (one 16-wave workgroup per CU), not by a CU-masked queue"}))
    return 0


def dual_bench(args, torch, pkv, dev) -> int:
    """A local and an offloaded attention batch per step ([P2] section 3.2.1: the decode
    instance's own attention and the attention it offloaded run at the same time), replayed
    from pkv_dual_step_graphs captured as two parallel branches, against the same two steps
    captured one after the other and against each alone.  Each variant cycles over R copies
    of both batches' inputs (at least 1 GiB of K/V reads per cycle, so none is cached); one
    graph launch per step, K steps, timed with events on the launch stream."""
    from workloads import get_config, make_workload, step_bytes
    from workloads.device import upload

    cfgs = [get_config(args.local), get_config(args.offloaded)]
    ws = [make_workload(c, (args.seed or 0) + 500 + i, append=True) for i, c in enumerate(cfgs)]
    ctx_cap = max(int(w.max_context_len) for w in ws)
    ctx_cap = -(-ctx_cap // 16) * 16
    sb = [step_bytes(c, w.context_lens, True) for c, w in zip(cfgs, ws)]
    per_step = sum(x["total"] for x in sb)
    reads = sum(x["kv_history"] for x in sb)
    R = max(2, math.ceil((1 << 30) / reads))

    def branch(w, cfg):
        d = upload(w, dev)
        W = w.block_tables.shape[1]
        bt = torch.full((cfg.B, -(-ctx_cap // 16)), -1, dtype=torch.int32, device=dev)
        bt[:, :W] = d["block_tables"]
        b = {"q": d["q"], "k_new": d["k_new"], "v_new": d["v_new"], "k_pool": d["k_pool"], "v_pool": d["v_pool"],
             "block_tables": bt, "positions": d["positions"],
             "out": torch.empty((cfg.B, cfg.H_q, cfg.D), dtype=torch.float32, device=dev),
             "partition_size": cfg.partition_size}
        if cfg.fp8 or cfg.mxfp4:
            b["k_scale"], b["v_scale"] = d["k_scale"], d["v_scale"]
        return b

    sets = [[branch(w, c) for w, c in zip(ws, cfgs)] for _ in range(R)]
    B0, B1 = cfgs[0].B, cfgs[1].B
    stream = torch.cuda.current_stream(dev)
    scale = float(ws[0].scale)
    if float(ws[1].scale) != scale:
        raise SystemExit("both batches need the same head dim (one scale)")

    def time_variant(caps0, caps1, parallel, n0, n1):
        objs = [pkv.DualStepGraphs(s[0], s[1], scale, caps0, caps1, ctx_cap, parallel=parallel) for s in sets]
        for k in range(2 * R):
            objs[k % R].launch(n0, n1, stream=stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for k in range(args.steps):
            objs[k % R].launch(n0, n1, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        gpu = e0.elapsed_time(e1) / 1e3
        for o in objs:
            o.close()
        return gpu / args.steps, wall / args.steps

    res = {}
    for name, c0, c1, par, n0, n1 in (("parallel", [B0], [B1], True, B0, B1),
                                      ("serialized", [B0], [B1], False, B0, B1),
                                      ("local_alone", [B0], [0], True, B0, 0),
                                      ("offloaded_alone", [0], [B1], True, 0, B1)):
        g, wall = time_variant(c0, c1, par, n0, n1)
        byt = (sb[0]["total"] if n0 else 0) + (sb[1]["total"] if n1 else 0)
        res[name] = {"us_per_step": round(g * 1e6, 2), "wall_us_per_step": round(wall * 1e6, 2),
                     "GBps": round(byt / g / 1e9, 1)}
        print(json.dumps({"variant": name, **res[name]}), file=sys.stderr, flush=True)
    print(json.dumps({
        "mode": "dual", "metric": "decode step with a local and an offloaded attention batch (HBM GB/s)",
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "config": {"local": workload_label(cfgs[0], "fused append + attention"),
                   "offloaded": workload_label(cfgs[1], "fused append + attention"),
                   "ctx_cap": ctx_cap, "input_rotation_sets": R, "algorithmic_bytes_per_step": int(per_step),
                   "graphs": "one pkv_dual_step_graphs launch per step (parallel or serialized branches)"},
        "variants": res,
        "overlap_gain": round(res["serialized"]["us_per_step"] / res["parallel"]["us_per_step"], 3),
        "data": "synthetic (seeded; resident in HBM, rotated past the Infinity Cache)",
    }))
    return 0


def loop_bench(args, torch, pkv, dev) -> int:
    """A decode loop driven by the library's block manager.

    The workload's requests are registered with a pkv.BlockManager; every step
    the host asks it for the step's positions, copy pairs and block tables
    (pkv_bm_append_batch, straight into one packed pinned buffer), enqueues
    the copy of that buffer to the device, and then either enqueues
    copy_blocks + the fused append + attention one call at a time, or
    (--graphs) replays the captured step graph of the smallest fitting
    (batch, context) bucket; --native does all of that in one
    pkv_decoder_step call.  Two metadata buffer sets alternate so the host
    prepares step k+1 while the GPU runs step k.  Reported next to the same
    fused step on static tables.
    """
    from workloads import draw_lengths, get_config, kv_bytes_per_token

    cfg = get_config(args.config)
    seed = args.seed if args.seed is not None else 1000 + int(cfg.name[1:])
    rng = np.random.default_rng(seed)
    hist = draw_lengths(cfg, rng).astype(np.int64) - 1          # tokens already cached
    hist = np.maximum(hist, 0)
    B, H_q, H_kv, D, bs = cfg.B, cfg.H_q, cfg.H_kv, cfg.D, cfg.block_size
    total_steps = args.warmup + args.steps
    final = hist + total_steps
    need = int(((final + bs - 1) // bs).sum())
    factor = cfg.pool[1] if cfg.pool[0] == "factor" else 1.0
    n_blocks = max(int(math.ceil(factor * need)), need)
    W = int(((final.max() + bs - 1) // bs))
    P = cfg.partition_size if args.partition is None else args.partition
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[cfg.dtype]

    ids = np.arange(B, dtype=np.int64)
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    k_pool = (torch.randn((n_blocks, H_kv, bs, D), generator=g, device=dev) * cfg.kv_std).to(tdt)
    v_pool = (torch.randn((n_blocks, H_kv, bs, D), generator=g, device=dev) * cfg.kv_std).to(tdt)
    q = (torch.randn((B, H_q, D), generator=g, device=dev) * cfg.q_std).to(tdt)
    k_new = (torch.randn((B, H_kv, D), generator=g, device=dev) * cfg.kv_std).to(tdt)
    v_new = (torch.randn((B, H_kv, D), generator=g, device=dev) * cfg.kv_std).to(tdt)
    out = torch.empty((B, H_q, D), dtype=torch.float32, device=dev)
    bucket = 256                                      # context-capacity interval of the graph grid
    max_ctx_bound = int(final.max()) + 1
    ctx_caps = list(range(bucket, max_ctx_bound + bucket, bucket))
    W = max(W, ctx_caps[-1] // bs)                    # table rows reach the top context bucket
    ws_bytes = pkv.decode_workspace_bytes(B, H_q, D, ctx_caps[-1], P) if P else 0
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(D)
    main = torch.cuda.current_stream(dev)

    dec = None
    if args.native:
        caps = dict(batch_caps=[B], ctx_caps=ctx_caps) if args.graphs else {}
        dec = pkv.Decoder(q, k_new, v_new, k_pool, v_pool, out, scale, W, partition_size=P,
                          workspace=ws if P else None, shuffle_seed=seed, **caps)
        bm = dec.block_manager
    else:
        bm = pkv.BlockManager(n_blocks, bs, shuffle_seed=seed)
    for b in range(B):
        bm.add_sequence(b, int(hist[b]))

    # packed metadata: positions [B] | cow_src [B] | cow_dst [B] | block tables [B][W]
    meta_len = 3 * B + B * W
    pin = [torch.empty(meta_len, dtype=torch.int32, pin_memory=True) for _ in range(2)]
    dmeta = [torch.empty(meta_len, dtype=torch.int32, device=dev) for _ in range(2)]
    hv = [(m.numpy(), m.numpy()[3 * B:].reshape(B, W)) for m in pin]
    dv = [(m[:B], m[B:2 * B], m[2 * B:3 * B], m[3 * B:].view(B, W)) for m in dmeta]
    graphs = None
    if args.graphs and not args.native:
        graphs = [pkv.StepGraphs(q, k_new, v_new, k_pool, v_pool, dv[s][3], dv[s][0], out, scale, [B], ctx_caps,
                                 partition_size=P, cow_src=dv[s][1], cow_dst=dv[s][2], workspace=ws)
                  for s in range(2)]
    done = [torch.cuda.Event() for _ in range(2)]
    host_bm_s, copies = 0.0, 0

    def step(k):
        nonlocal host_bm_s, copies
        if dec is not None:
            h0 = time.perf_counter()
            copies += dec.step(ids, stream=main)
            host_bm_s += time.perf_counter() - h0
            return
        s = k % 2
        done[s].synchronize()          # step k-2 (which used this buffer set) has finished
        flat, tab = hv[s]
        h0 = time.perf_counter()
        _, pos, cow = bm.append_batch(ids, W, out_tables=tab, out_positions=flat[:B])
        host_bm_s += time.perf_counter() - h0
        n = len(cow)
        flat[B:3 * B] = -1
        if n:
            flat[B:B + n] = cow[:, 0]
            flat[2 * B:2 * B + n] = cow[:, 1]
            copies += n
        max_ctx = int(pos.max()) + 1
        dmeta[s].copy_(pin[s], non_blocking=True)         # in order on the compute stream
        if graphs is not None:
            graphs[s].launch(B, max_ctx, n, stream=main)
        else:
            d_pos, d_cs, d_cd, d_tab = dv[s]
            if n:
                pkv.copy_blocks(k_pool, v_pool, d_cs[:n], d_cd[:n], stream=main)
            pkv.append_decode_attention(q, k_new, v_new, k_pool, v_pool, d_tab, d_pos, scale, max_ctx,
                                        partition_size=P, out=out, workspace=ws if P else None, stream=main)
        done[s].record(main)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    host_bm_s = 0.0
    kv_read = 0.0
    per_tok = kv_bytes_per_token(H_kv, D, {"f32": 4, "f16": 2, "bf16": 2}[cfg.dtype])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(main)
    for k in range(args.warmup, total_steps):
        kv_read += float((hist + k).sum()) * per_tok      # history the step reads (before its append)
        step(k)
    e1.record(main)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu = e0.elapsed_time(e1) / 1e3

    # the same fused step on fixed tables, launched back to back
    tabs, lens = bm.batch_tables(ids, W)
    st_t = torch.from_numpy(tabs).to(dev)
    st_p = torch.from_numpy(lens - 1).to(dev)
    for _ in range(5):
        pkv.append_decode_attention(q, k_new, v_new, k_pool, v_pool, st_t, st_p, scale, int(lens.max()),
                                    partition_size=P, out=out, workspace=ws if P else None, stream=main)
    torch.cuda.synchronize()
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    f0.record(main)
    for _ in range(args.steps):
        pkv.append_decode_attention(q, k_new, v_new, k_pool, v_pool, st_t, st_p, scale, int(lens.max()),
                                    partition_size=P, out=out, workspace=ws if P else None, stream=main)
    f1.record(main)
    torch.cuda.synchronize()
    static_s = f0.elapsed_time(f1) / 1e3 / args.steps

    print(json.dumps({
        "mode": "loop",
        "metric": "decode steps driven by the host block manager" + (" (native decoder," if dec else " (python loop,")
                  + (" step graphs)" if args.graphs else " eager)"),
        "value": round(B * args.steps / wall, 1),
        "unit": "tokens/s",
        "higher_is_better": True,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 5),
        "gpu_ms_per_step": round(gpu / args.steps * 1e3, 5),
        "static_tables_eager_gpu_ms_per_step": round(static_s * 1e3, 5),
        # python loop: time in pkv_bm_append_batch; native: time in the whole pkv_decoder_step call
        "host_us_per_step": round(host_bm_s / args.steps * 1e6, 2),
        "host_us_measures": "pkv_decoder_step call" if dec else "pkv_bm_append_batch call",
        "kv_read_GBps_wall": round(kv_read / wall / 1e9, 1),
        "cow_block_copies": copies,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded device normals; lengths drawn as the workload's)",
        "config": {"workload": workload_label(cfg, "manager-driven fused append + attention"
                                                   + (f" (split {P})" if P else "")),
                   "n_blocks": n_blocks, "bt_stride": W, "partition_size": P,
                   "graph_buckets": [[B], [ctx_caps[0], ctx_caps[-1], bucket]] if args.graphs else None},
    }))
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="c4", choices=["c1", "c2", "c3", "c4", "c5", "c3f8", "c5f8", "c3f4", "c5f4"],
                    help="the headline workload (default c4, the largest that fits one GPU)")
    ap.add_argument("--also", default="c2,c3,c5",
                    help="more workloads timed the same way in the same run, reported under other_workloads "
                         "(comma-separated; 'none' for only --config)")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--partition", type=int, default=None, help="split-KV partition size (default: the workload's)")
    ap.add_argument("--no-append", action="store_true", help="attention only (no kv_append in the step)")
    ap.add_argument("--rotate", type=int, default=0, help="input copies to rotate over (0 = enough to defeat MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--no-graph", action="store_true", help="launch every step eagerly (for counter runs)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes 5 times (scales HBM byte counters)")
    ap.add_argument("--local", default="c2", help="dual mode: the local batch's workload")
    ap.add_argument("--offloaded", default="c2", help="dual mode: the offloaded batch's workload")
    ap.add_argument("--mode", default="step", choices=["step", "loop", "cumask", "cufrac", "dual", "tileprobe"],
                    help="step: the headline step over resident inputs; loop: a block-manager-driven decode loop")
    ap.add_argument("--graphs", action="store_true", help="loop mode: replay captured step graphs")
    ap.add_argument("--native", action="store_true", help="loop mode: one pkv_decoder_step call per step")
    ap.add_argument("--neighbour", default="gemm", choices=["gemm", "mfma"],
                    help="cufrac mode: the work on the other CUs (an HBM-streaming GEMM or MFMA chains)")
    ap.add_argument("--gemm-only", type=int, default=0, metavar="N_WG",
                    help="only run the GEMM neighbour 3 times on N_WG workgroups (for its counter runs)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "one GPU only: the step has no cross-GPU exchange (each GPU would run its own "
                                   "shard of requests or KV heads); run with --gpus 1",
                          "n_gpus": args.gpus}))
        return 2

    if args.mode == "cumask":
        return cumask_bench(args)

    import torch
    import paged_kv_decode_blocks_amd as pkv
    from workloads import get_config, make_workload, step_bytes

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
    if args.gemm_only:
        g = 8192
        ga = torch.zeros((g, g), dtype=torch.bfloat16, device=dev)
        gc = torch.empty((g, g), dtype=torch.float32, device=dev)
        for _ in range(3):
            pkv.probe_gemm_bf16(ga, ga, gc, args.gemm_only)
        torch.cuda.synchronize()
        print(json.dumps({"gemm_only": args.gemm_only, "M": g, "N": g, "K": g, "dispatches": 3}))
        return 0
    if args.mode == "loop":
        return loop_bench(args, torch, pkv, dev)
    if args.mode == "dual":
        return dual_bench(args, torch, pkv, dev)
    if args.mode == "cufrac":
        return cufrac_bench(args, torch, pkv, dev, lib)
    if args.mode == "tileprobe":
        return tileprobe_bench(args, torch, pkv, dev)

    names = [args.config] + [c for c in (args.also.split(",") if args.also not in ("", "none") else [])
                             if c and c != args.config]
    result = None
    others = {}
    ceiling = read_ceiling(pkv, torch, dev)
    for i, name in enumerate(names):
        r = measure_step(name, args, torch, pkv, dev, lib, cpu=(i == 0 and not args.no_cpu_baseline), ceiling=ceiling)
        print(json.dumps({"measured": name, "pct_of_peak": r["pct_of_peak"], "frac": r["roofline"]["frac"]}),
              file=sys.stderr, flush=True)
        if i == 0:
            result = r
        else:
            others[name] = {k: r[k] for k in ("value", "unit", "pct_of_peak", "ms_per_step", "kv_tokens_per_s",
                                              "dtype")}
            others[name]["workload"] = r["config"]["workload"]
            others[name]["launch"] = r["config"]["launch"]
            others[name]["algorithmic_bytes_per_step"] = r["config"]["algorithmic_bytes_per_step"]
            others[name]["roofline"] = {k: r["roofline"][k] for k in ("achieved", "frac", "traffic", "gpu_us_per_step",
                                                                      "size_matched_read_probe")}
    if others:
        result["other_workloads"] = others
    print(json.dumps(result), flush=True)
    return 0


def size_matched_read_probe(pkv, torch, dev, nbytes: int, kernel_grid: int, reps: int = 32):
    """Best HBM read rate (GB/s) of the plain streaming-read probe over reads of the step's own
    size, at the attention launch's grid and at other grid sizes: a ceiling for one launch that
    moves that many bytes.  Successive launches read different slices of a buffer of at least
    1 GiB + 4x the Infinity Cache, so no slice is cached; launches are replayed from a graph."""
    nbytes = max(nbytes // 4096 * 4096, 4096)
    n_slices = max(2, math.ceil((4 * INFINITY_CACHE_BYTES + (1 << 30)) / nbytes))
    buf = torch.empty(n_slices * nbytes // 4, dtype=torch.int32, device=dev)
    buf.fill_(1)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    res = {}
    for grid in sorted({int(kernel_grid), 256, 1024, 2048, 4096, 8192, 16384}):
        if grid < 1:
            continue

        def launch(k):
            pkv.probe_stream_read(buf[(k % n_slices) * nbytes // 4:], sink, grid, nbytes=nbytes)

        for k in range(2):
            launch(k)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for k in range(reps):
                launch(k)
        gr.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        gr.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        res[grid] = round(nbytes * reps / (e0.elapsed_time(e1) / 1e3) / 1e9, 1)
        del gr
    del buf
    best = max(res, key=res.get)
    return {"bytes": nbytes, "best_GBps": res[best], "best_grid": best, "kernel_grid": int(kernel_grid),
            "GBps_by_grid": {str(k): v for k, v in sorted(res.items())}}


def measure_step(name, args, torch, pkv, dev, lib, cpu: bool, ceiling: float):
    """Time K decode steps of workload `name` (fused append + attention, + merge when split)
    over device-resident inputs; returns the bench's JSON record for it."""
    from workloads import get_config, make_workload, step_bytes

    cfg = get_config(name)
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
    calls, sets = resident_steps(lib, torch, pkv, dev, w, append, P, R)
    P_ = ctypes.c_void_p

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
    # region replays HIP graphs of steps (the library makes no allocation, memset
    # or synchronisation, so it captures as is): one of G >= GRAPH_MIN_STEPS steps
    # cycling over the R input sets (each replay also pays a fixed cost), and one
    # of the remaining steps.
    graph = tail = None
    G = R * max(1, math.ceil(GRAPH_MIN_STEPS / R))
    reps, rem = divmod(args.steps, G) if not args.no_graph else (0, args.steps)

    def capture(n):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for k in range(n):
                step(k)
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        return gr

    if not args.no_graph:
        graph = capture(G)
        if rem:
            tail = capture(rem)
    stream = torch.cuda.current_stream(dev)
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g0.record(stream)
    for _ in range(reps):
        graph.replay()
    if tail is not None:
        tail.replay()
    else:
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
    kernel_grid = int(launch.split("grid=")[1].split()[0]) if "grid=" in launch else 1024
    probe = size_matched_read_probe(pkv, torch, dev, int(read_per_step), kernel_grid)
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
        "dtype": "fp8_e4m3" if cfg.fp8 else ("mxfp4_e2m1" if cfg.mxfp4 else cfg.dtype),
        "data": "synthetic",
        "config": {
            "workload": workload_label(cfg, "kv_append + paged decode attention (fused)" if append
                                       else "paged decode attention"),
            "batch": B, "heads_q": H_q, "heads_kv": H_kv, "head_dim": D, "block_size": bs,
            "kv_tokens_per_step": kv_tokens, "max_context_len": max_ctx, "partition_size": P,
            "accumulate": "f32", "output": "f32", "seed": w.seed, "input_rotation_sets": R,
            "algorithmic_bytes_per_step": int(bytes_per_step), "launch": launch,
            "timed_loop": (f"{reps} replays of a HIP graph of {G} steps (input sets cycled)"
                           + (f" + one graph of {rem} steps" if rem else "") if graph is not None
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
            "size_matched_read_probe": probe,
            "frac_of_size_matched_read_probe": round(achieved / probe["best_GBps"], 4),
            "eager_launch_us": {"mean": round(float(launch_ms.mean()) * 1e3, 2),
                          "p10": round(float(np.percentile(launch_ms, 10)) * 1e3, 2),
                          "p50": round(float(np.median(launch_ms)) * 1e3, 2),
                          "p90": round(float(np.percentile(launch_ms, 90)) * 1e3, 2)},
            "kernel_src_digest": digest,
        },
    }
    if cpu:
        result["cpu_baseline"] = cpu_baseline(w, bytes_per_step, kv_tokens, args.cpu_budget)
    del calls, sets
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return result


if __name__ == "__main__":
    sys.exit(main())
