"""Benchmark of the flag-gated shard-decomposed AG+GEMM on one MI355X.

One step = one pass of the whole hot path over one batch: the producer fills
the inbox and raises the per-(shard, k-tile) flags on one stream while the
flag-gated consumer GEMM runs on another (the Push model of the "Eliminating
Multi-GPU Performance Taxes" analysis page). Inputs are seeded synthetic fp16
uniform[-1, 1] and resident in HBM before timing starts.

Before the counted warmup steps the step runs untimed for --prewarm-ms (default
300 ms), so that the engine clock, which needs a few tens of milliseconds of
continuous load to settle, is at its steady value when timing starts.

Prints one JSON line. Besides the required fields it carries:
  roofline      the consumer kernel (the dominant one) against the fp16 MFMA
                or HBM peak, timed with HIP events on the consumer's stream;
  cpu_baseline  the CPU oracle timed on a bounded sample of the same workload;
  ladder        the same-GPU BSP ladder: BSP with host barrier, BSP with a
                device-side dependency only, fused, consumer alone (flags set).
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

W_DEF, K_DEF, N_DEF = 8, 8192, 28672
WORKLOADS = {
    # name: (W, M, K, N, c_dtype, release schedule)
    "tiny_m8": (8, 8, 512, 256, "f32", None),
    "decode_m1": (W_DEF, 1, K_DEF, N_DEF, "f16", None),
    "xover_m128": (W_DEF, 128, K_DEF, N_DEF, "f16", None),
    "prefill_m4096": (W_DEF, 4096, K_DEF, N_DEF, "f16", None),
    "ooo_m512": (W_DEF, 512, K_DEF, N_DEF, "f16", "random"),
}
# Flash-Decode combine (the pages' Flash-Decode shape: 96 query heads, d = 128, W = 8 ranks):
# name: (W, H, D, heads per flag tile, output dtype, max delay between tile releases in ns)
FD_WORKLOADS = {
    "fd_combine_h96": (8, 96, 128, 16, "f16", 2_000),
}
# MI355X published peaks
PEAK_FP16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


CSRC = os.path.join(ROOT, "shard_decomposed_gemm_amd", "csrc")
KERNEL_SOURCES = {"mfma": ("gemm_mfma.hip", "mfma_sched.h", "agemm_internal.h", "guard_units.h"),
                  "small_m": ("gemm_small_m.hip", "agemm_internal.h", "guard_units.h"),
                  "fd": ("fd_combine.hip", "fd_internal.h", "agemm_internal.h")}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "consumer_hbm_traffic.md")


def device_peaks(measure: bool) -> dict:
    """The peaks the rooflines use (published), the same derived from the device
    properties, and the device's measured ceilings (register-only fp16 MFMA loop,
    streaming read of 2 GiB, beyond the 256 MB last-level cache) as secondary
    references."""
    import torch
    from shard_decomposed_gemm_amd import agemm
    info = agemm.device_info()
    derived = {
        # CDNA4: 4096 dense fp16 FLOP per clock per CU. HBM3E: 4 bits per pin per
        # reported memory clock (8 Gb/s per pin at the 2 GHz the properties give).
        "fp16_tflops": info["cus"] * 4096 * info["clock_khz"] * 1e3 / 1e12,
        "hbm_gbs": 4.0 * info["mem_clock_khz"] * 1e3 * info["bus_bits"] / 8 / 1e9,
    }
    out = {"published": {"fp16_tflops": PEAK_FP16_TFLOPS, "hbm_gbs": PEAK_HBM_GBS},
           "device_props": dict(info, **{k + "_from_props": v for k, v in derived.items()})}
    if measure:
        buf = torch.zeros(2 << 30, dtype=torch.uint8, device="cuda")
        out["measured"] = {"mfma_f16_register_loop_tflops": agemm.probe_mfma(100, 30),
                           "stream_read_gbs": agemm.probe_read(buf, 10, 20), "read_bytes": buf.numel()}
        del buf
        torch.cuda.synchronize()
    return out


def kernel_digest(kind: str) -> str:
    """Digest of the consumer kernel's sources, comments and blank space left out:
    counter figures taken from another version of the kernel's code are not reported."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind]:
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)   # block comments
        text = re.sub(r"//[^\n]*", " ", text)                 # line comments
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kind: str):
    """HBM bytes per launch of the consumer kernel, from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of known size); None if there is
    none for this workload or the kernel has changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    digest = kernel_digest(kind)
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if not line.startswith("traffic:"):
                continue
            kv = dict(x.split("=", 1) for x in line.split()[1:] if "=" in x)
            if kv.get("workload") == workload and kv.get("digest") == digest:
                return float(kv["bytes_per_launch"])
    return None


def algorithmic(W, M, K, N, c_bytes):
    flops = 2.0 * M * K * N
    consumer_bytes = 2.0 * K * N + 2.0 * M * K + c_bytes * M * N  # B once, A once, C once
    path_bytes = 2.0 * K * N + 6.0 * M * K + c_bytes * M * N      # + producer read and inbox write
    return flops, consumer_bytes, path_bytes


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(W, M, K, N, budget_s: float):
    """The oracle as it stands, on a bounded row sample of the same workload. The oracle
    splits rows over its threads, so the sample is a multiple of the thread count (one
    row per thread at M = 1 is all there is)."""
    import oracle
    import synth
    threads = oracle.default_threads()
    b = synth.matrix_f16(0xB002, K, N)
    a = synth.matrix_f16(0xA100 + M, M, K)
    # one row per thread first (this includes the oracle's own fp16 decode of B), then a
    # sample sized to the budget
    rows = min(M, threads)
    t0 = time.perf_counter()
    oracle.sharded_gemm(synth.shards(a[:rows], W), b, nthreads=threads)
    t1 = time.perf_counter() - t0
    # grow the sample until it takes at least half the budget (the decode of B is a
    # fixed cost of every call, so a first estimate undershoots)
    for _ in range(3):
        if t1 >= budget_s / 2 or rows >= M:
            break
        rows = min(M, rows * max(2, int(budget_s / t1)))
        t0 = time.perf_counter()
        oracle.sharded_gemm(synth.shards(a[:rows], W), b, nthreads=threads)
        t1 = time.perf_counter() - t0
    flops = 2.0 * rows * K * N
    cores = min(threads, rows)
    return {"value": flops / t1 / 1e12, "unit": "TFLOP/s", "cores": cores, "cpu_model": cpu_model(),
            "host_cpus": os.cpu_count(), "kind": "oracle",
            "sample": f"{rows} of {M} rows at full K={K}, N={N}, W={W} (binary64, {cores} threads, {t1:.2f} s, "
                      f"including the oracle's decode of B)",
            "seconds": t1}


def prewarm(step, ms: float) -> int:
    """Runs the step, untimed, for at least `ms` milliseconds of wall clock: the GPU's
    engine clock takes a few tens of milliseconds of continuous load to reach its
    steady value (measured: a register-only MFMA loop runs at 72 % of its steady rate
    in its first 3 ms launch and needs about 20 back-to-back launches to settle)."""
    import torch
    n, t0 = 0, time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            step(n)
            n += 1
        torch.cuda.synchronize()
    return n


def fd_cpu_baseline(W, H, D, budget_s: float):
    """The combine oracle as it stands (numpy, binary64, one thread), called repeatedly
    on the same partials for a bounded time."""
    import synth
    from oracle import fd as fdo
    o, lse = synth.fd_partials(0x7A00, W, H, D)
    n, t0 = 0, time.perf_counter()
    while True:
        fdo.combine(o, lse)
        n += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s or n >= 100000:
            break
    return {"value": dt / n * 1e6, "unit": "us per combine", "cores": 1, "kind": "oracle",
            "sample": f"{n} combines of W={W} partials (H={H}, D={D}, binary64) in {dt:.2f} s", "seconds": dt}


def interleaved_ladder(variants, n: int, reps: int, timeit):
    """Times each variant (name, step function, enter, leave; enter and leave may be None)
    in `reps` interleaved passes of n steps, the order rotated by one every pass, so that a
    drift of the clock hits every variant alike. Returns the best pass of each variant and
    every pass's value (microseconds per step)."""
    passes = {v[0]: [] for v in variants}
    for rep in range(reps):
        k = rep % len(variants)
        for name, fn, enter, leave in variants[k:] + variants[:k]:
            if enter:
                enter()
            passes[name].append(timeit(fn, n))
            if leave:
                leave()
    return ({name: float(min(v)) for name, v in passes.items()},
            {name: [round(float(x), 1) for x in v] for name, v in passes.items()})


def run_fd(args):
    """One step = producer of the W ranks' partial tiles (seeded release order and
    delays) || flag-gated combine, on two streams."""
    import numpy as np
    import torch
    import synth
    from shard_decomposed_gemm_amd import FdCombine

    W, H, D, HT, odt, max_delay = FD_WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] workload={args.workload} W={W} H={H} D={D} heads/tile={HT} out={odt}", file=sys.stderr, flush=True)
    o, lse = synth.fd_partials(0x7A00, W, H, D)
    do = [torch.from_numpy(x).to(dev) for x in o]
    dl = [torch.from_numpy(x).to(dev) for x in lse]
    Os = [torch.empty((H, D), dtype=torch.float16 if odt == "f16" else torch.float32, device=dev) for _ in range(2)]
    ctx = FdCombine(W, H, D, heads_per_tile=HT, out_dtype=odt)
    sched = synth.schedule(0x7A01, ctx.t, max_delay)
    sp, sc = ctx.streams()
    torch.cuda.synchronize()

    def step(i):
        ctx.produce(do, dl, schedule=sched, stream=sp)
        ctx.run_fused(Os[i & 1], stream=sc)

    def timeit(fn, n):
        for i in range(max(3, n // 5)):
            fn(i)
        torch.cuda.synchronize()
        t = time.perf_counter()
        for i in range(n):
            fn(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t) * 1e6 / n

    prewarm(step, args.prewarm_ms)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    us_step = (time.perf_counter() - t0) * 1e6 / args.steps
    ctx.check()
    ctx.timing_begin(args.steps)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    kern = ctx.timing_end()
    ctx.check()
    kavg = float(np.mean(kern))
    # algorithmic bytes of the combine kernel: every partial read once, the output written once
    obytes = 2 if odt == "f16" else 4
    cons_bytes = 4.0 * W * H * D + 4.0 * W * H + obytes * H * D
    roof = {"bound": "hbm", "achieved": cons_bytes / (kavg * 1e-6) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": cons_bytes / (kavg * 1e-6) / 1e9 / PEAK_HBM_GBS, "traffic": None,
            "kernel": "flag-gated Flash-Decode combine (one wave per head)", "kernel_digest": kernel_digest("fd"),
            "algorithmic_bytes_per_launch": cons_bytes, "kernel_us_avg": kavg, "kernel_us_min": float(np.min(kern)),
            "kernel_us_p10_p50_p90": [float(x) for x in np.percentile(kern, [10, 50, 90])],
            "note": "latency-bound: 0.4 MB per launch is far below what one launch takes to stream at HBM speed"}
    ladder = None
    if not args.no_ladder:
        def flags_up():
            ctx.produce(do, dl)
            torch.cuda.synchronize()

        best, passes = interleaved_ladder([
            ("bsp_host_sync_us", lambda i: ctx.run_bsp(do, dl, Os[i & 1], schedule=sched, host_sync=True, stream=sc),
             None, None),
            ("bsp_device_dep_us", lambda i: ctx.run_bsp(do, dl, Os[i & 1], schedule=sched, host_sync=False, stream=sc),
             None, None),
            ("fused_us", step, None, None),
            ("consumer_only_us", lambda i: ctx.run_fused(Os[i & 1], stream=sc), flags_up, None),
        ], max(20, args.steps // args.sweep_reps), args.sweep_reps, timeit)
        ctx.check()
        ladder = dict(best)
        ladder["fused_speedup_vs_bsp"] = best["bsp_host_sync_us"] / best["fused_us"]
        ladder["fused_speedup_vs_bsp_device_dep"] = best["bsp_device_dep_us"] / best["fused_us"]
        ladder["method"] = (f"best of {args.sweep_reps} interleaved passes of "
                            f"{max(20, args.steps // args.sweep_reps)} steps, order rotated each pass")
        ladder["passes"] = passes
        print(f"[bench] ladder: {json.dumps(ladder)}", file=sys.stderr, flush=True)
    peaks = device_peaks(not args.no_peaks)
    if "measured" in peaks:
        roof["frac_of_measured_ceiling"] = roof["achieved"] / peaks["measured"]["stream_read_gbs"]
    cpu = None if args.no_cpu else fd_cpu_baseline(W, H, D, min(args.cpu_budget, 10.0))
    line = {
        "metric": "Flash-Decode combine step latency (producer of W partials || flag-gated combine)",
        "value": us_step, "unit": "us", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "prewarm_ms": args.prewarm_ms,
        "ms_per_step": us_step * 1e-3, "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": args.workload, "W": W, "H": H, "D": D, "heads_per_tile": HT, "out_dtype": odt,
                   "tiles": ctx.t, "schedule": f"seeded permutation, cumulative U[0,{max_delay // 1000}] us delays",
                   "release_span_us": float(sched[1][-1]) / 1e3},
        "roofline": roof, "cpu_baseline": cpu, "ladder": ladder, "peaks": peaks,
    }
    print(json.dumps(line), flush=True)
    ctx.close()


def run_sweep(args):
    """The fused-vs-BSP ladder across M at the sweep shape of the analysis page's
    AG+GEMM experiments (W = 8, K = 8192, N = 28672, M varied), fp16 C, shard order."""
    import numpy as np
    import torch
    import synth
    from shard_decomposed_gemm_amd import Context

    Ms = [int(x) for x in args.sweep.split(",") if x.strip()]
    W, K, N = W_DEF, K_DEF, N_DEF
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    to_dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.float16)).to(dev)
    B0 = to_dev(synth.matrix_f16(0xB002, K, N))
    Bs = [B0, B0.clone()]
    rows = []

    def timeit(fn, n):
        for i in range(max(3, n // 5)):
            fn(i)
        torch.cuda.synchronize()
        t = time.perf_counter()
        for i in range(n):
            fn(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t) * 1e6 / n

    for M in Ms:
        print(f"[sweep] M={M}", file=sys.stderr, flush=True)
        shards = [to_dev(x) for x in synth.shards(synth.matrix_f16(0xA100 + M, M, K), W)]
        Cs = [torch.empty((M, N), dtype=torch.float16, device=dev) for _ in range(2)]
        ctx = Context(W, M, K, N, c_dtype="f16")
        sp, sc = ctx.streams()

        def fused_step(i):
            ctx.produce(shards, stream=sp)
            ctx.run_fused(Bs[i & 1], Cs[i & 1], stream=sc)

        prewarm(fused_step, args.prewarm_ms)
        n = args.steps
        r = {"M": M, "consumer": ctx.consumer_info()}
        # fused and the BSP variants interleaved, so a clock drift hits them alike;
        # each keeps its best of the passes
        for rep in range(args.sweep_reps):
            r.setdefault("fused_us", []).append(timeit(fused_step, n))
            r.setdefault("bsp_host_sync_us", []).append(timeit(
                lambda i: ctx.run_bsp(shards, Bs[i & 1], Cs[i & 1], host_sync=True, stream=sc), n))
            r.setdefault("bsp_device_dep_us", []).append(timeit(
                lambda i: ctx.run_bsp(shards, Bs[i & 1], Cs[i & 1], host_sync=False, stream=sc), n))
            r.setdefault("pull_us", []).append(timeit(
                lambda i: ctx.run_pull(shards, Bs[i & 1], Cs[i & 1], stream=sc), n))
            ctx.set_strict_acquire(True)
            r.setdefault("fused_strict_acquire_us", []).append(timeit(fused_step, n))
            ctx.set_strict_acquire(False)
        ctx.produce(shards)
        torch.cuda.synchronize()
        r["consumer_only_us"] = [timeit(lambda i: ctx.run_fused(Bs[i & 1], Cs[i & 1], stream=sc), n)]
        ctx.check()
        r["passes"] = {k: [round(float(x), 1) for x in v] for k, v in r.items() if k.endswith("_us")}
        for k in list(r):
            if k.endswith("_us"):
                r[k] = float(min(r[k]))
        r["tflops_fused"] = 2.0 * M * K * N / (r["fused_us"] * 1e-6) / 1e12
        print(json.dumps(r), flush=True)
        rows.append(r)
        ctx.close()
        del shards, Cs
    print("\n| M | consumer | fused | fused, strict acquire | BSP host sync | BSP device dep | Pull | consumer alone "
          "| fused vs BSP (host / device) |")
    print("|---|---|---|---|---|---|---|---|---|")
    for r in rows:
        c = r["consumer"]
        kern = ("small-M" if c["kind"] == "small_m" else
                f"cfg {c['tile_config']}, {c['tiles']} tiles / {c['grid']} WG" + (", split" if c["split"] else ""))
        print(f"| {r['M']} | {kern} | {r['fused_us']:.1f} | {r['fused_strict_acquire_us']:.1f} | "
              f"{r['bsp_host_sync_us']:.1f} | "
              f"{r['bsp_device_dep_us']:.1f} | {r['pull_us']:.1f} | {r['consumer_only_us']:.1f} | "
              f"{r['bsp_host_sync_us'] / r['fused_us']:.3f}x / {r['bsp_device_dep_us'] / r['fused_us']:.3f}x |")


def calibrate_copy(steps: int):
    """A plain device-to-device copy of 1 GiB: the known byte count (1 GiB read, 1 GiB
    written per dispatch) against which FETCH_SIZE / WRITE_SIZE are scaled."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(max(1, steps)):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / max(1, steps)
    print(json.dumps({"calibration": "copy", "bytes_read": n, "bytes_written": n, "us_per_copy": dt * 1e6,
                      "GBps_read_plus_write": 2 * n / dt / 1e9}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the pages' methodology: 500 timed iterations after 100 warmup iterations
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="prefill_m4096", choices=list(WORKLOADS) + list(FD_WORKLOADS))
    ap.add_argument("--sweep", default=None,
                    help="comma-separated M values at K=8192, N=28672, W=8: the fused / BSP / Pull ladder "
                         "per M (one JSON object per M, then a markdown table); no headline line")
    ap.add_argument("--sweep-reps", type=int, default=4,
                    help="interleaved passes per variant in the ladder and in --sweep (the best pass is kept)")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work for cpu_baseline (the timed sample takes 10 to 20 s)")
    ap.add_argument("--prewarm-ms", type=float, default=300.0,
                    help="untimed steps for this long before the warmup steps, so the engine clock has settled")
    ap.add_argument("--order", choices=["shard", "arrival"], default="shard",
                    help="flag-tile order of the fused consumer (agemm_set_order)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-ladder", action="store_true")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured ceilings (fp16 MFMA register loop, streaming read)")
    ap.add_argument("--one-stream", action="store_true",
                    help="producer and consumer on one stream (the consumer then finds every flag up); "
                         "for counter collection, which serialises kernel dispatches")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for the HBM byte counters)")
    ap.add_argument("--probe-mfma", type=int, default=0, metavar="LAUNCHES",
                    help="only run the register-only fp16 MFMA loop for LAUNCHES launches (about 1.8 ms each) "
                         "and print its rate: a pure MFMA load, e.g. to read clocks and power beside the GEMM's")
    args = ap.parse_args()
    if args.calibrate_copy:
        return calibrate_copy(args.steps)
    if args.probe_mfma > 0:
        from shard_decomposed_gemm_amd import agemm
        print(json.dumps({"probe": "fp16 MFMA register loop", "launches": args.probe_mfma,
                          "tflops": agemm.probe_mfma(10, args.probe_mfma)}), flush=True)
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the flag-gated path keeps all W inbox slots in one GPU's HBM "
              "and the library has no multi-GPU path. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.workload in FD_WORKLOADS:
        return run_fd(args)
    if args.sweep:
        return run_sweep(args)

    import numpy as np
    import torch
    import synth
    from shard_decomposed_gemm_amd import Context

    W, M, K, N, c_dtype, sched_kind = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] workload={args.workload} W={W} M={M} K={K} N={N} C={c_dtype}", file=sys.stderr, flush=True)

    to_dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.float16)).to(dev)
    a = synth.matrix_f16(0xA102, M, K)
    shards = [to_dev(s) for s in synth.shards(a, W)]
    B0 = to_dev(synth.matrix_f16(0xB002, K, N))
    # Two copies of B, used alternately, so that the 256 MB last-level cache cannot hold B across steps.
    Bs = [B0, B0.clone()]
    cdt = torch.float16 if c_dtype == "f16" else torch.float32
    c_bytes = 2 if c_dtype == "f16" else 4
    Cs = [torch.empty((M, N), dtype=cdt, device=dev) for _ in range(2)]
    ctx = Context(W, M, K, N, c_dtype=c_dtype)
    ctx.set_order(args.order)
    sched = synth.schedule(0x5005, ctx.t, 20_000) if sched_kind == "random" else None
    if args.one_stream:
        # counter collection serialises dispatches, so no pair of streams overlaps there
        sp = sc = torch.cuda.Stream()
    else:
        sp, sc = ctx.streams()  # a producer / consumer pair verified to run concurrently
    torch.cuda.synchronize()

    def fused_step(i):
        ctx.produce(shards, schedule=sched, stream=sp)
        ctx.run_fused(Bs[i & 1], Cs[i & 1], stream=sc)

    # ---- the timed fused steps (wall clock between two device synchronisations)
    prewarm(fused_step, args.prewarm_ms)
    for i in range(args.warmup):
        fused_step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        fused_step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ctx.check()
    # ---- the same steps again, with HIP events attached to each consumer dispatch on
    # the consumer stream (agemm_timing_begin/end): the dominant kernel's own
    # execution time. Attaching events costs a few microseconds per step between
    # kernels, so the headline value comes from the pass above.
    ctx.timing_begin(args.steps)
    t1 = time.perf_counter()
    for i in range(args.steps):
        fused_step(i)
    torch.cuda.synchronize()
    wall_timed = time.perf_counter() - t1
    kern_us = ctx.timing_end()
    ctx.check()
    # ---- a third pass with a timing event recorded on the consumer stream after each
    # step: the spacing of consecutive step ends gives each step's time (median and
    # spread) beside the mean of the first pass.
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ends[0].record(sc)
    for i in range(args.steps):
        fused_step(i)
        ends[i + 1].record(sc)
    torch.cuda.synchronize()
    ctx.check()
    step_us = np.array([ends[i].elapsed_time(ends[i + 1]) * 1e3 for i in range(args.steps)])
    ms_step = wall * 1e3 / args.steps
    flops, cons_bytes, path_bytes = algorithmic(W, M, K, N, c_bytes)
    value = flops / (ms_step * 1e-3) / 1e12
    kavg = float(np.mean(kern_us)) * 1e-3  # ms
    print(f"[bench] fused: {ms_step * 1e3:.1f} us/step ({wall_timed * 1e6 / args.steps:.1f} with kernel timing; "
          f"step p10/p50/p90 {'/'.join('%.1f' % x for x in np.percentile(step_us, [10, 50, 90]))}), "
          f"consumer kernel {kavg * 1e3:.1f} us avg over {len(kern_us)} launches", file=sys.stderr, flush=True)

    mfma_bound = flops / (PEAK_FP16_TFLOPS * 1e12) > cons_bytes / (PEAK_HBM_GBS * 1e9)
    if mfma_bound:
        achieved = flops / (kavg * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_FP16_TFLOPS, "traffic": None}
    else:
        achieved = cons_bytes / (kavg * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": None}
    kind, tile_cfg = ctx.consumer
    roof["traffic"] = measured_traffic(args.workload, kind)
    roof["kernel"] = ("flag-gated MFMA tile GEMM, tile config %d, %d workgroups%s"
                      % (tile_cfg, ctx.grid, ", stream-K split over (tile, shard) units" if ctx.split else "")
                      if kind == "mfma" else "flag-gated small-M split-K streaming GEMM")
    roof["kernel_digest"] = kernel_digest(kind)
    roof["algorithmic_bytes_per_launch"] = cons_bytes
    roof["flops_per_launch"] = flops
    roof["kernel_us_avg"] = kavg * 1e3
    roof["kernel_us_min"] = float(np.min(kern_us))
    roof["kernel_us_p10_p50_p90"] = [float(x) for x in np.percentile(kern_us, [10, 50, 90])]
    roof["kernel_timing"] = ("HIP events attached to each consumer dispatch, over a second pass of the same "
                             "timed steps")

    # ---- the BSP ladder on the same GPU
    ladder = None
    if not args.no_ladder:
        def timeit(fn, n):
            for i in range(max(3, n // 5)):
                fn(i)
            torch.cuda.synchronize()
            t = time.perf_counter()
            for i in range(n):
                fn(i)
            torch.cuda.synchronize()
            return (time.perf_counter() - t) * 1e6 / n

        def flags_up():
            ctx.produce(shards)
            torch.cuda.synchronize()

        n = max(20, args.steps // args.sweep_reps)
        best, passes = interleaved_ladder([
            ("bsp_host_sync_us", lambda i: ctx.run_bsp(shards, Bs[i & 1], Cs[i & 1], schedule=sched, host_sync=True,
                                                       stream=sc), None, None),
            ("bsp_device_dep_us", lambda i: ctx.run_bsp(shards, Bs[i & 1], Cs[i & 1], schedule=sched,
                                                        host_sync=False, stream=sc), None, None),
            ("fused_us", fused_step, None, None),
            ("fused_strict_acquire_us", fused_step, lambda: ctx.set_strict_acquire(True),
             lambda: ctx.set_strict_acquire(False)),
            ("consumer_only_us", lambda i: ctx.run_fused(Bs[i & 1], Cs[i & 1], stream=sc), flags_up, None),
            ("pull_us", lambda i: ctx.run_pull(shards, Bs[i & 1], Cs[i & 1], stream=sc), None, None),
        ], n, args.sweep_reps, timeit)
        ctx.check()
        ladder = dict(best)
        ladder["fused_speedup_vs_bsp"] = best["bsp_host_sync_us"] / best["fused_us"]
        ladder["fused_speedup_vs_bsp_device_dep"] = best["bsp_device_dep_us"] / best["fused_us"]
        ladder["method"] = f"best of {args.sweep_reps} interleaved passes of {n} steps, order rotated each pass"
        ladder["passes"] = passes
        print(f"[bench] ladder: {json.dumps(ladder)}", file=sys.stderr, flush=True)

    peaks = device_peaks(not args.no_peaks)
    if "measured" in peaks:
        m = peaks["measured"]
        ceil = m["mfma_f16_register_loop_tflops"] if roof["bound"] == "mfma" else m["stream_read_gbs"]
        roof["frac_of_measured_ceiling"] = roof["achieved"] / ceil
        print(f"[bench] measured ceilings: {m['mfma_f16_register_loop_tflops']:.0f} TFLOP/s fp16 MFMA loop, "
              f"{m['stream_read_gbs']:.0f} GB/s streaming read", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(W, M, K, N, args.cpu_budget)
        print(f"[bench] cpu oracle: {cpu['sample']}", file=sys.stderr, flush=True)

    line = {
        "metric": "TFLOP/s and % fp16 MFMA / HBM roofline, shard-split GEMM K=8192 N=28672",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "prewarm_ms": args.prewarm_ms,
        "ms_per_step": ms_step,
        "ms_per_step_with_kernel_timing": wall_timed * 1e3 / args.steps,
        "step_us_p10_p50_p90": [float(x) for x in np.percentile(step_us, [10, 50, 90])],
        "step_timing": "spacing of timing events recorded on the consumer stream after each step, a third "
                       "pass of the same steps",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": args.workload, "W": W, "M": M, "K": K, "N": N, "c_dtype": c_dtype,
                   "accumulate": "f32", "flag_ktile": ctx.bkf, "tiles": ctx.t,
                   "schedule": "seeded permutation, cumulative U[0,20] us delays" if sched else "shard order, no delay",
                   "path": "producer || flag-gated consumer on two streams", "order": args.order},
        "roofline": roof,
        "cpu_baseline": cpu,
        "ladder": ladder,
        "peaks": peaks,
    }
    print(json.dumps(line), flush=True)
    ctx.close()


if __name__ == "__main__":
    main()
