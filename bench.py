"""Benchmark of libgemm355 on one MI355X: TFLOP/s = 2MNK/t of C = alpha*A@B + beta*C.

One "step" is one library call over the whole path (for f16r: the operand
rounding passes and the GEMM).  The headline workload is the f32 GEMM at
M = N = K = 4096 (alpha 1, beta 0); the line also carries the beta = 1 run and
the f16r GEMM at 8192^3 (alpha 0.75, beta -0.25), each with its fraction of the
matrix-core roof re-measured on this chip (the Matrix Multiplication lab,
"Part 1 -- the two roofs, again"), and the CPU oracle timed on host cores.

Protocol (the lab's helpers): every result is checked against the oracle before
it is timed; clocks are settled with synchronised calls for a quarter second;
then exactly --steps calls are timed between two device synchronisations, with
an event pair around every call on the stream the library launches on.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--workloads a,b,...] [--no-tune] [--json-out path]
Prints progress on stderr and ONE JSON line on stdout.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "TFLOP/s (2MNK/t) at 4096^3 f32 and 8192^3 f16r/f32acc; % of MFMA peak"
PRIMARY = "f32_4096_a1_b0"
SCORED = ["f32_4096_a1_b0", "f32_4096_a1_b1", "f16r_8192_a0.75_b-0.25"]

# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s).
PEAK_TFLOPS = {"f32": 157.3, "f16r": 2500.0}
PEAK_HBM_GBS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workloads", default=",".join(SCORED))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-tune", action="store_true")
    ap.add_argument("--no-roofs", action="store_true")
    ap.add_argument("--roof-seconds", type=float, default=2.0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB copy kernel (byte-counter calibration)")
    ap.add_argument("--summarize-trace", metavar="DIR", default=None,
                    help="write a markdown summary of a rocprofv3 --kernel-trace --stats run")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"), default=None,
                    help="summarise FETCH_SIZE / WRITE_SIZE runs into an HBM-traffic table")
    ap.add_argument("--out", default=None, help="output file of the --summarize-* modes")
    ap.add_argument("--cmd", default="", help="the command that produced the profile")
    ap.add_argument("--sweep", metavar="OUT_MD", default=None,
                    help="shape and alignment sweep of both modes (sizes 128..8192, n = "
                         "4088..4104 and 2048..2304, fixed-tile steps); markdown to OUT_MD")
    ap.add_argument("--sweep-repeats", type=int, default=3)
    ap.add_argument("--precision", metavar="OUT_MD", default=None,
                    help="precision study (the lab's Part 4): f32, f16r and f16r with binary16 "
                         "output against float64 of the unrounded inputs; markdown to OUT_MD")
    ap.add_argument("--skinny", metavar="OUT_MD", default=None,
                    help="few-rows sweep (M = 1..2048 at K = N = 4096, both modes) against "
                         "the HBM and matrix-core roofs; markdown to OUT_MD")
    args = ap.parse_args()

    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.out, args.cmd)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.out, args.cmd)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs as a single process on one GPU.", file=sys.stderr)
        sys.exit(2)

    import torch

    import gemm_tiled_amd as g
    from workloads import WORKLOADS, sample_indices, workload_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(0)
    log(f"device {props.name} ({getattr(props, 'gcnArchName', '?')}), "
        f"{props.multi_processor_count} CUs; libgemm355 {g.version()}")

    if args.calibrate_copy:
        copy_calibration(g, torch, dev)

    if args.sweep:
        shape_sweep(g, torch, dev, args.sweep, args.sweep_repeats)
        return
    if args.skinny:
        skinny_sweep(g, torch, dev, args.skinny, args.sweep_repeats)
        return
    if args.precision:
        precision_study(g, torch, dev, args.precision)
        return

    # ------------------------------------------------------------------ roofs
    roofs = {}
    if not args.no_roofs:
        roofs = measure_roofs(g, torch, dev, args.roof_seconds)
        log(f"measured roofs: {json.dumps(roofs)}")

    # -------------------------------------------------------------- workloads
    names = [n for n in args.workloads.split(",") if n]
    runs = {}
    for name in names:
        w = WORKLOADS[name]
        runs[name] = bench_workload(g, torch, dev, w, args, roofs, workload_inputs,
                                    sample_indices)

    primary = PRIMARY if PRIMARY in runs else names[0]
    pr = runs[primary]
    w = WORKLOADS[primary]

    # --------------------------------------------------------- CPU baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_seconds, workload_inputs)

    line = {
        "metric": METRIC,
        "value": pr["tflops_job"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pr["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w.mode == "f32" else "f16r/f32acc",
        "data": "synthetic (seeded uniform/normal matrices; no dataset)",
        "config": {"workload": primary, "mode": w.mode, "M": w.M, "N": w.N, "K": w.K,
                   "alpha": w.alpha, "beta": w.beta, "tile": pr["tile"]},
        "roofline": pr["roofline"],
        "cpu_baseline": cpu,
        "measured_roof": roofs or None,
        "frac_of_measured_roof": pr.get("frac_of_measured_roof"),
        "workloads": runs,
    }
    text = json.dumps(line)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(text + "\n")
    print(text, flush=True)


def measure_roofs(g, torch, dev, seconds):
    import ctypes

    L = g.lib()
    out = {}
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    blocks = 256 * 4   # four workgroups of four waves per CU
    sink = torch.empty(blocks * 256, device=dev, dtype=torch.float32)
    for mode, name in ((0, "f32"), (1, "f16r")):
        iters = 2000 if mode == 0 else 4000
        flops = ctypes.c_double(0)

        def launch():
            st = L.gemm355_roof_mfma(mode, iters, blocks, ctypes.c_void_p(sink.data_ptr()),
                                     ctypes.byref(flops), sp)
            if st != 0:
                raise g.Gemm355Error(st, "gemm355_roof_mfma")

        launch()
        torch.cuda.synchronize()
        # sustained: back-to-back launches for `seconds`, synchronising every 4 calls
        s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s_ev.record()
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            launch()
            n += 1
            if n % 4 == 0:
                torch.cuda.synchronize()
        e_ev.record()
        e_ev.synchronize()
        t = s_ev.elapsed_time(e_ev) / 1e3 / n
        out[f"mfma_{name}_tflops"] = flops.value / t / 1e12
        out[f"mfma_{name}_published_tflops"] = PEAK_TFLOPS[name]
    # HBM read roof: 4 GiB, beyond the 256 MB last-level cache
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, device=dev, dtype=torch.float32)
    sink1 = torch.zeros(1, device=dev, dtype=torch.float32)

    def read():
        st = L.gemm355_roof_hbm(ctypes.c_void_p(buf.data_ptr()), nbytes, 256 * 8,
                                ctypes.c_void_p(sink1.data_ptr()), sp)
        if st != 0:
            raise g.Gemm355Error(st, "gemm355_roof_hbm")

    t = steady(read, torch, 0.5)
    out["hbm_read_gbs"] = nbytes / t / 1e9
    out["hbm_published_gbs"] = PEAK_HBM_GBS
    del buf
    torch.cuda.empty_cache()
    return out


def steady(fn, torch, seconds=0.5, min_calls=3, batch=1):
    """Median seconds per call after settling (the lab's steady()).  With
    batch > 1 each sample times `batch` back-to-back calls between two events
    and divides: for calls of a few microseconds, the GPU time per call in a
    stream of calls, without the host's per-call launch latency."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds / 2:
        fn()
        torch.cuda.synchronize()
    s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts, t0 = [], time.perf_counter()
    while time.perf_counter() - t0 < seconds or len(ts) < min_calls:
        s_ev.record()
        for _ in range(batch):
            fn()
        e_ev.record()
        e_ev.synchronize()
        ts.append(s_ev.elapsed_time(e_ev) / 1e3 / batch)
    return float(np.median(ts))


def bench_workload(g, torch, dev, w, args, roofs, workload_inputs, sample_indices):
    import oracle   # correctness check before timing (CPU, test infrastructure)

    log(f"{w.name}: generating inputs")
    A, B, C = workload_inputs(w)
    tA = torch.from_numpy(A).to(dev)
    tB = torch.from_numpy(B).to(dev)
    tC0 = torch.from_numpy(C).to(dev)
    tC = tC0.clone()
    fn = g.gemm_f32 if w.mode == "f32" else g.gemm_f16r_f32acc

    if not args.no_tune:
        log(f"{w.name}: tuning")
        g.tune(w.mode, tA, tB, tC, beta=w.beta)
    tile = g.get_config(w.mode, w.M, w.N, w.K, beta=w.beta)
    log(f"{w.name}: tile {tile}")

    # correctness first: one call on a fresh C, sampled oracle elements
    fn(tA, tB, tC, w.alpha, w.beta)
    torch.cuda.synchronize()
    got = tC.cpu().numpy()
    r, c = sample_indices(w.M, w.N, 2048, seed=1)
    ref, W = oracle.entries(w.mode, A, B, C, w.alpha, w.beta, r, c)
    err = np.abs(got[r, c].astype(np.float64) - ref)
    ratio = float(np.max(err / np.where(W > 0, W, 1.0)))
    ok = bool(np.all(err <= oracle.TOL[w.mode] * W))
    log(f"{w.name}: parity on {r.size} sampled elements: max err/W {ratio:.3e} "
        f"(bound {oracle.TOL[w.mode]:.0e}) -> {'ok' if ok else 'FAIL'}")
    if not ok:
        raise SystemExit(f"{w.name}: result outside the parity bound; not timing it")
    del got

    stream = torch.cuda.current_stream()
    call = lambda: fn(tA, tB, tC, w.alpha, w.beta)   # noqa: E731  (C drifts; timing is data-independent)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    # settle the clocks (synchronised calls, a quarter second)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.25:
        call()
        torch.cuda.synchronize()

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ev, e_ev in evs:
        s_ev.record(stream)
        call()
        e_ev.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = np.array([s.elapsed_time(e) / 1e3 for s, e in evs])
    gpu_total = float(per.sum())

    flops = w.flops
    tflops_job = flops * args.steps / wall / 1e12
    tflops_med = flops / float(np.median(per)) / 1e12
    avg = float(per.mean())
    achieved = flops / avg / 1e12
    peak = PEAK_TFLOPS[w.mode]
    roof = {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": None,
            "kernel": f32_kernel_name(tile) if w.mode == "f32" else
            "pack_kernel + gemm_f16_kernel (whole call)",
            "per_launch_flops": flops}
    res = {
        "mode": w.mode, "M": w.M, "N": w.N, "K": w.K, "alpha": w.alpha, "beta": w.beta,
        "tile": tile,
        "ms_per_step": wall / args.steps * 1e3,
        "ms_median_call": float(np.median(per)) * 1e3,
        "ms_mean_call": avg * 1e3,
        "gpu_busy_frac": gpu_total / wall,
        "tflops_job": tflops_job,
        "tflops_median_call": tflops_med,
        "parity_max_ratio_sampled": ratio,
        "roofline": roof,
    }
    tr = committed_traffic(w.mode, w.name, tile)
    if tr is not None:
        roof["traffic"] = tr["traffic_bytes_per_launch"]
        roof["traffic_source"] = tr["source"]
    key = "mfma_f32_tflops" if w.mode == "f32" else "mfma_f16r_tflops"
    if roofs.get(key):
        res["frac_of_measured_roof"] = round(tflops_med / roofs[key], 4)
    log(f"{w.name}: {tflops_job:.2f} TFLOP/s over {args.steps} steps "
        f"({res['ms_per_step']:.4f} ms/step, median call {res['ms_median_call']:.4f} ms, "
        f"{tflops_med:.2f} TFLOP/s median); frac of published peak {roof['frac']:.3f}"
        + (f", of measured roof {res['frac_of_measured_roof']:.3f}" if "frac_of_measured_roof" in res
           else ""))
    del tA, tB, tC, tC0
    torch.cuda.empty_cache()
    return res


def cpu_baseline(w, target_seconds, workload_inputs):
    """The oracle as it stands, timed on the host cores over the whole workload
    when that fits in ~30 s, else over a band of output rows sized to about
    target_seconds; throughput in TFLOP/s (2*rows*N*K / t)."""
    import oracle

    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    os.environ["OMP_NUM_THREADS"] = str(threads)
    A, B, C = workload_inputs(w)

    def timed(rows):
        t0 = time.perf_counter()
        oracle.check(w.mode, A, B, C, w.alpha, w.beta, C, rows=(0, rows))
        return time.perf_counter() - t0

    # per-row cost from two probes (the widening of A and B is a fixed cost)
    t16, t64 = timed(16), timed(64)
    per_row = max((t64 - t16) / 48.0, 1e-6)
    fixed = max(t16 - 16 * per_row, 0.0)
    if fixed + per_row * w.M <= 30.0:
        rows = w.M
    else:
        rows = int(min(w.M, max(64, (target_seconds - fixed) / per_row)))
    t = timed(rows)
    flops = 2.0 * rows * w.N * w.K
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    cpu_model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    what = "the whole workload" if rows == w.M else f"{rows} of {w.M} output rows"
    res = {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "sample": f"{what} of {w.name} (float64 triple loop incl. operand widening and "
                     f"the bound), {t:.1f} s", "cpu": cpu_model}
    log(f"cpu baseline: {res['value'] * 1e3:.2f} GFLOP/s on {threads} threads ({res['sample']})")
    return res


# ---------------------------------------------------------------------------
# Shape and alignment sweep (the Matrix Multiplication lab, "Part 5 -- cuBLAS,
# and what shape does to it": a size sweep, the one-element steps around 2048
# and 4096, and the same steps for a tiling that cannot change).
# ---------------------------------------------------------------------------
SWEEP_SIZES = [128, 256, 512, 1024, 1536, 2048, 3072, 4096, 6144, 8192]
SWEEP_QUANT = list(range(4088, 4105)) + [2048, 2049, 2056, 2064, 2080, 2112, 2176, 2304]
SWEEP_FIXED = [2048, 2049, 4096, 4097]
FIXED_TILE = {"f32": "BM=128 BN=128 BK=32 ST=2 WM=2 WN=2 GM=8",
              "f16r": "BM=128 BN=128 BK=64 ST=1 WM=2 WN=2 GM=8"}


def _tile_fields(tile):
    return {k: int(v) for k, v in (t.split("=") for t in tile.split() if "=" in t and
                                    t.split("=")[1].isdigit())}


def _plan_of(g, mode, n, pin=None):
    """How a square n^3 call runs (the library's own plan, gemm355_get_plan_ex):
    the kernel path and, when the ring runs only a block of C, that block."""
    if pin:
        g.set_config(mode, pin)
    try:
        plan = dict(kv.split("=") for kv in g.get_plan(mode, n, n, n, beta=0.0).split())
    finally:
        if pin:
            g.set_config(mode, None)
    text = plan["form"]
    if plan["block"] != f"{n}x{n}x{n}":
        text += f" on {plan['block']} + strips"
    if "rows" in plan:
        text += ", rows 4-byte aligned"
    return text


def shape_sweep(g, torch, dev, out, repeats):
    import random

    import oracle
    from workloads import make_inputs, sample_indices

    cases = [(mode, n, "tuned") for mode in ("f32", "f16r")
             for n in sorted(set(SWEEP_SIZES + SWEEP_QUANT))]
    cases += [(mode, n, "fixed") for mode in ("f32", "f16r") for n in SWEEP_FIXED]
    inputs = {}
    for n in sorted({c[1] for c in cases}):
        A, B, C = make_inputs(n, n, n, "normal", seed=n)
        r, c = sample_indices(n, n, 256, seed=2)
        refs = {mode: oracle.entries(mode, A, B, C, 1.0, 0.0, r, c) for mode in ("f32", "f16r")}
        inputs[n] = (torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev),
                     torch.from_numpy(C).to(dev), r, c, refs)
        del A, B, C
    log(f"sweep: {len(cases)} cases, {repeats} shuffled rounds")

    tiles, plans, calls = {}, {}, {}
    for case in cases:
        mode, n, kind = case
        tA, tB, tC, r, c, refs = inputs[n]
        fn = g.gemm_f32 if mode == "f32" else g.gemm_f16r_f32acc
        if kind == "tuned":
            g.tune(mode, tA, tB, tC, beta=0.0)
            tiles[case] = g.get_config(mode, n, n, n, beta=0.0)
            plans[case] = _plan_of(g, mode, n)
            call = (lambda fn=fn, tA=tA, tB=tB, tC=tC: fn(tA, tB, tC, 1.0, 0.0))
        else:
            tiles[case] = FIXED_TILE[mode] + " source=pin"
            plans[case] = _plan_of(g, mode, n, FIXED_TILE[mode])

            def call(fn=fn, tA=tA, tB=tB, tC=tC, mode=mode):
                g.set_config(mode, FIXED_TILE[mode])
                try:
                    fn(tA, tB, tC, 1.0, 0.0)
                finally:
                    g.set_config(mode, None)
        # correctness first: sampled elements against the oracle (beta = 0: C is not read)
        call()
        torch.cuda.synchronize()
        got = tC[torch.as_tensor(r, device=dev), torch.as_tensor(c, device=dev)].cpu().numpy()
        ref, W = refs[mode]
        err = np.abs(got.astype(np.float64) - ref)
        if not np.all(err <= oracle.TOL[mode] * W):
            raise SystemExit(f"sweep {case}: outside the parity bound")
        calls[case] = call

    times = {case: [] for case in cases}
    rng = random.Random(0)
    for rnd in range(repeats):
        order = list(cases)
        rng.shuffle(order)
        for case in order:
            times[case].append(steady(calls[case], torch, seconds=0.3))
        log(f"sweep: round {rnd + 1} of {repeats} done")

    rows = []
    for case in cases:
        mode, n, kind = case
        ts = times[case]
        med = float(np.median(ts))
        rows.append({"mode": mode, "n": n, "kind": kind, "tile": tiles[case].split(" source=")[0],
                     "path": plans[case], "seconds": med,
                     "seconds_min": min(ts), "seconds_max": max(ts),
                     "tflops": 2.0 * n ** 3 / med / 1e12})
    by = {(r["mode"], r["n"], r["kind"]): r for r in rows}

    def step(mode, kind, a, b):
        ra, rb = by[(mode, a, kind)], by[(mode, b, kind)]
        return 100 * (rb["seconds"] / ra["seconds"] - 1), 100 * (1 - rb["tflops"] / ra["tflops"])

    lines = ["# Shape and alignment sweep (both modes, one MI355X)", "",
             "Command:", "", "```", "python bench.py --sweep profiles/sweep_shapes.md", "```", "",
             "Square n x n x n, A, B, C iid N(0,1) (seed n), alpha = 1, beta = 0.  Every case is "
             "checked against the oracle on 256 sampled elements before it is timed; each time "
             f"is the median of {repeats} shuffled rounds of the lab's steady() (0.3 s each).  "
             "`tuned` lets the library's tuner pick the tile per shape; `fixed` pins one 128 x 128 "
             "tile, so its step isolates the cost of the ragged edge.", ""]
    lines += ["## One-element steps", "", "| mode | tiling | 2048 -> 2049 time | 4096 -> 4097 time |",
              "|---|---|---:|---:|"]
    for mode in ("f32", "f16r"):
        for kind in ("tuned", "fixed"):
            a, b = step(mode, kind, 2048, 2049), step(mode, kind, 4096, 4097)
            lines.append(f"| {mode} | {kind} | {a[0]:+.1f}% | {b[0]:+.1f}% |")
    for title, sel in (("## Size sweep", lambda r: r["n"] in SWEEP_SIZES and r["kind"] == "tuned"),
                       ("## Near 2048 and 4096", lambda r: r["n"] in SWEEP_QUANT and
                        r["kind"] == "tuned"),
                       ("## Fixed 128 x 128 tile", lambda r: r["kind"] == "fixed")):
        lines += ["", title, "", "| mode | n | TFLOP/s | min..max ms | tile | path |",
                  "|---|---:|---:|---|---|---|"]
        for r in sorted(filter(sel, rows), key=lambda r: (r["mode"], r["n"])):
            lines.append(f"| {r['mode']} | {r['n']} | {r['tflops']:.1f} | "
                         f"{r['seconds_min'] * 1e3:.3f}..{r['seconds_max'] * 1e3:.3f} | "
                         f"{r['tile']} | {r['path']} |")
    lines += ["", "```json", json.dumps(rows), "```", ""]
    _write(out, "\n".join(lines))


# ---------------------------------------------------------------------------
# Precision (the Matrix Multiplication lab, "Part 4 -- precision"): A, B =
# U[0,1) - 0.5, C = A@B; each variant against the float64 product of the
# UNROUNDED inputs, as the lab's normalised max error (max|err| / max|ref|)
# and relative Frobenius error, beside its speed and bytes per element of C.
# ---------------------------------------------------------------------------
PRECISION_SIZES = [2048, 4096]


def precision_study(g, torch, dev, out):
    import oracle
    from workloads import make_inputs

    rows = []
    for n in PRECISION_SIZES:
        A, B, _ = make_inputs(n, n, n, "centered", seed=0)
        zeros = np.zeros((n, n), dtype=np.float32)
        tA, tB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
        tC = torch.zeros((n, n), device=dev, dtype=torch.float32)
        tC16 = torch.zeros((n, n), device=dev, dtype=torch.float16)
        variants = [
            ("f32", 4, lambda: g.gemm_f32(tA, tB, tC, 1.0, 0.0), tC),
            ("f16r (f32 output)", 4, lambda: g.gemm_f16r_f32acc(tA, tB, tC, 1.0, 0.0), tC),
            ("f16r, f16 output", 2, lambda: g.gemm_f16r_f16out(tA, tB, tC16, 1.0, 0.0), tC16),
        ]
        for label, nbytes, fn, dst in variants:
            fn()
            torch.cuda.synchronize()
            got = dst.float().cpu().numpy()
            # against the float64 product of the unrounded inputs (the f32 reference)
            vs64 = oracle.check("f32", A, B, zeros, 1.0, 0.0, got, tol=1.0)
            # and against the float64 product of the binary16-rounded inputs
            vsr = oracle.check("f16r", A, B, zeros, 1.0, 0.0, got, tol=1.0)
            t = steady(fn, torch, 0.5)
            rows.append({"n": n, "variant": label, "seconds": t,
                         "tflops": 2.0 * n ** 3 / t / 1e12, "bytes_per_element": nbytes,
                         "err_max_norm": vs64["err_max_norm"], "err_fro": vs64["err_fro"],
                         "err_max_norm_vs_rounded": vsr["err_max_norm"],
                         "err_fro_vs_rounded": vsr["err_fro"]})
            log(f"precision n={n} {label}: {rows[-1]['tflops']:.1f} TFLOP/s, "
                f"max {vs64['err_max_norm']:.2e}, Frobenius {vs64['err_fro']:.2e}")
        del tA, tB, tC, tC16
        torch.cuda.empty_cache()
    for r_ in rows:
        base = next(x for x in rows if x["n"] == r_["n"] and x["variant"] == "f32")
        r_["speedup_vs_f32"] = r_["tflops"] / base["tflops"]
    lines = ["# Precision: f32, f16r and f16r with binary16 output (one MI355X)", "",
             "Command:", "", "```", "python bench.py --precision profiles/precision.md", "```", "",
             "A, B = U[0,1) - 0.5 (float32, seed 0), C = A @ B (alpha 1, beta 0).  Errors against "
             "the float64 product of the unrounded inputs, computed by the oracle: normalised "
             "max error max|C - ref| / max|ref| and relative Frobenius error "
             "||C - ref|| / ||ref||.  The last two columns measure the same against the float64 "
             "product of the binary16-rounded inputs, which separates the rounding of the "
             "operands (and of the output) from the f32 accumulation.  Times: steady(), "
             "median over 0.5 s.", "",
             "| n | variant | TFLOP/s | speedup vs f32 | bytes/element of C | max err (norm.) | "
             "Frobenius | max err vs rounded inputs | Frobenius vs rounded inputs |",
             "|---:|---|---:|---:|---:|---:|---:|---:|---:|"]
    for r_ in rows:
        lines.append(f"| {r_['n']} | {r_['variant']} | {r_['tflops']:.1f} | "
                     f"{r_['speedup_vs_f32']:.2f} | {r_['bytes_per_element']} | "
                     f"{r_['err_max_norm']:.2e} | {r_['err_fro']:.2e} | "
                     f"{r_['err_max_norm_vs_rounded']:.2e} | {r_['err_fro_vs_rounded']:.2e} |")
    lines += ["", "```json", json.dumps(rows), "```", ""]
    _write(out, "\n".join(lines))


# ---------------------------------------------------------------------------
# Few rows of C (the lab's "Part 5", the skinny shapes: M from 1 up at
# K = N = 4096).  Arithmetic intensity I = 2MNK / (4(MK + KN + MN)) bytes of
# f32 storage; below the ridge the HBM roof bounds the call.
# ---------------------------------------------------------------------------
SKINNY_M = [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048]
SKINNY_BATCH = 20   # calls per timed sample: the calls take microseconds


def skinny_sweep(g, torch, dev, out, repeats):
    import random

    import oracle
    from workloads import make_inputs, sample_indices

    roofs = measure_roofs(g, torch, dev, 1.0)
    log(f"skinny: roofs {json.dumps(roofs)}")
    K = N = 4096
    _, B, _ = make_inputs(1, N, K, "normal", seed=4096)
    tB = torch.from_numpy(B).to(dev)
    cases = []
    for M in SKINNY_M:
        A = make_inputs(M, 1, K, "normal", seed=M)[0]       # M x K
        C = make_inputs(M, N, 1, "normal", seed=M + 1)[2]   # M x N
        r, c = sample_indices(M, N, 256, seed=3)
        tA, tC = torch.from_numpy(A).to(dev), torch.from_numpy(C).to(dev)
        for mode in ("f32", "f16r"):
            ref, W = oracle.entries(mode, A, B, C, 1.0, 0.0, r, c)
            kinds = ("tuned", "split-K", "rows", "no split-K") + (("round on load",) if mode == "f16r" else ())
            for kind in kinds:
                cases.append((mode, M, kind, tA, tC, r, c, ref, W))
    calls, tiles = {}, {}
    for (mode, M, kind, tA, tC, r, c, ref, W) in cases:
        fn = g.gemm_f32 if mode == "f32" else g.gemm_f16r_f32acc
        key = (mode, M, kind)
        if kind == "tuned":
            g.tune(mode, tA, tB, tC, beta=0.0)
            tiles[key] = g.get_config(mode, M, N, K, beta=0.0)
            call = (lambda fn=fn, tA=tA, tC=tC: fn(tA, tB, tC, 1.0, 0.0))
        elif kind in ("split-K", "rows"):
            cfg = g.parse_config(mode, "KS=1" if kind == "split-K" else "KS=2")
            tiles[key] = cfg

            def call(fn=fn, tA=tA, tC=tC, mode=mode, cfg=cfg):
                g.set_config(mode, cfg)
                try:
                    fn(tA, tB, tC, 1.0, 0.0)
                finally:
                    g.set_config(mode, None)
        else:
            # the library's best configuration without split-K (tuned over the
            # rest), or the best of the f16r configurations that round the
            # operands as they stage them (KS=3)
            best, best_t = None, 1e30
            for cfg in g.list_configs(mode):
                if ("KS=3" not in cfg) if kind == "round on load" else ("KS=" in cfg):
                    continue
                g.set_config(mode, cfg)
                try:
                    t = steady(lambda fn=fn, tA=tA, tC=tC: fn(tA, tB, tC, 1.0, 0.0), torch, 0.05,
                               batch=SKINNY_BATCH)
                finally:
                    g.set_config(mode, None)
                if t < best_t:
                    best, best_t = cfg, t
            tiles[key] = best

            def call(fn=fn, tA=tA, tC=tC, mode=mode, cfg=best):
                g.set_config(mode, cfg)
                try:
                    fn(tA, tB, tC, 1.0, 0.0)
                finally:
                    g.set_config(mode, None)
        call()
        torch.cuda.synchronize()
        got = tC[torch.as_tensor(r, device=dev), torch.as_tensor(c, device=dev)].cpu().numpy()
        if not np.all(np.abs(got.astype(np.float64) - ref) <= oracle.TOL[mode] * W):
            raise SystemExit(f"skinny {key}: outside the parity bound")
        calls[key] = call
    times = {k: [] for k in calls}
    rng = random.Random(1)
    for rnd in range(repeats):
        order = list(calls)
        rng.shuffle(order)
        for k in order:
            times[k].append(steady(calls[k], torch, seconds=0.2, batch=SKINNY_BATCH))
        log(f"skinny: round {rnd + 1} of {repeats} done")
    rows = []
    hbm = roofs["hbm_read_gbs"] * 1e9
    for (mode, M, kind), ts in times.items():
        t = float(np.median(ts))
        flops = 2.0 * M * N * K
        nbytes = 4.0 * (M * K + K * N + M * N)
        intensity = flops / nbytes
        mfma = roofs["mfma_f32_tflops" if mode == "f32" else "mfma_f16r_tflops"] * 1e12
        roof = min(mfma, intensity * hbm)
        rows.append({"mode": mode, "M": M, "kind": kind, "tile": tiles[(mode, M, kind)].split(
            " source=")[0], "seconds": t, "tflops": flops / t / 1e12,
            "gbs": nbytes / t / 1e9, "intensity": intensity, "roof_tflops": roof / 1e12,
            "bound": "hbm" if intensity * hbm < mfma else "mfma", "frac_of_roof": flops / t / roof})
    lines = ["# Few rows of C: M = 1 .. 2048 at K = N = 4096 (both modes, one MI355X)", "",
             "Command:", "", "```", "python bench.py --skinny profiles/skinny_m.md", "```", "",
             "A (M x K), B (K x N), C iid N(0,1); alpha = 1, beta = 0.  Every case is checked "
             "against the oracle on 256 sampled elements before it is timed; the time is the "
             f"median of {repeats} shuffled rounds of steady() (0.2 s), each sample "
             f"{SKINNY_BATCH} back-to-back calls between two events (GPU time per call in a "
             "stream of calls: at M = 1 a call takes ~15 us, less than the host's per-call "
             "launch latency, which a single-call sample would add).  Bytes are the f32 "
             "storage the call must move at least once, 4(MK + KN + MN); the roof is "
             "min(measured matrix-core roof of the mode, intensity x measured HBM read roof "
             f"{roofs['hbm_read_gbs']:.0f} GB/s).  `tuned` is the library's own choice (all "
             "configurations are candidates); `split-K` is the 32x128-tile split-K "
             "configuration (KS=1), `rows` the few-rows configuration (KS=2: B streamed into "
             "registers, 16x16x4 matrix instructions, k split within and across workgroups); "
             "`round on load` (f16r) the fastest of the configurations that round A and B to "
             "binary16 as they stage them for the binary16 matrix instruction (KS=3, no packing "
             "pass); `no split-K` is the fastest configuration of none of these kinds.", "",
             "| mode | M | choice | TFLOP/s | GB/s | FLOP/B | bound | of roof | tile |",
             "|---|---:|---|---:|---:|---:|---|---:|---|"]
    for r_ in sorted(rows, key=lambda r_: (r_["mode"], r_["M"], r_["kind"])):
        lines.append(f"| {r_['mode']} | {r_['M']} | {r_['kind']} | {r_['tflops']:.2f} | "
                     f"{r_['gbs']:.0f} | {r_['intensity']:.1f} | {r_['bound']} | "
                     f"{r_['frac_of_roof']:.2f} | {r_['tile']} |")
    lines += ["", "```json", json.dumps({"roofs": roofs, "rows": rows}), "```", ""]
    _write(out, "\n".join(lines))


# ---------------------------------------------------------------------------
# Profile evidence: byte-counter calibration, committed summaries.
# ---------------------------------------------------------------------------
COPY_BYTES = 256 << 20          # one direction of the calibration copy
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {
    "f32": ["gemm_tiled_amd/csrc/gemm_f32.hip", "gemm_tiled_amd/csrc/gemm_f32_ring.hip",
            "gemm_tiled_amd/csrc/f32_kernel.hpp", "gemm_tiled_amd/csrc/internal.hpp"],
    "f16r": ["gemm_tiled_amd/csrc/gemm_f16r.hip", "gemm_tiled_amd/csrc/f16_kernel.hpp",
             "gemm_tiled_amd/csrc/internal.hpp"],
}


def copy_calibration(g, torch, dev):
    """A plain copy of COPY_BYTES (read) into COPY_BYTES (write), 5 launches:
    the kernel whose FETCH_SIZE / WRITE_SIZE calibrate the byte counters."""
    import ctypes
    n = COPY_BYTES // 4
    src = torch.ones(n, device=dev, dtype=torch.float32)
    dst = torch.empty(n, device=dev, dtype=torch.float32)
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for _ in range(5):
        st = g.lib().gemm355_copy_f32(ctypes.c_void_p(src.data_ptr()),
                                      ctypes.c_void_p(dst.data_ptr()), n, sp)
        if st != 0:
            raise g.Gemm355Error(st, "gemm355_copy_f32")
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()
    log(f"calibration copy: 5 x {COPY_BYTES >> 20} MiB")


def source_hash(mode):
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[mode]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def f32_kernel_name(tile):
    """The f32 kernel a configuration string runs on whole tiles: the
    direct-to-LDS ring for the configurations with three or more stages,
    the register-staged kernel otherwise."""
    m = re.search(r"ST=(\d+)", tile or "")
    return "gemm_f32_ring_kernel" if m and int(m.group(1)) >= 3 else "gemm_f32_kernel"


def committed_traffic(mode, workload, tile):
    """HBM bytes per launch from the committed counter summary of this
    workload and tile, if it was taken on the current kernel sources; else None."""
    import glob
    import re
    for path in sorted(glob.glob(os.path.join(PROFILES, "traffic", "*.md"))):
        text = open(path).read()
        m = re.search(r"```json\n(.*?)\n```", text, re.S)
        if not m:
            continue
        try:
            d = json.loads(m.group(1))
        except ValueError:
            continue
        if d.get("workload") != workload or d.get("mode") != mode:
            continue
        if d.get("tile", "").split(" source=")[0] != tile.split(" source=")[0]:
            continue
        if d.get("source_hash") != source_hash(mode):
            return None          # the kernel changed since the counters were taken
        return {"traffic_bytes_per_launch": d["traffic_bytes_per_launch"],
                "source": os.path.relpath(path, ROOT)}
    return None


def _csv_rows(directory, suffix):
    import csv
    import glob
    files = glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True)
    rows = []
    for f in files:
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def summarize_trace(directory, out, cmd):
    rows = _csv_rows(directory, "kernel_stats.csv")
    if not rows:
        raise SystemExit(f"no kernel_stats.csv under {directory}")
    lines = ["# Kernel trace summary", "", "Command:", "", "```", cmd, "```", "",
             "| kernel | calls | average us | min us | max us | share of GPU time |",
             "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        name = r["Name"].replace("|", "/")
        lines.append(f"| `{name[:150]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.1f}% |")
    text = "\n".join(lines) + "\n"
    _write(out, text)


def _per_dispatch(rows, counter):
    import collections
    per = collections.defaultdict(float)
    names = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        per[r["Dispatch_Id"]] += float(r["Counter_Value"])
        names[r["Dispatch_Id"]] = r["Kernel_Name"]
    by_kernel = collections.defaultdict(list)
    for d, v in per.items():
        by_kernel[names[d]].append(v)
    return {k: (sum(v) / len(v), len(v)) for k, v in by_kernel.items()}


def summarize_pmc(fetch_dir, write_dir, out, cmd):
    fetch = _per_dispatch(_csv_rows(fetch_dir, "counter_collection.csv"), "FETCH_SIZE")
    write = _per_dispatch(_csv_rows(write_dir, "counter_collection.csv"), "WRITE_SIZE")
    copy_f = [v[0] for k, v in fetch.items() if "copy_f32_kernel" in k]
    copy_w = [v[0] for k, v in write.items() if "copy_f32_kernel" in k]
    if not copy_f or not copy_w:
        raise SystemExit("no calibration copy kernel in the counter runs (--calibrate-copy)")
    kib = COPY_BYTES / 1024
    f_fac, w_fac = kib / copy_f[0], kib / copy_w[0]
    lines = ["# HBM traffic per launch (FETCH_SIZE, WRITE_SIZE)", "", "Commands:", "", "```",
             cmd, "```", "",
             f"Calibration: the plain copy of {COPY_BYTES >> 20} MiB read FETCH_SIZE "
             f"{copy_f[0]:.0f} KiB and WRITE_SIZE {copy_w[0]:.0f} KiB per launch against "
             f"{kib:.0f} KiB moved each way, so the factors are {f_fac:.4f} (fetch) and "
             f"{w_fac:.4f} (write).", "",
             "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | calibrated bytes |",
             "|---|---:|---:|---:|"]
    best = None
    for k in sorted(set(fetch) | set(write)):
        fb = fetch.get(k, (0.0, 0))[0] * f_fac * 1024
        wb = write.get(k, (0.0, 0))[0] * w_fac * 1024
        lines.append(f"| `{k[:150]}` | {fetch.get(k, (0.0, 0))[0]:.0f} | "
                     f"{write.get(k, (0.0, 0))[0]:.0f} | {fb + wb:.4g} |")
        calls = fetch.get(k, (0.0, 0))[1]
        if "gemm_" in k and (best is None or calls > best[2]):
            best = (k, fb + wb, calls)
    text = "\n".join(lines) + "\n"
    if best is not None:
        mode = "f32" if "gemm_f32" in best[0] else "f16r"
        kernel, total = best[0], best[1]
        if mode == "f16r":
            # one f16r call is one packing launch plus one GEMM launch; the
            # roofline of that mode is priced on the whole call, so is its traffic
            for k in set(fetch) | set(write):
                if "pack_kernel" in k:
                    total += (fetch.get(k, (0.0, 0))[0] * f_fac +
                              write.get(k, (0.0, 0))[0] * w_fac) * 1024
                    kernel = "pack_kernel + " + kernel
        meta = {"workload": os.environ.get("TRAFFIC_WORKLOAD", ""),
                "tile": os.environ.get("TRAFFIC_TILE", ""), "mode": mode, "kernel": kernel,
                "traffic_bytes_per_launch": total, "source_hash": source_hash(mode),
                "fetch_factor": f_fac, "write_factor": w_fac}
        text += "\nMachine-readable (read by bench.py while the kernel sources are unchanged):\n"
        text += "\n```json\n" + json.dumps(meta) + "\n```\n"
    _write(out, text)


def _write(out, text):
    if out:
        with open(out, "w") as f:
            f.write(text)
    print(text)


if __name__ == "__main__":
    main()
