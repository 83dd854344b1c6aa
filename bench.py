"""Benchmark of libgemm355 on one MI355X: TFLOP/s = 2MNK/t of C = alpha*A@B + beta*C.

One "step" is one library call over the whole path (for f16r: the operand
rounding pass and the GEMM).  The headline workload is the f32 GEMM at
M = N = K = 4096 (alpha 1, beta 0); the line also carries the beta = 1 run and
the f16r GEMM at 8192^3 (alpha 0.75, beta -0.25), each with its fraction of the
matrix-core roof re-measured on this chip in the same run (the Matrix
Multiplication lab, "Part 1 -- the two roofs, again"), the shader clocks,
board power and temperature sampled while it ran, and the CPU oracle timed on
the host cores (the lab, "Part 2 -- the ladder": every rung checked and timed
in the same run).

Protocol: every result is checked against the oracle before it is timed; the
clocks are brought to their working level with synchronised calls first; then
exactly --steps calls are timed between two device synchronisations, with an
event pair around every call on the stream the library launches on.  Tiles are
the library's own choice (its heuristic), the same choice a profiled run of the
same command makes; --tune runs the library's autotuner first.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--workloads a,b,...] [--tune] [--json-out path]
       python bench.py --profile WORKLOAD [--layout TN] [--calls N] [--calibrate-copy]
       python bench.py --summarize-trace DIR --out FILE --cmd "..."
       python bench.py --summarize-counters WORKLOAD DIR [DIR ...] --out FILE --cmd "..."
Prints progress on stderr and ONE JSON line on stdout.
"""
from __future__ import annotations

import argparse
import collections
import json
import os
import re
import sys
import threading
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
# Matrix instruction forms of the roof kernel (gemm355_roof_mfma's `form`).
ROOF_FORMS = {"f32": {0: "v_mfma_f32_32x32x2_f32", 1: "v_mfma_f32_16x16x4_f32"},
              "f16r": {0: "v_mfma_f32_32x32x16_f16", 1: "v_mfma_f32_16x16x32_f16"}}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workloads", default=",".join(SCORED))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tune", action="store_true",
                    help="run the library's autotuner for each workload before timing it")
    ap.add_argument("--no-roofs", action="store_true")
    ap.add_argument("--roof-seconds", type=float, default=2.0)
    ap.add_argument("--sustain-seconds", type=float, default=1.5,
                    help="back-to-back calls of each workload with the clocks and power sampled")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="target CPU time of each oracle sample")
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--profile", metavar="WORKLOAD", default=None,
                    help="run only this workload's call --calls times (for a profiler); a "
                         "workload name or mode:MxNxK (alpha 1, beta 0, U[-1,1] inputs)")
    ap.add_argument("--layout", choices=("NN", "TN", "NT", "TT"), default="NN",
                    help="operand layout of --profile and --summarize-counters: T stores "
                         "that operand transposed (op(A) = A^T from a K x M array, op(B) = "
                         "B^T from an N x K one)")
    ap.add_argument("--calls", type=int, default=20)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB copy kernel (byte-counter calibration)")
    ap.add_argument("--summarize-trace", metavar="DIR", default=None,
                    help="markdown summary of a rocprofv3 --kernel-trace --stats run")
    ap.add_argument("--summarize-counters", nargs="+", metavar="ARG", default=None,
                    help="WORKLOAD DIR [DIR ...]: markdown summary of rocprofv3 --pmc runs")
    ap.add_argument("--out", default=None, help="output file of the --summarize-* modes")
    ap.add_argument("--cmd", default="", help="the commands that produced the profile")
    ap.add_argument("--sweep", metavar="OUT_MD", default=None,
                    help="shape and alignment sweep of both modes (sizes 128..8192, n = "
                         "4088..4104 and 2048..2304, fixed-tile steps); markdown to OUT_MD")
    ap.add_argument("--sweep-repeats", type=int, default=3)
    ap.add_argument("--precision", metavar="OUT_MD", default=None,
                    help="precision study (the lab's Part 4): f32, f16r and f16r with binary16 "
                         "output against float64 of the unrounded inputs; markdown to OUT_MD")
    ap.add_argument("--choice", metavar="OUT_MD", default=None,
                    help="the untuned choice against every configuration timed pinned, at "
                         "square, few-row and ragged shapes of both modes; markdown to OUT_MD")
    ap.add_argument("--thin", metavar="OUT_MD", default=None,
                    help="few-columns sweep (N = 1..64 at M = K = 4096, both modes); markdown "
                         "to OUT_MD")
    ap.add_argument("--skinny", metavar="OUT_MD", default=None,
                    help="few-rows sweep (M = 1..2048 at K = N = 4096, both modes) against "
                         "the HBM and matrix-core roofs; markdown to OUT_MD")
    args = ap.parse_args()

    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.out, args.cmd)
        return
    if args.summarize_counters:
        if len(args.summarize_counters) < 2:
            raise SystemExit("--summarize-counters WORKLOAD DIR [DIR ...]")
        summarize_counters(args.summarize_counters[0], args.summarize_counters[1:], args.out,
                           args.cmd, args.layout)
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
    from workloads import WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(0)
    log(f"device {props.name} ({getattr(props, 'gcnArchName', '?')}), "
        f"{props.multi_processor_count} CUs; libgemm355 {g.version()}")

    if args.profile:
        profile_run(g, torch, dev, profile_target(args.profile), args.calls, args.calibrate_copy,
                    args.layout)
        return
    if args.calibrate_copy:
        copy_calibration(g, torch, dev)
    if args.sweep:
        shape_sweep(g, torch, dev, args.sweep, args.sweep_repeats)
        return
    if args.skinny:
        skinny_sweep(g, torch, dev, args.skinny, args.sweep_repeats)
        return
    if args.choice:
        choice_study(g, torch, dev, args.choice, args.sweep_repeats)
        return
    if args.thin:
        thin_sweep(g, torch, dev, args.thin, args.sweep_repeats)
        return
    if args.precision:
        precision_study(g, torch, dev, args.precision)
        return

    # ------------------------------------------------------------------ roofs
    roofs = {}
    if not args.no_roofs:
        roofs = measure_roofs(g, torch, dev, args.roof_seconds)
        log("measured roofs: " + json.dumps({k: v for k, v in roofs.items() if k != "forms"}))

    # -------------------------------------------------------------- workloads
    names = [n for n in args.workloads.split(",") if n]
    runs = {name: bench_workload(g, torch, dev, WORKLOADS[name], args, roofs) for name in names}

    # ------------------------------------------- the oracle on the host cores
    if not args.no_cpu_baseline:
        for name in names:
            runs[name]["oracle"] = oracle_rate(WORKLOADS[name], args.cpu_seconds)

    primary = PRIMARY if PRIMARY in runs else names[0]
    pr = runs[primary]
    w = WORKLOADS[primary]
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
        "cpu_baseline": pr.get("oracle"),
        "measured_roof": roofs or None,
        "frac_of_measured_roof": pr.get("frac_of_measured_roof"),
        "workloads": runs,
    }
    text = json.dumps(line)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(text + "\n")
    print(text, flush=True)


# ---------------------------------------------------------------------------
# Clocks, power and temperature while the GPU works (the lab's "Setup" keeps a
# sampler beside every sustained run: a roof or a timing means little without
# the clock it ran at).  Read through the amdsmi module of the ROCm install.
# ---------------------------------------------------------------------------
_AMDSMI = None


def _amdsmi_handle():
    """(module, processor handle) of the GPU, or None when amdsmi is missing."""
    global _AMDSMI
    if _AMDSMI is not None:
        return _AMDSMI or None
    try:
        rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
        path = os.path.join(rocm, "share", "amd_smi")
        if os.path.isdir(path) and path not in sys.path:
            sys.path.append(path)
        import amdsmi
        amdsmi.amdsmi_init()
        handles = amdsmi.amdsmi_get_processor_handles()
        _AMDSMI = (amdsmi, handles[0]) if handles else False
    except Exception as e:   # noqa: BLE001 -- the sampler is optional
        log(f"amdsmi unavailable ({e}); clocks and power are not recorded")
        _AMDSMI = False
    return _AMDSMI or None


class GpuSampler:
    """Background thread reading the shader clock of every XCD, the socket
    power and the hotspot temperature every `period` seconds while the block
    it guards runs; summary() gives medians and extremes."""

    def __init__(self, period=0.05):
        self.period = period
        self.rows = []
        self._stop = threading.Event()
        self._thread = None

    def _read(self, smi, h):
        m = smi.amdsmi_get_gpu_metrics_info(h)
        clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float))
                and 0 < c < 10000]
        power = m.get("current_socket_power")
        temp = m.get("temperature_hotspot")
        return (float(np.mean(clks)) if clks else None,
                float(power) if isinstance(power, (int, float)) else None,
                float(temp) if isinstance(temp, (int, float)) else None)

    def _loop(self, smi, h):
        while not self._stop.is_set():
            try:
                self.rows.append(self._read(smi, h))
            except Exception:   # noqa: BLE001 -- a failed read is skipped
                pass
            self._stop.wait(self.period)

    def __enter__(self):
        got = _amdsmi_handle()
        if got:
            self._thread = threading.Thread(target=self._loop, args=got, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread:
            self._thread.join()
        return False

    def summary(self):
        if not self.rows:
            return None
        out = {"samples": len(self.rows), "period_s": self.period, "source": "amdsmi"}
        for idx, key in ((0, "gfx_mhz"), (1, "power_w"), (2, "hotspot_c")):
            vals = [r[idx] for r in self.rows if r[idx] is not None]
            if vals:
                out[f"{key}_median"] = round(float(np.median(vals)), 1)
                out[f"{key}_min"] = round(float(np.min(vals)), 1)
                out[f"{key}_max"] = round(float(np.max(vals)), 1)
        return out


# ---------------------------------------------------------------------------
# GPU timing.
# ---------------------------------------------------------------------------
def warm_clocks(call, torch, seconds=0.25):
    """Synchronised calls for `seconds`, so the clocks sit at the level the
    work itself holds them at before anything is timed."""
    until = time.perf_counter() + seconds
    while True:
        call()
        torch.cuda.synchronize()
        if time.perf_counter() >= until:
            return


def call_times(call, torch, seconds=0.5, at_least=3, per_sample=1, chunk=8):
    """GPU seconds per call, one sample per event pair: chunks of `chunk`
    samples are queued back to back (each sample `per_sample` calls between its
    two events) and read after one synchronisation per chunk, until `seconds`
    have passed and at least `at_least` samples exist.  Warm the clocks first."""
    stream = torch.cuda.current_stream()
    out = []
    until = time.perf_counter() + seconds
    while len(out) < at_least or time.perf_counter() < until:
        marks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(chunk)]
        for begin, end in marks:
            begin.record(stream)
            for _ in range(per_sample):
                call()
            end.record(stream)
        marks[-1][1].synchronize()
        out.extend(b.elapsed_time(e) * 1e-3 / per_sample for b, e in marks)
    return out


def median_call_time(call, torch, seconds=0.5, per_sample=1):
    warm_clocks(call, torch, min(0.25, seconds / 2))
    return float(np.median(call_times(call, torch, seconds, per_sample=per_sample)))


def sustained(launch, torch, seconds, in_flight=4):
    """Keep up to `in_flight` launches queued for `seconds`; returns (launches,
    GPU seconds between an event before the first and one after the last)."""
    stream = torch.cuda.current_stream()
    first, last = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    queued = collections.deque()
    first.record(stream)
    launches = 0
    until = time.perf_counter() + seconds
    while time.perf_counter() < until:
        launch()
        launches += 1
        done = torch.cuda.Event()
        done.record(stream)
        queued.append(done)
        if len(queued) > in_flight:
            queued.popleft().synchronize()
    last.record(stream)
    last.synchronize()
    return launches, first.elapsed_time(last) * 1e-3


# ---------------------------------------------------------------------------
# Roofs (the lab's "Part 1 -- the two roofs, again"): a kernel of nothing but
# independent matrix instructions, in each instruction form of the mode, run
# for `seconds` with the clocks sampled; the fastest form is the mode's roof.
# The HBM read roof: a 16-byte grid-stride read of 4 GiB (beyond the 256 MB
# memory-side cache).
# ---------------------------------------------------------------------------
def measure_roofs(g, torch, dev, seconds):
    import ctypes

    L = g.lib()
    out = {"forms": {}}
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    blocks = 256 * 4   # four workgroups of four waves per CU
    sink = torch.empty(blocks * 256, device=dev, dtype=torch.float32)
    for mode, name in ((0, "f32"), (1, "f16r")):
        best = None
        for form, instr in ROOF_FORMS[name].items():
            iters = 2000 if mode == 0 else 4000
            flops = ctypes.c_double(0)

            def launch(mode=mode, form=form, iters=iters, flops=flops):
                st = L.gemm355_roof_mfma(mode, form, iters, blocks,
                                         ctypes.c_void_p(sink.data_ptr()), ctypes.byref(flops), sp)
                if st != 0:
                    raise g.Gemm355Error(st, "gemm355_roof_mfma")

            launch()
            torch.cuda.synchronize()
            with GpuSampler() as smp:
                n, span = sustained(launch, torch, seconds)
            rate = flops.value * n / span / 1e12
            out["forms"][f"{name}:{instr}"] = {"tflops": round(rate, 2), "launches": n,
                                               "seconds": round(span, 3), "gpu": smp.summary()}
            log(f"roof {name} {instr}: {rate:.1f} TFLOP/s over {span:.2f} s"
                + (f" at {smp.summary()['gfx_mhz_median']} MHz" if smp.summary() else ""))
            if best is None or rate > best[0]:
                best = (rate, instr, smp.summary())
        out[f"mfma_{name}_tflops"] = best[0]
        out[f"mfma_{name}_form"] = best[1]
        out[f"mfma_{name}_gpu"] = best[2]
        out[f"mfma_{name}_published_tflops"] = PEAK_TFLOPS[name]
    # the vector FMA roof (the lab's fma_peak), the cross-check of the f32 matrix
    # roof: one FMA per element, since no packed f32 instruction is built here
    fflops = ctypes.c_double(0)

    def launch_fma():
        st = L.gemm355_roof_fma(20000, blocks, ctypes.c_void_p(sink.data_ptr()),
                                ctypes.byref(fflops), sp)
        if st != 0:
            raise g.Gemm355Error(st, "gemm355_roof_fma")

    launch_fma()
    torch.cuda.synchronize()
    with GpuSampler() as smp:
        n, span = sustained(launch_fma, torch, seconds)
    out["fma_f32_tflops"] = fflops.value * n / span / 1e12
    out["fma_f32_gpu"] = smp.summary()
    log(f"roof f32 vector FMA (v_fma_f32): {out['fma_f32_tflops']:.1f} TFLOP/s over {span:.2f} s")
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, device=dev, dtype=torch.float32)
    sink1 = torch.zeros(1, device=dev, dtype=torch.float32)

    def read():
        st = L.gemm355_roof_hbm(ctypes.c_void_p(buf.data_ptr()), nbytes, 256 * 8,
                                ctypes.c_void_p(sink1.data_ptr()), sp)
        if st != 0:
            raise g.Gemm355Error(st, "gemm355_roof_hbm")

    with GpuSampler() as smp:
        t = median_call_time(read, torch, 0.5)
    out["hbm_read_gbs"] = nbytes / t / 1e9
    out["hbm_gpu"] = smp.summary()
    out["hbm_published_gbs"] = PEAK_HBM_GBS
    del buf
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------
# One workload: check, then time exactly --steps calls.
# ---------------------------------------------------------------------------
def _workload_tensors(w, torch, dev):
    from workloads import workload_inputs
    A, B, C = workload_inputs(w)
    return (A, B, C), (torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev),
                       torch.from_numpy(C).to(dev))


def bench_workload(g, torch, dev, w, args, roofs):
    import oracle   # correctness check before timing (CPU, test infrastructure)
    from workloads import sample_indices

    log(f"{w.name}: generating inputs")
    (A, B, C), (tA, tB, tC) = _workload_tensors(w, torch, dev)
    fn = g.gemm_f32 if w.mode == "f32" else g.gemm_f16r_f32acc
    if args.tune:
        log(f"{w.name}: tuning")
        g.tune(w.mode, tA, tB, tC, beta=w.beta)
    tile = g.get_config(w.mode, w.M, w.N, w.K, beta=w.beta)
    log(f"{w.name}: tile {tile}")

    # correctness first: one call on the workload's C, oracle-sampled elements
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

    def call():   # C drifts from call to call when beta != 0; the timing does not depend on it
        fn(tA, tB, tC, w.alpha, w.beta)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    warm_clocks(call, torch, 0.25)

    marks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.steps)]
    with GpuSampler(period=0.01) as smp:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for begin, end in marks:
            begin.record(stream)
            call()
            end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    per = np.array([b.elapsed_time(e) * 1e-3 for b, e in marks])
    # The timed steps last tens of milliseconds, about the update interval of
    # the board's power reading: the clocks and power of the call are sampled
    # over a sustained stretch of back-to-back calls as well.
    with GpuSampler() as held:
        n_held, span_held = sustained(call, torch, args.sustain_seconds)

    flops = w.flops
    avg = float(per.mean())
    achieved = flops / avg / 1e12
    peak = PEAK_TFLOPS[w.mode]
    roof = {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": None,
            "kernel": dominant_kernel(w.mode, tile),
            "per_launch_flops": flops,
            "timed_as": "mean of the event-timed library calls (one launch for the f32 ring; "
                        "the packing pass plus the GEMM launch for f16r)"}
    res = {
        "mode": w.mode, "M": w.M, "N": w.N, "K": w.K, "alpha": w.alpha, "beta": w.beta,
        "tile": tile,
        "ms_per_step": wall / args.steps * 1e3,
        "ms_median_call": float(np.median(per)) * 1e3,
        "ms_mean_call": avg * 1e3,
        "gpu_busy_frac": float(per.sum()) / wall,
        "tflops_job": flops * args.steps / wall / 1e12,
        "tflops_median_call": flops / float(np.median(per)) / 1e12,
        "parity_max_ratio_sampled": ratio,
        "gpu_timed_steps": smp.summary(),
        "sustained": {"tflops": w.flops * n_held / span_held / 1e12, "calls": n_held,
                      "seconds": round(span_held, 3), "gpu": held.summary()},
        "roofline": roof,
    }
    tr = committed_traffic(w.mode, w.name, tile)
    if tr is not None:
        roof["traffic"] = tr["traffic_bytes_per_launch"]
        roof["traffic_source"] = tr["source"]
        res["counters"] = {"source": tr["source"], "kernels": tr["kernels"]}
    key = f"mfma_{w.mode}_tflops"
    if roofs.get(key):
        res["frac_of_measured_roof"] = round(res["tflops_median_call"] / roofs[key], 4)
    gpu = res["sustained"]["gpu"] or {}
    log(f"{w.name}: {res['tflops_job']:.2f} TFLOP/s over {args.steps} steps "
        f"({res['ms_per_step']:.4f} ms/step, median call {res['ms_median_call']:.4f} ms); "
        f"of published peak {roof['frac']:.3f}"
        + (f", of measured roof {res['frac_of_measured_roof']:.3f}"
           if "frac_of_measured_roof" in res else "")
        + (f"; sustained {res['sustained']['tflops']:.1f} TFLOP/s at {gpu.get('gfx_mhz_median')} MHz, "
           f"{gpu.get('power_w_median')} W" if gpu else ""))
    del tA, tB, tC
    torch.cuda.empty_cache()
    return res


def oracle_rate(w, target_seconds):
    """The oracle as it stands (float64 triple loop, the bound alongside),
    timed on the host cores over the whole workload when that fits in ~30 s,
    else over a band of output rows sized to about target_seconds; the rate
    in TFLOP/s (2 * rows * N * K / t)."""
    import oracle
    from workloads import workload_inputs

    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    os.environ["OMP_NUM_THREADS"] = str(threads)
    A, B, C = workload_inputs(w)

    def run(rows):
        t0 = time.perf_counter()
        oracle.check(w.mode, A, B, C, w.alpha, w.beta, C, rows=(0, rows))
        return time.perf_counter() - t0

    # cost per row from two short bands (widening A and B is a fixed cost)
    t_a, t_b = run(16), run(64)
    per_row = max((t_b - t_a) / 48.0, 1e-6)
    fixed = max(t_a - 16 * per_row, 0.0)
    rows = w.M if fixed + per_row * w.M <= 30.0 else \
        int(min(w.M, max(64, (target_seconds - fixed) / per_row)))
    t = run(rows)
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f
                              if ln.startswith("model name")), "")
    except OSError:
        pass
    what = "the whole workload" if rows == w.M else f"{rows} of {w.M} output rows"
    res = {"value": 2.0 * rows * w.N * w.K / t / 1e12, "unit": "TFLOP/s", "cores": threads,
           "kind": "oracle", "seconds": round(t, 2),
           "sample": f"{what} of {w.name} (float64 triple loop incl. operand widening and "
                     f"the bound), {t:.1f} s", "cpu": cpu_model}
    log(f"oracle {w.name}: {res['value'] * 1e3:.2f} GFLOP/s on {threads} threads "
        f"({res['sample']})")
    return res


def profile_target(spec):
    """A scored workload by name, or mode:MxNxK (alpha 1, beta 0, U[-1,1])."""
    from workloads import WORKLOADS, Workload
    if spec in WORKLOADS:
        return WORKLOADS[spec]
    m = re.fullmatch(r"(f32|f16r):(\d+)x(\d+)x(\d+)", spec)
    if not m:
        raise SystemExit(f"unknown workload {spec!r}: a workload name or mode:MxNxK")
    return Workload(spec, m.group(1), int(m.group(2)), int(m.group(3)), int(m.group(4)), 1.0,
                    0.0, "uniform")


def profile_run(g, torch, dev, w, calls, calibrate, layout="NN"):
    """The workload's call, `calls` times after 3 untimed ones, with the tile
    the benchmark uses (nothing else runs on the GPU besides the optional
    calibration copy): what a profiler of this command sees.  A transposed
    layout stores that operand transposed (copied once, before the calls)."""
    (_, _, _), (tA, tB, tC) = _workload_tensors(w, torch, dev)
    ta, tb = layout[0] == "T", layout[1] == "T"
    if ta:
        tA = tA.t().contiguous()
    if tb:
        tB = tB.t().contiguous()
    tile = g.get_config(w.mode, w.M, w.N, w.K, beta=w.beta, transa=ta, transb=tb)
    log(f"profile {w.name} {layout}: tile {tile}, {calls} calls")
    for _ in range(3):
        g.gemm(w.mode, tA, tB, tC, w.alpha, w.beta, transa=ta, transb=tb)
    torch.cuda.synchronize()
    for _ in range(calls):
        g.gemm(w.mode, tA, tB, tC, w.alpha, w.beta, transa=ta, transb=tb)
    torch.cuda.synchronize()
    if calibrate:
        copy_calibration(g, torch, dev)
    print(json.dumps({"profile": w.name, "layout": layout, "tile": tile, "calls": calls}),
          flush=True)


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
        log(f"sweep: {mode} {n} {kind}: {tiles[case].split(' source=')[0]} ({plans[case]})")

    times = {case: [] for case in cases}
    rng = random.Random(0)
    for rnd in range(repeats):
        order = list(cases)
        rng.shuffle(order)
        for case in order:
            times[case].append(median_call_time(calls[case], torch, 0.3))
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
             "Command:", "", "```", f"python bench.py --sweep {out}", "```", "",
             "Square n x n x n, A, B, C iid N(0,1) (seed n), alpha = 1, beta = 0.  Every case is "
             "checked against the oracle on 256 sampled elements before it is timed; each time "
             f"is the median of {repeats} shuffled rounds, each the median of event-timed calls "
             "over 0.3 s after warming the clocks.  "
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
    # operand layouts at the scored sizes and for few rows of C (K = N = 4096):
    # op(A) = A^T and/or op(B) = B^T, stored transposed, against the plain
    # layout, the library's own choice
    lay = []
    layout_shapes = [("f32", 4096, 4096, 4096), ("f16r", 8192, 8192, 8192)] + [
        (mode, m, 4096, 4096) for mode in ("f32", "f16r") for m in (16, 128, 512)]
    for mode, M, N, K in layout_shapes:
        A, B, C = make_inputs(M, N, K, "normal", seed=M + 7)
        r, c = sample_indices(M, N, 256, seed=4)
        ref, W = oracle.entries(mode, A, B, C, 1.0, 0.0, r, c)
        tA, tB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
        tAt, tBt = tA.t().contiguous(), tB.t().contiguous()
        tC = torch.from_numpy(C).to(dev)
        batch = 1 if M * N * K >= 2 ** 36 else SKINNY_BATCH
        for ta, tb in ((False, False), (True, False), (False, True), (True, True)):
            def call(mode=mode, ta=ta, tb=tb, a=tAt if ta else tA, b=tBt if tb else tB, cc=tC):
                g.gemm(mode, a, b, cc, 1.0, 0.0, transa=ta, transb=tb)
            call()
            torch.cuda.synchronize()
            got = tC[torch.as_tensor(r, device=dev), torch.as_tensor(c, device=dev)].cpu().numpy()
            if not np.all(np.abs(got.astype(np.float64) - ref) <= oracle.TOL[mode] * W):
                raise SystemExit(f"sweep layouts {mode} {M}x{N}x{K} ta={ta} tb={tb}: outside the "
                                 "parity bound")
            t = float(np.median([median_call_time(call, torch, 0.3, per_sample=batch)
                                 for _ in range(repeats)]))
            plan = g.get_plan(mode, M, N, K, beta=0.0, transa=ta, transb=tb).split()[0].split("=")[1]
            tile = g.get_config(mode, M, N, K, beta=0.0, transa=ta, transb=tb).split(" source=")[0]
            lay.append({"mode": mode, "M": M, "N": N, "K": K, "ta": ta, "tb": tb, "seconds": t,
                        "tflops": 2.0 * M * N * K / t / 1e12, "path": plan, "tile": tile})
            log(f"sweep: layout {mode} {M}x{N}x{K} ta={ta} tb={tb}: {t * 1e6:.1f} us ({plan})")
        del tA, tB, tAt, tBt, tC
        torch.cuda.empty_cache()
    lines += ["", "## Operand layouts (the library's own choice; op(X) = X^T stored transposed)", "",
              "Few-row calls are timed in samples of " + str(SKINNY_BATCH) + " back-to-back calls "
              "(GPU time per call in a stream of calls).", "",
              "| mode | M x N x K | layout | us | TFLOP/s | against NN | path | tile |",
              "|---|---|---|---:|---:|---:|---|---|"]
    for r_ in lay:
        nn = next(x for x in lay if x["mode"] == r_["mode"] and x["M"] == r_["M"] and
                  x["N"] == r_["N"] and not x["ta"] and not x["tb"])
        name = ("T" if r_["ta"] else "N") + ("T" if r_["tb"] else "N")
        lines.append(f"| {r_['mode']} | {r_['M']}x{r_['N']}x{r_['K']} | {name} | "
                     f"{r_['seconds'] * 1e6:.1f} | {r_['tflops']:.1f} | "
                     f"{100 * (r_['seconds'] / nn['seconds'] - 1):+.1f}% | {r_['path']} | "
                     f"{r_['tile']} |")
    lines += ["", "```json", json.dumps({"shapes": rows, "layouts": lay}), "```", ""]
    _write(out, "\n".join(lines))


# ---------------------------------------------------------------------------
# The untuned choice (the phobos "gemm, f32" page, "Tuning": the best tile
# depends on the card and the sizes).  At each shape every configuration the
# heuristic weighs there is timed pinned -- in f32 every one that does not
# split K for few rows, in f16r the half-depth rings and the f32-panel ring --
# and the library's own choice without tuning is set beside the fastest.
# ---------------------------------------------------------------------------
CHOICE_SHAPES = {
    "f32": [(n, n, n) for n in (1024, 1536, 1792, 2048, 2304, 2560, 2816, 3072, 3328, 3584,
                                4096, 4608, 5120, 5632, 6144)] +
           [(n, n, n) for n in (1000, 1500, 1800, 2000, 2049, 2300, 2500, 2800, 3000, 3300,
                                3500, 4000, 4097, 4100, 4600, 5000, 5500, 6000, 7000)] +
           [(512, 4096, 4096), (768, 4096, 4096), (1024, 4096, 4096), (1536, 4096, 4096),
            (2048, 4096, 4096), (2048, 2048, 8192), (4096, 4096, 1024), (4000, 4097, 4093),
            (3000, 5000, 2000), (1000, 8000, 4000), (768, 1024, 1024), (1024, 512, 2048),
            (2000, 3000, 1000)],
    "f16r": [(n, n, n) for n in (1792, 2048, 2304, 2560, 2816, 3072, 3328, 3584, 3840, 4096,
                                 4352, 4608, 5120, 5632, 6144, 6656, 7168, 7680, 8192)] +
            [(n, n, n) for n in (1800, 2300, 2800, 3000, 3300, 4097, 4600, 5500, 6000, 7000)] +
            [(768, 4096, 4096), (1024, 4096, 4096), (1280, 4096, 4096), (1536, 4096, 4096),
             (2048, 4096, 4096), (3072, 4096, 4096), (2048, 2048, 8192), (4096, 4096, 1024),
             (8192, 8192, 2048), (4096, 8192, 4096), (1024, 8192, 8192), (3000, 5000, 2000),
             (1000, 8000, 4000), (2000, 3000, 1000),
             # small products: few packed tiles for a deep K, or a shallow K
             (1024, 2048, 4096), (1280, 1280, 4096), (1024, 1024, 8192), (1448, 1448, 4096),
             (1280, 1280, 2048), (1536, 1536, 1024), (2048, 2048, 512), (1280, 1024, 512),
             (2048, 2048, 1024), (1792, 1792, 1024), (1448, 1448, 2048), (1024, 1024, 2048),
             (2048, 1024, 2048), (1280, 1280, 1024)],
}


def _choice_candidates(g, mode):
    if mode == "f32":
        return [c for c in g.list_configs(mode) if "KS=1" not in c and "KS=2" not in c]
    # the half-depth rings of the packed path and the f32-panel ring that
    # rounds on load (no packing pass)
    return [c for c in g.list_configs(mode) if "BK=32" in c and ("KS=" not in c or "KS=3" in c)]


def choice_study(g, torch, dev, out, repeats):
    import random

    import oracle
    from workloads import make_inputs, sample_indices

    g.cache_clear()
    rows = []
    for mode in ("f32", "f16r"):
        cands = _choice_candidates(g, mode)
        for (M, N, K) in CHOICE_SHAPES[mode]:
            A, B, C = make_inputs(M, N, K, "normal", seed=M + 3 * N + 7 * K)
            r, c = sample_indices(M, N, 64, seed=3)
            ref, W = oracle.entries(mode, A, B, C, 1.0, 0.0, r, c)
            tA, tB, tC = (torch.from_numpy(x).to(dev) for x in (A, B, C))
            del A, B, C
            heur = g.get_config(mode, M, N, K, beta=0.0).split(" source=")[0]
            plan = g.get_plan(mode, M, N, K, beta=0.0)
            fn = g.gemm_f32 if mode == "f32" else g.gemm_f16r_f32acc
            cfgs = list(dict.fromkeys(cands + [heur]))
            calls, reps = {}, {}
            for cfg in cfgs:
                def call(fn=fn, cfg=cfg):
                    g.set_config(mode, cfg)
                    try:
                        fn(tA, tB, tC, 1.0, 0.0)
                    finally:
                        g.set_config(mode, None)
                call()
                torch.cuda.synchronize()
                got = tC[torch.as_tensor(r, device=dev), torch.as_tensor(c, device=dev)].cpu().numpy()
                if not np.all(np.abs(got.astype(np.float64) - ref) <= oracle.TOL[mode] * W):
                    raise SystemExit(f"choice {mode} {M}x{N}x{K} {cfg}: outside the parity bound")
                calls[cfg] = call
                t0 = median_call_time(call, torch, 0.02)
                reps[cfg] = max(1, min(10, int(2e-4 / max(t0, 1e-6))))
            times = {cfg: [] for cfg in cfgs}
            rng = random.Random(M * N + K)
            for _ in range(repeats):
                order = list(cfgs)
                rng.shuffle(order)
                for cfg in order:
                    times[cfg].append(median_call_time(calls[cfg], torch, 0.04, per_sample=reps[cfg]))
            med = {cfg: float(np.median(v)) for cfg, v in times.items()}
            best = min(med, key=med.get)
            rows.append({"mode": mode, "M": M, "N": N, "K": K, "heuristic": heur, "plan": plan,
                         "heuristic_s": med[heur], "best": best, "best_s": med[best],
                         "ratio": med[heur] / med[best], "times": med})
            log(f"choice: {mode} {M}x{N}x{K}: {heur} {med[heur] * 1e6:.1f} us, fastest {best} "
                f"{med[best] * 1e6:.1f} us ({med[heur] / med[best]:.3f})")
            del tA, tB, tC
            torch.cuda.empty_cache()

    lines = ["# The untuned choice against every configuration timed pinned (one MI355X)", "",
             "Command:", "", "```", f"python bench.py --choice {out}", "```", "",
             "A, B, C iid N(0,1), alpha = 1, beta = 0.  At each shape every candidate is checked "
             "against the oracle on 64 sampled elements, then timed pinned: the median of "
             f"{repeats} shuffled rounds, each the median of event-timed calls over 0.04 s after "
             "warming the clocks (calls under 0.2 ms in batches).  Candidates: in f32 every "
             "configuration that does not split K for few rows (the rings, the register-staged "
             "tiles and the f32-panel ring), in f16r the half-depth rings of the packed path and "
             "the f32-panel ring that rounds on load.  `ratio` is the "
             "untuned choice's time over the fastest candidate's.", ""]
    for mode in ("f32", "f16r"):
        sel = [r for r in rows if r["mode"] == mode]
        ratios = [r["ratio"] for r in sel]
        lines += [f"## {mode}", "",
                  f"{len(sel)} shapes: the untuned choice within 2% of the fastest at "
                  f"{sum(x <= 1.02 for x in ratios)}, within 5% at {sum(x <= 1.05 for x in ratios)}; "
                  f"mean ratio {np.mean(ratios):.3f}, worst {max(ratios):.3f}.", "",
                  "| M x N x K | untuned choice | plan | us | fastest pinned | us | ratio |",
                  "|---|---|---|---:|---|---:|---:|"]
        for r in sel:
            lines.append(f"| {r['M']}x{r['N']}x{r['K']} | {r['heuristic']} | {r['plan']} | "
                         f"{r['heuristic_s'] * 1e6:.1f} | {r['best']} | {r['best_s'] * 1e6:.1f} | "
                         f"{r['ratio']:.3f} |")
        lines.append("")
    brief = [{k: (round(v * 1e6, 1) if k.endswith("_s") else v) for k, v in r.items()
              if k != "times"} for r in rows]
    lines += ["```json", json.dumps(brief), "```", ""]
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
            t = median_call_time(fn, torch, 0.5)
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
             "Command:", "", "```", f"python bench.py --precision {out}", "```", "",
             "A, B = U[0,1) - 0.5 (float32, seed 0), C = A @ B (alpha 1, beta 0).  Errors against "
             "the float64 product of the unrounded inputs, computed by the oracle: normalised "
             "max error max|C - ref| / max|ref| and relative Frobenius error "
             "||C - ref|| / ||ref||.  The last two columns measure the same against the float64 "
             "product of the binary16-rounded inputs, which separates the rounding of the "
             "operands (and of the output) from the f32 accumulation.  Times: event-timed calls, "
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
            kinds = ("tuned", "split-K", "rows", "no split-K",
                     "round on load" if mode == "f16r" else "panel ring")
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
            # rest), or the best of the KS=3 configurations (f16r: those that
            # round the operands as they stage them; f32: the f32-panel ring)
            best, best_t = None, 1e30
            for cfg in g.list_configs(mode):
                if ("KS=3" not in cfg) if kind in ("round on load", "panel ring") else ("KS=" in cfg):
                    continue
                g.set_config(mode, cfg)
                try:
                    t = median_call_time(lambda fn=fn, tA=tA, tC=tC: fn(tA, tB, tC, 1.0, 0.0),
                                         torch, 0.05, per_sample=SKINNY_BATCH)
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
        log(f"skinny: {mode} M={M} {kind}: {tiles[key].split(' source=')[0]}")
    times = {k: [] for k in calls}
    rng = random.Random(1)
    for rnd in range(repeats):
        order = list(calls)
        rng.shuffle(order)
        for k in order:
            times[k].append(median_call_time(calls[k], torch, 0.2, per_sample=SKINNY_BATCH))
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
             "Command:", "", "```", f"python bench.py --skinny {out}", "```", "",
             "A (M x K), B (K x N), C iid N(0,1); alpha = 1, beta = 0.  Every case is checked "
             "against the oracle on 256 sampled elements before it is timed; the time is the "
             f"median of {repeats} shuffled rounds of event-timed samples (0.2 s), each sample "
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
             "pass), `panel ring` (f32) the fastest of the f32-panel ring's configurations (KS=3: "
             "direct-to-LDS f32 panels, K split, slices added in order by the tile's last "
             "workgroup); `no split-K` is the fastest configuration of none of these kinds.", "",
             "| mode | M | choice | TFLOP/s | GB/s | FLOP/B | bound | of roof | tile |",
             "|---|---:|---|---:|---:|---:|---|---:|---|"]
    for r_ in sorted(rows, key=lambda r_: (r_["mode"], r_["M"], r_["kind"])):
        lines.append(f"| {r_['mode']} | {r_['M']} | {r_['kind']} | {r_['tflops']:.2f} | "
                     f"{r_['gbs']:.0f} | {r_['intensity']:.1f} | {r_['bound']} | "
                     f"{r_['frac_of_roof']:.2f} | {r_['tile']} |")
    lines += ["", "```json", json.dumps({"roofs": roofs, "rows": rows}), "```", ""]
    _write(out, "\n".join(lines))


THIN_N = [1, 2, 4, 8, 16, 32, 64]


def thin_sweep(g, torch, dev, out, repeats):
    """Few columns of C: N = 1 .. 64 at M = K = 4096.  The calls stream A
    (64 MiB), so the bound is A's bytes over the HBM read roof; compared: the
    library's tuned choice, the few-rows configuration pinned (for N <= 16 its
    few-columns form, the transposed problem) and the fastest configuration of
    any other kind."""
    import random

    import oracle
    from workloads import make_inputs, sample_indices

    roofs = measure_roofs(g, torch, dev, 1.0)
    M = K = 4096
    A = make_inputs(M, 1, K, "normal", seed=4097)[0]
    tA = torch.from_numpy(A).to(dev)
    calls, tiles, plans = {}, {}, {}
    for N in THIN_N:
        B = make_inputs(1, N, K, "normal", seed=N)[1]
        C = make_inputs(M, N, 1, "normal", seed=N + 1)[2]
        r, c = sample_indices(M, N, 256, seed=3)
        tB, tC = torch.from_numpy(B).to(dev), torch.from_numpy(C).to(dev)
        for mode in ("f32", "f16r"):
            ref, W = oracle.entries(mode, A, B, C, 1.0, 0.0, r, c)
            fn = g.gemm_f32 if mode == "f32" else g.gemm_f16r_f32acc
            for kind in ("tuned", "rows", "other"):
                key = (mode, N, kind)
                if kind == "tuned":
                    g.tune(mode, tA, tB, tC, beta=0.0)
                    cfg = g.get_config(mode, M, N, K, beta=0.0).split(" source=")[0]
                    pin = None
                elif kind == "rows":
                    cfg = pin = g.parse_config(mode, "KS=2")
                else:
                    best, best_t = None, 1e30
                    for cand in g.list_configs(mode):
                        if "KS=2" in cand:
                            continue
                        g.set_config(mode, cand)
                        try:
                            t = median_call_time(lambda fn=fn, tB=tB, tC=tC: fn(tA, tB, tC, 1.0, 0.0),
                                                 torch, 0.05, per_sample=SKINNY_BATCH)
                        finally:
                            g.set_config(mode, None)
                        if t < best_t:
                            best, best_t = cand, t
                    cfg = pin = best

                def call(fn=fn, tB=tB, tC=tC, mode=mode, pin=pin):
                    if pin:
                        g.set_config(mode, pin)
                    try:
                        fn(tA, tB, tC, 1.0, 0.0)
                    finally:
                        if pin:
                            g.set_config(mode, None)
                call()
                torch.cuda.synchronize()
                got = tC[torch.as_tensor(r, device=dev), torch.as_tensor(c, device=dev)].cpu().numpy()
                if not np.all(np.abs(got.astype(np.float64) - ref) <= oracle.TOL[mode] * W):
                    raise SystemExit(f"thin {key}: outside the parity bound")
                if pin:
                    g.set_config(mode, pin)
                try:
                    plans[key] = g.get_plan(mode, M, N, K, beta=0.0).split()[0].split("=")[1]
                finally:
                    if pin:
                        g.set_config(mode, None)
                calls[key], tiles[key] = call, cfg
                log(f"thin: {mode} N={N} {kind}: {cfg} ({plans[key]})")
    times = {k: [] for k in calls}
    rng = random.Random(2)
    for rnd in range(repeats):
        order = list(calls)
        rng.shuffle(order)
        for k in order:
            times[k].append(median_call_time(calls[k], torch, 0.2, per_sample=SKINNY_BATCH))
        log(f"thin: round {rnd + 1} of {repeats} done")
    hbm = roofs["hbm_read_gbs"] * 1e9
    rows = []
    for (mode, N, kind), ts in times.items():
        t = float(np.median(ts))
        nbytes = 4.0 * (M * K + K * N + M * N)
        rows.append({"mode": mode, "N": N, "kind": kind, "tile": tiles[(mode, N, kind)],
                     "path": plans[(mode, N, kind)], "seconds": t, "gbs": nbytes / t / 1e9,
                     "frac_of_hbm_roof": nbytes / t / hbm})
    lines = ["# Few columns of C: N = 1 .. 64 at M = K = 4096 (both modes, one MI355X)", "",
             "Command:", "", "```", f"python bench.py --thin {out}", "```", "",
             "A (M x K), B (K x N), C iid N(0,1); alpha = 1, beta = 0.  Every case is checked "
             "against the oracle on 256 sampled elements before it is timed; the time is the "
             f"median of {repeats} shuffled rounds of event-timed samples (0.2 s), each sample "
             f"{SKINNY_BATCH} back-to-back calls between two events.  Bytes are the f32 storage "
             "the call must move at least once, 4(MK + KN + MN), against the measured HBM read "
             f"roof {roofs['hbm_read_gbs']:.0f} GB/s.  `tuned` is the library's own choice after "
             "tuning, `rows` the few-rows configuration pinned (KS=2: for N <= 16 its "
             "few-columns form, the transposed problem C^T = B^T A^T, streaming A), `other` the "
             "fastest configuration of any other kind.", "",
             "| mode | N | choice | us | GB/s | of HBM roof | path | tile |",
             "|---|---:|---|---:|---:|---:|---|---|"]
    for r_ in sorted(rows, key=lambda r_: (r_["mode"], r_["N"], r_["kind"])):
        lines.append(f"| {r_['mode']} | {r_['N']} | {r_['kind']} | {r_['seconds'] * 1e6:.1f} | "
                     f"{r_['gbs']:.0f} | {r_['frac_of_hbm_roof']:.2f} | {r_['path']} | "
                     f"{r_['tile']} |")
    lines += ["", "```json", json.dumps({"hbm_read_gbs": roofs["hbm_read_gbs"], "rows": rows}),
              "```", ""]
    _write(out, "\n".join(lines))


# ---------------------------------------------------------------------------
# Profile evidence: byte-counter calibration and the committed summaries of
# rocprofv3 runs (profiles/).  Every summary embeds the exact commands that
# produced it; the summarisers refuse to write one without them.
# ---------------------------------------------------------------------------
COPY_BYTES = 256 << 20          # one direction of the calibration copy
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {
    "f32": ["gemm_tiled_amd/csrc/gemm_f32.hip", "gemm_tiled_amd/csrc/gemm_f32_ring.hip",
            "gemm_tiled_amd/csrc/f32_ring.hpp", "gemm_tiled_amd/csrc/f32_kernel.hpp",
            "gemm_tiled_amd/csrc/internal.hpp"],
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


def _tile_fields(tile):
    return {k: int(v) for k, v in (t.split("=") for t in (tile or "").split()
                                   if "=" in t and t.split("=")[1].isdigit())}


def dominant_kernel(mode, tile):
    """The kernel that does the work of a call with this tile, by the name
    prefix rocprofv3 shows (for f16r, after its packing pass)."""
    f = _tile_fields(tile)
    ks = f.get("KS", 0)
    if ks == 2:
        return "gemm_rows_kernel"
    if ks == 3:
        if f.get("BK") == 32:
            return "gemm_panel_ring_kernel" + (" (no packing pass)" if mode == "f16r" else "")
        return "gemm_f16_direct_kernel (no packing pass)"
    if mode == "f32":
        ring = f.get("ST", 0) >= 3 and f.get("BK") == 16 and ks == 0
        return "gemm_f32_ring_kernel" if ring else "gemm_f32_kernel"
    return "pack_kernel + " + ("gemm_f16_ring_kernel" if f.get("BK") == 32 else "gemm_f16_kernel")


def committed_traffic(mode, workload, tile):
    """HBM bytes per call and the per-kernel counters from the committed
    counter summary of this workload and tile, if it was taken on the current
    kernel sources; else None."""
    import glob
    for path in sorted(glob.glob(os.path.join(PROFILES, "counters", "*.md"))):
        text = open(path).read()
        m = re.search(r"```json\n(.*?)\n```", text, re.S)
        if not m:
            continue
        try:
            d = json.loads(m.group(1))
        except ValueError:
            continue
        if d.get("workload") != workload or d.get("mode") != mode or d.get("layout", "NN") != "NN":
            continue
        if d.get("tile", "").split(" source=")[0] != tile.split(" source=")[0]:
            continue
        if d.get("source_hash") != source_hash(mode):
            return None          # the kernel changed since the counters were taken
        keep = ("duration_us", "cycles_per_xcd", "mfma_util_pct", "lds_bank_conflict_per_access",
                "lds_util_pct", "l2_hit", "hbm_read_bytes", "hbm_write_bytes")
        kernels = {_short(k, 80): {f: v.get(f) for f in keep}
                   for k, v in d.get("kernels", {}).items()}
        return {"traffic_bytes_per_launch": d["traffic_bytes_per_call"],
                "source": os.path.relpath(path, ROOT), "kernels": kernels}
    return None


def _csv_rows(directory, suffix):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True)):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _short(name, n=110):
    name = name.replace("|", "/").replace("g355::(anonymous namespace)::", "").replace("g355::", "")
    return name if len(name) <= n else name[:n] + "..."


def _commands_block(cmd):
    if not cmd.strip():
        raise SystemExit("a profile summary needs the commands that made it (--cmd)")
    return ["Commands (run from the repository root; rocprofv3 writes under gpurun_out/):", "",
            "```", cmd.strip(), "```", ""]


def _dispatch_runs(trace_rows, gap_s=0.1):
    """Dispatches of each kernel split into runs wherever the same kernel was
    idle for more than gap_s (the phases of a benchmark: roofs, each
    workload's check + warm-up + timed calls, tuning): (kernel, durations in
    us, start ns) per run, in time order."""
    by_kernel = collections.defaultdict(list)
    for r in trace_rows:
        by_kernel[r["Kernel_Name"]].append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    runs = []
    for k, ds in by_kernel.items():
        ds.sort()
        cur = [ds[0]]
        for d in ds[1:]:
            if d[0] - cur[-1][1] > gap_s * 1e9:
                runs.append((k, [(e - s) / 1e3 for s, e in cur], cur[0][0]))
                cur = []
            cur.append(d)
        runs.append((k, [(e - s) / 1e3 for s, e in cur], cur[0][0]))
    runs.sort(key=lambda r: r[2])
    return runs


def summarize_trace(directory, out, cmd):
    stats = _csv_rows(directory, "kernel_stats.csv")
    trace = _csv_rows(directory, "kernel_trace.csv")
    if not stats or not trace:
        raise SystemExit(f"no kernel_stats.csv / kernel_trace.csv under {directory}")
    lines = ["# Kernel trace summary", ""] + _commands_block(cmd)
    lines += ["## Runs of each kernel, in time order", "",
              "A run is the dispatches of one kernel with no gap above 0.1 s (the benchmark's "
              "phases: roof kernels, then for each workload its check, warm-up and timed "
              "calls).  Runs of 5 or more dispatches:", "",
              "| # | kernel | dispatches | mean us | median us | min us | max us |",
              "|---:|---|---:|---:|---:|---:|---:|"]
    n = 0
    for k, durs, _ in _dispatch_runs(trace):
        if len(durs) < 5:
            continue
        n += 1
        lines.append(f"| {n} | `{_short(k)}` | {len(durs)} | {np.mean(durs):.1f} | "
                     f"{np.median(durs):.1f} | {np.min(durs):.1f} | {np.max(durs):.1f} |")
    lines += ["", "## Every kernel (rocprofv3 --stats)", "",
              "| kernel | calls | average us | min us | max us | share of GPU time |",
              "|---|---:|---:|---:|---:|---:|"]
    for r in stats:
        lines.append(f"| `{_short(r['Name'])}` | {r['Calls']} | "
                     f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                     f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    _write(out, "\n".join(lines) + "\n")


def _counter_table(dirs):
    """Per kernel: the mean per dispatch of every counter found in the
    counter_collection.csv files of dirs, and the mean duration (us) of the
    same dispatches from the kernel traces of those runs."""
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    dur = {}
    for d in dirs:
        tag = os.path.abspath(d)
        for r in _csv_rows(d, "counter_collection.csv"):
            key = (tag, r["Dispatch_Id"])
            per[key][r["Counter_Name"]] += float(r["Counter_Value"])
            names[key] = r["Kernel_Name"]
        for r in _csv_rows(d, "kernel_trace.csv"):
            dur[(tag, r["Dispatch_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    table = collections.defaultdict(lambda: collections.defaultdict(list))
    for key, vals in per.items():
        for c, v in vals.items():
            table[names[key]][c].append(v)
        if key in dur:
            table[names[key]]["duration_us"].append(dur[key])
    return {k: {c: float(np.mean(v)) for c, v in cs.items()} for k, cs in table.items()}


def summarize_counters(workload, dirs, out, cmd, layout="NN"):
    w = profile_target(workload)
    ta, tb = layout[0] == "T", layout[1] == "T"
    tab = _counter_table(dirs)
    copy = next((v for k, v in tab.items() if "copy_f32_kernel" in k), None)
    if not copy or "FETCH_SIZE" not in copy or "WRITE_SIZE" not in copy:
        raise SystemExit("no calibration copy kernel with FETCH_SIZE and WRITE_SIZE "
                         "(run the profile with --calibrate-copy)")
    kib = COPY_BYTES / 1024
    f_fac, w_fac = kib / copy["FETCH_SIZE"], kib / copy["WRITE_SIZE"]
    mine = {k: v for k, v in tab.items() if "gemm_" in k or "pack_kernel" in k}
    import gemm_tiled_amd as g   # the tile the profiled run used: the library's own choice
    tile = g.get_config(w.mode, w.M, w.N, w.K, beta=w.beta, transa=ta,
                        transb=tb).split(" source=")[0]
    what = "" if layout == "NN" else (f", layout {layout}: " + "; ".join(
        x for x, t in (("A stored K x M", ta), ("B stored N x K", tb)) if t))
    lines = [f"# Counters of the {workload} call ({w.mode}, {w.M}x{w.N}x{w.K}, "
             f"alpha {w.alpha}, beta {w.beta}{what})", ""] + _commands_block(cmd)
    lines += [f"Tile: `{tile}` (the library's own choice for this call).", "",
              f"Byte calibration: the plain copy of {COPY_BYTES >> 20} MiB each way read "
              f"FETCH_SIZE {copy['FETCH_SIZE']:.0f} KiB and WRITE_SIZE {copy['WRITE_SIZE']:.0f} "
              f"KiB per launch, so HBM bytes = FETCH_SIZE x {f_fac:.4f} + WRITE_SIZE x "
              f"{w_fac:.4f} (KiB x 1024).", "",
              "Definitions (rocprofv3's own metrics on gfx950): MfmaUtil = matrix-unit busy "
              "cycles over (GRBM_GUI_ACTIVE x 1024 SIMDs); LdsBankConflict = bank-conflict "
              "cycles per LDS-active cycle not stalled (conflicts per access); LdsUtil = "
              "LDS-active cycles over (GUI-active cycles x 256 CUs); L2 hit = TCC_HIT / "
              "(TCC_HIT + TCC_MISS); cycles = GRBM_GUI_ACTIVE per XCD (the counter sums the 8 "
              "XCDs), over the kernel's duration in the same counted run for the clock (a "
              "counted dispatch runs longer than an uncounted one: divide the cycles by the "
              "kernel trace's duration for the clock of an ordinary run).", "",
              "| kernel | duration us | cycles/XCD (M) | clock MHz | MfmaUtil % | "
              "LdsBankConflict | LdsUtil % | L2 hit | HBM read MB | HBM write MB |",
              "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    meta_k = {}
    for k, v in sorted(mine.items(), key=lambda kv: -kv[1].get("duration_us", 0)):
        du = v.get("duration_us")
        clk = v["GRBM_GUI_ACTIVE"] / 8 / du if du and "GRBM_GUI_ACTIVE" in v else None
        hit = v.get("TCC_HIT_sum")
        miss = v.get("TCC_MISS_sum")
        l2 = hit / (hit + miss) if hit is not None and miss is not None and hit + miss > 0 else None
        rd = v["FETCH_SIZE"] * f_fac * 1024 if "FETCH_SIZE" in v else None
        wr = v["WRITE_SIZE"] * w_fac * 1024 if "WRITE_SIZE" in v else None

        def fmt(x, f):
            return "" if x is None else format(x, f)
        cyc = v["GRBM_GUI_ACTIVE"] / 8 / 1e6 if "GRBM_GUI_ACTIVE" in v else None
        lines.append(f"| `{_short(k)}` | {fmt(du, '.1f')} | {fmt(cyc, '.3f')} | {fmt(clk, '.0f')} | "
                     f"{fmt(v.get('MfmaUtil'), '.1f')} | {fmt(v.get('LdsBankConflict'), '.3f')} | "
                     f"{fmt(v.get('LdsUtil'), '.1f')} | {fmt(l2, '.3f')} | "
                     f"{fmt(rd and rd / 1e6, '.1f')} | {fmt(wr and wr / 1e6, '.1f')} |")
        meta_k[k] = {"duration_us": du, "cycles_per_xcd": cyc and cyc * 1e6, "clock_mhz": clk,
                     "mfma_util_pct": v.get("MfmaUtil"),
                     "lds_bank_conflict_per_access": v.get("LdsBankConflict"),
                     "lds_util_pct": v.get("LdsUtil"), "l2_hit": l2, "hbm_read_bytes": rd,
                     "hbm_write_bytes": wr, "raw": dict(v)}
    flops = 2.0 * w.M * w.N * w.K
    compulsory = 4.0 * (w.M * w.K + w.K * w.N) + 4.0 * w.M * w.N * (2 if w.beta != 0 else 1)
    traffic = sum((m["hbm_read_bytes"] or 0) + (m["hbm_write_bytes"] or 0) for m in meta_k.values())
    lines += ["", f"Per call (every kernel above): HBM traffic {traffic / 1e6:.1f} MB against "
              f"{compulsory / 1e6:.1f} MB compulsory (4(MK + KN) + 4MN read + 4MN written when "
              f"beta != 0, else written only): {traffic / compulsory:.2f}x; "
              f"{flops / max(traffic, 1):.0f} FLOP per HBM byte.", ""]
    meta = {"workload": workload, "layout": layout, "mode": w.mode, "tile": tile,
            "traffic_bytes_per_call": traffic, "compulsory_bytes": compulsory,
            "source_hash": source_hash(w.mode), "fetch_factor": f_fac, "write_factor": w_fac,
            "kernels": meta_k}
    lines += ["Machine-readable (bench.py reads `traffic_bytes_per_call` while the kernel "
              "sources hash to `source_hash`):", "", "```json", json.dumps(meta), "```", ""]
    _write(out, "\n".join(lines))


def _write(out, text):
    if out:
        os.makedirs(os.path.dirname(os.path.abspath(out)), exist_ok=True)
        with open(out, "w") as f:
            f.write(text)
    print(text)


if __name__ == "__main__":
    main()
