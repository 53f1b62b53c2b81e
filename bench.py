#!/usr/bin/env python3
"""Benchmark of the diagonal linear-recurrence scan on one MI355X.

Default workload (the headline metric): the very long forward + backward
fp32 scan, B=2, D=256, T=2^20, [B,D,T] layout (the largest forward+backward
fp32 configuration); one step = lrs_scan_fwd then lrs_scan_bwd over the same
resident inputs.  The same run also measures scan_fwd_bwd (B=8, D=512,
T=4096) and reports it inside the line under "also".  Other workloads
(--workload): scan_fwd_bwd, scan_fused (that step as one lrs_scan_fwd_bwd
call), scan_short (T = 32, sequential kernels), scan_fwd_bwd_bf16 and
scan_long_bf16 (the scans with bf16 arrays, fp32 state),
sru_fwd / sru_fwd_bwd (bf16 SRU layer), sru_deer (SRU with v_f*c_{t-1}
by DEER), lstm_fwd_bwd
(bf16 LSTM cell-state layer with input-only gates), deer / deer_fwd_bwd
(Newton solve, and its backward), scan_fwd_small.

Prints ONE JSON line.  `value` is scanned elements per second over K timed
steps launched back to back from Python (inputs resident in HBM before timing
starts; HIP events only at the two ends of the region).  `roofline` describes
the dominant kernel: algorithmic bytes per launch divided by its average
launch time, measured with HIP events recorded on the launch stream around
every call over a second run of K timed steps (those per-call events add a
few microseconds between launches, which is why they are kept out of the
first region).  `cpu_baseline` times the fp64 CPU oracle
on the host cores over a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "scanned elements/sec (B·D·T) and % of HBM roofline, fwd+bwd, fp32"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published peak

# algorithmic bytes per element of each kernel (every input read once, every
# output written once; per-channel vectors are negligible)
BYTES_PER_ELEM = {"scan_fwd_f32": 12, "scan_bwd_f32": 20, "sru_fwd_bf16": 8,
                  "scan_fwd_bf16": 6, "scan_bwd_bf16": 10,  # the scans with bf16 arrays
                  "sru_fwd_save_bf16": 12,  # + the fp32 cell states for the backward
                  "sru_bwd_bf16": 18,       # z_f, z_r, z_x, dL/dh, c in; three gradients out
                  "scan_fused_f32": 24,     # a, b, dL/dh in; h, dL/da, dL/db out
                  "deer_iter_first": 8, "deer_iter": 12,
                  "deer_fused": 8,          # u in, the last iterate out, all iterations in one pass
                  "deer_bwd_f32": 12,       # h, dL/dh in; dL/du out
                  "sru_deer_iter_first": 8,  # z_f, z_x in; c' out (from c = 0)
                  "sru_deer_iter": 12,       # z_f, z_x, c in; c' out
                  "sru_deer_out": 10,        # z_r, z_x, c in; h out
                  "sru_deer_fused": 8,       # z_f, z_x in; the last iterate out (all iterations)
                  "lstm_fwd_save_bf16": 14,  # four pre-activations in; h and c out
                  "lstm_bwd_bf16": 22}       # four pre-activations, dL/dh, c in; four gradients out
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_counters.json")

# The fused DEER solve is bound by vector-ALU issue, not by HBM: its roofline
# counts the floating-point work of the method's per-element Newton step
# (y'_t = z_t + J_t (y'_{t-1} - y_{t-1}), z_t = tanh(w y_{t-1} + u_t),
# J_t = w (1 - z_t^2), and the update norm):
#   pre-activation fma 2, tanh as exp + add + reciprocal + fma 5, J: mul + fma 3,
#   the update: sub + fma 3, |y' - y| folded into the max: sub + max 2.
DEER_FLOPS_PER_ELEM_ITER = 15
# MI355X published fp32 vector peak (256 CUs x 4 SIMDs x 16 lanes x 2 flops per
# FMA x 2 for packed fp32, 2.4 GHz); code built without packed fp32 issues at
# most half of it.
FP32_VECTOR_PEAK_TFLOPS = 157.3


def deer_fused_applies(T: int, k_max: int, C: int, cus: int) -> bool:
    """The library's default rule for the fused DEER solve: K_max <= 8 and
    channels of at most 8192 steps or at least as many channels as the device
    has compute units (`cus`)."""
    return k_max <= 8 and (T <= 8192 or C >= cus)


def sru_deer_fused_applies(C: int, k_max: int) -> bool:
    """The library's default rule for the fused SRU-by-DEER walk: the
    persistent plan (at least one 128-channel block per compute unit, 256 on
    MI355X) and K_max <= 8."""
    import torch
    min_blocks = torch.cuda.get_device_properties(0).multi_processor_count
    return (C + 127) // 128 >= min_blocks and k_max <= 8


def csrc_hash() -> str:
    d = os.path.join(ROOT, "linear_recurrence_scan_diagonal_amd", "csrc")
    h = hashlib.sha256()
    for fn in sorted(os.listdir(d)):
        with open(os.path.join(d, fn), "rb") as f:
            h.update(fn.encode() + f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel_key: str):
    """HBM bytes per launch of a kernel on a workload from the committed
    counter summary, or None when there is none or the kernel sources changed
    since the counters were taken."""
    try:
        with open(COUNTERS_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    k = rec.get(f"{workload}/{kernel_key}")
    if k is None or k.get("csrc_hash") != csrc_hash():
        return None
    return k.get("hbm_bytes_per_launch")


# rocprof kernel names of each timed entry point (substring match)
KERNEL_NAMES = {"scan_fwd_f32": ("k_scan_fwd_bdt<float", "k_scan_fwd_tbd<float",
                                 "k_scan_fwd_serial<float", "k_scan_fwd_packed<float"),
                "scan_bwd_f32": ("k_scan_bwd_bdt<float", "k_scan_bwd_tbd<float",
                                 "k_scan_bwd_serial<float", "k_scan_bwd_packed<float"),
                "scan_fwd_bf16": ("k_scan_fwd_bdt<unsigned short", "k_scan_fwd_tbd<unsigned short",
                                  "k_scan_fwd_serial<unsigned short",
                                  "k_scan_fwd_packed<unsigned short"),
                "scan_bwd_bf16": ("k_scan_bwd_bdt<unsigned short", "k_scan_bwd_tbd<unsigned short",
                                  "k_scan_bwd_serial<unsigned short",
                                  "k_scan_bwd_packed<unsigned short"),
                "scan_fused_f32": ("k_scan_fused_bdt<float",),
                "sru_fwd_bf16": ("k_sru_fwd<unsigned short", "k_sru_fwd_persist<unsigned short"),
                "sru_fwd_save_bf16": ("k_sru_fwd<unsigned short",
                                      "k_sru_fwd_persist<unsigned short"),
                "sru_bwd_bf16": ("k_sru_bwd<unsigned short",),
                "deer_solve": ("k_deer_fused<", "k_deer_iter"),
                "sru_deer_bf16": ("k_sru_deer_fused<unsigned short", "k_sru_deer_iter<unsigned short",
                                  "k_sru_deer_iter_persist<unsigned short"),
                "deer_bwd_f32": ("k_deer_bwd",),
                "lstm_fwd_save_bf16": ("k_lstm_fwd<unsigned short",
                                       "k_lstm_fwd_persist<unsigned short"),
                "lstm_bwd_bf16": ("k_lstm_bwd<unsigned short",)}
# entry points timed by each workload
WORKLOAD_KERNELS = {"scan_fwd_small": ("scan_fwd_f32",),
                    "scan_fwd_bwd": ("scan_fwd_f32", "scan_bwd_f32"),
                    "scan_long": ("scan_fwd_f32", "scan_bwd_f32"),
                    "scan_fwd_bwd_bf16": ("scan_fwd_bf16", "scan_bwd_bf16"),
                    "scan_long_bf16": ("scan_fwd_bf16", "scan_bwd_bf16"),
                    "scan_fused": ("scan_fused_f32",),
                    "scan_short": ("scan_fwd_f32", "scan_bwd_f32"),
                    "sru_fwd": ("sru_fwd_bf16",),
                    "sru_fwd_bwd": ("sru_fwd_save_bf16", "sru_bwd_bf16"),
                    "deer": ("deer_solve",),
                    "deer_fwd_bwd": ("deer_solve", "deer_bwd_f32"),
                    "sru_deer": ("sru_deer_bf16",),
                    "lstm_fwd_bwd": ("lstm_fwd_save_bf16", "lstm_bwd_bf16")}
# entry points that launch one kernel per Newton iteration
SOLVE_KEYS = ("deer_solve", "sru_deer_bf16")
CALIB_NAME = "CUDAFunctor_add<float>"  # the stream reference kernel
CALIB_READ = 2 * 4 * (1 << 26)
CALIB_WRITE = 4 * (1 << 26)


def summarize(args):
    """Turn rocprofv3 CSV output (kernel trace + stats, and one --pmc run each
    for FETCH_SIZE and WRITE_SIZE) into profiles/<workload>.md (every kernel the
    workload launches) and
    the per-launch HBM traffic record in profiles/hbm_counters.json."""
    import csv
    import glob
    d = args.summarize
    wl = args.workload
    tag = wl if args.layout == "bdt" else f"{wl}_{args.layout}"  # output and record name
    cmd_base = (f"python3 bench.py --workload {wl}" +
                (f" --layout {args.layout}" if args.layout != "bdt" else "") + " --also none")

    def rows(pattern):
        out = []
        for f in sorted(glob.glob(os.path.join(d, pattern), recursive=True)):
            with open(f) as fh:
                out.extend(csv.DictReader(fh))
        return out

    stats = rows(f"trace_{tag}/**/*kernel_stats.csv")
    pmc = {c: rows(f"{c.lower()}_{tag}/**/*counter_collection.csv") for c in ("FETCH_SIZE", "WRITE_SIZE")}
    bench_line = None
    for f in glob.glob(os.path.join(d, f"trace_{tag}.json")):
        with open(f) as fh:
            for line in fh:
                if line.startswith("{"):
                    bench_line = json.loads(line)

    def per_dispatch(counter, pat):
        vals = [float(r["Counter_Value"]) * 1024 for r in pmc[counter] if pat in r["Kernel_Name"]]
        return sum(vals) / len(vals) if vals else None

    factor = {}
    for c, known in (("FETCH_SIZE", CALIB_READ), ("WRITE_SIZE", CALIB_WRITE)):
        v = per_dispatch(c, CALIB_NAME)
        factor[c] = known / v if v else None
    try:
        with open(COUNTERS_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    lines = [f"# rocprofv3 summary: workload `{tag}`", "",
             "Commands (repo root, one MI355X):", "",
             f"    rocprofv3 --kernel-trace --stats -f csv -d <out>/trace_{tag} -o t -- {cmd_base} --steps 20 --warmup 3 --no-cpu-baseline > <out>/trace_{tag}.json",
             f"    rocprofv3 --pmc FETCH_SIZE -f csv -d <out>/fetch_size_{tag} -o p -- {cmd_base} --steps 3 --warmup 1 --no-cpu-baseline",
             f"    rocprofv3 --pmc WRITE_SIZE -f csv -d <out>/write_size_{tag} -o p -- {cmd_base} --steps 3 --warmup 1 --no-cpu-baseline",
             f"    python3 bench.py --summarize <out> --workload {wl}" + (f" --layout {args.layout}" if args.layout != "bdt" else ""),
             "", "## Kernel trace (--stats)", "",
             "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for r in stats:
        if "lrs::" in r["Name"] or CALIB_NAME in r["Name"]:
            lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs'])/1e3:.2f} | "
                         f"{float(r['MinNs'])/1e3:.2f} | {float(r['MaxNs'])/1e3:.2f} |")
    fused = [r for r in stats if "lrs::k_deer_fused<" in r["Name"]]
    if fused:
        from linear_recurrence_scan_diagonal_amd import inputs as I
        us = float(fused[0]["AverageNs"]) / 1e3
        n = I.WORKLOADS[wl].N
        tf = DEER_FLOPS_PER_ELEM_ITER * n * 5 / (us * 1e-6) / 1e12
        lines += ["", f"ALU view of `k_deer_fused` (vector-ALU bound): {DEER_FLOPS_PER_ELEM_ITER} flops "
                  f"per element and Newton iteration x {n} elements x 5 iterations / {us:.2f} us = "
                  f"{tf:.2f} TFLOP/s, {100 * tf / FP32_VECTOR_PEAK_TFLOPS:.1f}% of the "
                  f"{FP32_VECTOR_PEAK_TFLOPS} TFLOP/s fp32 vector peak."]
    # an entry point that needs look-back state launches the reset kernel
    # first; bench.py's events bracket the whole call
    reset = [r for r in stats if "k_reset" in r["Name"]]
    reset_us = float(reset[0]["AverageNs"]) / 1e3 if reset else 0.0
    reset_calls = int(reset[0]["Calls"]) if reset else 0
    ep = []
    keys = WORKLOAD_KERNELS[wl]
    mains = [r for r in stats for key in keys
             if key not in SOLVE_KEYS and any(p in r["Name"] for p in KERNEL_NAMES[key])]
    main_calls = sum(int(r["Calls"]) for r in mains)
    for key in keys:
        pats = KERNEL_NAMES[key]
        for r in stats:
            if any(p in r["Name"] for p in pats) and key not in SOLVE_KEYS:
                share = reset_calls / main_calls if main_calls else 0.0
                ep.append(f"{key}: {float(r['AverageNs'])/1e3:.2f} us kernel"
                          + (f" + {share:.0f} x {reset_us:.2f} us reset = "
                             f"{float(r['AverageNs'])/1e3 + share * reset_us:.2f} us per call"
                             if share >= 1 else ""))
    if ep:
        lines += ["", "Per entry-point call (rocprof averages): " + "; ".join(ep) + "."]
    if bench_line:
        lines += ["", "Same run, bench.py's own per-kernel HIP-event averages (ms, one event "
                  "after each entry-point call of queued steps): "
                  f"{bench_line.get('per_kernel_ms')}; value {bench_line['value']:.4g} elements/s, "
                  f"{bench_line['ms_per_step']:.5f} ms/step."]
    lines += ["", "## HBM traffic (--pmc, per dispatch)", "",
              f"Calibration: torch add over 3 x 256 MiB reads {CALIB_READ} B and writes {CALIB_WRITE} B; "
              f"its FETCH_SIZE/WRITE_SIZE scale to those byte counts by factors "
              f"{factor['FETCH_SIZE'] and round(factor['FETCH_SIZE'], 3)} and "
              f"{factor['WRITE_SIZE'] and round(factor['WRITE_SIZE'], 3)}.", "",
              "| kernel | raw FETCH KiB | raw WRITE KiB | scaled HBM bytes | algorithmic bytes | ratio |",
              "|---|---|---|---|---|---|"]
    # the sources the profiled run was built from (its bench line), else these
    src_hash = (bench_line or {}).get("csrc_hash") or csrc_hash()
    if src_hash != csrc_hash():
        print(f"note: the profiled run used kernel sources {src_hash}, this tree has {csrc_hash()}",
              file=sys.stderr)
    from linear_recurrence_scan_diagonal_amd import inputs as I
    w = I.WORKLOADS[wl]
    for key in WORKLOAD_KERNELS[wl]:
        pats = KERNEL_NAMES[key]
        for pat in pats:
            f_ = per_dispatch("FETCH_SIZE", pat)
            w_ = per_dispatch("WRITE_SIZE", pat)
            if f_ is None or w_ is None or not factor["FETCH_SIZE"] or not factor["WRITE_SIZE"]:
                continue
            hbm = f_ * factor["FETCH_SIZE"] + w_ * factor["WRITE_SIZE"]
            a = BYTES_PER_ELEM[key] * w.N if key in BYTES_PER_ELEM else None
            if pat in ("k_deer_fused<", "k_sru_deer_fused<unsigned short"):
                # one launch per solve (all iterations)
                a = BYTES_PER_ELEM["deer_fused" if pat == "k_deer_fused<" else "sru_deer_fused"] * w.N
                rec[f"{tag}/{key}"] = {"hbm_bytes_per_launch": round(hbm), "csrc_hash": src_hash,
                                      "algorithmic_bytes": a}
            elif key in SOLVE_KEYS:
                # one launch per Newton iteration: first iteration 8 B/elem, then 12 B/elem
                n_it = len([r for r in pmc["FETCH_SIZE"] if pat in r["Kernel_Name"]])
                a = None
                hbm_solve = hbm * 5  # five iterations per solve on this workload
                rec[f"{tag}/{key}"] = {"hbm_bytes_per_launch": round(hbm_solve), "csrc_hash": src_hash,
                                      "per_iteration_bytes": round(hbm), "dispatches": n_it}
            else:
                rec[f"{tag}/{key}"] = {"hbm_bytes_per_launch": round(hbm), "csrc_hash": src_hash,
                                      "algorithmic_bytes": a}
            lines.append(f"| `{pat}` | {f_/1024:.0f} | {w_/1024:.0f} | {hbm:.4g} | "
                         f"{a if a else 'n/a'} | {hbm / a if a else float('nan'):.3f} |")
    lines += ["", f"Kernel sources hash of the profiled run: `{src_hash}` (bench.py reports "
              "`traffic` only while it matches the sources it runs)."]
    os.makedirs(os.path.dirname(COUNTERS_FILE), exist_ok=True)
    with open(COUNTERS_FILE, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    out = os.path.join(ROOT, "profiles", f"{tag}.md")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {out}")


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="scan_long",
                   choices=["scan_fwd_bwd", "scan_fused", "scan_short", "scan_long",
                            "scan_fwd_bwd_bf16", "scan_long_bf16", "sru_fwd",
                            "sru_deer", "sru_fwd_bwd", "lstm_fwd_bwd",
                            "deer", "deer_fwd_bwd", "scan_fwd_small"])
    p.add_argument("--layout", default="bdt", choices=["bdt", "tbd"])
    p.add_argument("--also", default=None,
                   help="comma-separated workloads also measured in the same run and reported "
                        "inside the line under 'also' (default: scan_fwd_bwd when the workload "
                        "is scan_long, else none; 'none' disables)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--graph", action="store_true",
                   help="also time the step captured as a HIP graph and replayed")
    p.add_argument("--no-stream-ref", action="store_true",
                   help="skip the read-2/write-1 stream reference kernel")
    p.add_argument("--crossover", action="store_true",
                   help="time the sequential and the parallel scan kernels at T = 4 .. 8192 "
                        "(2^24 elements) and print a table, instead of the bench line")
    p.add_argument("--deer-crossover", action="store_true",
                   help="time the DEER solve against the sequential loop (lrs_rnn_seq) over "
                        "channel counts and lengths and print a table, instead of the bench line")
    p.add_argument("--deer-warm", action="store_true",
                   help="time warm-started DEER solves (K_max 5 and K_max matched to the count) "
                        "against the sequential loop at the DEER workload and print a table")
    p.add_argument("--summarize", metavar="DIR",
                   help="summarise rocprofv3 CSV output under DIR into profiles/ and exit")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="minimum CPU time for the oracle baseline sample")
    return p.parse_args()


class DeviceEvent:
    """A HIP timing event recorded with a device-scope release
    (hipEventReleaseToDevice) instead of the default system-scope one, whose
    cache writeback would add several microseconds to every interval that
    ends in it.  Uses the HIP runtime the process already loaded (torch's)."""

    _hip = None
    RELEASE_TO_DEVICE = 0x40000000

    @classmethod
    def hip(cls):
        if cls._hip is None:
            cls._hip = ctypes.CDLL("libamdhip64.so.7")
        return cls._hip

    def __init__(self):
        self.h = ctypes.c_void_p()
        rc = self.hip().hipEventCreateWithFlags(ctypes.byref(self.h),
                                                ctypes.c_uint(self.RELEASE_TO_DEVICE))
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self, stream):
        rc = self.hip().hipEventRecord(self.h, ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def ms_until(self, later):
        ms = ctypes.c_float()
        rc = self.hip().hipEventElapsedTime(ctypes.byref(ms), self.h, later.h)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        if self._hip is not None and self.h:
            self._hip.hipEventDestroy(self.h)


def step_kernel_ms(torch, calls, reps):
    """Duration of every call of each entry point (lists of ms), from HIP
    events recorded on the launch stream after every call of `reps` consecutive
    steps.  A GPU-side spin issued first lets the host queue all of them
    before the device reaches the first, so host launch latency stays out of
    the measurement, and each kernel sees the same cache state as in the
    timed steps (the previous kernel of the step ran just before it)."""
    stream = torch.cuda.current_stream().cuda_stream
    ev = [DeviceEvent() for _ in range(reps * len(calls) + 1)]
    torch.cuda.synchronize()
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(5_000_000)
    ev[0].record(stream)
    i = 1
    for _ in range(reps):
        for fn in calls.values():
            fn()
            ev[i].record(stream)
            i += 1
    torch.cuda.synchronize()
    per_call = {k: [] for k in calls}
    i = 1
    for _ in range(reps):
        for k in calls:
            per_call[k].append(ev[i - 1].ms_until(ev[i]))
            i += 1
    return per_call


def cold_kernel_ms(torch, calls, reps, flush):
    """Average duration of each entry point when every call starts with cold
    caches: a 1 GiB buffer is read (summed) just before it, which evicts the
    L2s and the memory-side cache without leaving dirty lines whose write-back
    would compete with the call; the call is bracketed by two HIP events."""
    stream = torch.cuda.current_stream().cuda_stream
    out = {k: 0.0 for k in calls}
    for _ in range(reps):
        for k, fn in calls.items():
            flush.sum()
            s, e = DeviceEvent(), DeviceEvent()
            s.record(stream)
            fn()
            e.record(stream)
            torch.cuda.synchronize()
            out[k] += s.ms_until(e) / reps
    return out


def cpu_threads() -> int:
    n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        n = min(n, int(env))
    return max(1, n)


def main():
    args = parse()
    if args.summarize:
        summarize(args)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); every channel is "
              "independent, so several GPUs would each run this same per-GPU workload.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import linear_recurrence_scan_diagonal_amd as lrs
    from linear_recurrence_scan_diagonal_amd import inputs as I

    lrs.load()  # fail loudly if the HIP library is not built
    dev = torch.device("cuda:0")
    if args.crossover:
        crossover(args, np, torch, lrs, I, dev)
        return
    if args.deer_crossover:
        deer_crossover(args, np, torch, lrs, I, dev)
        return
    if args.deer_warm:
        deer_warm(args, np, torch, lrs, I, dev)
        return
    line, w = measure(args, np, torch, lrs, I, dev)
    also = args.also
    if also is None:
        also = "scan_fwd_bwd" if args.workload == "scan_long" else "none"
    extra_lines = {}
    for name in [x for x in also.split(",") if x and x != "none"]:
        torch.cuda.empty_cache()
        sub = argparse.Namespace(**vars(args))
        sub.workload, sub.layout, sub.graph, sub.no_stream_ref = name, "bdt", False, True
        sl, _ = measure(sub, np, torch, lrs, I, dev)
        extra_lines[name] = {k: sl[k] for k in ("value", "unit", "ms_per_step", "config",
                                                "roofline", "per_kernel_ms", "per_kernel_stats_ms", "step_hbm_frac",
                                                "cold") if k in sl}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args, np, I)
    line["cpu_baseline"] = cpu
    if extra_lines:
        line["also"] = extra_lines
    line["csrc_hash"] = csrc_hash()
    print(json.dumps(line), flush=True)


def measure(args, np, torch, lrs, I, dev):
    """Time one workload (args.workload, args.layout): returns the bench line
    (without the CPU baseline) and the workload."""
    w = I.WORKLOADS[args.workload]
    B, D, T = w.B, w.D, w.T
    N = w.N
    extra = {}

    def to_dev(x_ct, layout):
        if layout == "bdt":
            return torch.from_numpy(np.ascontiguousarray(x_ct).reshape(B, D, T)).to(dev)
        return torch.from_numpy(np.ascontiguousarray(x_ct.T).reshape(T, B, D)).to(dev)

    print(f"# generating inputs for {w.name}: {w.desc}", file=sys.stderr, flush=True)
    if w.kind == "scan":
        layout = args.layout
        fwd_only = args.workload == "scan_fwd_small"
        bf16 = w.io == "bf16"
        x = (I.scan_inputs_bf16 if bf16 else I.scan_inputs)(w, with_grad=not fwd_only)
        if bf16:  # a, b, dL/dh as bf16 bit patterns (one rounding from the fp64 draw)
            def to_dev16(bits_ct, layout):
                return to_dev(bits_ct.view(np.int16), layout).view(torch.bfloat16)
            a, b = to_dev16(x["a"], layout), to_dev16(x["b"], layout)
            g = None if fwd_only else to_dev16(x["g"], layout)
        else:
            a, b = to_dev(x["a"], layout), to_dev(x["b"], layout)
            g = None if fwd_only else to_dev(x["g"], layout)
        h0 = torch.from_numpy(x["h0"].reshape(B, D)).to(dev)
        h = torch.empty_like(a)
        ga, gb = torch.empty_like(a), torch.empty_like(a)
        gh0 = torch.empty((B, D), dtype=torch.float32, device=dev)
        ws_bytes = lrs.scan_workspace_bytes(B, D, T, layout, a.dtype)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        sfx = "bf16" if bf16 else "f32"

        calls = {f"scan_fwd_{sfx}": lambda: lrs.scan_fwd(a, b, h0, layout=layout, out=h,
                                                          workspace=ws)}
        if args.workload == "scan_fused":
            calls = {"scan_fused_f32": lambda: lrs.scan_fwd_bwd(a, b, g, h0, layout=layout,
                                                                out=(h, ga, gb, gh0), workspace=ws)}
        elif not fwd_only:
            calls[f"scan_bwd_{sfx}"] = lambda: lrs.scan_bwd(a, h, g, h0, layout=layout, grad_a=ga,
                                                            grad_b=gb, grad_h0=gh0, workspace=ws)

        def step():
            for fn in calls.values():
                fn()
        kernels = list(calls)
        dtype = "bf16 I/O, f32 state" if bf16 else "f32"
        config = {"workload": w.name, "B": B, "D": D, "T": T, "layout": layout,
                  "pass": "fwd" if fwd_only else ("fwd+bwd, one call" if args.workload == "scan_fused"
                                                   else "fwd+bwd")}
    elif w.kind == "sru":
        s = I.sru_inputs(w)
        z = {k: torch.from_numpy(s[k].view(np.int16)).view(torch.bfloat16).to(dev)
             for k in ("zf", "zr", "zx")}
        bf = torch.from_numpy(s["bias_f"]).to(dev)
        br = torch.from_numpy(s["bias_r"]).to(dev)
        hs = torch.empty_like(z["zf"])
        ws = torch.empty(max(1, lrs.load().lrs_sru_workspace_bytes(T, B, D)), dtype=torch.uint8,
                         device=dev)

        if w.name == "sru_fwd":
            calls = {"sru_fwd_bf16": lambda: lrs.sru_fwd(z["zf"], z["zr"], z["zx"], bf, br, out=hs,
                                                         workspace=ws)}
        else:  # forward saving the cell states, then the backward
            gh = torch.from_numpy(I.sru_grad_inputs(w)["gh"].view(np.int16)).view(
                torch.bfloat16).to(dev)
            cs = torch.empty((T, B, D), dtype=torch.float32, device=dev)
            grads = (torch.empty_like(z["zf"]), torch.empty_like(z["zf"]), torch.empty_like(z["zf"]),
                     torch.empty(D, dtype=torch.float32, device=dev),
                     torch.empty(D, dtype=torch.float32, device=dev),
                     torch.empty((B, D), dtype=torch.float32, device=dev))
            wsb = torch.empty(max(1, lrs.load().lrs_sru_bwd_workspace_bytes(T, B, D)),
                              dtype=torch.uint8, device=dev)
            calls = {"sru_fwd_save_bf16": lambda: lrs.sru_fwd(z["zf"], z["zr"], z["zx"], bf, br,
                                                              out=hs, workspace=ws, c_states=cs),
                     "sru_bwd_bf16": lambda: lrs.sru_bwd(z["zf"], z["zr"], z["zx"], bf, br, cs, gh,
                                                         out=grads, workspace=wsb)}

        def step():
            for fn in calls.values():
                fn()
        kernels = list(calls)
        dtype = "bf16 I/O, f32 state"
        config = {"workload": w.name, "B": B, "D": D, "T": T, "layout": "tbd",
                  "pass": "fwd+bwd" if w.name == "sru_fwd_bwd" else "fwd"}
    elif w.kind == "lstm":  # forward saving the cell states, then the backward
        s = I.lstm_inputs(w)
        s["gh"] = I.sru_grad_inputs(w)["gh"]
        z = {k: torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).to(dev)
             for k, v in s.items()}
        hs = torch.empty_like(z["zf"])
        cs = torch.empty((T, B, D), dtype=torch.float32, device=dev)
        grads = tuple(torch.empty_like(z["zf"]) for _ in range(4)) + (
            torch.empty((B, D), dtype=torch.float32, device=dev),)
        ws = torch.empty(max(1, lrs.load().lrs_lstm_workspace_bytes(T, B, D)), dtype=torch.uint8,
                         device=dev)
        zg = (z["zf"], z["zi"], z["zc"], z["zo"])
        calls = {"lstm_fwd_save_bf16": lambda: lrs.lstm_fwd(*zg, out=hs, workspace=ws,
                                                            c_states=cs),
                 "lstm_bwd_bf16": lambda: lrs.lstm_bwd(*zg, cs, z["gh"], out=grads,
                                                       workspace=ws)}

        def step():
            for fn in calls.values():
                fn()
        kernels = list(calls)
        dtype = "bf16 I/O, f32 state"
        config = {"workload": w.name, "B": B, "D": D, "T": T, "layout": "tbd",
                  "pass": "fwd+bwd"}
    elif w.kind == "sru_deer":
        s = I.sru_inputs(w)
        z = {k: torch.from_numpy(s[k].view(np.int16)).view(torch.bfloat16).to(dev)
             for k in ("zf", "zr", "zx")}
        pr = {k: torch.from_numpy(v).to(dev) for k, v in
              (("bf", s["bias_f"]), ("br", s["bias_r"]), ("vf", I.sru_vf(w)))}
        hs = torch.empty_like(z["zf"])
        cs = torch.empty((T, B, D), dtype=torch.float32, device=dev)
        ws = torch.empty(lrs.load().lrs_sru_deer_workspace_bytes(T, B, D, 5), dtype=torch.uint8,
                         device=dev)

        def sru_solve():
            lrs.sru_deer_fwd(z["zf"], z["zr"], z["zx"], pr["bf"], pr["br"], pr["vf"], eps=1e-5,
                             k_max=5, out=hs, c_states=cs, workspace=ws, sync=False)
        calls = {"sru_deer_bf16": sru_solve}

        def step():
            sru_solve()
        kernels = list(calls)
        dtype = "bf16 I/O, f32 state"
        config = {"workload": w.name, "B": B, "D": D, "T": T, "layout": "tbd", "eps": 1e-5,
                  "k_max": 5, "pass": "solve"}
    else:  # deer
        x = I.deer_inputs(w)
        wd = torch.from_numpy(x["w"]).to(dev)
        u = torch.from_numpy(x["u"].reshape(B, D, T)).to(dev)
        h0 = torch.from_numpy(x["h0"].reshape(B, D)).to(dev)
        hd = torch.empty_like(u)
        ws = torch.empty(lrs.load().lrs_deer_workspace_bytes(B, D, T, 5), dtype=torch.uint8,
                         device=dev)

        # the timed solve is the asynchronous form (no host outputs): the
        # iteration record is read once afterwards with deer_stats
        def solve_async():
            lrs.deer_solve(wd, u, h0, None, eps=1e-5, k_max=5, out=hd, workspace=ws, sync=False)

        def solve_sync():
            return lrs.deer_solve(wd, u, h0, None, eps=1e-5, k_max=5, out=hd, workspace=ws)
        calls = {"deer_solve": solve_async}
        if w.name == "deer_fwd_bwd":  # then the backward at the solution
            gd = torch.from_numpy(I.series(w.seed, "g", w.dists["g"], np.arange(w.C), T,
                                           np.float32).reshape(B, D, T)).to(dev)
            dgrads = (torch.empty_like(u), torch.empty(D, dtype=torch.float32, device=dev),
                      torch.empty((B, D), dtype=torch.float32, device=dev))
            wsd = torch.empty(max(1, lrs.load().lrs_deer_bwd_workspace_bytes(B, D, T)),
                              dtype=torch.uint8, device=dev)
            calls["deer_bwd_f32"] = lambda: lrs.deer_bwd(wd, hd, gd, h0, out=dgrads, workspace=wsd)

        def step():
            for fn in calls.values():
                fn()
        kernels = list(calls)
        dtype = "f32"
        config = {"workload": w.name, "B": B, "D": D, "T": T, "layout": "bdt", "eps": 1e-5,
                  "k_max": 5, "pass": "solve+bwd" if w.name == "deer_fwd_bwd" else "solve"}

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    def timed(fn, steps):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        t0.record()
        for _ in range(steps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps, time.perf_counter() - w0

    # (1) eager steps, HIP events only at the two ends of the timed region
    ms_per_step, wall = timed(step, args.steps)
    extra["timing"] = "eager launches, events at both ends"
    # (2) the same step captured once as a HIP graph and replayed (reported
    #     beside the eager figure); DEER is captured in its asynchronous form
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(2):
            graph.replay()
        extra["ms_per_step_graph"] = round(timed(graph.replay, args.steps)[0], 5)
    # (3) per-kernel launch durations for the roofline: `steps` more steps
    #     with a HIP event after every entry point, on its launch stream
    per_call = step_kernel_ms(torch, calls, args.steps)
    per_kernel = {k: sum(v) / len(v) for k, v in per_call.items()}
    extra["per_kernel_stats_ms"] = {k: {"median": round(float(np.median(v)), 5),
                                        "min": round(min(v), 5), "max": round(max(v), 5),
                                        "calls": len(v)} for k, v in per_call.items()}
    extra["per_kernel_timing"] = ("HIP event (device-scope release) after every call of "
                                  "queued steps")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    if w.kind == "sru_deer":
        info = lrs.deer_stats(ws, 5)
    if w.kind == "deer":
        # the synchronous form reads the record back after every solve
        extra["ms_per_step_sync"] = round(timed(solve_sync, args.steps)[0], 5)
        info = lrs.deer_stats(ws, 5)
        # the same recurrence evaluated step after step, one lane per channel
        # (T dependent steps whatever the channel count): the sequential
        # reference the solve replaces, with the largest difference between
        # the two results relative to the largest |h|
        h_seq = torch.empty_like(u)
        seq_ms = timed(lambda: lrs.rnn_seq(wd, u, h0, out=h_seq), args.steps)[0]
        diff = ((h_seq - hd).abs().max() / hd.abs().max().clamp_min(1e-30)).item()
        extra["seq_ref"] = {"kernel": "rnn_seq, one lane per channel, T dependent steps",
                            "ms": round(seq_ms, 5), "elements_per_s": N / (seq_ms / 1e3),
                            "solve_speedup": round(seq_ms / ms_per_step, 3),
                            "max_rel_diff_vs_solve": diff}
        del h_seq
    value = N / (ms_per_step / 1e3)
    # (4) the same entry points with cold caches before every call
    flush = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
    cold = cold_kernel_ms(torch, calls, max(3, args.steps // 2), flush)
    del flush

    if w.kind == "scan":
        bytes_step = sum(BYTES_PER_ELEM[k] * N for k in kernels)
        dom = max(kernels, key=lambda k: per_kernel[k])
        dom_bytes = BYTES_PER_ELEM[dom] * N
        dom_ms = per_kernel[dom]
    elif w.kind in ("sru", "lstm"):
        bytes_step = sum(BYTES_PER_ELEM[k] * N for k in kernels)
        dom = max(kernels, key=lambda k: per_kernel[k])
        dom_bytes, dom_ms = BYTES_PER_ELEM[dom] * N, per_kernel[dom]
    elif w.kind == "sru_deer":
        iters = info["iters"]
        if sru_deer_fused_applies(w.B * w.D, 5):
            # one pass over all K_max iterations (a second when the stop rule
            # fired earlier), then the output kernel
            bytes_step = (BYTES_PER_ELEM["sru_deer_fused"] * (1 if iters == 5 else 2) +
                          BYTES_PER_ELEM["sru_deer_out"]) * N
        else:
            bytes_step = (BYTES_PER_ELEM["sru_deer_iter_first"] + (iters - 1) *
                          BYTES_PER_ELEM["sru_deer_iter"] + BYTES_PER_ELEM["sru_deer_out"]) * N
        dom, dom_bytes, dom_ms = "sru_deer_bf16", bytes_step, per_kernel["sru_deer_bf16"]
        extra["deer_iters"] = iters
        extra["deer_deltas"] = info["deltas"]
    else:
        iters = info["iters"]
        if deer_fused_applies(w.T, 5, w.C, cus):
            # one pass over all K_max iterations, and a second one when the stop
            # rule fired earlier
            solve_bytes = BYTES_PER_ELEM["deer_fused"] * N * (1 if iters == 5 else 2)
        else:
            solve_bytes = (BYTES_PER_ELEM["deer_iter_first"] + (iters - 1) *
                           BYTES_PER_ELEM["deer_iter"]) * N
        bytes_step = solve_bytes + sum(BYTES_PER_ELEM[k] * N for k in kernels if k != "deer_solve")
        dom, dom_bytes, dom_ms = "deer_solve", solve_bytes, per_kernel["deer_solve"]
        extra["deer_iters"] = iters
        extra["deer_deltas"] = info["deltas"]
    achieved = dom_bytes / (dom_ms / 1e3) / 1e9
    traffic = measured_traffic(w.name if args.layout == "bdt" else f"{w.name}_{args.layout}", dom)
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic, "algorithmic_bytes": dom_bytes,
                "avg_launch_ms": round(dom_ms, 5)}
    if w.kind == "deer" and deer_fused_applies(w.T, 5, w.C, cus):
        # vector-ALU bound: the method's flops over the iterations it performed
        flops = DEER_FLOPS_PER_ELEM_ITER * N * iters
        tflops = flops / (dom_ms / 1e3) / 1e12
        roofline = {"bound": "alu", "kernel": dom, "achieved": round(tflops, 2),
                    "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tflops / FP32_VECTOR_PEAK_TFLOPS, 4), "traffic": traffic,
                    "algorithmic_flops": flops, "algorithmic_bytes": dom_bytes,
                    "hbm_frac": round(achieved / HBM_PEAK_GBS, 4),
                    "avg_launch_ms": round(dom_ms, 5)}
    extra["per_kernel_ms"] = {k: round(v, 5) for k, v in per_kernel.items()}
    extra["step_hbm_frac"] = round(bytes_step / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4)
    cold_ms = sum(cold.values())
    extra["cold"] = {"per_kernel_ms": {k: round(v, 5) for k, v in cold.items()},
                     "ms_per_step": round(cold_ms, 5),
                     "step_hbm_frac": round(bytes_step / (cold_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                     "how": "1 GiB read before every call (evicts L2 and the memory-side "
                            "cache), HIP events around the call"}
    extra["wall_s"] = round(wall, 3)

    if not args.no_stream_ref:
        extra["stream_ref"] = stream_reference(torch, dev)

    line = {"metric": METRIC, "value": value, "unit": "elements/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
            "data": "synthetic", "config": config, "roofline": roofline, "cpu_baseline": None,
            **extra}
    return line, w


def crossover(args, np, torch, lrs, I, dev):
    """Kernel families for short channels: sequential (one lane per channel),
    packed (whole channels per workgroup) and one channel per workgroup, on
    the B=8 D=512 T=4096 workload's 2^24 elements of a, b, dL/dh regrouped as
    [1, 2^24/T, T] for T = 4 .. 8192, each forced through the plan options
    (serial_fwd_max_t, serial_bwd_max_t, packed_max_t), timed with HIP events
    over --steps calls."""
    w = I.WORKLOADS["scan_fwd_bwd"]
    x = I.scan_inputs(w)
    N = w.N
    flat = {k: torch.from_numpy(np.ascontiguousarray(x[k]).reshape(-1)).to(dev)
            for k in ("a", "b", "g")}
    h = torch.empty(N, device=dev)
    ga, gb = torch.empty(N, device=dev), torch.empty(N, device=dev)
    ws = torch.empty(max(1, lrs.scan_workspace_bytes(1, N // 4, 4)), dtype=torch.uint8,
                     device=dev)

    def timed(fn):
        for _ in range(3):
            fn()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record()
        for _ in range(args.steps):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) * 1e3 / args.steps

    big = 1 << 40
    modes = (("sequential", (big, big, 0)), ("packed", (0, 0, big)),
             ("one channel per workgroup", (0, 0, 0)))
    rows = []
    T = 4
    while T <= 8192:
        D = N // T
        a, b, g = (flat[k].view(1, D, T) for k in ("a", "b", "g"))
        hv, gav, gbv = h.view(1, D, T), ga.view(1, D, T), gb.view(1, D, T)
        res = {}
        for mode, (sf, sb, pk) in modes:
            if mode == "packed" and T > 2048:
                res[mode] = None  # no channel fits a packed workgroup
                continue
            opts = {"serial_fwd_max_t": sf, "serial_bwd_max_t": sb, "packed_max_t": pk}
            res[mode] = (timed(lambda: lrs.scan_fwd(a, b, None, out=hv, workspace=ws,
                                                    options=opts)),
                         timed(lambda: lrs.scan_bwd(a, hv, g, None, need_grad_h0=False,
                                                    grad_a=gav, grad_b=gbv, workspace=ws,
                                                    options=opts)))
        rows.append((T, D, res))
        T *= 2
    pct = lambda us, bpe: 100.0 * bpe * N / (us * 1e-6) / 1e9 / HBM_PEAK_GBS
    cell = lambda v, bpe: "n/a" if v is None else f"{v:.1f} ({pct(v, bpe):.0f}%)"
    print(f"# crossover, {N} elements (fwd 12 B, bwd 20 B per element), us and % of 8 TB/s")
    print("| T | channels | " + " | ".join(f"{m} fwd | {m} bwd" for m, _ in modes) + " |")
    print("|---|---|" + "---|---|" * len(modes))
    for T, D, res in rows:
        cells = []
        for m, _ in modes:
            v = res[m]
            cells += [cell(None if v is None else v[0], 12), cell(None if v is None else v[1], 20)]
        print(f"| {T} | {D} | " + " | ".join(cells) + " |", flush=True)


def deer_crossover(args, np, torch, lrs, I, dev):
    """The DEER solve (eps 1e-5, K_max 5, asynchronous form) under the default
    plan, with the fused pass forced (deer_fuse = 1) and with one launch per
    iteration (deer_fuse = 0), against the sequential loop (lrs_rnn_seq, one
    lane per channel), on the DEER workload's distributions (w ~ U(-0.9, 0.9)
    per feature, u ~ N(0, 1), h0 = 0) drawn on the device, over channel counts
    and lengths.  HIP events over --steps calls each."""
    dw = I.WORKLOADS["deer"]
    shapes = ([(1, c, 8192) for c in (64, 512, 2048)] +
              [(dw.B, dw.D, T) for T in (1024, 2048, 4096, 8192, 16384, 32768)] +
              [(1, c, 32768) for c in (256, 512, 1024, 2048)] + [(64, 1024, 8192)])

    def timed(fn):
        for _ in range(3):
            fn()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record()
        for _ in range(args.steps):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) * 1e3 / args.steps

    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    print(f"| channels | T | DEER default us (iterations) | fused | one launch per iteration | "
          f"sequential us | sequential / DEER default |")
    print("|---|---|---|---|---|---|---|")
    for B, D, T in shapes:
        u = I.device_draw(dw.seed + T, dw.dists["u"], (B, D, T), dev)
        wd = I.device_draw(dw.seed + 1, dw.dists["w"], (D,), dev)
        h, hs = torch.empty_like(u), torch.empty_like(u)
        ws = torch.empty(max(1, lrs.load().lrs_deer_workspace_bytes(B, D, T, 5)),
                         dtype=torch.uint8, device=dev)
        t = {}
        for mode, opts in (("default", None), ("fused", {"deer_fuse": 1}),
                           ("per-iteration", {"deer_fuse": 0})):
            t[mode] = timed(lambda: lrs.deer_solve(wd, u, None, None, eps=1e-5, k_max=5, out=h,
                                                   workspace=ws, sync=False, options=opts))
            if mode == "default":
                iters = lrs.deer_stats(ws, 5)["iters"]
        t_seq = timed(lambda: lrs.rnn_seq(wd, u, None, out=hs))
        plan = "fused" if deer_fused_applies(T, 5, B * D, cus) else "per-iteration"
        print(f"| {B * D} | {T} | {t['default']:.1f} ({iters}, {plan}) | {t['fused']:.1f} | "
              f"{t['per-iteration']:.1f} | {t_seq:.1f} | {t_seq / t['default']:.2f} |",
              flush=True)
        del u, h, hs, ws


def deer_warm(args, np, torch, lrs, I, dev):
    """DEER solves at the DEER workload's shape and distributions (drawn on the
    device), cold (h_init = 0) and warm-started from the sequential solution of
    the inputs perturbed by N(0, sigma^2), with K_max 5 and with K_max set to
    the count the stop rule reaches, against the sequential loop; HIP events
    over --steps calls each."""
    dw = I.WORKLOADS["deer"]
    B, D, T = dw.B, dw.D, dw.T
    u = I.device_draw(dw.seed + T, dw.dists["u"], (B, D, T), dev)
    wd = I.device_draw(dw.seed + 1, dw.dists["w"], (D,), dev)
    h = torch.empty_like(u)
    ws = torch.empty(lrs.load().lrs_deer_workspace_bytes(B, D, T, 5), dtype=torch.uint8,
                     device=dev)

    def timed(fn):
        for _ in range(3):
            fn()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record()
        for _ in range(args.steps):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) * 1e3 / args.steps

    t_seq = timed(lambda: lrs.rnn_seq(wd, u, None, out=h))
    print(f"| start | K_max | iterations | solve us | sequential {t_seq:.1f} us / solve |")
    print("|---|---|---|---|---|")
    for sigma, k_max in ((0.0, 5), (0.01, 5), (0.01, 3), (0.01, 2), (0.05, 5), (0.05, 4)):
        h_init = None
        if sigma > 0:
            pert = I.device_draw(dw.seed + 2, ("normal", 0.0, 1.0), (B, D, T), dev)
            h_init = lrs.rnn_seq(wd, u + sigma * pert, None)
            del pert
        t = timed(lambda: lrs.deer_solve(wd, u, None, h_init, eps=1e-5, k_max=k_max, out=h,
                                         workspace=ws, sync=False))
        st = lrs.deer_stats(ws, k_max)
        start = "cold" if sigma == 0 else f"warm, inputs perturbed by N(0, {sigma}^2)"
        print(f"| {start} | {k_max} | {st['iters']} ({'converged' if st['converged'] else 'K_max'}) "
              f"| {t:.1f} | {t_seq / t:.2f} |", flush=True)


STREAM_REF_ELEMS = 1 << 26  # 256 MiB per fp32 operand


def stream_reference(torch, dev, reps: int = 10):
    """Practical HBM ceiling on this device: torch's elementwise add z = x + y
    over three 256 MiB fp32 arrays (reads 512 MiB, writes 256 MiB per call,
    far beyond the caches).  Its per-dispatch counters also calibrate the
    FETCH_SIZE / WRITE_SIZE readings of the scan kernels."""
    x = torch.ones(STREAM_REF_ELEMS, device=dev)
    y = torch.ones(STREAM_REF_ELEMS, device=dev)
    z = torch.empty(STREAM_REF_ELEMS, device=dev)
    for _ in range(3):
        torch.add(x, y, out=z)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        torch.add(x, y, out=z)
    e.record()
    torch.cuda.synchronize()
    sec = s.elapsed_time(e) / 1e3 / reps
    gbs = 3 * 4 * STREAM_REF_ELEMS / sec / 1e9
    return {"kernel": "torch add, read 2 x 256 MiB + write 256 MiB", "GB/s": round(gbs, 1),
            "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}


def cpu_baseline(w, args, np, I):
    """Time the fp64 oracle on the host cores over a bounded sample: whole
    passes over the workload's channels (or a channel subset for the largest
    workloads), repeated until at least --cpu-seconds of CPU time."""
    import oracle
    threads = cpu_threads()
    C, T = w.C, w.T
    if w.kind == "scan":
        nch = C if C * T <= (1 << 26) else max(1, (1 << 26) // T)
        ch = np.arange(nch)
        if w.io == "bf16":  # the oracle on the bf16 values the GPU receives
            x = I.scan_inputs_bf16(w, channels=ch, with_grad=w.name != "scan_fwd_small")
            x = {k: (I.bf16_bits_to_f64(v) if k != "h0" else v) for k, v in x.items()}
        else:
            x = I.scan_inputs(w, channels=ch, with_grad=w.name != "scan_fwd_small")
        a, b = x["a"].astype(np.float64), x["b"].astype(np.float64)
        h0 = x["h0"].astype(np.float64)
        g = x["g"].astype(np.float64) if "g" in x else None

        def once(nt=threads):
            h = oracle.scan_fwd(a, b, h0, nthreads=nt)
            if g is not None:
                oracle.scan_bwd(a, h, h0, g, nthreads=nt)
        sample = f"{nch} of {C} channels x T={T}, fwd{'+bwd' if g is not None else ''}"
        n_el = nch * T
    elif w.kind == "sru":
        sub = I.scaled(w, B=1, D=min(w.D, 1024))
        s = I.sru_inputs(sub)
        z = [I.bf16_bits_to_f64(s[k]) for k in ("zf", "zr", "zx")]

        with_bwd = w.name == "sru_fwd_bwd"
        gh64 = I.bf16_bits_to_f64(I.sru_grad_inputs(sub)["gh"]) if with_bwd else None

        def once(nt=threads):
            oracle.sru_fwd(*z, s["bias_f"], s["bias_r"], nthreads=nt)
            if with_bwd:
                oracle.sru_bwd(*z, s["bias_f"], s["bias_r"], gh64, nthreads=nt)
        sample = (f"B=1 of {w.B}, D={sub.D}, T={T} (same recipe), "
                  f"fwd{'+bwd' if with_bwd else ''}")
        n_el = sub.N
    elif w.kind == "sru_deer":
        sub = I.scaled(w, B=1, D=min(w.D, 1024))
        s = I.sru_inputs(sub)
        z = [I.bf16_bits_to_f64(s[k]) for k in ("zf", "zr", "zx")]
        vf = I.sru_vf(sub)

        def once(nt=threads):
            oracle.sru_deer(*z, s["bias_f"], s["bias_r"], vf, eps=1e-5, k_max=5, nthreads=nt)
        sample = f"B=1 of {w.B}, D={sub.D}, T={T} (same recipe), eps=1e-5, K_max=5"
        n_el = sub.N
    elif w.kind == "lstm":
        sub = I.scaled(w, B=1, D=min(w.D, 1024))
        s = I.lstm_inputs(sub)
        z = [I.bf16_bits_to_f64(s[k]) for k in ("zf", "zi", "zc", "zo")]
        gh64 = I.bf16_bits_to_f64(I.sru_grad_inputs(sub)["gh"])

        def once(nt=threads):
            oracle.lstm_fwd(*z, nthreads=nt)
            oracle.lstm_bwd(*z, gh64, nthreads=nt)
        sample = f"B=1 of {w.B}, D={sub.D}, T={T} (same recipe), fwd+bwd"
        n_el = sub.N
    else:
        sub = I.scaled(w, B=1)
        x = I.deer_inputs(sub)
        u = x["u"].reshape(1, sub.D, T).astype(np.float64)

        with_bwd = w.name == "deer_fwd_bwd"
        g64 = (I.series(w.seed, "g", w.dists["g"], np.arange(sub.C), T).reshape(1, sub.D, T)
               if with_bwd else None)

        def once(nt=threads):
            hs, _, _ = oracle.deer(x["w"], u, None, eps=1e-5, k_max=5, nthreads=nt)
            if with_bwd:
                oracle.deer_bwd(x["w"], hs, g64, nthreads=nt)
        sample = (f"B=1 of {w.B}, D={sub.D}, T={T}, eps=1e-5, K_max=5"
                  f"{', solve+bwd' if with_bwd else ''}")
        n_el = sub.N
    def time_it(nt):
        reps, t_total = 0, 0.0
        while t_total < args.cpu_seconds and reps < 10000:
            t0 = time.perf_counter()
            once(nt)
            t_total += time.perf_counter() - t0
            reps += 1
        return reps, t_total

    reps, t_total = time_it(threads)
    reps1, t1 = time_it(1)
    return {"value": n_el * reps / t_total, "unit": "elements/s", "cores": threads,
            "kind": "oracle", "sample": f"{sample}; {reps} repetitions, {t_total:.1f} s",
            "single_thread": {"value": n_el * reps1 / t1, "unit": "elements/s", "cores": 1,
                              "sample": f"{sample}; {reps1} repetitions, {t1:.1f} s"},
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}


def cpu_model() -> str:
    """The host CPU's model name (first processor entry of /proc/cpuinfo), with
    its family / model / stepping numbers, which identify the core generation
    where a virtual machine reports only a generic name."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if not line.strip():
                    if fields:
                        break  # end of the first processor entry
                    continue
                key, _, val = line.partition(":")
                fields.setdefault(key.strip().lower(), val.strip())
    except OSError:
        pass
    name = fields.get("model name", "unknown")
    ids = [f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping") if k in fields]
    return f"{name} ({', '.join(ids)})" if ids else name


if __name__ == "__main__":
    main()
