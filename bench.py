"""Throughput of the batched fp32 FFT on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload w2] [--configs all|none]
    python bench.py --summarize-trace KERNEL_TRACE.csv [--windows WINDOWS.jsonl]

One step is one pass of the whole hot path over one batch: for the default
workload (w2: 16384 rows of N = 4096 complex64, U[-1,1]) a forward transform
followed by the inverse of its output, two kernel launches.  Inputs are
resident in HBM before timing starts.  Each workload first runs for 200 ms
(settle, untimed, reported), then W warm-up steps, then the K timed steps.
Prints ONE JSON line.

value     = 5 N log2(N) * rows * directions / time  (GFLOP/s, the pages'
            flop convention)
roofline  = algorithmic HBM bytes of one launch (read + write of every
            element once) / the average launch duration, timed with HIP events
            on the stream the kernels run on, against the 8 TB/s HBM peak
cpu_baseline = the f64 oracle (untuned reference) on a bounded sample of the
            same workload on the host cores
configs   = (default run) every configuration of the metric measured in the
            same run: c1 1024 x 8, c2 4096 x 16384 forward + inverse (the
            headline above), c3 2^22 x 32 (four-step), c4 real rows 1024 x 2048
            (C2R then R2C, mmax 682), c5 8192^2 2D with the fused shift.  Each
            with its time per exec over the timed region, GFLOP/s, algorithmic
            GB/s and fraction of HBM peak, the median and geometric mean of
            per-exec event timings, 100 back-to-back steps for c1 and c4, the
            relative L2 error against the oracle over the whole output, and
            the oracle's own time on that reference (the CPU baseline)
--summarize-trace: per-kernel durations of a rocprofv3 kernel trace of a
            bench run; with --windows (the --timed-windows file the traced run
            wrote: host CLOCK_MONOTONIC windows around its timed regions, the
            clock of the trace's timestamps) only the timed launches
"""
import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "batched C2C fp32 FFT GFLOP/s (5N log2N) + achieved HBM GB/s vs peak"
HBM_PEAK_GBPS = 8000.0
FP32_MFMA_PEAK_TFLOPS = 157.3   # dense fp32 matrix-core peak of the MI355X
PROFILES = os.path.join(ROOT, "profiles")


_TOKENS = re.compile(r'"(?:\\.|[^"\\\n])*"|//[^\n]*|/\*.*?\*/', re.S)


def code_only(text):
    """Source text without comments and blank lines (string literals kept)."""
    text = _TOKENS.sub(lambda m: m.group(0) if m.group(0).startswith('"') else " ", text)
    return "\n".join(l.rstrip() for l in text.splitlines() if l.strip())


def kernel_source_hash():
    """Hash of the kernel sources, comments left out; stored HBM-traffic
    counters are used only while it matches."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fourier_transform_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hpp", ".hip")):
            h.update(f.encode() + b"\0")
            h.update(code_only(open(os.path.join(csrc, f), encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def stored_traffic(kernel_key):
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except ValueError:
        return None
    e = d.get(kernel_key)
    if not e or e.get("source_hash") != kernel_source_hash():
        return None
    return e.get("bytes_per_launch")


def workload_spec(name):
    from fourier_transform_amd import workloads as W
    if name == "w1":
        return dict(kind="c2c", n=W.W1["n"], batch=W.W1["batch"], dirs=(-1,), gen=W.workload1,
                    passes=1, label="1D C2C fp32 forward N=1024 batch=8")
    if name == "w2":
        return dict(kind="c2c", n=W.W2["n"], batch=W.W2["batch"], dirs=(-1, 1), gen=W.workload2,
                    passes=1, label="1D C2C fp32 forward+inverse N=4096 batch=16384")
    if name == "w3":
        return dict(kind="c2c", n=W.W3["n"], batch=W.W3["batch"], dirs=(-1,), gen=W.workload3,
                    passes=2, label="1D C2C fp32 forward N=2^22 batch=32 (four-step)")
    if name == "w4":
        return dict(kind="real", n=W.W4["nphi"], batch=W.W4["nlat"], mmax=W.W4["mmax"], dirs=(1, -1),
                    gen=W.workload4_spectrum, passes=1,
                    label="real rows nlat=1024 x nphi=2048, C2R synthesis then R2C analysis, "
                          "mmax=682, m-major spectrum")
    if name == "w5":
        return dict(kind="2d", n=W.W5["ny"] * W.W5["nx"], ny=W.W5["ny"], nx=W.W5["nx"], batch=1,
                    dirs=(-1,), gen=W.workload5, passes=2,
                    label="2D C2C fp32 forward 8192x8192 with fused chessboard shift")
    if name == "w6":
        return dict(kind="c2c", n=W.W6["n"], batch=W.W6["batch"], dirs=(-1, 1), gen=W.workload6,
                    passes=1, label="1D C2C fp32 forward+inverse N=1000 batch=65536 "
                                    "(length not a power of two)")
    raise SystemExit(f"unknown workload {name}")


def any_length_spec(n):
    """Workload 6 at another length: about the same 512 MiB, rows of n values."""
    from fourier_transform_amd import workloads as W
    batch = max(1, (1000 * 65536) // n)
    return dict(kind="c2c", n=n, batch=batch, dirs=(-1, 1),
                gen=lambda: W.workload6(n=n, batch=batch), passes=1,
                label=f"1D C2C fp32 forward+inverse N={n} batch={batch} (length not a power of two)")


def cpu_baseline(spec, x_host, reps=3, direct=False):
    """Time the f64 oracle (as it stands, untuned) on the host cores.

    The sample is the whole workload when it is small enough, else its first
    rows up to 2^27 points (a few seconds of work at most); the reported time
    is the median of `reps` runs and excludes the fp32 -> f64 widening.
    """
    import numpy as np
    import oracle
    n = spec["n"]
    one_thread = None
    if spec["kind"] == "real" and direct:
        rows = min(spec["batch"], 64)           # the direct sums: O(n mmax) per row
        xs = np.ascontiguousarray(x_host.T[:rows]).astype(np.complex128)

        def run():
            oracle.dft_analys_direct(oracle.dft_synth_direct(xs, n, spec["mmax"]), spec["mmax"])
        flops = 2.5 * n * math.log2(n) * rows * 2
        desc = f"{rows} of {spec['batch']} rows, direct synthesis then direct analysis"
    elif spec["kind"] == "real":
        rows = spec["batch"]
        xs = np.ascontiguousarray(x_host.T).astype(np.complex128)   # [rows][mmax+1]

        def run():
            oracle.r2c(oracle.c2r(xs, n, spec["mmax"]), spec["mmax"])
        flops = 2.5 * n * math.log2(n) * rows * 2
        desc = f"all {rows} rows, C2R then R2C"
    elif spec["kind"] == "2d":
        xs = x_host.astype(np.complex128)

        def run():
            for s in spec["dirs"]:
                oracle.c2c_2d(xs, s)
        flops = 5.0 * n * math.log2(n) * len(spec["dirs"])
        desc = f"whole {spec['ny']}x{spec['nx']} image, {len(spec['dirs'])} direction(s)"
    else:
        pow2 = n & (n - 1) == 0
        # the radix-2 oracle for powers of two, else the definition (O(n^2)
        # per row, so a smaller sample)
        rows = max(1, min(spec["batch"], (1 << 27) // n if pow2 else (1 << 25) // (n * n) + 64))
        xs = x_host[:rows].astype(np.complex128)

        def run():
            for s in spec["dirs"]:
                oracle.c2c(xs, s) if pow2 else oracle.dft(xs, s)
        flops = 5.0 * n * math.log2(n) * rows * len(spec["dirs"])
        desc = f"{rows} of {spec['batch']} rows, {len(spec['dirs'])} direction(s)"
        if pow2:
            # the same transform on one thread, on 1/16 of the sample: a per-core figure
            rows1 = max(1, rows // 16)
            x1 = xs[:rows1]
            t0 = time.perf_counter()
            for s in spec["dirs"]:
                oracle.c2c(x1, s, nthreads=1)
            dt1 = time.perf_counter() - t0
            one_thread = {"value": round(5.0 * n * math.log2(n) * rows1 * len(spec["dirs"]) / dt1 / 1e9, 3),
                          "sample": f"{rows1} rows, {len(spec['dirs'])} direction(s), one run"}
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        run()
        times.append(time.perf_counter() - t0)
    dt = sorted(times)[len(times) // 2]
    out = {"value": round(flops / dt / 1e9, 3), "unit": "GFLOP/s", "cores": oracle.threads(0),
           "kind": "oracle", "sample": desc + f", median of {reps} runs, {dt:.3f} s each"}
    if one_thread is not None:
        out["one_thread"] = one_thread
    return out


# configurations of the metric (c1..c5) and the workloads that implement them
CONFIGS = (("c1", "w1"), ("c2", "w2"), ("c3", "w3"), ("c4", "w4"), ("c5", "w5"))
BAR = 0.60              # fraction of HBM peak the large batched C2C and 2D configs must sustain
BAR_CONFIGS = ("c2", "c3", "c5")
BACK_TO_BACK = 100      # c1 and c4 (launch-bound) are also timed as this many back-to-back steps
TRAFFIC_KEY = {"w1": "c2c_rows_1024", "w2": "c2c_rows_4096", "w3": "fourstep_2^22", "w4": "real_2048",
               "w5": "2d_8192x8192"}


def cpu_model():
    """The host CPU's model name (first processor in /proc/cpuinfo)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def make_plans(F, spec, direct=False, real_pairs=False):
    n, batch = spec["n"], spec["batch"]
    plans = []
    for s in spec["dirs"]:
        if spec["kind"] == "real":
            if direct:
                kind = F.FFT_C2R_DIRECT if s > 0 else F.FFT_R2C_DIRECT
            else:
                kind = F.FFT_C2R if s > 0 else F.FFT_R2C
            p = F.fft_plan_create(n, batch, kind, s)
            F.fft_plan_set(p, F.FFT_OPT_MMAX, spec["mmax"])
            F.fft_plan_set(p, F.FFT_OPT_SPEC_LAYOUT, 1)
            if real_pairs:
                F.fft_plan_set(p, F.FFT_OPT_REAL_PAIRS, 1)
        elif spec["kind"] == "2d":
            p = F.fft_plan_create_2d(spec["ny"], spec["nx"], batch, F.FFT_C2C, s)
            F.fft_plan_set(p, F.FFT_OPT_SHIFT, 1)
        else:
            p = F.fft_plan_create(n, batch, F.FFT_C2C, s)
        plans.append(p)
    return plans


SETTLE_MS = 200.0       # the workload runs this long before its warm-up steps (see time_workload)


class _Windows:
    """Host-clock windows (CLOCK_MONOTONIC, ns: the clock of rocprofv3's
    kernel timestamps) around each timed region, appended to a JSON-lines
    file when --timed-windows is given.  The device is idle when a window
    opens and has finished when it closes, so the launches whose start lies
    inside it are exactly the timed ones (--summarize-trace --windows)."""

    def __init__(self):
        self.path = None
        self.label = ""
        self.t0 = None

    def open(self):
        self.t0 = time.clock_gettime_ns(time.CLOCK_MONOTONIC)

    def close(self):
        t1 = time.clock_gettime_ns(time.CLOCK_MONOTONIC)
        if self.path:
            os.makedirs(os.path.dirname(os.path.abspath(self.path)), exist_ok=True)
            with open(self.path, "a") as f:
                f.write(json.dumps({"label": self.label, "t0_ns": self.t0, "t1_ns": t1}) + "\n")


WINDOWS = _Windows()


def time_workload(F, torch, plans, xd, bufs, stream, steps, warmup, back_to_back=0, settle_ms=SETTLE_MS):
    """Settle, warm-up steps, then `steps` steps between one pair of HIP
    events on the exec stream (no events between launches), then the same
    steps with an event before every exec (median and geometric mean per exec
    and plan), then optionally `back_to_back` steps between one event pair.

    Settle: the workload itself runs for `settle_ms` of wall time before the
    warm-up steps.  Measured on MI355X, a process's first ~100 launches of the
    4096-point pass take 213-215 us and later ones 190 us, whatever the
    launch order (the GPU ramping up from idle); the settle keeps that ramp
    out of the timed region, which then measures the steady state."""
    def step():
        src = xd
        for p, dst in zip(plans, bufs):
            F.fft_exec(p, src, dst, stream.cuda_stream)
            src = dst

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    settle_steps = 0
    while True:
        step()
        settle_steps += 1
        if settle_steps % 8 == 0:
            torch.cuda.synchronize()
            if (time.perf_counter() - t0) * 1e3 >= settle_ms:
                break
    settle = {"ms": round((time.perf_counter() - t0) * 1e3, 1), "steps": settle_steps}
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    WINDOWS.open()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    WINDOWS.close()
    out = {"ms_per_step": ev0.elapsed_time(ev1) / steps, "wall_ms_per_step": wall * 1e3 / steps, "settle": settle}
    out["ms_per_exec"] = out["ms_per_step"] / len(plans)

    # an event before every exec: per-exec durations (the events themselves
    # add a little between launches)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps * len(plans) + 1)]
    k = 0
    for _ in range(steps):
        src = xd
        for p, dst in zip(plans, bufs):
            evs[k].record(stream)
            F.fft_exec(p, src, dst, stream.cuda_stream)
            src = dst
            k += 1
    evs[k].record(stream)
    torch.cuda.synchronize()
    d = [evs[i].elapsed_time(evs[i + 1]) for i in range(k)]
    per_plan = []
    for j in range(len(plans)):
        dj = sorted(d[j::len(plans)])
        per_plan.append({"median_ms": round(dj[len(dj) // 2], 5),
                         "geomean_ms": round(math.exp(sum(math.log(max(v, 1e-9)) for v in dj) / len(dj)), 5)})
    out["per_exec_events"] = per_plan
    if back_to_back:
        b0 = torch.cuda.Event(enable_timing=True)
        b1 = torch.cuda.Event(enable_timing=True)
        b0.record(stream)
        for _ in range(back_to_back):
            step()
        b1.record(stream)
        torch.cuda.synchronize()
        out["back_to_back"] = {"steps": back_to_back,
                               "ms_per_exec": round(b0.elapsed_time(b1) / (back_to_back * len(plans)), 5)}
    return out


def work_per_exec(spec):
    """(flops, algorithmic HBM bytes) of one exec (one direction)."""
    n, batch = spec["n"], spec["batch"]
    if spec["kind"] == "real":
        # 2.5 N log2 N per row and direction; the real rows (4 B) once and the kept bins (8 B) once
        return 2.5 * n * math.log2(n) * batch, batch * n * 4 + (spec["mmax"] + 1) * batch * 8
    return 5.0 * n * math.log2(n) * batch, 2 * spec["passes"] * batch * n * 8   # read + write per HBM pass


def rel(got, want):
    import numpy as np
    d = np.asarray(got, np.complex128) - np.asarray(want, np.complex128)
    return float(np.linalg.norm(d.ravel()) / np.linalg.norm(np.asarray(want, np.complex128).ravel()))


def parity_and_oracle(spec, x_host, outs):
    """Relative L2 error of the GPU outputs against the oracle over the whole
    output of the configuration, and the oracle's own time on that work (one
    run, all host threads; the widening to f64 is not timed)."""
    import numpy as np
    import oracle
    n = spec["n"]
    res = {}
    t_oracle = 0.0
    flops = 0.0

    def timed(fn, *a):
        nonlocal t_oracle
        t0 = time.perf_counter()
        r = fn(*a)
        t_oracle += time.perf_counter() - t0
        return r

    if spec["kind"] == "real":
        mmax = spec["mmax"]
        xs = np.ascontiguousarray(x_host.T).astype(np.complex128)        # [rows][mmax+1]
        rows_gpu = outs[0]                                                 # C2R output [rows][n]
        res["synthesis"] = rel(rows_gpu, timed(oracle.c2r, xs, n, mmax))
        xr = rows_gpu.astype(np.float64)
        res["analysis"] = rel(outs[1].T, timed(oracle.r2c, xr, mmax))      # same rows the GPU analysed
        res["closed_form_r2c_c2r_eq_nF"] = rel(outs[1] / n, x_host)
        flops = 2.5 * n * math.log2(n) * spec["batch"] * 2
        sample = "whole output: C2R against the oracle's synthesis of F, R2C against the oracle's analysis " \
                 "of the GPU's rows, and R2C(C2R(F)) = n F"
    elif spec["kind"] == "2d":
        want = timed(lambda v: oracle.fftshift_2d(oracle.c2c_2d(v, -1)), x_host)
        res["forward_shifted"] = rel(outs[0], want)
        flops = 5.0 * n * math.log2(n)
        sample = "whole image, against the oracle's 2D transform followed by the index rotation"
    elif len(spec["dirs"]) == 2:
        res["forward"] = rel(outs[0], timed(oracle.c2c, x_host, -1))
        res["inverse"] = rel(outs[1], timed(oracle.c2c, outs[0], +1))
        res["round_trip"] = rel(outs[1] / n, x_host)
        flops = 5.0 * n * math.log2(n) * spec["batch"] * 2
        sample = "whole output: forward against the oracle, inverse against the oracle on the GPU's forward " \
                 "output, and the round trip"
    else:
        # row chunks (16 rows each: one oracle thread per row)
        err2 = ref2 = 0.0
        for r0 in range(0, x_host.shape[0], 16):
            want = timed(oracle.c2c, x_host[r0:r0 + 16], spec["dirs"][0])
            d = outs[0][r0:r0 + 16].astype(np.complex128) - want
            err2 += float(np.sum(np.abs(d) ** 2))
            ref2 += float(np.sum(np.abs(want) ** 2))
        res["forward"] = math.sqrt(err2 / ref2)
        flops = 5.0 * n * math.log2(n) * spec["batch"]
        sample = "whole output (all rows), oracle on chunks of 16 rows"
    res = {k: float(f"{v:.4g}") for k, v in res.items()}
    cpu = {"value": round(flops / t_oracle / 1e9, 3), "unit": "GFLOP/s", "cores": oracle.threads(0),
           "kind": "oracle", "sample": f"the parity reference: {sample}; one run, {t_oracle:.3f} s"}
    return res, sample, cpu


def measure_config(F, torch, name, steps, warmup):
    """One configuration end to end: inputs, plans, timing, parity, oracle time."""
    spec = workload_spec(name)
    x_host = spec["gen"]()
    xd = torch.from_numpy(x_host).cuda()
    if spec["kind"] == "real":
        bufs = [torch.empty((spec["batch"], spec["n"]), dtype=torch.float32, device="cuda"), torch.empty_like(xd)]
    else:
        bufs = [torch.empty_like(xd) for _ in spec["dirs"]]
    plans = make_plans(F, spec)
    stream = torch.cuda.current_stream()
    WINDOWS.label = name
    try:
        tm = time_workload(F, torch, plans, xd, bufs, stream, steps, warmup,
                           back_to_back=BACK_TO_BACK if name in ("w1", "w4") else 0)
        torch.cuda.synchronize()
        outs = [b.cpu().numpy() for b in bufs]
    finally:
        for p in plans:
            F.fft_plan_destroy(p)
    del xd, bufs
    torch.cuda.empty_cache()
    flops, nbytes = work_per_exec(spec)
    ms = tm["ms_per_exec"]
    gbps = nbytes / (ms * 1e-3) / 1e9
    entry = {
        "workload": spec["label"],
        "ms_per_exec": round(ms, 5),
        "ms_per_step": round(tm["ms_per_step"], 5),
        "execs_per_step": len(plans),
        "gflops": round(flops / (ms * 1e-3) / 1e9, 2),
        "flop_convention": "2.5 N log2 N per real row" if spec["kind"] == "real" else "5 N log2 N",
        "algorithmic_bytes_per_exec": nbytes,
        "hbm_passes": spec["passes"],
        "algorithmic_gbps": round(gbps, 1),
        "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
        "traffic": stored_traffic(TRAFFIC_KEY[name]),
        "per_exec_events": tm["per_exec_events"],
        "settle": tm["settle"],
    }
    if "back_to_back" in tm:
        entry["back_to_back"] = tm["back_to_back"]
    rl2, sample, cpu = parity_and_oracle(spec, x_host, outs)
    entry["rel_l2"] = rl2
    entry["rel_l2_sample"] = sample
    entry["cpu_baseline"] = cpu
    return entry


def summarize_trace(path, windows=None, out=sys.stdout):
    """Per-kernel durations of a rocprofv3 kernel trace (CSV) of a bench run:
    with `windows` (the --timed-windows file of that run) only the launches
    that started inside a timed region.  Prints a markdown table:
    dispatches, median, mean, min and max duration (us), VGPRs, LDS."""
    import csv
    rows = list(csv.DictReader(open(path)))
    if windows:
        wins = [json.loads(l) for l in open(windows) if l.strip()]
        rows = [r for r in rows if any(w["t0_ns"] <= int(r["Start_Timestamp"]) <= w["t1_ns"] for w in wins)]
    by = {}
    for r in rows:
        by.setdefault(r["Kernel_Name"], []).append(r)
    print("| kernel | dispatches | median us | mean us | min us | max us | VGPR | AGPR | LDS B | scratch B |",
          file=out)
    print("|---|---|---|---|---|---|---|---|---|---|", file=out)
    for name, rs in by.items():
        d = sorted((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rs)
        r0 = rs[0]
        short = name if len(name) <= 90 else name[:87] + "..."
        print(f"| `{short}` | {len(d)} | {d[len(d) // 2]:.1f} | {sum(d) / len(d):.1f} | {d[0]:.1f} | "
              f"{d[-1]:.1f} | {r0.get('VGPR_Count', r0.get('Arch_VGPR_Count', ''))} | "
              f"{r0.get('Accum_VGPR_Count', '')} | {r0.get('LDS_Block_Size', r0.get('Group_Segment_Size', ''))} | "
              f"{r0.get('Scratch_Size', r0.get('Private_Segment_Size', ''))} |", file=out)


# kernels of each stored traffic record: (name prefix, launches per record)
TRAFFIC_KERNELS = {
    "c2c_rows_1024": [("fftamd::k_c2c_rows<1024,", 1.0)],
    "c2c_rows_4096": [("fftamd::k_c2c_rows<4096,", 1.0)],      # per launch (both directions averaged)
    "fourstep_2^22": [("fftamd::k_fs_cols<2048,", 1.0), ("fftamd::k_fs_rows<2048,", 1.0)],
    "real_2048": [("fftamd::k_c2r<1024,", 0.5), ("fftamd::k_r2c<1024,", 0.5)],   # per exec (one direction)
    "2d_8192x8192": [("fftamd::k_rows_fold<8192,", 1.0), ("fftamd::k_fold_cols<2048,", 1.0)],
}
COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_BYTES = 1 << 29     # the bench's reference copy: 512 MiB read and 512 MiB written


NUM_CUS = 256  # MI355X compute units
XCDS = 8   # GRBM_GUI_ACTIVE is summed over the XCDs' instances in rocprofv3's counter CSV


def summarize_pmc(paths, out=sys.stdout):
    """LDS and VALU activity per kernel from rocprofv3 --pmc counter CSVs of a
    bench run (one counter group per run; the files are merged by kernel
    name).  Per dispatch, each counter is summed over its instances (one CSV
    row per dispatch and counter); the table gives the mean over dispatches
    and, where their counters are present, the conflict share
    SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE, VALUBusy = 100 *
    SQ_ACTIVE_INST_VALU / CUs / (GRBM_GUI_ACTIVE / XCDs) and VALUUtilization =
    100 * SQ_THREAD_CYCLES_VALU / (64 * SQ_ACTIVE_INST_VALU)."""
    import csv
    acc = {}
    for path in paths:
        for r in csv.DictReader(open(path)):
            name = r["Kernel_Name"]
            if "fftamd::" not in name:
                continue
            acc.setdefault(name, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    cols = ["SQ_INSTS_LDS", "SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_VALU"]
    print("| kernel | dispatches | LDS instructions | LDS-active clocks | bank-conflict clocks | conflict share | "
          "VALU instructions | VALUBusy % | VALUUtilization % |", file=out)
    print("|---|---|---|---|---|---|---|---|---|", file=out)
    for name, cs in acc.items():
        mean = {k: sum(v) / len(v) for k, v in cs.items()}
        n = max(len(v) for v in cs.values())
        cell = [f"{mean[c]:.4g}" if c in mean else "-" for c in cols]
        share = (f"{mean['SQ_LDS_BANK_CONFLICT'] / mean['SQ_LDS_IDX_ACTIVE']:.3f}"
                 if mean.get("SQ_LDS_IDX_ACTIVE") else "-")
        busy = (f"{100 * mean['SQ_ACTIVE_INST_VALU'] / NUM_CUS / (mean['GRBM_GUI_ACTIVE'] / XCDS):.1f}"
                if mean.get("SQ_ACTIVE_INST_VALU") and mean.get("GRBM_GUI_ACTIVE") else "-")
        util = (f"{100 * mean['SQ_THREAD_CYCLES_VALU'] / (64 * mean['SQ_ACTIVE_INST_VALU']):.1f}"
                if mean.get("SQ_ACTIVE_INST_VALU") and "SQ_THREAD_CYCLES_VALU" in mean else "-")
        short = name.replace("void ", "").split("(")[0]
        print(f"| `{short}` | {n} | {cell[0]} | {cell[1]} | {cell[2]} | {share} | {cell[3]} | {busy} | {util} |",
              file=out)


def summarize_counters(fetch_csv, write_csv, out=sys.stdout, write_traffic=False):
    """HBM bytes per dispatch from two rocprofv3 --pmc runs of the bench
    (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by what the
    same counter reads for the bench's 512 MiB reference copy.  Prints a markdown table per kernel and the bytes of each
    stored traffic record; with write_traffic, stores them in
    profiles/traffic.json under the current kernel-source hash."""
    import csv

    def per_kernel(path, counter):
        acc = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        for k in acc:
            if k.startswith(COPY_KERNEL):
                # the copy kernel also serves torch's small staging copies:
                # keep the dispatches of the 512 MiB reference copy (the largest)
                top = max(acc[k])
                acc[k] = [v for v in acc[k] if v >= 0.9 * top]
        return {k: sum(v) / len(v) for k, v in acc.items()}, {k: len(v) for k, v in acc.items()}

    fetch, nf = per_kernel(fetch_csv, "FETCH_SIZE")
    write, nw = per_kernel(write_csv, "WRITE_SIZE")
    copy_name = next(k for k in fetch if k.startswith(COPY_KERNEL))
    fscale = COPY_BYTES / (fetch[copy_name] * 1024)
    wscale = COPY_BYTES / (write[copy_name] * 1024)
    print(f"Calibration: `{copy_name}` of {COPY_BYTES >> 20} MiB reads FETCH_SIZE {fetch[copy_name]:.0f} KiB and "
          f"WRITE_SIZE {write[copy_name]:.0f} KiB per dispatch: scale x{fscale:.3f} and x{wscale:.3f}.\n", file=out)
    print("| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled bytes |", file=out)
    print("|---|---|---|---|---|", file=out)
    scaled = {}
    for k in fetch:
        if k not in write:
            continue
        scaled[k] = fetch[k] * 1024 * fscale + write[k] * 1024 * wscale
        short = k if len(k) <= 90 else k[:87] + "..."
        print(f"| `{short}` | {nf[k]} / {nw[k]} | {fetch[k]:.0f} | {write[k]:.0f} | {scaled[k]:.4g} |", file=out)
    print("", file=out)
    rec = {}
    for key, parts in TRAFFIC_KERNELS.items():
        total, ok = 0.0, True
        for prefix, w in parts:
            ks = [k for k in scaled if k.split("(")[0].replace("void ", "").startswith(prefix)]
            if not ks:
                ok = False
                break
            total += w * sum(scaled[k] for k in ks) / len(ks)
        if ok:
            rec[key] = int(round(total))
            print(f"- `{key}`: {rec[key]} bytes per record ({' + '.join(p for p, _ in parts)})", file=out)
    if write_traffic:
        path = os.path.join(PROFILES, "traffic.json")
        h = kernel_source_hash()
        d = {key: {"source_hash": h, "bytes_per_launch": v,
                   "evidence": "profiles/hbm_traffic_counters.md",
                   "kernels": [p for p, _ in TRAFFIC_KERNELS[key]]} for key, v in rec.items()}
        json.dump(d, open(path, "w"), indent=1)
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="w2", choices=["w1", "w2", "w3", "w4", "w5", "w6"])
    ap.add_argument("--configs", choices=["all", "none"], default=None,
                    help="also measure configurations c1-c5 (default: all with the w2 headline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--real-pairs", action="store_true",
                    help="w4: two real rows per complex transform of length n")
    ap.add_argument("--n", type=int, default=None,
                    help="w6 only: the row length (default 1000; rows scaled to keep ~512 MiB)")
    ap.add_argument("--direct", action="store_true",
                    help="w4: the band-limited direct sums on the matrix cores instead of the FFT")
    ap.add_argument("--summarize-counters", metavar=("FETCH_CSV", "WRITE_CSV"), nargs=2, default=None,
                    help="HBM bytes per kernel from two rocprofv3 --pmc counter_collection.csv files "
                         "(FETCH_SIZE, then WRITE_SIZE) of a bench run, calibrated on the reference copy")
    ap.add_argument("--summarize-pmc", metavar="CSV", nargs="+", default=None,
                    help="LDS and VALU activity per kernel from rocprofv3 --pmc counter_collection.csv files "
                         "of a bench run (one counter group per file)")
    ap.add_argument("--write-traffic", action="store_true",
                    help="with --summarize-counters: store the records in profiles/traffic.json")
    ap.add_argument("--summarize-trace", metavar="CSV", default=None,
                    help="print the per-kernel durations of a rocprofv3 kernel trace of a bench run and exit "
                         "(with --windows: only the launches of its timed regions)")
    ap.add_argument("--windows", metavar="JSONL", default=None,
                    help="with --summarize-trace: the --timed-windows file of the traced run")
    ap.add_argument("--timed-windows", metavar="JSONL", default=None,
                    help="append the host-clock window of every timed region to this file")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.windows)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, write_traffic=args.write_traffic)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "the transforms are not sharded across devices", file=sys.stderr)
        sys.exit(2)
    if (args.direct or args.real_pairs) and args.workload != "w4":
        raise SystemExit("--direct and --real-pairs apply to the real-transform workload w4")
    if args.direct and args.real_pairs:
        raise SystemExit("--direct and --real-pairs exclude each other")
    if args.n is not None and args.workload != "w6":
        raise SystemExit("--n applies to the any-length workload w6")
    if args.n is not None and (args.n < 3 or args.n & (args.n - 1) == 0):
        raise SystemExit("--n takes a length >= 3 that is not a power of two")
    plain_headline = args.workload == "w2" and not (args.direct or args.real_pairs or args.n)
    WINDOWS.path = args.timed_windows
    configs = args.configs or ("all" if plain_headline else "none")

    import numpy as np
    import torch
    from fourier_transform_amd import fft as F

    if not torch.cuda.is_available():
        raise SystemExit("no HIP device")
    F.lib()  # fail loudly if the library is missing
    spec = any_length_spec(args.n) if args.n is not None else workload_spec(args.workload)
    n, batch = spec["n"], spec["batch"]
    x_host = spec["gen"]()
    xd = torch.from_numpy(x_host).cuda()
    if spec["kind"] == "real":
        # synthesis: m-major spectrum -> real rows; analysis: real rows -> spectrum
        bufs = [torch.empty((batch, n), dtype=torch.float32, device="cuda"), torch.empty_like(xd)]
    else:
        bufs = [torch.empty_like(xd) for _ in spec["dirs"]]
    plans = make_plans(F, spec, direct=args.direct, real_pairs=args.real_pairs)
    stream = torch.cuda.current_stream()
    WINDOWS.label = args.workload
    tm = time_workload(F, torch, plans, xd, bufs, stream, args.steps, args.warmup)
    avg_exec_ms = tm["ms_per_exec"]

    # each direction on its own (same buffers), outside the timed region
    per_dir = None
    if len(plans) == 2:
        per_dir = {}
        src = xd
        for name, p, dst in zip(("forward", "inverse") if spec["dirs"][0] < 0 else ("inverse", "forward"),
                                plans, bufs):
            d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            d0.record(stream)
            for _ in range(args.steps):
                F.fft_exec(p, src, dst, stream.cuda_stream)
            d1.record(stream)
            torch.cuda.synchronize()
            per_dir[name] = round(d0.elapsed_time(d1) / args.steps, 5)
            src = dst

    # correctness guard for the numbers: the round trip must return N x
    check = None
    if len(spec["dirs"]) == 2 and spec["kind"] != "real":
        z = bufs[-1]
        check = float(torch.linalg.vector_norm(z / n - xd) / torch.linalg.vector_norm(xd))

    # attainable-bandwidth reference: a plain 512 MiB device-to-device copy
    a = torch.empty(1 << 27, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    WINDOWS.label = "copy 512 MiB"
    WINDOWS.open()     # the calibration of the HBM byte counters
    c0.record(stream)
    for _ in range(10):
        b.copy_(a)
    c1.record(stream)
    torch.cuda.synchronize()
    WINDOWS.close()
    copy_gbps = 10 * 2 * a.numel() * 4 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del a, b

    ms_per_step = tm["wall_ms_per_step"]
    flops_exec, bytes_per_exec = work_per_exec(spec)
    value = flops_exec * len(plans) / (ms_per_step * 1e-3) / 1e9
    key = TRAFFIC_KEY.get(args.workload, f"any_{n}")
    if args.direct:
        # a real matrix product of batch x n x 2(mmax+1) per launch, on the
        # fp32 matrix cores
        key = "direct_2048"
        flops_mm = 2.0 * batch * n * 2 * (spec["mmax"] + 1)
        achieved = flops_mm / (avg_exec_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": FP32_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / FP32_MFMA_PEAK_TFLOPS, 4),
                "traffic": stored_traffic(key), "kernel": key, "avg_launch_ms": round(avg_exec_ms, 5),
                "algorithmic_flops_per_launch": flops_mm,
                "algorithmic_bytes_per_launch": bytes_per_exec}
    else:
        achieved = bytes_per_exec / (avg_exec_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": stored_traffic(key), "kernel": key,
                "avg_launch_ms": round(avg_exec_ms, 5),
                "algorithmic_bytes_per_launch": bytes_per_exec}
    suffix = ""
    if args.real_pairs:
        suffix = ", two rows per complex transform"
    if args.direct:
        suffix = ", band-limited direct sums (matrix cores)"
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": spec["label"] + suffix, "n": n, "batch": batch,
                   "directions": len(spec["dirs"]),
                   "layout": "float32 rows / m-major complex64 spectrum" if spec["kind"] == "real"
                   else "interleaved complex64"},
        "roofline": roof,
        "copy_gbps": round(copy_gbps, 1),
        "per_exec_events": tm["per_exec_events"],
        "settle": dict(tm["settle"], note="the workload ran this long before the warm-up steps, so that "
                                          "the timed region sees the GPU's steady state, not its ramp from idle"),
    }
    if check is not None:
        out["round_trip_rel_l2"] = check
    if per_dir is not None:
        out["ms_per_direction"] = per_dir
    outs = [b.cpu().numpy() for b in bufs] if configs == "all" else None
    for p in plans:
        F.fft_plan_destroy(p)
    del xd, bufs
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(spec, x_host, direct=args.direct)
        out["cpu_baseline"]["cpu_model"] = cpu_model()

    if configs == "all":
        # every configuration of the metric in the same run; c2 is the
        # headline measurement above (its timed region, parity on its outputs)
        recs = {}
        for cname, wname in CONFIGS:
            print(f"[bench] {cname} ({wname})", file=sys.stderr, flush=True)
            if wname == args.workload:
                rl2, sample, cpu = parity_and_oracle(spec, x_host, outs)
                flops, nbytes = work_per_exec(spec)
                gbps = nbytes / (avg_exec_ms * 1e-3) / 1e9
                recs[cname] = {"workload": spec["label"], "ms_per_exec": round(avg_exec_ms, 5),
                               "ms_per_step": round(tm["ms_per_step"], 5), "execs_per_step": len(plans),
                               "gflops": round(flops / (avg_exec_ms * 1e-3) / 1e9, 2),
                               "flop_convention": "5 N log2 N", "algorithmic_bytes_per_exec": nbytes,
                               "hbm_passes": spec["passes"], "algorithmic_gbps": round(gbps, 1),
                               "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4), "traffic": roof["traffic"],
                               "per_exec_events": tm["per_exec_events"], "settle": tm["settle"], "rel_l2": rl2,
                               "rel_l2_sample": sample, "cpu_baseline": cpu}
            else:
                recs[cname] = measure_config(F, torch, wname, args.steps, args.warmup)
            if cname in BAR_CONFIGS:
                recs[cname]["bar_frac"] = BAR
                recs[cname]["meets_bar"] = recs[cname]["frac_of_hbm_peak"] >= BAR
            else:
                recs[cname]["bar_frac"] = None      # launch-bound parity configurations
            recs[cname]["parity_ok"] = all(v <= 1e-5 for v in recs[cname]["rel_l2"].values())
            recs[cname]["cpu_baseline"]["cpu_model"] = cpu_model()
        out["configs"] = recs
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
