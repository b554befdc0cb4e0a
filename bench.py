"""Throughput of the batched fp32 FFT on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload w2]

One step is one pass of the whole hot path over one batch: for the default
workload (w2: 16384 rows of N = 4096 complex64, U[-1,1]) a forward transform
followed by the inverse of its output, two kernel launches.  Inputs are
resident in HBM before timing starts.  Prints ONE JSON line.

value     = 5 N log2(N) * rows * directions / time  (GFLOP/s, the pages'
            flop convention)
roofline  = algorithmic HBM bytes of one launch (read + write of every
            element once) / the average launch duration, timed with HIP events
            on the stream the kernels run on, against the 8 TB/s HBM peak
cpu_baseline = the f64 oracle (untuned reference) on a bounded sample of the
            same workload on the host cores
"""
import argparse
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="w2", choices=["w1", "w2", "w3", "w4", "w5", "w6"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--real-pairs", action="store_true",
                    help="w4: two real rows per complex transform of length n")
    ap.add_argument("--n", type=int, default=None,
                    help="w6 only: the row length (default 1000; rows scaled to keep ~512 MiB)")
    ap.add_argument("--direct", action="store_true",
                    help="w4: the band-limited direct sums on the matrix cores instead of the FFT")
    args = ap.parse_args()
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
    plans = []
    for s in spec["dirs"]:
        if spec["kind"] == "real":
            if args.direct:
                kind = F.FFT_C2R_DIRECT if s > 0 else F.FFT_R2C_DIRECT
            else:
                kind = F.FFT_C2R if s > 0 else F.FFT_R2C
            p = F.fft_plan_create(n, batch, kind, s)
            F.fft_plan_set(p, F.FFT_OPT_MMAX, spec["mmax"])
            F.fft_plan_set(p, F.FFT_OPT_SPEC_LAYOUT, 1)
            if args.real_pairs:
                F.fft_plan_set(p, F.FFT_OPT_REAL_PAIRS, 1)
        elif spec["kind"] == "2d":
            p = F.fft_plan_create_2d(spec["ny"], spec["nx"], batch, F.FFT_C2C, s)
            F.fft_plan_set(p, F.FFT_OPT_SHIFT, 1)
        else:
            p = F.fft_plan_create(n, batch, F.FFT_C2C, s)
        plans.append(p)
    stream = torch.cuda.current_stream()

    def step():
        src = xd
        for p, dst in zip(plans, bufs):
            F.fft_exec(p, src, dst, stream.cuda_stream)
            src = dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K steps between two synchronisations, bracketed by HIP
    # events on the stream the kernels are launched on (no events between
    # launches, which would insert gaps)
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
    avg_exec_ms = ev0.elapsed_time(ev1) / (args.steps * len(plans))

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
    if len(spec["dirs"]) == 2:
        z = bufs[-1]
        check = float(torch.linalg.vector_norm(z / n - xd) / torch.linalg.vector_norm(xd))

    # attainable-bandwidth reference: a plain 512 MiB device-to-device copy
    a = torch.empty(1 << 27, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(10):
        b.copy_(a)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 10 * 2 * a.numel() * 4 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del a, b

    ms_per_step = wall * 1e3 / args.steps
    if spec["kind"] == "real":
        # real transforms: 2.5 N log2 N per row and direction; bytes per exec:
        # the real rows (4 B) once and the kept bins (8 B) once
        flops_step = 2.5 * n * math.log2(n) * batch * len(spec["dirs"])
        bytes_per_exec = batch * n * 4 + (spec["mmax"] + 1) * batch * 8
    else:
        flops_step = 5.0 * n * math.log2(n) * batch * len(spec["dirs"])
        bytes_per_exec = 2 * spec["passes"] * x_host.nbytes      # read + write per HBM pass
    value = flops_step / (ms_per_step * 1e-3) / 1e9
    key = {"w1": "c2c_rows_1024", "w2": "c2c_rows_4096", "w3": "fourstep_2^22",
           "w4": "real_2048", "w5": "2d_8192x8192", "w6": f"any_{n}"}[args.workload]
    if args.direct:
        # a real matrix product of batch x n x 2(mmax+1) per launch, on the
        # fp32 matrix cores
        key = "direct_2048"
        flops_exec = 2.0 * batch * n * 2 * (spec["mmax"] + 1)
        achieved = flops_exec / (avg_exec_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": FP32_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / FP32_MFMA_PEAK_TFLOPS, 4),
                "traffic": stored_traffic(key), "kernel": key, "avg_launch_ms": round(avg_exec_ms, 5),
                "algorithmic_flops_per_launch": flops_exec,
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
    }
    if check is not None:
        out["round_trip_rel_l2"] = check
    if per_dir is not None:
        out["ms_per_direction"] = per_dir
    for p in plans:
        F.fft_plan_destroy(p)
    del xd, bufs
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(spec, x_host, direct=args.direct)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
