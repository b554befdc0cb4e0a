"""Build libfft_amd.so: hand-written HIP kernels for gfx950 plus the C-ABI runtime.

    python -m fourier_transform_amd.build [--force] [--variant default|poison|all]

Objects go to ``fourier_transform_amd/_build/`` (``_build_poison/`` for the
debug variant); the libraries are written in-tree next to this file so that
they travel with the source tree.

Variants:
  default  libfft_amd.so, the product library
  poison   libfft_amd_poison.so, the LDS-poison debug build: the same sources
           with -DFFTAMD_LDS_POISON=1, so that every kernel fills its LDS with
           NaNs before use (a read of LDS nothing wrote shows up as NaNs in
           the output); the GPU tests run a parity sweep on it
"""
import argparse
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfft_amd.so")
POISON_LIB = os.path.join(HERE, "libfft_amd_poison.so")
VARIANTS = {
    "default": (OBJ, LIB, []),
    "poison": (os.path.join(HERE, "_build_poison"), POISON_LIB, ["-DFFTAMD_LDS_POISON=1"]),
}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming packed fp32 instructions
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-x", "hip",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def headers():
    return glob.glob(os.path.join(CSRC, "*.hpp")) + [os.path.join(ROOT, "include", "fft.h")]


def _compile(src, obj, extra, verbose):
    cmd = [HIPCC] + FLAGS + extra + ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    return src


def build(force: bool = False, verbose: bool = False, jobs: int = None, variants=("default",)) -> str:
    """Compile every HIP source for gfx950 and link the libraries of the given
    variants (one job pool for all of them); returns the first library's path."""
    newest_hdr = max(os.path.getmtime(h) for h in headers())
    todo, links = [], []
    for v in variants:
        obj_dir, lib, extra = VARIANTS[v]
        os.makedirs(obj_dir, exist_ok=True)
        objs = []
        for src in sources():
            obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
            objs.append(obj)
            if force or not os.path.exists(obj) or os.path.getmtime(obj) < max(
                    os.path.getmtime(src), newest_hdr):
                todo.append((src, obj, extra))
        links.append((lib, objs))
    # longest compilations first (the sources with the most instantiations)
    heavy = ["k_fourstep_cols.hip", "k_fourstep_rows.hip", "k_fold.hip", "k_c2c_cols.hip", "k_real.hip"]
    todo.sort(key=lambda t: heavy.index(os.path.basename(t[0])) if os.path.basename(t[0]) in heavy
              else len(heavy))
    jobs = jobs or min(8, os.cpu_count() or 1, max(1, len(todo)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for f in [ex.submit(_compile, s, o, x, verbose) for s, o, x in todo]:
            f.result()
    for lib, objs in links:
        if todo or force or not os.path.exists(lib):
            tmp = lib + ".tmp"
            cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC"] + objs + ["-o", tmp]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True)
            os.replace(tmp, lib)
    return links[0][0]


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--force", action="store_true")
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("--variant", choices=["default", "poison", "all"], default="default")
    args = ap.parse_args()
    variants = ("default", "poison") if args.variant == "all" else (args.variant,)
    print(build(force=args.force, verbose=args.verbose, variants=variants))
    sys.exit(0)
