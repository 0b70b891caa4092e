"""Build libqlq.so (HIP, gfx950) in-tree with hipcc.

    python -m bit_weight_quantized_qlq_amd.build [--verbose]

Sources under csrc/ are compiled in parallel into csrc/../_build/*.o and
linked into bit_weight_quantized_qlq_amd/libqlq.so.  The build always
recompiles (it is the "does it build" check); nothing is cached across calls.
"""

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libqlq.so")
SOURCES = ["api.cpp", "pack.hip", "gemv.hip", "gemm.hip", "ternary.hip", "int8.hip", "pergroup.hip", "w4a8.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# -ffp-contract=off: every fused multiply-add in the kernels is written out
# explicitly, so the rounding of each step is the one the source states.
# The packed-fp32 feature is disabled for the device code.
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=off",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src, extra, verbose):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC] + CFLAGS + extra + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def build(verbose=False, extra_flags=None, jobs=None):
    """Compile every source and link libqlq.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    extra = list(extra_flags or [])
    jobs = jobs or min(len(SOURCES), 8)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("-D", action="append", default=[], help="extra preprocessor define")
    args = ap.parse_args()
    path = build(verbose=args.verbose, extra_flags=[f"-D{d}" for d in args.D])
    print(path)


if __name__ == "__main__":
    main()
