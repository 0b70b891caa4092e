"""Build libqlq.so (HIP, gfx950) in-tree with hipcc.

    python -m bit_weight_quantized_qlq_amd.build [--verbose]

Sources under csrc/ are compiled in parallel into csrc/../_build/*.o and
linked into bit_weight_quantized_qlq_amd/libqlq.so; the read-rate probes the
benchmark uses (csrc/probe.hip) go into their own libqlq_probe.so.  The build
always recompiles (it is the "does it build" check); nothing is cached across
calls.
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
PROBE_LIB = os.path.join(PKG, "libqlq_probe.so")
PROBE_SOURCES = ["probe.hip"]

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


def _link(objs, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose=False, extra_flags=None, jobs=None, only=None):
    """Compile every source (or only those named in `only`, relinking with the
    objects already built for the others), link libqlq.so and
    libqlq_probe.so; returns the path of libqlq.so."""
    os.makedirs(BUILD, exist_ok=True)
    extra = list(extra_flags or [])
    srcs = SOURCES + PROBE_SOURCES
    todo = srcs if not only else [s for s in srcs if s in only]
    if only and len(todo) != len(set(only)):
        raise ValueError(f"unknown sources {sorted(set(only) - set(srcs))}; sources: {srcs}")
    jobs = jobs or min(len(todo), 8)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = dict(zip(todo, ex.map(lambda s: _compile(s, extra, verbose), todo)))
    for s in srcs:
        if s not in objs:
            o = os.path.join(BUILD, os.path.splitext(s)[0] + ".o")
            if not os.path.exists(o):
                raise RuntimeError(f"{o} is not built: run a full build first")
            objs[s] = o
    _link([objs[s] for s in SOURCES], LIB, verbose)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB, verbose)
    return LIB


# Address and undefined-behaviour sanitizers on the host code only (each
# -fsanitize directly after -Xarch_host: the device code is built as usual).
HOST_SANITIZE = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
]
ABI_DRIVER = os.path.join(ROOT, "tests", "abi_sanitize_driver.cpp")


def build_abi_sanitize_driver(verbose=False):
    """The C ABI's host code (api.cpp) under the address and undefined-behaviour
    sanitizers, linked with the kernel objects of the last full build and the
    host-side validation driver (tests/abi_sanitize_driver.cpp) into one
    executable; returns its path."""
    sdir = os.path.join(BUILD, "sanitize")
    os.makedirs(sdir, exist_ok=True)
    objs = []
    for src, out in ((os.path.join(CSRC, "api.cpp"), os.path.join(sdir, "api.o")),
                     (ABI_DRIVER, os.path.join(sdir, "abi_sanitize_driver.o"))):
        cmd = [HIPCC] + [f for f in CFLAGS if f != "-O3"] + ["-O1", "-g"] + HOST_SANITIZE + \
              ["-x", "hip", "-c", src, "-o", out]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        objs.append(out)
    for s in SOURCES[1:]:  # the kernels, as the last full build left them
        o = os.path.join(BUILD, os.path.splitext(s)[0] + ".o")
        if not os.path.exists(o):
            raise RuntimeError(f"{o} is not built: run a full build first")
        objs.append(o)
    exe = os.path.join(sdir, "abi_sanitize_driver")
    cmd = [HIPCC, f"--offload-arch={ARCH}"] + HOST_SANITIZE + ["-o", exe] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    return exe


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("-D", action="append", default=[], help="extra preprocessor define")
    ap.add_argument("--only", nargs="+", help="compile only these sources (e.g. gemv.hip) and relink")
    args = ap.parse_args()
    path = build(verbose=args.verbose, extra_flags=[f"-D{d}" for d in args.D], only=args.only)
    print(path)


if __name__ == "__main__":
    main()
