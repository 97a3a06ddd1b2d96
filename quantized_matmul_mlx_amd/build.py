"""Builds libqaff.so (HIP, gfx950 only) in-tree with hipcc, and beside it libqaff_bench.so (the
benchmark's measurement aids, include/qaff_bench.h; not linked into libqaff.so).

    python -m quantized_matmul_mlx_amd.build          # or __graft_entry__.build()

Each source compiles to an object under _build/ in parallel, then they link into
quantized_matmul_mlx_amd/libqaff.so and libqaff_bench.so. Always recompiles.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqaff.so")
BENCH_LIB = os.path.join(PKG, "libqaff_bench.so")

# every .hip and .cpp file under csrc/ goes into libqaff.so, except the benchmark's aids
BENCH_SOURCES = ["bench_aux.hip"]
SOURCES = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")) and f not in BENCH_SOURCES)

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-std=c++17", "-O3", f"--offload-arch={ARCH}", "-fPIC",
    # Packed-FP32 instructions are kept out of every kernel (hipcc -O3 would otherwise form them
    # from ordinary float code); the host pass warns that it does not know the feature.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    # The first kernel arguments arrive in SGPRs at dispatch instead of through a scalar load at
    # the start of every wave: the decode GEMV (a single round trip to HBM) took 3.78 instead of
    # 4.03 us per call.
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if noise not in l]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
    if msgs and verbose:
        print("\n".join(msgs), flush=True)
    return obj


def _link(lib: str, objs, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + BENCH_SOURCES
    with ThreadPoolExecutor(max_workers=min(len(srcs), 8)) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
    _link(LIB, [objs[s] for s in SOURCES], verbose)
    _link(BENCH_LIB, [objs[s] for s in BENCH_SOURCES], verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
