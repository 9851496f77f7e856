"""Builds libqmv.so (the C-ABI library) in-tree for gfx950.

    python gguf_block_quantized_qmv_amd/build.py [-v]

The HIP kernel files are compiled with hipcc for gfx950 only; the ABI layer
(qmv_api.cpp, pure host code with no HIP call) with g++. Objects go to
_build/ at the repository root, the library next to this file.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqmv.so")

HIP_SOURCES = ["q4k_gemv.hip", "q8_0.hip", "q4k_dequant.hip", "q4k_moe.hip", "q4k_prefill.hip", "iq4xs_gemv.hip", "iq4xs_moe.hip", "q6k_gemv.hip", "q4k_moe_grouped.hip", "calib_read.hip"]
HOST_SOURCES = ["qmv_api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    # keep hipcc from forming packed fp32 instructions (v_pk_{add,mul,fma}_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I" + INCLUDE,
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I" + INCLUDE]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}):\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if verbose and noise:
        print("\n".join(noise), file=sys.stderr)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source and link libqmv.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    steps = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        steps.append([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        steps.append(["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    workers = jobs or min(len(steps), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        for f in [ex.submit(_run, s, verbose) for s in steps]:
            f.result()
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
