"""Build liboscar.so in-tree with hipcc for gfx950.

Usage: ``python -m bit_rotated_kv_int2_amd.build`` (or call ``build()``).
The library lands next to this file; tests, the benchmark and the binding
load it from there.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "liboscar.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

SOURCES = [
    "oscar_api.cpp",
    "oscar_calibrate.cpp",
    "oscar_write.hip",
    "oscar_decode_kernels.hip",
    "oscar_bf16.hip",
]

# Benchmark-only helper library (streaming-read probe); liboscar.so does not
# contain or load it.
PROBE_SOURCE = "bench_read_probe.hip"
PROBE_LIB_PATH = os.path.join(HERE, "libbench_probe.so")

# Packed-FP32 VALU forms are disabled for all device code.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-pthread",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build liboscar.so)")


def _compile(src: str, obj: str, verbose: bool) -> None:
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, *lang, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{r.stdout}\n{r.stderr}")
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if verbose and noise:
        print("\n".join(noise), file=sys.stderr)


def build(verbose: bool = False, jobs: int = 6) -> str:
    """Compile every source and link liboscar.so; returns its path."""
    from concurrent.futures import ThreadPoolExecutor

    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    objs = []
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = []
        for s in SOURCES:
            src = os.path.join(CSRC, s)
            obj = os.path.join(obj_dir, os.path.splitext(s)[0] + ".o")
            objs.append(obj)
            futs.append(ex.submit(_compile, src, obj, verbose))
        for f in futs:
            f.result()
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-pthread", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    _build_probe(verbose)
    return LIB_PATH


def _build_probe(verbose: bool) -> None:
    tmp = PROBE_LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-x", "hip", "-shared", os.path.join(CSRC, PROBE_SOURCE), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {PROBE_SOURCE}:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBE_LIB_PATH)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
