"""Build libkq.so (the HIP C-ABI library) in-tree for gfx950.

    python post_weight_quantization_amd/build.py

Every source under csrc/ is compiled with hipcc to an object under _build/,
then linked into post_weight_quantization_amd/libkq.so. Packed fp32 vector
instructions are disabled for device code (-packed-fp32-ops).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libkq.so")

SOURCES = ["kq_api.hip", "gemm_f32.hip", "cov.hip", "biip.hip", "chol.hip", "gptaq.hip",
           "objective.hip", "deploy.hip", "yaqa.hip"]

# microbenchmarks of the part's own ceilings, for the benchmark (not the ABI)
PEAKS_SOURCES = ["peaks.hip"]
PEAKS_LIB = os.path.join(HERE, "libkq_peaks.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 1)
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES + PEAKS_SOURCES))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PEAKS_LIB)
    if verbose:
        print(f"built {LIB} and {PEAKS_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
