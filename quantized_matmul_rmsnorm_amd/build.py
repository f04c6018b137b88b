"""Build libmmq.so (the gfx950 HIP kernels and the C-ABI host library) in-tree,
and libmmq_peak.so (measured MFMA ceilings; loaded by the benchmark only).

hipcc cross-compiles for gfx950 without a GPU.  Every HIP translation unit is
built with -O3, no fast-math (the quantiser relies on IEEE division and
round-half-even), and packed-FP32 instruction generation disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmmq.so")
LIB_PEAK = os.path.join(PKG, "libmmq_peak.so")
SOURCES = ["quant.hip", "repack.hip", "gemm.hip", "mmvq.hip", "host.cpp"]
PEAK_SOURCES = ["peak.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs: list, lib: str) -> None:
    tmp = lib + ".tmp"
    r = subprocess.run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs,
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build() -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PEAK_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PEAK_SOURCES], LIB_PEAK)
    return LIB


if __name__ == "__main__":
    print(build())
