"""Builds libsinkattn.so (the HIP kernels and the C ABI) in-tree for gfx950.

Each source is compiled to an object with hipcc in parallel, then linked into
``streamingllm_sink_attn_amd/libsinkattn.so``; the microbenchmarks of
``csrc/peaks`` become ``libsinkattn_peaks.so``.  Run ``python -m
streamingllm_sink_attn_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsinkattn.so")
PEAKS_LIB = os.path.join(PKG, "libsinkattn_peaks.so")
ARCH = os.environ.get("SINK_ATTN_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

COMMON = [
    "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-I", os.path.join(ROOT, "include"),
    # Packed FP32 arithmetic stays off: plain float code only.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def peaks_sources():
    return sorted(glob.glob(os.path.join(CSRC, "peaks", "*.hip")))


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True, jobs: int = 8) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    srcs, psrcs = sources(), peaks_sources()
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(srcs) + len(psrcs))) as ex:
        objs = list(ex.map(_compile, srcs + psrcs))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], PEAKS_LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources and {PEAKS_LIB} from {len(psrcs)}")
    return LIB


if __name__ == "__main__":
    build(jobs=int(sys.argv[1]) if len(sys.argv) > 1 else 8)
