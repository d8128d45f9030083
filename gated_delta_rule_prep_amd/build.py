"""Build libkda.so (the C-ABI library) from csrc/ with hipcc for gfx950.

Every HIP source is compiled for gfx950 only, with the packed-fp32 target
feature switched off; objects go to _build/ and the shared library is written
next to this file, where kda.py loads it from.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkda.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -amdgpu-mfma-vgpr-form keeps MFMA accumulators in ordinary VGPRs: the
# recurrence scales and converts its state accumulators with VALU instructions
# every chunk, and accumulators placed in AGPRs cost a copy each way.
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form=1",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]
SOURCES = ["kda_api.cpp", "kda_sched.hip", "kda_prep.hip", "kda_recur.hip", "kda_prep32.hip", "kda_recur32.hip", "kda_prep64.hip", "kda_recur64.hip", "kda_fused.hip", "kda_segment.hip",
           "kda_decode.hip"]


def _compile(src: str) -> str:
    out = os.path.join(OBJ, os.path.basename(src) + ".o")
    lang = ["-x", "hip"]
    cmd = [HIPCC, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed on %s" % src)
    return out


def build(verbose: bool = False) -> str:
    """Compile every source (always) and link libkda.so; returns its path."""
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link of libkda.so failed")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
