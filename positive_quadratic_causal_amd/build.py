"""Build liboal.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Every source under csrc/ is compiled with hipcc for --offload-arch=gfx950 and
linked into positive_quadratic_causal_amd/liboal.so.  Packed fp32 vector
instructions are disabled for all device code (-packed-fp32-ops).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(os.path.dirname(HERE), "_build")
LIB = os.path.join(HERE, "liboal.so")
ARCH = "gfx950"

SOURCES = [
    "oal_api.hip",
    "oal_expand.hip",
    "oal_state.hip",
    "oal_decode.hip",
    "oal_prefill_vec.hip",
    "oal_prefill_mfma.hip",
    "oal_state_mfma.hip",
    "oal_softmax.hip",
    "oal_backward.hip",
    "oal_calib.hip",
    "oal_grouping.hip",
]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
    "-Rpass-analysis=kernel-resource-usage",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if warn:
        print(f"[build] {src}:\n{warn}", file=sys.stderr)
    return obj


def build(jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
