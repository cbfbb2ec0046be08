"""Ahead-of-time build of libqlinear.so for gfx950 with hipcc.

Each HIP source is compiled to an object (in parallel), then linked into one
shared library next to this file.  Flags:
  -ffp-contract=off   quantizer arithmetic must round once per operation;
                      the kernels write every FMA they want explicitly.
  -packed-fp32-ops    off: no packed fp32 VALU instructions are generated.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqlinear.so")
OBJDIR = os.path.join(HERE, "_build")
SOURCES = ["api.hip", "isq.hip", "gemv.hip", "gemv_fp8.hip", "gemm.hip", "probe.hip"]
ARCH = os.environ.get("QLINEAR_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I", os.path.join(HERE, "..", "include"),
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    # the host pass does not know the packed-fp32 feature; that note is harmless
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [ln for ln in r.stderr.splitlines() if noise not in ln and ln.strip()]
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def build() -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
