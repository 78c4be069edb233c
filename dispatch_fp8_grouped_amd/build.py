"""Build libmegamoe.so (HIP, gfx950 only) in-tree with hipcc.

    python -m dispatch_fp8_grouped_amd.build          # or: python dispatch_fp8_grouped_amd/build.py

Every source in csrc/ is compiled to an object for gfx950, then linked into
dispatch_fp8_grouped_amd/libmegamoe.so.  Packed fp32 instructions are disabled for the device code, and
the build fails if any kernel spills registers or uses scratch memory.
"""
from __future__ import annotations

import concurrent.futures
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libmegamoe.so")
BUILD_DIR = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-disable-promote-alloca-to-lds",
]
SOURCES = ["route.hip", "fill.hip", "gemm.hip", "combine.hip", "pack.hip", "host.hip"]


def _check_resources(src: str, remarks: str) -> None:
    """Fail on any kernel that spills or uses scratch: a scratch access makes the compiler wait for
    every outstanding vector-memory operation, which would drain the GEMM's LDS-DMA pipeline."""
    kernel = None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            kernel = m.group(1)
            continue
        m = re.search(r"(VGPRs Spill|SGPRs Spill|ScratchSize \[bytes/lane\]): (\d+)", line)
        if m and int(m.group(2)) != 0 and not (m.group(1) == "SGPRs Spill"):
            raise RuntimeError(f"{src}: kernel {kernel} has {m.group(1)} = {m.group(2)}")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, "-Rpass-analysis=kernel-resource-usage", "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    _check_resources(src, res.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
