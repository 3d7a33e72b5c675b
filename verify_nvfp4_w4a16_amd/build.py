"""Build libnvfp4_w4a16.so in-tree: host C++ with g++, HIP kernels for gfx950.

Usage: python -m verify_nvfp4_w4a16_amd.build   (or __graft_entry__.build()).
Always recompiles every source.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB_DIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIB_DIR, "libnvfp4_w4a16.so")
ARCH = "gfx950"

HOST_SOURCES = ["host/pack.cpp", "host/tiles.cpp"]
HIP_SOURCES = ["kernels/nvfp4_linear.hip", "kernels/nvfp4_gemm.hip", "kernels/nvfp4_fused.hip",
               "kernels/w8a16.hip", "kernels/read_probe.hip", "kernels/library_gemm.hip"]

# -ffp-contract=off keeps the packer's float64 steps unfused (bit-exact rule).
HOST_FLAGS = ["-std=c++17", "-O3", "-fPIC", "-ffp-contract=off", "-Wall", "-Wextra",
              "-pthread", "-I", INCLUDE]
# Packed fp32 instructions are kept out of the device code on purpose.
HIP_FLAGS = ["-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-I", INCLUDE]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd: list[str]) -> str:
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in proc.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"build step failed ({proc.returncode}): {' '.join(cmd)}\n{out}")
    return out


# The compiler's per-kernel resource report (one remark block per kernel).
RESOURCE_REMARKS = "-Rpass-analysis=kernel-resource-usage"


def scratch_users(report: str) -> list[tuple[str, int]]:
    """(kernel, bytes per lane) for every kernel in a resource report that
    spills to scratch memory."""
    users = []
    name = None
    for line in report.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name is not None and int(m.group(1)) > 0:
            users.append((name, int(m.group(1))))
    return users


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    hipcc = _hipcc()
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        cmd = ["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        _run(cmd)
        objs.append(obj)
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        cmd = [hipcc, *HIP_FLAGS, RESOURCE_REMARKS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        spills = scratch_users(_run(cmd))
        if spills:
            # every kernel the library can launch must keep its registers
            raise RuntimeError(f"{src}: kernels spill to scratch: {spills}")
        objs.append(obj)
    tmp = LIB + ".tmp"
    # hipBLASLt: the library GEMM of the expand path
    cmd = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-pthread", *objs, "-lhipblaslt", "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    _run(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
