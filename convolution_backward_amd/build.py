"""Build libconv2d_dgrad.so in-tree with hipcc for gfx950.

Usage: python -m convolution_backward_amd.build   (always recompiles)
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libconv2d_dgrad.so")
OBJDIR = os.path.join(PKG, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed-fp32 VALU forms are kept out of generated code on purpose.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function"]

SOURCES = ["dgrad_kernels.hip", "dgrad_wide.hip", "dgrad_halo.hip", "dgrad_pgemm.hip", "dgrad_halo1.hip", "dgrad_pwide.hip", "chain_kernels.hip", "dgrad_api.cpp", "dgrad_plan.cpp"]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    remarks = ["-Rpass-analysis=kernel-resource-usage"] if src.endswith(".hip") else []
    cmd = [HIPCC, *COMMON, *lang, *remarks, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, check=True, capture_output=True, text=True)
    if remarks:
        _check_no_scratch(src, res.stderr)
    return obj


def _check_no_scratch(src: str, remarks: str) -> None:
    """The kernels count their own vector-memory operations to wait for
    exactly the loads they need; a scratch (private memory) access would be
    an operation they do not count. Refuse a build in which any kernel uses
    scratch."""
    kernel, bad, seen = None, [], 0
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            kernel = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m:
            seen += 1
            if int(m.group(1)) != 0:
                bad.append(f"{kernel}: {m.group(1)} bytes/lane")
    if seen == 0:
        raise RuntimeError(f"{src}: no kernel resource-usage remarks from the compiler")
    if bad:
        raise RuntimeError(f"{src}: kernels use scratch memory: " + "; ".join(bad))


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], check=True)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
