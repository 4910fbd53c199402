"""The host code of the library under AddressSanitizer and
UndefinedBehaviorSanitizer (host side only: the kernels are built as usual
and never launched). tests/abi_stress.cpp drives the host-only entry points
from eight threads at once: validation, plans, workspace-size queries and the
tile-config table (query, save, load, clear)."""
import os
import subprocess

import pytest

from convolution_backward_amd.build import SOURCES

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "convolution_backward_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

pytestmark = pytest.mark.slow


def test_abi_under_asan_ubsan_with_eight_threads(tmp_path):
    exe = str(tmp_path / "abi_stress")
    sources = [os.path.join(ROOT, "tests", "abi_stress.cpp")] + [os.path.join(CSRC, f) for f in SOURCES]
    cmd = [HIPCC, "-O1", "-g", "-std=c++17", "--offload-arch=gfx950",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, *sources, "-pthread", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    res = subprocess.run([exe, str(tmp_path)], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-4000:]
    assert "0 failures" in res.stdout
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr[-4000:]
