"""The kernels' multiply-shift division, checked exhaustively on the CPU.

The header compiles as plain C++ without HIP; a small driver built with g++
compares it with hardware division over every divisor up to 4096 and many
numerators, including the largest the kernels use (2^31 - 1)."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "convolution_backward_amd", "csrc")

DRIVER = r"""
#include <cstdio>
#include <cstdint>
#include "fastdiv.h"
int main() {
    uint64_t bad = 0, checked = 0;
    uint32_t ds[] = {4097u, 50176u, 200704u, 3136u, 784u, 65535u, 65536u, 1000003u, 2147483647u};
    auto test = [&](uint32_t d) {
        cbw::FastDiv f = cbw::make_fastdiv(d);
        auto one = [&](uint32_t n) { ++checked; if (cbw::fastdiv(n, f) != n / d) ++bad; };
        for (uint32_t n = 0; n < 70000; ++n) one(n);
        for (uint32_t k = 1; k < 4000; ++k) { uint64_t m = (uint64_t)d * (k * 524287ull % 2147483647ull / d + 1);
            if (m < 2147483648ull) { one((uint32_t)m); one((uint32_t)(m - 1)); } }
        one(2147483647u); one(2147483646u);
    };
    for (uint32_t d = 1; d <= 4096; ++d) test(d);
    for (uint32_t d : ds) test(d);
    std::printf("%llu %llu\n", (unsigned long long)checked, (unsigned long long)bad);
    return bad != 0;
}
"""


def test_fastdiv_exhaustive(tmp_path):
    src = tmp_path / "drv.cpp"
    src.write_text(DRIVER)
    exe = tmp_path / "drv"
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    checked, bad = (int(v) for v in out.stdout.split())
    assert bad == 0 and checked > 1_000_000
