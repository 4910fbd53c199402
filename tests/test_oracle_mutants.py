"""The pins must catch plausible mistakes in the oracle.

Each case below rewrites one expression of ``oracle/dgrad_oracle.c`` (a
dropped condition, a wrong sign or index, a transposed operand, a different
rounding or kink reading), builds that copy with gcc in a temporary
directory, and runs the pin battery on it in a child process (a mutant may
also crash). At least one pin must fail for every mutant. The committed
oracle itself is never modified.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "flip_tap_sign": ("const int a = h + pad - r;", "const int a = h - pad + r;"),
    "drop_stride_divisibility": ("if (a < 0 || a % stride != 0)", "if (a < 0)"),
    "upper_bound_P_off_by_one": ("if (p >= P)", "if (p > P - 1 + (P > 1))"),
    "swap_filter_RS_index": ("(((int64_t)k * R + r) * S + t) * C", "(((int64_t)k * S + t) * R + r) * C"),
    "swap_dy_PQ_index": ("(((int64_t)n * P + p) * Q + q) * K", "(((int64_t)n * Q + q) * P + p) * K"),
    "filter_flip": ("const double* wrow = wd + (((int64_t)k * R + r) * S + t) * C;",
                    "const double* wrow = wd + (((int64_t)k * R + (R - 1 - r)) * S + (S - 1 - t)) * C;"),
    "hardswish_slope": ("return z / 3.0 + 0.5;", "return z / 6.0 + 0.5;"),
    "hardswish_left_kink_open": ("if (z < -3.0)", "if (z <= -3.0)"),
    "relu_at_zero": ("return z > 0.0 ? 1.0 : 0.0;", "return z >= 0.0 ? 1.0 : 0.0;"),
    "half_exponent_bias": ("expo - 25", "expo - 24"),
    "half_subnormal_scale": ("ldexp((double)frac, -24)", "ldexp((double)frac, -25)"),
    "rounding_truncates": ("nearbyint(a / quantum)", "floor(a / quantum)"),
    "epilogue_skipped": ("o[c] = acc[c] * epilogue_factor(epi, lut[zrow[c]]);", "o[c] = acc[c];"),
    "pad_used_once": ("const int b = x + pad - t;", "const int b = x - t;"),
    "wgrad_pad_sign": ("const int h = p * stride - pad + r;", "const int h = p * stride + pad - r;"),
    "wgrad_column_bound": ("if (w < 0 || w >= W)", "if (w < 0 || w > W)"),
    "wgrad_filter_row_decode": ("const int r = (int)((fr / S) % R);\n            const int t = (int)(fr % S);",
                                "const int t = (int)((fr / R) % S);\n            const int r = (int)(fr % R);"),
    "wgrad_input_transposed": ("x + (((int64_t)n * H + h) * W + w) * C", "x + (((int64_t)n * W + w) * H + h) * C"),
    "wgrad_signed_magnitude": ("mag[c] += fabs(v);", "mag[c] += v;"),
    "wgrad_stride_ignored": ("const int w = q * stride - pad + t;", "const int w = q - pad + t;"),
    "forward_bias_dropped": ("acc[k] = lut[bias[k]];", "acc[k] = 0.0;"),
    "forward_hardswish_clamp": ("if (g > 6.0)", "if (g > 3.0)"),
    "forward_filter_taps_swapped": ("wt + (((int64_t)k * R + r) * S + t) * C", "wt + (((int64_t)k * S + t) * R + r) * C"),
    "forward_output_decode": ("const int p = (int)((pix / Q) % P);", "const int p = (int)((pix / P) % Q);"),
    "chain_t_unrounded": ("oracle_half_to_double(oracle_double_to_half_rne(t[it * (int64_t)Cm + c]))",
                          "t[it * (int64_t)Cm + c]"),
    "chain_w2_transposed": ("o[ci] += tc * wrow[ci];", "o[ci] += tc * w2d[(int64_t)ci * Cm + c];"),
    "chain_epilogue_dropped": ("1, pad, epi, rows, nrows, t, nthreads", "1, pad, 0, rows, nrows, t, nthreads"),
}

_CHILD = r"""
import sys
sys.path.insert(0, {root!r})
import oracle
from tests import oracle_pins
lib = oracle.load({lib!r})
failed = oracle_pins.run_all(lib)
print("FAILED:" + ";".join(failed))
"""


def _run_battery(lib_path):
    code = _CHILD.format(root=ROOT, lib=lib_path)
    proc = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600)
    if proc.returncode != 0:
        return ["crashed"]
    line = [l for l in proc.stdout.splitlines() if l.startswith("FAILED:")][-1]
    return [f for f in line[len("FAILED:"):].split(";") if f]


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    src = open(oracle.SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new)
    path = tmp_path / "mutant.c"
    path.write_text(mutated)
    lib = str(tmp_path / "libmutant.so")
    oracle.build(src=str(path), out=lib)
    failed = _run_battery(lib)
    assert failed, f"no pin caught mutant {name}"
