"""The fused hardswish' epilogue forms z/3 without a division (kernel_common.h,
epilogue_factor): q0 = z * RN(1/3), e = fma(-3, q0, z), q = fma(e, RN(1/3), q0).
This test emulates those fp32 operations exactly on the host and checks that
q is the correctly rounded fp32 quotient z/3 for every fp16 value z in
[-3, 3] (the only inputs the kernels feed it: z is an fp16 tensor, and g is
0 or 1 outside that interval), so the replacement changes no result bit."""
from fractions import Fraction

import numpy as np

THIRD_RN = np.float32(float.fromhex("0x1.555556p-2"))


def _rn32(x: Fraction) -> np.float32:
    """x rounded to the nearest fp32 value, ties to even (exact: the
    candidates around a double approximation are compared as fractions)."""
    c = np.float32(float(x))
    best = None
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        d = abs(Fraction(float(cand)) - x)
        even = (int(np.float32(cand).view(np.uint32)) & 1) == 0
        if best is None or d < best[0] or (d == best[0] and even):
            best = (d, np.float32(cand))
    return best[1]


def _fma32(a, b, c) -> np.float32:
    return _rn32(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c)))


def test_third_constant_is_rn_of_one_third():
    assert THIRD_RN == _rn32(Fraction(1, 3))
    assert THIRD_RN.view(np.uint32) == np.uint32(0x3EAAAAAB)


def test_rn32_helper_on_known_ties():
    # 1 + 2^-24 lies halfway between 1 and 1 + 2^-23: ties to even gives 1
    assert _rn32(Fraction(1) + Fraction(1, 2 ** 24)) == np.float32(1.0)
    # 1 + 3*2^-24 lies halfway between 1 + 2^-23 and 1 + 2^-22: even is 1 + 2^-22
    assert _rn32(Fraction(1) + Fraction(3, 2 ** 24)) == np.float32(1.0 + 2.0 ** -22)


def test_division_free_third_is_correctly_rounded_for_every_fp16_input():
    checked = 0
    for bits in range(1 << 16):
        z16 = np.uint16(bits).view(np.float16)
        if not np.isfinite(z16) or not (-3.0 <= float(z16) <= 3.0):
            continue
        z = np.float32(z16)
        q0 = np.float32(z * THIRD_RN)              # one fp32 multiply, rounded once
        q = _fma32(_fma32(np.float32(-3.0), q0, z), THIRD_RN, q0)
        want = _rn32(Fraction(float(z)) / 3)
        assert float(q) == float(want), (float(z), float(q), float(want))
        checked += 1
    assert checked > 30000
