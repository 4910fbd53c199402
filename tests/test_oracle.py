"""The oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle
from tests import oracle_pins as pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(oracle_lib, check):
    check(oracle_lib)


def test_invalid_arguments_rejected(oracle_lib):
    dy = np.zeros((1, 3, 3, 1), np.float16)
    w = np.zeros((1, 3, 3, 1), np.float16)
    with pytest.raises(ValueError):
        oracle.dgrad(dy, w, 3, 3, 1, 1, epilogue=2, z=None, lib=oracle_lib)
    with pytest.raises(ValueError):
        oracle.dgrad(dy, w, 4, 3, 1, 1, lib=oracle_lib)       # P mismatch
    assert oracle_lib.oracle_out_extent(2, 3, 1, 0) == 0     # filter larger than input


def test_configs_extents_match_recipe():
    """The measured layers' dy extents (28, 56, 14, 7) follow from H, R, s, pad."""
    from workloads import CONFIGS
    want = {"tiny_n1_14x14_256_3x3_s1": 14, "r50_stage2_3x3_n8": 56, "r50_3x3_s2_n256": 28,
            "r50_1x1_s2_downsample_n256": 28, "r50_1x1_s1_reduce_n256": 14,
            "r50_stage4_3x3_dhardswish_n256": 7}
    for c in CONFIGS:
        assert c.P == c.Q == want[c.name]
        assert oracle.out_extent(c.H, c.R, c.stride, c.pad) == c.P
