"""GPU parity: the HIP path against the fp64 oracle, through the C ABI.

Tolerance: |gpu - ref| <= 1e-3 + 1e-2 |ref| elementwise; bit-exact where the
arithmetic is exact (integer inputs, zero phases, one-hot dy, epilogue ties).
dx is filled with NaN before every call so an unwritten element fails.
"""
import numpy as np
import pytest

import convolution_backward_amd as cb
import oracle
from workloads import (CONFIGS, EPI_DHARDSWISH, EPI_DRELU, EPI_NONE, integer_inputs, make_inputs,
                       one_hot_dy, small_config)
from tests.gpu_util import assert_close, note, ref_full, ref_rows, run, to_dev

pytestmark = pytest.mark.gpu

# N, H, W, C, K, R, S, stride, pad: several tiles, ragged tails in M, C and K,
# every stride-phase situation (zero phases carried by GEMM tiles or left to
# standalone chunks, empty lattices, >16 phases).
SMALL = [
    (2, 15, 13, 136, 72, 3, 3, 1, 1),
    (2, 17, 16, 64, 128, 3, 3, 2, 1),
    (3, 11, 12, 40, 24, 3, 3, 2, 0),
    (1, 20, 19, 32, 16, 1, 1, 2, 0),
    (2, 9, 9, 16, 16, 5, 5, 3, 2),
    (1, 14, 14, 264, 56, 1, 1, 1, 0),
    (2, 8, 10, 24, 8, 2, 4, 2, 1),
    (1, 23, 23, 16, 16, 3, 3, 5, 1),
    (1, 5, 5, 8, 8, 7, 7, 1, 3),
    (1, 1, 1, 8, 8, 1, 1, 1, 0),
    (1, 3, 3, 8, 8, 3, 3, 4, 2),
    (1, 33, 35, 8, 8, 3, 3, 16, 1),
    (4, 28, 28, 192, 320, 3, 3, 1, 1),
    (2, 12, 12, 16, 8, 1, 1, 4, 0),
    (2, 30, 30, 48, 136, 1, 1, 3, 0),
]


def _cfg(shape, epi=EPI_NONE, seed=7):
    return small_config(*shape, epilogue=epi, seed=seed)


@pytest.fixture(scope="module")
def small_refs():
    out = {}
    for shape in SMALL:
        for epi in (EPI_NONE, EPI_DRELU, EPI_DHARDSWISH):
            cfg = _cfg(shape, epi)
            inp = make_inputs(cfg)
            out[(shape, epi)] = (cfg, inp, ref_full(cfg, inp))
    return out


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_small_every_config(small_refs, shape):
    cfg, inp, ref = small_refs[(shape, EPI_NONE)]
    for cid in range(cb.conv2d_dgrad_num_configs()):
        note(f"small {shape} config {cid} {cb.conv2d_dgrad_config_name(cid)}")
        assert_close(run(cfg, inp, config_id=cid), ref, f"{shape} config {cid}")


@pytest.mark.parametrize("epi", [EPI_DRELU, EPI_DHARDSWISH])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_small_epilogues(small_refs, shape, epi):
    cfg, inp, ref = small_refs[(shape, epi)]
    note(f"small {shape} epilogue {epi} (selected config)")
    assert_close(run(cfg, inp), ref, f"{shape} epi {epi}")
    note(f"small {shape} epilogue {epi} config 0")
    assert_close(run(cfg, inp, config_id=0), ref, f"{shape} epi {epi} config 0")


def _wide_configs():
    return [cid for cid in range(cb.conv2d_dgrad_num_configs()) if cb.conv2d_dgrad_config_name(cid).endswith("w")]


# Shapes without zero phases (the one-tile-per-workgroup kernel runs them
# itself): ragged M, C and K, several phases, a pixel tile past the end, a
# single pixel, 5x5 and 7x7 filters.
WIDE_SHAPES = [
    (2, 15, 13, 136, 72, 3, 3, 1, 1),
    (2, 17, 16, 64, 128, 3, 3, 2, 1),
    (2, 9, 9, 16, 16, 5, 5, 3, 2),
    (1, 14, 14, 264, 56, 1, 1, 1, 0),
    (1, 5, 5, 8, 8, 7, 7, 1, 3),
    (1, 1, 1, 8, 8, 1, 1, 1, 0),
    (4, 28, 28, 192, 320, 3, 3, 1, 1),
    (3, 7, 7, 512, 136, 3, 3, 1, 1),
]


@pytest.mark.parametrize("epi", [EPI_NONE, EPI_DRELU, EPI_DHARDSWISH])
@pytest.mark.parametrize("shape", WIDE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_wide_kernel_every_epilogue(shape, epi):
    cfg = _cfg(shape, epi, seed=9)
    inp = make_inputs(cfg)
    ref = ref_full(cfg, inp)
    for cid in _wide_configs():
        note(f"wide kernel {shape} epilogue {epi} config {cid}")
        assert_close(run(cfg, inp, config_id=cid), ref, f"{shape} epi {epi} config {cid}")


def _halo_configs():
    return [cid for cid in range(cb.conv2d_dgrad_num_configs()) if cb.conv2d_dgrad_config_name(cid).endswith("h")]


# 3x3 stride-1 layers with pad 1 (P = H, Q = W; the halo kernel runs them
# itself): ragged M, C and K; one k chunk (K <= 64, and K = 64 exactly), two,
# three, four and five chunks (the chunk walk pairs chunks after one alone
# when their count before the last is odd); a pixel tile past the end; a
# single pixel, whose taps all but one leave the image; and the widest halo
# the buffers hold (W = 67: 256 + 2*68 rows).
HALO_SHAPES = [
    (2, 15, 13, 136, 72, 3, 3, 1, 1),
    (4, 28, 28, 192, 320, 3, 3, 1, 1),
    (3, 7, 7, 512, 136, 3, 3, 1, 1),
    (2, 10, 10, 16, 40, 3, 3, 1, 1),
    (1, 5, 5, 8, 64, 3, 3, 1, 1),
    (1, 9, 9, 64, 128, 3, 3, 1, 1),
    (1, 6, 67, 24, 24, 3, 3, 1, 1),
    (1, 1, 1, 8, 8, 3, 3, 1, 1),
    (2, 3, 40, 264, 200, 3, 3, 1, 1),
]


@pytest.mark.parametrize("epi", [EPI_NONE, EPI_DRELU, EPI_DHARDSWISH])
@pytest.mark.parametrize("shape", HALO_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_halo_kernel_every_epilogue(shape, epi):
    cfg = _cfg(shape, epi, seed=11)
    inp = make_inputs(cfg)
    ref = ref_full(cfg, inp)
    for cid in _halo_configs():
        note(f"halo kernel {shape} epilogue {epi} config {cid}")
        assert_close(run(cfg, inp, config_id=cid), ref, f"{shape} epi {epi} config {cid}")


@pytest.mark.parametrize("shape", [(2, 15, 13, 136, 72, 3, 3, 1, 1), (1, 6, 67, 24, 24, 3, 3, 1, 1),
                                   (2, 3, 40, 264, 200, 3, 3, 1, 1)],
                         ids=lambda s: "x".join(map(str, s)))
def test_halo_kernel_integer_bit_exact(shape):
    """Integer inputs (every product and partial sum exact in fp32): the
    halo kernel's output equals the rounded oracle bit for bit, so no tap
    reads a wrong row, a stale halo buffer or a nonzero padding row."""
    cfg = _cfg(shape, EPI_NONE, seed=12)
    inp = integer_inputs(cfg, lo=-3, hi=3, seed=13)
    ref16 = oracle.round_to_half(ref_full(cfg, inp))
    for cid in _halo_configs():
        note(f"halo kernel integer {shape} config {cid}")
        _bits_equal(run(cfg, inp, config_id=cid), ref16)


def _halo1_configs():
    return [cid for cid in range(cb.conv2d_dgrad_num_configs()) if cb.conv2d_dgrad_config_name(cid).endswith("s")]


# The single-chunk halo kernel (3x3, stride 1, pad 1, K <= 64, all loads at
# once): ragged M, C and K (K of 8, 24, 40 and 64), images down to 1x1 and 5
# wide, one up to 67 wide (the widest halo the buffer takes at 128 pixels is
# 103 wide), one and many tiles.
HALO1_SHAPES = [
    (2, 15, 13, 136, 40, 3, 3, 1, 1),
    (4, 28, 28, 64, 64, 3, 3, 1, 1),
    (3, 7, 7, 72, 64, 3, 3, 1, 1),
    (2, 10, 10, 16, 24, 3, 3, 1, 1),
    (1, 5, 5, 8, 8, 3, 3, 1, 1),
    (1, 6, 67, 24, 64, 3, 3, 1, 1),
    (1, 1, 1, 8, 8, 3, 3, 1, 1),
    (2, 3, 103, 200, 56, 3, 3, 1, 1),
    (8, 56, 56, 64, 64, 3, 3, 1, 1),
]


@pytest.mark.parametrize("shape", HALO1_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_halo1_kernel(shape):
    cfg = _cfg(shape, EPI_NONE, seed=18)
    inp = make_inputs(cfg)
    ref = ref_full(cfg, inp)
    for cid in _halo1_configs():
        note(f"single-chunk halo kernel {shape} config {cid}")
        assert_close(run(cfg, inp, config_id=cid), ref, f"{shape} config {cid}")


@pytest.mark.parametrize("shape", [(2, 15, 13, 136, 40, 3, 3, 1, 1), (1, 6, 67, 24, 64, 3, 3, 1, 1),
                                   (8, 56, 56, 64, 64, 3, 3, 1, 1)],
                         ids=lambda s: "x".join(map(str, s)))
def test_halo1_kernel_integer_bit_exact(shape):
    """Integer inputs: the single-chunk halo kernel's output equals the
    rounded oracle bit for bit (no tap reads a wrong row, a padding row or
    channels past K)."""
    cfg = _cfg(shape, EPI_NONE, seed=19)
    inp = integer_inputs(cfg, lo=-3, hi=3, seed=20)
    ref16 = oracle.round_to_half(ref_full(cfg, inp))
    for cid in _halo1_configs():
        note(f"single-chunk halo kernel integer {shape} config {cid}")
        _bits_equal(run(cfg, inp, config_id=cid, repeat=2), ref16)


# The same kernel with K above 64, split by k chunk: one workgroup per tile
# and chunk, the partial sums in the workspace, the last chunk to arrive adds
# them in chunk order. 2, 4 and 8 chunks, a ragged last chunk (8 channels),
# ragged C and M, the suite's N=1 layer; without a workspace the host runs
# these layers on the plain kernel of the same tile.
HALO1_SPLIT_SHAPES = [
    (1, 14, 14, 256, 256, 3, 3, 1, 1),
    (2, 15, 13, 136, 200, 3, 3, 1, 1),
    (1, 7, 7, 512, 512, 3, 3, 1, 1),
    (3, 9, 11, 72, 128, 3, 3, 1, 1),
]


@pytest.mark.parametrize("shape", HALO1_SPLIT_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_halo1_split_kernel(shape):
    cfg = _cfg(shape, EPI_NONE, seed=25)
    inp = make_inputs(cfg)
    ref = ref_full(cfg, inp)
    for cid in _halo1_configs():
        note(f"split single-chunk halo kernel {shape} config {cid}")
        before = cb.conv2d_dgrad_streamk_launches()
        assert_close(run(cfg, inp, config_id=cid), ref, f"{shape} config {cid}")
        assert cb.conv2d_dgrad_streamk_launches() > before      # the chunks were split
        note(f"split single-chunk halo config {cid} without a workspace {shape}")
        assert_close(run(cfg, inp, config_id=cid, workspace=None), ref, f"{shape} config {cid}, no workspace")


@pytest.mark.parametrize("shape", [(1, 14, 14, 256, 256, 3, 3, 1, 1), (2, 15, 13, 136, 200, 3, 3, 1, 1)],
                         ids=lambda s: "x".join(map(str, s)))
def test_halo1_split_kernel_integer_bit_exact(shape):
    """Integer inputs: the chunk sums meet in a fixed order, so the split
    kernel's output equals the rounded oracle bit for bit, call after call."""
    cfg = _cfg(shape, EPI_NONE, seed=26)
    inp = integer_inputs(cfg, lo=-3, hi=3, seed=27)
    ref16 = oracle.round_to_half(ref_full(cfg, inp))
    for cid in _halo1_configs():
        note(f"split single-chunk halo kernel integer {shape} config {cid}")
        _bits_equal(run(cfg, inp, config_id=cid, repeat=3), ref16)


# Layers outside its class, asked for by its config id, run on the plain
# kernel of the same tile: K above 512 (more chunks than a split takes), a
# halo wider than the buffer, stride 2, 5x5, and fused epilogue factors.
@pytest.mark.parametrize("shape,epi", [((1, 7, 7, 64, 576, 3, 3, 1, 1), EPI_NONE),
                                       ((1, 4, 150, 64, 64, 3, 3, 1, 1), EPI_NONE),
                                       ((2, 14, 14, 64, 64, 3, 3, 2, 1), EPI_NONE),
                                       ((2, 9, 9, 64, 32, 5, 5, 1, 2), EPI_NONE),
                                       ((2, 15, 13, 136, 40, 3, 3, 1, 1), EPI_DRELU),
                                       ((2, 15, 13, 136, 40, 3, 3, 1, 1), EPI_DHARDSWISH)],
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_halo1_config_outside_its_layers(shape, epi):
    cfg = _cfg(shape, epi, seed=21)
    inp = make_inputs(cfg)
    ref = ref_full(cfg, inp)
    for cid in _halo1_configs():
        note(f"single-chunk halo config {cid} on {shape} epilogue {epi}")
        assert_close(run(cfg, inp, config_id=cid), ref, f"{shape} epi {epi} config {cid}")


def _pgemm_configs():
    return [cid for cid in range(cb.conv2d_dgrad_num_configs()) if cb.conv2d_dgrad_config_name(cid).endswith("p")]


# The persistent GEMM kernel (1x1, stride 1, no padding, K a multiple of 64):
# ragged M and C; 1, 4, 5 and 8 k steps; one tile per workgroup, and one to
# two and three to four tiles per workgroup (the slice requests cross tile
# boundaries, the first slice after an epilogue lets its stores stay in
# flight). The full-size 1x1 layer of the every-config tests walks six to
# seven.
PGEMM_SHAPES = [
    (2, 15, 13, 136, 256, 1, 1, 1, 0),
    (1, 7, 9, 64, 512, 1, 1, 1, 0),
    (3, 9, 11, 200, 64, 1, 1, 1, 0),
    (4, 28, 28, 192, 320, 1, 1, 1, 0),
    (32, 28, 28, 512, 64, 1, 1, 1, 0),
    (256, 14, 14, 512, 256, 1, 1, 1, 0),
    (128, 14, 14, 1024, 256, 1, 1, 1, 0),
]


@pytest.mark.parametrize("shape", PGEMM_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_pgemm_kernel(shape):
    cfg = _cfg(shape, EPI_NONE, seed=14)
    inp = make_inputs(cfg)
    ref = ref_full(cfg, inp)
    for cid in _pgemm_configs():
        note(f"persistent GEMM kernel {shape} config {cid}")
        assert_close(run(cfg, inp, config_id=cid), ref, f"{shape} config {cid}")


@pytest.mark.parametrize("shape", [(4, 28, 28, 192, 320, 1, 1, 1, 0), (32, 28, 28, 512, 64, 1, 1, 1, 0),
                                   (256, 14, 14, 512, 256, 1, 1, 1, 0)],
                         ids=lambda s: "x".join(map(str, s)))
def test_pgemm_kernel_integer_bit_exact(shape):
    """Integer inputs: the persistent GEMM kernel's output equals the rounded
    oracle bit for bit, two calls in a row (every tile of every round)."""
    cfg = _cfg(shape, EPI_NONE, seed=15)
    inp = integer_inputs(cfg, lo=-3, hi=3, seed=16)
    ref16 = oracle.round_to_half(ref_full(cfg, inp))
    for cid in _pgemm_configs():
        note(f"persistent GEMM kernel integer {shape} config {cid}")
        _bits_equal(run(cfg, inp, config_id=cid, repeat=2), ref16)


# Layers outside the GEMM kernel's class, asked for by its config id: the
# host runs the plain kernel of the same tile (a 3x3 stride-2 layer, a 1x1
# stride-2 layer with zero phases, a 1x1 layer with padding, K not a multiple
# of 64, fused epilogue factors).
@pytest.mark.parametrize("shape,epi", [((4, 28, 28, 96, 128, 3, 3, 2, 1), EPI_NONE),
                                       ((8, 28, 28, 128, 256, 1, 1, 2, 0), EPI_NONE),
                                       ((2, 9, 9, 64, 128, 1, 1, 1, 1), EPI_NONE),
                                       ((3, 9, 11, 200, 72, 1, 1, 1, 0), EPI_NONE),
                                       ((2, 15, 13, 136, 256, 1, 1, 1, 0), EPI_DRELU),
                                       ((2, 15, 13, 136, 256, 1, 1, 1, 0), EPI_DHARDSWISH)],
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_pgemm_config_outside_its_layers(shape, epi):
    cfg = _cfg(shape, epi, seed=17)
    inp = make_inputs(cfg)
    ref = ref_full(cfg, inp)
    for cid in _pgemm_configs():
        note(f"persistent GEMM config {cid} on {shape} epilogue {epi}")
        assert_close(run(cfg, inp, config_id=cid), ref, f"{shape} epi {epi} config {cid}")


def _pwide_configs():
    return [cid for cid in range(cb.conv2d_dgrad_num_configs()) if cb.conv2d_dgrad_config_name(cid).endswith("q")]


# The persistent four-wave kernel for strided layers without zero phases: 3x3
# stride 2 (four phases of 1, 2, 2 and 4 taps in one launch; even sizes take
# the phase-interleaved order, odd ones the phase-major one), ragged M, C
# and K, 5x5 stride 3 (phases with taps past the image), 3x3 stride 2 at 392
# tiles (workgroups walk one or two tiles, the slice requests crossing tile
# and phase boundaries).
PWIDE_SHAPES = [
    (4, 28, 28, 96, 128, 3, 3, 2, 1),
    (2, 27, 29, 72, 136, 3, 3, 2, 1),
    (2, 17, 19, 64, 80, 5, 5, 3, 2),
    (3, 14, 14, 200, 40, 3, 3, 2, 1),
    (64, 28, 28, 256, 64, 3, 3, 2, 1),
]


@pytest.mark.parametrize("shape", PWIDE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_pwide_kernel(shape):
    cfg = _cfg(shape, EPI_NONE, seed=14)
    inp = make_inputs(cfg)
    ref = ref_full(cfg, inp)
    for cid in _pwide_configs():
        note(f"persistent wide kernel {shape} config {cid}")
        assert_close(run(cfg, inp, config_id=cid), ref, f"{shape} config {cid}")


@pytest.mark.parametrize("shape", [(64, 28, 28, 256, 64, 3, 3, 2, 1), (2, 27, 29, 72, 136, 3, 3, 2, 1)],
                         ids=lambda s: "x".join(map(str, s)))
def test_pwide_kernel_integer_bit_exact(shape):
    """Integer inputs: the persistent four-wave kernel's output equals the
    rounded oracle bit for bit, two calls in a row (every tile of every
    phase)."""
    cfg = _cfg(shape, EPI_NONE, seed=15)
    inp = integer_inputs(cfg, lo=-3, hi=3, seed=16)
    ref16 = oracle.round_to_half(ref_full(cfg, inp))
    for cid in _pwide_configs():
        note(f"persistent wide kernel integer {shape} config {cid}")
        _bits_equal(run(cfg, inp, config_id=cid, repeat=2), ref16)


# Layers outside its class, asked for by its config id, run on the plain
# kernel of the same tile: stride 1, a strided layer with zero phases (1x1
# stride 2), and fused epilogue factors.
@pytest.mark.parametrize("shape,epi", [((2, 14, 14, 128, 96, 3, 3, 1, 1), EPI_NONE),
                                       ((8, 28, 28, 128, 256, 1, 1, 2, 0), EPI_NONE),
                                       ((4, 28, 28, 96, 128, 3, 3, 2, 1), EPI_DRELU),
                                       ((4, 28, 28, 96, 128, 3, 3, 2, 1), EPI_DHARDSWISH)],
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_pwide_config_outside_its_layers(shape, epi):
    cfg = _cfg(shape, epi, seed=17)
    inp = make_inputs(cfg)
    ref = ref_full(cfg, inp)
    for cid in _pwide_configs():
        note(f"persistent wide config {cid} on {shape} epilogue {epi}")
        assert_close(run(cfg, inp, config_id=cid), ref, f"{shape} epi {epi} config {cid}")


# Launches of a few rounds of tiles: the grid is trimmed to the fewest
# workgroups that keep the number of rounds (the persistent GEMM config:
# 259 tiles on 130 workgroups; the persistent strided config: 546 tiles of
# four phases on 184), and the workgroups past the last whole span of groups
# go to the XCDs in contiguous ranges, a tail that is not a multiple of
# eight. Every config, every element against the oracle.
@pytest.mark.parametrize("shape", [(337, 14, 14, 128, 64, 1, 1, 1, 0), (67, 30, 31, 200, 64, 3, 3, 1, 1),
                                   (160, 29, 30, 136, 64, 3, 3, 2, 1)],
                         ids=lambda s: "x".join(map(str, s)))
def test_trimmed_grids_every_config(shape):
    cfg = _cfg(shape, EPI_NONE, seed=23)
    inp = make_inputs(cfg)
    ref = ref_full(cfg, inp)
    for cid in range(cb.conv2d_dgrad_num_configs()):
        note(f"trimmed grid {shape} config {cid} {cb.conv2d_dgrad_config_name(cid)}")
        assert_close(run(cfg, inp, config_id=cid), ref, f"{shape} config {cid}")


# ---------------------------------------------------------------- full sizes

@pytest.mark.parametrize("idx", range(len(CONFIGS)), ids=[c.name for c in CONFIGS])
def test_measured_layer(idx):
    """Each measured layer at full size in the configuration the table picks
    (the one bench.py times), with and without a workspace: every element
    against the oracle. Each call after the first goes into a fresh
    NaN-filled dx, so the chosen configuration alone must write every element
    (the first call profiles every candidate into the same buffer)."""
    cfg = CONFIGS[idx]
    inp = make_inputs(cfg)
    ref = ref_full(cfg, inp)
    wsz = cb.conv2d_dgrad_workspace_size(cfg.N, cfg.H, cfg.W, cfg.C, cfg.K, cfg.R, cfg.S, cfg.stride, cfg.pad,
                                         cfg.epilogue)
    for ws in ("auto", None):
        note(f"measured layer {cfg.name} (table-selected config, workspace {ws})")
        gpu = run(cfg, inp, workspace=ws, repeat=2)
        assert_close(gpu, ref, f"{cfg.name} workspace {ws}")
        cid, cached = cb.conv2d_dgrad_query_config(cfg.N, cfg.H, cfg.W, cfg.C, cfg.K, cfg.R, cfg.S, cfg.stride,
                                                   cfg.pad, cfg.epilogue, with_workspace=ws is not None and wsz > 0)
        assert cached


@pytest.mark.parametrize("idx", range(2, len(CONFIGS)), ids=[c.name for c in CONFIGS[2:]])
def test_measured_layer_every_config(idx):
    """Every compiled tile configuration on the full-size batch-256 layers:
    every element against the oracle."""
    cfg = CONFIGS[idx]
    inp = make_inputs(cfg)
    ref = ref_full(cfg, inp)
    for cid in range(cb.conv2d_dgrad_num_configs()):
        note(f"measured layer {cfg.name} config {cid} {cb.conv2d_dgrad_config_name(cid)}")
        assert_close(run(cfg, inp, config_id=cid), ref, f"{cfg.name} config {cid}")


def _measured_integer_inputs(cfg, seed):
    """Integer dy, w in [-2, 2] (every product and partial sum an exact fp32
    integer; K*R*S*4 < 2^24) and, for the fused layer, z on hardswish' kinks
    and zero crossings, where g is exact in fp32."""
    return integer_inputs(cfg, lo=-2, hi=2, seed=seed)


@pytest.mark.parametrize("idx", [2, 3, 5], ids=[CONFIGS[i].name for i in (2, 3, 5)])
def test_measured_layer_integer_bit_exact(idx):
    """The full-size layers in the table-selected configuration (the
    persistent walks with several tiles per workgroup, cross-tile prefetch,
    companion zero stores and the phase-interleaved order), on integer
    inputs: every element bit-exact, each call into a fresh NaN-filled dx."""
    cfg = CONFIGS[idx]
    inp = _measured_integer_inputs(cfg, seed=300 + idx)
    ref16 = oracle.round_to_half(ref_full(cfg, inp))
    note(f"integer bit-exact measured layer {cfg.name} (table-selected config)")
    _bits_equal(run(cfg, inp, repeat=2), ref16)


def test_fused_layer_streamk_forced_bit_exact():
    """The fused stage-4 layer with the stream-K split forced in every
    configuration that has it: every element bit-exact on integer inputs, and
    the split taken."""
    cfg = CONFIGS[5]
    inp = _measured_integer_inputs(cfg, seed=305)
    ref16 = oracle.round_to_half(ref_full(cfg, inp))
    prev = cb.conv2d_dgrad_set_streamk(1)
    try:
        for cid in range(cb.conv2d_dgrad_num_configs()):
            name = cb.conv2d_dgrad_config_name(cid)
            if name == "256x64x64/4x1" or name.endswith(("w", "h", "p", "s", "q")):
                continue   # no stream-K variant
            before = cb.conv2d_dgrad_streamk_launches()
            note(f"fused layer, stream-K forced, config {cid} {name}")
            _bits_equal(run(cfg, inp, config_id=cid), ref16)
            assert cb.conv2d_dgrad_streamk_launches() > before, f"{name}: the split was not taken"
    finally:
        cb.conv2d_dgrad_set_streamk(prev)


def test_downsample_zero_pattern():
    """1x1 stride 2: three of the four lattices are exact zeros."""
    cfg = CONFIGS[3]
    inp = make_inputs(cfg)
    note("zero pattern, 1x1 stride 2 at full size")
    gpu = run(cfg, inp)
    assert np.all(gpu[:, 1::2, :, :] == 0) and np.all(gpu[:, :, 1::2, :] == 0)
    assert np.count_nonzero(gpu[:, ::2, ::2, :]) > 0.99 * gpu[:, ::2, ::2, :].size


# ---------------------------------------------------------------- bit-exact cases

def _bits_equal(gpu, ref16):
    g = np.asarray(gpu, dtype=np.float16)
    assert not np.isnan(g).any()
    # +0 and -0 compare equal; everything else must be the same fp16 value
    assert np.array_equal(g, ref16), f"{np.sum(g != ref16)} elements differ"


@pytest.mark.parametrize("shape", [(2, 12, 12, 64, 64, 3, 3, 1, 1), (2, 13, 14, 72, 64, 3, 3, 2, 1),
                                   (1, 9, 9, 16, 136, 1, 1, 2, 0), (1, 10, 11, 24, 40, 5, 3, 3, 2),
                                   (2, 16, 18, 72, 64, 3, 3, 2, 1), (2, 18, 18, 16, 24, 3, 3, 3, 1)],
                         ids=lambda s: "x".join(map(str, s)))
def test_integer_inputs_bit_exact(shape):
    """Integer dy, w in [-8, 8]: every partial sum is an exact fp32 integer,
    and sums above 2048 exercise fp16 round-to-nearest-even. The last two
    shapes have 4 and 9 phases of equal lattice size, whose tiles run in the
    phase-interleaved order."""
    cfg = _cfg(shape)
    inp = integer_inputs(cfg, lo=-8, hi=8, seed=21)
    ref16 = oracle.round_to_half(ref_full(cfg, inp))
    for cid in range(cb.conv2d_dgrad_num_configs()):
        note(f"integer bit-exact {shape} config {cid}")
        _bits_equal(run(cfg, inp, config_id=cid), ref16)


def test_fp16_rounding_is_nearest_even():
    """1x1, stride 1, w = 1: dx = dy[...,0] + dy[...,1] = 2048 + {1,3,5,7}.
    fp16 spacing is 2 there, so 2049/2051/2053/2055 are exact ties that
    round-to-nearest-even sends to 2048/2052/2052/2056 (truncation would
    give 2048/2050/2052/2054)."""
    cfg = _cfg((1, 8, 8, 16, 8, 1, 1, 1, 0))
    rng = np.random.Generator(np.random.PCG64(24))
    dy = np.zeros((1, 8, 8, 8), np.float16)
    dy[..., 0] = 2048
    dy[..., 1] = rng.choice([1, 3, 5, 7], size=(1, 8, 8))
    w = np.zeros((8, 1, 1, 16), np.float16)
    w[0:2] = 1
    inp = {"dy": dy, "w": w, "z": None}
    note("fp16 rounding ties")
    gpu = run(cfg, inp)
    want = {2049: 2048, 2051: 2052, 2053: 2052, 2055: 2056}
    exact = 2048 + dy[..., 1].astype(np.float64)
    for v, r in want.items():
        sel = exact[0] == v
        assert np.all(gpu[0][sel] == r), v
    _bits_equal(gpu, oracle.round_to_half(ref_full(cfg, inp)))


@pytest.mark.parametrize("epi", [EPI_DRELU, EPI_DHARDSWISH])
def test_epilogue_ties_bit_exact(epi):
    """z at the kinks and zero crossings (-4, -3, -1.5, 0, 1.5, 3, 4), where
    g is exact in fp32: the fused result is bit-exact."""
    cfg = _cfg((2, 14, 14, 64, 32, 3, 3, 1, 1), epi)
    inp = integer_inputs(cfg, lo=-2, hi=2, seed=22)
    ref16 = oracle.round_to_half(ref_full(cfg, inp))
    note(f"epilogue ties epi {epi}")
    _bits_equal(run(cfg, inp), ref16)


@pytest.mark.parametrize("stride,pad", [(2, 1), (3, 1), (2, 0)])
def test_one_hot_footprints(stride, pad):
    """One nonzero dy element lands exactly on the taps p*s - pad + r."""
    cfg = _cfg((2, 11, 10, 16, 8, 3, 3, stride, pad))
    base = integer_inputs(cfg, lo=-4, hi=4, seed=23)
    positions = [(0, 0, 0, 0), (1, cfg.P - 1, cfg.Q - 1, 7), (0, cfg.P // 2, 1, 3), (1, 0, cfg.Q - 1, 5)]
    for (n, p, q, k) in positions:
        inp = {"dy": one_hot_dy(cfg, n, p, q, k), "w": base["w"], "z": None}
        ref = ref_full(cfg, inp)
        note(f"one-hot stride {stride} pad {pad} at {(n, p, q, k)}")
        gpu = run(cfg, inp)
        _bits_equal(gpu, oracle.round_to_half(ref))
        support = {(int(a), int(b)) for a, b in zip(*np.nonzero(np.any(gpu[n] != 0, axis=-1)))}
        want = {(p * stride - pad + r, q * stride - pad + t) for r in range(3) for t in range(3)
                if 0 <= p * stride - pad + r < cfg.H and 0 <= q * stride - pad + t < cfg.W}
        assert support <= want
        assert np.all(gpu[1 - n] == 0)


# ---------------------------------------------------------------- behaviour

def test_deterministic():
    cfg = CONFIGS[2]
    inp = make_inputs(cfg)
    note("determinism, strided 3x3 at full size")
    a = run(cfg, inp)
    b = run(cfg, inp)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_non_default_stream():
    import torch
    cfg = _cfg((2, 15, 13, 136, 72, 3, 3, 2, 1), EPI_DHARDSWISH)
    inp = make_inputs(cfg)
    s = torch.cuda.Stream()
    note("non-default stream")
    assert_close(run(cfg, inp, stream=s), ref_full(cfg, inp), "side stream")


def test_autotune_off_uses_heuristic():
    cfg = _cfg((1, 16, 16, 64, 64, 3, 3, 1, 1))
    inp = make_inputs(cfg)
    prev = cb.conv2d_dgrad_set_autotune(False)
    try:
        want, cached = cb.conv2d_dgrad_query_config(cfg.N, cfg.H, cfg.W, cfg.C, cfg.K, cfg.R, cfg.S,
                                                    cfg.stride, cfg.pad)
        assert not cached
        note("autotune off")
        assert_close(run(cfg, inp, workspace=None), ref_full(cfg, inp), "heuristic")
        got, cached = cb.conv2d_dgrad_query_config(cfg.N, cfg.H, cfg.W, cfg.C, cfg.K, cfg.R, cfg.S,
                                                   cfg.stride, cfg.pad)
        assert cached and got == want
    finally:
        cb.conv2d_dgrad_set_autotune(prev)


@pytest.mark.parametrize("with_ws", [False, True])
def test_fault_injection_falls_back_to_heuristic(with_ws):
    """With every profiled candidate failing, a new key keeps the shape
    heuristic's choice ("Get" after a failed "Find"), caches it, and the call
    still gives the oracle's result in every element."""
    cfg = _cfg((3, 19, 17, 72, 40, 3, 3, 1, 1), EPI_DHARDSWISH, seed=41)
    inp = make_inputs(cfg)
    want, cached = cb.conv2d_dgrad_query_config(cfg.N, cfg.H, cfg.W, cfg.C, cfg.K, cfg.R, cfg.S, cfg.stride,
                                                cfg.pad, cfg.epilogue, with_workspace=with_ws)
    assert not cached
    prev = cb.conv2d_dgrad_set_fault_inject(True)
    try:
        note(f"fault injection, workspace {with_ws}")
        gpu = run(cfg, inp, workspace="auto" if with_ws else None, repeat=2)
    finally:
        cb.conv2d_dgrad_set_fault_inject(prev)
    got, cached = cb.conv2d_dgrad_query_config(cfg.N, cfg.H, cfg.W, cfg.C, cfg.K, cfg.R, cfg.S, cfg.stride,
                                               cfg.pad, cfg.epilogue, with_workspace=with_ws)
    assert cached and got == want
    assert_close(gpu, ref_full(cfg, inp), "fault-injected tuning")


def test_first_calls_allocate_no_device_memory():
    """New problem keys (each profiled on its first call, split candidates
    included) change no byte of free device memory: the library allocates
    nothing; the workspace is the caller's."""
    import torch
    shapes = [(2, 15, 13, 136, 72, 3, 3, 1, 1), (1, 14, 14, 256, 256, 3, 3, 1, 1),
              (2, 17, 16, 64, 128, 3, 3, 2, 1), (4, 28, 28, 192, 320, 3, 3, 1, 1)]
    cases = []
    for i, shape in enumerate(shapes):
        cfg = _cfg(shape, seed=50 + i)
        d = {k: to_dev(v) for k, v in make_inputs(cfg).items()}
        dx = torch.empty((cfg.N, cfg.H, cfg.W, cfg.C), dtype=torch.float16, device="cuda")
        x = torch.zeros((cfg.N, cfg.H, cfg.W, cfg.C), dtype=torch.float16, device="cuda")
        dw = torch.empty((cfg.K, cfg.R, cfg.S, cfg.C), dtype=torch.float32, device="cuda")
        ws = cb.workspace(1 << 26)
        cases.append((cfg, d, dx, x, dw, ws))

    def calls(cfg, d, dx, x, dw, ws):
        cb.dgrad(d["dy"], d["w"], cfg.H, cfg.W, cfg.stride, cfg.pad, out=dx, workspace=ws)
        cb.dgrad(d["dy"], d["w"], cfg.H, cfg.W, cfg.stride, cfg.pad, out=dx)
        cb.wgrad(d["dy"], x, cfg.R, cfg.S, cfg.stride, cfg.pad, out=dw, workspace=ws)
        cb.wgrad(d["dy"], x, cfg.R, cfg.S, cfg.stride, cfg.pad, out=dw)
        torch.cuda.synchronize()

    # the first case loads the code object and creates the runtime's own state
    note("allocation check: warm-up key")
    calls(*cases[0])
    torch.cuda.empty_cache()
    free0, _ = torch.cuda.mem_get_info()
    for case in cases[1:]:
        cfg = case[0]
        note(f"allocation check: new key {cfg.N, cfg.H, cfg.W, cfg.C, cfg.K, cfg.stride}")
        calls(*case)
        torch.cuda.empty_cache()
        free1, _ = torch.cuda.mem_get_info()
        assert free1 == free0, f"free device memory changed by {free0 - free1} bytes"


# ---------------------------------------------------------------- maximum sizes

def _int8_inputs(cfg, seed):
    """Small-integer dy and w drawn as int8 (host memory stays near the tensor
    size): every product and partial sum is an exact fp16/fp32 integer."""
    rng = np.random.Generator(np.random.PCG64(seed))
    dy = rng.integers(-2, 3, size=(cfg.N, cfg.P, cfg.Q, cfg.K), dtype=np.int8).astype(np.float16)
    w = rng.integers(-2, 3, size=(cfg.K, cfg.R, cfg.S, cfg.C), dtype=np.int8).astype(np.float16)
    return {"dy": dy, "w": w, "z": None}


def _compare_in_row_chunks(cfg, inp, gpu, bit_exact, pixels_per_chunk=1 << 16):
    """Every pixel row of gpu against the oracle, computed chunk by chunk so
    that host memory stays near the tensor size."""
    flat = gpu.reshape(-1, cfg.C)
    npix = flat.shape[0]
    for p0 in range(0, npix, pixels_per_chunk):
        rows = np.arange(p0, min(npix, p0 + pixels_per_chunk), dtype=np.int64)
        ref = ref_rows(cfg, inp, rows)
        if bit_exact:
            _bits_equal(flat[rows], oracle.round_to_half(ref))
        else:
            assert_close(flat[rows], ref, f"{cfg.name} pixels {p0}..")


# One tensor just below the 2^30-element limit in each case, so byte offsets,
# the last pixels and (for 1x1 stride 2) the companion zero stores reach the
# top of the 32-bit offset range.
MAX_SHAPES = [
    ("dx_1x1_s1", (63, 128, 128, 1024, 64, 1, 1, 1, 0)),       # dx 1,056,964,608 elements
    ("dy_1x1_s1", (63, 128, 128, 64, 1024, 1, 1, 1, 0)),       # dy 1,056,964,608 elements
    ("dx_3x3_s2", (40, 448, 448, 128, 64, 3, 3, 2, 1)),        # dx 1,027,604,480 elements, 4 phases
    ("dx_1x1_s2", (20, 448, 448, 256, 64, 1, 1, 2, 0)),        # dx 1,027,604,480 elements, 3 zero phases
]


@pytest.mark.parametrize("name,shape", MAX_SHAPES, ids=[n for n, _ in MAX_SHAPES])
def test_maximum_sizes_bit_exact(name, shape):
    """Every element bit-exact on small-integer inputs."""
    cfg = small_config(*shape, name=name)
    assert max(cfg.N * cfg.P * cfg.Q * cfg.K, cfg.N * cfg.H * cfg.W * cfg.C) < 2 ** 30
    inp = _int8_inputs(cfg, seed=17)
    note(f"maximum size {name} {shape}")
    gpu = run(cfg, inp)
    if cfg.stride == 2 and cfg.R == 1:    # the three zero lattices, everywhere
        assert not np.any(gpu[:, 1::2, :, :]) and not np.any(gpu[:, :, 1::2, :])
    _compare_in_row_chunks(cfg, inp, gpu, bit_exact=True)


# The persistent GEMM kernel ("p") and the single-chunk halo kernel ("s"),
# asked for by config id, on dx tensors just below the 2^30-element limit, so
# their dx byte offsets reach the top of the 32-bit range: bit-exact on small
# integers on the first and last pixel rows and a seeded sample between them
# (the whole 3x3 tensor would keep the oracle busy for minutes), and no
# element left unwritten.
MAX_NEW_KERNELS = [("p", (63, 128, 128, 1024, 64, 1, 1, 1, 0)), ("s", (100, 100, 100, 1024, 64, 3, 3, 1, 1))]


@pytest.mark.parametrize("suffix,shape", MAX_NEW_KERNELS, ids=[s for s, _ in MAX_NEW_KERNELS])
def test_new_kernels_at_maximum_offsets(suffix, shape):
    cfg = small_config(*shape, name=f"max_{suffix}")
    npix = cfg.N * cfg.H * cfg.W
    assert npix * cfg.C < 2 ** 30 and npix * cfg.C > 2 ** 29
    ids = [c for c in range(cb.conv2d_dgrad_num_configs()) if cb.conv2d_dgrad_config_name(c).endswith(suffix)]
    assert ids
    inp = _int8_inputs(cfg, seed=23)
    rng = np.random.Generator(np.random.PCG64(24))
    rows = np.unique(np.concatenate([np.arange(0, 2048), np.arange(npix - 8192, npix),
                                     rng.integers(0, npix, size=4096)])).astype(np.int64)
    ref16 = oracle.round_to_half(ref_rows(cfg, inp, rows))
    for cid in ids:
        note(f"maximum offsets, config {cid} {cb.conv2d_dgrad_config_name(cid)} {shape}")
        gpu = run(cfg, inp, config_id=cid)
        assert not np.isnan(gpu).any()
        _bits_equal(gpu.reshape(npix, cfg.C)[rows], ref16)
        del gpu


# ResNet-50 dgrad layers at batch 256 beyond the measured suite (dx channels C,
# dy channels K): the stage-2/3/4 3x3 convolutions, the stage-4 strided 3x3
# and a 1x1 expansion, each with one of the epilogues.
RESNET50_N256 = [
    ("stage2_3x3", (256, 56, 56, 64, 64, 3, 3, 1, 1), EPI_DHARDSWISH),
    ("stage2_3x3_plain", (256, 56, 56, 64, 64, 3, 3, 1, 1), EPI_NONE),
    ("stage3_3x3", (256, 28, 28, 128, 128, 3, 3, 1, 1), EPI_DRELU),
    ("stage4_3x3", (256, 14, 14, 256, 256, 3, 3, 1, 1), EPI_NONE),
    ("stage4_3x3_s2", (256, 28, 28, 256, 256, 3, 3, 2, 1), EPI_DHARDSWISH),
    ("stage2_1x1_expand", (256, 56, 56, 64, 256, 1, 1, 1, 0), EPI_DRELU),
]


@pytest.mark.parametrize("name,shape,epi", RESNET50_N256, ids=[n for n, _, _ in RESNET50_N256])
def test_resnet50_batch256_layers(name, shape, epi):
    """Full-size layers in the table-selected configuration: every element
    against the oracle (the second call into a fresh NaN-filled dx)."""
    cfg = small_config(*shape, epilogue=epi, seed=17)
    inp = make_inputs(cfg)
    note(f"resnet50 batch-256 layer {name} {shape} epilogue {epi}")
    gpu = run(cfg, inp, repeat=2)
    assert_close(gpu, ref_full(cfg, inp), name)
