"""GPU parity of the stream-K split (a launch's reduction slices cut into equal
ranges, one per resident workgroup; the last share of a split tile adds the
others' fp32 partial sums). Forced on with conv2d_dgrad_set_streamk(1), it must
give the oracle's result: bit-exact on integer inputs (every partial sum is an
exact fp32 integer, so the order of the fix-up adds cannot matter), within the
fp16 tolerance on random inputs, and the same bits on every call."""
import numpy as np
import pytest

import convolution_backward_amd as cb
import oracle
from workloads import CONFIGS, EPI_DHARDSWISH, EPI_DRELU, EPI_NONE, integer_inputs, make_inputs, small_config
from tests.gpu_util import assert_close, note, ref_full, run

pytestmark = pytest.mark.gpu

# Launches without zero phases (stream-K never splits those): stride 1, and
# strided shapes where every lattice has taps. Ragged tails in M, C and K,
# one to four GEMM phases with different slice counts, tiles shorter than
# one workgroup's share and tiles split over many workgroups.
SHAPES = [
    (2, 15, 13, 136, 72, 3, 3, 1, 1),
    (2, 17, 16, 64, 128, 3, 3, 2, 1),     # four phases: 4, 2, 2, 1 taps
    (1, 14, 14, 264, 56, 1, 1, 1, 0),
    (2, 9, 9, 16, 16, 5, 5, 3, 2),        # nine phases
    (1, 5, 5, 8, 8, 7, 7, 1, 3),
    (1, 1, 1, 8, 8, 1, 1, 1, 0),          # one slice
    (4, 28, 28, 192, 320, 3, 3, 1, 1),
    (2, 13, 14, 72, 200, 3, 3, 2, 1),
]


def _streamk_configs():
    """Configurations with a split variant: all but 256x64/4x1 and the
    kernels without stream-K ("w", "h", "p", "s", "q")."""
    return [cid for cid in range(cb.conv2d_dgrad_num_configs())
            if cb.conv2d_dgrad_config_name(cid) != "256x64x64/4x1"
            and not cb.conv2d_dgrad_config_name(cid).endswith(("w", "h", "p", "s", "q"))]


@pytest.fixture
def forced_streamk():
    prev = cb.conv2d_dgrad_set_streamk(1)
    try:
        yield
    finally:
        cb.conv2d_dgrad_set_streamk(prev)


def _bits_equal(gpu, ref16, what):
    g = np.asarray(gpu, dtype=np.float16)
    assert not np.isnan(g).any(), f"{what}: unwritten element"
    assert np.array_equal(g, ref16), f"{what}: {np.sum(g != ref16)} elements differ"


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_streamk_integer_bit_exact(forced_streamk, shape):
    cfg = small_config(*shape)
    inp = integer_inputs(cfg, lo=-8, hi=8, seed=33)
    ref16 = oracle.round_to_half(ref_full(cfg, inp))
    for cid in _streamk_configs():
        before = cb.conv2d_dgrad_streamk_launches()
        note(f"stream-K integer {shape} config {cid} {cb.conv2d_dgrad_config_name(cid)}")
        _bits_equal(run(cfg, inp, config_id=cid), ref16, f"{shape} config {cid}")
        assert cb.conv2d_dgrad_streamk_launches() > before, "the split was not taken"


@pytest.mark.parametrize("epi", [EPI_NONE, EPI_DRELU, EPI_DHARDSWISH])
@pytest.mark.parametrize("shape", SHAPES[:4], ids=lambda s: "x".join(map(str, s)))
def test_streamk_random_inputs(forced_streamk, shape, epi):
    cfg = small_config(*shape, epilogue=epi, seed=11)
    inp = make_inputs(cfg)
    ref = ref_full(cfg, inp)
    for cid in _streamk_configs():
        note(f"stream-K random {shape} epi {epi} config {cid}")
        assert_close(run(cfg, inp, config_id=cid), ref, f"{shape} epi {epi} config {cid}")


def test_streamk_unsplit_config_runs_whole_tiles(forced_streamk):
    """The one configuration without a stream-K variant still runs (whole tiles)."""
    names = [cb.conv2d_dgrad_config_name(c) for c in range(cb.conv2d_dgrad_num_configs())]
    cid = names.index("256x64x64/4x1")
    cfg = small_config(*SHAPES[0])
    inp = integer_inputs(cfg, lo=-8, hi=8, seed=34)
    before = cb.conv2d_dgrad_streamk_launches()
    note(f"stream-K forced, config {cid} without a variant")
    _bits_equal(run(cfg, inp, config_id=cid), oracle.round_to_half(ref_full(cfg, inp)), "256x64")
    assert cb.conv2d_dgrad_streamk_launches() == before


@pytest.mark.parametrize("idx", [2, 5], ids=[CONFIGS[2].name, CONFIGS[5].name])
def test_streamk_measured_layer(forced_streamk, idx):
    """The strided 3x3 and fused layers at full size with the split forced:
    every element against the oracle, and the same bits on a second call.
    The fused layer's 196-784 tiles leave workgroups idle, so every
    configuration splits; the strided layer has more than four rounds of
    tiles per workgroup in every configuration, so no launch splits (a split
    cannot pay there) and whole tiles run."""
    cfg = CONFIGS[idx]
    inp = make_inputs(cfg)
    ref = ref_full(cfg, inp)
    for cid in _streamk_configs():
        name = cb.conv2d_dgrad_config_name(cid)
        note(f"stream-K measured layer {cfg.name} config {cid} {name}")
        before = cb.conv2d_dgrad_streamk_launches()
        a = run(cfg, inp, config_id=cid)
        assert (cb.conv2d_dgrad_streamk_launches() > before) == (idx == 5), name
        assert_close(a, ref, f"{cfg.name} config {cid}")
        b = run(cfg, inp, config_id=cid)
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), "stream-K result changed between calls"


def test_streamk_without_workspace_runs_whole_tiles(forced_streamk):
    """Forced split but no workspace: the launch runs whole tiles (nothing to
    hold the partial sums) and still gives the oracle's bits."""
    cfg = small_config(*SHAPES[0])
    inp = integer_inputs(cfg, lo=-8, hi=8, seed=36)
    before = cb.conv2d_dgrad_streamk_launches()
    note("stream-K forced without a workspace")
    _bits_equal(run(cfg, inp, config_id=0, workspace=None), oracle.round_to_half(ref_full(cfg, inp)), "no ws")
    assert cb.conv2d_dgrad_streamk_launches() == before


def test_streamk_workspace_shared_across_shapes(forced_streamk):
    """One workspace serves split launches of different shapes in turn (the
    counters each launch used are back at zero after it): bit-exact on
    integer inputs for every call, twice over."""
    import torch
    ws = cb.workspace(max(cb.conv2d_dgrad_workspace_size(*s[:9]) for s in SHAPES[:4]))
    for rnd in range(2):
        for shape in SHAPES[:4]:
            cfg = small_config(*shape)
            inp = integer_inputs(cfg, lo=-8, hi=8, seed=37)
            before = cb.conv2d_dgrad_streamk_launches()
            note(f"shared workspace round {rnd} {shape}")
            _bits_equal(run(cfg, inp, config_id=0, workspace=ws), oracle.round_to_half(ref_full(cfg, inp)),
                        f"{shape} round {rnd}")
            assert cb.conv2d_dgrad_streamk_launches() > before
    torch.cuda.synchronize()
    assert int(ws[:65536].count_nonzero()) == 0, "a counter was left nonzero"


def test_streamk_modes_agree_on_integer_inputs():
    """Never split, always split and the default give the same bits when every
    sum is exact; the default mode is restored."""
    cfg = small_config(*SHAPES[6])
    inp = integer_inputs(cfg, lo=-8, hi=8, seed=35)
    outs = []
    prev = cb.conv2d_dgrad_set_streamk(0)
    try:
        for mode in (0, 1, 2):
            cb.conv2d_dgrad_set_streamk(mode)
            note(f"stream-K mode {mode}")
            outs.append(run(cfg, inp, config_id=0).view(np.uint16))
    finally:
        cb.conv2d_dgrad_set_streamk(prev)
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
