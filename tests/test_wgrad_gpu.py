"""GPU parity of wgrad (the filter gradient) through the C ABI against the
fp64 oracle.

Tolerance. Every fp16 x fp16 product is exact in fp32. The kernel adds them
in fp32: 16 at a time inside an MFMA, then along its slice range (at most a
few hundred sequential adds of partial sums per output), then the split
partials in order. Each add rounds by at most 2^-24 of a partial sum, which
is bounded by sum|dy * x|, so |gpu - ref| <= ~400 * 2^-24 * sum|dy * x|;
the test allows 1e-4 * sum|dy * x| + 1e-6 (4x that). Integer inputs make
every partial sum an exact fp32 integer: there the result is bit-exact.
"""
import numpy as np
import pytest

import convolution_backward_amd as cb
import oracle
from workloads import CONFIGS, integer_inputs, make_inputs, small_config
from tests.gpu_util import note, to_dev

pytestmark = pytest.mark.gpu

SMALL = [
    (2, 15, 13, 136, 72, 3, 3, 1, 1),
    (2, 17, 16, 64, 128, 3, 3, 2, 1),
    (3, 11, 12, 40, 24, 3, 3, 2, 0),
    (1, 20, 19, 32, 16, 1, 1, 2, 0),
    (2, 9, 9, 16, 16, 5, 5, 3, 2),
    (1, 14, 14, 264, 56, 1, 1, 1, 0),
    (2, 8, 10, 24, 8, 2, 4, 2, 1),
    (1, 1, 1, 8, 8, 1, 1, 1, 0),
    (1, 5, 5, 8, 8, 7, 7, 1, 3),
    (4, 28, 28, 192, 320, 3, 3, 1, 1),
]


def _x_like(cfg, seed, integer=False):
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (cfg.N, cfg.H, cfg.W, cfg.C)
    if integer:
        return rng.integers(-2, 3, size=shape).astype(np.float16)
    return rng.standard_normal(shape).astype(np.float16)


def run_wgrad(cfg, dy, x, config_id=None, splits=0, stream=None, workspace="auto", repeat=1):
    """dw from the HIP path, pre-filled with NaN. workspace: "auto" (sized for
    the problem's largest split), None (no workspace: one split per tile,
    written directly) or a tensor. With repeat > 1 each further call goes into
    a freshly NaN-filled dw (the first may profile candidates into it)."""
    import torch
    d_dy, d_x = to_dev(dy), to_dev(x)
    ws = (cb.wgrad_workspace(cfg.N, cfg.H, cfg.W, cfg.C, cfg.K, cfg.R, cfg.S, cfg.stride, cfg.pad)
          if isinstance(workspace, str) else workspace)
    dw = torch.empty((cfg.K, cfg.R, cfg.S, cfg.C), dtype=torch.float32, device="cuda")
    for _ in range(repeat):
        dw.fill_(float("nan"))
        if stream is None:
            cb.wgrad(d_dy, d_x, cfg.R, cfg.S, cfg.stride, cfg.pad, config_id=config_id, splits=splits, out=dw,
                     workspace=ws)
        else:
            with torch.cuda.stream(stream):
                cb.wgrad(d_dy, d_x, cfg.R, cfg.S, cfg.stride, cfg.pad, config_id=config_id, splits=splits, out=dw,
                         workspace=ws)
            stream.synchronize()
        torch.cuda.synchronize()
    return dw.cpu().numpy()


def assert_wgrad_close(got, ref, mag, what):
    g = np.asarray(got, dtype=np.float64)
    assert not np.isnan(g).any(), f"{what}: NaN (unwritten element?)"
    err = np.abs(g - ref)
    bound = 1e-4 * mag + 1e-6
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} out of tolerance; max err {err.max():.3g}, "
                           f"worst ratio {np.max(err / bound):.3g}")


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_wgrad_small_every_config(shape):
    cfg = small_config(*shape)
    dy = make_inputs(cfg)["dy"]
    x = _x_like(cfg, 41)
    ref, mag = oracle.wgrad(dy, x, cfg.R, cfg.S, cfg.stride, cfg.pad, with_abs=True)
    for cid in range(cb.conv2d_wgrad_num_configs()):
        for splits in (0, 1, 3):
            note(f"wgrad small {shape} config {cid} splits {splits}")
            assert_wgrad_close(run_wgrad(cfg, dy, x, cid, splits), ref, mag, f"{shape} config {cid} splits {splits}")
        note(f"wgrad small {shape} config {cid} without a workspace")
        assert_wgrad_close(run_wgrad(cfg, dy, x, cid, 0, workspace=None), ref, mag, f"{shape} config {cid} direct")


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_wgrad_integer_bit_exact(shape):
    cfg = small_config(*shape)
    dy = integer_inputs(cfg, lo=-2, hi=2, seed=42)["dy"]
    x = _x_like(cfg, 43, integer=True)
    ref = oracle.wgrad(dy, x, cfg.R, cfg.S, cfg.stride, cfg.pad)
    for cid in range(cb.conv2d_wgrad_num_configs()):
        note(f"wgrad integer {shape} config {cid}")
        got = run_wgrad(cfg, dy, x, cid, 0)
        assert not np.isnan(got).any()
        assert np.array_equal(got.astype(np.float64), ref), f"{np.sum(got != ref)} elements differ"


@pytest.mark.parametrize("idx", range(1, len(CONFIGS)), ids=[c.name for c in CONFIGS[1:]])
def test_wgrad_measured_layer(idx):
    """Each measured layer's shape at full size (table-selected config and
    split, with a workspace): every element of dw against the oracle (the
    second call into a fresh NaN-filled dw), and the same bits on a third."""
    cfg = CONFIGS[idx]
    dy = make_inputs(cfg)["dy"]
    x = _x_like(cfg, 44)
    note(f"wgrad measured layer {cfg.name}")
    got = run_wgrad(cfg, dy, x, repeat=2)
    ref, mag = oracle.wgrad(dy, x, cfg.R, cfg.S, cfg.stride, cfg.pad, with_abs=True)
    assert_wgrad_close(got, ref, mag, cfg.name)
    again = run_wgrad(cfg, dy, x)
    assert np.array_equal(got.view(np.uint32), again.view(np.uint32)), "wgrad changed between calls"


@pytest.mark.parametrize("idx", [1, 5], ids=[CONFIGS[1].name, CONFIGS[5].name])
def test_wgrad_measured_layer_without_workspace(idx):
    """Without a workspace each tile runs its whole reduction and writes dw
    directly: every element against the oracle."""
    cfg = CONFIGS[idx]
    dy = make_inputs(cfg)["dy"]
    x = _x_like(cfg, 48)
    note(f"wgrad measured layer {cfg.name} without a workspace")
    got = run_wgrad(cfg, dy, x, workspace=None, repeat=2)
    ref, mag = oracle.wgrad(dy, x, cfg.R, cfg.S, cfg.stride, cfg.pad, with_abs=True)
    assert_wgrad_close(got, ref, mag, f"{cfg.name} direct")


def test_wgrad_side_stream():
    import torch
    cfg = small_config(2, 15, 13, 136, 72, 3, 3, 2, 1)
    dy = make_inputs(cfg)["dy"]
    x = _x_like(cfg, 46)
    ref, mag = oracle.wgrad(dy, x, cfg.R, cfg.S, cfg.stride, cfg.pad, with_abs=True)
    note("wgrad side stream")
    assert_wgrad_close(run_wgrad(cfg, dy, x, stream=torch.cuda.Stream()), ref, mag, "side stream")


# One tensor just below the 2^30-element limit in each case (x of a 1x1 layer
# and of a strided 3x3 layer), so byte offsets near 2^31 and the last pixels
# of the reduction are exercised. Small-integer inputs keep every sum exact
# (each filter element sums at most ~2*10^6 products of magnitude <= 4,
# below 2^24), so every filter element must match the oracle bit for bit.
MAX_SHAPES = [
    ("x_1x1_s1", (63, 128, 128, 1024, 64, 1, 1, 1, 0)),       # x 1,056,964,608 elements
    ("x_3x3_s2", (40, 448, 448, 128, 64, 3, 3, 2, 1)),        # x 1,027,604,480 elements
]


def _int8(rng, shape):
    return rng.integers(-2, 3, size=shape, dtype=np.int8).astype(np.float16)


@pytest.mark.parametrize("name,shape", MAX_SHAPES, ids=[n for n, _ in MAX_SHAPES])
def test_wgrad_maximum_sizes_bit_exact(name, shape):
    cfg = small_config(*shape, name=name)
    assert cfg.N * cfg.H * cfg.W * cfg.C < 2 ** 30
    rng = np.random.Generator(np.random.PCG64(47))
    dy = _int8(rng, (cfg.N, cfg.P, cfg.Q, cfg.K))
    x = _int8(rng, (cfg.N, cfg.H, cfg.W, cfg.C))
    note(f"wgrad maximum size {name} {shape}")
    got = run_wgrad(cfg, dy, x)
    assert not np.isnan(got).any()
    ref = oracle.wgrad(dy, x, cfg.R, cfg.S, cfg.stride, cfg.pad)
    assert np.array_equal(got.astype(np.float64), ref), f"{np.sum(got != ref)} elements differ"
