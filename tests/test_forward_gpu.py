"""GPU parity of the forward layer with its fused bias + hardswish epilogue
through the C ABI against the fp64 oracle.

z and y are fp16 results of fp32 accumulation (each rounded once), so the
tolerance is dgrad's: |gpu - ref| <= 1e-3 + 1e-2 |ref|. With integer x, w
and bias every partial sum is an exact fp32 integer, and z equals the
oracle's value rounded to nearest even, bit for bit.
"""
import numpy as np
import pytest

import convolution_backward_amd as cb
import oracle
from workloads import CONFIGS, make_inputs, make_x, small_config
from tests.gpu_util import assert_close, note, to_dev

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


def _inputs(cfg, seed, integer=False):
    rng = np.random.Generator(np.random.PCG64(seed))
    if integer:
        x = rng.integers(-2, 3, size=(cfg.N, cfg.H, cfg.W, cfg.C)).astype(np.float16)
        w = rng.integers(-2, 3, size=(cfg.K, cfg.R, cfg.S, cfg.C)).astype(np.float16)
        b = rng.integers(-4, 5, size=cfg.K).astype(np.float16)
        return x, w, b
    x = make_x(cfg, seed=seed)
    w = make_inputs(cfg)["w"]
    b = (rng.standard_normal(cfg.K) * 0.5).astype(np.float16)
    return x, w, b


def run_forward(cfg, x, w, b, act, config_id=None, with_z=True):
    import torch
    P, Q = cfg.P, cfg.Q
    y = torch.full((cfg.N, P, Q, cfg.K), float("nan"), dtype=torch.float16, device="cuda")
    z = torch.full((cfg.N, P, Q, cfg.K), float("nan"), dtype=torch.float16, device="cuda") if with_z else None
    cb.forward(to_dev(x), to_dev(w), to_dev(b), cfg.stride, cfg.pad, act=act, with_z=with_z,
               config_id=config_id, out=y, z_out=z)
    torch.cuda.synchronize()
    return (None if z is None else z.cpu().numpy()), y.cpu().numpy()


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_forward_small_every_config(shape):
    cfg = small_config(*shape)
    x, w, b = _inputs(cfg, 51)
    for act in (cb.ACT_HARDSWISH, cb.ACT_NONE):
        zr, yr = oracle.forward(x, w, b, cfg.stride, cfg.pad, act=act)
        for cid in range(cb.conv2d_forward_num_configs()):
            note(f"forward small {shape} act {act} config {cid}")
            z, y = run_forward(cfg, x, w, b, act, cid)
            assert_close(z, zr, f"{shape} z act {act} config {cid}")
            assert_close(y, yr, f"{shape} y act {act} config {cid}")


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_forward_integer_bit_exact(shape):
    cfg = small_config(*shape)
    x, w, b = _inputs(cfg, 52, integer=True)
    zr, yr = oracle.forward(x, w, b, cfg.stride, cfg.pad, act=1)
    z16 = oracle.round_to_half(zr)
    for cid in range(cb.conv2d_forward_num_configs()):
        note(f"forward integer {shape} config {cid}")
        z, y = run_forward(cfg, x, w, b, 1, cid)
        assert not np.isnan(z).any()
        assert np.array_equal(z, z16), f"{np.sum(z != z16)} z elements differ"
        assert_close(y, yr, f"{shape} y config {cid}")


def test_forward_without_z():
    cfg = small_config(2, 15, 13, 136, 72, 3, 3, 2, 1)
    x, w, b = _inputs(cfg, 53)
    _, yr = oracle.forward(x, w, b, cfg.stride, cfg.pad, act=1)
    note("forward without z")
    z, y = run_forward(cfg, x, w, b, 1, with_z=False)
    assert z is None
    assert_close(y, yr, "y without z")


@pytest.mark.parametrize("idx", range(1, len(CONFIGS)), ids=[c.name for c in CONFIGS[1:]])
def test_forward_measured_layer(idx):
    """Each measured layer's shape at full size (table-selected config): every
    element of z and y against the oracle, and the same bits on a second
    call."""
    cfg = CONFIGS[idx]
    x, w, b = _inputs(cfg, 54)
    note(f"forward measured layer {cfg.name}")
    z, y = run_forward(cfg, x, w, b, 1)
    zr, yr = oracle.forward(x, w, b, cfg.stride, cfg.pad, act=1)
    assert_close(z, zr, f"{cfg.name} z")
    assert_close(y, yr, f"{cfg.name} y")
    del zr, yr
    z2, y2 = run_forward(cfg, x, w, b, 1)
    assert np.array_equal(y.view(np.uint16), y2.view(np.uint16))
    assert np.array_equal(z.view(np.uint16), z2.view(np.uint16))


# x just below the 2^30-element limit (1x1 and strided 3x3), small-integer
# inputs: z is exact and must equal the oracle's RNE fp16 value bit for bit
# in every element.
MAX_SHAPES = [
    ("x_1x1_s1", (63, 128, 128, 1024, 64, 1, 1, 1, 0)),       # x 1,056,964,608 elements
    ("x_3x3_s2", (40, 448, 448, 128, 64, 3, 3, 2, 1)),        # x 1,027,604,480 elements
]


@pytest.mark.parametrize("name,shape", MAX_SHAPES, ids=[n for n, _ in MAX_SHAPES])
def test_forward_maximum_sizes_bit_exact(name, shape):
    cfg = small_config(*shape, name=name)
    assert cfg.N * cfg.H * cfg.W * cfg.C < 2 ** 30
    rng = np.random.Generator(np.random.PCG64(57))
    x = rng.integers(-2, 3, size=(cfg.N, cfg.H, cfg.W, cfg.C), dtype=np.int8).astype(np.float16)
    w = rng.integers(-2, 3, size=(cfg.K, cfg.R, cfg.S, cfg.C), dtype=np.int8).astype(np.float16)
    b = rng.integers(-4, 5, size=cfg.K).astype(np.float16)
    note(f"forward maximum size {name} {shape}")
    z, y = run_forward(cfg, x, w, b, 1)
    npq = cfg.N * cfg.P * cfg.Q
    zf, yf = z.reshape(-1, cfg.K), y.reshape(-1, cfg.K)
    for p0 in range(0, npq, 1 << 20):    # chunks of output pixels keep host memory bounded
        rows = np.arange(p0, min(npq, p0 + (1 << 20)), dtype=np.int64)
        zr, yr = oracle.forward(x, w, b, cfg.stride, cfg.pad, act=1, rows=rows)
        assert np.array_equal(zf[rows], oracle.round_to_half(zr)), f"z differs in pixels {p0}.."
        assert_close(yf[rows], yr, f"{name} y pixels {p0}..")
