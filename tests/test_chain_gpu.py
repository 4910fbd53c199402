"""GPU parity of the fused chain of two dgrad steps (an RxS stride-1 dgrad,
the activation derivative, then the 1x1 dgrad in front of it) through the C
ABI against the fp64 oracle.

Tolerance, from the arithmetic: the kernel rounds t to fp16 after an fp32
sum, the oracle after an fp64 sum. The two t can land on neighbouring fp16
values when the sum sits next to a rounding midpoint, a difference of at
most one fp16 spacing, 2^-10 |t| (or 2^-24 for subnormal t). Each such
difference reaches dx multiplied by w2, so
    |gpu - ref| <= 1e-3 + 1e-2 |ref| + 2^-10 * sum_c |t_c| |w2[c, ci]|,
where the first two terms are the dgrad bound (final fp16 rounding and fp32
accumulation) and the sum is the oracle's magnitude output. With inputs in
{-1, 0, 1} and z chosen so that g(z) is 0, 1/2 or 1, every sum is exact in
fp32 and every t exact in fp16, and dx equals the oracle rounded to nearest
even bit for bit.
"""
import numpy as np
import pytest

import convolution_backward_amd as cb
import oracle
from workloads import CHAIN_BY_NAME, ChainConfig, integer_chain_inputs, make_chain_inputs
from tests.gpu_util import note, to_dev

pytestmark = pytest.mark.gpu

EPIS = (cb.EPI_NONE, cb.EPI_DRELU, cb.EPI_DHARDSWISH)

# (N, H, W, Cm, K, R, S, pad, C): several pixel tiles with a ragged last one,
# both resident widths (Cm <= 64 and Cm <= 128) with ragged Cm, ragged K and
# C, 1x1 and non-square filters, and a single pixel; stage-1 walks of nine
# and eighteen slices (the unrolled variants) and of other lengths.
SMALL = [
    (2, 14, 13, 64, 64, 3, 3, 1, 256),
    (1, 9, 11, 128, 32, 3, 3, 1, 136),
    (3, 7, 6, 72, 40, 3, 3, 1, 64),
    (2, 10, 9, 8, 16, 1, 1, 0, 24),
    (1, 12, 7, 40, 24, 5, 3, 2, 128),
    (2, 6, 8, 120, 72, 3, 3, 0, 200),
    (1, 1, 1, 16, 8, 1, 1, 0, 8),
    (1, 16, 16, 64, 136, 3, 3, 1, 384),
    (2, 10, 9, 48, 96, 3, 3, 1, 72),
]


def _cfg(shape, epi, seed=31):
    N, H, W, Cm, K, R, S, pad, C = shape
    return ChainConfig(name="small", N=N, H=H, W=W, Cm=Cm, K=K, R=R, S=S, pad=pad, C=C, epilogue=epi, seed=seed)


def run_chain(cfg, inp):
    import torch
    dx = torch.full((cfg.N, cfg.H, cfg.W, cfg.C), float("nan"), dtype=torch.float16, device="cuda")
    z = to_dev(inp["z"]) if inp["z"] is not None else None
    cb.dgrad_chain(to_dev(inp["dy"]), to_dev(inp["w1"]), z, to_dev(inp["w2"]), cfg.pad, cfg.epilogue, out=dx)
    torch.cuda.synchronize()
    return dx.cpu().numpy()


def _ref(cfg, inp, rows=None):
    return oracle.chain(inp["dy"], inp["w1"], inp["z"], inp["w2"], cfg.H, cfg.W, cfg.pad, cfg.epilogue,
                        rows=rows, with_abs=True)


def assert_chain_close(got, ref, mag, what):
    got = got.astype(np.float64)
    assert not np.isnan(got).any(), f"{what}: NaN in the output (an element was never written)"
    bound = 1e-3 + 1e-2 * np.abs(ref) + 2.0 ** -10 * mag
    err = np.abs(got - ref)
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} elements out of tolerance; "
                           f"worst error {err.max():.3g} at {np.unravel_index(np.argmax(err - bound), err.shape)}")


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_chain_small_every_epilogue(shape):
    for epi in EPIS:
        cfg = _cfg(shape, epi)
        inp = make_chain_inputs(cfg)
        note(f"chain small {shape} epilogue {epi}")
        ref, mag = _ref(cfg, inp)
        assert_chain_close(run_chain(cfg, inp), ref, mag, f"{shape} epilogue {epi}")


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_chain_integer_bit_exact(shape):
    for epi in (cb.EPI_DRELU, cb.EPI_DHARDSWISH):
        cfg = _cfg(shape, epi)
        inp = integer_chain_inputs(cfg)
        note(f"chain integer {shape} epilogue {epi}")
        ref = oracle.chain(inp["dy"], inp["w1"], inp["z"], inp["w2"], cfg.H, cfg.W, cfg.pad, epi)
        got = run_chain(cfg, inp)
        want = oracle.round_to_half(ref)
        assert np.array_equal(got.view(np.uint16), want.view(np.uint16)), \
            f"{int(np.sum(got.view(np.uint16) != want.view(np.uint16)))} elements differ"


def test_chain_matches_the_unfused_pair_on_integer_inputs():
    """The fused kernel equals this library's two separate dgrad calls (the
    second on the fp16 t the first stores), bit for bit where both are exact."""
    import torch
    cfg = _cfg((2, 14, 13, 64, 64, 3, 3, 1, 256), cb.EPI_DHARDSWISH)
    inp = integer_chain_inputs(cfg, seed=5)
    fused = run_chain(cfg, inp)
    t = cb.dgrad(to_dev(inp["dy"]), to_dev(inp["w1"]), cfg.H, cfg.W, 1, cfg.pad,
                 epilogue=cb.EPI_DHARDSWISH, z=to_dev(inp["z"]))
    w2 = to_dev(inp["w2"])
    dx = cb.dgrad(t.contiguous(), w2, cfg.H, cfg.W, 1, 0)
    torch.cuda.synchronize()
    assert np.array_equal(fused.view(np.uint16), dx.cpu().numpy().view(np.uint16))


def test_chain_with_workspace_chooses_a_path():
    """With a workspace that holds t, the first call times the fused kernel
    against the two-call pair and caches the faster; whichever runs, the
    result is bit-exact against the oracle on integer inputs (t is rounded to
    fp16 once on both paths), and a workspace too small for t keeps the
    fused kernel."""
    import torch
    for shape in [(2, 14, 13, 64, 64, 3, 3, 1, 256), (1, 9, 11, 128, 32, 3, 3, 1, 136)]:
        cfg = _cfg(shape, cb.EPI_DHARDSWISH, seed=41)
        inp = integer_chain_inputs(cfg, seed=13)
        want = oracle.round_to_half(oracle.chain(inp["dy"], inp["w1"], inp["z"], inp["w2"], cfg.H, cfg.W, cfg.pad,
                                                 cfg.epilogue))
        need = cb.conv2d_dgrad_chain_workspace_size(cfg.N, cfg.H, cfg.W, cfg.Cm, cfg.K, cfg.R, cfg.S, cfg.pad, cfg.C,
                                                    cfg.epilogue)
        assert need >= 65536 + 2 * cfg.N * cfg.H * cfg.W * cfg.Cm
        d = {k: to_dev(v) for k, v in inp.items()}
        for ws_bytes in (need, 65536 + 256):
            ws = cb.workspace(ws_bytes)
            for rep in range(2):   # the first call may time both paths into dx; the second runs the choice
                dx = torch.full((cfg.N, cfg.H, cfg.W, cfg.C), float("nan"), dtype=torch.float16, device="cuda")
                note(f"chain with workspace {ws_bytes} {shape} call {rep}")
                cb.dgrad_chain(d["dy"], d["w1"], d["z"], d["w2"], cfg.pad, cfg.epilogue, out=dx, workspace=ws)
                torch.cuda.synchronize()
                got = dx.cpu().numpy()
                assert np.array_equal(got.view(np.uint16), want.view(np.uint16)), f"{shape} ws {ws_bytes}"
        pair, cached = cb.conv2d_dgrad_chain_query(cfg.N, cfg.H, cfg.W, cfg.Cm, cfg.K, cfg.R, cfg.S, cfg.pad, cfg.C,
                                                   cfg.epilogue)
        assert cached


def test_chain_deterministic():
    cfg = _cfg(SMALL[0], cb.EPI_DHARDSWISH)
    inp = make_chain_inputs(cfg)
    a = run_chain(cfg, inp)
    b = run_chain(cfg, inp)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def _check_in_row_chunks(cfg, inp, got, bit_exact=False, pixels_per_chunk=1 << 17):
    """Every pixel row of dx against the oracle, computed chunk by chunk so
    that host memory stays bounded."""
    flat = got.reshape(-1, cfg.C)
    M = flat.shape[0]
    for p0 in range(0, M, pixels_per_chunk):
        rows = np.arange(p0, min(M, p0 + pixels_per_chunk), dtype=np.int64)
        if bit_exact:
            ref = oracle.chain(inp["dy"], inp["w1"], inp["z"], inp["w2"], cfg.H, cfg.W, cfg.pad, cfg.epilogue,
                               rows=rows)
            want = oracle.round_to_half(ref)
            assert np.array_equal(flat[rows].view(np.uint16), want.view(np.uint16)), f"pixels {p0}.. differ"
        else:
            ref, mag = _ref(cfg, inp, rows=rows)
            assert_chain_close(flat[rows], ref, mag, f"{cfg.name} pixels {p0}..")


@pytest.mark.parametrize("name", sorted(CHAIN_BY_NAME))
def test_chain_full_size(name):
    """The full-size chains: every element of dx against the oracle."""
    cfg = CHAIN_BY_NAME[name]
    inp = make_chain_inputs(cfg)
    note(f"chain full size {name}")
    _check_in_row_chunks(cfg, inp, run_chain(cfg, inp))


def test_chain_maximum_size_integer():
    """dx just below 2^30 elements (the largest tensor the library admits):
    every element bit-exact, the last pixels included."""
    import torch
    cfg = ChainConfig(name="max", N=1023, H=32, W=32, Cm=64, K=8, R=3, S=3, pad=1, C=1024,
                      epilogue=cb.EPI_DRELU)
    assert cfg.N * cfg.H * cfg.W * cfg.C < 2 ** 30
    inp = integer_chain_inputs(cfg, seed=9)
    note("chain maximum size")
    dx = torch.full((cfg.N, cfg.H, cfg.W, cfg.C), float("nan"), dtype=torch.float16, device="cuda")
    cb.dgrad_chain(to_dev(inp["dy"]), to_dev(inp["w1"]), to_dev(inp["z"]), to_dev(inp["w2"]), cfg.pad,
                   cfg.epilogue, out=dx)
    got = dx.cpu().numpy()
    del dx
    torch.cuda.empty_cache()
    _check_in_row_chunks(cfg, inp, got, bit_exact=True)
