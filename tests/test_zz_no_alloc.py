"""The no-allocation entry point (conv2d_dgrad_nhwc_noalloc) through the C
ABI: its output against conv2d_dgrad_nhwc_ws with a caller workspace (same
table entry, so the same tile configuration and split: the same bits) and
against the oracle, on two calls in a row, the second with a smaller input;
no device memory is allocated by either call after the first set-up; and a
problem whose split candidates need more than the static array is rejected
before anything is enqueued."""
import numpy as np
import pytest

import convolution_backward_amd as cb
from workloads import CONFIGS, make_inputs, small_config
from tests.gpu_util import assert_close, note, ref_full, to_dev

pytestmark = pytest.mark.gpu


def _both(cfg, inp):
    """(noalloc result, workspace-entry result), each into a NaN-filled dx."""
    import torch
    dy, w, z = to_dev(inp["dy"]), to_dev(inp["w"]), to_dev(inp.get("z"))
    dx_a = torch.full((cfg.N, cfg.H, cfg.W, cfg.C), float("nan"), dtype=torch.float16, device="cuda")
    dx_b = torch.full_like(dx_a, float("nan"))
    need = cb.conv2d_dgrad_workspace_size(cfg.N, cfg.H, cfg.W, cfg.C, cfg.K, cfg.R, cfg.S, cfg.stride, cfg.pad,
                                          cfg.epilogue)
    assert need <= cb.conv2d_dgrad_noalloc_max_bytes(), f"{cfg.name} needs {need} bytes"
    ws = cb.workspace(need)
    note(f"no-alloc entry {cfg.name}")
    cb.conv2d_dgrad_nhwc_noalloc(dy, w, dx_a, cfg.N, cfg.H, cfg.W, cfg.C, cfg.K, cfg.R, cfg.S, cfg.stride, cfg.pad,
                                 cfg.epilogue, z)
    note(f"workspace entry {cfg.name}")
    cb.conv2d_dgrad_nhwc_ws(dy, w, dx_b, cfg.N, cfg.H, cfg.W, cfg.C, cfg.K, cfg.R, cfg.S, cfg.stride, cfg.pad,
                            cfg.epilogue, z, ws)
    torch.cuda.synchronize()
    return dx_a.cpu().numpy(), dx_b.cpu().numpy()


def test_noalloc_matches_workspace_entry_on_two_calls():
    """The fused batch-256 layer (stream-K candidates in its table entry),
    then the smaller N=1 layer (split in its table entry): each equals the
    workspace entry point's output bit for bit and the oracle within the
    tolerance, with every element written."""
    for idx in (5, 0):
        cfg = CONFIGS[idx]
        inp = make_inputs(cfg)
        a, b = _both(cfg, inp)
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), f"{cfg.name}: entry points differ"
        assert_close(a, ref_full(cfg, inp), f"{cfg.name} no-alloc")


def test_noalloc_allocates_nothing():
    """After the first call on the device (which finds the array's address),
    calls on new problems leave free device memory unchanged."""
    import torch
    cases = []
    for i, shape in enumerate([(1, 14, 14, 256, 256, 3, 3, 1, 1), (2, 15, 13, 136, 72, 3, 3, 1, 1),
                               (3, 11, 12, 40, 24, 3, 3, 2, 0)]):
        cfg = small_config(*shape, seed=60 + i)
        d = {k: to_dev(v) for k, v in make_inputs(cfg).items()}
        dx = torch.empty((cfg.N, cfg.H, cfg.W, cfg.C), dtype=torch.float16, device="cuda")
        cases.append((cfg, d, dx))

    def call(cfg, d, dx):
        cb.conv2d_dgrad_nhwc_noalloc(d["dy"], d["w"], dx, cfg.N, cfg.H, cfg.W, cfg.C, cfg.K, cfg.R, cfg.S,
                                     cfg.stride, cfg.pad, cfg.epilogue, d["z"])
        torch.cuda.synchronize()

    note("no-alloc set-up call")
    call(*cases[0])
    torch.cuda.empty_cache()
    free0, _ = torch.cuda.mem_get_info()
    for case in cases[1:]:
        note(f"no-alloc new key {case[0].N, case[0].H, case[0].W, case[0].C, case[0].K, case[0].stride}")
        call(*case)
        torch.cuda.empty_cache()
        assert torch.cuda.mem_get_info()[0] == free0


def test_noalloc_rejects_problems_beyond_the_array():
    import torch
    cfg = small_config(256, 14, 14, 512, 512, 3, 3, 1, 1)
    need = cb.conv2d_dgrad_workspace_size(cfg.N, cfg.H, cfg.W, cfg.C, cfg.K, cfg.R, cfg.S, cfg.stride, cfg.pad)
    assert need > cb.conv2d_dgrad_noalloc_max_bytes()
    dy = torch.zeros((cfg.N, cfg.P, cfg.Q, cfg.K), dtype=torch.float16, device="cuda")
    w = torch.zeros((cfg.K, cfg.R, cfg.S, cfg.C), dtype=torch.float16, device="cuda")
    dx = torch.full((cfg.N, cfg.H, cfg.W, cfg.C), float("nan"), dtype=torch.float16, device="cuda")
    note("no-alloc rejection")
    with pytest.raises(cb.DgradError) as e:
        cb.conv2d_dgrad_nhwc_noalloc(dy, w, dx, cfg.N, cfg.H, cfg.W, cfg.C, cfg.K, cfg.R, cfg.S, cfg.stride, cfg.pad)
    assert e.value.code == cb.UNSUPPORTED and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.isnan(dx).all(), "a rejected call must enqueue nothing"
