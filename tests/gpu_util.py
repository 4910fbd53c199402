"""Helpers for the GPU tests: move seeded inputs to the device, run the HIP
path through the C ABI, compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np

import convolution_backward_amd as cb
import oracle

# |gpu - ref| <= ATOL + RTOL * |ref|, elementwise (fp16 output, fp32 accumulate)
ATOL = 1e-3
RTOL = 1e-2


def note(msg: str):
    """Name the case before a GPU step, flushed, so a crash still says which."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(a):
    import torch
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run(cfg, inp, config_id=None, poison=True, stream=None):
    """dx from the HIP path (dx pre-filled with NaN so unwritten elements show)."""
    import torch
    dy, w, z = to_dev(inp["dy"]), to_dev(inp["w"]), to_dev(inp.get("z"))
    dx = torch.empty((cfg.N, cfg.H, cfg.W, cfg.C), dtype=torch.float16, device="cuda")
    if poison:
        dx.fill_(float("nan"))
    if stream is None:
        cb.dgrad(dy, w, cfg.H, cfg.W, cfg.stride, cfg.pad, cfg.epilogue, z, config_id=config_id, out=dx)
    else:
        with torch.cuda.stream(stream):
            cb.dgrad(dy, w, cfg.H, cfg.W, cfg.stride, cfg.pad, cfg.epilogue, z, config_id=config_id, out=dx)
        stream.synchronize()
    torch.cuda.synchronize()
    return dx.cpu().numpy()


def ref_full(cfg, inp):
    return oracle.dgrad(inp["dy"], inp["w"], cfg.H, cfg.W, cfg.stride, cfg.pad, cfg.epilogue, inp.get("z"))


def ref_rows(cfg, inp, rows):
    return oracle.dgrad(inp["dy"], inp["w"], cfg.H, cfg.W, cfg.stride, cfg.pad, cfg.epilogue, inp.get("z"),
                        rows=rows)


def assert_close(gpu, ref, what=""):
    g = np.asarray(gpu, dtype=np.float64)
    assert not np.isnan(g).any(), f"{what}: NaN in output (unwritten element?)"
    err = np.abs(g - ref)
    bound = ATOL + RTOL * np.abs(ref)
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements out of tolerance; "
                             f"first {idx.tolist()}: gpu {g[tuple(idx[0])]} ref {ref[tuple(idx[0])]}; "
                             f"max err {err.max():.3g}")


def sample_rows(cfg, count, seed=0):
    """Seeded pixel sample plus every corner/edge pixel of the first and last
    images (the halo cases)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    npix = cfg.N * cfg.H * cfg.W
    rows = set(rng.choice(npix, size=min(count, npix), replace=False).tolist())
    for n in {0, cfg.N - 1}:
        for h in {0, 1, cfg.H - 2, cfg.H - 1}:
            for x in {0, 1, cfg.W - 2, cfg.W - 1}:
                if 0 <= h < cfg.H and 0 <= x < cfg.W:
                    rows.add((n * cfg.H + h) * cfg.W + x)
    return np.array(sorted(rows), dtype=np.int64)
