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


def problem_workspace(cfg):
    """A zeroed workspace big enough for every split candidate of cfg (or None)."""
    return cb.dgrad_workspace(cfg.N, cfg.H, cfg.W, cfg.C, cfg.K, cfg.R, cfg.S, cfg.stride, cfg.pad, cfg.epilogue)


def run(cfg, inp, config_id=None, poison=True, stream=None, workspace="auto", repeat=1):
    """dx from the HIP path (dx pre-filled with NaN so unwritten elements show).

    workspace: "auto" (a zeroed workspace sized for the problem, so split
    launches are candidates), None (none: whole tiles only) or a tensor.
    repeat > 1 calls again that many times in total, each into a freshly
    NaN-filled dx, and returns the last result: after the first call has
    filled the tile-config table (profiling every candidate into dx), the
    chosen configuration alone must write every element."""
    import torch
    dy, w, z = to_dev(inp["dy"]), to_dev(inp["w"]), to_dev(inp.get("z"))
    ws = problem_workspace(cfg) if isinstance(workspace, str) else workspace
    dx = torch.empty((cfg.N, cfg.H, cfg.W, cfg.C), dtype=torch.float16, device="cuda")
    for _ in range(repeat):
        if poison:
            dx.fill_(float("nan"))
        if stream is None:
            cb.dgrad(dy, w, cfg.H, cfg.W, cfg.stride, cfg.pad, cfg.epilogue, z, config_id=config_id, out=dx,
                     workspace=ws)
        else:
            with torch.cuda.stream(stream):
                cb.dgrad(dy, w, cfg.H, cfg.W, cfg.stride, cfg.pad, cfg.epilogue, z, config_id=config_id, out=dx,
                         workspace=ws)
            stream.synchronize()
        torch.cuda.synchronize()
    out = dx.cpu().numpy()
    del dx, dy, w, z, ws
    return out


def ref_full(cfg, inp):
    return oracle.dgrad(inp["dy"], inp["w"], cfg.H, cfg.W, cfg.stride, cfg.pad, cfg.epilogue, inp.get("z"))


def ref_rows(cfg, inp, rows):
    return oracle.dgrad(inp["dy"], inp["w"], cfg.H, cfg.W, cfg.stride, cfg.pad, cfg.epilogue, inp.get("z"),
                        rows=rows)


def assert_close(gpu, ref, what="", chunk=1 << 24):
    """Every element: |gpu - ref| <= ATOL + RTOL*|ref| (in chunks, so that
    full-size tensors need little extra host memory)."""
    gf = np.asarray(gpu).reshape(-1)
    rf = np.asarray(ref).reshape(-1)
    assert gf.size == rf.size, f"{what}: {gf.size} elements against {rf.size}"
    nbad, first, worst = 0, None, 0.0
    for i in range(0, gf.size, chunk):
        g = gf[i:i + chunk].astype(np.float64)
        r = rf[i:i + chunk]
        if np.isnan(g).any():
            raise AssertionError(f"{what}: NaN in output (unwritten element?) at flat index "
                                 f"{i + int(np.argmax(np.isnan(g)))}")
        err = np.abs(g - r)
        bad = err > ATOL + RTOL * np.abs(r)
        worst = max(worst, float(err.max()) if err.size else 0.0)
        if bad.any():
            nbad += int(bad.sum())
            if first is None:
                j = int(np.argmax(bad))
                first = (i + j, float(g[j]), float(r[j]))
    if nbad:
        raise AssertionError(f"{what}: {nbad} of {gf.size} elements out of tolerance; first at flat index "
                             f"{first[0]}: gpu {first[1]} ref {first[2]}; max err {worst:.3g}")


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
