"""Four host threads, each on a stream of its own with a workspace of its own,
call dgrad on problems the tile-config table has not seen, so every first
call profiles its candidates while the other threads' calls run. Each result
must match the oracle (every element), and each problem must end up in the
table. This is the concurrency the algorithm cache has to survive ("not good
for multi-threading", CUDA.jl PR #321, "Performance improvements by calling
cuDNN API"). Four streams stay within the box's four hardware queues."""
import threading

import numpy as np
import pytest

import convolution_backward_amd as cb
from workloads import EPI_DHARDSWISH, EPI_DRELU, EPI_NONE, make_inputs, small_config
from tests.gpu_util import assert_close, note, problem_workspace, ref_full, to_dev

pytestmark = pytest.mark.gpu

# shapes no other test uses (new table keys), strided and not, every epilogue
SHAPES = [
    ((2, 11, 13, 40, 24, 3, 3, 1, 1), EPI_NONE),
    ((1, 9, 9, 48, 56, 3, 3, 2, 1), EPI_DRELU),
    ((3, 7, 5, 24, 32, 1, 1, 1, 0), EPI_DHARDSWISH),
    ((2, 10, 10, 16, 40, 5, 5, 2, 2), EPI_NONE),
]


def test_four_threads_on_four_streams_profile_new_problems():
    import torch
    cfgs = [small_config(*shape, epilogue=epi, seed=61 + i) for i, (shape, epi) in enumerate(SHAPES)]
    inps = [make_inputs(c) for c in cfgs]
    refs = [ref_full(c, inp) for c, inp in zip(cfgs, inps)]
    with_ws = [cb.conv2d_dgrad_workspace_size(c.N, c.H, c.W, c.C, c.K, c.R, c.S, c.stride, c.pad, c.epilogue) > 0
               for c in cfgs]
    outs = [None] * len(cfgs)
    errors = []
    start = threading.Barrier(len(cfgs))

    def worker(i):
        try:
            cfg, inp = cfgs[i], inps[i]
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                dy, w, z = to_dev(inp["dy"]), to_dev(inp["w"]), to_dev(inp.get("z"))
                ws = problem_workspace(cfg)
                dx = torch.full((cfg.N, cfg.H, cfg.W, cfg.C), float("nan"), dtype=torch.float16, device="cuda")
                stream.synchronize()
                start.wait(timeout=60)
                for _ in range(2):   # the first call profiles, the second runs the cached choice
                    dx.fill_(float("nan"))
                    cb.dgrad(dy, w, cfg.H, cfg.W, cfg.stride, cfg.pad, cfg.epilogue, z, out=dx, workspace=ws)
                stream.synchronize()
                outs[i] = dx.cpu().numpy()
        except Exception as e:   # reported in the main thread
            errors.append((i, repr(e)))

    note("four host threads, four streams, four new problems")
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cfgs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    for i, (cfg, out) in enumerate(zip(cfgs, outs)):
        assert_close(out, refs[i], f"thread {i} {SHAPES[i]}")
        _, cached = cb.conv2d_dgrad_query_config(cfg.N, cfg.H, cfg.W, cfg.C, cfg.K, cfg.R, cfg.S, cfg.stride,
                                                 cfg.pad, cfg.epilogue, with_workspace=with_ws[i])
        assert cached, f"{SHAPES[i]} not cached"
