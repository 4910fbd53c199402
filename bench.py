#!/usr/bin/env python3
"""Throughput of the conv2d dgrad hot path on one MI355X.

A step is one pass over the measured ResNet-50 dgrad suite: the N=1 14x14
3x3 layer, the batch-8 stage-2 3x3 layer and the batch-256 layers (3x3
stride 2, the 1x1 stride-2 downsample, the 1x1 stride-1 reduce, and the
stage-4 3x3 with the fused hardswish' epilogue), each a single call of the C
ABI (with a caller-owned workspace) on synthetic seeded inputs already
resident in HBM. That covers every part of the path: the stride-phase plan,
zero phases, the MFMA implicit GEMM, the stream-K split, the fused epilogue
and the tile-config table (filled during warm-up).

Timing is cold, as the headline: before every layer call a read of a
512 MiB buffer evicts the layer's operands from L2 and the Infinity Cache
(a read, so that no dirty lines are left whose write-back would land inside
the timed kernel), and HIP events on the launch stream bracket the call
alone. value = useful FLOPs of the suite (2*N*P*Q*K*C*R*S per layer) / the
mean over the K steps of the summed per-layer times. The warm (back to
back) and end-to-end (host call + synchronise) timings are reported beside.

Prints one JSON line (see the fields at the end of main()).
Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--cpu-fraction F]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from workloads import CONFIGS, EPI_NAMES, make_inputs, make_x  # noqa: E402

SUITE = [0, 1, 2, 3, 4, 5]         # indices into CONFIGS
MFMA_PEAK_TFLOPS = 2500.0          # MI355X dense fp16 matrix-core peak
HBM_PEAK_GBS = 8000.0              # MI355X HBM3E peak
RIDGE = MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)   # FLOP per byte
METRIC = "dgrad TFLOP/s and % of fp16 MFMA peak, ResNet-50 layer shapes at N=8/256"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def roofline_of(cfg, seconds):
    flops = cfg.useful_flops()
    nbytes = cfg.algorithmic_bytes()
    ai = flops / nbytes
    if ai >= RIDGE:
        achieved = flops / seconds / 1e12
        return {"bound": "mfma", "achieved": achieved, "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / MFMA_PEAK_TFLOPS}
    achieved = nbytes / seconds / 1e9
    return {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS}


KERNEL_SOURCES = ("dgrad_kernels.hip", "dgrad_wide.hip", "dgrad_halo.hip", "dgrad_pgemm.hip", "dgrad_halo1.hip", "dgrad_pwide.hip", "kernel_common.h", "dgrad_internal.h")


def kernel_source_digest():
    """First 16 hex digits of the SHA-256 of the dgrad kernel sources, in order."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "convolution_backward_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key, tile_config):
    """HBM bytes per launch from the committed rocprofv3 counter summary, when
    it was taken on the current kernel source with the same tile config; else
    None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_digest():
        return None
    return t.get("by_tile_config", {}).get(kernel_key, {}).get(tile_config)


def kernel_of(tile_config):
    """The kernel template a tile-config name runs (its suffix, stream-K aside)."""
    base = tile_config.split("+")[0]
    kind = {"w": "dgrad_wide", "h": "dgrad_halo", "p": "dgrad_pgemm", "s": "dgrad_halo1", "q": "dgrad_pwide"}.get(base[-1], "dgrad_igemm")
    return f"{kind}<{base}>"


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inputs, fraction, suite, seed=99):
    """The oracle, untuned, on a seeded `fraction` of each layer's output
    pixels with every host thread, the full-suite time extrapolated by
    1/fraction per layer; plus one-thread runs of the two small layers."""
    import oracle
    lib = oracle.load()
    threads = oracle.max_threads(lib)
    total_t = 0.0
    rows_done = 0
    per_layer = []
    for idx in suite:
        cfg = CONFIGS[idx]
        npix = cfg.N * cfg.H * cfg.W
        k = max(1, int(round(npix * fraction)))
        rng = np.random.Generator(np.random.PCG64(seed + idx))
        rows = np.sort(rng.choice(npix, size=k, replace=False))
        inp = inputs[idx]
        t0 = time.perf_counter()
        oracle.dgrad(inp["dy"], inp["w"], cfg.H, cfg.W, cfg.stride, cfg.pad, cfg.epilogue, inp["z"],
                     rows=rows, lib=lib)
        dt = time.perf_counter() - t0
        total_t += dt * npix / k
        rows_done += k
        per_layer.append({"layer": cfg.name, "seconds": dt * npix / k,
                          "gflops": cfg.useful_flops() / (dt * npix / k) / 1e9})
        log(f"[cpu] {cfg.name}: {k} of {npix} pixels in {dt:.2f} s ({threads} threads)")
    one_thread = []
    for idx in (0, 1):
        if idx not in inputs:
            continue
        cfg, inp = CONFIGS[idx], inputs[idx]
        t0 = time.perf_counter()
        oracle.dgrad(inp["dy"], inp["w"], cfg.H, cfg.W, cfg.stride, cfg.pad, cfg.epilogue, inp["z"],
                     threads=1, lib=lib)
        dt = time.perf_counter() - t0
        one_thread.append({"layer": cfg.name, "seconds": dt, "gflops": cfg.useful_flops() / dt / 1e9})
        log(f"[cpu] {cfg.name}: every pixel on 1 thread in {dt:.2f} s")
    flops = sum(CONFIGS[i].useful_flops() for i in suite)
    return {"value": flops / total_t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"seeded {fraction:.0%} of the output pixels of each suite layer "
                      f"({rows_done} pixel rows, all channels, fp64, {threads} OpenMP threads); full-suite "
                      f"time extrapolated per layer by pixel count: {total_t:.2f} s per step",
            "layers": per_layer, "one_thread": one_thread}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100,
                    help="timed steps; each layer is launched once per step, cold")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-fraction", type=float, default=1.0,
                    help="share of each layer's pixels the oracle computes for cpu_baseline (0 skips it)")
    ap.add_argument("--warm-steps", type=int, default=50,
                    help="back-to-back steps timed as the warm figure (0 skips)")
    ap.add_argument("--e2e-reps", type=int, default=20,
                    help="host-timed calls per layer, each followed by a stream synchronisation (0 skips)")
    ap.add_argument("--wgrad-reps", type=int, default=10,
                    help="timed wgrad (filter gradient) calls per layer, after the dgrad timing (0 skips)")
    ap.add_argument("--forward-reps", type=int, default=10,
                    help="timed forward (conv + bias + hardswish) calls per layer shape, after the rest (0 skips)")
    ap.add_argument("--chain-reps", type=int, default=10,
                    help="timed calls of the fused two-step chain and of the unfused pair, after the rest (0 skips)")
    ap.add_argument("--only", default="",
                    help="comma-separated layer names: time only these (for profiler runs)")
    ap.add_argument("--flush", choices=("write", "read"), default="write",
                    help="how the cold mode evicts the caches before each layer call: a 512 MiB write "
                         "(the protocol's cache-flush write) or a 512 MiB read")
    ap.add_argument("--copy-calibrate-mb", type=float, default=0.0,
                    help="run only a plain device-to-device copy of this many MB, 10 times "
                         "(reference for the HBM byte counters) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); this library has no multi-GPU path: "
              "dgrad shards over the batch with no exchange, so N GPUs run N independent copies.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import convolution_backward_amd as cb
    cb.get_lib()    # fails loudly if the HIP library is not built
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibrate_mb > 0:
        n = int(args.copy_calibrate_mb * 1e6) // 2
        src = torch.empty(n, dtype=torch.float16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 2 * n, "copy_bytes_written": 2 * n, "launches": 10}), flush=True)
        return

    suite = SUITE
    if args.only:
        names = set(args.only.split(","))
        suite = [i for i in SUITE if CONFIGS[i].name in names]
        if not suite:
            print(f"--only matched no layer of {[CONFIGS[i].name for i in SUITE]}", file=sys.stderr)
            sys.exit(2)

    # ---- inputs, resident in HBM before timing; one workspace (zeroed once,
    # owned by PyTorch's allocator) serves every layer, as the C ABI allows
    host_inputs, layers = {}, []
    ws_bytes = 0
    for idx in suite:
        cfg = CONFIGS[idx]
        inp = make_inputs(cfg)
        host_inputs[idx] = inp
        d = {k: (None if v is None else torch.from_numpy(v).to(dev)) for k, v in inp.items()}
        d["dx"] = torch.empty((cfg.N, cfg.H, cfg.W, cfg.C), dtype=torch.float16, device=dev)
        layers.append((cfg, d))
        ws_bytes = max(ws_bytes, cb.conv2d_dgrad_workspace_size(cfg.N, cfg.H, cfg.W, cfg.C, cfg.K, cfg.R, cfg.S,
                                                                cfg.stride, cfg.pad, cfg.epilogue))
    workspace = cb.workspace(ws_bytes, dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)

    def one_layer(cfg, d):
        cb.conv2d_dgrad_nhwc_ws(d["dy"], d["w"], d["dx"], cfg.N, cfg.H, cfg.W, cfg.C, cfg.K, cfg.R, cfg.S,
                                cfg.stride, cfg.pad, cfg.epilogue, d["z"], workspace, stream.cuda_stream)

    # ---- warm-up (the first call per layer fills the tile-config table)
    for _ in range(args.warmup):
        for cfg, d in layers:
            one_layer(cfg, d)
    torch.cuda.synchronize()

    # ---- timed steps, cold: before each layer call a 512 MiB write (or read,
    # --flush read) evicts L2 (4 MiB per XCD) and the 256 MiB Infinity Cache;
    # the event pair on the launch stream brackets the layer call alone
    flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev).fill_(1.0)
    evict = (lambda: flush.fill_(0.0)) if args.flush == "write" else (lambda: flush.sum())
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in layers] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        for li, (cfg, d) in enumerate(layers):
            evict()
            ev[s][li][0].record(stream)
            one_layer(cfg, d)
            ev[s][li][1].record(stream)
    torch.cuda.synchronize()
    cold_wall = time.perf_counter() - t0
    step_ms = [sum(ev[s][li][0].elapsed_time(ev[s][li][1]) for li in range(len(layers))) for s in range(args.steps)]
    ms_per_step = float(np.mean(step_ms))

    per_layer = []
    for li, (cfg, d) in enumerate(layers):
        ms = np.array([ev[s][li][0].elapsed_time(ev[s][li][1]) for s in range(args.steps)])
        avg = float(np.mean(ms))
        cid, _, split = cb.conv2d_dgrad_query_config(cfg.N, cfg.H, cfg.W, cfg.C, cfg.K, cfg.R, cfg.S, cfg.stride,
                                                     cfg.pad, cfg.epilogue, with_workspace=ws_bytes > 0,
                                                     with_split=True)
        rl = roofline_of(cfg, avg * 1e-3)
        per_layer.append({
            "layer": cfg.name, "avg_us": avg * 1e3, "median_us": float(np.median(ms)) * 1e3,
            "min_us": float(np.min(ms)) * 1e3, "launches": int(len(ms)),
            "tflops": cfg.useful_flops() / (avg * 1e-3) / 1e12,
            "mfma_frac": cfg.useful_flops() / (avg * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS,
            "alg_gbs": cfg.algorithmic_bytes() / (avg * 1e-3) / 1e9,
            "hbm_frac": cfg.algorithmic_bytes() / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "bound": rl["bound"], "roofline_frac": rl["frac"],
            "tile_config": cb.conv2d_dgrad_config_name(cid) + ("+sk" if split else ""),
            "useful_gflop": cfg.useful_flops() / 1e9, "alg_mb": cfg.algorithmic_bytes() / 1e6,
        })
        log(f"[cold] {cfg.name:34s} {avg*1e3:9.2f} us  {per_layer[-1]['tflops']:7.1f} TFLOP/s  "
            f"{per_layer[-1]['alg_gbs']:7.0f} GB/s  {rl['bound']} {rl['frac']:.1%}  [{per_layer[-1]['tile_config']}]")

    # ---- the same cold loop with the other eviction (context, not `value`):
    # a write leaves dirty lines in the Infinity Cache whose write-back lands
    # inside the timed call, a read does not
    flops_total = sum(cfg.useful_flops() for cfg, _ in layers)
    other = "read" if args.flush == "write" else "write"
    evict2 = (lambda: flush.fill_(0.0)) if other == "write" else (lambda: flush.sum())
    ev2 = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in layers] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        for li, (cfg, d) in enumerate(layers):
            evict2()
            ev2[s][li][0].record(stream)
            one_layer(cfg, d)
            ev2[s][li][1].record(stream)
    torch.cuda.synchronize()
    ms2 = float(np.mean([sum(ev2[s][li][0].elapsed_time(ev2[s][li][1]) for li in range(len(layers)))
                         for s in range(args.steps)]))
    other_flush = {"flush": other, "note": f"the cold loop with a 512 MiB {other} before each layer call instead",
                   "value": flops_total / (ms2 * 1e-3) / 1e12, "ms_per_step": ms2,
                   "layers": [{"layer": cfg.name,
                               "avg_us": float(np.mean([ev2[s][li][0].elapsed_time(ev2[s][li][1])
                                                        for s in range(args.steps)])) * 1e3}
                              for li, (cfg, d) in enumerate(layers)]}
    log(f"[cold, {other} flush] " + "  ".join(f"{x['layer'][:18]} {x['avg_us']:.1f}" for x in other_flush["layers"]))
    del flush

    # ---- warm: the layers back to back (operands partly in the caches, like
    # the pages' nvprof averages), wall clock over the steps, then per-layer
    # HIP events in a second pass
    warm = None
    if args.warm_steps > 0:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.warm_steps):
            for cfg, d in layers:
                one_layer(cfg, d)
        torch.cuda.synchronize()
        warm_ms = (time.perf_counter() - t0) * 1e3 / args.warm_steps
        wev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in layers] for _ in range(args.warm_steps)]
        for s in range(args.warm_steps):
            for li, (cfg, d) in enumerate(layers):
                wev[s][li][0].record(stream)
                one_layer(cfg, d)
                wev[s][li][1].record(stream)
        torch.cuda.synchronize()
        wl = []
        for li, (cfg, d) in enumerate(layers):
            ms = [wev[s][li][0].elapsed_time(wev[s][li][1]) for s in range(args.warm_steps)]
            avg = float(np.mean(ms))
            wl.append({"layer": cfg.name, "avg_us": avg * 1e3, "min_us": float(np.min(ms)) * 1e3,
                       "tflops": cfg.useful_flops() / (avg * 1e-3) / 1e12,
                       "roofline_frac": roofline_of(cfg, avg * 1e-3)["frac"]})
            log(f"[warm] {cfg.name:34s} {avg*1e3:9.2f} us  {wl[-1]['tflops']:7.1f} TFLOP/s")
        warm = {"note": "layers back to back, no flush; value = suite FLOPs / wall time per step",
                "value": sum(cfg.useful_flops() for cfg, _ in layers) / (warm_ms * 1e-3) / 1e12,
                "unit": "TFLOP/s", "ms_per_step": warm_ms, "layers": wl}

    # ---- end to end: host time of one C-ABI call plus a stream
    # synchronisation, the tile table already filled (launch overhead included)
    e2e = None
    if args.e2e_reps > 0:
        el = []
        for cfg, d in layers:
            ts = []
            for _ in range(args.e2e_reps):
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                one_layer(cfg, d)
                stream.synchronize()
                ts.append((time.perf_counter() - t0) * 1e6)
            el.append({"layer": cfg.name, "median_us": float(np.median(ts)), "min_us": float(np.min(ts))})
            log(f"[e2e] {cfg.name:34s} {el[-1]['median_us']:9.2f} us (median of {args.e2e_reps})")
        e2e = {"note": "host wall time of conv2d_dgrad_nhwc_ws + stream synchronise, operands warm", "layers": el}

    # ---- wgrad (the filter gradient, a NEXT row of the same layer): each
    # layer's dy with a seeded x, the table's tile config and split count with
    # a caller-owned workspace, HIP events around each call (its two
    # kernels); not part of `value`
    wgrad = None
    if args.wgrad_reps > 0:
        wlayers = []
        for cfg, d in layers:
            x = torch.from_numpy(make_x(cfg)).to(dev)
            dw = torch.empty((cfg.K, cfg.R, cfg.S, cfg.C), dtype=torch.float32, device=dev)
            wws = cb.wgrad_workspace(cfg.N, cfg.H, cfg.W, cfg.C, cfg.K, cfg.R, cfg.S, cfg.stride, cfg.pad, dev)

            def wcall():
                cb.conv2d_wgrad_nhwc_ws(d["dy"], x, dw, cfg.N, cfg.H, cfg.W, cfg.C, cfg.K, cfg.R, cfg.S,
                                        cfg.stride, cfg.pad, wws, stream.cuda_stream)
            for _ in range(3):
                wcall()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.wgrad_reps)]
            for e0, e1 in evs:
                e0.record(stream)
                wcall()
                e1.record(stream)
            torch.cuda.synchronize()
            ms = [e0.elapsed_time(e1) for e0, e1 in evs]
            avg = float(np.mean(ms))
            fl = cfg.useful_flops()
            nbytes = 2 * (cfg.N * cfg.P * cfg.Q * cfg.K + cfg.N * cfg.H * cfg.W * cfg.C) + 4 * cfg.K * cfg.R * cfg.S * cfg.C
            ai = fl / nbytes
            if ai >= RIDGE:
                rl = {"bound": "mfma", "achieved": fl / (avg * 1e-3) / 1e12, "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s"}
            else:
                rl = {"bound": "hbm", "achieved": nbytes / (avg * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
            rl["frac"] = rl["achieved"] / rl["peak"]
            wlayers.append({"layer": cfg.name, "avg_us": avg * 1e3, "min_us": float(np.min(ms)) * 1e3,
                            "tflops": fl / (avg * 1e-3) / 1e12, "alg_mb": nbytes / 1e6, "roofline": rl})
            log(f"[wgrad] {cfg.name:34s} {avg*1e3:9.2f} us  {wlayers[-1]['tflops']:7.1f} TFLOP/s  "
                f"{rl['bound']} {rl['frac']:.1%}")
            del x, dw, wws
        wsum = sum(w["avg_us"] for w in wlayers) * 1e-6
        wgrad = {"note": "dw[k,r,s,c] = sum dy*x (fp32 out), x = max(N(0,1),0) seeded; split-K GEMM plus an "
                         "ordered reduction kernel, partial sums in a caller-owned workspace; warm; suite value = "
                         "useful FLOPs / sum of per-layer means",
                 "value": sum(cfg.useful_flops() for cfg, _ in layers) / wsum / 1e12, "unit": "TFLOP/s",
                 "layers": wlayers}

    # ---- forward layer with the fused bias + hardswish epilogue (a NEXT row):
    # each layer shape's x and w, seeded bias, z and y both stored; not part of `value`
    fwd = None
    if args.forward_reps > 0:
        flayers = []
        for cfg, d in layers:
            x = torch.from_numpy(make_x(cfg)).to(dev)
            bias = torch.from_numpy((np.random.Generator(np.random.PCG64(cfg.seed + 700))
                                     .standard_normal(cfg.K) * 0.5).astype(np.float16)).to(dev)
            y = torch.empty((cfg.N, cfg.P, cfg.Q, cfg.K), dtype=torch.float16, device=dev)
            z = torch.empty_like(y)

            def fcall():
                cb.conv2d_forward_nhwc(x, d["w"], bias, z, y, cfg.N, cfg.H, cfg.W, cfg.C, cfg.K, cfg.R, cfg.S,
                                       cfg.stride, cfg.pad, cb.ACT_HARDSWISH, stream.cuda_stream)
            for _ in range(3):
                fcall()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.forward_reps)]
            for e0, e1 in evs:
                e0.record(stream)
                fcall()
                e1.record(stream)
            torch.cuda.synchronize()
            ms = [e0.elapsed_time(e1) for e0, e1 in evs]
            avg = float(np.mean(ms))
            fl = cfg.useful_flops()
            nbytes = 2 * (cfg.N * cfg.H * cfg.W * cfg.C + cfg.K * cfg.R * cfg.S * cfg.C + cfg.K
                          + 2 * cfg.N * cfg.P * cfg.Q * cfg.K)
            if fl / nbytes >= RIDGE:
                rl = {"bound": "mfma", "achieved": fl / (avg * 1e-3) / 1e12, "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s"}
            else:
                rl = {"bound": "hbm", "achieved": nbytes / (avg * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
            rl["frac"] = rl["achieved"] / rl["peak"]
            flayers.append({"layer": cfg.name, "avg_us": avg * 1e3, "min_us": float(np.min(ms)) * 1e3,
                            "tflops": fl / (avg * 1e-3) / 1e12, "alg_mb": nbytes / 1e6, "roofline": rl})
            log(f"[fwd] {cfg.name:34s} {avg*1e3:9.2f} us  {flayers[-1]['tflops']:7.1f} TFLOP/s  "
                f"{rl['bound']} {rl['frac']:.1%}")
            del x, bias, y, z
        fsum = sum(f["avg_us"] for f in flayers) * 1e-6
        fwd = {"note": "z = bias + conv(x, w), y = hardswish(z), both fp16 and stored; x = max(N(0,1),0), bias "
                       "N(0,0.25) seeded; suite value = useful FLOPs / sum of per-layer means",
               "value": sum(cfg.useful_flops() for cfg, _ in layers) / fsum / 1e12, "unit": "TFLOP/s",
               "layers": flayers}

    # ---- persistent fusion (a NEXT row): the stage-2 bottleneck's 3x3 dgrad,
    # hardswish', then the 1x1 dgrad, fused in one kernel, against the same two
    # steps as two calls of this library (t stored in fp16 between them); not
    # part of `value`
    def chain_block(name):
        from workloads import CHAIN_BY_NAME, make_chain_inputs
        ccfg = CHAIN_BY_NAME[name]
        ci = {k: (None if v is None else torch.from_numpy(v).to(dev)) for k, v in make_chain_inputs(ccfg).items()}
        cdx = torch.empty((ccfg.N, ccfg.H, ccfg.W, ccfg.C), dtype=torch.float16, device=dev)
        ct = torch.empty((ccfg.N, ccfg.H, ccfg.W, ccfg.Cm), dtype=torch.float16, device=dev)
        cdx2 = torch.empty_like(cdx)

        def fused():
            cb.conv2d_dgrad_chain_nhwc(ci["dy"], ci["w1"], ci["z"], ci["w2"], cdx, ccfg.N, ccfg.H, ccfg.W, ccfg.Cm,
                                       ccfg.K, ccfg.R, ccfg.S, ccfg.pad, ccfg.C, ccfg.epilogue, stream.cuda_stream)

        def pair():
            cb.conv2d_dgrad_nhwc(ci["dy"], ci["w1"], ct, ccfg.N, ccfg.H, ccfg.W, ccfg.Cm, ccfg.K, ccfg.R, ccfg.S, 1,
                                 ccfg.pad, ccfg.epilogue, ci["z"], stream.cuda_stream)
            cb.conv2d_dgrad_nhwc(ct, ci["w2"], cdx2, ccfg.N, ccfg.H, ccfg.W, ccfg.C, ccfg.Cm, 1, 1, 1, 0,
                                 cb.EPI_NONE, None, stream.cuda_stream)

        def timed(fn):
            for _ in range(3):
                fn()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.chain_reps)]
            for e0, e1 in evs:
                e0.record(stream)
                fn()
                e1.record(stream)
            torch.cuda.synchronize()
            ms = [e0.elapsed_time(e1) for e0, e1 in evs]
            return float(np.mean(ms)), float(np.min(ms))

        cws = cb.workspace(cb.conv2d_dgrad_chain_workspace_size(ccfg.N, ccfg.H, ccfg.W, ccfg.Cm, ccfg.K, ccfg.R,
                                                                ccfg.S, ccfg.pad, ccfg.C, ccfg.epilogue), dev)

        def chosen():
            cb.conv2d_dgrad_chain_nhwc_ws(ci["dy"], ci["w1"], ci["z"], ci["w2"], cdx, ccfg.N, ccfg.H, ccfg.W,
                                          ccfg.Cm, ccfg.K, ccfg.R, ccfg.S, ccfg.pad, ccfg.C, ccfg.epilogue, cws,
                                          stream.cuda_stream)

        f_avg, f_min = timed(fused)
        p_avg, p_min = timed(pair)
        c_avg, c_min = timed(chosen)
        use_pair, _ = cb.conv2d_dgrad_chain_query(ccfg.N, ccfg.H, ccfg.W, ccfg.Cm, ccfg.K, ccfg.R, ccfg.S, ccfg.pad,
                                                  ccfg.C, ccfg.epilogue)
        fl = ccfg.useful_flops()
        nbytes = ccfg.algorithmic_bytes()
        t_bytes = 2 * 2 * ccfg.N * ccfg.H * ccfg.W * ccfg.Cm     # t written and read back by the pair
        if fl / nbytes >= RIDGE:
            rl = {"bound": "mfma", "achieved": fl / (f_avg * 1e-3) / 1e12, "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s"}
        else:
            rl = {"bound": "hbm", "achieved": nbytes / (f_avg * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
        rl["frac"] = rl["achieved"] / rl["peak"]
        chain = {"note": f"dx = dgrad_1x1(fp16(dgrad_3x3(dy, w1) * hardswish'(z)), w2), ResNet-50 bottleneck "
                         f"(3x3 {ccfg.Cm}->{ccfg.K} and 1x1 {ccfg.C}->{ccfg.Cm} convolutions, {ccfg.H}x{ccfg.W}) at "
                         f"N={ccfg.N}, seeded synthetic; fused = one kernel with the intermediate tile in LDS, "
                         "pair = two dgrad calls with t in HBM",
                 "workload": ccfg.name, "fused_us": f_avg * 1e3, "fused_min_us": f_min * 1e3,
                 "pair_us": p_avg * 1e3, "pair_min_us": p_min * 1e3, "speedup": p_avg / f_avg,
                 "chosen": "pair" if use_pair else "fused", "chosen_us": c_avg * 1e3,
                 "chosen_note": "conv2d_dgrad_chain_nhwc_ws with a workspace that holds t: the library times both "
                                "paths on the first call and keeps the faster",
                 "tflops": fl / (f_avg * 1e-3) / 1e12, "alg_mb": nbytes / 1e6,
                 "pair_alg_mb": (nbytes + t_bytes) / 1e6, "roofline": rl}
        log(f"[chain] {ccfg.name:34s} fused {f_avg*1e3:9.2f} us  pair {p_avg*1e3:9.2f} us  "
            f"chosen ({chain['chosen']}) {c_avg*1e3:9.2f} us  {chain['tflops']:7.1f} TFLOP/s  "
            f"{rl['bound']} {rl['frac']:.1%}")
        del ci, cdx, ct, cdx2, cws
        return chain

    chain = chain3 = None
    if args.chain_reps > 0 and not args.only:
        chain = chain_block("r50_stage2_chain_3x3_1x1_n256")
        chain3 = chain_block("r50_stage3_chain_3x3_1x1_n256")

    flops = sum(cfg.useful_flops() for cfg, _ in layers)
    value = flops / (ms_per_step * 1e-3) / 1e12

    dom = max(range(len(layers)), key=lambda i: per_layer[i]["avg_us"])
    dcfg = layers[dom][0]
    roof = roofline_of(dcfg, per_layer[dom]["avg_us"] * 1e-6)
    roof["kernel"] = f"{kernel_of(per_layer[dom]['tile_config'])} on {dcfg.name}"
    roof["unit_of_work"] = ("one layer call = one launch; algorithmic bytes dy + w + dx (+ z), each once, "
                            f"{dcfg.algorithmic_bytes()} B; cold mean of {args.steps} launches")
    roof["traffic"] = measured_traffic(dcfg.name, per_layer[dom]["tile_config"])
    roof["kernel_source_sha256_16"] = kernel_source_digest()

    cpu = None
    if args.cpu_fraction > 0:
        cpu = cpu_baseline(host_inputs, args.cpu_fraction, suite)

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "resnet50_dgrad_suite: " + ", ".join(
                f"{c.name} (N={c.N} {c.H}x{c.W} C={c.C} K={c.K} {c.R}x{c.S} s{c.stride} p{c.pad}"
                f"{'' if c.epilogue == 0 else ' +' + EPI_NAMES[c.epilogue]})" for c, _ in layers),
            "accumulate": "f32",
            "layout": "NHWC fp16 dy/dx/z, KRSC fp16 filter",
            "useful_gflop_per_step": flops / 1e9,
            "timing": "cold",
        },
        "mfma_frac_of_peak": value / MFMA_PEAK_TFLOPS,
        "timing": f"cold: each layer call after a 512 MiB {args.flush}; per-layer HIP events on the launch stream; "
                  f"{args.steps} launches per layer; wall time of the timed loop {cold_wall:.3f} s "
                  "(flushes included)",
        "roofline": roof,
        "cpu_baseline": cpu,
        "layers": per_layer,
        "cold_other_flush": other_flush,
        "warm": warm,
        "e2e": e2e,
        "workspace_bytes": ws_bytes,
        "wgrad": wgrad,
        "forward": fwd,
        "chain": chain,
        "chain_stage3": chain3,
        "device": torch.cuda.get_device_name(dev),
        "build": cb.conv2d_dgrad_build_info(),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
