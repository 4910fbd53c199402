"""The C ABI on the CPU: the library loads, exports what the header declares,
validates arguments before any HIP call, and plans stride phases correctly.
No test here launches a kernel."""
import ctypes
import itertools
import os
import re

import numpy as np
import pytest

import convolution_backward_amd as cb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "conv2d_dgrad.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(conv2d_(?:dgrad|wgrad|forward)_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(cb.LIB_PATH)
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n


def test_header_status_codes_match_binding():
    text = open(HEADER).read()
    for name, val in [("OK", cb.OK), ("INVALID_ARGUMENT", cb.INVALID_ARGUMENT),
                      ("UNSUPPORTED", cb.UNSUPPORTED), ("HIP_ERROR", cb.HIP_ERROR),
                      ("EPI_NONE", cb.EPI_NONE), ("EPI_DRELU", cb.EPI_DRELU),
                      ("EPI_DHARDSWISH", cb.EPI_DHARDSWISH)]:
        m = re.search(rf"#define CONV2D_DGRAD_{name} (\d+)", text)
        assert m and int(m.group(1)) == val, name


def test_build_info_names_target():
    info = cb.conv2d_dgrad_build_info()
    assert "gfx950" in info and "HIP" in info


def test_config_names():
    n = cb.conv2d_dgrad_num_configs()
    assert n >= 4
    names = [cb.conv2d_dgrad_config_name(i) for i in range(n)]
    assert len(set(names)) == n
    for nm in names:
        assert re.fullmatch(r"\d+x\d+x64/\d+x\d+[whpsq]?", nm)
    with pytest.raises(cb.DgradError):
        cb.conv2d_dgrad_config_name(n)


# Fake, aligned, non-overlapping addresses: validation never dereferences them.
DY, WP, DX, Z = 0x10000000, 0x20000000, 0x30000000, 0x40000000
GOOD = dict(N=2, H=8, W=8, C=16, K=8, R=3, S=3, stride=2, pad=1)


def check(dy=DY, w=WP, dx=DX, z=None, epi=0, **kw):
    args = dict(GOOD)
    args.update(kw)
    return cb.conv2d_dgrad_check(dy, w, dx, args["N"], args["H"], args["W"], args["C"], args["K"],
                                 args["R"], args["S"], args["stride"], args["pad"], epi, z)


@pytest.mark.parametrize("kw,code", [
    ({}, cb.OK),
    ({"N": 0}, cb.INVALID_ARGUMENT), ({"H": 0}, cb.INVALID_ARGUMENT), ({"C": -8}, cb.INVALID_ARGUMENT),
    ({"R": 0}, cb.INVALID_ARGUMENT), ({"stride": 0}, cb.INVALID_ARGUMENT), ({"pad": -1}, cb.INVALID_ARGUMENT),
    ({"H": 1, "R": 5, "pad": 0}, cb.INVALID_ARGUMENT),             # P < 1
    ({"epi": 7}, cb.INVALID_ARGUMENT), ({"epi": cb.EPI_DHARDSWISH}, cb.INVALID_ARGUMENT),  # z missing
    ({"epi": cb.EPI_DRELU, "z": Z}, cb.OK),
    ({"dy": 0}, cb.INVALID_ARGUMENT), ({"dx": 0}, cb.INVALID_ARGUMENT), ({"w": 0}, cb.INVALID_ARGUMENT),
    ({"dy": DY + 8}, cb.INVALID_ARGUMENT),                           # misaligned
    ({"dx": DY + 16}, cb.INVALID_ARGUMENT),                          # dx overlaps dy
    ({"C": 12}, cb.UNSUPPORTED), ({"K": 4}, cb.UNSUPPORTED), ({"stride": 17, "H": 40, "W": 40}, cb.UNSUPPORTED),
    ({"N": 70000, "H": 200, "W": 200}, cb.UNSUPPORTED),               # 2^31 elements
])
def test_validation_codes(kw, code):
    assert check(**kw) == code
    if code != cb.OK:
        assert cb.conv2d_dgrad_last_error() != ""


WG = dict(N=2, H=8, W=8, C=16, K=8, R=3, S=3, stride=2, pad=1)


def wcheck(dy=DY, x=DX, dw=WP, **kw):
    args = dict(WG)
    args.update(kw)
    return cb.conv2d_wgrad_check(dy, x, dw, args["N"], args["H"], args["W"], args["C"], args["K"],
                                 args["R"], args["S"], args["stride"], args["pad"])


@pytest.mark.parametrize("kw,code", [
    ({}, cb.OK),
    ({"N": 0}, cb.INVALID_ARGUMENT), ({"stride": 0}, cb.INVALID_ARGUMENT), ({"H": 1, "R": 5, "pad": 0}, cb.INVALID_ARGUMENT),
    ({"dy": 0}, cb.INVALID_ARGUMENT), ({"x": 0}, cb.INVALID_ARGUMENT), ({"dw": 0}, cb.INVALID_ARGUMENT),
    ({"dw": WP + 8}, cb.INVALID_ARGUMENT),                          # misaligned
    ({"dw": DY + 64}, cb.INVALID_ARGUMENT),                         # dw overlaps dy
    ({"dw": DX + 16}, cb.INVALID_ARGUMENT),                         # dw overlaps x
    ({"C": 12}, cb.UNSUPPORTED), ({"K": 4}, cb.UNSUPPORTED),
])
def test_wgrad_validation_codes(kw, code):
    assert wcheck(**kw) == code
    if code != cb.OK:
        assert cb.conv2d_dgrad_last_error() != ""


def test_wgrad_configs_and_bad_calls():
    assert cb.conv2d_wgrad_num_configs() >= 2
    with pytest.raises(cb.DgradError) as e:
        cb.conv2d_wgrad_nhwc(DY, DX, WP, 2, 8, 8, 12, 8, 3, 3, 1, 1, stream=0)
    assert e.value.code == cb.UNSUPPORTED
    with pytest.raises(cb.DgradError) as e:
        cb.conv2d_wgrad_nhwc_config(DY, DX, WP, 2, 8, 8, 16, 8, 3, 3, 1, 1, config_id=99, stream=0)
    assert e.value.code == cb.INVALID_ARGUMENT


FB = 0x50000000   # bias
FG = dict(N=2, H=8, W=8, C=16, K=8, R=3, S=3, stride=2, pad=1)


def fcheck(x=DX, w=WP, bias=FB, z=Z, y=DY, act=1, **kw):
    args = dict(FG)
    args.update(kw)
    return cb.conv2d_forward_check(x, w, bias, z, y, args["N"], args["H"], args["W"], args["C"], args["K"],
                                   args["R"], args["S"], args["stride"], args["pad"], act)


@pytest.mark.parametrize("kw,code", [
    ({}, cb.OK), ({"z": 0}, cb.OK),                                 # z is optional
    ({"act": 2}, cb.INVALID_ARGUMENT), ({"act": -1}, cb.INVALID_ARGUMENT),
    ({"x": 0}, cb.INVALID_ARGUMENT), ({"w": 0}, cb.INVALID_ARGUMENT), ({"bias": 0}, cb.INVALID_ARGUMENT),
    ({"y": 0}, cb.INVALID_ARGUMENT),
    ({"y": DY + 8}, cb.INVALID_ARGUMENT), ({"bias": FB + 4}, cb.INVALID_ARGUMENT),   # misaligned
    ({"y": DX + 16}, cb.INVALID_ARGUMENT),                          # y overlaps x
    ({"z": DY + 16}, cb.INVALID_ARGUMENT),                          # z overlaps y
    ({"C": 12}, cb.UNSUPPORTED), ({"K": 4}, cb.UNSUPPORTED), ({"N": 0}, cb.INVALID_ARGUMENT),
])
def test_forward_validation_codes(kw, code):
    assert fcheck(**kw) == code
    if code != cb.OK:
        assert cb.conv2d_dgrad_last_error() != ""


def test_forward_configs_and_bad_calls():
    assert cb.conv2d_forward_num_configs() >= 2
    with pytest.raises(cb.DgradError) as e:
        cb.conv2d_forward_nhwc(DX, WP, FB, Z, DY, 2, 8, 8, 12, 8, 3, 3, 1, 1, 1, stream=0)
    assert e.value.code == cb.UNSUPPORTED
    with pytest.raises(cb.DgradError) as e:
        cb.conv2d_forward_nhwc_config(DX, WP, FB, Z, DY, 2, 8, 8, 16, 8, 3, 3, 1, 1, 1, config_id=99, stream=0)
    assert e.value.code == cb.INVALID_ARGUMENT


W2 = 0x60000000   # second filter of the chain
CG = dict(N=2, H=8, W=8, Cm=64, K=32, R=3, S=3, pad=1, C=128)


def ccheck(dy=DY, w1=WP, z=Z, w2=W2, dx=DX, epi=cb.EPI_DHARDSWISH, **kw):
    a = dict(CG)
    a.update(kw)
    return cb.conv2d_dgrad_chain_check(dy, w1, z, w2, dx, a["N"], a["H"], a["W"], a["Cm"], a["K"], a["R"], a["S"],
                                       a["pad"], a["C"], epi)


@pytest.mark.parametrize("kw,code", [
    ({}, cb.OK), ({"epi": cb.EPI_NONE, "z": 0}, cb.OK), ({"Cm": 128}, cb.OK), ({"Cm": 8, "C": 8}, cb.OK),
    ({"epi": cb.EPI_DRELU, "z": 0}, cb.INVALID_ARGUMENT),          # z missing
    ({"epi": 3}, cb.INVALID_ARGUMENT),
    ({"N": 0}, cb.INVALID_ARGUMENT), ({"C": 0}, cb.INVALID_ARGUMENT), ({"pad": -1}, cb.INVALID_ARGUMENT),
    ({"H": 1, "R": 5, "pad": 0}, cb.INVALID_ARGUMENT),             # P < 1
    ({"dy": 0}, cb.INVALID_ARGUMENT), ({"w1": 0}, cb.INVALID_ARGUMENT), ({"w2": 0}, cb.INVALID_ARGUMENT),
    ({"dx": 0}, cb.INVALID_ARGUMENT),
    ({"w2": W2 + 8}, cb.INVALID_ARGUMENT),                          # misaligned
    ({"dx": DY + 16}, cb.INVALID_ARGUMENT),                         # dx overlaps dy
    ({"dx": W2 + 64}, cb.INVALID_ARGUMENT),                         # dx overlaps w2
    ({"dx": Z + 16}, cb.INVALID_ARGUMENT),                          # dx overlaps z
    ({"Cm": 136}, cb.UNSUPPORTED),                                  # more than one resident tile of channels
    ({"Cm": 60}, cb.UNSUPPORTED), ({"C": 12}, cb.UNSUPPORTED), ({"K": 4}, cb.UNSUPPORTED),
    ({"N": 70000, "H": 64, "W": 64, "C": 8, "Cm": 8, "K": 8}, cb.UNSUPPORTED),   # dx of 2^31 elements
])
def test_chain_validation_codes(kw, code):
    assert ccheck(**kw) == code
    if code != cb.OK:
        assert cb.conv2d_dgrad_last_error() != ""


def test_chain_bad_call_raises_before_launch():
    with pytest.raises(cb.DgradError) as e:
        cb.conv2d_dgrad_chain_nhwc(DY, WP, Z, W2, DX, 2, 8, 8, 200, 32, 3, 3, 1, 128, cb.EPI_DHARDSWISH, stream=0)
    assert e.value.code == cb.UNSUPPORTED


def test_invalid_call_returns_before_any_hip_call():
    # conv2d_dgrad_nhwc with a bad argument fails with the validation code,
    # not a HIP error, on a host without a GPU.
    with pytest.raises(cb.DgradError) as e:
        cb.conv2d_dgrad_nhwc(DY, WP, DX, 2, 8, 8, 12, 8, 3, 3, 1, 1, stream=0)
    assert e.value.code == cb.UNSUPPORTED
    with pytest.raises(cb.DgradError) as e:
        cb.conv2d_dgrad_nhwc_config(DY, WP, DX, 2, 8, 8, 16, 8, 3, 3, 1, 1, config_id=99, stream=0)
    assert e.value.code == cb.INVALID_ARGUMENT


WS = 0x70000000   # a workspace address


@pytest.mark.parametrize("ws,nbytes,code", [
    (None, 16, cb.INVALID_ARGUMENT),            # NULL with a size
    (WS + 8, 1 << 20, cb.INVALID_ARGUMENT),     # misaligned
    (WS, 65535, cb.INVALID_ARGUMENT),           # smaller than the counter area
    (DX - 4096, 1 << 20, cb.INVALID_ARGUMENT),  # overlaps dx
    (DY + 256, 1 << 20, cb.INVALID_ARGUMENT),   # overlaps dy (512 bytes)
])
def test_workspace_validation(ws, nbytes, code):
    for fn in (lambda: cb.conv2d_dgrad_nhwc_ws(DY, WP, DX, 2, 8, 8, 16, 8, 3, 3, 2, 1, workspace=(ws, nbytes),
                                               stream=0),
               lambda: cb.conv2d_dgrad_nhwc_config(DY, WP, DX, 2, 8, 8, 16, 8, 3, 3, 2, 1, config_id=0,
                                                   workspace=(ws, nbytes), stream=0),
               lambda: cb.conv2d_wgrad_nhwc_ws(DY, DX, WP, 2, 8, 8, 16, 8, 3, 3, 2, 1, workspace=(ws, nbytes),
                                               stream=0)):
        with pytest.raises(cb.DgradError) as e:
            fn()
        assert e.value.code == code and "workspace" in str(e.value)


def test_workspace_size_queries():
    from workloads import CONFIGS
    sizes = {c.name: cb.conv2d_dgrad_workspace_size(c.N, c.H, c.W, c.C, c.K, c.R, c.S, c.stride, c.pad, c.epilogue)
             for c in CONFIGS}
    # layers whose tiles leave workgroups idle can split: counters + partial sums
    assert sizes["tiny_n1_14x14_256_3x3_s1"] > 65536
    assert sizes["r50_stage4_3x3_dhardswish_n256"] > 65536
    # zero phases never split
    assert sizes["r50_1x1_s2_downsample_n256"] == 0
    for n in sizes.values():
        assert n == 0 or 65536 < n <= 65536 + (1 << 30)
    c = CONFIGS[2]
    wsz = cb.conv2d_wgrad_workspace_size(c.N, c.H, c.W, c.C, c.K, c.R, c.S, c.stride, c.pad)
    assert 65536 < wsz <= 65536 + (1 << 30)
    assert cb.conv2d_wgrad_workspace_size(1, 1, 1, 8, 8, 1, 1, 1, 0) == 0   # one slice: nothing to split
    with pytest.raises(cb.DgradError):
        cb.conv2d_dgrad_workspace_size(2, 8, 8, 12, 8, 3, 3, 2, 1)


def test_library_imports_no_allocator():
    """The library never allocates device (or pinned host) memory: it imports
    no allocation, free or memset routine of the HIP runtime."""
    import subprocess
    out = subprocess.run(["nm", "-D", "--undefined-only", cb.LIB_PATH], check=True, capture_output=True,
                         text=True).stdout
    hip = [ln.split()[-1] for ln in out.splitlines() if "hip" in ln.lower()]
    assert hip, "no HIP import found (nm output changed?)"
    bad = [n for n in hip if re.search(r"alloc|free|memset|hostregister", n, re.I)]
    assert not bad, bad


def test_library_sources_call_no_allocator():
    csrc = os.path.join(ROOT, "convolution_backward_amd", "csrc")
    for fn in os.listdir(csrc):
        text = open(os.path.join(csrc, fn)).read()
        text = re.sub(r"//[^\n]*", "", text)
        assert not re.search(r"\bhip(Ext)?Malloc|\bhipFree|\bhipMemset|\bhipHostMalloc", text), fn


def _meta(shape, dtype=None):
    import torch
    return torch.empty(shape, dtype=dtype or torch.float16, device="meta")


@pytest.mark.parametrize("case", ["dy_pq", "w_k", "z_shape", "z_dtype", "out_shape", "out_dtype", "cpu"])
def test_dgrad_wrapper_checks_shapes(case):
    """Every tensor is checked against the shape the C call is told, before
    any C call (a mismatch would let the kernel run past a buffer)."""
    import torch
    N, H, W, C, K = 2, 8, 8, 16, 8
    dy, w = _meta((N, 4, 4, K)), _meta((K, 3, 3, C))        # stride 2, pad 1: P = Q = 4
    z, out = _meta((N, H, W, C)), _meta((N, H, W, C))
    kw = dict(epilogue=cb.EPI_DHARDSWISH, z=z, out=out)
    if case == "dy_pq":
        dy = _meta((N, 5, 4, K))
    elif case == "w_k":
        w = _meta((K + 8, 3, 3, C))
    elif case == "z_shape":
        kw["z"] = _meta((N, H, W - 1, C))
    elif case == "z_dtype":
        kw["z"] = _meta((N, H, W, C), torch.float32)
    elif case == "out_shape":
        kw["out"] = _meta((N, H, W, C + 8))
    elif case == "out_dtype":
        kw["out"] = _meta((N, H, W, C), torch.float32)
    with pytest.raises(ValueError):
        cb.dgrad(dy, w, H, W, 2, 1, **kw)


@pytest.mark.parametrize("case", ["dy_pq", "out_shape", "out_dtype"])
def test_wgrad_wrapper_checks_shapes(case):
    import torch
    dy, x = _meta((2, 4, 4, 8)), _meta((2, 8, 8, 16))
    out = _meta((8, 3, 3, 16), torch.float32)
    if case == "dy_pq":
        dy = _meta((2, 4, 3, 8))
    elif case == "out_shape":
        out = _meta((8, 3, 3, 24), torch.float32)
    elif case == "out_dtype":
        out = _meta((8, 3, 3, 16))
    with pytest.raises(ValueError):
        cb.wgrad(dy, x, 3, 3, 2, 1, out=out)


@pytest.mark.parametrize("case", ["bias", "out", "z_out", "w_c"])
def test_forward_wrapper_checks_shapes(case):
    x, w, bias = _meta((2, 8, 8, 16)), _meta((8, 3, 3, 16)), _meta((8,))
    kw = dict(out=_meta((2, 4, 4, 8)), z_out=_meta((2, 4, 4, 8)))
    if case == "bias":
        bias = _meta((16,))
    elif case == "out":
        kw["out"] = _meta((2, 4, 5, 8))
    elif case == "z_out":
        kw["z_out"] = _meta((2, 4, 4, 16))
    elif case == "w_c":
        w = _meta((8, 3, 3, 24))
    with pytest.raises(ValueError):
        cb.forward(x, w, bias, 2, 1, **kw)


@pytest.mark.parametrize("case", ["z", "out", "w2"])
def test_chain_wrapper_checks_shapes(case):
    dy, w1, w2 = _meta((2, 8, 8, 32)), _meta((32, 3, 3, 64)), _meta((64, 1, 1, 128))
    z, out = _meta((2, 8, 8, 64)), _meta((2, 8, 8, 128))
    if case == "z":
        z = _meta((2, 8, 8, 128))
    elif case == "out":
        out = _meta((2, 8, 9, 128))
    elif case == "w2":
        w2 = _meta((64, 3, 1, 128))
    with pytest.raises(ValueError):
        cb.dgrad_chain(dy, w1, z, w2, 1, cb.EPI_DHARDSWISH, out=out)


def test_table_under_concurrent_callers(tmp_path):
    """Eight host threads query, save, load and clear the table at once
    (ctypes releases the GIL in every call): no crash, every query answers,
    and the table ends in a state one of the writers left."""
    import threading
    names = [cb.conv2d_dgrad_config_name(i) for i in range(cb.conv2d_dgrad_num_configs())]
    lines = "".join(f"{n} 8 8 16 8 3 3 1 1 0 none 256 0 {names[n % len(names)]}\n" for n in range(1, 65))
    src = tmp_path / "table.txt"
    src.write_text(lines)
    errors = []

    def worker(k):
        try:
            for i in range(300):
                op = (i + k) % 5
                if op == 0:
                    cid, _ = cb.conv2d_dgrad_query_config(1 + i % 64, 8, 8, 16, 8, 3, 3, 1, 1)
                    assert 0 <= cid < len(names)
                elif op == 1:
                    cb.conv2d_dgrad_cache_load(str(src))
                elif op == 2:
                    cb.conv2d_dgrad_cache_save(str(tmp_path / f"out{k}.txt"))
                elif op == 3 and i % 50 == 0:
                    cb.conv2d_dgrad_cache_clear()
                else:
                    assert cb.conv2d_dgrad_workspace_size(1 + i % 64, 8, 8, 16, 8, 3, 3, 1, 1) >= 0
                    assert 0 <= cb.conv2d_dgrad_cache_size() <= 64
        except Exception as e:   # noqa: BLE001
            errors.append(repr(e))

    cb.conv2d_dgrad_cache_clear()
    threads = [threading.Thread(target=worker, args=(k,)) for k in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:3]
    cb.conv2d_dgrad_cache_load(str(src))
    assert cb.conv2d_dgrad_cache_size() == 64
    for k in range(8):   # every saved file is a whole table: lines of 14 fields
        for ln in (tmp_path / f"out{k}.txt").read_text().splitlines():
            assert len(ln.split()) == 14
    cb.conv2d_dgrad_cache_clear()


def brute_phase(H, R, stride, pad, ph):
    """Taps reaching output rows h = ph + s*i, found by trying every r."""
    rows = list(range(ph, H, stride))
    taps = [r for r in range(R) if (ph + pad - r) % stride == 0]
    deltas = [(ph + pad - r) // stride for r in taps]
    return len(rows), taps, deltas


@pytest.mark.parametrize("stride", [1, 2, 3, 4, 5])
def test_plan_matches_brute_force(stride):
    for H, W, R, S, pad in itertools.product(range(1, 9), (3, 7), (1, 2, 3, 5), (1, 3), (0, 1, 2, 3)):
        if (H + 2 * pad - R) < 0 or (W + 2 * pad - S) < 0:
            continue
        N, K = 2, 8
        P, Q, phases = cb.conv2d_dgrad_plan(N, H, W, 8, K, R, S, stride, pad)
        assert P == (H + 2 * pad - R) // stride + 1 and Q == (W + 2 * pad - S) // stride + 1
        seen = set()
        for p in phases:
            hp, rt, rd = brute_phase(H, R, stride, pad, p["ph"])
            wp, tt, td = brute_phase(W, S, stride, pad, p["pw"])
            assert (p["Hp"], p["Wp"]) == (hp, wp)
            assert [p["r0"] + a * stride for a in range(p["nr"])] == rt
            assert [p["t0"] + b * stride for b in range(p["nt"])] == tt
            assert [p["dr0"] - a for a in range(p["nr"])] == rd
            assert [p["dt0"] - b for b in range(p["nt"])] == td
            assert p["M"] == N * hp * wp and p["Kg"] == K * len(rt) * len(tt)
            seen.add((p["ph"], p["pw"]))
        # every non-empty lattice appears once; lattices cover dx exactly
        want = {(a, b) for a in range(min(stride, H)) for b in range(min(stride, W))}
        assert seen == want
        assert sum(p["M"] for p in phases) == N * H * W
        # heaviest first
        taps = [p["nr"] * p["nt"] for p in phases]
        assert taps == sorted(taps, reverse=True)


def test_plan_of_measured_layers():
    from workloads import CONFIGS
    c = CONFIGS[2]   # 3x3, stride 2, pad 1 on 56x56
    P, Q, phases = cb.conv2d_dgrad_plan(c.N, c.H, c.W, c.C, c.K, c.R, c.S, c.stride, c.pad)
    assert (P, Q) == (28, 28)
    assert [p["nr"] * p["nt"] for p in phases] == [4, 2, 2, 1]
    assert all(p["M"] == 256 * 28 * 28 for p in phases)
    c = CONFIGS[3]   # 1x1, stride 2: one GEMM phase, three zero phases
    _, _, phases = cb.conv2d_dgrad_plan(c.N, c.H, c.W, c.C, c.K, c.R, c.S, c.stride, c.pad)
    assert [p["Kg"] for p in phases] == [512, 0, 0, 0]
    assert (phases[0]["ph"], phases[0]["pw"]) == (0, 0)


def test_query_config_without_gpu_uses_heuristic():
    cb.conv2d_dgrad_cache_clear()
    cid, cached = cb.conv2d_dgrad_query_config(8, 56, 56, 64, 64, 3, 3, 1, 1)
    assert 0 <= cid < cb.conv2d_dgrad_num_configs() and not cached
    assert "x64x" in cb.conv2d_dgrad_config_name(cid)   # narrow layer -> 64-channel tile


def test_cache_save_load_roundtrip(tmp_path):
    cb.conv2d_dgrad_cache_clear()
    assert cb.conv2d_dgrad_cache_size() == 0
    # A saved line for a CPU-only host ("none", 256 CUs) is what a query here looks up.
    name = cb.conv2d_dgrad_config_name(1)
    f = tmp_path / "table.txt"
    f.write_text(f"2 8 8 16 8 3 3 2 1 0 none 256 0 {name}\nthis line is ignored\n")
    cb.conv2d_dgrad_cache_load(str(f))
    assert cb.conv2d_dgrad_cache_size() == 1
    cid, cached = cb.conv2d_dgrad_query_config(2, 8, 8, 16, 8, 3, 3, 2, 1)
    assert cached and cid == 1
    cid, cached = cb.conv2d_dgrad_query_config(2, 8, 8, 16, 8, 3, 3, 2, 1, with_workspace=True)
    assert not cached   # calls with a workspace have their own entry
    out = tmp_path / "saved.txt"
    cb.conv2d_dgrad_cache_save(str(out))
    assert out.read_text().split() == f"2 8 8 16 8 3 3 2 1 0 none 256 0 {name}".split()
    cb.conv2d_dgrad_cache_clear()
    assert cb.conv2d_dgrad_cache_size() == 0


def test_cache_keeps_stream_k_choice(tmp_path):
    """A table line may mark its choice as split ("+sk"); configurations
    without a stream-K variant cannot carry the mark (the line is skipped)."""
    cb.conv2d_dgrad_cache_clear()
    names = [cb.conv2d_dgrad_config_name(i) for i in range(cb.conv2d_dgrad_num_configs())]
    split_ok = names.index("256x128x64/4x2")
    no_variant = names.index("256x64x64/4x1")
    f = tmp_path / "table.txt"
    f.write_text(f"256 7 7 512 512 3 3 1 1 2 none 256 1 {names[split_ok]}+sk\n"
                 f"256 7 7 512 512 3 3 1 1 2 none 256 0 {names[split_ok]}+sk\n"     # a split needs a workspace
                 f"2 8 8 16 8 3 3 2 1 0 none 256 1 {names[no_variant]}+sk\n"
                 f"2 8 8 16 8 3 3 1 1 0 none 256 0 {names[no_variant]}\n")
    cb.conv2d_dgrad_cache_load(str(f))
    assert cb.conv2d_dgrad_cache_size() == 2
    cid, cached, split = cb.conv2d_dgrad_query_config(256, 7, 7, 512, 512, 3, 3, 1, 1, cb.EPI_DHARDSWISH,
                                                      with_workspace=True, with_split=True)
    assert cached and cid == split_ok and split
    out = tmp_path / "saved.txt"
    cb.conv2d_dgrad_cache_save(str(out))
    lines = sorted(out.read_text().splitlines())
    assert lines == sorted([f"256 7 7 512 512 3 3 1 1 2 none 256 1 {names[split_ok]}+sk",
                            f"2 8 8 16 8 3 3 1 1 0 none 256 0 {names[no_variant]}"])
    cb.conv2d_dgrad_cache_clear()


def test_streamk_mode_setting():
    prev = cb.conv2d_dgrad_set_streamk(0)
    try:
        assert cb.conv2d_dgrad_set_streamk(1) == 0
        assert cb.conv2d_dgrad_set_streamk(2) == 1
        with pytest.raises(cb.DgradError) as e:
            cb.conv2d_dgrad_set_streamk(3)
        assert e.value.code == cb.INVALID_ARGUMENT
        assert cb.conv2d_dgrad_set_streamk(2) == 2
    finally:
        cb.conv2d_dgrad_set_streamk(prev)
    assert cb.conv2d_dgrad_streamk_launches() == 0   # nothing launched without a GPU


def test_autotune_toggle():
    prev = cb.conv2d_dgrad_set_autotune(False)
    assert cb.conv2d_dgrad_set_autotune(prev) is False


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    import importlib
    mod = importlib.import_module("convolution_backward_amd")
    monkeypatch.setattr(mod, "_lib", None)
    monkeypatch.setattr(mod, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(ImportError):
        mod.get_lib()
