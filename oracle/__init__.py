"""ctypes front end of the fp64 CPU oracle for conv2d dgrad (and wgrad).

TEST INFRASTRUCTURE: only tests/, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package. The product package
``convolution_backward_amd`` never imports it and shares no code with it.

The arithmetic lives in ``dgrad_oracle.c`` (plain C, built with gcc and
OpenMP); this file only builds/loads it and marshals numpy arrays.
Functions whose results have no independent pin are listed in the C file's
header; at present every function here is pinned by ``tests/test_oracle.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "dgrad_oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")

EPI_NONE, EPI_DRELU, EPI_DHARDSWISH = 0, 1, 2

# Portable ISA level: the library is built here and may run on another host.
CFLAGS = ["-O3", "-march=x86-64-v3", "-fopenmp", "-fPIC", "-shared", "-std=c11"]


def build(src: str = SRC, out: str = LIB, extra=()) -> str:
    """Compile the oracle with gcc. Always recompiles."""
    cmd = ["gcc", *CFLAGS, *extra, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_lib = None


def _bind(lib):
    u16p = ctypes.POINTER(ctypes.c_uint16)
    f64p = ctypes.POINTER(ctypes.c_double)
    i64p = ctypes.POINTER(ctypes.c_int64)
    i = ctypes.c_int
    lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_half_to_double.restype = ctypes.c_double
    lib.oracle_double_to_half_rne.argtypes = [ctypes.c_double]
    lib.oracle_double_to_half_rne.restype = ctypes.c_uint16
    lib.oracle_relu_grad.argtypes = [ctypes.c_double]
    lib.oracle_relu_grad.restype = ctypes.c_double
    lib.oracle_hardswish_grad.argtypes = [ctypes.c_double]
    lib.oracle_hardswish_grad.restype = ctypes.c_double
    lib.oracle_out_extent.argtypes = [i, i, i, i]
    lib.oracle_out_extent.restype = i
    lib.oracle_dgrad_rows.argtypes = [u16p, u16p, u16p] + [i] * 10 + [i64p, ctypes.c_int64, f64p, i]
    lib.oracle_dgrad_rows.restype = i
    lib.oracle_dgrad_full.argtypes = [u16p, u16p, u16p] + [i] * 10 + [f64p, i]
    lib.oracle_dgrad_full.restype = i
    lib.oracle_wgrad_rows.argtypes = [u16p, u16p] + [i] * 9 + [i64p, ctypes.c_int64, f64p, f64p, i]
    lib.oracle_wgrad_rows.restype = i
    lib.oracle_forward_rows.argtypes = [u16p, u16p, u16p] + [i] * 10 + [i64p, ctypes.c_int64, f64p, f64p, i]
    lib.oracle_forward_rows.restype = i
    lib.oracle_chain_rows.argtypes = [u16p, u16p, u16p, u16p] + [i] * 10 + [i64p, ctypes.c_int64, f64p, f64p, i]
    lib.oracle_chain_rows.restype = i
    lib.oracle_hardswish.argtypes = [ctypes.c_double]
    lib.oracle_hardswish.restype = ctypes.c_double
    lib.oracle_round_to_half.argtypes = [f64p, u16p, ctypes.c_int64]
    lib.oracle_round_to_half.restype = None
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = i
    return lib


def load(path: str = LIB):
    """Load the built oracle (building it only if no library exists)."""
    global _lib
    if path == LIB and _lib is not None:
        return _lib
    if not os.path.exists(path):
        build(out=path)
    lib = _bind(ctypes.CDLL(path))
    if path == LIB:
        _lib = lib
    return lib


def _u16(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.float16:
        raise TypeError("oracle inputs are float16 arrays")
    return a.view(np.uint16), a.view(np.uint16).ctypes.data_as(ctypes.POINTER(ctypes.c_uint16))


def out_extent(n_in, filt, stride, pad, lib=None):
    return (lib or load()).oracle_out_extent(n_in, filt, stride, pad)


def dgrad(dy, w, H, W, stride, pad, epilogue=EPI_NONE, z=None, rows=None,
          threads=0, lib=None):
    """fp64 dgrad of float16 dy [N,P,Q,K] and w [K,R,S,C].

    Returns [N,H,W,C] float64, or [len(rows), C] when ``rows`` (linear pixel
    indices (n*H+h)*W+w) is given.
    """
    lib = lib or load()
    N, P, Q, K = dy.shape
    K2, R, S, C = w.shape
    if K2 != K:
        raise ValueError("dy and w disagree on K")
    if (lib.oracle_out_extent(H, R, stride, pad), lib.oracle_out_extent(W, S, stride, pad)) != (P, Q):
        raise ValueError("dy spatial shape does not match H, W, R, S, stride, pad")
    dyk, dyp = _u16(dy)
    wk, wp = _u16(w)
    zk = zp = None
    if epilogue != EPI_NONE:
        if z is None or tuple(z.shape) != (N, H, W, C):
            raise ValueError("epilogue needs z of shape [N,H,W,C]")
        zk, zp = _u16(z)
    f64p = ctypes.POINTER(ctypes.c_double)
    if rows is None:
        out = np.empty((N, H, W, C), dtype=np.float64)
        rc = lib.oracle_dgrad_full(dyp, wp, zp, N, H, W, C, K, R, S, stride, pad,
                                   epilogue, out.ctypes.data_as(f64p), int(threads))
    else:
        rr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        out = np.empty((len(rr), C), dtype=np.float64)
        rc = lib.oracle_dgrad_rows(dyp, wp, zp, N, H, W, C, K, R, S, stride, pad,
                                   epilogue, rr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                   len(rr), out.ctypes.data_as(f64p), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_dgrad failed with code {rc}")
    del dyk, wk, zk
    return out


def wgrad(dy, x, R, S, stride, pad, rows=None, with_abs=False, threads=0, lib=None):
    """fp64 filter gradient of float16 dy [N,P,Q,K] and x [N,H,W,C].

    Returns [K,R,S,C] float64, or [len(rows), C] when ``rows`` (linear filter
    rows (k*R + r)*S + t) is given. With ``with_abs`` also returns the sums of
    |dy * x| of the same shape.
    """
    lib = lib or load()
    N, P, Q, K = dy.shape
    N2, H, W, C = x.shape
    if N2 != N:
        raise ValueError("dy and x disagree on N")
    if (lib.oracle_out_extent(H, R, stride, pad), lib.oracle_out_extent(W, S, stride, pad)) != (P, Q):
        raise ValueError("dy spatial shape does not match H, W, R, S, stride, pad")
    dyk, dyp = _u16(dy)
    xk, xp = _u16(x)
    rr = np.arange(K * R * S, dtype=np.int64) if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    out = np.empty((len(rr), C), dtype=np.float64)
    mag = np.empty((len(rr), C), dtype=np.float64) if with_abs else None
    f64p = ctypes.POINTER(ctypes.c_double)
    rc = lib.oracle_wgrad_rows(dyp, xp, N, H, W, C, K, R, S, stride, pad,
                               rr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), len(rr),
                               out.ctypes.data_as(f64p), mag.ctypes.data_as(f64p) if with_abs else None,
                               int(threads))
    if rc != 0:
        raise ValueError(f"oracle_wgrad failed with code {rc}")
    del dyk, xk
    if rows is None:
        out = out.reshape(K, R, S, C)
        mag = mag.reshape(K, R, S, C) if with_abs else None
    return (out, mag) if with_abs else out


def forward(x, w, bias, stride, pad, act=1, rows=None, threads=0, lib=None):
    """fp64 forward layer of float16 x [N,H,W,C], w [K,R,S,C], bias [K]:
    z = bias + conv(x, w) and y = hardswish(z) (act=1) or z (act=0).

    Returns (z, y) of shape [N,P,Q,K], or [len(rows), K] when ``rows`` (linear
    output pixels (n*P + p)*Q + q) is given.
    """
    lib = lib or load()
    N, H, W, C = x.shape
    K, R, S, C2 = w.shape
    if C2 != C or tuple(bias.shape) != (K,):
        raise ValueError("x, w and bias disagree on C or K")
    P, Q = lib.oracle_out_extent(H, R, stride, pad), lib.oracle_out_extent(W, S, stride, pad)
    xk, xp = _u16(x)
    wk, wp = _u16(w)
    bk, bp = _u16(bias)
    rr = np.arange(N * P * Q, dtype=np.int64) if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    z = np.empty((len(rr), K), dtype=np.float64)
    y = np.empty((len(rr), K), dtype=np.float64)
    f64p = ctypes.POINTER(ctypes.c_double)
    rc = lib.oracle_forward_rows(xp, wp, bp, N, H, W, C, K, R, S, stride, pad, act,
                                 rr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), len(rr),
                                 z.ctypes.data_as(f64p), y.ctypes.data_as(f64p), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_forward failed with code {rc}")
    del xk, wk, bk
    if rows is None:
        return z.reshape(N, P, Q, K), y.reshape(N, P, Q, K)
    return z, y


def chain(dy, w1, z, w2, H, W, pad, epilogue=EPI_NONE, rows=None, with_abs=False, threads=0, lib=None):
    """fp64 chain of two dgrad steps: t = fp16(dgrad(dy, w1; stride 1, pad) * g(z)),
    then dx = t @ w2 over the Cm channels.

    dy [N,P,Q,K], w1 [K,R,S,Cm], z [N,H,W,Cm] (for an epilogue), w2 [Cm,1,1,C]
    or [Cm,C], all float16. Returns dx [N,H,W,C] float64 (unrounded), or
    [len(rows), C] for linear pixel indices ``rows``; with ``with_abs`` also
    sum_c |t||w2| of the same shape.
    """
    lib = lib or load()
    N, P, Q, K = dy.shape
    K2, R, S, Cm = w1.shape
    w2m = np.asarray(w2).reshape(w2.shape[0], -1)
    if K2 != K or w2m.shape[0] != Cm:
        raise ValueError("dy, w1 and w2 disagree on K or Cm")
    C = w2m.shape[1]
    if (lib.oracle_out_extent(H, R, 1, pad), lib.oracle_out_extent(W, S, 1, pad)) != (P, Q):
        raise ValueError("dy spatial shape does not match H, W, R, S, pad at stride 1")
    dyk, dyp = _u16(dy)
    w1k, w1p = _u16(w1)
    w2k, w2p = _u16(np.ascontiguousarray(w2m))
    zk = zp = None
    if epilogue != EPI_NONE:
        if z is None or tuple(z.shape) != (N, H, W, Cm):
            raise ValueError("epilogue needs z of shape [N,H,W,Cm]")
        zk, zp = _u16(z)
    rr = np.arange(N * H * W, dtype=np.int64) if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    out = np.empty((len(rr), C), dtype=np.float64)
    mag = np.empty((len(rr), C), dtype=np.float64) if with_abs else None
    f64p = ctypes.POINTER(ctypes.c_double)
    rc = lib.oracle_chain_rows(dyp, w1p, zp, w2p, N, H, W, Cm, K, R, S, pad, C, epilogue,
                               rr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), len(rr),
                               out.ctypes.data_as(f64p), mag.ctypes.data_as(f64p) if with_abs else None,
                               int(threads))
    if rc != 0:
        raise ValueError(f"oracle_chain failed with code {rc}")
    del dyk, w1k, w2k, zk
    if rows is None:
        out = out.reshape(N, H, W, C)
        mag = mag.reshape(N, H, W, C) if with_abs else None
    return (out, mag) if with_abs else out


def hardswish(zv: float, lib=None) -> float:
    return (lib or load()).oracle_hardswish(zv)


def round_to_half(x, lib=None) -> np.ndarray:
    """RNE fp16 encoding of an fp64 array, returned as float16."""
    lib = lib or load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    lib.oracle_round_to_half(x.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                             out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)), x.size)
    return out.view(np.float16)


def half_to_double(bits: int, lib=None) -> float:
    return (lib or load()).oracle_half_to_double(bits)


def hardswish_grad(zv: float, lib=None) -> float:
    return (lib or load()).oracle_hardswish_grad(zv)


def relu_grad(zv: float, lib=None) -> float:
    return (lib or load()).oracle_relu_grad(zv)


def max_threads(lib=None) -> int:
    return (lib or load()).oracle_max_threads()
