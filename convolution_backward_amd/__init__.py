"""Python binding of libconv2d_dgrad.so, the MI355X conv2d backward-data library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/conv2d_dgrad.h``. PyTorch
supplies device memory and the current stream. There is no CPU fallback: if
the library is missing, every call raises.

The functions carry the C ABI's names. Tensor arguments may be torch tensors
(float16, contiguous, on the GPU) or raw device addresses (int).
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libconv2d_dgrad.so")

OK = 0
INVALID_ARGUMENT = 1
UNSUPPORTED = 2
HIP_ERROR = 3

EPI_NONE = 0
EPI_DRELU = 1
EPI_DHARDSWISH = 2


class DgradError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"conv2d_dgrad status {code}: {message}")
        self.code = code


class _Phase(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("ph", "pw", "Hp", "Wp", "r0", "t0", "nr", "nt", "dr0", "dt0")] + [
        ("M", ctypes.c_longlong), ("Kg", ctypes.c_longlong)]


_lib = None


def _bind(lib):
    vp, i = ctypes.c_void_p, ctypes.c_int
    ip = ctypes.POINTER(ctypes.c_int)
    lib.conv2d_dgrad_nhwc.argtypes = [vp, vp, vp] + [i] * 10 + [vp, vp]
    lib.conv2d_dgrad_nhwc_config.argtypes = [vp, vp, vp] + [i] * 10 + [vp, i, vp]
    lib.conv2d_dgrad_num_configs.argtypes = []
    lib.conv2d_dgrad_config_name.argtypes = [i, ctypes.c_char_p, i]
    lib.conv2d_dgrad_query_config.argtypes = [i] * 10 + [ip, ip]
    lib.conv2d_dgrad_set_autotune.argtypes = [i]
    lib.conv2d_dgrad_set_streamk.argtypes = [i]
    lib.conv2d_dgrad_streamk_launches.argtypes = []
    lib.conv2d_dgrad_streamk_launches.restype = ctypes.c_longlong
    lib.conv2d_dgrad_cache_clear.argtypes = []
    lib.conv2d_dgrad_cache_size.argtypes = []
    lib.conv2d_dgrad_cache_save.argtypes = [ctypes.c_char_p]
    lib.conv2d_dgrad_cache_load.argtypes = [ctypes.c_char_p]
    lib.conv2d_dgrad_plan.argtypes = [i] * 9 + [ctypes.POINTER(_Phase), i, ip, ip, ip]
    lib.conv2d_dgrad_check.argtypes = [vp, vp, vp] + [i] * 10 + [vp]
    lib.conv2d_wgrad_nhwc.argtypes = [vp, vp, vp] + [i] * 9 + [vp]
    lib.conv2d_wgrad_nhwc_config.argtypes = [vp, vp, vp] + [i] * 9 + [i, i, vp]
    lib.conv2d_wgrad_num_configs.argtypes = []
    lib.conv2d_wgrad_check.argtypes = [vp, vp, vp] + [i] * 9
    lib.conv2d_forward_nhwc.argtypes = [vp] * 5 + [i] * 10 + [vp]
    lib.conv2d_forward_nhwc_config.argtypes = [vp] * 5 + [i] * 10 + [i, vp]
    lib.conv2d_forward_num_configs.argtypes = []
    lib.conv2d_forward_check.argtypes = [vp] * 5 + [i] * 10
    lib.conv2d_dgrad_chain_nhwc.argtypes = [vp] * 5 + [i] * 10 + [vp]
    lib.conv2d_dgrad_chain_check.argtypes = [vp] * 5 + [i] * 10
    lib.conv2d_dgrad_last_error.argtypes = []
    lib.conv2d_dgrad_last_error.restype = ctypes.c_char_p
    lib.conv2d_dgrad_build_info.argtypes = []
    lib.conv2d_dgrad_build_info.restype = ctypes.c_char_p
    for name in ("conv2d_dgrad_nhwc", "conv2d_dgrad_nhwc_config", "conv2d_dgrad_num_configs",
                 "conv2d_dgrad_config_name", "conv2d_dgrad_query_config", "conv2d_dgrad_set_autotune",
                 "conv2d_dgrad_set_streamk", "conv2d_dgrad_streamk_launches", "conv2d_dgrad_cache_clear", "conv2d_dgrad_cache_size", "conv2d_dgrad_cache_save",
                 "conv2d_dgrad_cache_load", "conv2d_dgrad_plan", "conv2d_dgrad_check",
                 "conv2d_wgrad_nhwc", "conv2d_wgrad_nhwc_config", "conv2d_wgrad_num_configs", "conv2d_wgrad_check",
                 "conv2d_forward_nhwc", "conv2d_forward_nhwc_config", "conv2d_forward_num_configs",
                 "conv2d_forward_check", "conv2d_dgrad_chain_nhwc", "conv2d_dgrad_chain_check"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


def get_lib():
    """The loaded HIP library; raises if it has not been built.

    PyTorch carries its own HIP runtime (same soname as ROCm's). It is loaded
    first so that this library binds to that one runtime instead of bringing
    a second copy into the process."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m convolution_backward_amd.build` (hipcc, gfx950)")
        try:
            import torch  # noqa: F401  (loads the HIP runtime the tensors live in)
        except ImportError:
            pass
        _lib = _bind(ctypes.CDLL(LIB_PATH))
    return _lib


def _check(rc: int) -> int:
    if rc != OK:
        raise DgradError(rc, get_lib().conv2d_dgrad_last_error().decode())
    return rc


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream, *tensors):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    for t in tensors:
        if t is not None and not isinstance(t, int):
            import torch
            if t.is_cuda:
                return torch.cuda.current_stream(t.device).cuda_stream
    return 0


def conv2d_dgrad_nhwc(dy, w, dx, N, H, W, C, K, R, S, stride, pad, epilogue=EPI_NONE, z=None, stream=None):
    """dx = dgrad(dy, w) [* g(z)], enqueued on `stream` (default: torch's current stream)."""
    lib = get_lib()
    return _check(lib.conv2d_dgrad_nhwc(_ptr(dy), _ptr(w), _ptr(dx), N, H, W, C, K, R, S, stride, pad,
                                        epilogue, _ptr(z), _stream(stream, dy, dx)))


def conv2d_dgrad_nhwc_config(dy, w, dx, N, H, W, C, K, R, S, stride, pad, epilogue=EPI_NONE, z=None,
                             config_id=0, stream=None):
    lib = get_lib()
    return _check(lib.conv2d_dgrad_nhwc_config(_ptr(dy), _ptr(w), _ptr(dx), N, H, W, C, K, R, S, stride, pad,
                                               epilogue, _ptr(z), config_id, _stream(stream, dy, dx)))


def conv2d_dgrad_check(dy, w, dx, N, H, W, C, K, R, S, stride, pad, epilogue=EPI_NONE, z=None) -> int:
    """Validation only: the status code, no exception, no HIP call."""
    return get_lib().conv2d_dgrad_check(_ptr(dy), _ptr(w), _ptr(dx), N, H, W, C, K, R, S, stride, pad,
                                        epilogue, _ptr(z))


def conv2d_wgrad_nhwc(dy, x, dw, N, H, W, C, K, R, S, stride, pad, stream=None):
    """dw (fp32 [K,R,S,C]) = wgrad(dy, x), enqueued on `stream` (default: torch's current stream)."""
    return _check(get_lib().conv2d_wgrad_nhwc(_ptr(dy), _ptr(x), _ptr(dw), N, H, W, C, K, R, S, stride, pad,
                                              _stream(stream, dy, dw)))


def conv2d_wgrad_nhwc_config(dy, x, dw, N, H, W, C, K, R, S, stride, pad, config_id=0, splits=0, stream=None):
    return _check(get_lib().conv2d_wgrad_nhwc_config(_ptr(dy), _ptr(x), _ptr(dw), N, H, W, C, K, R, S, stride,
                                                     pad, config_id, splits, _stream(stream, dy, dw)))


def conv2d_wgrad_check(dy, x, dw, N, H, W, C, K, R, S, stride, pad) -> int:
    """Validation only: the status code, no exception, no HIP call."""
    return get_lib().conv2d_wgrad_check(_ptr(dy), _ptr(x), _ptr(dw), N, H, W, C, K, R, S, stride, pad)


def conv2d_wgrad_num_configs() -> int:
    return get_lib().conv2d_wgrad_num_configs()


def wgrad(dy, x, R, S, stride, pad, config_id=None, splits=0, out=None):
    """Allocate dw [K,R,S,C] float32 with torch.empty and fill it on the current stream.

    dy [N,P,Q,K] and x [N,H,W,C] are float16 GPU tensors.
    """
    import torch
    for name, t in (("dy", dy), ("x", x)):
        if t.dtype != torch.float16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float16 GPU tensor")
    N, _, _, K = dy.shape
    N2, H, W, C = x.shape
    if N2 != N:
        raise ValueError("dy and x disagree on N")
    dw = out if out is not None else torch.empty((K, R, S, C), dtype=torch.float32, device=dy.device)
    if config_id is None and splits == 0:
        conv2d_wgrad_nhwc(dy, x, dw, N, H, W, C, K, R, S, stride, pad)
    else:
        conv2d_wgrad_nhwc_config(dy, x, dw, N, H, W, C, K, R, S, stride, pad,
                                 0 if config_id is None else config_id, splits)
    return dw


ACT_NONE, ACT_HARDSWISH = 0, 1


def conv2d_forward_nhwc(x, w, bias, z, y, N, H, W, C, K, R, S, stride, pad, act=ACT_HARDSWISH, stream=None):
    """z = bias + conv(x, w) (if z is given) and y = act(z), enqueued on `stream`."""
    return _check(get_lib().conv2d_forward_nhwc(_ptr(x), _ptr(w), _ptr(bias), _ptr(z), _ptr(y), N, H, W, C, K, R,
                                                S, stride, pad, act, _stream(stream, x, y)))


def conv2d_forward_nhwc_config(x, w, bias, z, y, N, H, W, C, K, R, S, stride, pad, act=ACT_HARDSWISH,
                               config_id=0, stream=None):
    return _check(get_lib().conv2d_forward_nhwc_config(_ptr(x), _ptr(w), _ptr(bias), _ptr(z), _ptr(y), N, H, W, C,
                                                       K, R, S, stride, pad, act, config_id, _stream(stream, x, y)))


def conv2d_forward_check(x, w, bias, z, y, N, H, W, C, K, R, S, stride, pad, act=ACT_HARDSWISH) -> int:
    """Validation only: the status code, no exception, no HIP call."""
    return get_lib().conv2d_forward_check(_ptr(x), _ptr(w), _ptr(bias), _ptr(z), _ptr(y), N, H, W, C, K, R, S,
                                          stride, pad, act)


def conv2d_forward_num_configs() -> int:
    return get_lib().conv2d_forward_num_configs()


def forward(x, w, bias, stride, pad, act=ACT_HARDSWISH, with_z=True, config_id=None, out=None, z_out=None):
    """Allocate y (and z) [N,P,Q,K] float16 with torch.empty and fill them on the
    current stream. Returns (z, y) (z is None when with_z is False).

    x [N,H,W,C], w [K,R,S,C] and bias [K] are float16 GPU tensors.
    """
    import torch
    for name, t in (("x", x), ("w", w), ("bias", bias)):
        if t.dtype != torch.float16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float16 GPU tensor")
    N, H, W, C = x.shape
    K, R, S, C2 = w.shape
    if C2 != C:
        raise ValueError("x and w disagree on C")
    P, Q = (H + 2 * pad - R) // stride + 1, (W + 2 * pad - S) // stride + 1
    y = out if out is not None else torch.empty((N, P, Q, K), dtype=torch.float16, device=x.device)
    z = None
    if with_z:
        z = z_out if z_out is not None else torch.empty((N, P, Q, K), dtype=torch.float16, device=x.device)
    if config_id is None:
        conv2d_forward_nhwc(x, w, bias, z, y, N, H, W, C, K, R, S, stride, pad, act)
    else:
        conv2d_forward_nhwc_config(x, w, bias, z, y, N, H, W, C, K, R, S, stride, pad, act, config_id)
    return z, y


def conv2d_dgrad_chain_nhwc(dy, w1, z, w2, dx, N, H, W, Cm, K, R, S, pad, C, epilogue=EPI_NONE, stream=None):
    """Two dgrad steps of a bottleneck in one kernel: t = fp16(dgrad(dy, w1) * g(z))
    at stride 1, then dx = t @ w2 (the 1x1 step), enqueued on `stream`."""
    return _check(get_lib().conv2d_dgrad_chain_nhwc(_ptr(dy), _ptr(w1), _ptr(z), _ptr(w2), _ptr(dx), N, H, W, Cm, K,
                                                    R, S, pad, C, epilogue, _stream(stream, dy, dx)))


def conv2d_dgrad_chain_check(dy, w1, z, w2, dx, N, H, W, Cm, K, R, S, pad, C, epilogue=EPI_NONE) -> int:
    """Validation alone; returns the status code (no exception)."""
    return get_lib().conv2d_dgrad_chain_check(_ptr(dy), _ptr(w1), _ptr(z), _ptr(w2), _ptr(dx), N, H, W, Cm, K, R, S,
                                              pad, C, epilogue)


def dgrad_chain(dy, w1, z, w2, pad, epilogue=EPI_NONE, out=None):
    """Allocate dx [N,H,W,C] float16 with torch.empty (unless `out` is given)
    and fill it on the current stream with the fused chain.

    dy [N,P,Q,K], w1 [K,R,S,Cm], z [N,H,W,Cm] (or None for EPI_NONE) and
    w2 [Cm,1,1,C] are float16 GPU tensors; H = P - 2*pad + R - 1 (stride 1).
    """
    import torch
    for name, t in (("dy", dy), ("w1", w1), ("w2", w2)) + ((("z", z),) if z is not None else ()):
        if t.dtype != torch.float16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float16 GPU tensor")
    N, P, Q, K = dy.shape
    K2, R, S, Cm = w1.shape
    if K2 != K or w2.shape[0] != Cm or w2.dim() != 4 or tuple(w2.shape[1:3]) != (1, 1):
        raise ValueError("dy, w1 and w2 [Cm,1,1,C] disagree on K or Cm")
    C = w2.shape[3]
    H, W = P - 2 * pad + R - 1, Q - 2 * pad + S - 1
    dx = out if out is not None else torch.empty((N, H, W, C), dtype=torch.float16, device=dy.device)
    conv2d_dgrad_chain_nhwc(dy, w1, z, w2, dx, N, H, W, Cm, K, R, S, pad, C, epilogue)
    return dx


def conv2d_dgrad_num_configs() -> int:
    return get_lib().conv2d_dgrad_num_configs()


def conv2d_dgrad_config_name(config_id: int) -> str:
    buf = ctypes.create_string_buffer(64)
    _check(get_lib().conv2d_dgrad_config_name(config_id, buf, len(buf)))
    return buf.value.decode()


def conv2d_dgrad_query_config(N, H, W, C, K, R, S, stride, pad, epilogue=EPI_NONE):
    """(config_id, cached) for a problem key, without launching."""
    cid, cached = ctypes.c_int(), ctypes.c_int()
    _check(get_lib().conv2d_dgrad_query_config(N, H, W, C, K, R, S, stride, pad, epilogue,
                                               ctypes.byref(cid), ctypes.byref(cached)))
    return cid.value, bool(cached.value)


def conv2d_dgrad_set_autotune(on: bool) -> bool:
    return bool(get_lib().conv2d_dgrad_set_autotune(1 if on else 0))


def conv2d_dgrad_set_streamk(mode: int) -> int:
    """0 never split the reduction, 1 whenever eligible, 2 (default) when it pays;
    returns the previous mode."""
    prev = get_lib().conv2d_dgrad_set_streamk(int(mode))
    if prev < 0:
        raise DgradError(INVALID_ARGUMENT, conv2d_dgrad_last_error())
    return prev


def conv2d_dgrad_streamk_launches() -> int:
    """Kernel launches enqueued with a stream-K split since the library loaded."""
    return int(get_lib().conv2d_dgrad_streamk_launches())


def conv2d_dgrad_cache_clear():
    return _check(get_lib().conv2d_dgrad_cache_clear())


def conv2d_dgrad_cache_size() -> int:
    return get_lib().conv2d_dgrad_cache_size()


def conv2d_dgrad_cache_save(path: str):
    return _check(get_lib().conv2d_dgrad_cache_save(os.fsencode(path)))


def conv2d_dgrad_cache_load(path: str):
    return _check(get_lib().conv2d_dgrad_cache_load(os.fsencode(path)))


def conv2d_dgrad_plan(N, H, W, C, K, R, S, stride, pad):
    """(P, Q, phases): the stride-phase plan, heaviest phase first."""
    lib = get_lib()
    n, P, Q = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    arr = (_Phase * 256)()
    _check(lib.conv2d_dgrad_plan(N, H, W, C, K, R, S, stride, pad, arr, 256,
                                 ctypes.byref(n), ctypes.byref(P), ctypes.byref(Q)))
    phases = [{f: getattr(arr[i], f) for f, _ in _Phase._fields_} for i in range(min(n.value, 256))]
    return P.value, Q.value, phases


def conv2d_dgrad_last_error() -> str:
    return get_lib().conv2d_dgrad_last_error().decode()


def conv2d_dgrad_build_info() -> str:
    return get_lib().conv2d_dgrad_build_info().decode()


def dgrad(dy, w, H, W, stride, pad, epilogue=EPI_NONE, z=None, config_id=None, out=None):
    """Allocate dx [N,H,W,C] with torch.empty and fill it on the current stream.

    dy [N,P,Q,K] and w [K,R,S,C] (and z [N,H,W,C]) are float16 GPU tensors.
    """
    import torch
    for name, t in (("dy", dy), ("w", w), ("z", z)):
        if t is None:
            continue
        if t.dtype != torch.float16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float16 GPU tensor")
    N, _, _, K = dy.shape
    K2, R, S, C = w.shape
    if K2 != K:
        raise ValueError("dy and w disagree on K")
    dx = out if out is not None else torch.empty((N, H, W, C), dtype=torch.float16, device=dy.device)
    if config_id is None:
        conv2d_dgrad_nhwc(dy, w, dx, N, H, W, C, K, R, S, stride, pad, epilogue, z)
    else:
        conv2d_dgrad_nhwc_config(dy, w, dx, N, H, W, C, K, R, S, stride, pad, epilogue, z, config_id)
    return dx


__all__ = [
    "conv2d_dgrad_nhwc", "conv2d_dgrad_nhwc_config", "conv2d_dgrad_check", "conv2d_dgrad_num_configs",
    "conv2d_dgrad_config_name", "conv2d_dgrad_query_config", "conv2d_dgrad_set_autotune",
    "conv2d_dgrad_set_streamk", "conv2d_dgrad_streamk_launches",
    "conv2d_dgrad_cache_clear", "conv2d_dgrad_cache_size", "conv2d_dgrad_cache_save", "conv2d_dgrad_cache_load",
    "conv2d_dgrad_plan", "conv2d_dgrad_last_error", "conv2d_dgrad_build_info", "dgrad", "get_lib",
    "conv2d_wgrad_nhwc", "conv2d_wgrad_nhwc_config", "conv2d_wgrad_check", "conv2d_wgrad_num_configs", "wgrad",
    "conv2d_forward_nhwc", "conv2d_forward_nhwc_config", "conv2d_forward_check", "conv2d_forward_num_configs",
    "forward", "ACT_NONE", "ACT_HARDSWISH",
    "DgradError", "EPI_NONE", "EPI_DRELU", "EPI_DHARDSWISH",
]
