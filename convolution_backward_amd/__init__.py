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
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    ip = ctypes.POINTER(ctypes.c_int)
    szp = ctypes.POINTER(ctypes.c_size_t)
    lib.conv2d_dgrad_nhwc.argtypes = [vp, vp, vp] + [i] * 10 + [vp, vp]
    lib.conv2d_dgrad_nhwc_ws.argtypes = [vp, vp, vp] + [i] * 10 + [vp, vp, sz, vp]
    lib.conv2d_dgrad_workspace_size.argtypes = [i] * 10 + [szp]
    lib.conv2d_dgrad_nhwc_noalloc.argtypes = [vp, vp, vp] + [i] * 10 + [vp, vp]
    lib.conv2d_dgrad_noalloc_max_bytes.argtypes = []
    lib.conv2d_dgrad_noalloc_max_bytes.restype = ctypes.c_size_t
    lib.conv2d_dgrad_nhwc_config.argtypes = [vp, vp, vp] + [i] * 10 + [vp, i, vp, sz, vp]
    lib.conv2d_dgrad_num_configs.argtypes = []
    lib.conv2d_dgrad_config_name.argtypes = [i, ctypes.c_char_p, i]
    lib.conv2d_dgrad_query_config.argtypes = [i] * 11 + [ip, ip, ip]
    lib.conv2d_dgrad_set_autotune.argtypes = [i]
    lib.conv2d_dgrad_set_fault_inject.argtypes = [i]
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
    lib.conv2d_wgrad_nhwc_ws.argtypes = [vp, vp, vp] + [i] * 9 + [vp, sz, vp]
    lib.conv2d_wgrad_workspace_size.argtypes = [i] * 9 + [szp]
    lib.conv2d_wgrad_nhwc_config.argtypes = [vp, vp, vp] + [i] * 9 + [i, i, vp, sz, vp]
    lib.conv2d_wgrad_num_configs.argtypes = []
    lib.conv2d_wgrad_check.argtypes = [vp, vp, vp] + [i] * 9
    lib.conv2d_forward_nhwc.argtypes = [vp] * 5 + [i] * 10 + [vp]
    lib.conv2d_forward_nhwc_config.argtypes = [vp] * 5 + [i] * 10 + [i, vp]
    lib.conv2d_forward_num_configs.argtypes = []
    lib.conv2d_forward_check.argtypes = [vp] * 5 + [i] * 10
    lib.conv2d_dgrad_chain_nhwc.argtypes = [vp] * 5 + [i] * 10 + [vp]
    lib.conv2d_dgrad_chain_nhwc_ws.argtypes = [vp] * 5 + [i] * 10 + [vp, sz, vp]
    lib.conv2d_dgrad_chain_workspace_size.argtypes = [i] * 10 + [szp]
    lib.conv2d_dgrad_chain_query.argtypes = [i] * 10 + [ip, ip]
    lib.conv2d_dgrad_chain_check.argtypes = [vp] * 5 + [i] * 10
    lib.conv2d_dgrad_last_error.argtypes = []
    lib.conv2d_dgrad_last_error.restype = ctypes.c_char_p
    lib.conv2d_dgrad_build_info.argtypes = []
    lib.conv2d_dgrad_build_info.restype = ctypes.c_char_p
    for name in ("conv2d_dgrad_nhwc", "conv2d_dgrad_nhwc_ws", "conv2d_dgrad_workspace_size", "conv2d_dgrad_nhwc_noalloc",
                 "conv2d_dgrad_nhwc_config", "conv2d_dgrad_num_configs",
                 "conv2d_dgrad_config_name", "conv2d_dgrad_query_config", "conv2d_dgrad_set_autotune",
                 "conv2d_dgrad_set_fault_inject", "conv2d_wgrad_nhwc_ws", "conv2d_wgrad_workspace_size",
                 "conv2d_dgrad_set_streamk", "conv2d_dgrad_streamk_launches", "conv2d_dgrad_cache_clear", "conv2d_dgrad_cache_size", "conv2d_dgrad_cache_save",
                 "conv2d_dgrad_cache_load", "conv2d_dgrad_plan", "conv2d_dgrad_check",
                 "conv2d_wgrad_nhwc", "conv2d_wgrad_nhwc_config", "conv2d_wgrad_num_configs", "conv2d_wgrad_check",
                 "conv2d_forward_nhwc", "conv2d_forward_nhwc_config", "conv2d_forward_num_configs",
                 "conv2d_forward_check", "conv2d_dgrad_chain_nhwc", "conv2d_dgrad_chain_check",
                 "conv2d_dgrad_chain_nhwc_ws", "conv2d_dgrad_chain_workspace_size", "conv2d_dgrad_chain_query"):
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


def _ws(workspace):
    """(pointer, bytes) of an optional workspace tensor."""
    if workspace is None:
        return None, 0
    if isinstance(workspace, tuple):
        return workspace
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


# ------------------------------------------------------------------ raw C ABI

def conv2d_dgrad_nhwc(dy, w, dx, N, H, W, C, K, R, S, stride, pad, epilogue=EPI_NONE, z=None, stream=None):
    """dx = dgrad(dy, w) [* g(z)], enqueued on `stream` (default: torch's current stream)."""
    lib = get_lib()
    return _check(lib.conv2d_dgrad_nhwc(_ptr(dy), _ptr(w), _ptr(dx), N, H, W, C, K, R, S, stride, pad,
                                        epilogue, _ptr(z), _stream(stream, dy, dx)))


def conv2d_dgrad_nhwc_ws(dy, w, dx, N, H, W, C, K, R, S, stride, pad, epilogue=EPI_NONE, z=None,
                         workspace=None, stream=None):
    """conv2d_dgrad_nhwc with a caller-owned workspace (a tensor, or a (pointer, bytes) pair)."""
    wp, wb = _ws(workspace)
    return _check(get_lib().conv2d_dgrad_nhwc_ws(_ptr(dy), _ptr(w), _ptr(dx), N, H, W, C, K, R, S, stride, pad,
                                                 epilogue, _ptr(z), wp, wb, _stream(stream, dy, dx)))


def conv2d_dgrad_nhwc_noalloc(dy, w, dx, N, H, W, C, K, R, S, stride, pad, epilogue=EPI_NONE, z=None, stream=None):
    """conv2d_dgrad_nhwc_ws with the library's static per-device scratch as the
    workspace: allocates nothing (for callers that cannot allocate)."""
    return _check(get_lib().conv2d_dgrad_nhwc_noalloc(_ptr(dy), _ptr(w), _ptr(dx), N, H, W, C, K, R, S, stride, pad,
                                                      epilogue, _ptr(z), _stream(stream, dy, dx)))


def conv2d_dgrad_noalloc_max_bytes() -> int:
    return int(get_lib().conv2d_dgrad_noalloc_max_bytes())


def conv2d_dgrad_workspace_size(N, H, W, C, K, R, S, stride, pad, epilogue=EPI_NONE) -> int:
    """Workspace bytes that let every candidate of the problem split its reduction (0: none splits)."""
    b = ctypes.c_size_t()
    _check(get_lib().conv2d_dgrad_workspace_size(N, H, W, C, K, R, S, stride, pad, epilogue, ctypes.byref(b)))
    return b.value


def conv2d_dgrad_nhwc_config(dy, w, dx, N, H, W, C, K, R, S, stride, pad, epilogue=EPI_NONE, z=None,
                             config_id=0, workspace=None, stream=None):
    wp, wb = _ws(workspace)
    return _check(get_lib().conv2d_dgrad_nhwc_config(_ptr(dy), _ptr(w), _ptr(dx), N, H, W, C, K, R, S, stride,
                                                     pad, epilogue, _ptr(z), config_id, wp, wb,
                                                     _stream(stream, dy, dx)))


def conv2d_dgrad_check(dy, w, dx, N, H, W, C, K, R, S, stride, pad, epilogue=EPI_NONE, z=None) -> int:
    """Validation only: the status code, no exception, no HIP call."""
    return get_lib().conv2d_dgrad_check(_ptr(dy), _ptr(w), _ptr(dx), N, H, W, C, K, R, S, stride, pad,
                                        epilogue, _ptr(z))


def conv2d_wgrad_nhwc(dy, x, dw, N, H, W, C, K, R, S, stride, pad, stream=None):
    """dw (fp32 [K,R,S,C]) = wgrad(dy, x), enqueued on `stream` (default: torch's current stream)."""
    return _check(get_lib().conv2d_wgrad_nhwc(_ptr(dy), _ptr(x), _ptr(dw), N, H, W, C, K, R, S, stride, pad,
                                              _stream(stream, dy, dw)))


def conv2d_wgrad_nhwc_ws(dy, x, dw, N, H, W, C, K, R, S, stride, pad, workspace=None, stream=None):
    wp, wb = _ws(workspace)
    return _check(get_lib().conv2d_wgrad_nhwc_ws(_ptr(dy), _ptr(x), _ptr(dw), N, H, W, C, K, R, S, stride, pad,
                                                 wp, wb, _stream(stream, dy, dw)))


def conv2d_wgrad_workspace_size(N, H, W, C, K, R, S, stride, pad) -> int:
    b = ctypes.c_size_t()
    _check(get_lib().conv2d_wgrad_workspace_size(N, H, W, C, K, R, S, stride, pad, ctypes.byref(b)))
    return b.value


def conv2d_wgrad_nhwc_config(dy, x, dw, N, H, W, C, K, R, S, stride, pad, config_id=0, splits=0,
                             workspace=None, stream=None):
    wp, wb = _ws(workspace)
    return _check(get_lib().conv2d_wgrad_nhwc_config(_ptr(dy), _ptr(x), _ptr(dw), N, H, W, C, K, R, S, stride,
                                                     pad, config_id, splits, wp, wb, _stream(stream, dy, dw)))


def conv2d_wgrad_check(dy, x, dw, N, H, W, C, K, R, S, stride, pad) -> int:
    """Validation only: the status code, no exception, no HIP call."""
    return get_lib().conv2d_wgrad_check(_ptr(dy), _ptr(x), _ptr(dw), N, H, W, C, K, R, S, stride, pad)


def conv2d_wgrad_num_configs() -> int:
    return get_lib().conv2d_wgrad_num_configs()


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


def conv2d_dgrad_chain_nhwc(dy, w1, z, w2, dx, N, H, W, Cm, K, R, S, pad, C, epilogue=EPI_NONE, stream=None):
    """Two dgrad steps of a bottleneck in one kernel: t = fp16(dgrad(dy, w1) * g(z))
    at stride 1, then dx = t @ w2 (the 1x1 step), enqueued on `stream`."""
    return _check(get_lib().conv2d_dgrad_chain_nhwc(_ptr(dy), _ptr(w1), _ptr(z), _ptr(w2), _ptr(dx), N, H, W, Cm, K,
                                                    R, S, pad, C, epilogue, _stream(stream, dy, dx)))


def conv2d_dgrad_chain_nhwc_ws(dy, w1, z, w2, dx, N, H, W, Cm, K, R, S, pad, C, epilogue=EPI_NONE, workspace=None,
                               stream=None):
    """The chain with a caller-owned workspace: where it holds t, the faster of
    the fused kernel and the two-call pair runs (chosen once per problem)."""
    wp, wb = _ws(workspace)
    return _check(get_lib().conv2d_dgrad_chain_nhwc_ws(_ptr(dy), _ptr(w1), _ptr(z), _ptr(w2), _ptr(dx), N, H, W, Cm,
                                                       K, R, S, pad, C, epilogue, wp, wb, _stream(stream, dy, dx)))


def conv2d_dgrad_chain_workspace_size(N, H, W, Cm, K, R, S, pad, C, epilogue=EPI_NONE) -> int:
    b = ctypes.c_size_t()
    _check(get_lib().conv2d_dgrad_chain_workspace_size(N, H, W, Cm, K, R, S, pad, C, epilogue, ctypes.byref(b)))
    return b.value


def conv2d_dgrad_chain_query(N, H, W, Cm, K, R, S, pad, C, epilogue=EPI_NONE):
    """(pair, cached): the chain path cached for this problem on the current device."""
    pair, cached = ctypes.c_int(), ctypes.c_int()
    _check(get_lib().conv2d_dgrad_chain_query(N, H, W, Cm, K, R, S, pad, C, epilogue, ctypes.byref(pair),
                                              ctypes.byref(cached)))
    return bool(pair.value), bool(cached.value)


def conv2d_dgrad_chain_check(dy, w1, z, w2, dx, N, H, W, Cm, K, R, S, pad, C, epilogue=EPI_NONE) -> int:
    """Validation alone; returns the status code (no exception)."""
    return get_lib().conv2d_dgrad_chain_check(_ptr(dy), _ptr(w1), _ptr(z), _ptr(w2), _ptr(dx), N, H, W, Cm, K, R, S,
                                              pad, C, epilogue)


def conv2d_dgrad_num_configs() -> int:
    return get_lib().conv2d_dgrad_num_configs()


def conv2d_dgrad_config_name(config_id: int) -> str:
    buf = ctypes.create_string_buffer(64)
    _check(get_lib().conv2d_dgrad_config_name(config_id, buf, len(buf)))
    return buf.value.decode()


def conv2d_dgrad_query_config(N, H, W, C, K, R, S, stride, pad, epilogue=EPI_NONE, with_workspace=False,
                              with_split=False):
    """(config_id, cached) for a problem key, without launching; with
    ``with_split`` also whether the cached choice splits the reduction."""
    cid, cached, split = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(get_lib().conv2d_dgrad_query_config(N, H, W, C, K, R, S, stride, pad, epilogue, 1 if with_workspace else 0,
                                               ctypes.byref(cid), ctypes.byref(cached), ctypes.byref(split)))
    if with_split:
        return cid.value, bool(cached.value), bool(split.value)
    return cid.value, bool(cached.value)


def conv2d_dgrad_set_autotune(on: bool) -> bool:
    return bool(get_lib().conv2d_dgrad_set_autotune(1 if on else 0))


def conv2d_dgrad_set_fault_inject(on: bool) -> bool:
    """While on, every profiled candidate counts as failed (the heuristic's choice is kept)."""
    return bool(get_lib().conv2d_dgrad_set_fault_inject(1 if on else 0))


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


# ------------------------------------------------------------------ tensor API
#
# These check every tensor against the shape the C call will be told (the C
# side sizes each buffer's hardware range from the claimed shape, so a tensor
# smaller than claimed would be read or written past its end), then allocate
# outputs with torch.empty and launch on the current stream.

def _out_extent(n, f, stride, pad):
    # the forward layer's output size; it only sizes and checks tensors here
    return (n + 2 * pad - f) // stride + 1


def _check_tensor(name, t, shape, dtype, device=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def workspace(nbytes: int, device=None):
    """A zero-filled uint8 device tensor of `nbytes` (at least 64 KiB) to pass as
    `workspace`: PyTorch's allocator owns it; its counter area starts at zero
    as the C ABI requires, and every call leaves it so."""
    import torch
    return torch.zeros(max(int(nbytes), 65536), dtype=torch.uint8, device=device or "cuda")


def _check_ws(ws, device):
    import torch
    if ws is None:
        return
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or ws.device != device or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor on the same device as the inputs")


def dgrad_workspace(N, H, W, C, K, R, S, stride, pad, epilogue=EPI_NONE, device=None):
    """A zeroed workspace that lets every candidate of this dgrad problem split (None if none splits)."""
    n = conv2d_dgrad_workspace_size(N, H, W, C, K, R, S, stride, pad, epilogue)
    return workspace(n, device) if n > 0 else None


def wgrad_workspace(N, H, W, C, K, R, S, stride, pad, device=None):
    """A zeroed workspace for the largest wgrad split of this problem (None if none splits)."""
    n = conv2d_wgrad_workspace_size(N, H, W, C, K, R, S, stride, pad)
    return workspace(n, device) if n > 0 else None


def dgrad(dy, w, H, W, stride, pad, epilogue=EPI_NONE, z=None, config_id=None, out=None, workspace=None):
    """dx [N,H,W,C] = dgrad(dy, w) [* g(z)] on the current stream (allocated with
    torch.empty unless `out` is given).

    dy [N,P,Q,K] and w [K,R,S,C] (and z [N,H,W,C] for an epilogue) are
    contiguous float16 GPU tensors with P, Q the forward layer's output size
    for H, W, R, S, stride, pad. `workspace` (see ``dgrad_workspace``) lets
    small-tile problems split their reduction.
    """
    import torch
    if not isinstance(dy, torch.Tensor) or not isinstance(w, torch.Tensor) or dy.dim() != 4 or w.dim() != 4:
        raise ValueError("dy [N,P,Q,K] and w [K,R,S,C] must be 4-d torch tensors")
    N, K = dy.shape[0], dy.shape[3]
    K2, R, S, C = w.shape
    if K2 != K:
        raise ValueError("dy and w disagree on K")
    if stride < 1 or pad < 0:
        raise ValueError("stride must be >= 1 and pad >= 0")
    P, Q = _out_extent(H, R, stride, pad), _out_extent(W, S, stride, pad)
    dev = dy.device
    _check_tensor("dy", dy, (N, P, Q, K), torch.float16, dev)
    _check_tensor("w", w, (K, R, S, C), torch.float16, dev)
    if epilogue != EPI_NONE:
        if z is None:
            raise ValueError("the epilogue needs z")
        _check_tensor("z", z, (N, H, W, C), torch.float16, dev)
    else:
        z = None
    _check_ws(workspace, dev)
    if out is not None:
        _check_tensor("out", out, (N, H, W, C), torch.float16, dev)
    dx = out if out is not None else torch.empty((N, H, W, C), dtype=torch.float16, device=dev)
    if config_id is None:
        conv2d_dgrad_nhwc_ws(dy, w, dx, N, H, W, C, K, R, S, stride, pad, epilogue, z, workspace)
    else:
        conv2d_dgrad_nhwc_config(dy, w, dx, N, H, W, C, K, R, S, stride, pad, epilogue, z, config_id, workspace)
    return dx


def wgrad(dy, x, R, S, stride, pad, config_id=None, splits=0, out=None, workspace=None):
    """dw [K,R,S,C] float32 = wgrad(dy, x) on the current stream (allocated with
    torch.empty unless `out` is given).

    dy [N,P,Q,K] and x [N,H,W,C] are contiguous float16 GPU tensors, P and Q
    the forward output size. Without `workspace` (see ``wgrad_workspace``)
    each tile runs its whole reduction in one workgroup.
    """
    import torch
    if not isinstance(dy, torch.Tensor) or not isinstance(x, torch.Tensor) or dy.dim() != 4 or x.dim() != 4:
        raise ValueError("dy [N,P,Q,K] and x [N,H,W,C] must be 4-d torch tensors")
    N, _, _, K = dy.shape
    N2, H, W, C = x.shape
    if N2 != N:
        raise ValueError("dy and x disagree on N")
    if stride < 1 or pad < 0 or R < 1 or S < 1:
        raise ValueError("R, S, stride must be >= 1 and pad >= 0")
    P, Q = _out_extent(H, R, stride, pad), _out_extent(W, S, stride, pad)
    dev = dy.device
    _check_tensor("dy", dy, (N, P, Q, K), torch.float16, dev)
    _check_tensor("x", x, (N, H, W, C), torch.float16, dev)
    _check_ws(workspace, dev)
    if out is not None:
        _check_tensor("out", out, (K, R, S, C), torch.float32, dev)
    dw = out if out is not None else torch.empty((K, R, S, C), dtype=torch.float32, device=dev)
    if config_id is None and splits == 0:
        conv2d_wgrad_nhwc_ws(dy, x, dw, N, H, W, C, K, R, S, stride, pad, workspace)
    else:
        conv2d_wgrad_nhwc_config(dy, x, dw, N, H, W, C, K, R, S, stride, pad,
                                 0 if config_id is None else config_id, splits, workspace)
    return dw


def forward(x, w, bias, stride, pad, act=ACT_HARDSWISH, with_z=True, config_id=None, out=None, z_out=None):
    """(z, y), each [N,P,Q,K] float16, of the forward layer with its fused
    bias + activation epilogue, on the current stream (z is None when
    with_z is False; outputs allocated with torch.empty unless given).

    x [N,H,W,C], w [K,R,S,C] and bias [K] are contiguous float16 GPU tensors.
    """
    import torch
    if not isinstance(x, torch.Tensor) or not isinstance(w, torch.Tensor) or x.dim() != 4 or w.dim() != 4:
        raise ValueError("x [N,H,W,C] and w [K,R,S,C] must be 4-d torch tensors")
    N, H, W, C = x.shape
    K, R, S, C2 = w.shape
    if C2 != C:
        raise ValueError("x and w disagree on C")
    if stride < 1 or pad < 0:
        raise ValueError("stride must be >= 1 and pad >= 0")
    P, Q = _out_extent(H, R, stride, pad), _out_extent(W, S, stride, pad)
    dev = x.device
    _check_tensor("x", x, (N, H, W, C), torch.float16, dev)
    _check_tensor("w", w, (K, R, S, C), torch.float16, dev)
    _check_tensor("bias", bias, (K,), torch.float16, dev)
    if out is not None:
        _check_tensor("out", out, (N, P, Q, K), torch.float16, dev)
    if z_out is not None:
        _check_tensor("z_out", z_out, (N, P, Q, K), torch.float16, dev)
    y = out if out is not None else torch.empty((N, P, Q, K), dtype=torch.float16, device=dev)
    z = None
    if with_z:
        z = z_out if z_out is not None else torch.empty((N, P, Q, K), dtype=torch.float16, device=dev)
    if config_id is None:
        conv2d_forward_nhwc(x, w, bias, z, y, N, H, W, C, K, R, S, stride, pad, act)
    else:
        conv2d_forward_nhwc_config(x, w, bias, z, y, N, H, W, C, K, R, S, stride, pad, act, config_id)
    return z, y


def dgrad_chain(dy, w1, z, w2, pad, epilogue=EPI_NONE, out=None, workspace=None):
    """dx [N,H,W,C] float16 of the two-step chain on the current stream
    (allocated with torch.empty unless `out` is given): the fused kernel, or,
    with a `workspace` that holds t (``conv2d_dgrad_chain_workspace_size``),
    whichever of it and the two-call pair was timed faster for the problem.

    dy [N,P,Q,K], w1 [K,R,S,Cm], z [N,H,W,Cm] (for an epilogue) and
    w2 [Cm,1,1,C] are contiguous float16 GPU tensors; H = P - 2*pad + R - 1
    (stride 1).
    """
    import torch
    for name, t in (("dy", dy), ("w1", w1), ("w2", w2)):
        if not isinstance(t, torch.Tensor) or t.dim() != 4:
            raise ValueError(f"{name} must be a 4-d torch tensor")
    N, P, Q, K = dy.shape
    K2, R, S, Cm = w1.shape
    if K2 != K or w2.shape[0] != Cm or tuple(w2.shape[1:3]) != (1, 1):
        raise ValueError("dy, w1 and w2 [Cm,1,1,C] disagree on K or Cm")
    C = w2.shape[3]
    H, W = P - 2 * pad + R - 1, Q - 2 * pad + S - 1
    if pad < 0 or H < 1 or W < 1:
        raise ValueError("pad must be >= 0 and the chain's H, W >= 1")
    dev = dy.device
    _check_tensor("dy", dy, (N, P, Q, K), torch.float16, dev)
    _check_tensor("w1", w1, (K, R, S, Cm), torch.float16, dev)
    _check_tensor("w2", w2, (Cm, 1, 1, C), torch.float16, dev)
    if epilogue != EPI_NONE:
        if z is None:
            raise ValueError("the epilogue needs z")
        _check_tensor("z", z, (N, H, W, Cm), torch.float16, dev)
    else:
        z = None
    if out is not None:
        _check_tensor("out", out, (N, H, W, C), torch.float16, dev)
    _check_ws(workspace, dev)
    dx = out if out is not None else torch.empty((N, H, W, C), dtype=torch.float16, device=dev)
    conv2d_dgrad_chain_nhwc_ws(dy, w1, z, w2, dx, N, H, W, Cm, K, R, S, pad, C, epilogue, workspace)
    return dx


__all__ = [
    "conv2d_dgrad_nhwc", "conv2d_dgrad_nhwc_ws", "conv2d_dgrad_workspace_size", "conv2d_dgrad_nhwc_config",
    "conv2d_dgrad_nhwc_noalloc", "conv2d_dgrad_noalloc_max_bytes",
    "conv2d_dgrad_check", "conv2d_dgrad_num_configs",
    "conv2d_dgrad_config_name", "conv2d_dgrad_query_config", "conv2d_dgrad_set_autotune",
    "conv2d_dgrad_set_fault_inject", "conv2d_dgrad_set_streamk", "conv2d_dgrad_streamk_launches",
    "conv2d_dgrad_cache_clear", "conv2d_dgrad_cache_size", "conv2d_dgrad_cache_save", "conv2d_dgrad_cache_load",
    "conv2d_dgrad_plan", "conv2d_dgrad_last_error", "conv2d_dgrad_build_info", "dgrad", "get_lib",
    "conv2d_wgrad_nhwc", "conv2d_wgrad_nhwc_ws", "conv2d_wgrad_workspace_size", "conv2d_wgrad_nhwc_config",
    "conv2d_wgrad_check", "conv2d_wgrad_num_configs", "wgrad",
    "conv2d_forward_nhwc", "conv2d_forward_nhwc_config", "conv2d_forward_check", "conv2d_forward_num_configs",
    "forward", "ACT_NONE", "ACT_HARDSWISH", "conv2d_dgrad_chain_nhwc", "conv2d_dgrad_chain_check", "dgrad_chain",
    "conv2d_dgrad_chain_nhwc_ws", "conv2d_dgrad_chain_workspace_size", "conv2d_dgrad_chain_query",
    "workspace", "dgrad_workspace", "wgrad_workspace",
    "DgradError", "EPI_NONE", "EPI_DRELU", "EPI_DHARDSWISH",
]
