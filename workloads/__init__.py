"""Seeded synthetic inputs for conv2d backward-data (dgrad).

This module only draws numbers. It holds none of the operation's arithmetic:
no output sizes beyond the forward-convolution shape rule needed to size dy,
no index algebra, no epilogue. Both the fp64 oracle (``oracle/``) and the HIP
path (``convolution_backward_amd``) consume what it returns, and neither
imports the other.

Shapes and value distributions stand in for the ResNet-50 dgrad workloads
that the TVM pull request "[CUTLASS] Conv2d dgrad" (apache/tvm #10110, the
opening benchmark comment) measures at batch 8 and batch 256. The pages do
not print the layer list, so the layers below are the standard ResNet-50
shapes of those families.

Conventions:
  * dy  [N][P][Q][K]  fp16, NHWC (K = channels of the forward output)
  * w   [K][R][S][C]  fp16, KRSC (C = channels of the forward input)
  * z   [N][H][W][C]  fp16, saved pre-activation (only for epilogue configs)
  * In "N(0, a)" the second number is the standard deviation.
  * Values are drawn in fp64 with numpy's PCG64 and rounded to fp16 with
    round-to-nearest-even (``astype(np.float16)``). Draw order: dy, w, z.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, asdict

import numpy as np

EPI_NONE = 0
EPI_DRELU = 1
EPI_DHARDSWISH = 2
EPI_NAMES = {EPI_NONE: "none", EPI_DRELU: "drelu", EPI_DHARDSWISH: "dhardswish"}


@dataclass(frozen=True)
class DgradConfig:
    name: str
    N: int
    H: int
    W: int
    C: int
    K: int
    R: int
    S: int
    stride: int
    pad: int
    epilogue: int = EPI_NONE
    dy_dist: str = "normal"      # "normal" (N(0,1)) or "uniform" (U[-1,1])
    w_std: float = 1.0
    z_std: float = 1.5
    seed: int = 0
    note: str = ""

    @property
    def P(self) -> int:
        # forward-convolution output height: sizes the dy tensor
        return (self.H + 2 * self.pad - self.R) // self.stride + 1

    @property
    def Q(self) -> int:
        return (self.W + 2 * self.pad - self.S) // self.stride + 1

    def useful_flops(self) -> int:
        """2*N*P*Q*K*C*R*S: the multiply-adds of the forward layer."""
        return 2 * self.N * self.P * self.Q * self.K * self.C * self.R * self.S

    def algorithmic_bytes(self) -> int:
        """dy + w + dx (+ z) in fp16, each moved once."""
        b = 2 * (self.N * self.P * self.Q * self.K
                 + self.K * self.R * self.S * self.C
                 + self.N * self.H * self.W * self.C)
        if self.epilogue != EPI_NONE:
            b += 2 * self.N * self.H * self.W * self.C
        return b

    def as_dict(self) -> dict:
        d = asdict(self)
        d["P"], d["Q"] = self.P, self.Q
        return d

    def replace(self, **kw) -> "DgradConfig":
        d = asdict(self)
        d.update(kw)
        return DgradConfig(**d)


def _cfg(idx, **kw):
    return DgradConfig(seed=1000 + idx, **kw)


# The six layers of the measured suite. Seeds are 1000 + position.
CONFIGS = [
    _cfg(0, name="tiny_n1_14x14_256_3x3_s1", N=1, H=14, W=14, C=256, K=256,
         R=3, S=3, stride=1, pad=1, dy_dist="uniform",
         w_std=1.0 / math.sqrt(9 * 256),
         note="latency-sized single-sample layer"),
    _cfg(1, name="r50_stage2_3x3_n8", N=8, H=56, W=56, C=64, K=64,
         R=3, S=3, stride=1, pad=1, w_std=1.0 / math.sqrt(576)),
    _cfg(2, name="r50_3x3_s2_n256", N=256, H=56, W=56, C=128, K=128,
         R=3, S=3, stride=2, pad=1, w_std=1.0 / math.sqrt(1152),
         note="stride 2: four phases with 1/2/2/4 taps"),
    _cfg(3, name="r50_1x1_s2_downsample_n256", N=256, H=56, W=56, C=256, K=512,
         R=1, S=1, stride=2, pad=0, w_std=1.0 / math.sqrt(512),
         note="stride 2 1x1: one GEMM phase and three all-zero phases"),
    _cfg(4, name="r50_1x1_s1_reduce_n256", N=256, H=14, W=14, C=1024, K=256,
         R=1, S=1, stride=1, pad=0, w_std=1.0 / math.sqrt(256)),
    _cfg(5, name="r50_stage4_3x3_dhardswish_n256", N=256, H=7, W=7, C=512, K=512,
         R=3, S=3, stride=1, pad=1, epilogue=EPI_DHARDSWISH,
         w_std=1.0 / math.sqrt(4608), z_std=1.5,
         note="dy and w distributions assumed as in the other batch-256 layers"),
]
CONFIG_BY_NAME = {c.name: c for c in CONFIGS}


def get_config(key) -> DgradConfig:
    if isinstance(key, DgradConfig):
        return key
    if isinstance(key, int):
        return CONFIGS[key]
    return CONFIG_BY_NAME[key]


def _normal16(rng, shape, std):
    x = rng.standard_normal(size=shape, dtype=np.float64)
    if std != 1.0:
        x *= std
    return x.astype(np.float16)


def make_inputs(cfg, seed=None) -> dict:
    """dy, w (and z for epilogue configs) as C-contiguous float16 arrays."""
    cfg = get_config(cfg)
    rng = np.random.Generator(np.random.PCG64(cfg.seed if seed is None else seed))
    dy_shape = (cfg.N, cfg.P, cfg.Q, cfg.K)
    if cfg.dy_dist == "uniform":
        dy = rng.uniform(-1.0, 1.0, size=dy_shape).astype(np.float16)
    else:
        dy = _normal16(rng, dy_shape, 1.0)
    w = _normal16(rng, (cfg.K, cfg.R, cfg.S, cfg.C), cfg.w_std)
    out = {"dy": dy, "w": w, "z": None}
    if cfg.epilogue != EPI_NONE:
        out["z"] = _normal16(rng, (cfg.N, cfg.H, cfg.W, cfg.C), cfg.z_std)
    return out


def make_x(cfg, seed=None) -> np.ndarray:
    """The forward layer's input x [N,H,W,C] for wgrad: post-ReLU activations,
    max(N(0,1), 0) rounded to float16 (half of the values are exact zeros)."""
    cfg = get_config(cfg)
    rng = np.random.Generator(np.random.PCG64((cfg.seed + 500) if seed is None else seed))
    x = rng.standard_normal(size=(cfg.N, cfg.H, cfg.W, cfg.C), dtype=np.float64)
    return np.maximum(x, 0.0).astype(np.float16)


def small_config(N, H, W, C, K, R, S, stride, pad, epilogue=EPI_NONE,
                 seed=7, w_std=None, name="small") -> DgradConfig:
    """An arbitrary shape with the batch-256 value recipe (dy ~ N(0,1),
    w ~ N(0, 1/sqrt(K*R*S)), z ~ N(0,1.5))."""
    if w_std is None:
        w_std = 1.0 / math.sqrt(K * R * S)
    return DgradConfig(name=name, N=N, H=H, W=W, C=C, K=K, R=R, S=S,
                       stride=stride, pad=pad, epilogue=epilogue,
                       w_std=w_std, seed=seed)


def integer_inputs(cfg, lo=-2, hi=2, seed=11, z_values=None) -> dict:
    """Small-integer dy and w (fp16-exact), for tests where every product and
    partial sum is an exactly representable integer. ``z_values`` (if given)
    are drawn uniformly for z."""
    cfg = get_config(cfg)
    rng = np.random.Generator(np.random.PCG64(seed))
    dy = rng.integers(lo, hi + 1, size=(cfg.N, cfg.P, cfg.Q, cfg.K)).astype(np.float16)
    w = rng.integers(lo, hi + 1, size=(cfg.K, cfg.R, cfg.S, cfg.C)).astype(np.float16)
    z = None
    if cfg.epilogue != EPI_NONE:
        vals = np.asarray(z_values if z_values is not None else [-4, -3, -1.5, 0, 1.5, 3, 4],
                          dtype=np.float64)
        z = vals[rng.integers(0, len(vals), size=(cfg.N, cfg.H, cfg.W, cfg.C))].astype(np.float16)
    return {"dy": dy, "w": w, "z": z}


def one_hot_dy(cfg, n, p, q, k, value=1.0) -> np.ndarray:
    """dy that is zero except for one element."""
    cfg = get_config(cfg)
    dy = np.zeros((cfg.N, cfg.P, cfg.Q, cfg.K), dtype=np.float16)
    dy[n, p, q, k] = value
    return dy


@dataclass(frozen=True)
class ChainConfig:
    """Two dgrad steps of a bottleneck: the RxS stride-1 convolution
    (Cm -> K channels, filter w1 [K][R][S][Cm]) and the 1x1 convolution in
    front of it (C -> Cm, filter w2 [Cm][1][1][C]), with the activation
    derivative between them taken from z [N][H][W][Cm]."""
    name: str
    N: int
    H: int
    W: int
    Cm: int
    K: int
    R: int
    S: int
    pad: int
    C: int
    epilogue: int = EPI_DHARDSWISH
    z_std: float = 1.5
    seed: int = 0

    @property
    def P(self) -> int:
        return self.H + 2 * self.pad - self.R + 1

    @property
    def Q(self) -> int:
        return self.W + 2 * self.pad - self.S + 1

    def useful_flops(self) -> int:
        """Multiply-adds of both forward layers, times 2."""
        return 2 * (self.N * self.P * self.Q * self.K * self.Cm * self.R * self.S
                    + self.N * self.H * self.W * self.Cm * self.C)

    def algorithmic_bytes(self) -> int:
        """dy + w1 + z + w2 + dx in fp16, each moved once (t stays on chip)."""
        b = 2 * (self.N * self.P * self.Q * self.K + self.K * self.R * self.S * self.Cm
                 + self.Cm * self.C + self.N * self.H * self.W * self.C)
        if self.epilogue != EPI_NONE:
            b += 2 * self.N * self.H * self.W * self.Cm
        return b


# ResNet-50 bottlenecks: the 3x3 conv2 and the 1x1 conv1 in front of it, in
# stage 2 (56x56, 64 mid channels, 256 block channels) and stage 3 (28x28,
# 128 mid channels, 512 block channels).
CHAINS = [
    ChainConfig(name="r50_stage2_chain_3x3_1x1_n8", N=8, H=56, W=56, Cm=64, K=64, R=3, S=3, pad=1, C=256,
                seed=2001),
    ChainConfig(name="r50_stage2_chain_3x3_1x1_n256", N=256, H=56, W=56, Cm=64, K=64, R=3, S=3, pad=1, C=256,
                seed=2002),
    ChainConfig(name="r50_stage3_chain_3x3_1x1_n256", N=256, H=28, W=28, Cm=128, K=128, R=3, S=3, pad=1, C=512,
                seed=2003),
]
CHAIN_BY_NAME = {c.name: c for c in CHAINS}


def make_chain_inputs(cfg: ChainConfig, seed=None) -> dict:
    """dy ~ N(0,1), w1 ~ N(0, 1/sqrt(K*R*S)), z ~ N(0, z_std) (if the chain
    has an activation derivative), w2 ~ N(0, 1/sqrt(Cm)); float16, drawn in
    that order."""
    rng = np.random.Generator(np.random.PCG64(cfg.seed if seed is None else seed))
    dy = _normal16(rng, (cfg.N, cfg.P, cfg.Q, cfg.K), 1.0)
    w1 = _normal16(rng, (cfg.K, cfg.R, cfg.S, cfg.Cm), 1.0 / math.sqrt(cfg.K * cfg.R * cfg.S))
    z = _normal16(rng, (cfg.N, cfg.H, cfg.W, cfg.Cm), cfg.z_std) if cfg.epilogue != EPI_NONE else None
    w2 = _normal16(rng, (cfg.Cm, 1, 1, cfg.C), 1.0 / math.sqrt(cfg.Cm))
    return {"dy": dy, "w1": w1, "z": z, "w2": w2}


def integer_chain_inputs(cfg: ChainConfig, seed=11) -> dict:
    """dy, w1, w2 in {-1, 0, 1} and z from {-4, -1.5, 0, 1.5, 4} (relu' and
    hardswish' are then 0, 1/2 or 1): every intermediate sum is exact in fp32
    and every t exact in fp16."""
    rng = np.random.Generator(np.random.PCG64(seed))
    dy = rng.integers(-1, 2, size=(cfg.N, cfg.P, cfg.Q, cfg.K)).astype(np.float16)
    w1 = rng.integers(-1, 2, size=(cfg.K, cfg.R, cfg.S, cfg.Cm)).astype(np.float16)
    vals = np.array([-4.0, -1.5, 0.0, 1.5, 4.0])
    z = vals[rng.integers(0, len(vals), size=(cfg.N, cfg.H, cfg.W, cfg.Cm))].astype(np.float16)
    w2 = rng.integers(-1, 2, size=(cfg.Cm, 1, 1, cfg.C)).astype(np.float16)
    return {"dy": dy, "w1": w1, "z": z if cfg.epilogue != EPI_NONE else None, "w2": w2}


__all__ = [
    "DgradConfig", "CONFIGS", "CONFIG_BY_NAME", "get_config", "make_inputs",
    "small_config", "integer_inputs", "one_hot_dy",
    "ChainConfig", "CHAINS", "CHAIN_BY_NAME", "make_chain_inputs", "integer_chain_inputs",
    "EPI_NONE", "EPI_DRELU", "EPI_DHARDSWISH", "EPI_NAMES",
]
