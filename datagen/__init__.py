"""Seeded synthetic inputs for the fused W8A8 linear workloads.

This module only draws random numbers and casts them to bf16; it holds none of
the quantize / GEMM / dequant arithmetic.  Both the CPU oracle tests and the
GPU path take their inputs from here, so the two sides see the same bf16 bits.

Recipe (the pages give no layer shapes; these are diffusion-transformer-typical
stand-ins for the linear layers of the model named in the abstract of
"Realizing Native INT8 Compute for Diffusion Transformers on Consumer GPUs"):

* every stream is ``numpy.random.default_rng`` seeded from a
  ``numpy.random.SeedSequence(seed)`` spawn child; X, W and b of one linear use
  children 0, 1, 2 of that linear's own child;
* values are drawn in float32 (normal or Student-t), multiplied by the standard
  deviation in float32 and cast to bf16 with round-to-nearest-even by torch;
* the outlier workload scales 8 fixed activation channels (the same for every
  token) by 50 after drawing Student-t(nu=3) samples.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

X_STD = 1.0
W_STD = 0.02
B_STD = 0.01
OUTLIER_CHANNELS = 8
OUTLIER_GAIN = 50.0


@dataclass(frozen=True)
class LinearShape:
    name: str
    M: int
    K: int
    N: int
    act: str = "normal"  # "normal", "student_t3_outliers" or "gelu_of_prev"


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    seed: int
    linears: tuple
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def ops(self) -> int:
        return sum(2 * l.M * l.N * l.K for l in self.linears)


WORKLOADS = (
    Workload(0, "tiny_linear_64x256x128", 0,
             (LinearShape("tiny", 64, 256, 128),)),
    Workload(1, "dit768_attn_proj_2304x3072x3072", 1,
             (LinearShape("attn_proj", 2304, 3072, 3072),)),
    Workload(2, "dit768_mlp_pair_2304", 2,
             (LinearShape("mlp_up", 2304, 3072, 12288),
              LinearShape("mlp_down", 2304, 12288, 3072, act="gelu_of_prev"))),
    Workload(3, "dit1024_qkv_outliers_4096x3072x9216", 3,
             (LinearShape("qkv", 4096, 3072, 9216, act="student_t3_outliers"),)),
    Workload(4, "dit1024_block_cfg2_m8192", 4,
             (LinearShape("qkv", 8192, 3072, 9216),
              LinearShape("out_proj", 8192, 3072, 3072),
              LinearShape("mlp_up", 8192, 3072, 12288),
              LinearShape("mlp_down", 8192, 12288, 3072))),
)


def to_bf16(a: np.ndarray) -> torch.Tensor:
    """float32 numpy array -> bf16 CPU tensor (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def _streams(seed: int, n: int):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def _normal(rng, shape, std):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def outlier_channels(K: int, seed: int = 3) -> np.ndarray:
    """The 8 fixed outlier channel indices of the outlier workload."""
    return np.sort(np.random.default_rng(seed).choice(K, OUTLIER_CHANNELS, replace=False))


def gen_weight(shape: LinearShape, seed: int, idx: int = 0):
    """(W bf16 [N,K], b bf16 [N]) for linear ``idx`` of a workload."""
    child = np.random.SeedSequence(seed).spawn(idx + 1)[idx]
    _, rw, rb = [np.random.default_rng(s) for s in child.spawn(3)]
    w = to_bf16(_normal(rw, (shape.N, shape.K), W_STD))
    b = to_bf16(_normal(rb, (shape.N,), B_STD))
    return w, b


def gen_act(shape: LinearShape, seed: int, idx: int = 0, rows=None):
    """X bf16 [M,K] (or the selected rows of it) for linear ``idx``."""
    if shape.act == "gelu_of_prev":
        raise ValueError("this activation is produced by the previous linear")
    child = np.random.SeedSequence(seed).spawn(idx + 1)[idx]
    rx = np.random.default_rng(child.spawn(3)[0])
    if shape.act == "normal":
        x = _normal(rx, (shape.M, shape.K), X_STD)
    elif shape.act == "student_t3_outliers":
        x = rx.standard_t(3, size=(shape.M, shape.K)).astype(np.float32)
        x[:, outlier_channels(shape.K, seed)] *= np.float32(OUTLIER_GAIN)
    else:
        raise ValueError(shape.act)
    if rows is not None:
        x = x[rows]
    return to_bf16(x)


def random_bf16(shape, seed: int, std: float = 1.0, dist: str = "normal") -> torch.Tensor:
    """Free-form seeded bf16 tensor for edge-case tests."""
    rng = np.random.default_rng(seed)
    if dist == "normal":
        a = _normal(rng, shape, std)
    elif dist == "uniform":
        a = rng.uniform(-std, std, size=shape).astype(np.float32)
    elif dist == "student_t3":
        a = rng.standard_t(3, size=shape).astype(np.float32) * np.float32(std)
    else:
        raise ValueError(dist)
    return to_bf16(a)


def random_int8(shape, seed: int, lo: int = -127, hi: int = 127) -> np.ndarray:
    """Seeded int8 codes in [lo, hi] (for GEMM-only edge cases)."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=shape, dtype=np.int64).astype(np.int8)
