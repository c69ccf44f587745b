"""Comparison helpers shared by the GPU parity tests and the smoke entry."""
from __future__ import annotations

import numpy as np
import torch

COS_MIN = 0.9999
REL_MAX = 1e-2
REL_FLOOR = 1e-3   # relative-error denominator floor, as a fraction of max |y32|


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_metrics(y_bits: np.ndarray, y_ref: np.ndarray) -> dict:
    """Tolerance metrics of a bf16 output against an fp32/fp64 reference."""
    y = bits_to_f32(y_bits).astype(np.float64)
    r = np.asarray(y_ref, dtype=np.float64)
    finite = bool(np.isfinite(y).all())
    scale = np.abs(r).max() if r.size else 0.0
    den = np.maximum(np.abs(r), REL_FLOOR * scale) if scale > 0 else np.ones_like(r)
    rel = float((np.abs(y - r) / den).max()) if r.size else 0.0
    nrm = float(np.linalg.norm(y) * np.linalg.norm(r))
    cos = float((y * r).sum() / nrm) if nrm > 0 else (1.0 if np.array_equal(y, r) else 0.0)
    normwise = float(np.abs(y - r).max() / scale) if scale > 0 else 0.0
    return dict(finite=finite, rel=rel, cos=cos, normwise=normwise)


def assert_bf16_close(y_bits: np.ndarray, y32: np.ndarray, y64: np.ndarray | None = None) -> dict:
    m = bf16_metrics(y_bits, y32)
    assert m["finite"], "NaN/Inf in the bf16 output"
    assert m["cos"] >= COS_MIN, m
    assert m["rel"] <= REL_MAX, m
    if y64 is not None:
        m64 = bf16_metrics(y_bits, y64)
        assert m64["cos"] >= COS_MIN and m64["rel"] <= REL_MAX, m64
    return m
