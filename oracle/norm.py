"""RMSNorm before the layer and the residual add after it (CPU oracle).

Test infrastructure (see oracle/__init__.py).

"Day 0 support for Mistral Large 4 on vLLM", fusions of the decode round: the all-reduce,
the residual add and the RMSNorm run as one kernel; "Inkling 2 Small on vLLM: Day-0
Support", kernel fusion: the memory-bound steps between sublayers (residual update,
RMSNorm) are folded into neighbouring kernels. On one GPU (no all-reduce) the MoE
sublayer of a pre-norm block is

    x   = RMSNorm(r) = r / sqrt(mean(r^2) + eps) * gamma      (the layer's input, BF16)
    out = r + MoE(x)                                            (the residual stream, BF16)

Readings the pages leave open: gamma is a BF16 vector of H values; x is rounded to BF16
(round to nearest even) because the layer takes BF16 tokens; the residual add is one
FP32-or-wider sum rounded once to BF16. The oracle evaluates both in FP64.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_to_f64


def rms_norm(r_bits: np.ndarray, gamma_bits: np.ndarray, eps: float) -> np.ndarray:
    """x[t, h] = r[t, h] / sqrt(mean_h r[t, h]^2 + eps) * gamma[h], FP64."""
    r = bf16_to_f64(r_bits)
    g = bf16_to_f64(gamma_bits)
    ms = np.mean(r * r, axis=1, keepdims=True)
    return r / np.sqrt(ms + eps) * g[None, :]


def to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """FP64 -> BF16 bit patterns, rounded once, to nearest with ties to even (finite values
    in BF16's range). BF16 keeps 8 significant bits down to 2^-126 and a fixed quantum of
    2^-133 below: the value is divided by its quantum, rounded to an integer (numpy's round
    is half to even) and scaled back, which is exact in FP32."""
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)                                 # |v| in [2^(e-1), 2^e)
    q = np.ldexp(1.0, np.maximum(e, -125) - 8)         # the BF16 quantum at |v|
    out = (np.round(v / q) * q).astype(np.float32)
    return (out.view(np.uint32) >> 16).astype(np.uint16)


def residual_out(r_bits: np.ndarray, y: np.ndarray) -> np.ndarray:
    """The residual stream after the layer, FP64: r + y."""
    return bf16_to_f64(r_bits) + np.asarray(y, dtype=np.float64)
