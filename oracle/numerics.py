"""fp64 building blocks of the oracle (test infrastructure only).

bf16 rounding mirrors the points where a bf16 GPU kernel must round a GEMM
operand; everything else stays in fp64.
"""
from __future__ import annotations

import numpy as np


def round_bf16(x) -> np.ndarray:
    """Round fp64 values to the nearest bfloat16 value (8 significant bits,
    round half to even), returned as fp64.  bf16 has fp32's exponent range, so
    for the magnitudes met here only the significand is rounded."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)  # x = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def round_f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def rmsnorm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gain, row-wise."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gain, dtype=np.float64)


def rope_rotate_half(x: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """Rotary position embedding of one head vector x [hd] at position pos,
    pairing element i with element i + hd/2, frequency theta^(-2i/hd)."""
    x = np.asarray(x, dtype=np.float64)
    hd = x.shape[-1]
    half = hd // 2
    i = np.arange(half, dtype=np.float64)
    ang = float(pos) * theta ** (-2.0 * i / hd)
    c, s = np.cos(ang), np.sin(ang)
    out = np.empty_like(x)
    out[..., :half] = x[..., :half] * c - x[..., half:] * s
    out[..., half:] = x[..., half:] * c + x[..., :half] * s
    return out


def silu(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def logsumexp(v: np.ndarray) -> float:
    v = np.asarray(v, dtype=np.float64)
    m = np.max(v)
    return float(m + np.log(np.sum(np.exp(v - m))))


def softmax(v: np.ndarray) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    e = np.exp(v - np.max(v))
    return e / np.sum(e)


def matmul_t(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y = x W^T in fp64 (W row-major [out, in])."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T
