"""Elementary float64 operations of the oracle (test infrastructure only).

Each is the textbook definition written out; the drafter-level citations are
in ``oracle.model``.
"""
from __future__ import annotations

import numpy as np


def round_bf16(x) -> np.ndarray:
    """Nearest bf16 value (round half to even), returned as float64.

    bf16 keeps the top 16 bits of an IEEE binary32 number; rounding first to
    binary32 and then to bf16 is what a GPU storing a float32 result as bf16
    does.
    """
    x32 = np.asarray(x, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def rms_norm(x, gain, eps: float) -> np.ndarray:
    """y = x / sqrt(mean(x^2) + eps) * gain over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gain, dtype=np.float64)


def rope(x, positions, theta: float) -> np.ndarray:
    """Rotary embedding, rotate-half convention.

    ``x`` is [rows, heads, D]; row r is rotated by ``positions[r]``.  Pair
    (d, d + D/2) is rotated by angle pos * theta**(-2d/D).
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    half = D // 2
    d = np.arange(half, dtype=np.float64)
    inv_freq = theta ** (-2.0 * d / D)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def sigmoid(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def softmax(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x, axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=-1, keepdims=True)
