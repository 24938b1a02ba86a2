"""Batched draft sampler (test infrastructure only).

Ollama ``mlxrunner/dflash.go`` (``selectBlock``) samples rows 1..n from one
batched distribution (``Sampler.Distribution`` then ``SampleDistribution``),
and each row's penalties see only the committed history, never the other
rows of the block.  The pages name no penalty formula and no draw method;
the readings taken here are:

* repetition penalty (CTRL, Keskar et al. 2019): for each distinct token t in
  the last ``history`` committed tokens, z_t / rho if z_t > 0 else z_t * rho;
* temperature T: scores z'/T; probabilities softmax(z'/T); T == 0 is greedy
  (argmax of z', lowest index on an exact tie) and returns no probabilities;
* the draw is Gumbel-max: id = argmax_t (z'_t/T + g_t), g_t = -log(-log u_t),
  u_t = (b_t + 1/2) * 2**-23, a value exactly representable in float32, where
  b_t is a 23-bit field of word ((t mod 8) div 2) of Philox4x64-10 at counter
  (t div 8, row, round, 0) under key (seed, stream): bits 63..41 of the word
  for even t, bits 40..18 for odd t (one generator call serves eight tokens).

Philox4x64-10 is written from its published definition (Salmon, Moraes, Dror,
Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11): ten rounds of
two 64x64->128 multiplies with a Weyl key schedule.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

_M64 = np.uint64(0xFFFFFFFFFFFFFFFF)
_M32 = np.uint64(0xFFFFFFFF)
PHILOX_M0 = np.uint64(0xD2E7470EE14C6C93)
PHILOX_M1 = np.uint64(0xCA5A826395121157)
PHILOX_W0 = np.uint64(0x9E3779B97F4A7C15)
PHILOX_W1 = np.uint64(0xBB67AE8584CAA73B)


def _mulhilo(a: np.ndarray, b: np.uint64):
    """(high, low) 64-bit halves of the 128-bit product a*b, by 32-bit limbs."""
    a = np.asarray(a, dtype=np.uint64)
    s32 = np.uint64(32)
    a0, a1 = a & _M32, a >> s32
    b0, b1 = b & _M32, b >> s32
    p00, p01, p10, p11 = a0 * b0, a0 * b1, a1 * b0, a1 * b1
    mid = (p00 >> s32) + (p01 & _M32) + (p10 & _M32)
    lo = (p00 & _M32) | ((mid & _M32) << s32)
    hi = p11 + (p01 >> s32) + (p10 >> s32) + (mid >> s32)
    return hi, lo


def philox4x64_10(ctr, key):
    """Philox4x64 with 10 rounds on arrays of counters; returns 4 uint64 arrays."""
    c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint64) for c in ctr)
    k0, k1 = np.uint64(key[0]), np.uint64(key[1])
    with np.errstate(over="ignore"):
        for r in range(10):
            if r:
                k0 = np.uint64((int(k0) + int(PHILOX_W0)) & 0xFFFFFFFFFFFFFFFF)
                k1 = np.uint64((int(k1) + int(PHILOX_W1)) & 0xFFFFFFFFFFFFFFFF)
            hi0, lo0 = _mulhilo(c0, PHILOX_M0)
            hi1, lo1 = _mulhilo(c2, PHILOX_M1)
            c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def uniforms(seed: int, stream: int, rnd: int, row: int, vocab: int) -> np.ndarray:
    """u_t in (0, 1) for t in 0..vocab-1 (exact float32 values, returned float64)."""
    t = np.arange(vocab, dtype=np.uint64)
    o = t >> np.uint64(3)
    words = philox4x64_10((o, np.full_like(o, row), np.full_like(o, rnd), np.zeros_like(o)),
                          (seed, stream))
    w = np.stack(words, axis=0)[((t >> np.uint64(1)) & np.uint64(3)).astype(np.int64), np.arange(vocab)]
    hi = w >> np.uint64(41)
    lo = (w >> np.uint64(18)) & np.uint64(0x7FFFFF)
    bits = np.where((t & np.uint64(1)) == 0, hi, lo).astype(np.float64)
    return (bits + 0.5) * 2.0 ** -23


def penalize(z: np.ndarray, history: Sequence[int], rho: float) -> np.ndarray:
    z = np.array(z, dtype=np.float64)
    if rho == 1.0:
        return z
    for t in sorted(set(int(x) for x in history)):
        z[t] = z[t] / rho if z[t] > 0 else z[t] * rho
    return z


def sample_row(z, history: Sequence[int], temperature: float, rho: float,
               seed: int, stream: int, rnd: int, row: int):
    """One drafted row: returns (id, probs or None, sorted scores for margins)."""
    zp = penalize(z, history, rho)
    if temperature == 0.0:
        return int(np.argmax(zp)), None, zp
    s = zp / temperature
    m = np.max(s)
    e = np.exp(s - m)
    probs = e / e.sum()
    u = uniforms(seed, stream, rnd, row, zp.shape[0])
    score = s - np.log(-np.log(u))
    return int(np.argmax(score)), probs, score


def top2_gap(scores: np.ndarray) -> float:
    """Gap between the best and second-best score (the tie margin's input)."""
    part = np.partition(np.asarray(scores, dtype=np.float64), -2)[-2:]
    return float(part[1] - part[0])
