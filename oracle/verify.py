"""Speculative verification of a drafted block (test infrastructure only).

The pages fix what verification must achieve, not its formula: Ollama
``mlxrunner/dflash.go`` (``propose``) hands the verifier each position's
actual proposal distribution so that the output stays exact, and the mlxcel
Laguna PR's round loop verifies greedily by a raw per-position argmax.  The
readings taken here:

* greedy (T == 0): the target row i (i = 0..n) scores the token after
  position F + i; draft token i+1 is accepted while it equals the row's
  argmax (lowest index on an exact tie); ``accepted`` is the number of leading
  matches a and ``next`` is the argmax of row a (the correction, or with
  a == n the bonus token);
* sampling (T > 0): the standard speculative-sampling rule (Leviathan, Kalman,
  Matias 2023; Chen et al. 2023), which makes every emitted token an exact draw
  from the target: p_i = softmax(row_i / T), q_i = the draft distribution the
  drafted token x_{i+1} was drawn from; x_{i+1} is accepted iff
  u_i * q_i(x_{i+1}) <= p_i(x_{i+1}); at the first rejection (row a) ``next``
  is drawn from max(0, p_a - q_a) renormalised, and if all n are accepted from
  p_n;
* draws: Philox4x64-10 under the session's key (seed, stream): u_i = (top 23
  bits of word 0 at counter (0, i, round, 1)) + 1/2, times 2**-23; ``next``
  from row a by Gumbel-max over the row's scores (log of the residual mass,
  or row/T for the bonus row) with g_t from counter (t div 4, a, round, 2),
  word t mod 4, mapped to u as the drafter's sampler maps its draws;
* a draft id outside [0, V) (the pages' drafts are always tokens; the call
  takes the ids as device data it cannot check first) is never accepted, as
  a draft the target gives probability zero would not be, and ``next`` is
  then drawn at that row as after any rejection.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from oracle.sampler import philox4x64_10


def _u23(word: np.ndarray) -> np.ndarray:
    return ((np.asarray(word, dtype=np.uint64) >> np.uint64(41)).astype(np.float64) + 0.5) * 2.0 ** -23


def accept_uniform(seed: int, stream: int, rnd: int, i: int) -> float:
    """u_i of the acceptance test of draft token i+1."""
    w = philox4x64_10((np.array([0], np.uint64), np.array([i], np.uint64), np.array([rnd], np.uint64),
                       np.array([1], np.uint64)), (seed, stream))
    return float(_u23(w[0])[0])


def next_uniforms(seed: int, stream: int, rnd: int, row: int, vocab: int) -> np.ndarray:
    """u_t (t = 0..vocab-1) of the Gumbel-max draw of ``next`` from target row ``row``."""
    t = np.arange(vocab, dtype=np.uint64)
    q = t >> np.uint64(2)
    words = philox4x64_10((q, np.full_like(q, row), np.full_like(q, rnd), np.full_like(q, 2)), (seed, stream))
    w = np.stack(words, axis=0)[(t & np.uint64(3)).astype(np.int64), np.arange(vocab)]
    return _u23(w)


def softmax(z: np.ndarray, temperature: float) -> np.ndarray:
    s = np.asarray(z, dtype=np.float64) / temperature
    e = np.exp(s - s.max())
    return e / e.sum()


def verify_block(target: np.ndarray, draft_ids, draft_probs: Optional[np.ndarray], temperature: float,
                 seed: int, stream: int, rnd: int):
    """target [n+1, V] logits, draft_ids [n], draft_probs [n, V] (T > 0).

    Returns (accepted, next, info): info holds, for margins, the acceptance
    tests' (u*q, p) pairs up to the decision and the scores ``next`` was
    drawn from."""
    target = np.asarray(target, dtype=np.float64)
    n = len(draft_ids)
    assert target.shape[0] == n + 1
    info = {"tests": [], "scores": None}
    if temperature == 0.0:
        a = 0
        while a < n and int(np.argmax(target[a])) == int(draft_ids[a]):
            a += 1
        info["scores"] = target[a]
        return a, int(np.argmax(target[a])), info
    a = 0
    p_rows = [softmax(target[i], temperature) for i in range(n + 1)]
    V = target.shape[1]
    while a < n:
        x = int(draft_ids[a])
        if not 0 <= x < V:
            info["tests"].append((np.inf, 0.0))
            break
        p, q = p_rows[a][x], float(draft_probs[a][x])
        u = accept_uniform(seed, stream, rnd, a)
        info["tests"].append((u * q, p))
        if u * q <= p:
            a += 1
        else:
            break
    g = -np.log(-np.log(next_uniforms(seed, stream, rnd, a, target.shape[1])))
    if a < n:
        r = np.maximum(0.0, p_rows[a] - np.asarray(draft_probs[a], dtype=np.float64))
        with np.errstate(divide="ignore"):
            scores = np.where(r > 0, np.log(r), -np.inf) + g
    else:
        scores = target[n] / temperature + g
    info["scores"] = scores
    return a, int(np.argmax(scores)), info
