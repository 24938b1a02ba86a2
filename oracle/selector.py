"""DFlash2 candidate selector (test infrastructure only).

What the pages fix (Ollama ``mlxrunner/dflash.go``, the commit note "dflash:
add the DFlash2 draft model" and ``selectBlock``'s ``BlockSelector``
branch): after the block forward and the unembedding of rows 1..n, a DFlash2
draft hands the rows' hidden states, their logits and the anchor token to a
selector, which proposes each token conditioned on the token before it and
returns, per position, the candidate ids and their probabilities; the
verifier uses that candidate distribution to keep the output exact, and the
draft samples with the request's temperature only (no penalties).

The pages name the selector but give neither its candidate rule nor its
conditioning network.  The reading taken here (each part a configuration
field), the plainest one the rest supports:

* candidates of position i: the K highest logits of row i, ties to the
  lower id, ranked by logit (K = ``sel_candidates``);
* conditioning: candidate c at position i scores
  s_i(c) = z_i(c) + <P[t_{i-1}], Q[c]>, with P and Q the selector's two
  [V, Ds] tables (a learned bigram term on top of the row's own logit) and
  t_0 the anchor, t_{i-1} the token selected at position i-1;
* distribution: q_i = softmax over the K candidates of s_i / T; greedy
  (T = 0) takes the highest score (the lower candidate rank on a tie);
* draw: Gumbel-max over the candidates, u_k (candidate rank k) the top 23
  bits of word k mod 4 of Philox4x64-10 at counter (k div 4, i, round, 3)
  under the session's key (seed, stream), plus 1/2, times 2^-23.

Every part is pinned in ``tests/test_oracle_selector.py``.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from oracle.sampler import philox4x64_10


def candidates(z: np.ndarray, k: int) -> np.ndarray:
    """Ids of the k highest values of row z, highest first, ties to the lower id."""
    z = np.asarray(z, dtype=np.float64)
    order = np.lexsort((np.arange(z.size), -z))      # by value descending, then id ascending
    return order[:k]


def selector_uniforms(seed: int, stream: int, rnd: int, pos: int, k: int) -> np.ndarray:
    """u_0..u_{k-1} of the candidate draw at block position pos (1-based)."""
    j = np.arange(k, dtype=np.uint64)
    q = j >> np.uint64(2)
    words = philox4x64_10((q, np.full_like(q, pos), np.full_like(q, rnd), np.full_like(q, 3)), (seed, stream))
    w = np.stack(words, axis=0)[(j & np.uint64(3)).astype(np.int64), np.arange(k)]
    return ((w >> np.uint64(41)).astype(np.float64) + 0.5) * 2.0 ** -23


def select_block(logits: np.ndarray, anchor: int, P: np.ndarray, Q: np.ndarray, k: int, temperature: float,
                 seed: int, stream: int, rnd: int) -> Tuple[np.ndarray, np.ndarray, Optional[np.ndarray], list]:
    """logits [n, V] of rows 1..n.  Returns (tokens [n], candidate ids [n, k],
    candidate probabilities [n, k] or None when greedy, per-position scores
    (the values the choice was made on, for tie margins))."""
    z = np.asarray(logits, dtype=np.float64)
    n = z.shape[0]
    P = np.asarray(P, dtype=np.float64)
    Q = np.asarray(Q, dtype=np.float64)
    tokens = np.zeros(n, dtype=np.int64)
    cand = np.zeros((n, k), dtype=np.int64)
    probs = np.zeros((n, k)) if temperature > 0 else None
    scores = []
    prev = int(anchor)
    for i in range(n):
        c = candidates(z[i], k)
        s = z[i, c] + Q[c] @ P[prev]
        cand[i] = c
        if temperature > 0:
            a = s / temperature
            e = np.exp(a - a.max())
            probs[i] = e / e.sum()
            g = -np.log(-np.log(selector_uniforms(seed, stream, rnd, i + 1, k)))
            key = a + g
        else:
            key = s
        j = int(np.argmax(key))                     # first maximum: the lower rank on a tie
        tokens[i] = c[j]
        scores.append(key)
        prev = int(c[j])
    return tokens, cand, probs, scores


def dense_rows(cand: np.ndarray, probs: np.ndarray, vocab: int) -> np.ndarray:
    """The candidate distribution as full rows [n, V] (zero off the candidates)."""
    out = np.zeros((cand.shape[0], vocab))
    for i in range(cand.shape[0]):
        out[i, cand[i]] = probs[i]
    return out
