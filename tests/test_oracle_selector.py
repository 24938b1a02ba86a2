"""Pins of the DFlash2 candidate selector's oracle (CPU only).

Ollama ``mlxrunner/dflash.go`` (DFlash2 commit note; ``selectBlock``): the
selector proposes each token conditioned on its predecessor and returns each
position's candidate distribution, which verification uses to keep the
output exact; the draft samples with temperature only.  The reading (top-K
candidates, a bigram term <P[prev], Q[c]> on the row's logit, softmax over
the candidates, Gumbel-max with its own Philox counter field) is pinned by:
brute-force candidate sets; the closed forms with no conditioning (greedy =
the row argmax; all-vocabulary candidates = torch's softmax); a chain of
predecessor-driven choices that only sequential conditioning produces; the
draw frequencies (chi-square against the candidate softmax); and the
exactness of speculative verification with the sparse candidate
distribution (the emitted token follows the target, by Monte Carlo).
"""
import numpy as np
import pytest
import torch
from scipy import stats

from oracle.selector import candidates, dense_rows, select_block, selector_uniforms
from oracle.verify import accept_uniform, next_uniforms, softmax, verify_block


def test_candidates_brute_force_with_ties():
    rng = np.random.default_rng(0)
    for _ in range(50):
        z = rng.integers(0, 6, size=17).astype(np.float64)     # many exact ties
        k = int(rng.integers(1, 17))
        brute = [i for _, i in sorted((-z[i], i) for i in range(z.size))][:k]
        assert list(candidates(z, k)) == brute


def test_no_conditioning_greedy_is_row_argmax():
    rng = np.random.default_rng(1)
    z = rng.normal(size=(6, 40))
    z[3, 7] = z[3, 2] = z[3].max() + 1.0                         # a tie: the lower id wins
    zeros = np.zeros((40, 8))
    tok, cand, probs, _ = select_block(z, 5, zeros, zeros, 4, 0.0, 1, 2, 3)
    assert probs is None
    assert list(tok) == [int(np.argmax(r)) for r in z] and tok[3] == 2
    assert all(cand[i, 0] == tok[i] for i in range(6))


def test_all_candidates_is_the_temperature_softmax():
    rng = np.random.default_rng(2)
    z = rng.normal(scale=2.0, size=(3, 30))
    zeros = np.zeros((30, 4))
    _, cand, probs, _ = select_block(z, 0, zeros, zeros, 30, 0.7, 1, 2, 3)
    ref = torch.softmax(torch.from_numpy(z) / 0.7, dim=1).numpy()
    for i in range(3):
        np.testing.assert_allclose(probs[i], ref[i, cand[i]], rtol=1e-12, atol=1e-15)


def test_each_choice_follows_its_predecessor():
    """A bigram chain anchor -> 11 -> 4 -> 9: position i picks the successor
    of the token chosen at i - 1, never the successor of the anchor or of the
    same position's own best logit.  Each row's logits rank those tokens
    second to fifth, so only the conditioning can pick them."""
    V, Ds = 20, 6
    z = np.zeros((3, V))
    for i in range(3):
        z[i] = np.linspace(1.0, 0.0, V)                             # id 0 best, then 1, 2, ...
        z[i, [11, 4, 9]] = [0.95, 0.94, 0.93]                       # inside every row's top 5
    P = np.zeros((V, Ds))
    Q = np.zeros((V, Ds))
    chain = [(17, 11, 0), (11, 4, 1), (4, 9, 2)]                    # (prev, next, feature)
    for a, b, f in chain:
        P[a, f] = 10.0
        Q[b, f] = 1.0
    tok, _, _, _ = select_block(z, 17, P, Q, 5, 0.0, 0, 0, 0)
    assert list(tok) == [11, 4, 9]
    tok2, _, _, _ = select_block(z, 3, P, Q, 5, 0.0, 0, 0, 0)       # another anchor: no chain
    assert list(tok2) == [0, 0, 0]


def test_draws_follow_the_candidate_softmax():
    """Gumbel-max over the candidates with the selector's uniforms: the drawn
    rank of position 1 follows q over 20000 keys (chi-square p > 1e-3)."""
    rng = np.random.default_rng(3)
    z = rng.normal(size=(1, 24))
    P = rng.normal(scale=0.3, size=(24, 3))
    Q = rng.normal(scale=0.3, size=(24, 3))
    counts = np.zeros(6)
    q = None
    for key in range(20000):
        tok, cand, probs, _ = select_block(z, 5, P, Q, 6, 0.8, 7, key, 0)
        counts[int(np.flatnonzero(cand[0] == tok[0])[0])] += 1
        q = probs[0]
    chi = stats.chisquare(counts, q * counts.sum())
    assert chi.pvalue > 1e-3, (counts, q)


def test_uniforms_are_in_the_open_interval_and_disjoint_from_the_other_draws():
    u = selector_uniforms(1, 2, 3, 4, 16)
    assert np.all((u > 0) & (u < 1)) and len(set(u)) == 16
    assert not np.isclose(u[0], accept_uniform(1, 2, 3, 4))          # counter field 3 vs 1
    assert not np.allclose(u[:4], next_uniforms(1, 2, 3, 4, 4))      # vs 2


def test_verification_with_candidate_distributions_is_exact():
    """The first emitted token of a round drafted by the selector (sparse q on
    K candidates) and verified by speculative sampling is an exact draw from
    the target's p (Leviathan et al. 2023, theorem 1): 12000 seeded rounds,
    chi-square p > 1e-3."""
    rng = np.random.default_rng(4)
    V, K, T = 10, 4, 1.0
    z_draft = rng.normal(size=(2, V))
    target = rng.normal(size=(3, V))
    P = rng.normal(scale=0.5, size=(V, 3))
    Q = rng.normal(scale=0.5, size=(V, 3))
    p0 = softmax(target[0], T)
    counts = np.zeros(V)
    for key in range(12000):
        tok, cand, probs, _ = select_block(z_draft, 1, P, Q, K, T, 3, key, 0)
        q = dense_rows(cand, probs, V)
        a, x, _ = verify_block(target, tok, q, T, 3, key, 0)
        first = int(tok[0]) if a >= 1 else x
        counts[first] += 1
    keep = p0 * counts.sum() >= 5                                  # rare tokens share one bin
    obs, exp = counts[keep], p0[keep] * counts.sum()
    if not keep.all():
        obs, exp = np.append(obs, counts[~keep].sum()), np.append(exp, p0[~keep].sum() * counts.sum())
    chi = stats.chisquare(obs, exp)
    assert chi.pvalue > 1e-3, (counts, p0)


def test_dense_rows_hold_the_candidate_probabilities():
    cand = np.array([[3, 1], [0, 2]])
    probs = np.array([[0.75, 0.25], [0.5, 0.5]])
    d = dense_rows(cand, probs, 5)
    np.testing.assert_array_equal(d, [[0, 0.25, 0, 0.75, 0], [0.5, 0, 0.5, 0, 0]])
