"""Pins of the verification oracle (CPU only).

The greedy rule is checked on hand-built logits; the sampling rule against
what it exists to guarantee (rejection-sampling theorem: every emitted token
is an exact draw from the target, and a draft is accepted with probability
sum_t min(p_t, q_t)), with independent draft draws, so that a dropped term,
a wrong sign or a missing renormalisation of the residual fails."""
import numpy as np
import pytest

from oracle.verify import accept_uniform, next_uniforms, softmax, verify_block


def _logits(argmaxes, V=11, seed=0):
    rng = np.random.default_rng(seed)
    z = rng.normal(size=(len(argmaxes), V))
    for i, a in enumerate(argmaxes):
        z[i, a] = z[i].max() + 1.0
    return z


def test_greedy_accepts_leading_argmax_matches_and_corrects():
    z = _logits([3, 5, 7, 2])
    a, nxt, _ = verify_block(z, [3, 5, 6], None, 0.0, 1, 2, 0)
    assert (a, nxt) == (2, 7)
    a, nxt, _ = verify_block(z, [4, 5, 7], None, 0.0, 1, 2, 0)
    assert (a, nxt) == (0, 3)
    a, nxt, _ = verify_block(z, [3, 5, 7], None, 0.0, 1, 2, 0)
    assert (a, nxt) == (3, 2)                       # all accepted: the bonus token
    a, nxt, _ = verify_block(z[:1], [], None, 0.0, 1, 2, 0)
    assert (a, nxt) == (0, 3)                       # nothing drafted


def test_draft_equal_to_target_is_always_accepted():
    rng = np.random.default_rng(1)
    z = rng.normal(size=(5, 9)) * 2
    q = np.stack([softmax(z[i], 0.7) for i in range(4)])
    for rnd in range(50):
        ids = [int(rng.choice(9, p=q[i])) for i in range(4)]
        a, nxt, info = verify_block(z, ids, q, 0.7, 3, 4, rnd)
        assert a == 4
        assert all(uq <= p for uq, p in info["tests"])


def test_zero_target_mass_is_rejected_and_never_emitted():
    z = np.zeros((2, 6))
    z[0, 2] = -np.inf                               # p_0(2) = 0
    q = np.zeros((1, 6))
    q[0, 2] = 1.0                                   # the draft was sure of token 2
    seen = set()
    for rnd in range(200):
        a, nxt, _ = verify_block(z, [2], q, 1.0, 5, 6, rnd)
        assert a == 0 and nxt != 2
        seen.add(nxt)
    assert seen == {0, 1, 3, 4, 5}                  # the residual is p_0 itself: uniform over the rest


def test_out_of_vocabulary_draft_acts_as_a_zero_probability_draft():
    """A draft id outside [0, V) is never accepted: the outcome equals that of
    a real token y the target row gives probability 0 (its logit -inf) while
    the draft distribution gives it mass, with the same rows otherwise (so the
    residual the correction is drawn from is the same).  Greedy: the same as
    any draft that is not the row's argmax."""
    rng = np.random.default_rng(4)
    V, y = 13, 6
    for rnd in range(40):
        z = rng.normal(size=(4, V)) * 1.5
        z[1, y] = -np.inf
        q = np.stack([softmax(rng.normal(size=V), 1.0) for _ in range(3)])
        ids = [int(rng.choice(V, p=softmax(z[0], 0.8))), y, 2]
        ref = verify_block(z, ids, q, 0.8, 7, 1, rnd)
        assert ref[0] <= 1
        for bad in (-1, V, V + 1000):
            out = verify_block(z, [ids[0], bad, 2], q, 0.8, 7, 1, rnd)
            assert out[:2] == ref[:2], (rnd, bad, out[:2], ref[:2])
        zg = z.copy()
        zg[1, y] = 0.0
        gref = verify_block(zg, [int(np.argmax(zg[0])), (int(np.argmax(zg[1])) + 1) % V, 2], None, 0.0, 7, 1, rnd)
        for bad in (-1, V):
            assert verify_block(zg, [int(np.argmax(zg[0])), bad, 2], None, 0.0, 7, 1, rnd)[:2] == gref[:2] == (1, int(np.argmax(zg[1])))


@pytest.mark.parametrize("temperature", [1.0, 0.6])
def test_emitted_token_is_an_exact_draw_from_the_target(temperature):
    """n = 1: the first emitted token (the draft if accepted, else the
    residual draw) is distributed as p_0, and the draft is accepted with
    probability sum_t min(p_t, q_t) (Leviathan et al. 2023, theorem 1)."""
    V, N = 6, 12000
    rng = np.random.default_rng(7)
    z = np.array([[1.2, -0.3, 0.5, 2.0, -1.0, 0.1], [0.0] * 6])
    p = softmax(z[0], temperature)
    q = np.array([0.05, 0.30, 0.25, 0.10, 0.20, 0.10])
    counts = np.zeros(V)
    accepted = 0
    for rnd in range(N):
        x = int(rng.choice(V, p=q))                 # the draft, drawn independently of the oracle's draws
        a, nxt, _ = verify_block(z, [x], q[None, :], temperature, 11, 3, rnd)
        counts[x if a == 1 else nxt] += 1
        accepted += a
    chi2 = float(np.sum((counts - N * p) ** 2 / (N * p)))
    assert chi2 < 25.0, (chi2, counts / N, p)       # 5 degrees of freedom: 99.99% quantile ~ 25.7
    rate = np.minimum(p, q).sum()
    assert abs(accepted / N - rate) < 4 * np.sqrt(rate * (1 - rate) / N), (accepted / N, rate)


def test_draws_are_in_the_open_unit_interval_and_keyed():
    u = [accept_uniform(1, 2, r, i) for r in range(3) for i in range(4)]
    assert all(0.0 < x < 1.0 for x in u) and len(set(u)) == len(u)
    g = next_uniforms(1, 2, 0, 0, 1000)
    assert g.min() > 0 and g.max() < 1 and abs(g.mean() - 0.5) < 0.05
    assert not np.array_equal(g, next_uniforms(1, 2, 0, 1, 1000))     # row is part of the counter
    assert not np.array_equal(g, next_uniforms(1, 3, 0, 0, 1000))     # and the stream part of the key
