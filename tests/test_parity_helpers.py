"""Host checks of the GPU parity harness's own arithmetic (CPU only)."""
import math

import numpy as np
import pytest

from tests.parity import Report, tie_probability


def test_tie_probability_matches_monte_carlo():
    """P(top-1 minus top-2 Gumbel-max score <= tau) from the closed form
    equals the frequency over 2e5 seeded Gumbel draws (within 4 sigma)."""
    rng = np.random.default_rng(0)
    for V, tau in ((12, 0.05), (40, 0.3), (200, 0.01)):
        a = rng.normal(scale=1.5, size=V)
        p = np.exp(a - a.max())
        p /= p.sum()
        g = -np.log(-np.log(rng.uniform(size=(200_000, V))))
        s = np.sort(a + g, axis=1)
        freq = float(np.mean(s[:, -1] - s[:, -2] <= tau))
        pt = tie_probability(p, tau)
        sd = math.sqrt(pt * (1 - pt) / 200_000)
        assert abs(freq - pt) <= 4 * sd + 1e-4, (V, tau, freq, pt)


def test_tie_probability_limits():
    p = np.full(50, 1 / 50)
    assert tie_probability(p, 0.0) == 0.0
    assert tie_probability(p, 50.0) > 0.999
    one = np.zeros(10)
    one[3] = 1.0
    assert tie_probability(one, 2.0) < 1e-12       # a certain winner never ties


def test_skip_bound():
    """Skips may exceed their expected count by 3 sqrt(E) + 2 (Poisson slack)."""
    r = Report(sampled_expected_skips=4.0, sampled_skipped=12, greedy_expected_skips=1.0, greedy_skipped=6)
    assert r.skip_bound_ok()
    r.sampled_skipped = 13
    assert not r.skip_bound_ok()
    r.sampled_skipped = 0
    r.greedy_skipped = 7
    assert not r.skip_bound_ok()


def test_greedy_tie_probability_matches_monte_carlo():
    """The spacing-model estimate of P(top-2 logit gap <= tau), averaged over
    rows of iid normal logits, is within 25% (relative) of the observed
    frequency, from vocabularies of 3001 to 151936."""
    from tests.parity import greedy_tie_probability
    rng = np.random.default_rng(1)
    for V, tau, rows in ((151936, 0.05, 200), (5003, 0.02, 1500), (3001, 0.1, 800)):
        zs = [rng.normal(size=V) for _ in range(rows)]
        est = float(np.mean([greedy_tie_probability(z, tau) for z in zs]))
        freq = float(np.mean([np.diff(np.partition(z, -2)[-2:])[0] <= tau for z in zs]))
        assert abs(est - freq) <= 0.25 * freq + 3 * math.sqrt(freq * (1 - freq) / rows), (V, tau, est, freq)


@pytest.mark.parametrize("temperature", [0.0, 0.8])
def test_id_margin_is_the_argmax_stability_bound(temperature):
    """Two score vectors within d of each other per token agree on the argmax
    whenever the reference's top-1/top-2 gap exceeds the margin id_margin
    returns (greedy rows included): perturb seeded rows by up to d per logit,
    adversarially on the top two and at random elsewhere, and check every
    row whose gap clears the margin keeps its argmax; the margin is never
    below the one-ulp tie margin and does not exceed 2d (+ 1e-4 / T)."""
    from tests.parity import id_margin, margin, top2_gap
    import synth
    cfg = synth.config("qwen", layers=1, vocab=2000)
    rng = np.random.default_rng(3)
    kept = 0
    for trial in range(400):
        z = rng.normal(scale=3.0, size=2000)
        d = float(rng.choice([0.0, 0.01, 0.05, 0.1]))
        delta = rng.uniform(-d, d, size=2000)
        top = np.argsort(z)[-2:]
        delta[top[1]], delta[top[0]] = -d, d                  # the worst case for the top two
        zg = z + delta
        tau = id_margin(cfg, zg, z, temperature)
        m = margin(cfg, float(np.max(np.abs(z))), temperature)
        assert tau >= m - 1e-15
        assert tau <= max(m, 2 * d / (temperature or 1.0) + (1e-4 if temperature else 0.0)) + 1e-12
        s = z / temperature if temperature else z
        sg = zg / temperature if temperature else zg
        if top2_gap(s) > tau:
            kept += 1
            assert int(np.argmax(sg)) == int(np.argmax(s)), (trial, d, tau)
    assert kept >= 150, kept
