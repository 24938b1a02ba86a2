"""Pins of the oracle sampler (CPU only): hand-worked penalty cases, the
softmax normalisation, the greedy limit and a chi-square test that the
Gumbel-max draw follows softmax(z/T)."""
import numpy as np
import pytest

from oracle.sampler import penalize, sample_row, top2_gap, uniforms
from tests.helpers import load_golden


def test_penalty_golden_cases():
    for c in load_golden("sampler_cases.json")["cases"]:
        z = penalize(np.array(c["logits"]), c["history"], c["rho"])
        np.testing.assert_array_equal(z, c["penalized"])
        i, p, _ = sample_row(np.array(c["logits"]), c["history"], 0.0, c["rho"], 0, 0, 0, 0)
        assert i == c["greedy_id"] and p is None


def test_penalty_unit_rho_and_untouched_tokens():
    rng = np.random.default_rng(0)
    z = rng.standard_normal(100)
    np.testing.assert_array_equal(penalize(z, [1, 5, 7], 1.0), z)
    zp = penalize(z, [1, 5, 7, 5], 1.3)
    other = np.setdiff1d(np.arange(100), [1, 5, 7])
    np.testing.assert_array_equal(zp[other], z[other])
    for t in (1, 5, 7):
        assert zp[t] == (z[t] / 1.3 if z[t] > 0 else z[t] * 1.3)


def test_probs_normalised_and_small_temperature_is_argmax():
    rng = np.random.default_rng(1)
    z = rng.standard_normal(4099) * 3
    for T in (0.7, 1.0, 2.5):
        _, p, _ = sample_row(z, [3, 4], T, 1.1, 5, 6, 7, 0)
        assert abs(p.sum() - 1.0) < 1e-12 and (p > 0).all()
    zp = penalize(z, [3, 4], 1.1)
    i, _, _ = sample_row(z, [3, 4], 1e-4, 1.1, 5, 6, 7, 0)
    assert top2_gap(zp) > 1e-2 and i == int(np.argmax(zp))


def test_gumbel_max_follows_softmax_chi_square():
    from scipy.stats import chisquare
    rng = np.random.default_rng(2)
    V, T, N = 32, 0.8, 20000
    z = rng.standard_normal(V)
    _, p, _ = sample_row(z, [], T, 1.0, 9, 1, 0, 0)
    counts = np.zeros(V)
    for r in range(N):
        i, _, _ = sample_row(z, [], T, 1.0, 9, 1, r, 0)
        counts[i] += 1
    stat, pval = chisquare(counts, N * p)
    assert pval > 1e-3, (stat, pval)


def test_draws_depend_on_every_key_and_counter_field():
    base = uniforms(1, 2, 3, 4, 64)
    for args in [(9, 2, 3, 4), (1, 9, 3, 4), (1, 2, 9, 4), (1, 2, 3, 9)]:
        assert not np.array_equal(base, uniforms(*args, 64))


def test_both_fields_of_a_word_are_independent_uniforms():
    """Tokens 2i and 2i + 1 take disjoint bit fields of one generator word:
    each marginal is uniform on (0, 1) and the pair is uncorrelated (a field
    taken twice, or overlapping fields, would fail one of these)."""
    from scipy.stats import kstest
    u = np.concatenate([uniforms(3, 1, r, 0, 4096) for r in range(8)])
    even, odd = u[0::2], u[1::2]
    assert kstest(even, "uniform").pvalue > 1e-3 and kstest(odd, "uniform").pvalue > 1e-3
    assert abs(np.corrcoef(even, odd)[0, 1]) < 0.02
    assert not np.array_equal(even, odd)
