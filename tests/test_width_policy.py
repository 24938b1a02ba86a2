"""The draft width controller (host library, no GPU): per-position acceptance
estimates against simulated rounds, and its choice against the closed form of
the expected tokens of a round at a constant acceptance rate a,
E(n) = (1 - a^(n+1)) / (1 - a) (Leviathan, Kalman, Matias 2023, eq. 1)."""
import numpy as np
import pytest

from block_diffusion_drafter_fwd_amd import abi
from block_diffusion_drafter_fwd_amd.drafter import WidthPolicy


@pytest.fixture(scope="module")
def lib():
    return abi.load("host")


def _simulate(pol, alpha, rounds, rng, width):
    for _ in range(rounds):
        acc = 0
        while acc < width and rng.random() < alpha:
            acc += 1
        pol.observe(width, acc)


def test_always_and_never_accepted(lib):
    p = WidthPolicy(15, 440.0, 4.0, 0.0, 0.0, 0.9, lib=lib)
    for _ in range(200):
        p.observe(15, 15)
    assert min(p.rates()) > 0.99 and p.choose() == 15
    q = WidthPolicy(15, 440.0, 4.0, 300.0, 20.0, 0.9, lib=lib)
    for _ in range(200):
        q.observe(15, 0)
    assert q.rates()[0] < 0.01 and q.choose() == 1
    assert q.rates()[1] == pytest.approx(0.5)          # never tested: still the prior


@pytest.mark.parametrize("alpha,costs", [(0.5, (440.0, 4.0, 300.0, 20.0)), (0.8, (440.0, 4.0, 300.0, 20.0)),
                                         (0.9, (100.0, 50.0, 100.0, 50.0)), (0.7, (10.0, 30.0, 0.0, 0.0))])
def test_choice_matches_the_closed_form(lib, alpha, costs):
    rng = np.random.default_rng(int(alpha * 100))
    p = WidthPolicy(15, *costs, decay=1.0, lib=lib)
    _simulate(p, alpha, 6000, rng, 15)
    rates = np.array(p.rates())
    tested = rates[:6]
    assert np.all(np.abs(tested - alpha) < 0.05), rates
    df, dp, vf, vp = costs
    n = np.arange(1, 16)
    a_hat = float(np.mean(tested))
    expect = (1 - a_hat ** (n + 1)) / (1 - a_hat)
    rate = expect / (df + dp * n + vf + vp * (n + 1))
    best = int(n[np.argmax(rate)])
    # the estimates of deep positions are noisier: accept a neighbour whose
    # closed-form rate is within 2% of the best
    got = p.choose()
    assert rate[got - 1] >= 0.98 * rate.max(), (got, best, rate)


def test_bad_arguments_are_refused(lib):
    with pytest.raises(abi.DFlashError):
        WidthPolicy(0, 1.0, 1.0, lib=lib)
    with pytest.raises(abi.DFlashError):
        WidthPolicy(8, 1.0, 1.0, decay=0.0, lib=lib)
    p = WidthPolicy(8, 1.0, 1.0, lib=lib)
    with pytest.raises(abi.DFlashError):
        p.observe(3, 4)
