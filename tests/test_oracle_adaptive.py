"""Pins for the oracle's adaptive speculation length (runs on the CPU).

[Handbook] "adaptive": after each verification round the accepted draft
count feeds an exponential moving average, and the next round's speculation
length is one of a few fixed tiers (default 1, 3, 7) chosen from it; only
the length changes, never the verification, so the output is unchanged.
The checks below use what the mathematics fixes: the closed form of the
average under a constant input, the limit it converges to, the
no-smoothing case, and the tier rule's defining properties.
"""
import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("a,ema0,beta", [(2.5, 0.0, 0.2), (0.0, 6.0, 0.3), (7.0, 1.0, 0.05)])
def test_constant_input_closed_form(a, ema0, beta):
    """ema_n = a + (ema0 - a) (1 - beta)^n for a constant accepted count a."""
    n = 60
    _, emas = oracle.adaptive_lengths([a] * n, beta=beta, ema0=ema0)
    closed = [a + (ema0 - a) * (1.0 - beta) ** (i + 1) for i in range(n)]
    np.testing.assert_allclose(emas, closed, rtol=0, atol=1e-12)


def test_no_smoothing_follows_the_last_round():
    """beta = 1: the average is the last round's count, so the length
    follows it one round later."""
    acc = [0, 2, 6, 1, 3, 7, 0]
    ks, emas = oracle.adaptive_lengths(acc, beta=1.0, ema0=0.0)
    assert emas == [float(a) for a in acc]
    assert ks == [1] + [oracle.adaptive_tier(a, (1, 3, 7)) for a in acc[:-1]]
    assert ks == [1, 1, 7, 7, 3, 7, 7]


def test_tier_rule():
    """The smallest tier of at least twice the average, else the largest:
    a tier, non-decreasing in the average, never below twice the average
    unless the largest tier is, and the tier below it always is."""
    tiers = (1, 3, 7)
    prev = 0
    for e in np.linspace(0.0, 10.0, 1001):
        k = oracle.adaptive_tier(e, tiers)
        assert k in tiers and k >= prev
        prev = k
        if 2.0 * e <= tiers[-1]:
            assert k >= 2.0 * e and all(t < 2.0 * e for t in tiers if t < k)
        else:
            assert k == tiers[-1]
    assert oracle.adaptive_tier(0.5, tiers) == 1 and oracle.adaptive_tier(0.51, tiers) == 3
    assert oracle.adaptive_tier(1.5, tiers) == 3 and oracle.adaptive_tier(1.51, tiers) == 7


def test_moves_both_ways_from_the_ends():
    """At length 1 the average never exceeds 1, yet drafts accepted 60% of
    the time move the length up; under sustained full rejection the average
    only approaches 0, yet the length comes back down to 1."""
    ks, emas = oracle.adaptive_lengths([0.6] * 20, ema0=0.0)
    assert ks[0] == 1 and ks[-1] == 3
    assert all(k == oracle.adaptive_tier(e, (1, 3, 7)) for k, e in zip(ks[1:], emas))
    ks, _ = oracle.adaptive_lengths([0.0] * 20, ema0=7.0)
    assert ks[0] == 7 and ks[-1] == 1


def test_converges_to_the_matching_tier():
    """Sustained full acceptance at the largest tier keeps it; sustained
    rejection of everything brings the length down to the smallest tier."""
    ks, _ = oracle.adaptive_lengths([7] * 40, ema0=0.0)
    assert ks[0] == 1 and ks[-1] == 7 and ks == sorted(ks)
    ks, _ = oracle.adaptive_lengths([0] * 40, ema0=7.0)
    assert ks[0] == 7 and ks[-1] == 1 and ks == sorted(ks, reverse=True)
