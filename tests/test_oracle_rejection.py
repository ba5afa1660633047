"""Pins for the oracle's rejection-sampling verification (runs on the CPU).

The pages state that rejection sampling keeps the target distribution
(vLLM features 03, '1. principle', citing Leviathan et al. and Chen et al.)
and name it as the usual verifier (Arctic blog, 'what is speculative
decoding').  These tests check the oracle against consequences of that rule
that do not depend on the oracle's own code: the output distribution
(chi-square at V = 8), the per-position acceptance probability
sum_x min(p(x), q(x)), special cases that reduce to greedy verification or
to a point mass, scipy's softmax, and the worked example in sampling form.
"""
import numpy as np
import pytest
from scipy import special, stats

from conftest import golden

NEG = np.float32(-1.0e4)   # exp(-1e4 - M) is exactly 0 in fp64


def _softmax64(logits32):
    return special.softmax(np.asarray(logits32, np.float64), axis=-1)


def _sample_rows(rng, probs, n):
    """n draws from each row of probs (inverse CDF in numpy)."""
    c = np.cumsum(probs, axis=-1)
    c[:, -1] = 1.0
    u = rng.random((n, probs.shape[0]))
    return np.stack([np.searchsorted(c[i], u[:, i], side="right") for i in range(probs.shape[0])],
                    axis=1).astype(np.int32)


@pytest.mark.parametrize("K", [1, 3])
def test_output_distribution_chisquare_v8(orc, K):
    """Given position j is reached, the emitted token is distributed as the
    target's p_j; the accept frequency at position i is sum_x min(p_i, q_i)."""
    rng = np.random.default_rng(100 + K)
    V, T = 8, 200_000
    p = rng.dirichlet(np.ones(V), size=K + 1)
    q = rng.dirichlet(np.ones(V), size=K)
    tl = np.log(p).astype(np.float32)
    dl = np.log(q).astype(np.float32)
    p_eff = _softmax64(tl)          # what the fp32 logits really encode
    q_eff = _softmax64(dl)
    target = np.broadcast_to(tl, (T, K + 1, V)).copy()
    draftl = np.broadcast_to(dl, (T, K, V)).copy()
    x = _sample_rows(rng, q_eff, T)
    u = rng.random((T, K + 1), dtype=np.float32)
    out = orc.verify_rejection(target, draftl, x, u)
    n = out["accepted"]
    for j in range(K + 1):
        reached = n >= j
        tok = out["emitted"][reached, j]
        counts = np.bincount(tok, minlength=V)
        assert stats.chisquare(counts, p_eff[j] * reached.sum()).pvalue > 1e-3
    for i in range(K):
        reached = n >= i
        acc = (n[reached] > i).astype(np.float64)
        beta = np.minimum(p_eff[i], q_eff[i]).sum()
        assert abs(acc.mean() - beta) < 4 * np.sqrt(beta * (1 - beta) / reached.sum())
    # reported probabilities are the softmax values at the drafted ids
    np.testing.assert_allclose(out["p_draft"], p_eff[np.arange(K), x], rtol=1e-12)
    np.testing.assert_allclose(out["q_draft"], q_eff[np.arange(K), x], rtol=1e-12)


def test_probabilities_match_scipy_softmax_with_temperature(orc):
    """p_i(x_i), q_i(x_i) equal scipy.special.softmax(logits / T) at x_i."""
    rng = np.random.default_rng(7)
    B, K, V = 6, 4, 333
    for T in (0.5, 1.0, 1.7):
        tl = (rng.standard_normal((B, K + 1, V)) * 3).astype(np.float32)
        dl = (rng.standard_normal((B, K, V)) * 3).astype(np.float32)
        x = rng.integers(0, V, (B, K)).astype(np.int32)
        u = rng.random((B, K + 1), dtype=np.float32)
        out = orc.verify_rejection(tl, dl, x, u, temperature=T)
        ps = special.softmax(tl.astype(np.float64) / T, axis=-1)
        qs = special.softmax(dl.astype(np.float64) / T, axis=-1)
        bi, ki = np.meshgrid(np.arange(B), np.arange(K), indexing="ij")
        np.testing.assert_allclose(out["p_draft"], ps[bi, ki, x], rtol=1e-12)
        np.testing.assert_allclose(out["q_draft"], qs[bi, ki, x], rtol=1e-12)


def test_identical_draft_accepts_everything(orc):
    """q = p: p/q = 1 > u, so every draft is accepted and the bonus ~ p_K."""
    rng = np.random.default_rng(8)
    V, K, T = 8, 3, 100_000
    tl = np.log(rng.dirichlet(np.ones(V), size=K + 1)).astype(np.float32)
    target = np.broadcast_to(tl, (T, K + 1, V)).copy()
    draftl = target[:, :K, :].copy()
    x = _sample_rows(rng, _softmax64(tl[:K]), T)
    u = rng.random((T, K + 1), dtype=np.float32)
    out = orc.verify_rejection(target, draftl, x, u)
    assert (out["accepted"] == K).all()
    counts = np.bincount(out["emitted"][:, K], minlength=V)
    assert stats.chisquare(counts, _softmax64(tl[K]) * T).pvalue > 1e-3


def test_one_hot_target_is_greedy(orc):
    """A one-hot target p makes rejection sampling deterministic: a draft is
    accepted iff it is the target's token, and the residual after a
    rejection is a point mass on that token -- greedy verification."""
    rng = np.random.default_rng(9)
    B, K, V = 400, 4, 50
    t = rng.integers(0, V, (B, K + 1))
    tl = np.full((B, K + 1, V), NEG, np.float32)
    np.put_along_axis(tl, t[..., None], 0.0, axis=-1)
    dl = rng.standard_normal((B, K, V)).astype(np.float32)
    x = np.where(rng.random((B, K)) < 0.7, t[:, :K], rng.integers(0, V, (B, K))).astype(np.int32)
    u = rng.random((B, K + 1), dtype=np.float32)
    rej = orc.verify_rejection(tl, dl, x, u)
    gre = orc.verify_greedy(tl, x)
    assert np.array_equal(rej["accepted"], gre["accepted"])
    assert np.array_equal(rej["emitted"], gre["emitted"])


def test_one_hot_draft_accepts_with_p(orc):
    """q one-hot at x gives p/q = p(x): accepted with probability p(x)."""
    rng = np.random.default_rng(10)
    V, T = 8, 200_000
    tl = np.log(rng.dirichlet(np.ones(V), size=2)).astype(np.float32)
    x0 = 3
    dl = np.full((1, V), NEG, np.float32)
    dl[0, x0] = 0.0
    target = np.broadcast_to(tl, (T, 2, V)).copy()
    draftl = np.broadcast_to(dl, (T, 1, V)).copy()
    x = np.full((T, 1), x0, np.int32)
    u = rng.random((T, 2), dtype=np.float32)
    out = orc.verify_rejection(target, draftl, x, u)
    pa = _softmax64(tl[0])[x0]
    freq = out["accepted"].mean()
    assert abs(freq - pa) < 4 * np.sqrt(pa * (1 - pa) / T)
    # after a rejection the residual max(0, p - q) excludes x0 entirely
    rej = out["accepted"] == 0
    assert not (out["emitted"][rej, 0] == x0).any()


def test_worked_example_sampling_form(orc):
    """Arctic blog, 'a simple example', with a sampling verifier: the target
    favours 13 and 578 (ratio >= 1: accepted for any u); at the third
    position p = {7301: 0.1, 21747: 0.9}, q = {7301: 0.5, 6: 0.5} and
    u = 0.9 > p/q = 0.2 rejects 7301; the residual max(0, p - q) is a point
    mass on 21747, which is emitted whatever the final uniform."""
    g = golden("worked_example.json")
    V = g["vocab_for_test"]
    d = g["drafts"]

    def row(mass):
        r = np.full(V, NEG, np.float32)
        for k, v in mass.items():
            r[k] = np.log(v)
        return r
    tl = np.stack([row({d[0]: 0.9, 5: 0.1}), row({d[1]: 0.8, 5: 0.2}),
                   row({d[2]: 0.1, g["target_token"]: 0.9}), row({1: 1.0})])[None]
    dl = np.stack([row({d[0]: 0.5, 6: 0.5}), row({d[1]: 0.4, 6: 0.6}),
                   row({d[2]: 0.5, 6: 0.5})])[None]
    for ufin in (0.0, 0.5, 0.999):
        u = np.array([[0.99, 0.99, 0.9, ufin]], np.float32)
        out = orc.verify_rejection(tl, dl, np.array([d], np.int32), u)
        assert out["accepted"][0] == 2
        assert out["emitted"][0].tolist() == g["accepted_drafts"] + [g["target_token"], -1]
        assert out["p_draft"][0, 2] == pytest.approx(0.1, rel=1e-6)
        assert out["q_draft"][0, 2] == pytest.approx(0.5, rel=1e-6)


def test_flags_and_draft_len(orc):
    """Out-of-range draft ids are rejected (flagged); draft_len 0 samples the
    bonus from p_0; lengths outside [0, K] are clamped and flagged; a
    near-tie accept test is reported."""
    rng = np.random.default_rng(11)
    B, K, V = 4, 3, 16
    tl = rng.standard_normal((B, K + 1, V)).astype(np.float32)
    dl = tl[:, :K, :].copy()                  # q = p: valid drafts always accepted
    x = rng.integers(0, V, (B, K)).astype(np.int32)
    x[1, 1] = -3
    u = rng.random((B, K + 1), dtype=np.float32)
    dlen = np.array([0, 3, 7, 2], np.int32)
    out = orc.verify_rejection(tl, dl, x, u, draft_len=dlen)
    assert out["accepted"].tolist() == [0, 1, 3, 2]
    assert out["flags"].tolist() == [0, orc.FLAG_DRAFT_OOR, orc.FLAG_BAD_LEN, 0]
    assert (out["emitted"][0, 1:] == -1).all()
    assert out["p_draft"][1, 1] == 0.0 and out["q_draft"][1, 1] == 0.0
    # draft_len 0: the emitted token is a sample of p_0 with u[b][K]
    c = np.cumsum(_softmax64(tl[0, 0]))
    assert out["emitted"][0, 0] == int(np.searchsorted(c, u[0, K] * c[-1], side="right"))
    # a uniform planted just below p/q is flagged as an accept tie
    tl2 = np.log(np.array([[[0.3, 0.7], [0.5, 0.5]]])).astype(np.float32)
    dl2 = np.log(np.array([[[0.6, 0.4]]])).astype(np.float32)
    ratio = _softmax64(tl2[0, 0])[0] / _softmax64(dl2[0, 0])[0]
    u2 = np.array([[np.nextafter(np.float32(ratio), np.float32(0)), 0.5]], np.float32)
    out2 = orc.verify_rejection(tl2, dl2, np.array([[0]], np.int32), u2)
    assert out2["accept_tie"][0]


def test_masked_entries_equal_smaller_vocabulary(orc):
    """A -inf logit has probability 0, so a row with masked entries is the
    same distribution as the row with those entries removed: embedding a
    V'-token problem into V > V' ids (kept ids increasing, the rest -inf in
    both target and draft) must give the same decisions, the same p and q,
    and the same emitted tokens mapped through the embedding."""
    rng = np.random.default_rng(77)
    B, K, Vs, V = 24, 4, 40, 300
    for T in (1.0, 0.7):
        tl = (2.0 * rng.standard_normal((B, K + 1, Vs))).astype(np.float32)
        dl = (tl[:, :K] + 0.5 * rng.standard_normal((B, K, Vs))).astype(np.float32)
        x = rng.integers(0, Vs, size=(B, K)).astype(np.int32)
        u = rng.random((B, K + 1), dtype=np.float32)
        ids = np.sort(rng.choice(V, size=Vs, replace=False)).astype(np.int32)
        tL = np.full((B, K + 1, V), -np.inf, np.float32)
        dL = np.full((B, K, V), -np.inf, np.float32)
        tL[..., ids] = tl
        dL[..., ids] = dl
        small = orc.verify_rejection(tl, dl, x, u, T)
        large = orc.verify_rejection(tL, dL, ids[x], u, T)
        np.testing.assert_array_equal(large["accepted"], small["accepted"])
        np.testing.assert_array_equal(large["p_draft"], small["p_draft"])
        np.testing.assert_array_equal(large["q_draft"], small["q_draft"])
        for b in range(B):
            n = small["accepted"][b]
            np.testing.assert_array_equal(large["emitted"][b, :n + 1], ids[small["emitted"][b, :n + 1]])
            assert (large["emitted"][b, n + 1:] == -1).all()


# ------------------------------------------------------- probability input

@pytest.mark.parametrize("K", [1, 3])
def test_probability_input_chisquare_v8(orc, K):
    """With the target and draft given as probabilities (the verifier's
    interface takes logits or probabilities), the emitted token at each
    reached position is distributed as p and the accept frequency is
    sum_x min(p, q); rows need not be normalised (the row's sum divides)."""
    rng = np.random.default_rng(300 + K)
    V, T = 8, 200_000
    p = rng.dirichlet(np.ones(V), size=K + 1).astype(np.float32)
    q = rng.dirichlet(np.ones(V), size=K).astype(np.float32)
    p[0, 3] = 0.0                                  # an impossible target token
    q[0, 5] = 0.0                                  # and an impossible draft token
    p3 = (p * np.float32(3.0)).astype(np.float32)                         # unnormalised
    p_eff = p3.astype(np.float64) / p3.astype(np.float64).sum(axis=1, keepdims=True)
    q_eff = q.astype(np.float64) / q.astype(np.float64).sum(axis=1, keepdims=True)
    target = np.broadcast_to(p3, (T, K + 1, V)).copy()
    draftp = np.broadcast_to(q, (T, K, V)).copy()
    x = _sample_rows(rng, q_eff, T)
    u = rng.random((T, K + 1), dtype=np.float32)
    out = orc.verify_rejection(target, draftp, x, u, probs=True)
    n = out["accepted"]
    for j in range(K + 1):
        reached = n >= j
        counts = np.bincount(out["emitted"][reached, j], minlength=V)
        assert counts[3] == 0 or j != 0
        expect = p_eff[j] * reached.sum()
        live = expect > 0
        assert stats.chisquare(counts[live], expect[live]).pvalue > 1e-3
    for i in range(K):
        reached = n >= i
        acc = (n[reached] > i).astype(np.float64)
        beta = np.minimum(p_eff[i], q_eff[i]).sum()
        assert abs(acc.mean() - beta) < 4 * np.sqrt(beta * (1 - beta) / reached.sum())
    np.testing.assert_allclose(out["p_draft"], p_eff[np.arange(K), x], rtol=1e-12)


def test_probability_input_equals_logit_input(orc):
    """Probabilities exp(l) / sum exp(l) rounded to fp32 give the logit
    path's decisions except within the rounding band of a tie; scaling
    every row by a power of two changes nothing at all."""
    from proposal_sv_verify_amd import workloads as W
    wl = W.rejection_workload(64, 4, 500, 1.0, 0.5, 1.0, seed=311, dtype="f32")
    P = _softmax64(wl["target"]).astype(np.float32)
    Q = _softmax64(wl["draft_logits"]).astype(np.float32)
    a = orc.verify_rejection(wl["target"], wl["draft_logits"], wl["draft"], wl["uniforms"])
    b = orc.verify_rejection(P, Q, wl["draft"], wl["uniforms"], probs=True)
    tie = a["accept_tie"] | a["sample_tie"] | b["accept_tie"] | b["sample_tie"]
    same = (a["emitted"] == b["emitted"]).all(axis=1)
    assert (same | tie).all() and same.sum() >= 60
    c = orc.verify_rejection(P * np.float32(0.25), Q * np.float32(8.0), wl["draft"], wl["uniforms"],
                             probs=True)
    for k in ("accepted", "emitted", "p_draft", "q_draft", "accept_tie", "sample_tie"):
        np.testing.assert_array_equal(b[k], c[k], err_msg=k)


def test_probability_input_zero_draft_probability_accepts(orc):
    """q(x) = 0 makes the ratio infinite: the draft is accepted whatever u."""
    V = 6
    p = np.array([[0.1, 0.2, 0.3, 0.4, 0.0, 0.0], [0.5, 0.5, 0, 0, 0, 0]], np.float32)[None]
    q = np.array([[0.0, 0.5, 0.5, 0.0, 0.0, 0.0]], np.float32)[None]
    x = np.array([[0]], np.int32)
    u = np.array([[0.999, 0.7]], np.float32)
    out = orc.verify_rejection(p, q, x, u, probs=True)
    assert out["accepted"][0] == 1 and out["emitted"][0, 0] == 0
    assert out["emitted"][0, 1] == 1                 # bonus from p_1 = (0.5, 0.5): u 0.7 -> id 1
    assert V == p.shape[-1]


# ------------------------------------------------------------- tie flags
#
# GPU parity for rejection sampling compares every decision except those the
# oracle flags as ties, so the flags themselves are pinned here on rows whose
# probabilities are exact binary fractions (given as probabilities, so p and
# q are the row values over an exactly representable sum).  An accept test
# is a tie when |u - p/q| < 1e-6 (the band the problem statement fixes); a
# final sample is a tie when u*S lies within SAMPLE_BAND_SCALE * sqrt(sum p^2
# + sum q^2) probability mass of an end of the chosen token's CDF interval
# (q only after a rejection).  The square roots below are worked by hand.

def _probs(rows):
    return np.array(rows, np.float32)[None]


def _u_at(target, side):
    """The fp32 uniform nearest target + side, and its exact distance from
    target (fp64)."""
    u = np.float32(target + side)
    return u, abs(float(u) - target)


@pytest.mark.parametrize("side", [-3e-7, 3e-7, -9e-7, 9e-7, -1.1e-6, 1.1e-6, -3e-6, 3e-6])
def test_accept_tie_flag_band(orc, side):
    """p(x)/q(x) = 0.125/0.25 = 0.5 exactly.  A uniform within 1e-6 of 0.5
    is flagged whichever way the test goes; one outside is not; the
    decision itself is u < 0.5 either way."""
    tl = _probs([[0.5, 0.25, 0.125, 0.125], [0.25, 0.25, 0.25, 0.25]])
    dl = _probs([[0.25, 0.25, 0.25, 0.25]])
    u0, dist = _u_at(0.5, side)
    assert abs(dist - 1e-6) > 5e-8                    # fp32 rounding keeps the side of the band
    u = np.array([[u0, 0.3]], np.float32)
    out = orc.verify_rejection(tl, dl, np.array([[2]], np.int32), u, probs=True)
    assert out["p_draft"][0, 0] == 0.125 and out["q_draft"][0, 0] == 0.25
    assert out["accepted"][0] == (1 if u0 < np.float32(0.5) else 0)
    assert out["accept_tie"][0] == (dist < 1e-6)
    assert not out["sample_tie"][0]


def test_accept_tie_counts_only_decisions_taken(orc):
    """A near-tie uniform at a position after the first rejection, past
    draft_len, at an out-of-range id (ratio 0 against u = 0) or where the
    draft has q(x) = 0 (ratio +inf) is not a decision the verifier takes on
    a ratio: none is flagged.  A clear decision (|u - p/q| >= 1e-3) is not
    flagged either."""
    half = [0.25, 0.25, 0.25, 0.25]
    tl = _probs([[0.5, 0.25, 0.125, 0.125], [0.5, 0.25, 0.125, 0.125], half])
    dl = _probs([half, half])
    x = np.array([[2, 2]], np.int32)                  # ratios 0.5 and 0.5
    cases = [
        (np.array([[0.9, 0.5 - 1e-7, 0.3]], np.float32), None, 0),   # rejected at 0; 1 not taken
        (np.array([[0.1, 0.5 - 1e-7, 0.3]], np.float32), np.array([1], np.int32), 1),   # past len
        (np.array([[0.499, 0.501, 0.3]], np.float32), None, 1),       # clear both ways
    ]
    for u, dlen, acc in cases:
        out = orc.verify_rejection(tl, dl, x, u, draft_len=dlen, probs=True)
        assert out["accepted"][0] == acc
        assert not out["accept_tie"][0], (u, dlen)
    bad = orc.verify_rejection(tl, dl, np.array([[-1, 2]], np.int32),
                               np.array([[0.0, 0.2, 0.3]], np.float32), probs=True)
    assert bad["accepted"][0] == 0 and not bad["accept_tie"][0]
    qz = _probs([[0.0, 0.5, 0.5, 0.0], half])
    inf = orc.verify_rejection(tl, qz, np.array([[0, 2]], np.int32),
                               np.array([[0.9999999, 0.9, 0.3]], np.float32), probs=True)
    assert inf["accepted"][0] >= 1 and not inf["accept_tie"][0]
    # the same near-tie uniform at position 1 when position 0 is accepted is flagged
    near = orc.verify_rejection(tl, dl, x, np.array([[0.1, 0.5 - 3e-7, 0.3]], np.float32),
                                probs=True)
    assert near["accepted"][0] == 2 and near["accept_tie"][0]


# The bonus row p = (1/2, 1/4, 1/8, 1/8): sum p^2 = 1/4 + 1/16 + 2/64 = 11/32,
# so the band is SCALE * sqrt(11/32); interval ends at 1/2, 3/4, 7/8.
BONUS_P = [0.5, 0.25, 0.125, 0.125]
BONUS_ROOT = np.sqrt(11.0 / 32.0)


@pytest.mark.parametrize("end,token_below", [(0.5, 0), (0.75, 1), (0.875, 2)])
@pytest.mark.parametrize("frac", [-1.5, -0.8, 0.8, 1.5])
def test_sample_tie_flag_band_bonus(orc, end, token_below, frac):
    """The bonus draw (draft_len 0, r = p, S = 1): u*S placed frac bands
    from an interval end.  Within the band (|frac| < 1) the draw is flagged,
    outside it is not; the token is the one whose interval holds u*S."""
    band = orc.SAMPLE_BAND_SCALE * BONUS_ROOT
    tl = _probs([BONUS_P])
    uK, dist = _u_at(end, frac * band)
    assert abs(dist / band - abs(frac)) < 0.1
    out = orc.verify_rejection(tl, np.zeros((1, 0, 4), np.float32), np.zeros((1, 0), np.int32),
                               np.array([[uK]], np.float32), probs=True)
    assert out["emitted"][0, 0] == (token_below + 1 if frac > 0 else token_below)
    assert out["sample_tie"][0] == (abs(frac) < 1.0)
    assert not out["accept_tie"][0]


# After a rejection: p = (3/8, 3/8, 1/8, 1/8), q = (1/8, 1/8, 3/8, 3/8):
# r = (1/4, 1/4, 0, 0), S = 1/2, one interval end inside at 1/4.  sum p^2 =
# sum q^2 = 2 (9/64) + 2 (1/64) = 5/16, so the band is SCALE * sqrt(5/8); a
# band without the draft's terms would be SCALE * sqrt(5/16), 0.707 of it.
RESID_P = [0.375, 0.375, 0.125, 0.125]
RESID_Q = [0.125, 0.125, 0.375, 0.375]
RESID_ROOT = np.sqrt(5.0 / 8.0)


@pytest.mark.parametrize("frac", [-1.25, -0.85, 0.85, 1.25])
def test_sample_tie_flag_band_residual(orc, frac):
    """x = 2 (ratio 1/3) rejected by u = 0.9; the residual is drawn with
    u_K * S placed frac bands from the interval end 1/4 (u_K near 1/2)."""
    band = orc.SAMPLE_BAND_SCALE * RESID_ROOT
    tl = _probs([RESID_P, BONUS_P])
    dl = _probs([RESID_Q])
    uK, dist2 = _u_at(0.5, 2.0 * frac * band)           # u_K * S = u_K / 2
    assert abs(dist2 / 2.0 / band - abs(frac)) < 0.1
    out = orc.verify_rejection(tl, dl, np.array([[2]], np.int32),
                               np.array([[0.9, uK]], np.float32), probs=True)
    assert out["accepted"][0] == 0
    assert out["emitted"][0, 0] == (1 if frac > 0 else 0)
    assert out["sample_tie"][0] == (abs(frac) < 1.0)
    assert not out["accept_tie"][0]


def test_sample_tie_at_the_top_of_the_distribution(orc):
    """u_K = the largest fp32 below 1 puts u*S within 6e-8 of the top of the
    last token's interval: flagged; u_K = 0 sits at the bottom of the first
    token's interval: flagged."""
    tl = _probs([BONUS_P])
    empty = (np.zeros((1, 0, 4), np.float32), np.zeros((1, 0), np.int32))
    top = orc.verify_rejection(tl, *empty, np.array([[np.nextafter(np.float32(1), np.float32(0))]],
                                                    np.float32), probs=True)
    assert top["emitted"][0, 0] == 3 and top["sample_tie"][0]
    bottom = orc.verify_rejection(tl, *empty, np.array([[0.0]], np.float32), probs=True)
    assert bottom["emitted"][0, 0] == 0 and bottom["sample_tie"][0]


def test_flagged_fraction_at_the_rejection_workload_size(orc):
    """On full-size rejection rows (V = 128256, bf16 N(0, 2) target and
    target + N(0, 0.5) draft) the tie flags mark a small fraction of draws:
    a band wider than the stated one would flag far more, so the GPU parity
    tests would compare little.  Uniforms are redrawn over the same rows."""
    from proposal_sv_verify_amd import workloads as W
    wl = W.rejection_workload(8, 5, 128256, seed=W.seed_for(3, salt=7))
    flags = accept = 0
    trials = 0
    rng = np.random.default_rng(12)
    for rep in range(6):
        u = rng.random((8, 6), dtype=np.float32)
        out = orc.verify_rejection(wl["target"], wl["draft_logits"], wl["draft"], u)
        flags += int(out["sample_tie"].sum())
        accept += int(out["accept_tie"].sum())
        trials += 8
    assert accept == 0
    assert flags <= 0.1 * trials


def test_sample_cdf_hand_worked(orc):
    """The residual of the rows above is (1/4, 1/4, 0, 0) with S = 1/2; with
    no draft row the CDF is p's; q = p leaves no residual, so p is drawn;
    S equals the total-variation distance 1 - sum min(p, q) on random rows."""
    C, S = orc.sample_cdf(np.array(RESID_P, np.float32), np.array(RESID_Q, np.float32), probs=True)
    assert S == 0.5 and C.tolist() == [0.25, 0.5, 0.5, 0.5]
    C, S = orc.sample_cdf(np.array(BONUS_P, np.float32), probs=True)
    assert S == 1.0 and C.tolist() == [0.5, 0.75, 0.875, 1.0]
    C, S = orc.sample_cdf(np.array(RESID_P, np.float32), np.array(RESID_P, np.float32), probs=True)
    assert S == 1.0 and C.tolist() == [0.375, 0.75, 0.875, 1.0]
    rng = np.random.default_rng(13)
    for T in (0.7, 1.0):
        t = (2 * rng.standard_normal(500)).astype(np.float32)
        d = (t + 0.5 * rng.standard_normal(500)).astype(np.float32)
        C, S = orc.sample_cdf(t, d, T)
        p, q = _softmax64(t / np.float32(T) if T == 1.0 else t.astype(np.float64) / T), \
            _softmax64(d / np.float32(T) if T == 1.0 else d.astype(np.float64) / T)
        assert S == pytest.approx(1.0 - np.minimum(p, q).sum(), rel=1e-12)
        assert np.all(np.diff(C) >= 0) and C[-1] == S
