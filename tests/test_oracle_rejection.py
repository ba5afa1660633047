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
