"""Pins for the oracle's greedy verification (runs on the CPU).

Each test checks the oracle against something other than itself: values the
pages print for a worked example, the tau closed form under planted
acceptance, output identity with plain greedy decoding, and numpy's argmax.
"""
import numpy as np
import pytest
from scipy import stats

from conftest import golden
from proposal_sv_verify_amd import workloads as W


def _rows_with_argmax(V, ids, seed):
    """fp32 rows whose unique maximum sits at the given ids."""
    rng = np.random.default_rng(seed)
    rows = rng.standard_normal((len(ids), V)).astype(np.float32)
    for r, i in enumerate(ids):
        rows[r, i] = 10.0
    return rows


def test_worked_example(orc):
    """Arctic blog, 'a simple example': drafts 13, 578, 7301 after token 16;
    13 and 578 are accepted and the target supplies 21747 (2/3 = 66.7%)."""
    g = golden("worked_example.json")
    V = g["vocab_for_test"]
    K = len(g["drafts"])
    # rows 0..2 score the drafts; the target's choices are the accepted drafts
    # followed by its own token; row 3 (after the third draft) is never used.
    choices = g["accepted_drafts"] + [g["target_token"], 0]
    logits = _rows_with_argmax(V, choices, seed=1)[None]
    out = orc.verify_greedy(logits, np.array([g["drafts"]], np.int32))
    n = int(out["accepted"][0])
    assert n == len(g["accepted_drafts"])
    assert out["emitted"][0].tolist() == g["accepted_drafts"] + [g["target_token"], -1]
    assert round(100.0 * n / K, 1) == g["acceptance_rate_percent"]


def test_all_accepted_plus_one(orc):
    """vLLM features 03, '1. principle': four correct drafts plus the big
    model's own token settle five tokens in one step."""
    g = golden("all_accept.json")
    K = g["drafts"]
    V = 50
    ids = [7, 3, 41, 19, 22]
    logits = _rows_with_argmax(V, ids, seed=2)[None]
    out = orc.verify_greedy(logits, np.array([ids[:K]], np.int32))
    assert out["accepted"][0] == K
    emitted = out["emitted"][0]
    assert (emitted >= 0).sum() == g["tokens_settled"]
    assert emitted[K] == ids[K]


def test_argmax_matches_numpy_with_ties(orc):
    """Lowest id among equal maxima, as numpy.argmax, on bf16 rows with
    planted duplicate maxima, including -0/+0 and all-equal rows."""
    rng = np.random.default_rng(3)
    for trial in range(300):
        V = int(rng.integers(1, 300))
        x = rng.standard_normal(V).astype(np.float32) * 2
        bits = W.f32_to_bf16_bits(x)
        if V > 2 and trial % 3 == 0:
            m = bits[np.argmax(W.bf16_bits_to_f32(bits))]
            where = rng.choice(V, size=min(V, 3), replace=False)
            bits[where] = m
        if trial % 50 == 1:
            bits[:] = 0x8000          # -0.0 everywhere
            bits[V // 2:] = 0x0000    # +0.0 in the second half: still all equal
        ref = int(np.argmax(W.bf16_bits_to_f32(bits)))
        assert orc.argmax(bits) == ref
        f = W.bf16_bits_to_f32(bits).copy()
        assert orc.argmax(f) == ref


@pytest.mark.parametrize("case", golden("tau_values.json")["cases"],
                         ids=lambda c: "a%.1f_g%d" % (c["alpha"], c["gamma"]))
def test_tau_closed_form(orc, case):
    """Handbook, 'key metrics': under independent acceptance alpha with gamma
    drafts the mean tokens per step is (1 - alpha^(gamma+1)) / (1 - alpha);
    the number accepted follows P(n=j) = alpha^j (1-alpha), P(n=gamma) =
    alpha^gamma.  Drafts are planted at rate alpha (the handbook's simulated
    acceptance) on random rows; the oracle verifies them."""
    a, K = case["alpha"], case["gamma"]
    tau = (1 - a ** (K + 1)) / (1 - a)
    assert tau == pytest.approx(case["tau"], abs=1e-4)
    B, V = 200_000, 16
    rng = np.random.default_rng(int(a * 100) + K)
    logits = rng.standard_normal((B, K + 1, V)).astype(np.float32)
    top = np.argmax(logits[:, :K, :], axis=-1)
    draft = W.planted_acceptance_drafts(top, V, a, seed=int(a * 1000) + K)
    out = orc.verify_greedy(logits, draft)
    n = out["accepted"].astype(np.float64)
    mean, se = (n + 1).mean(), (n + 1).std(ddof=1) / np.sqrt(B)
    assert abs(mean - tau) < 4 * se
    counts = np.bincount(out["accepted"], minlength=K + 1)
    expected = np.array([a ** j * (1 - a) for j in range(K)] + [a ** K]) * B
    assert stats.chisquare(counts, expected).pvalue > 1e-3


def test_metric_identity(orc):
    """vLLM features 03, results 1 and 4: tokens per step = 1 + sum of the
    per-position acceptance fractions (84.2/79.4/77.0/74.7% -> 4.15;
    7.7 of 8 -> 8.7).  The oracle's outputs obey the same identity."""
    g = golden("metric_identities.json")
    assert 1 + sum(g["per_position_acceptance_k4"]) == pytest.approx(g["tokens_per_step_k4"], abs=5e-3)
    assert 1 + g["accepted_of_8_k8"] == pytest.approx(g["tokens_per_step_k8"])
    gw = W.greedy_workload(2000, 4, 64, "f32", 1.0, (0.8,), seed=5)
    out = orc.verify_greedy(gw["logits"], gw["drafts"][0.8])
    n = out["accepted"]
    per_pos = np.array([(n > i).mean() for i in range(4)])
    settled = (out["emitted"] >= 0).sum(axis=1)
    assert np.array_equal(settled, n + 1)
    assert settled.mean() == pytest.approx(1 + per_pos.sum())


def _toy_target(V=64, table_rows=97, seed=11):
    """A deterministic 'target model': the next-token logits are a fixed
    function of the last three tokens (bf16-rounded, so ties occur)."""
    rng = np.random.default_rng(seed)
    table = W.f32_to_bf16_bits(rng.standard_normal((table_rows, V)).astype(np.float32) * 2)

    def logits(ctx):
        a, b, c = ctx[-3:]
        return table[(a * 4099 + b * 131 + c * 7) % table_rows]
    return logits


def _plain_greedy(target, prompt, n_new):
    ctx = list(prompt)
    for _ in range(n_new):
        ctx.append(int(np.argmax(W.bf16_bits_to_f32(target(ctx)))))
    return ctx


def _speculative(orc, target, prompt, n_new, K, proposer):
    ctx = list(prompt)
    steps = 0
    while len(ctx) < len(prompt) + n_new:
        draft, dlen = proposer(ctx, K)
        rows = []
        for i in range(K + 1):
            rows.append(target(ctx + [int(t) for t in draft[:min(i, dlen)]]))
        out = orc.verify_greedy(np.stack(rows)[None], np.array([draft], np.int32),
                                draft_len=np.array([dlen], np.int32))
        n = int(out["accepted"][0])
        ctx.extend(int(t) for t in out["emitted"][0][:n + 1])
        steps += 1
    return ctx[:len(prompt) + n_new], steps


@pytest.mark.parametrize("K", [2, 4, 8])
def test_greedy_identity_ngram_proposer(orc, K):
    """Handbook 'why' / vLLM features 03 '1. principle': with greedy decoding
    the speculative output equals what the target alone produces.  Proposer:
    the oracle's n-gram lookup (n = 5..2), which often proposes nothing."""
    target = _toy_target()
    prompt = [5, 9, 17, 33, 5, 9]
    ref = _plain_greedy(target, prompt, 512)

    def ngram(ctx, K):
        o = orc.ngram_propose(np.array([ctx], np.int32), np.array([len(ctx)], np.int32), 2, 5, K)
        return o["proposal"][0], int(o["proposal_len"][0])
    got, steps = _speculative(orc, target, prompt, 512, K, ngram)
    assert got == ref
    assert steps < 512          # lookups do hit on this repetitive target


@pytest.mark.parametrize("alpha", [0.3, 0.9])
def test_greedy_identity_planted_proposer(orc, alpha):
    """Same identity with a proposer that is right with probability alpha."""
    target = _toy_target(seed=12)
    prompt = [1, 2, 3]
    ref = _plain_greedy(target, prompt, 512)
    rng = np.random.default_rng(int(alpha * 10))

    def planted(ctx, K):
        d = []
        for _ in range(K):
            true = int(np.argmax(W.bf16_bits_to_f32(target(ctx + d))))
            d.append(true if rng.random() < alpha else (true + 1 + int(rng.integers(0, 63))) % 64)
        return np.array(d, np.int32), K
    got, steps = _speculative(orc, target, prompt, 512, 4, planted)
    assert got == ref


def test_draft_len_and_flags(orc):
    """Variable-length drafts (no match -> no draft, vLLM features 03 '3-1'):
    draft_len 0 emits only the target's token; out-of-range lengths are
    clamped and flagged; out-of-range ids never match and are flagged."""
    V, K = 40, 3
    ids = [4, 8, 15, 16]
    logits = np.stack([_rows_with_argmax(V, ids, seed=s) for s in range(5)])
    draft = np.array([ids[:3]] * 5, np.int32)
    draft[4, 1] = V + 7                    # id out of range at position 1
    dl = np.array([0, 2, 5, -1, 3], np.int32)
    out = orc.verify_greedy(logits, draft, draft_len=dl)
    assert out["accepted"].tolist() == [0, 2, 3, 0, 1]
    assert out["emitted"][0].tolist() == [4, -1, -1, -1]
    assert out["emitted"][1].tolist() == [4, 8, 15, -1]
    assert out["emitted"][2].tolist() == [4, 8, 15, 16]
    assert out["flags"].tolist() == [0, 0, orc.FLAG_BAD_LEN, orc.FLAG_BAD_LEN, orc.FLAG_DRAFT_OOR]
    assert out["argmax"][0].tolist() == [4, -1, -1, -1]
