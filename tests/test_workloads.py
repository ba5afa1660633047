"""Input generators: determinism, distributions and planting (CPU)."""
import numpy as np
import pytest
import torch
from scipy import stats

from proposal_sv_verify_amd import workloads as W


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(100_000).astype(np.float32) * 3,
                        np.array([0.0, -0.0, 1e-30, -1e-30, 3.0e38, 1.00390625, 1.01171875], np.float32)])
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(W.bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generators_are_deterministic():
    a = W.greedy_workload(3, 4, 500, "bf16", 2.0, (0.3, 0.9), seed=5)
    b = W.greedy_workload(3, 4, 500, "bf16", 2.0, (0.3, 0.9), seed=5)
    assert np.array_equal(a["logits"], b["logits"])
    assert all(np.array_equal(a["drafts"][k], b["drafts"][k]) for k in a["drafts"])
    r1 = W.rejection_workload(2, 3, 300, seed=6)
    r2 = W.rejection_workload(2, 3, 300, seed=6)
    for k in ("target", "draft_logits", "draft", "uniforms"):
        assert np.array_equal(r1[k], r2[k])
    n1 = W.ngram_workload(4, 2048, seed=7)
    n2 = W.ngram_workload(4, 2048, seed=7)
    assert np.array_equal(n1["tokens"], n2["tokens"])
    t1 = W.tree_workload(2, 20, 100, seed=8)
    t2 = W.tree_workload(2, 20, 100, seed=8)
    assert np.array_equal(t1["parent"], t2["parent"]) and np.array_equal(t1["token"], t2["token"])


def test_philox_uniforms_are_uniform():
    u = W.philox_uniforms((200_000,), seed=9)
    assert u.dtype == np.float32 and u.min() >= 0.0 and u.max() < 1.0
    assert stats.kstest(u.astype(np.float64), "uniform").pvalue > 1e-3


def test_planted_acceptance_rate():
    top = np.zeros((100_000,), np.int64) + 3
    d = W.planted_acceptance_drafts(top, 10, 0.6, seed=10)
    hit = (d == 3).mean()
    assert abs(hit - 0.6) < 4 * np.sqrt(0.24 / 1e5)
    assert d.min() >= 0 and d.max() < 10


def test_gumbel_max_draws_follow_softmax():
    rng = np.random.Generator(np.random.PCG64(11))
    logits = np.array([[0.0, 1.0, -0.5, 2.0]], np.float32)
    rows = np.repeat(logits, 100_000, axis=0)
    x = W.gumbel_max_sample(rows, 1.0, rng)
    p = np.exp(logits[0].astype(np.float64))
    p /= p.sum()
    assert stats.chisquare(np.bincount(x, minlength=4), p * len(x)).pvalue > 1e-3


def test_tree_shape_limits():
    t = W.tree_workload(4, 64, 1000, seed=12)
    for par in t["parent"]:
        assert par[0] == -1 and all(0 <= par[j] < j for j in range(1, 64))
        depth = np.zeros(64, int)
        for j in range(1, 64):
            depth[j] = depth[par[j]] + 1
        assert depth.max() <= 6
        assert np.bincount(par[1:], minlength=64).max() <= 4
    # children of one node carry distinct ids
    for b in range(4):
        for i in range(64):
            kids = np.nonzero(t["parent"][b] == i)[0]
            assert len(set(t["token"][b, kids].tolist())) == len(kids)


def test_ngram_spans_and_zipf():
    wl = W.ngram_workload(8, 8192, seed=13)
    toks = wl["tokens"]
    assert toks.min() >= 0 and toks.max() < 151936
    # rank-1 token frequency close to the truncated Zipf(1.1) mass (~13%)
    h = (np.arange(1, 151937, dtype=np.float64) ** -1.1).sum()
    assert abs((toks == 0).mean() - 1 / h) < 0.02
