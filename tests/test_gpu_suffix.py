"""GPU parity: suffix-decoding proposals against the oracle, bit-exact
(proposal, proposal_len, score, match_len, source, flags)."""
import numpy as np
import pytest
import torch

import proposal_sv_verify_amd as sv
from proposal_sv_verify_amd import workloads as W
from gpu_util import host, say, to_dev

pytestmark = pytest.mark.gpu


def _case(orc, tokens, lengths, history, m_min, m_max, K, min_prob, label=""):
    say("suffix", label, tokens.shape, None if history is None else history.shape, m_min, m_max, K,
        min_prob)
    g = sv.suffix_propose(to_dev(tokens), to_dev(lengths),
                          None if history is None else to_dev(history), m_min, m_max, K, min_prob)
    r = orc.suffix_propose(tokens, lengths, history, m_min, m_max, K, min_prob)
    for k in ("proposal", "proposal_len", "match_len", "source"):
        np.testing.assert_array_equal(host(g[k]), r[k], err_msg="%s %s" % (label, k))
    np.testing.assert_array_equal(host(g["score"]), r["score"], err_msg="%s score" % label)
    np.testing.assert_array_equal(host(g["flags"]).astype(np.uint32), r["flags"])
    return r


def test_suffix_workload_full_size(orc):
    """64 contexts of 8192 tokens with planted copies, a 262144-token history
    of documents copying spans of them; patterns up to 32, K 16."""
    c = W.SUFFIX
    wl = W.suffix_workload(c["B"], c["L"], c["H"], seed=W.seed_for(2, salt=7))
    r = _case(orc, wl["tokens"], wl["lengths"], wl["history"], c["m_min"], c["m_max"], c["K"],
              c["min_prob"], "full size")
    assert (r["source"] == 1).any() and (r["source"] == 0).any()


@pytest.mark.parametrize("m_min,m_max,K,min_prob", [(1, 4, 8, 0.0), (2, 32, 32, 0.3), (3, 7, 1, 1.0),
                                                    (1, 32, 5, 0.5)])
def test_suffix_small_alphabets(orc, m_min, m_max, K, min_prob):
    """Small vocabularies (many occurrences, frequent ties and capped
    occurrence lists), ragged lengths including 0, 1 and bad ones, strides
    that are not multiples of 4, histories with separators."""
    rng = np.random.default_rng(m_max * 7 + K)
    for trial, (B, stride, H, V) in enumerate([(7, 37, 0, 3), (16, 300, 1001, 4), (5, 20000, 40000, 6),
                                               (33, 1024, 5, 2), (9, 17000, 70001, 50)]):
        tok = rng.integers(0, V, size=(B, stride)).astype(np.int32)
        lens = rng.integers(0, stride + 1, size=B).astype(np.int32)
        lens[0] = stride
        if B > 3:
            lens[1], lens[2], lens[3] = 0, 1, stride + 5       # the last one is flagged
        hist = None
        if H:
            hist = rng.integers(-1, V, size=H).astype(np.int32)
        _case(orc, tok, lens, hist, m_min, m_max, K, min_prob, "trial %d" % trial)


def test_suffix_long_repeats_and_cap(orc):
    """A periodic context (every end is a full-length match: the cap of
    most recent occurrences and the early stop decide), a history made of
    the same period, and contexts whose suffix appears only in history."""
    per = np.array([11, 12, 13, 14, 15, 16, 17], np.int32)
    B, L = 4, 9000
    tok = np.tile(per, (B, L // len(per) + 1))[:, :L].copy()
    tok[2] = np.arange(L, dtype=np.int32) + 1000                     # no repeat in the context
    tok[3] = np.arange(L, dtype=np.int32) + 1000
    tok[3, -5:] = [21, 22, 23, 24, 25]
    hist = np.concatenate([np.tile(per, 5000), [-1], [21, 22, 23, 24, 25, 26, 27], [-1],
                           np.arange(2000, dtype=np.int32) + 1000, [-1, 21, 22, 23, 24, 25, 26, 28]])
    hist = hist.astype(np.int32)
    lens = np.full(B, L, np.int32)
    r = _case(orc, tok, lens, hist, 1, 32, 16, 0.0, "periodic")
    assert r["source"].tolist()[3] == 1
    _case(orc, tok, lens, hist, 1, 32, 16, 0.6, "periodic p0.6")
    _case(orc, tok, lens, None, 2, 5, 3, 0.0, "periodic no history")


def test_suffix_unaligned_views(orc):
    """Token rows and history taken as views at odd offsets (the 4-byte
    loads path)."""
    wl = W.suffix_workload(6, 3001, 20003, seed=99)
    big = np.zeros((7, 3003), np.int32)              # a spare row: rows read up to their stride
    big[:6, 1:3002] = wl["tokens"]
    t = to_dev(big)[:6, 1:3002]
    hbig = np.zeros(20004, np.int32)
    hbig[1:] = wl["history"]
    h = to_dev(hbig)[1:]
    say("suffix unaligned views")
    g = sv.suffix_propose(t, to_dev(wl["lengths"]), h, 1, 32, 12, 0.2)
    r = orc.suffix_propose(wl["tokens"], wl["lengths"], wl["history"], 1, 32, 12, 0.2)
    for k in ("proposal", "proposal_len", "match_len", "source", "score"):
        np.testing.assert_array_equal(host(g[k]), r[k], err_msg=k)


@pytest.mark.parametrize("n7,n3,want", [(40, 40, 3), (41, 39, 7)])
def test_suffix_counts_on_a_sorted_step(orc, n7, n3, want):
    """More than 64 occurrences continue the first step (the step sorts
    their tokens across the wave): the pattern is followed n7 times by
    token 7 and n3 times by token 3 in the history.  Equal counts go to
    the lower id; one more occurrence decides otherwise."""
    rng = np.random.default_rng(5)
    ctx = rng.integers(1000, 2000, size=300).astype(np.int32)
    ctx[-2:] = [500, 501]
    docs = []
    for t in rng.permutation([7] * n7 + [3] * n3):
        docs += list(rng.integers(2000, 3000, size=int(rng.integers(3, 9)))) + [500, 501, int(t)]
        docs += list(rng.integers(2000, 3000, size=3)) + [-1]
    hist = np.array(docs, np.int32)
    r = _case(orc, ctx[None, :], np.array([300], np.int32), hist, 1, 8, 4, 0.1,
              "counts %d/%d" % (n7, n3))
    assert r["source"][0] == 1 and r["proposal"][0, 0] == want
