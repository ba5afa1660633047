"""GPU parity at the limits the header states: the largest vocabulary, the
most drafts, the longest proposals, vocabularies past the selection's
staging size.  Bit-exact against the oracle (rejection: up to flagged
ties)."""
import numpy as np
import pytest
import torch

import proposal_sv_verify_amd as sv
from proposal_sv_verify_amd import workloads as W
from gpu_util import check_rejection, dev, host, say, to_dev

pytestmark = pytest.mark.gpu

SV_MAX_V = 1 << 30
SV_MAX_DRAFTS = 4096
SV_MAX_PROPOSAL = 4096


def test_greedy_largest_vocabulary(orc):
    """One sequence, K 1, V = SV_MAX_V - 3 (2 GiB per bf16 row): row 0's
    maximum sits at the last id, row 1 has the same maximum at two ids far
    apart (the lower one wins)."""
    V = SV_MAX_V - 3
    rng = np.random.default_rng(17)
    say("greedy largest vocabulary V", V)
    lg = rng.integers(0x3000, 0x3f80, size=(1, 2, V), dtype=np.uint16)    # bf16 in [2^-31, 1)
    lg[0, 0, V - 1] = 0x4000                                             # 2.0
    lg[0, 1, 123456789] = 0x4040                                         # 3.0 ...
    lg[0, 1, V - 7] = 0x4040                                             # ... twice
    draft = np.array([[V - 1]], np.int32)
    g = sv.verify_greedy(to_dev(lg), to_dev(draft))
    r = orc.verify_greedy(lg, draft)
    for k in ("accepted", "emitted", "argmax"):
        np.testing.assert_array_equal(host(g[k]), r[k], err_msg=k)
    assert r["argmax"].tolist() == [[V - 1, 123456789]] and r["accepted"][0] == 1
    del g
    torch.cuda.empty_cache()


def test_greedy_and_rejection_most_drafts(orc):
    """K = SV_MAX_DRAFTS with a small vocabulary and ragged draft lengths."""
    B, K, V = 3, SV_MAX_DRAFTS, 64
    wl = W.greedy_workload(B, K, V, dtype="f32", sigma=2.0, alphas=(0.999,), seed=21)
    dl = np.array([K, 17, 4000], np.int32)
    say("greedy most drafts K", K)
    g = sv.verify_greedy(to_dev(wl["logits"]), to_dev(wl["drafts"][0.999]), to_dev(dl))
    r = orc.verify_greedy(wl["logits"], wl["drafts"][0.999], dl)
    for k in ("accepted", "emitted", "argmax"):
        np.testing.assert_array_equal(host(g[k]), r[k], err_msg=k)
    rw = W.rejection_workload(2, K, 8, 0.3, 1e-4, 1.0, seed=22, dtype="f32")   # q close to p: long runs
    say("rejection most drafts K", K)
    g = sv.verify_rejection(to_dev(rw["target"]), to_dev(rw["draft_logits"]), to_dev(rw["draft"]),
                            to_dev(rw["uniforms"]), 1.0)
    r = orc.verify_rejection(rw["target"], rw["draft_logits"], rw["draft"], rw["uniforms"], 1.0)
    check_rejection(g, r, "K4096", max_flagged=1)


def test_rejection_vocabulary_past_selection_staging(orc):
    """V = 3,000,001: more sub-chunk masses than the selection stages in
    LDS (2048 sub-chunks of 1024), so it reads them from memory."""
    wl = W.rejection_workload(3, 2, 3000001, 2.0, 0.5, 1.0, seed=23, dtype="bf16")
    say("rejection V 3000001")
    g = sv.verify_rejection(to_dev(wl["target"]), to_dev(wl["draft_logits"]), to_dev(wl["draft"]),
                            to_dev(wl["uniforms"]), 1.0)
    r = orc.verify_rejection(wl["target"], wl["draft_logits"], wl["draft"], wl["uniforms"], 1.0)
    check_rejection(g, r, "V3000001", max_flagged=1)


def test_ngram_longest_proposal(orc):
    """K = SV_MAX_PROPOSAL and n_max = SV_MAX_NGRAM on long periodic and
    planted contexts: proposals run to the end of the context or to K."""
    rng = np.random.default_rng(24)
    L = 100000
    per = rng.integers(0, 1000, size=5003).astype(np.int32)
    tok = np.stack([np.tile(per, L // len(per) + 1)[:L],
                    W.ngram_workload(1, L, seed=25)["tokens"][0]]).astype(np.int32)
    lens = np.array([L, L - 1], np.int32)
    say("ngram longest proposal K", SV_MAX_PROPOSAL)
    g = sv.ngram_propose(to_dev(tok), to_dev(lens), 1, 31, SV_MAX_PROPOSAL)
    r = orc.ngram_propose(tok, lens, 1, 31, SV_MAX_PROPOSAL)
    for k in ("proposal", "proposal_len", "match_n", "match_pos"):
        np.testing.assert_array_equal(host(g[k]), r[k], err_msg=k)
    assert r["proposal_len"][0] == SV_MAX_PROPOSAL
