"""GPU parity: rejection sampling on given probabilities
(sv_verify_rejection_probs) against the oracle's probability mode:
decisions identical except oracle-flagged ties, p_i(x_i) and q_i(x_i)
within 1e-5 relative."""
import numpy as np
import pytest
import torch

import proposal_sv_verify_amd as sv
from proposal_sv_verify_amd import workloads as W
from gpu_util import check_rejection, dev, host, say, to_dev

pytestmark = pytest.mark.gpu


def _softmax32(logits):
    x = np.asarray(logits, np.float64)
    x = np.exp(x - x.max(axis=-1, keepdims=True))
    return (x / x.sum(axis=-1, keepdims=True)).astype(np.float32)


def _case(orc, P, Q, draft, u, draft_len=None, label=""):
    say("rejection probs", label, P.shape)
    K = P.shape[1] - 1
    stats = torch.zeros(3 + K, dtype=torch.int64, device=dev())
    g = sv.verify_rejection_probs(to_dev(P), to_dev(Q), to_dev(draft), to_dev(u),
                                  to_dev(draft_len) if draft_len is not None else None, stats=stats)
    r = orc.verify_rejection(P, Q, draft, u, 1.0, draft_len, probs=True)
    check_rejection(g, r, label)
    np.testing.assert_array_equal(host(g["flags"]).astype(np.uint32), r["flags"])
    acc = host(g["accepted"]).astype(np.int64)
    assert host(stats)[0] == acc.sum()
    return r


def test_probs_dirichlet_v8_with_zeros(orc):
    """4096 sequences, K 3, V 8: Dirichlet rows with zero entries on both
    sides (drafts where q = 0 are accepted outright), rows not normalised."""
    rng = np.random.default_rng(41)
    B, K, V = 4096, 3, 8
    P = rng.dirichlet(np.ones(V), size=(B, K + 1)).astype(np.float32)
    Q = rng.dirichlet(np.ones(V), size=(B, K)).astype(np.float32)
    P[rng.random(P.shape) < 0.15] = 0.0
    Q[rng.random(Q.shape) < 0.15] = 0.0
    P[..., 0] += np.float32(1e-3)                  # every row keeps some mass
    Q[..., 1] += np.float32(1e-3)
    P *= np.float32(3.0)
    x = rng.integers(0, V, size=(B, K)).astype(np.int32)
    u = rng.random((B, K + 1), dtype=np.float32)
    dl = rng.integers(-1, K + 2, size=B).astype(np.int32)
    _case(orc, P, Q, x, u, None, "V8")
    _case(orc, P, Q, x, u, dl, "V8 ragged")


def test_probs_full_vocabulary(orc):
    """The rejection workload's logits turned into fp32 probabilities
    (V 128256, B 16, K 5), drafts sampled from the draft distribution."""
    wl = W.rejection_workload(16, 5, 128256, 2.0, 0.5, 1.0, seed=42, dtype="f32")
    P = _softmax32(wl["target"])
    Q = _softmax32(wl["draft_logits"])
    _case(orc, P, Q, wl["draft"], wl["uniforms"], None, "V128256")


def test_probs_one_hot_and_bonus_only(orc):
    """One-hot targets reduce to greedy decisions; K = 0 samples the bonus
    from p alone."""
    rng = np.random.default_rng(43)
    B, K, V = 64, 4, 3000
    P = np.zeros((B, K + 1, V), np.float32)
    top = rng.integers(0, V, size=(B, K + 1))
    P[np.arange(B)[:, None], np.arange(K + 1)[None, :], top] = 1.0
    Q = rng.random((B, K, V)).astype(np.float32)
    x = np.where(rng.random((B, K)) < 0.7, top[:, :K], rng.integers(0, V, size=(B, K))).astype(np.int32)
    u = rng.random((B, K + 1), dtype=np.float32)
    r = _case(orc, P, Q, x, u, None, "one-hot")
    greedy_n = np.array([next((i for i in range(K) if x[b, i] != top[b, i]), K) for b in range(B)])
    np.testing.assert_array_equal(r["accepted"], greedy_n)
    P0 = rng.random((B, 1, V)).astype(np.float32)
    _case(orc, P0, np.zeros((B, 0, V), np.float32), np.zeros((B, 0), np.int32),
          rng.random((B, 1), dtype=np.float32), None, "K0")
