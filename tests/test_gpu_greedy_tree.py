"""GPU parity: greedy and tree verification against the oracle, bit-exact
(accepted counts, emitted tokens, argmaxes, tree paths, flags)."""
import numpy as np
import pytest
import torch

import proposal_sv_verify_amd as sv
from proposal_sv_verify_amd import workloads as W
from gpu_util import dev, host, say, to_dev

pytestmark = pytest.mark.gpu


def _greedy_case(orc, logits, draft, draft_len=None, label=""):
    say("greedy", label, logits.shape, logits.dtype)
    t = to_dev(logits)
    d = to_dev(draft)
    dl = to_dev(draft_len) if draft_len is not None else None
    stats = torch.zeros(3 + draft.shape[1], dtype=torch.int64, device=dev())
    g = sv.verify_greedy(t, d, dl, stats=stats)
    r = orc.verify_greedy(logits, draft, draft_len)
    for k in ("accepted", "emitted", "argmax"):
        np.testing.assert_array_equal(host(g[k]), r[k], err_msg="%s %s" % (label, k))
    np.testing.assert_array_equal(host(g["flags"]).astype(np.uint32), r["flags"])
    n = r["accepted"].astype(np.int64)
    K = draft.shape[1]
    lens = np.clip(draft_len, 0, K) if draft_len is not None else np.full(len(n), K)
    want = [n.sum(), lens.sum(), (n + 1).sum()] + [(n > i).sum() for i in range(K)]
    np.testing.assert_array_equal(host(stats), np.array(want, np.int64))
    return g, r


def test_greedy_small_workload(orc):
    """fp32 logits N(0,1), B=4, K=4, V=32000, planted acceptance 0.7."""
    wl = W.greedy_workload(**W.GREEDY_SMALL, seed=W.seed_for(1))
    _greedy_case(orc, wl["logits"], wl["drafts"][0.7], label="B4K4V32000")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_greedy_ragged_shapes_and_ties(orc, dtype):
    rng = np.random.default_rng(5)
    for trial, V in enumerate([1, 2, 7, 8, 9, 63, 64, 65, 1000, 4097, 33333]):
        for K in (0, 1, 7):
            B = int(rng.integers(1, 18))
            wl = W.greedy_workload(B, K, V, dtype, 2.0, (0.6,), seed=100 * trial + K)
            logits = wl["logits"]
            if V > 3:                     # plant duplicate maxima in some rows
                wide = W.bf16_bits_to_f32(logits) if dtype == "bf16" else logits
                for b in range(B):
                    for i in range(K + 1):
                        if rng.random() < 0.5:
                            j = rng.choice(V, size=3, replace=False)
                            m = logits[b, i, np.argmax(wide[b, i])]
                            logits[b, i, j] = m
                top = np.argmax(W.bf16_bits_to_f32(logits) if dtype == "bf16" else logits,
                                axis=-1)[:, :K]
                draft = W.planted_acceptance_drafts(top, V, 0.7, seed=trial)
            else:
                draft = wl["drafts"][0.6]
            dl = rng.integers(-1, K + 2, size=B).astype(np.int32) if trial % 2 else None
            if K > 0 and trial % 3 == 0:
                draft[0, 0] = V + 5        # out-of-range id: flagged, never matches
            _greedy_case(orc, logits, draft, dl, label="V%d K%d B%d" % (V, K, B))


def test_greedy_split_rows_and_padded_stride(orc):
    """Rows cut into many segments (merged by the per-sequence kernel) and a row
    stride larger than V."""
    sv.set_tuning(sv.TUNE_MIN_SEGMENT_BYTES, 1024)
    try:
        for dtype in ("f32", "bf16"):
            wl = W.greedy_workload(5, 6, 20011, dtype, 2.0, (0.5,), seed=77)
            _greedy_case(orc, wl["logits"], wl["drafts"][0.5], label="split " + dtype)
            big = np.zeros((5, 7, 20011 + 13), wl["logits"].dtype)
            big[:, :, :20011] = wl["logits"]
            say("greedy padded stride", dtype)
            t = to_dev(big)[:, :, :20011]
            g = sv.verify_greedy(t, to_dev(wl["drafts"][0.5]))
            r = orc.verify_greedy(wl["logits"], wl["drafts"][0.5])
            np.testing.assert_array_equal(host(g["emitted"]), r["emitted"])
            np.testing.assert_array_equal(host(g["argmax"]), r["argmax"])
    finally:
        sv.set_tuning(sv.TUNE_MIN_SEGMENT_BYTES, 0)


def test_greedy_negative_zero_and_constant_rows(orc):
    V = 300
    rows = np.zeros((2, 3, V), np.uint16)
    rows[0, 0, :] = 0x8000                # -0.0 everywhere -> id 0
    rows[0, 1, 150:] = 0x8000             # +0 then -0: all equal -> id 0
    rows[0, 2, :] = 0xC000                # -2.0 everywhere
    rows[1, 0, :] = 0x8000
    rows[1, 0, 299] = 0x0000              # -0 .. +0: equal -> id 0
    rows[1, 1, 7] = 0x3F80                # a single 1.0
    rows[1, 2, :] = 0xFF7F                # the most negative finite bf16
    draft = np.array([[0, 0], [0, 7]], np.int32)
    _greedy_case(orc, rows, draft, label="signed zeros")


def test_greedy_full_size_three_alphas(orc):
    """bf16 N(0,2), B=256, K=8, V=151936, planted alpha 0.3 / 0.6 / 0.9."""
    wl = W.greedy_workload(**W.GREEDY_LARGE, seed=W.seed_for(4))
    t = to_dev(wl["logits"])
    for a in W.GREEDY_LARGE["alphas"]:
        say("greedy full size alpha", a)
        g = sv.verify_greedy(t, to_dev(wl["drafts"][a]))
        r = orc.verify_greedy(wl["logits"], wl["drafts"][a])
        for k in ("accepted", "emitted", "argmax"):
            np.testing.assert_array_equal(host(g[k]), r[k], err_msg="alpha %s %s" % (a, k))
        tau = (1 - a ** 9) / (1 - a)
        assert abs(r["accepted"].mean() + 1 - tau) < 0.6


def _plant_ties(logits, dtype, rng, frac=0.5):
    """Copy each chosen row's maximum to 3 more random ids (lowest id wins)."""
    B, R, V = logits.shape
    wide = W.bf16_bits_to_f32(logits) if dtype == "bf16" else logits
    for b in range(B):
        for i in range(R):
            if rng.random() < frac:
                j = rng.choice(V, size=3, replace=False)
                logits[b, i, j] = logits[b, i, np.argmax(wide[b, i])]


@pytest.mark.parametrize("B,K,V,dtype", [
    (256, 8, 32000, "bf16"),
    (512, 3, 4096, "bf16"),
    (256, 15, 8200, "f32"),
    (256, 0, 5000, "f32"),       # the bonus row alone
    (256, 6, 800, "bf16"),       # short rows, many of them
    (256, 16, 4096, "bf16"),
    (256, 8, 32001, "bf16"),     # V not a whole number of 16-byte vectors
    (240, 8, 32000, "bf16"),
])
def test_greedy_large_batches(orc, B, K, V, dtype):
    """Batches of 240-512 sequences, bit-exact: planted ties between ids far
    apart in a row, the statistics counters and the out-of-range draft
    flag."""
    rng = np.random.default_rng(B + K + V)
    wl = W.greedy_workload(B, K, V, dtype, 2.0, (0.6,), seed=B * 1000 + K)
    logits = wl["logits"]
    _plant_ties(logits, dtype, rng)
    top = np.argmax(W.bf16_bits_to_f32(logits) if dtype == "bf16" else logits, axis=-1)[:, :K]
    draft = W.planted_acceptance_drafts(top, V, 0.7, seed=K)
    if K > 0:
        draft[3, 0] = -2                  # flagged, never matches
    _greedy_case(orc, logits, draft, label="B%d K%d V%d %s" % (B, K, V, dtype))


def test_greedy_repeat_is_bit_identical(orc):
    """Same inputs, same (reused) workspace: identical outputs every time."""
    wl = W.greedy_workload(64, 8, 50000, "bf16", 2.0, (0.6,), seed=9)
    t, d = to_dev(wl["logits"]), to_dev(wl["drafts"][0.6])
    say("greedy repeat")
    first = {k: host(v) for k, v in sv.verify_greedy(t, d).items()}
    for _ in range(5):
        again = sv.verify_greedy(t, d)
        for k in first:
            np.testing.assert_array_equal(host(again[k]), first[k])


def _tree_case(orc, wl, parent=None, token=None, label=""):
    parent = wl["parent"] if parent is None else parent
    token = wl["token"] if token is None else token
    say("tree", label, wl["logits"].shape)
    g = sv.verify_tree(to_dev(wl["logits"]), to_dev(parent), to_dev(token))
    r = orc.verify_tree(wl["logits"], parent, token)
    for k in ("accepted", "path", "emitted", "argmax"):
        np.testing.assert_array_equal(host(g[k]), r[k], err_msg="%s %s" % (label, k))
    np.testing.assert_array_equal(host(g["flags"]).astype(np.uint32), r["flags"])


def test_tree_full_size(orc):
    """bf16 N(0,2), B=32, 64-node trees (depth <= 6, branching <= 4), V=128256."""
    wl = W.tree_workload(**W.TREE, seed=W.seed_for(5))
    _tree_case(orc, wl, label="B32N64V128256")


def test_tree_random_and_malformed(orc):
    rng = np.random.default_rng(12)
    for trial in range(12):
        B = int(rng.integers(1, 9))
        N = int(rng.integers(1, 80))
        V = int(rng.integers(5, 3000))
        dtype = "bf16" if trial % 2 else "f32"
        wl = W.tree_workload(B, N, V, 2.0, 0.8, 6, 4, seed=500 + trial, dtype=dtype)
        parent, token = wl["parent"].copy(), wl["token"].copy()
        if N > 3:
            parent[0, N - 1] = N + 1
            parent[B - 1, 0] = 3
            token[0, 1] = -2
            for b in range(B):            # equal-depth ties: duplicate sibling tokens
                kids = np.nonzero(parent[b] == 0)[0]
                if len(kids) > 1:
                    token[b, kids[1]] = token[b, kids[0]]
        _tree_case(orc, wl, parent, token, label="trial %d N%d V%d" % (trial, N, V))


def test_tree_large_node_count(orc):
    wl = W.tree_workload(2, 1024, 700, 2.0, 0.9, 40, 2, seed=3)
    _tree_case(orc, wl, label="N1024")
