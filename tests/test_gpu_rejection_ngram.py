"""GPU parity: rejection sampling (decisions identical except oracle-flagged
ties; p_i(x_i), q_i(x_i) within 1e-5 relative) and the n-gram proposer
(bit-exact) against the oracle."""
import itertools

import numpy as np
import pytest
import torch

import proposal_sv_verify_amd as sv
from proposal_sv_verify_amd import workloads as W
from gpu_util import check_rejection, dev, host, say, to_dev

pytestmark = pytest.mark.gpu


def _rej_case(orc, wl, draft=None, draft_len=None, label="", max_flagged=None):
    draft = wl["draft"] if draft is None else draft
    say("rejection", label, wl["target"].shape)
    K = wl["target"].shape[1] - 1
    stats = torch.zeros(3 + K, dtype=torch.int64, device=dev())
    g = sv.verify_rejection(to_dev(wl["target"]), to_dev(wl["draft_logits"]), to_dev(draft),
                            to_dev(wl["uniforms"]), wl["temperature"],
                            to_dev(draft_len) if draft_len is not None else None, stats=stats)
    r = orc.verify_rejection(wl["target"], wl["draft_logits"], draft, wl["uniforms"],
                             wl["temperature"], draft_len)
    flagged, mism = check_rejection(g, r, label, max_flagged)
    np.testing.assert_array_equal(host(g["flags"]).astype(np.uint32), r["flags"])
    acc = host(g["accepted"]).astype(np.int64)
    assert host(stats)[0] == acc.sum() and host(stats)[2] == (acc + 1).sum()
    return flagged, mism


def test_rejection_full_size(orc):
    """bf16 target N(0,2), draft = target + N(0,0.5), B=64, K=5, V=128256,
    T=1, drafts sampled from the draft distribution, Philox uniforms."""
    wl = W.rejection_workload(**W.REJECTION, seed=W.seed_for(3))
    flagged, mism = _rej_case(orc, wl, label="B64K5V128256", max_flagged=4)
    say("rejection full size: flagged %d, mismatched %d of 64" % (flagged, mism))
    assert mism == 0


def test_rejection_full_size_more_seeds(orc):
    """Four more seeds of the full-size workload (256 sequences): every
    decision that differs from the oracle's lies in a flagged tie, and the
    flagged sequences stay few."""
    total_flag = total_mism = 0
    for salt in range(4):
        wl = W.rejection_workload(**W.REJECTION, seed=W.seed_for(3, salt=100 + salt))
        f, m = _rej_case(orc, wl, label="B64K5V128256 salt %d" % salt, max_flagged=6)
        total_flag += f
        total_mism += m
    say("rejection full size, 4 seeds: flagged %d, mismatched %d of 256" % (total_flag, total_mism))
    assert total_flag <= 12 and total_mism == 0


@pytest.mark.parametrize("T", [0.6, 1.0, 1.7])
def test_rejection_small_shapes_temperatures(orc, T):
    rng = np.random.default_rng(int(T * 10))
    total_flag = total_mism = 0
    for trial, V in enumerate([1, 2, 8, 9, 100, 4095, 4096, 4097, 9000]):
        for K in (0, 1, 4):
            B = int(rng.integers(1, 40))
            dtype = "bf16" if trial % 2 else "f32"
            wl = W.rejection_workload(B, K, V, 2.0, 0.7, T, seed=1000 * trial + K, dtype=dtype)
            dl = rng.integers(-1, K + 2, size=B).astype(np.int32) if trial % 3 == 1 else None
            draft = wl["draft"].copy()
            if K > 0 and trial % 4 == 2:
                draft[0, 0] = -7          # out of range: rejected, flagged
            f, m = _rej_case(orc, wl, draft, dl, label="T%.1f V%d K%d B%d" % (T, V, K, B))
            total_flag += f
            total_mism += m
    say("small shapes T %.1f: flagged %d, mismatched %d" % (T, total_flag, total_mism))


@pytest.mark.parametrize("dtype,T,top_k", [("bf16", 1.0, 50), ("f32", 0.7, 4000), ("bf16", 1.3, 1)])
def test_rejection_masked_logits(orc, dtype, T, top_k):
    """Top-k truncated rows: every entry outside a row's top_k is -inf in
    the target and draft logits (the two keep different sets, so drafts can
    have p = 0).  Masked entries carry probability 0 on both sides."""
    wl = W.rejection_workload(24, 4, 50000, 2.0, 0.7, T, seed=4242 + top_k, dtype=dtype, top_k=top_k)
    _rej_case(orc, wl, label="masked top%d %s T%.1f" % (top_k, dtype, T))
    sv.set_tuning(sv.TUNE_MIN_SEGMENT_BYTES, 2048)
    try:
        _rej_case(orc, wl, label="masked top%d %s T%.1f split" % (top_k, dtype, T))
    finally:
        sv.set_tuning(sv.TUNE_MIN_SEGMENT_BYTES, 0)


@pytest.mark.parametrize("case", ["shift+60", "shift-90", "outlier+70", "shift+20_T0.3"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rejection_extreme_logits(orc, case, dtype):
    """Logits far from 0: every row shifted up (terms above e^44 against a
    zero reference), shifted down (terms below e^-41), one large outlier
    per row, and a low temperature.  Softmax is shift-invariant, so the
    drafts sampled before the shift keep their distribution."""
    T = 0.3 if "T0.3" in case else 1.0
    seed = {"shift+60": 61, "shift-90": 62, "outlier+70": 63, "shift+20_T0.3": 64}[case]
    wl = W.rejection_workload(12, 3, 5000, 2.0, 0.5, T, seed=seed, dtype=dtype)
    widen = W.bf16_bits_to_f32 if dtype == "bf16" else (lambda a: a)
    narrow = W.f32_to_bf16_bits if dtype == "bf16" else (lambda a: a.astype(np.float32))
    t32, d32 = widen(wl["target"]).copy(), widen(wl["draft_logits"]).copy()
    if case.startswith("shift"):
        off = np.float32(float(case.split("_")[0][5:]))
        t32 += off
        d32 += off
    else:
        rng = np.random.default_rng(5)
        for a in (t32, d32):
            flat = a.reshape(-1, a.shape[-1])
            flat[np.arange(flat.shape[0]), rng.integers(0, flat.shape[1], flat.shape[0])] = 70.0
    wl = dict(wl, target=narrow(t32), draft_logits=narrow(d32))
    _rej_case(orc, wl, label="extreme %s %s" % (case, dtype))


@pytest.mark.parametrize("T", [0.05, 0.12, 8.0, 50.0])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rejection_extreme_temperatures(orc, T, dtype):
    """Temperatures far from 1: at T = 0.05 the terms of N(0, 2) logits
    reach e^±160, far outside fp32 against a zero reference (the careful
    path), and at large T the rows are nearly flat.  Drafts are sampled at
    the same temperature."""
    wl = W.rejection_workload(16, 4, 30011, 2.0, 0.5, T, seed=int(T * 1000) + (7 if dtype == "f32" else 0),
                              dtype=dtype)
    flagged, mism = _rej_case(orc, wl, label="T%g %s" % (T, dtype), max_flagged=2)
    assert mism == 0


@pytest.mark.parametrize("K", [63, 64, 130])
def test_rejection_long_drafts(orc, K):
    """Draft lengths at and past one 64-position block of the accept scan
    (which works in blocks of 64 positions), with and without per-sequence
    lengths."""
    wl = W.rejection_workload(4, K, 3000, 2.0, 0.15, 1.0, seed=700 + K, dtype="bf16")
    _rej_case(orc, wl, label="K%d" % K)
    dl = np.array([K, 0, K // 2, 65], np.int32)
    _rej_case(orc, wl, draft_len=dl, label="K%d ragged" % K)


def test_rejection_split_rows_and_repeat(orc):
    sv.set_tuning(sv.TUNE_MIN_SEGMENT_BYTES, 2048)
    try:
        wl = W.rejection_workload(6, 3, 50000, seed=31)
        _rej_case(orc, wl, label="split rows")
        t, d = to_dev(wl["target"]), to_dev(wl["draft_logits"])
        x, u = to_dev(wl["draft"]), to_dev(wl["uniforms"])
        first = {k: host(v) for k, v in sv.verify_rejection(t, d, x, u).items()}
        for _ in range(4):
            again = sv.verify_rejection(t, d, x, u)
            for k in first:
                np.testing.assert_array_equal(host(again[k]), first[k])
    finally:
        sv.set_tuning(sv.TUNE_MIN_SEGMENT_BYTES, 0)


def test_rejection_identical_draft_and_one_hot_target(orc):
    """q = p accepts every draft; a one-hot target turns rejection sampling
    into greedy verification (both paths agree with the oracle exactly)."""
    rng = np.random.default_rng(41)
    B, K, V = 16, 4, 3000
    tl = rng.standard_normal((B, K + 1, V)).astype(np.float32)
    wl = dict(target=tl, draft_logits=tl[:, :K].copy(),
              draft=rng.integers(0, V, (B, K)).astype(np.int32),
              uniforms=rng.random((B, K + 1), dtype=np.float32), temperature=1.0)
    _rej_case(orc, wl, label="q == p")
    g = sv.verify_rejection(to_dev(tl), to_dev(tl[:, :K].copy()), to_dev(wl["draft"]),
                            to_dev(wl["uniforms"]))
    assert (host(g["accepted"]) == K).all()
    t = rng.integers(0, V, (B, K + 1))
    oh = np.full((B, K + 1, V), -1.0e4, np.float32)
    np.put_along_axis(oh, t[..., None], 0.0, axis=-1)
    x = np.where(rng.random((B, K)) < 0.6, t[:, :K], rng.integers(0, V, (B, K))).astype(np.int32)
    wl2 = dict(target=oh, draft_logits=rng.standard_normal((B, K, V)).astype(np.float32),
               draft=x, uniforms=wl["uniforms"], temperature=1.0)
    _rej_case(orc, wl2, label="one-hot target")
    gr = orc.verify_greedy(oh, x)
    g2 = sv.verify_rejection(to_dev(oh), to_dev(wl2["draft_logits"]), to_dev(x),
                             to_dev(wl["uniforms"]))
    np.testing.assert_array_equal(host(g2["emitted"]), gr["emitted"])


# ------------------------------------------------------------------ n-gram

def _ngram_case(orc, tokens, lengths, n_min, n_max, K, label=""):
    say("ngram", label, tokens.shape, n_min, n_max, K)
    g = sv.ngram_propose(to_dev(tokens), to_dev(lengths), n_min, n_max, K)
    r = orc.ngram_propose(tokens, lengths, n_min, n_max, K)
    for k in ("proposal", "proposal_len", "match_n", "match_pos"):
        np.testing.assert_array_equal(host(g[k]), r[k], err_msg="%s %s" % (label, k))
    np.testing.assert_array_equal(host(g["flags"]).astype(np.uint32), r["flags"])
    return r


def test_ngram_workload(orc):
    """64 contexts of 8192 Zipf(1.1) ids with 8 planted copied spans each;
    n = 5..2, K = 8."""
    wl = W.ngram_workload(64, 8192, seed=W.seed_for(2))
    r = _ngram_case(orc, wl["tokens"], wl["lengths"], 2, 5, 8, "B64L8192")
    assert (r["match_n"][0::2] == 5).all()


def test_ngram_bandwidth_size_sampled(orc):
    """The same generator at 16384 contexts (512 MiB) in one call; the oracle
    checks every context."""
    wl = W.ngram_workload(16384, 8192, seed=W.seed_for(2, salt=1))
    _ngram_case(orc, wl["tokens"], wl["lengths"], 2, 5, 8, "B16384")


def test_ngram_many_contexts_ragged(orc):
    """The grouped kernel (16384 contexts and more, 32 per workgroup, tiles in
    groups of 16): a batch that leaves the last workgroup part-filled,
    ragged and invalid lengths, rows of 20 tiles (two groups, the second
    short), long planted repeats, Zipf ids from a small vocabulary so that
    matches of every length occur; element loads (stride % 4 != 0) and
    16-byte loads."""
    rng = np.random.default_rng(20261203)
    B, stride = 16384 + 37, 5003
    tokens = W.zipf_tokens(rng, (B, stride), 3000, 1.1).astype(np.int32)
    lengths = rng.integers(0, stride + 1, B).astype(np.int32)
    lengths[rng.random(B) < 0.3] = stride
    lengths[[5, 77, B - 1]] = [-1, stride + 1, -7]
    for b in range(0, B, 5):               # long repeats at every depth
        L = int(lengths[b])
        if L > 200:
            n = int(rng.integers(8, 40))
            s0 = int(rng.integers(0, L - n))
            tokens[b, L - n:L] = tokens[b, s0:s0 + n]
    for n_min, n_max, K in [(2, 5, 8), (1, 31, 16), (3, 3, 70)]:
        _ngram_case(orc, tokens, lengths, n_min, n_max, K, "many ragged n%d-%d" % (n_min, n_max))
    aligned = np.zeros((B, 5004), np.int32)
    aligned[:, :stride] = tokens
    _ngram_case(orc, aligned, np.clip(lengths, -1, 5004), 2, 5, 8, "many aligned")


def test_ngram_many_contexts_short_rows(orc):
    """The grouped kernel on rows of one tile and less: every context's only
    group, contexts too short for n_min, and the empty context."""
    rng = np.random.default_rng(7)
    B, stride = 20000, 200
    tokens = rng.integers(0, 6, (B, stride)).astype(np.int32)
    lengths = rng.integers(0, stride + 1, B).astype(np.int32)
    lengths[:64] = np.arange(64)
    for n_min, n_max, K in [(1, 4, 5), (4, 31, 3)]:
        _ngram_case(orc, tokens, lengths, n_min, n_max, K, "many short n%d-%d" % (n_min, n_max))
    # short contexts in long rows: the groups follow the lengths, not the stride
    B, stride = 16384, 4096
    tokens = rng.integers(0, 20, (B, stride)).astype(np.int32)
    lengths = rng.integers(0, 700, B).astype(np.int32)
    lengths[::997] = stride
    _ngram_case(orc, tokens, lengths, 2, 6, 4, "many short in long rows")


def test_full_size_calls_repeat_bit_identically():
    """Run-twice identity at full size, the launch shapes with the most
    workgroups and the LDS atomic combines: rejection sampling (2048
    final-sample workgroups; p and q compared as bits) and the grouped
    n-gram kernel (16384 contexts, group claims and key maxima in LDS)."""
    wl = W.rejection_workload(**W.REJECTION, seed=W.seed_for(3, salt=2))
    t, d = to_dev(wl["target"]), to_dev(wl["draft_logits"])
    x, u = to_dev(wl["draft"]), to_dev(wl["uniforms"])
    first = {k: host(v) for k, v in sv.verify_rejection(t, d, x, u).items()}
    for _ in range(2):
        again = sv.verify_rejection(t, d, x, u)
        for k in first:
            np.testing.assert_array_equal(host(again[k]).view(np.uint32) if first[k].dtype == np.float32
                                          else host(again[k]),
                                          first[k].view(np.uint32) if first[k].dtype == np.float32 else first[k],
                                          err_msg="rejection repeat %s" % k)
    ng = W.ngram_workload(16384, 8192, seed=W.seed_for(2, salt=4))
    tok, lens = to_dev(ng["tokens"]), to_dev(ng["lengths"])
    first = {k: host(v) for k, v in sv.ngram_propose(tok, lens, 2, 5, 8).items()}
    for _ in range(2):
        again = sv.ngram_propose(tok, lens, 2, 5, 8)
        for k in first:
            np.testing.assert_array_equal(host(again[k]), first[k], err_msg="ngram repeat %s" % k)


def test_ngram_exhaustive_ternary(orc):
    """Every context in {0,1,2}^L, L <= 9, at one stride (ragged lengths),
    for several lookup ranges and K."""
    ctxs, lens = [], []
    for L in range(0, 10):
        for c in itertools.product(range(3), repeat=L):
            ctxs.append(list(c) + [7] * (9 - L))
            lens.append(L)
    tokens = np.array(ctxs, np.int32)
    lengths = np.array(lens, np.int32)
    for (n_min, n_max) in [(1, 1), (1, 4), (2, 3), (2, 5), (3, 4)]:
        for K in (0, 1, 3, 8):
            _ngram_case(orc, tokens, lengths, n_min, n_max, K, "ternary")


def test_ngram_ragged_long_and_bad_lengths(orc):
    rng = np.random.default_rng(8)
    B, stride = 40, 5003                   # stride not a multiple of 4: scalar loads
    tokens = rng.integers(0, 50, (B, stride)).astype(np.int32)
    lengths = rng.integers(0, stride + 1, B).astype(np.int32)
    lengths[0], lengths[1], lengths[2] = -1, stride + 1, stride
    for b in range(3, B, 3):               # plant long repeats
        L = lengths[b]
        if L > 600:
            s = int(rng.integers(0, L - 500))
            tokens[b, L - 40:L] = tokens[b, s:s + 40]
    for n_min, n_max, K in [(1, 31, 16), (2, 5, 8), (5, 5, 3), (3, 20, 100)]:
        _ngram_case(orc, tokens, lengths, n_min, n_max, K, "ragged n%d-%d" % (n_min, n_max))
    aligned = np.zeros((B, 5004), np.int32)
    aligned[:, :stride] = tokens
    _ngram_case(orc, aligned, np.clip(lengths, -1, 5004), 2, 5, 8, "aligned stride")
