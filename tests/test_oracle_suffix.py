"""Pins for the oracle's suffix-decoding proposer (runs on the CPU).

[Arctic] "suffix decoding": the most recent tokens are looked up in suffix
trees of the current prompt and of earlier outputs; candidate tokens are
ranked by how often they followed (an empirical probability), and the
candidate sequence grows while it stays likely.  The pages leave the
scoring open; the oracle's reading (longest matched suffix, counts over
its most recent occurrences, greedy most-frequent path cut at a minimum
probability, score = the path's expected accepted tokens, the better of the
two texts) is pinned here by a hand-worked example, by a second,
independent implementation on exhaustive tiny inputs, by its reduction to
the n-gram lookup when one occurrence is counted, and by invariants.
"""
import itertools
from collections import Counter
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _run(o, contexts, history=None, m_min=1, m_max=8, K=4, min_prob=0.0, cap=oracle.SUFFIX_OCC_CAP):
    L = max(1, max(len(c) for c in contexts))
    tok = np.full((len(contexts), L), 99, np.int32)
    for b, c in enumerate(contexts):
        tok[b, :len(c)] = c
    lens = np.array([len(c) for c in contexts], np.int32)
    h = None if history is None else np.asarray(history, np.int32)
    return o.suffix_propose(tok, lens, h, m_min, m_max, K, min_prob, cap)


def test_worked_example(orc):
    """Context 5 1 2 3 9 1 2 3 7 1 2 3 9 4 1 2 3: its longest suffix seen
    before is 1 2 3 (4 1 2 3 is new), at ends 11, 7, 3.  They are followed
    by 9, 7, 9: token 9 with probability 2/3.  After 1 2 3 9 come 4 (end
    11) and 1 (end 3): a tie, the lower id 1 wins, 1/3.  Then only end 3
    continues: 2 and 3, 1/3 each.  Score 2/3 + 3 * 1/3 = 5/3."""
    r = _run(orc, [[5, 1, 2, 3, 9, 1, 2, 3, 7, 1, 2, 3, 9, 4, 1, 2, 3]], K=4)
    assert r["proposal"][0].tolist() == [9, 1, 2, 3]
    assert r["proposal_len"][0] == 4 and r["match_len"][0] == 3 and r["source"][0] == 0
    assert r["score"][0] == 5.0 / 3.0
    # a minimum probability of 1/2 keeps only the first token
    r = _run(orc, [[5, 1, 2, 3, 9, 1, 2, 3, 7, 1, 2, 3, 9, 4, 1, 2, 3]], K=4,
             min_prob=0.5)
    assert r["proposal"][0].tolist() == [9, -1, -1, -1] and r["score"][0] == 2.0 / 3.0


def test_history_tree_and_separators(orc):
    """The context 9 9 7 8 has no earlier 8; the history holds 7 8 twice,
    followed by 4 4 and a document separator, and by 4 6 2.  Step 1: 4
    (probability 1); step 2: 4 and 6 tie, the lower id 4 wins (1/2); step
    3: the path 7 8 4 4 is followed only by the separator, so it stops."""
    hist = [1, 7, 8, 4, 4, -1, 3, 7, 8, 4, 6, 2]
    r = _run(orc, [[9, 9, 7, 8]], history=hist, K=5)
    assert r["source"][0] == 1 and r["match_len"][0] == 2
    assert r["proposal"][0].tolist() == [4, 4, -1, -1, -1]
    assert r["score"][0] == 1.0 + 0.5
    # a separator never matches and never continues: 8 at the end of a
    # document is not an occurrence
    r = _run(orc, [[9, 9, 7, 8]], history=[7, 8, -1, 7, 8, -1], K=3)
    assert r["proposal_len"][0] == 0 and r["source"][0] == -1 and r["score"][0] == 0.0


def test_better_text_wins_and_context_wins_ties(orc):
    """The text whose path has the higher score (expected accepted tokens)
    gives the proposal; on equal scores the context does."""
    ctx = [3, 1, 2, 5, 3, 1, 2]       # 3 1 2 seen once before, followed by 5 3 1 2
    # history: only 1 2 matches, followed by 6, 6, 7 (6 at 2/3, then 0 at
    # 2/3): score 4/3 against the context's 2
    r = _run(orc, [ctx], history=[1, 2, 6, 0, 1, 2, 6, 0, 1, 2, 7], K=2)
    assert r["source"][0] == 0 and r["proposal"][0].tolist() == [5, 3]
    # history: 3 1 2 twice, followed by 8 8 8 and 8 8: score 2, a tie
    r = _run(orc, [ctx], history=[3, 1, 2, 8, 8, 8, 3, 1, 2, 8, 8], K=2)
    assert r["source"][0] == 0
    # K = 3: the context's 5 3 1 scores 3, the history's 8 8 8 scores
    # 1 + 1 + 1/2 (one occurrence has no third token)
    r = _run(orc, [ctx], history=[3, 1, 2, 8, 8, 8, 3, 1, 2, 8, 8], K=3)
    assert r["source"][0] == 0 and r["score"][0] == 3.0
    # a context whose 1 2 was followed by 5 once and by 6 once scores
    # 1/2 + 1/2; the history's 1 2 -> 9 9 (twice) scores 2 and wins
    r = _run(orc, [[1, 2, 5, 1, 2, 6, 1, 2]], history=[1, 2, 9, 9, 1, 2, 9, 9], K=2)
    assert r["source"][0] == 1 and r["proposal"][0].tolist() == [9, 9] and r["score"][0] == 2.0


def test_periodic_context_continues_the_period(orc):
    """Context (4 7 2) x 10, L = 30, patterns up to 6: the suffix 4 7 2 4 7 2
    ends at 26, 23, ..., 5 (8 occurrences).  The one at 26 has only 3 tokens
    after it and the one at 23 only 6, so the path's probabilities are 1
    for three steps, 7/8 for three and 6/8 for two: score 3 + 21/8 + 12/8.
    With a minimum probability of 1 the path stops after three tokens."""
    per = [4, 7, 2]
    ctx = per * 10
    r = _run(orc, [ctx], m_max=6, K=8, min_prob=0.0)
    assert r["proposal"][0].tolist() == (per * 3)[:8]
    assert r["score"][0] == 3 + 21 / 8 + 12 / 8 and r["match_len"][0] == 6
    r = _run(orc, [ctx], m_max=6, K=8, min_prob=1.0)
    assert r["proposal"][0].tolist() == per + [-1] * 5 and r["score"][0] == 3.0


def test_one_occurrence_reduces_to_ngram_lookup(orc):
    """Counting only the most recent occurrence, with no probability cut
    and no history, the proposal is the n-gram lookup's: the longest
    recent match (n_max down to n_min) and the tokens after it."""
    o = orc
    rng = np.random.default_rng(5)
    for trial in range(300):
        L = int(rng.integers(1, 40))
        ctx = rng.integers(0, 3 if trial % 2 else 5, size=L).astype(np.int32)
        n_min, n_max = sorted(rng.integers(1, 6, size=2).tolist())
        K = int(rng.integers(1, 9))
        s = o.suffix_propose(ctx[None, :], np.array([L], np.int32), None, n_min, n_max, K, 0.0, 1)
        g = o.ngram_propose(ctx[None, :], np.array([L], np.int32), n_min, n_max, K)
        assert s["proposal"].tolist() == g["proposal"].tolist(), (ctx, n_min, n_max, K)
        assert s["proposal_len"][0] == g["proposal_len"][0]
        assert s["match_len"][0] == g["match_n"][0]


# ---------------------------------------------------------------- brute force

def _brute_text(c, text, m_min, m_max, K, min_prob, cap):
    """Independent reading: enumerate pattern lengths from the longest,
    find occurrences by slice comparison, count continuation prefixes as
    tuples.  Returns (path, counts, n, m*)."""
    L, T = len(c), len(text)
    ends = [e for e in range(T - 2, -1, -1) if text[e + 1] >= 0]
    for m in range(min(m_max, L), m_min - 1, -1):
        pat = list(c[L - m:])
        if any(t < 0 for t in pat):
            continue
        occ = [e for e in ends if e - m + 1 >= 0 and list(text[e - m + 1:e + 1]) == pat]
        if occ:
            break
    else:
        return [], [], 0, 0
    occ = occ[:cap]
    conts = []
    for e in occ:
        t = []
        for j in range(1, K + 1):
            if e + j >= T or text[e + j] < 0:
                break
            t.append(int(text[e + j]))
        conts.append(tuple(t))
    path, counts = [], []
    for j in range(K):
        cnt = Counter(t[j] for t in conts if len(t) > j and t[:j] == tuple(path))
        if not cnt:
            break
        tok, n = min(cnt.items(), key=lambda kv: (-kv[1], kv[0]))
        if n < min_prob * len(occ):       # min_prob * len(occ) is exact in fp64 here
            break
        path.append(tok)
        counts.append(n)
    return path, counts, len(occ), m


def _brute(c, history, m_min, m_max, K, min_prob, cap):
    pc, cc, nc, mc = _brute_text(c, c, m_min, m_max, K, min_prob, cap)
    ph, ch, nh, mh = (_brute_text(c, history, m_min, m_max, K, min_prob, cap) if history
                      else ([], [], 0, 0))
    sc = Fraction(sum(cc), nc) if pc else Fraction(0)
    sh = Fraction(sum(ch), nh) if ph else Fraction(0)
    if pc and (not ph or sc >= sh):
        return pc, float(sc), mc, 0
    if ph:
        return ph, float(sh), mh, 1
    return [], 0.0, 0, -1


@pytest.mark.parametrize("m_min,m_max,K,min_prob,cap", [(1, 3, 3, 0.0, 256), (2, 4, 2, 0.5, 2),
                                                       (1, 2, 4, 0.34, 3), (1, 5, 1, 1.0, 1)])
def test_exhaustive_ternary_against_brute_force(orc, m_min, m_max, K, min_prob, cap):
    """Every context over {0, 1, 2} of length <= 6, against four histories
    (none, separators inside, a repetitive one, a random one)."""
    o = orc
    rng = np.random.default_rng(m_max * 10 + K)
    histories = [None, [0, 1, -1, 2, 0, 1, 2, -1, 1], [0, 1, 2] * 4,
                 rng.integers(-1, 3, size=15).tolist()]
    ctxs = [list(t) for L in range(0, 7) for t in itertools.product(range(3), repeat=L)]
    for h in histories:
        r = _run(o, ctxs, history=h, m_min=m_min, m_max=m_max, K=K, min_prob=min_prob, cap=cap)
        for b, c in enumerate(ctxs):
            path, score, ml, src = _brute(c, h, m_min, m_max, K, min_prob, cap)
            got = r["proposal"][b][:r["proposal_len"][b]].tolist()
            assert got == path, (c, h)
            assert r["score"][b] == score and r["match_len"][b] == ml and r["source"][b] == src, (c, h)


def test_invariants_on_repetitive_text(orc):
    """On planted-copy contexts: every proposal is what follows some
    occurrence of the matched suffix, the score is at most the length, and
    at least the length times the minimum probability."""
    from proposal_sv_verify_amd import workloads as W
    wl = W.ngram_workload(8, 2000, seed=77)
    o = orc
    r = o.suffix_propose(wl["tokens"], wl["lengths"], None, 1, 16, 12, 0.25)
    for b in range(8):
        n = r["proposal_len"][b]
        if n == 0:
            continue
        c = wl["tokens"][b, :wl["lengths"][b]]
        L, m = len(c), r["match_len"][b]
        prop = r["proposal"][b][:n].tolist()
        hits = [e for e in range(L - 1) if e - m + 1 >= 0 and (c[e - m + 1:e + 1] == c[L - m:]).all()
                and c[e + 1:e + 1 + n].tolist() == prop]
        assert hits, b
        assert 0.25 * n - 1e-12 <= r["score"][b] <= n + 1e-12
