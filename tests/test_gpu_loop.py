"""GPU: the propose -> verify loop end to end, on the device.

[Handbook] "how it works": a draft of up to K tokens is scored by the target
in one pass and the longest agreeing prefix plus one target token is kept;
with greedy decoding the output is exactly what the target alone would
produce ([Handbook] "why", [vLLM-03] "1. principle").  [vLLM-03] "3-1": a
proposer that finds no match proposes nothing, and the step still emits the
target's token.

Each step here runs sv_ngram_propose on the current contexts, builds the
toy target's logits for the K+1 positions of the drafted continuation,
verifies with sv_verify_greedy using the proposal lengths as draft_len, and
appends the emitted tokens -- all on the device, with no host round trip
inside the loop.  The result must equal plain greedy decoding of the same
toy target, computed on the host with numpy.  The per-call counters must
add up to what the loop emitted.
"""
import numpy as np
import pytest
import torch

import proposal_sv_verify_amd as sv
from proposal_sv_verify_amd import workloads as W
from gpu_util import dev, host, say

pytestmark = pytest.mark.gpu

V, ROWS = 64, 13


def _table(seed, scale=2.0):
    """The toy target: next-token logits are a fixed bf16 row chosen by a
    hash of the last three tokens (bf16 rounding makes ties common)."""
    rng = np.random.default_rng(seed)
    return W.f32_to_bf16_bits(rng.standard_normal((ROWS, V)).astype(np.float32) * np.float32(scale))


def _row_index(a, b, c):
    return (a * 4099 + b * 131 + c * 7) % ROWS


def _plain_greedy(table, prompt, n_new):
    ctx = list(prompt)
    for _ in range(n_new):
        row = W.bf16_bits_to_f32(table[_row_index(ctx[-3], ctx[-2], ctx[-1])])
        ctx.append(int(np.argmax(row)))
    return ctx


@pytest.mark.parametrize("K", [2, 4, 8])
def test_greedy_loop_equals_plain_greedy(K):
    B, steps, cap = 256, 48, 1024
    table_h = _table(seed=100 + K)
    rng = np.random.default_rng(7 + K)
    plen = rng.integers(6, 21, size=B)
    prompts = [list(rng.integers(0, V, size=int(n))) for n in plen]

    d = dev()
    table = torch.from_numpy(table_h.view(np.int16)).to(d).view(torch.bfloat16)
    ctx = torch.zeros(B, cap + K + 1, dtype=torch.int32, device=d)   # tail columns: scratch
    for b, p in enumerate(prompts):
        ctx[b, :len(p)] = torch.tensor(p, dtype=torch.int32)
    lengths = torch.tensor(plen, dtype=torch.int32, device=d)
    stats = torch.zeros(3 + K, dtype=torch.int64, device=d)
    drafted = torch.zeros((), dtype=torch.int64, device=d)
    cols = torch.arange(K + 1, device=d)[None, :]
    trash = cap + K                                                    # a column no result reads

    say("greedy loop", B, "sequences", steps, "steps, K", K)
    for _ in range(steps):
        prop = sv.ngram_propose(ctx[:, :cap], lengths, 2, 5, K)
        draft, dlen = prop["proposal"], prop["proposal_len"]
        drafted += dlen.sum()
        # the last three tokens of context ++ draft[0..i) for i = 0..K
        L = lengths.long()[:, None]
        tail = torch.cat([ctx.gather(1, (L - 3 + torch.arange(3, device=d)[None, :])),
                          draft.clamp(min=0)], dim=1).long()
        idx = _row_index(tail[:, 0:K + 1], tail[:, 1:K + 2], tail[:, 2:K + 3])
        logits = table[idx]                                            # [B, K+1, V] bf16
        out = sv.verify_greedy(logits, draft, dlen, stats=stats)
        acc, emi = out["accepted"].long(), out["emitted"]
        pos = torch.where(cols <= acc[:, None], L + cols, torch.full_like(cols, trash))
        ctx.scatter_(1, pos, emi)
        lengths += (acc + 1).int()
    torch.cuda.synchronize()

    final = host(lengths).astype(np.int64)
    ctx_h = host(ctx)
    new = final - plen
    assert (new >= steps).all() and (final <= cap).all()
    for b in range(B):
        ref = _plain_greedy(table_h, prompts[b], int(new[b]))
        assert list(ctx_h[b, :final[b]]) == ref, "sequence %d diverges from plain greedy" % b
    st = host(stats)
    assert st[2] == new.sum()                       # emitted total
    assert st[0] == new.sum() - B * steps           # accepted = emitted minus one per step
    assert st[1] == int(host(drafted))              # drafted = sum of proposal lengths
    assert st[3:].sum() == st[0]                    # per-position acceptances add up
    say("greedy loop: %.2f tokens per step, %d drafts proposed, %d accepted"
        % (new.mean() / steps, st[1], st[0]))
    assert st[0] > 0                                # the lookups do hit on this target


def test_rejection_loop_matches_oracle_loop(orc):
    """Rejection sampling in the loop ([vLLM-03] "1. principle"), with the
    n-gram proposal as a point-mass draft distribution (q = 1 at the
    proposed token, -inf logits elsewhere; rows past the proposal length
    are not read).  The same loop runs on the host with the oracle and the
    same Philox uniforms; every step must agree, except that a sequence
    whose step the oracle flags as a tie may diverge from then on."""
    B, K, steps, cap, T = 64, 4, 32, 512, 0.8
    table_h = _table(seed=211, scale=5.0)
    rng = np.random.default_rng(21)
    # prompts are the target's own greedy continuations of random starts, so
    # they repeat (the toy target cycles), lookups propose from the start,
    # and the drafts are likely but not certain under sampling
    prompts = [_plain_greedy(table_h, list(rng.integers(0, V, size=3)), int(n))
               for n in rng.integers(40, 81, size=B)]
    plen = np.array([len(q) for q in prompts])
    ctx_h = np.zeros((B, cap), np.int32)
    for b in range(B):
        ctx_h[b, :plen[b]] = prompts[b]
    len_h = plen.astype(np.int32).copy()

    d = dev()
    table = torch.from_numpy(table_h.view(np.int16)).to(d).view(torch.bfloat16)
    ctx = torch.from_numpy(ctx_h.copy()).to(d)
    lengths = torch.from_numpy(len_h.copy()).to(d)
    cols = torch.arange(K + 1, device=d)[None, :]
    live = np.ones(B, bool)                          # not yet diverged at a flagged tie
    flagged = proposed = 0
    say("rejection loop", B, "sequences", steps, "steps, K", K)
    for step in range(steps):
        u_h = W.philox_uniforms((B, K + 1), 5000 + step)
        # device step
        prop = sv.ngram_propose(ctx, lengths, 2, 5, K)
        draft, dlen = prop["proposal"], prop["proposal_len"]
        L = lengths.long()[:, None]
        tail = torch.cat([ctx.gather(1, (L - 3 + torch.arange(3, device=d)[None, :])),
                          draft.clamp(min=0)], dim=1).long()
        tl = table[_row_index(tail[:, 0:K + 1], tail[:, 1:K + 2], tail[:, 2:K + 3])]
        dl = torch.full((B, K, V), float("-inf"), device=d)
        dl.scatter_(2, draft.clamp(min=0).long()[:, :, None], 0.0)
        dl = dl.to(torch.bfloat16)
        out = sv.verify_rejection(tl, dl, draft, torch.from_numpy(u_h).to(d), T, dlen)
        acc, emi = out["accepted"].long(), out["emitted"]
        pos = torch.where(cols <= acc[:, None], L + cols, torch.full_like(cols, cap - 1))
        ctx.scatter_(1, pos, emi)
        lengths += (acc + 1).int()

        # host step with the oracle, from the host copy of the contexts
        ph = orc.ngram_propose(ctx_h, len_h, 2, 5, K)
        proposed += int(ph["proposal_len"].sum())
        np.testing.assert_array_equal(host(prop["proposal"])[live], ph["proposal"][live])
        dr, dn = ph["proposal"], ph["proposal_len"]
        tail_h = np.concatenate([np.stack([ctx_h[b, len_h[b] - 3:len_h[b]] for b in range(B)]),
                                 np.maximum(dr, 0)], axis=1).astype(np.int64)
        tl_h = table_h[_row_index(tail_h[:, 0:K + 1], tail_h[:, 1:K + 2], tail_h[:, 2:K + 3])]
        dl_h = np.full((B, K, V), -np.inf, np.float32)
        np.put_along_axis(dl_h, np.maximum(dr, 0)[:, :, None].astype(np.int64), 0.0, axis=2)
        r = orc.verify_rejection(tl_h, W.f32_to_bf16_bits(dl_h), dr, u_h, T, dn)
        acc_g, emi_g = host(out["accepted"]), host(emi)
        for b in np.nonzero(live)[0]:
            same = acc_g[b] == r["accepted"][b] and np.array_equal(emi_g[b], r["emitted"][b])
            if not same:
                assert r["accept_tie"][b] or r["sample_tie"][b], \
                    "step %d seq %d: GPU (%d, %s) vs oracle (%d, %s), no tie" % (
                        step, b, acc_g[b], emi_g[b], r["accepted"][b], r["emitted"][b])
                live[b] = False
                flagged += 1
        for b in range(B):
            n = int(r["accepted"][b])
            ctx_h[b, len_h[b]:len_h[b] + n + 1] = r["emitted"][b, :n + 1]
            len_h[b] += n + 1
    assert live.sum() >= B - 2, "too many flagged divergences: %d" % flagged
    ctx_g, len_g = host(ctx), host(lengths)
    for b in np.nonzero(live)[0]:
        assert len_g[b] == len_h[b]
        np.testing.assert_array_equal(ctx_g[b, :len_g[b]], ctx_h[b, :len_h[b]])
    say("rejection loop: %.2f tokens per step, %d drafts proposed, %d accepted, %d flagged divergences"
        % ((len_h - plen).mean() / steps, proposed, (len_h - plen).sum() - B * steps, flagged))
    assert proposed > B and (len_h - plen).sum() > B * steps + B   # drafts proposed and accepted


def test_adaptive_length_loop_stays_lossless():
    """[Handbook] "adaptive": the speculation length changes between rounds
    (tiers 1, 3, 7 from the moving average of accepted drafts, read from the
    verifier's counters), and the output is still plain greedy decoding."""
    B, rounds, cap, tiers = 128, 40, 1024, (1, 3, 7)
    table_h = _table(seed=333)
    rng = np.random.default_rng(33)
    # prompts that already follow the target (its greedy continuation of a
    # random start), so lookups hit and the length has a reason to grow
    prompts = [_plain_greedy(table_h, list(rng.integers(0, V, size=3)), int(n))
               for n in rng.integers(20, 60, size=B)]
    plen = np.array([len(q) for q in prompts])
    d = dev()
    table = torch.from_numpy(table_h.view(np.int16)).to(d).view(torch.bfloat16)
    ctx = torch.zeros(B, cap + 8, dtype=torch.int32, device=d)
    for b, p in enumerate(prompts):
        ctx[b, :len(p)] = torch.tensor(p, dtype=torch.int32)
    lengths = torch.tensor(plen, dtype=torch.int32, device=d)
    ctl = sv.Adaptive(tiers, beta=0.3)
    used = []
    say("adaptive loop", B, "sequences", rounds, "rounds")
    for _ in range(rounds):
        K = ctl.k
        used.append(K)
        prop = sv.ngram_propose(ctx[:, :cap], lengths, 2, 5, K)
        draft, dlen = prop["proposal"], prop["proposal_len"]
        L = lengths.long()[:, None]
        tail = torch.cat([ctx.gather(1, (L - 3 + torch.arange(3, device=d)[None, :])),
                          draft.clamp(min=0)], dim=1).long()
        logits = table[_row_index(tail[:, 0:K + 1], tail[:, 1:K + 2], tail[:, 2:K + 3])]
        stats = torch.zeros(3 + K, dtype=torch.int64, device=d)
        out = sv.verify_greedy(logits, draft, dlen, stats=stats)
        acc, emi = out["accepted"].long(), out["emitted"]
        cols = torch.arange(K + 1, device=d)[None, :]
        pos = torch.where(cols <= acc[:, None], L + cols, torch.full_like(cols, cap + 7))
        ctx.scatter_(1, pos, emi)
        lengths += (acc + 1).int()
        ctl.update(float(host(stats)[0]) / B)
    final, ctx_h = host(lengths).astype(np.int64), host(ctx)
    for b in range(B):
        ref = _plain_greedy(table_h, prompts[b], int(final[b] - plen[b]))
        assert list(ctx_h[b, :final[b]]) == ref, "sequence %d diverges" % b
    say("adaptive loop: lengths used", used)
    assert len(set(used)) >= 2                      # the length did adapt
