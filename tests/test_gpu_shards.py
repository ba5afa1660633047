"""GPU: verification from vocabulary-shard partials.

Greedy and tree verification depend on each row's maximum and the lowest id
holding it ([Arctic] "inference pipeline optimisation": only drafts equal to
the greedy choice are kept; [Handbook] "Medusa"), and those merge across
vocabulary shards in the same total order.  Each shard's partials come from
sv_argmax_shard on a column slice of the logits; sv_verify_*_partials must
then give exactly what the unsharded call and the oracle give.
"""
import numpy as np
import pytest
import torch

import proposal_sv_verify_amd as sv
from proposal_sv_verify_amd import workloads as W
from gpu_util import dev, host, say, to_dev

pytestmark = pytest.mark.gpu


def _cuts(V, P, rng):
    """Boundaries of P shards over [0, V): random interior cuts, plus a
    1-column shard (P >= 3) and a 7-column one (P >= 4) in the middle."""
    n_fixed = 0 if P < 3 else (2 if P == 3 else 3)
    fixed = [V // 2, V // 2 + 1, V // 2 + 8][:n_fixed]
    free = [c for c in range(1, V) if c not in fixed]
    inner = set(fixed) | set(int(c) for c in rng.choice(free, size=P - 1 - len(fixed), replace=False))
    cuts = [0] + sorted(inner) + [V]
    assert len(cuts) == P + 1
    return list(zip(cuts[:-1], cuts[1:]))


def _shard_partials(logits_t, shards):
    rows = logits_t.numel() // logits_t.shape[-1]
    parts = torch.empty(len(shards), rows, dtype=torch.int64, device=logits_t.device)
    for p, (a, b) in enumerate(shards):
        sv.argmax_shard(logits_t[..., a:b], a, out=parts[p])
    return parts


def _check_partials(parts, logits_h, shards):
    got = host(parts).view(sv.PARTIAL_DTYPE)
    wide = W.bf16_bits_to_f32(logits_h) if logits_h.dtype == np.uint16 else logits_h
    flat = wide.reshape(-1, wide.shape[-1])
    for p, (a, b) in enumerate(shards):
        sl = flat[:, a:b]
        top = sl.max(axis=1)
        idx = np.argmax(sl, axis=1) + a            # numpy: the lowest index of the maximum
        none = top == -np.inf
        np.testing.assert_array_equal(got[p]["value"], top)
        np.testing.assert_array_equal(got[p]["index"], np.where(none, sv.NO_INDEX, idx))


def _planted_greedy_logits(B, K, V, dtype, shards, seed):
    """Greedy workload logits with equal maxima in two shards, a whole shard
    at -inf, and whole rows at -inf."""
    wl = W.greedy_workload(B, K, V, dtype=dtype, sigma=2.0, alphas=(0.6,), seed=seed)
    lg = wl["logits"].copy()
    flat = lg.reshape(-1, V)
    neg = np.uint16(0xFF80) if dtype == "bf16" else np.float32(-np.inf)
    big = W.f32_to_bf16_bits(np.array([40.0], np.float32))[0] if dtype == "bf16" else np.float32(40.0)
    (a0, b0), (a1, b1) = shards[0], shards[-1]
    flat[0, b0 - 1] = big                     # the same maximum at the end of shard 0 ...
    flat[0, a1] = big                         # ... and at the start of the last shard
    flat[1, a0:b0] = neg                      # a row whose first shard is all -inf
    flat[2, :] = neg                          # a row that is all -inf
    return lg, wl["drafts"][0.6]


@pytest.mark.parametrize("dtype,P", [("bf16", 1), ("bf16", 5), ("f32", 8), ("bf16", 3)])
def test_greedy_partials_equal_unsharded(orc, dtype, P):
    B, K, V = 16, 6, 50000
    rng = np.random.default_rng(40 + P)
    shards = _cuts(V, P, rng)
    logits_h, draft_h = _planted_greedy_logits(B, K, V, dtype, shards, seed=900 + P)
    say("greedy partials", dtype, "P", len(shards), shards[:4])
    lt, dr = to_dev(logits_h), to_dev(draft_h)
    dl_h = rng.integers(-1, K + 2, size=B).astype(np.int32)
    parts = _shard_partials(lt, shards)
    _check_partials(parts, logits_h, shards)
    for dl in (None, to_dev(dl_h)):
        got = sv.verify_greedy_partials(parts, dr, V, dl)
        ref = sv.verify_greedy(lt, dr, dl)
        for k in ("accepted", "emitted", "argmax", "flags"):
            np.testing.assert_array_equal(host(got[k]), host(ref[k]), err_msg=k)
        o = orc.verify_greedy(logits_h, draft_h, None if dl is None else dl_h)
        np.testing.assert_array_equal(host(got["accepted"]), o["accepted"])
        np.testing.assert_array_equal(host(got["emitted"]), o["emitted"])


@pytest.mark.parametrize("P", [2, 7])
def test_tree_partials_equal_unsharded(orc, P):
    wl = W.tree_workload(8, 64, 30000, seed=950 + P)
    rng = np.random.default_rng(60 + P)
    shards = _cuts(30000, P, rng)
    say("tree partials P", len(shards))
    lt = to_dev(wl["logits"])
    par, tok = to_dev(wl["parent"]), to_dev(wl["token"])
    parts = _shard_partials(lt, shards)
    _check_partials(parts, wl["logits"], shards)
    got = sv.verify_tree_partials(parts, par, tok, 30000)
    ref = sv.verify_tree(lt, par, tok)
    for k in ("accepted", "path", "emitted", "argmax", "flags"):
        np.testing.assert_array_equal(host(got[k]), host(ref[k]), err_msg=k)
    o = orc.verify_tree(wl["logits"], wl["parent"], wl["token"])
    for k in ("accepted", "path", "emitted"):
        np.testing.assert_array_equal(host(got[k]), o[k], err_msg=k)


def test_greedy_partials_full_size_eight_shards():
    """The large greedy workload (B 256, K 8, V 151936, bf16) split into the
    eight 18992-column shards of an 8-way tensor-parallel output layer."""
    wl = W.greedy_workload(**W.GREEDY_LARGE, seed=W.seed_for(4))
    V = 151936
    shards = [(i * V // 8, (i + 1) * V // 8) for i in range(8)]
    say("greedy partials full size, 8 shards")
    lt = to_dev(wl["logits"])
    parts = _shard_partials(lt, shards)
    for a in (0.3, 0.6, 0.9):
        dr = to_dev(wl["drafts"][a])
        got = sv.verify_greedy_partials(parts, dr, V)
        ref = sv.verify_greedy(lt, dr)
        for k in ("accepted", "emitted", "argmax"):
            np.testing.assert_array_equal(host(got[k]), host(ref[k]), err_msg="%s alpha %.1f" % (k, a))
