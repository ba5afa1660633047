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
from gpu_util import check_rejection, dev, host, say, to_dev

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


def test_greedy_partials_full_size_eight_shards(orc):
    """The large greedy workload (B 256, K 8, V 151936, bf16) split into the
    eight 18992-column shards of an 8-way tensor-parallel output layer: the
    same results as the oracle on the whole rows, and as the unsharded call."""
    wl = W.greedy_workload(**W.GREEDY_LARGE, seed=W.seed_for(4))
    V = 151936
    shards = [(i * V // 8, (i + 1) * V // 8) for i in range(8)]
    say("greedy partials full size, 8 shards")
    lt = to_dev(wl["logits"])
    parts = _shard_partials(lt, shards)
    for a in (0.3, 0.6, 0.9):
        dr = to_dev(wl["drafts"][a])
        got = sv.verify_greedy_partials(parts, dr, V)
        o = orc.verify_greedy(wl["logits"], wl["drafts"][a])
        for k in ("accepted", "emitted", "argmax"):
            np.testing.assert_array_equal(host(got[k]), o[k], err_msg="oracle %s alpha %.1f" % (k, a))
        ref = sv.verify_greedy(lt, dr)
        for k in ("accepted", "emitted", "argmax"):
            np.testing.assert_array_equal(host(got[k]), host(ref[k]), err_msg="%s alpha %.1f" % (k, a))


# ------------------------------------------------------------ rejection sampling
#
# Sharded rejection sampling takes four steps per call: per-shard row
# statistics, the accept test on all shards' partials, per-shard sample
# masses, and the owner shard's sample.  Its decisions must match the oracle
# (and the unsharded call) except within the rounding band of a tie, which
# the oracle flags.

def _rejection_sharded(wl, shards, draft_len=None):
    B, K, V, T = wl["B"], wl["K"], wl["V"], wl["temperature"]
    tg, dg = to_dev(wl["target"]), to_dev(wl["draft_logits"])
    dr, u = to_dev(wl["draft"]), to_dev(wl["uniforms"])
    dl = to_dev(draft_len) if draft_len is not None else None
    P = len(shards)
    parts = torch.empty(P, B * (2 * K + 1), 2, dtype=torch.float64, device=dev())
    for p, (a, b) in enumerate(shards):
        sv.rejection_shard_stats(tg[..., a:b], dg[..., a:b], dr, a, T, dl, out=parts[p])
    stats = torch.zeros(3 + K, dtype=torch.int64, device=dev())
    dec = sv.verify_rejection_partials(parts, dr, u, V, T, dl, stats=stats)
    masses = torch.empty(P, B, 2, dtype=torch.float64, device=dev())
    wss = []
    for p, (a, b) in enumerate(shards):
        m = sv.rejection_shard_mass(tg[..., a:b], dg[..., a:b], dec["state"], T, out=masses[p])
        wss.append(m["workspace"])
    emitted = torch.full((B, K + 1), -7, dtype=torch.int32, device=dev())
    for p, (a, b) in enumerate(shards):
        sv.rejection_shard_sample(tg[..., a:b], dg[..., a:b], dr, u, dec["state"], masses, p, a,
                                  wss[p], emitted, T)
    out = dict(dec)
    out["emitted"] = emitted
    out["stats"] = stats
    out["parts"] = parts
    return out


def _check_soft_partials(parts, wl, shards, draft_len=None):
    """Each shard's per-row (z, m) gives the shard's log-sum-exp of l / T,
    and lx is the logit at the row's draft token when the shard holds it."""
    B, K, T = wl["B"], wl["K"], wl["temperature"]
    got = host(parts).view(sv.SOFT_PARTIAL_DTYPE).reshape(len(shards), B, 2 * K + 1)
    wide = lambda a: (W.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)
    tg, dg = wide(wl["target"]), wide(wl["draft_logits"])
    lens = np.full(B, K) if draft_len is None else np.clip(draft_len, 0, K)
    for p, (a, b) in enumerate(shards):
        for bb in range(B):
            for r in range(2 * K + 1):
                is_t = r <= K
                i = r if is_t else r - K - 1
                g = got[p, bb, r]
                if not (i <= lens[bb] if is_t else i < lens[bb]):
                    assert g["z"] == 0.0 and g["m"] == -np.inf
                    continue
                row = (tg[bb, i] if is_t else dg[bb, i])[a:b] / T
                lse = np.logaddexp.reduce(row)
                mine = np.log(g["z"]) + np.float64(g["m"]) / T
                np.testing.assert_allclose(mine, lse, rtol=0, atol=1e-6 * max(1.0, abs(lse)))
                x = wl["draft"][bb, i] if i < K else -1
                if i < K and a <= x < b:
                    src = (tg[bb, i] if is_t else dg[bb, i])
                    assert np.float64(g["lx"]) == src[x]
                else:
                    assert np.isnan(g["lx"])


def _rejection_shard_case(orc, wl, shards, draft_len=None, label=""):
    say("sharded rejection", label, "P", len(shards), shards[:4])
    g = _rejection_sharded(wl, shards, draft_len)
    r = orc.verify_rejection(wl["target"], wl["draft_logits"], wl["draft"], wl["uniforms"],
                             wl["temperature"], draft_len)
    flagged, mism = check_rejection(g, r, label)
    np.testing.assert_array_equal(host(g["flags"]).astype(np.uint32), r["flags"])
    acc = host(g["accepted"]).astype(np.int64)
    assert host(g["stats"])[0] == acc.sum() and host(g["stats"])[2] == (acc + 1).sum()
    # the unsharded call on the same inputs: the same except at flagged ties
    u = sv.verify_rejection(to_dev(wl["target"]), to_dev(wl["draft_logits"]), to_dev(wl["draft"]),
                            to_dev(wl["uniforms"]), wl["temperature"],
                            to_dev(draft_len) if draft_len is not None else None)
    tie = r["accept_tie"] | r["sample_tie"]
    same = (host(u["emitted"]) == host(g["emitted"])).all(axis=1)
    assert (same | tie).all(), "%s: sharded and unsharded differ outside flagged ties" % label
    return g, flagged, mism


@pytest.mark.parametrize("dtype,T,P,ragged", [("bf16", 1.0, 3, False), ("f32", 0.7, 5, True),
                                              ("bf16", 1.3, 2, True), ("f32", 1.0, 16, False)])
def test_rejection_sharded_matches_oracle(orc, dtype, T, P, ragged):
    B, K, V = 12, 5, 30000
    wl = W.rejection_workload(B, K, V, 2.0, 0.5, T, seed=700 + P, dtype=dtype)
    rng = np.random.default_rng(80 + P)
    shards = _cuts(V, P, rng)
    dl = rng.integers(-1, K + 2, size=B).astype(np.int32) if ragged else None
    g, _, _ = _rejection_shard_case(orc, wl, shards, dl, "%s T%.1f P%d" % (dtype, T, P))
    _check_soft_partials(g["parts"], wl, shards, dl)


def test_rejection_sharded_bonus_only_and_masked(orc):
    """K = 0 (every call samples the bonus from p) and top-k masked rows,
    where whole shards of a row are -inf."""
    wl = W.rejection_workload(9, 0, 7000, 2.0, 0.5, 1.0, seed=733, dtype="bf16")
    _rejection_shard_case(orc, wl, _cuts(7000, 4, np.random.default_rng(3)), label="K0 P4")
    wl = W.rejection_workload(16, 4, 40000, 2.0, 0.7, 1.0, seed=734, dtype="bf16", top_k=40)
    _rejection_shard_case(orc, wl, [(i * 5000, (i + 1) * 5000) for i in range(8)],
                          label="top40 P8")


def test_rejection_sharded_full_size_eight_shards(orc):
    """B 64, K 5, V 128256 bf16 in the eight 16032-column shards of an
    8-way tensor-parallel output layer."""
    wl = W.rejection_workload(**W.REJECTION, seed=W.seed_for(3))
    V = wl["V"]
    shards = [(i * V // 8, (i + 1) * V // 8) for i in range(8)]
    _, flagged, mism = _rejection_shard_case(orc, wl, shards, label="full size P8")
    say("sharded rejection full size: flagged %d, mismatched %d of 64" % (flagged, mism))
    assert flagged <= 4 and mism == 0
