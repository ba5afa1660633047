"""GPU parity on seeded random mixes of the parameters the other tests vary
one at a time: shapes, dtypes, row strides padded past V, base pointers a
few elements into their allocation, draft lengths, out-of-range ids,
temperatures, masked vocabularies, malformed trees, bad context lengths.
Each case is checked against the oracle: bit-exact for greedy, tree and
n-gram; decisions equal except oracle-flagged ties for rejection sampling
(logits and probabilities)."""
import numpy as np
import pytest
import torch

import proposal_sv_verify_amd as sv
from proposal_sv_verify_amd import workloads as W
from gpu_util import check_rejection, dev, host, say

pytestmark = pytest.mark.gpu

CASES = 60


def _view(a, pad, off):
    """a [..., V] on the device with row stride V + pad, its first element
    `off` elements into the allocation."""
    V = a.shape[-1]
    rows = int(np.prod(a.shape[:-1]))
    stride = V + pad
    flat = np.zeros(rows * stride + off + 8, a.dtype)
    flat[off:off + rows * stride].reshape(rows, stride)[:, :V] = a.reshape(rows, V)
    if a.dtype == np.uint16:
        t = torch.from_numpy(flat.view(np.int16)).to(dev()).view(torch.bfloat16)
    else:
        t = torch.from_numpy(flat).to(dev())
    return t[off:off + rows * stride].view(*a.shape[:-1], stride)[..., :V]


def _dv(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def _same(g, r, keys, label):
    for k in keys:
        np.testing.assert_array_equal(host(g[k]).astype(np.int64), np.asarray(r[k]).astype(np.int64),
                                      err_msg="%s %s" % (label, k))


def test_random_greedy(orc):
    rng = np.random.default_rng(101)
    for i in range(CASES):
        dtype = str(rng.choice(["f32", "bf16"]))
        B, K = int(rng.integers(1, 13)), int(rng.integers(0, 10))
        V = int(rng.choice([1, 2, 3, 7, 8, 13, 100, 1000, 4099, 20000, 65539]))
        wl = W.greedy_workload(B, K, V, dtype, 2.0, (0.6,), seed=1000 + i)
        lg = wl["logits"]
        if V > 4 and rng.random() < 0.5:              # duplicate the maximum in one row
            wide = W.bf16_bits_to_f32(lg) if dtype == "bf16" else lg
            b, r = int(rng.integers(0, B)), int(rng.integers(0, K + 1))
            lg[b, r, rng.choice(V, size=3, replace=False)] = lg[b, r, np.argmax(wide[b, r])]
        draft = wl["drafts"][0.6].copy()
        if K > 0 and rng.random() < 0.2:
            draft[0, 0] = V + 4
        dl = rng.integers(-1, K + 2, size=B).astype(np.int32) if rng.random() < 0.4 else None
        pad, off = int(rng.choice([0, 1, 5, 64])), int(rng.choice([0, 1, 3]))
        label = "greedy %d %s B%d K%d V%d pad%d off%d" % (i, dtype, B, K, V, pad, off)
        say(label)
        g = sv.verify_greedy(_view(lg, pad, off), _dv(draft), _dv(dl) if dl is not None else None)
        _same(g, orc.verify_greedy(lg, draft, dl), ("accepted", "emitted", "argmax", "flags"), label)


def test_random_tree(orc):
    rng = np.random.default_rng(102)
    for i in range(CASES):
        dtype = str(rng.choice(["f32", "bf16"]))
        B, N = int(rng.integers(1, 9)), int(rng.integers(1, 70))
        V = int(rng.choice([9, 12, 64, 777, 3001, 40000]))
        wl = W.tree_workload(B, N, V, 2.0, 0.8, N, int(rng.choice([2, 4, 8])), seed=2000 + i, dtype=dtype)
        parent, token = wl["parent"].copy(), wl["token"].copy()
        if N > 3 and rng.random() < 0.3:
            parent[0, N - 1] = N + 2
            token[0, 1] = -3
        pad, off = int(rng.choice([0, 1, 7])), int(rng.choice([0, 2]))
        label = "tree %d %s B%d N%d V%d pad%d off%d" % (i, dtype, B, N, V, pad, off)
        say(label)
        g = sv.verify_tree(_view(wl["logits"], pad, off), _dv(parent), _dv(token))
        _same(g, orc.verify_tree(wl["logits"], parent, token),
              ("accepted", "path", "emitted", "argmax", "flags"), label)


def test_random_rejection(orc):
    rng = np.random.default_rng(103)
    total_flag = total_mism = 0
    for i in range(CASES):
        dtype = str(rng.choice(["f32", "bf16"]))
        B, K = int(rng.integers(1, 13)), int(rng.integers(0, 8))
        V = int(rng.choice([1, 2, 8, 9, 100, 1000, 4097, 9000, 30000, 70001]))
        T = float(rng.choice([0.4, 1.0, 1.9]))
        top_k = int(rng.choice([0, 0, 1, 5, 50])) if V > 50 else 0
        wl = W.rejection_workload(B, K, V, 2.0, 0.7, T, seed=3000 + i, dtype=dtype, top_k=top_k or None)
        draft = wl["draft"].copy()
        if K > 0 and rng.random() < 0.2:
            draft[0, 0] = V + 3
        dl = rng.integers(-1, K + 2, size=B).astype(np.int32) if rng.random() < 0.4 else None
        pad, off = int(rng.choice([0, 1, 8])), int(rng.choice([0, 1]))
        label = "rejection %d %s B%d K%d V%d T%.1f top%d pad%d off%d" % (i, dtype, B, K, V, T, top_k, pad, off)
        say(label)
        tg = _view(wl["target"], pad, off)
        dg = _view(wl["draft_logits"], pad, off) if K > 0 else None
        g = sv.verify_rejection(tg, dg, _dv(draft), _dv(wl["uniforms"]), T,
                                _dv(dl) if dl is not None else None)
        r = orc.verify_rejection(wl["target"], wl["draft_logits"], draft, wl["uniforms"], T, dl)
        f, m = check_rejection(g, r, label)
        _same(g, r, ("flags",), label)
        total_flag += f
        total_mism += m
    say("random rejection mix: flagged %d, mismatched %d" % (total_flag, total_mism))


def test_random_rejection_probs(orc):
    rng = np.random.default_rng(104)
    for i in range(CASES):
        B, K = int(rng.integers(1, 10)), int(rng.integers(0, 6))
        V = int(rng.choice([1, 3, 8, 64, 1001, 5000]))
        P = rng.dirichlet(np.full(V, 0.3), size=(B, K + 1)).astype(np.float32)
        Q = rng.dirichlet(np.full(V, 0.3), size=(B, K)).astype(np.float32)
        P[P < 1e-4] = 0.0                             # zero entries, rows not normalised
        P[..., 0] += 1e-3
        Q[Q < 1e-4] = 0.0
        if K > 0:
            Q[..., -1] += 1e-3
        P *= np.float32(rng.uniform(0.5, 3.0))
        draft = np.array([[rng.choice(V, p=Q[b, k] / Q[b, k].sum()) for k in range(K)] for b in range(B)],
                         np.int32).reshape(B, K)
        u = rng.random((B, K + 1), dtype=np.float32)
        pad, off = int(rng.choice([0, 1, 4])), int(rng.choice([0, 1]))
        label = "probs %d B%d K%d V%d pad%d off%d" % (i, B, K, V, pad, off)
        say(label)
        g = sv.verify_rejection_probs(_view(P, pad, off), _view(Q, pad, off) if K > 0 else None,
                                      _dv(draft), _dv(u))
        f, m = check_rejection(g, orc.verify_rejection(P, Q, draft, u, 1.0, None, probs=True), label)
        assert m <= f


def test_random_ngram(orc):
    rng = np.random.default_rng(105)
    for i in range(CASES):
        B = int(rng.integers(1, 40))
        stride = int(rng.choice([1, 5, 31, 256, 1000, 4099]))
        alpha = int(rng.choice([2, 3, 5, 50]))
        tokens = rng.integers(0, alpha, (B, stride)).astype(np.int32)
        lengths = rng.integers(-2, stride + 3, size=B).astype(np.int32)
        n_min = int(rng.integers(1, 5))
        n_max = int(rng.integers(n_min, 9))
        K = int(rng.integers(0, 12))
        label = "ngram %d B%d stride%d alphabet%d n%d-%d K%d" % (i, B, stride, alpha, n_min, n_max, K)
        say(label)
        g = sv.ngram_propose(_dv(tokens), _dv(lengths), n_min, n_max, K)
        _same(g, orc.ngram_propose(tokens, lengths, n_min, n_max, K),
              ("proposal", "proposal_len", "match_n", "match_pos", "flags"), label)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_one_row_draft_beside_padded_target(orc, dtype):
    """B = 1, K = 1: the draft tensor is a single row, so its own stride is
    unconstrained and the call uses the padded target's."""
    wl = W.rejection_workload(1, 1, 3001, 2.0, 0.7, 1.0, seed=77, dtype=dtype)
    tg, dg = _view(wl["target"], 5, 1), _view(wl["draft_logits"], 5, 1)
    say("one-row draft", dtype, tuple(tg.shape), tg.stride(), tuple(dg.shape), dg.stride())
    g = sv.verify_rejection(tg, dg, _dv(wl["draft"]), _dv(wl["uniforms"]), 1.0)
    r = orc.verify_rejection(wl["target"], wl["draft_logits"], wl["draft"], wl["uniforms"], 1.0)
    f, m = check_rejection(g, r, "one-row draft " + dtype)
    assert m <= f
    if dtype == "f32":
        P = np.exp(wl["target"] - wl["target"].max(-1, keepdims=True)).astype(np.float32)
        Q = np.exp(wl["draft_logits"] - wl["draft_logits"].max(-1, keepdims=True)).astype(np.float32)
        g = sv.verify_rejection_probs(_view(P, 5, 1), _view(Q, 5, 1), _dv(wl["draft"]), _dv(wl["uniforms"]))
        r = orc.verify_rejection(P, Q, wl["draft"], wl["uniforms"], 1.0, None, probs=True)
        f, m = check_rejection(g, r, "one-row draft probs")
        assert m <= f


def _cuts(rng, V, P):
    P = min(P, V)
    inner = sorted(int(c) for c in rng.choice(np.arange(1, V), size=P - 1, replace=False)) if P > 1 else []
    c = [0] + inner + [V]
    return list(zip(c[:-1], c[1:]))


def test_random_vocabulary_shards(orc):
    """Greedy and rejection sampling over 1-8 vocabulary shards cut at random
    columns of padded, offset rows: the shard calls' combined results equal
    the oracle's on the whole rows."""
    rng = np.random.default_rng(106)
    for i in range(40):
        dtype = str(rng.choice(["f32", "bf16"]))
        B, K = int(rng.integers(1, 9)), int(rng.integers(0, 6))
        V = int(rng.choice([2, 9, 100, 3001, 20000]))
        pad, off = int(rng.choice([0, 3])), int(rng.choice([0, 1]))
        dl = rng.integers(-1, K + 2, size=B).astype(np.int32) if rng.random() < 0.4 else None
        dlt = _dv(dl) if dl is not None else None
        if i % 2 == 0:
            wl = W.greedy_workload(B, K, V, dtype, 2.0, (0.6,), seed=5000 + i)
            shards = _cuts(rng, V, int(rng.integers(1, 9)))
            label = "shard greedy %d %s B%d K%d V%d P%d" % (i, dtype, B, K, V, len(shards))
            say(label)
            lg = _view(wl["logits"], pad, off)
            parts = torch.empty(len(shards), B * (K + 1), dtype=torch.int64, device=dev())
            for p, (a, b) in enumerate(shards):
                sv.argmax_shard(lg[..., a:b], a, out=parts[p])
            g = sv.verify_greedy_partials(parts, _dv(wl["drafts"][0.6]), V, dlt)
            _same(g, orc.verify_greedy(wl["logits"], wl["drafts"][0.6], dl),
                  ("accepted", "emitted", "argmax", "flags"), label)
        else:
            V = max(V, 9)
            T = float(rng.choice([0.5, 1.0, 1.6]))
            wl = W.rejection_workload(B, K, V, 2.0, 0.7, T, seed=6000 + i, dtype=dtype)
            shards = _cuts(rng, V, int(rng.integers(1, 7)))
            label = "shard rejection %d %s B%d K%d V%d P%d T%.1f" % (i, dtype, B, K, V, len(shards), T)
            say(label)
            tg = _view(wl["target"], pad, off)
            dg = _view(wl["draft_logits"], pad, off) if K > 0 else None
            dr, u = _dv(wl["draft"]), _dv(wl["uniforms"])
            P = len(shards)
            parts = torch.empty(P, B * (2 * K + 1), 2, dtype=torch.float64, device=dev())
            for p, (a, b) in enumerate(shards):
                sv.rejection_shard_stats(tg[..., a:b], dg[..., a:b] if K > 0 else None, dr, a, T, dlt,
                                         out=parts[p])
            dec = sv.verify_rejection_partials(parts, dr, u, V, T, dlt)
            masses = torch.empty(P, B, 2, dtype=torch.float64, device=dev())
            wss = []
            for p, (a, b) in enumerate(shards):
                m = sv.rejection_shard_mass(tg[..., a:b], dg[..., a:b] if K > 0 else None, dec["state"], T,
                                            out=masses[p])
                wss.append(m["workspace"])
            emitted = torch.full((B, K + 1), -7, dtype=torch.int32, device=dev())
            for p, (a, b) in enumerate(shards):
                sv.rejection_shard_sample(tg[..., a:b], dg[..., a:b] if K > 0 else None, dr, u, dec["state"],
                                          masses, p, a, wss[p], emitted, T)
            out = dict(dec)
            out["emitted"] = emitted
            r = orc.verify_rejection(wl["target"], wl["draft_logits"], wl["draft"], wl["uniforms"], T, dl)
            f, m = check_rejection(out, r, label)
            assert m <= f


def test_random_suffix(orc):
    rng = np.random.default_rng(107)
    for i in range(40):
        B = int(rng.integers(1, 20))
        stride = int(rng.choice([3, 40, 333, 2048, 5003]))
        alpha = int(rng.choice([2, 3, 6, 40]))
        tokens = rng.integers(0, alpha, (B, stride)).astype(np.int32)
        lengths = rng.integers(-1, stride + 2, size=B).astype(np.int32)
        H = int(rng.choice([0, 1, 500, 20000]))
        hist = rng.integers(-1, alpha, size=H).astype(np.int32) if H else None
        m_min = int(rng.integers(1, 4))
        m_max = int(rng.integers(m_min, 33))
        K = int(rng.integers(0, 17))
        mp = float(rng.choice([0.0, 0.1, 0.5, 1.0]))
        label = "suffix %d B%d stride%d alphabet%d H%d m%d-%d K%d p%.1f" % (i, B, stride, alpha, H, m_min, m_max, K, mp)
        say(label)
        g = sv.suffix_propose(_dv(tokens), _dv(lengths), _dv(hist) if hist is not None else None,
                              m_min, m_max, K, mp)
        r = orc.suffix_propose(tokens, lengths, hist, m_min, m_max, K, mp)
        _same(g, r, ("proposal", "proposal_len", "match_len", "source", "flags"), label)
        np.testing.assert_array_equal(host(g["score"]), r["score"], err_msg=label + " score")
