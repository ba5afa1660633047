"""Seeded synthetic workloads for the verifier and the n-gram proposer.

This module only draws inputs.  It holds none of the verification or
proposal arithmetic: no softmax, no acceptance test, no prefix scan, no
n-gram search.  Both the GPU path (tests, benchmark) and the CPU oracle take
their inputs from here and from nowhere else.

Two input-construction steps need facts about the drawn logits:

* planting greedy acceptance at a chosen rate alpha needs each row's argmax
  id, taken with ``numpy.argmax`` (lowest id on ties) on the bf16-rounded
  values, purely to decide which draft ids to plant;
* drawing rejection-sampling drafts from the draft distribution uses the
  Gumbel-max trick (argmax of logits/T plus Gumbel noise), which samples
  from softmax(logits/T) without ever forming it.

Neither result is an expected value: the oracle and the kernels each compute
every output on their own from the arrays returned here.

Value streams: numpy PCG64 for values, numpy Philox for the per-position
uniforms of rejection sampling.  bf16 arrays are returned as raw uint16 bit
patterns, rounded to nearest-even from float32.
"""
from __future__ import annotations

import numpy as np

BASE_SEED = 20261202

# Sizes of the five synthetic workloads (vocabularies of the Llama-3.x /
# Qwen model families the pages measure with).
GREEDY_SMALL = dict(B=4, K=4, V=32000, dtype="f32", sigma=1.0, alphas=(0.7,))
NGRAM = dict(B=64, L=8192, vocab=151936, zipf_s=1.1, n_spans=8, span_min=32, span_max=256,
             n_min=2, n_max=5, K=8)
REJECTION = dict(B=64, K=5, V=128256, sigma=2.0, noise_sigma=0.5, temperature=1.0)
GREEDY_LARGE = dict(B=256, K=8, V=151936, dtype="bf16", sigma=2.0, alphas=(0.3, 0.6, 0.9))
TREE = dict(B=32, N=64, V=128256, sigma=2.0, alpha_tree=0.6, max_depth=6, max_children=4)


def seed_for(config_number: int, salt: int = 0) -> int:
    return BASE_SEED + config_number + 1000 * salt


# --------------------------------------------------------------------------
# bf16 helpers (input construction only)
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16, nearest-even, returning uint16 bit patterns.
    Finite values and +-inf map correctly; NaN handling is not needed."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))
    return ((bits + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _widen(logits: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(logits) if logits.dtype == np.uint16 else logits


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _normal_logits(rng, shape, sigma, dtype):
    x = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def _plant(rng, top: np.ndarray, V: int, alpha: float) -> np.ndarray:
    """Draft = the row's argmax id with probability alpha, else a uniform id
    among the V-1 others (so every draft is accepted with probability alpha
    exactly, independently per position)."""
    hit = rng.random(top.shape) < alpha
    if V == 1:                      # no other id exists: every draft is the argmax
        return np.asarray(top, np.int32).copy()
    other = rng.integers(0, V - 1, size=top.shape)
    other = other + (other >= top)
    return np.where(hit, top, other).astype(np.int32)


def _row_argmax(logits: np.ndarray, rows_per_chunk: int = 256) -> np.ndarray:
    """numpy argmax (lowest index on ties) over the last axis, in chunks."""
    flat = logits.reshape(-1, logits.shape[-1])
    out = np.empty(flat.shape[0], np.int64)
    for s in range(0, flat.shape[0], rows_per_chunk):
        out[s:s + rows_per_chunk] = np.argmax(_widen(flat[s:s + rows_per_chunk]), axis=-1)
    return out.reshape(logits.shape[:-1])


# --------------------------------------------------------------------------
# greedy verification inputs
# --------------------------------------------------------------------------

def greedy_workload(B, K, V, dtype="bf16", sigma=2.0, alphas=(0.7,), seed=0):
    """logits [B, K+1, V] ~ N(0, sigma) (sigma = standard deviation), drafts
    [B, K] planted with acceptance alpha per position, one draft set per
    alpha, all on the same logits."""
    rng = _rng(seed)
    logits = _normal_logits(rng, (B, K + 1, V), sigma, dtype)
    top = _row_argmax(logits[:, :K, :]) if K > 0 else np.zeros((B, 0), np.int64)
    drafts = {}
    for a in alphas:
        drafts[a] = _plant(rng, top, V, a)
    return dict(logits=logits, drafts=drafts, B=B, K=K, V=V)


def planted_acceptance_drafts(top: np.ndarray, V: int, alpha: float, seed: int) -> np.ndarray:
    """Stand-alone planter: given reference ids `top`, plant acceptance alpha."""
    return _plant(_rng(seed), np.asarray(top), V, alpha)


# --------------------------------------------------------------------------
# rejection-sampling inputs
# --------------------------------------------------------------------------

def philox_uniforms(shape, seed) -> np.ndarray:
    """float32 uniforms in [0, 1) from numpy's Philox counter-based generator."""
    return np.random.Generator(np.random.Philox(seed)).random(shape, dtype=np.float32)


def gumbel_max_sample(logits_f32: np.ndarray, temperature: float, rng) -> np.ndarray:
    """One draw per row from softmax(logits / T) by the Gumbel-max trick."""
    flat = logits_f32.reshape(-1, logits_f32.shape[-1])
    out = np.empty(flat.shape[0], np.int64)
    for s in range(0, flat.shape[0], 64):
        blk = flat[s:s + 64].astype(np.float64) / temperature
        u = rng.random(blk.shape)
        u = np.maximum(u, np.finfo(np.float64).tiny)
        out[s:s + 64] = np.argmax(blk - np.log(-np.log(u)), axis=-1)
    return out.reshape(logits_f32.shape[:-1])


def mask_top_k(logits_f32: np.ndarray, top_k: int) -> np.ndarray:
    """Copy of logits with every entry outside its row's top_k set to -inf
    (top-k truncation of a sampler; ties at the cut keep the lower ids)."""
    flat = logits_f32.reshape(-1, logits_f32.shape[-1])
    out = np.full_like(flat, -np.inf)
    if top_k > 0:
        keep = np.argsort(-flat, axis=-1, kind="stable")[:, :top_k]
        rows = np.arange(flat.shape[0])[:, None]
        out[rows, keep] = flat[rows, keep]
    return out.reshape(logits_f32.shape)


def rejection_workload(B, K, V, sigma=2.0, noise_sigma=0.5, temperature=1.0, seed=0,
                       dtype="bf16", top_k=None):
    """target [B, K+1, V] = round(N(0, sigma)); draft logits [B, K, V] =
    round(target + N(0, noise_sigma)); with top_k, each row of both keeps
    only its top_k entries and the rest are -inf; draft ids x ~
    softmax(draft/T) (a separate PCG64 stream); uniforms [B, K+1] from
    Philox."""
    rng = _rng(seed)
    tgt32 = rng.standard_normal((B, K + 1, V), dtype=np.float32)
    if sigma != 1.0:
        tgt32 *= np.float32(sigma)
    noise = rng.standard_normal((B, K, V), dtype=np.float32)
    if noise_sigma != 1.0:
        noise *= np.float32(noise_sigma)
    if dtype == "bf16":
        target = f32_to_bf16_bits(tgt32)
        d32 = bf16_bits_to_f32(target[:, :K, :]) + noise
        draft_logits = f32_to_bf16_bits(d32)
        dwide = bf16_bits_to_f32(draft_logits)
    else:
        target = tgt32
        draft_logits = (tgt32[:, :K, :] + noise).astype(np.float32)
        dwide = draft_logits
    del noise
    if top_k is not None:
        tw = bf16_bits_to_f32(target) if dtype == "bf16" else target
        target = mask_top_k(tw, top_k)
        dwide = mask_top_k(dwide, top_k)
        if dtype == "bf16":
            target = f32_to_bf16_bits(target)
            draft_logits = f32_to_bf16_bits(dwide)
        else:
            draft_logits = dwide
    xs = gumbel_max_sample(dwide, temperature, _rng(seed + 7919)).astype(np.int32) if K > 0 \
        else np.zeros((B, 0), np.int32)
    u = philox_uniforms((B, K + 1), seed)
    return dict(target=target, draft_logits=draft_logits, draft=xs.reshape(B, K), uniforms=u,
                temperature=float(temperature), B=B, K=K, V=V)


# --------------------------------------------------------------------------
# tree verification inputs
# --------------------------------------------------------------------------

def random_tree(rng, N, max_depth=6, max_children=4):
    """parent[0] = -1; node j picks a uniform parent among earlier nodes that
    are shallower than max_depth and have fewer than max_children children."""
    parent = np.full(N, -1, np.int32)
    depth = np.zeros(N, np.int32)
    nchild = np.zeros(N, np.int32)
    for j in range(1, N):
        ok = np.nonzero((depth[:j] < max_depth) & (nchild[:j] < max_children))[0]
        p = int(ok[rng.integers(0, len(ok))])
        parent[j] = p
        depth[j] = depth[p] + 1
        nchild[p] += 1
    return parent


def tree_workload(B, N, V, sigma=2.0, alpha_tree=0.6, max_depth=6, max_children=4, seed=0,
                  dtype="bf16"):
    """logits [B, N, V] ~ N(0, sigma); a random tree per sequence; for every
    internal node, with probability alpha_tree one uniformly chosen child
    carries the node row's argmax id and every other child a distinct id
    different from it.  The root token is random."""
    rng = _rng(seed)
    logits = _normal_logits(rng, (B, N, V), sigma, dtype)
    top = _row_argmax(logits)
    parent = np.zeros((B, N), np.int32)
    token = np.zeros((B, N), np.int32)
    for b in range(B):
        par = random_tree(rng, N, max_depth, max_children)
        parent[b] = par
        token[b, 0] = rng.integers(0, V)
        for i in range(N):
            kids = np.nonzero(par == i)[0]
            if len(kids) == 0:
                continue
            t = int(top[b, i])
            others = rng.choice(V - 1, size=len(kids), replace=False)
            others = others + (others >= t)
            if rng.random() < alpha_tree:
                others[rng.integers(0, len(kids))] = t
            token[b, kids] = others
    return dict(logits=logits, parent=parent, token=token, B=B, N=N, V=V)


# --------------------------------------------------------------------------
# n-gram proposer inputs
# --------------------------------------------------------------------------

_ZIPF_CDF = {}


def _zipf_cdf(vocab, s):
    key = (vocab, s)
    if key not in _ZIPF_CDF:
        w = np.arange(1, vocab + 1, dtype=np.float64) ** (-s)
        c = np.cumsum(w)
        c /= c[-1]
        c[-1] = 1.0
        _ZIPF_CDF[key] = c
    return _ZIPF_CDF[key]


def zipf_tokens(rng, shape, vocab, s):
    """Token id = rank - 1 for a Zipf(s) law truncated to ranks 1..vocab."""
    cdf = _zipf_cdf(vocab, s)
    u = rng.random(shape)
    return np.minimum(np.searchsorted(cdf, u, side="right"), vocab - 1).astype(np.int32)


def plant_spans(rng, ctx, n_spans, span_min, span_max, end_at_tail):
    """Copy n_spans earlier stretches over non-overlapping destinations,
    applied in destination order; each source ends before its destination
    starts.  When end_at_tail, the last destination ends exactly at the end
    of the context (the context stops in the middle of a copy)."""
    L = len(ctx)
    lens = rng.integers(span_min, span_max + 1, size=n_spans)
    reserve = span_max                      # room for the first source
    free = L - reserve - int(lens.sum())
    if free < 0:
        raise ValueError("context too short for the planted spans")
    ngaps = n_spans if end_at_tail else n_spans + 1
    cuts = np.sort(rng.integers(0, free + 1, size=ngaps - 1))
    gaps = np.diff(np.concatenate([[0], cuts, [free]]))
    pos = reserve
    for k in range(n_spans):
        pos += int(gaps[k])
        ln = int(lens[k])
        src = int(rng.integers(0, pos - ln + 1))
        ctx[pos:pos + ln] = ctx[src:src + ln]
        pos += ln
    if end_at_tail:
        assert pos == L
    return ctx


def ngram_workload(B, L, vocab=151936, zipf_s=1.1, n_spans=8, span_min=32, span_max=256, seed=0,
                   chunk=1024):
    """tokens [B, L] int32: Zipf background with planted copied spans; for
    even b the last span ends at the end of the context, for odd b the
    spans are placed uniformly.  lengths [B] = L."""
    rng = _rng(seed)
    toks = np.empty((B, L), np.int32)
    for s in range(0, B, chunk):
        e = min(B, s + chunk)
        toks[s:e] = zipf_tokens(rng, (e - s, L), vocab, zipf_s)
        for b in range(s, e):
            plant_spans(rng, toks[b], n_spans, span_min, span_max, end_at_tail=(b % 2 == 0))
    return dict(tokens=toks, lengths=np.full(B, L, np.int32), B=B, L=L)


# Suffix decoding: the n-gram contexts, plus a shared history of earlier
# outputs.  [Arctic] "suffix decoding" targets agent loops that regenerate
# earlier material; the history stands in for those earlier outputs:
# documents of Zipf background, each carrying copies of spans taken from
# the contexts (so that a context's recent tokens can have been generated
# before) and copies of its own earlier spans, separated by -1.
SUFFIX = dict(B=64, L=8192, H=262144, m_min=1, m_max=32, K=16, min_prob=0.1)


def suffix_workload(B, L, H, vocab=151936, zipf_s=1.1, seed=0, doc_min=256, doc_max=4096,
                    copies_per_doc=4, span_min=16, span_max=256):
    """contexts as ngram_workload(B, L); history [H] int32 of documents
    (length U[doc_min, doc_max]) split by -1 separators."""
    wl = ngram_workload(B, L, vocab=vocab, zipf_s=zipf_s, seed=seed)
    rng = _rng(seed + 104729)
    hist = zipf_tokens(rng, (H,), vocab, zipf_s).astype(np.int32)
    pos = 0
    while pos < H:
        n = int(rng.integers(doc_min, doc_max + 1))
        end = min(H, pos + n)
        doc = hist[pos:end]
        for _ in range(copies_per_doc):
            ln = int(rng.integers(span_min, span_max + 1))
            if ln >= len(doc):
                break
            dst = int(rng.integers(0, len(doc) - ln + 1))
            b = int(rng.integers(0, B))
            src = int(rng.integers(0, L - ln + 1))
            doc[dst:dst + ln] = wl["tokens"][b, src:src + ln]
        if end < H:
            hist[end] = -1
        pos = end + 1
    wl["history"] = hist
    wl["H"] = H
    return wl
