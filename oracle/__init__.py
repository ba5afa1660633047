"""CPU oracle for the speculative-decoding hot path (TEST INFRASTRUCTURE ONLY).

Plain fp64 C (``oracle.c``) behind ctypes.  Only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import this package; the
product library never does, and it shares no code with the GPU path.

Each wrapper takes numpy arrays (host memory) and returns numpy arrays.
bf16 inputs are passed as their raw ``uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32 = 0
BF16 = 1
PROBS = 2

FLAG_DRAFT_OOR = 1
FLAG_BAD_LEN = 2
FLAG_BAD_PARENT = 4

# Decision tie bands.  Accept tests: |u - p/q| < ACCEPT_BAND.  Final
# samples: u*S within SAMPLE_BAND_SCALE * sqrt(sum p^2 + sum q^2)
# probability mass of an end of the chosen token's CDF interval (the q terms
# after a rejection only).  The form follows the arithmetic of a kernel whose
# per-element probabilities carry independent rounding errors of about one
# fp32 ulp: the CDF error then grows like 2^-23 * sqrt(sum p^2 + sum q^2).
# The scale, 6 * 2^-23, is 2.9 times the largest CDF error measured on the
# GPU over 14 distributions (fp32 and bf16 logits, temperatures 0.3 to 1.3,
# masked rows, bonus-only and residual draws): 2.1 * 2^-23 times the same
# root.
# Suffix decoding counts the continuations of at most this many of the
# matched pattern's most recent occurrences in each text.
SUFFIX_OCC_CAP = 256

ACCEPT_BAND = 1e-6
SAMPLE_BAND_SCALE = 6.0 * 2.0 ** -23

GCC_FLAGS = ["-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC"]


def compile_source(src: str, out: str) -> str:
    """gcc a C source of the oracle into a shared library (IEEE fp64)."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc"] + GCC_FLAGS + ["-I", _HERE, "-o", tmp, src, "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile oracle.c into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        compile_source(_SRC, _LIB_PATH)
    return _LIB_PATH


def _ptr(a):
    return None if a is None else a.ctypes.data


def _dtype_code(arr):
    if arr.dtype == np.float32:
        return F32
    if arr.dtype == np.uint16:
        return BF16
    raise TypeError("logits must be float32 or uint16 (bf16 bits), got %s" % arr.dtype)


def _i32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


class Oracle:
    """The oracle's functions bound to one compiled library (the default
    build, or a deliberately altered copy in the mutation tests)."""

    F32, BF16 = F32, BF16
    FLAG_DRAFT_OOR, FLAG_BAD_LEN, FLAG_BAD_PARENT = FLAG_DRAFT_OOR, FLAG_BAD_LEN, FLAG_BAD_PARENT
    ACCEPT_BAND, SAMPLE_BAND_SCALE = ACCEPT_BAND, SAMPLE_BAND_SCALE

    def __init__(self, path):
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64, dbl = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.orc_argmax.argtypes = [P, ctypes.c_int, i64]
        L.orc_argmax.restype = i32
        L.orc_verify_greedy.argtypes = [P, ctypes.c_int, i64, P, P, i32, i32, i32, P, P, P, P]
        L.orc_verify_greedy.restype = None
        L.orc_verify_rejection.argtypes = [P, P, ctypes.c_int, i64, P, P, P, dbl, i32, i32, i32,
                                           dbl, dbl, P, P, P, P, P, P, P]
        L.orc_verify_rejection.restype = None
        L.orc_sample_cdf.argtypes = [P, P, ctypes.c_int, i32, dbl, P]
        L.orc_sample_cdf.restype = dbl
        L.orc_verify_tree.argtypes = [P, ctypes.c_int, i64, P, P, i32, i32, i32, P, P, P, P, P]
        L.orc_verify_tree.restype = None
        L.orc_ngram_propose.argtypes = [P, i64, P, i32, i32, i32, i32, P, P, P, P, P]
        L.orc_ngram_propose.restype = None
        L.orc_suffix_propose.argtypes = [P, i64, P, i32, P, i64, i32, i32, i32, dbl, i32, P, P, P,
                                         P, P, P]
        L.orc_suffix_propose.restype = None
        self.lib = L
        self.path = path

    def argmax(self, row):
        row = np.ascontiguousarray(row)
        return int(self.lib.orc_argmax(_ptr(row), _dtype_code(row), row.shape[-1]))

    def verify_greedy(self, logits, draft, draft_len=None):
        """logits [B, K+1, V] (float32 or bf16 bits), draft [B, K] int32."""
        logits = np.ascontiguousarray(logits)
        B, K1, V = logits.shape
        K = K1 - 1
        draft = _i32(draft).reshape(B, K)
        draft_len = _i32(draft_len)
        acc = np.zeros(B, np.int32)
        emi = np.zeros((B, K1), np.int32)
        amx = np.zeros((B, K1), np.int32)
        flg = np.zeros(B, np.uint32)
        self.lib.orc_verify_greedy(_ptr(logits), _dtype_code(logits), V, _ptr(draft),
                                   _ptr(draft_len), B, K, V, _ptr(acc), _ptr(emi), _ptr(amx),
                                   _ptr(flg))
        return dict(accepted=acc, emitted=emi, argmax=amx, flags=flg)

    def verify_rejection(self, target, draft_logits, draft, uniforms, temperature=1.0,
                         draft_len=None, accept_band=ACCEPT_BAND,
                         sample_band_scale=SAMPLE_BAND_SCALE, probs=False):
        """target [B, K+1, V], draft_logits [B, K, V], draft [B, K],
        uniforms [B, K+1] float32.  probs: the rows are float32
        probabilities (each row divided by its sum; temperature unused)."""
        target = np.ascontiguousarray(target)
        draft_logits = np.ascontiguousarray(draft_logits)
        B, K1, V = target.shape
        K = K1 - 1
        if draft_logits.shape != (B, K, V) or draft_logits.dtype != target.dtype:
            raise ValueError("draft logits must be [B, K, V] of the target's dtype")
        draft = _i32(draft).reshape(B, K)
        u = np.ascontiguousarray(uniforms, dtype=np.float32).reshape(B, K1)
        draft_len = _i32(draft_len)
        acc = np.zeros(B, np.int32)
        emi = np.zeros((B, K1), np.int32)
        pd = np.zeros((B, K), np.float64)
        qd = np.zeros((B, K), np.float64)
        at = np.zeros(B, np.uint8)
        st = np.zeros(B, np.uint8)
        flg = np.zeros(B, np.uint32)
        if probs and target.dtype != np.float32:
            raise TypeError("probabilities must be float32")
        code = PROBS if probs else _dtype_code(target)
        self.lib.orc_verify_rejection(_ptr(target), _ptr(draft_logits), code, V,
                                      _ptr(draft), _ptr(draft_len), _ptr(u), float(temperature),
                                      B, K, V, float(accept_band), float(sample_band_scale),
                                      _ptr(acc), _ptr(emi), _ptr(pd), _ptr(qd), _ptr(at),
                                      _ptr(st), _ptr(flg))
        return dict(accepted=acc, emitted=emi, p_draft=pd, q_draft=qd,
                    accept_tie=at.astype(bool), sample_tie=st.astype(bool), flags=flg)

    def sample_cdf(self, target_row, draft_row=None, temperature=1.0, probs=False):
        """The final sample's distribution for one row pair: returns (C, S)
        with C[v] the cumulative mass of r = max(0, p - q) (or of p when
        draft_row is None or the residual is empty) up to token v, S = C[-1]."""
        target_row = np.ascontiguousarray(target_row)
        V = target_row.shape[-1]
        if draft_row is not None:
            draft_row = np.ascontiguousarray(draft_row)
            if draft_row.shape != target_row.shape or draft_row.dtype != target_row.dtype:
                raise ValueError("draft_row must match target_row")
        if probs and target_row.dtype != np.float32:
            raise TypeError("probabilities must be float32")
        code = PROBS if probs else _dtype_code(target_row)
        cdf = np.zeros(V, np.float64)
        S = self.lib.orc_sample_cdf(_ptr(target_row), _ptr(draft_row), code, V, float(temperature),
                                    _ptr(cdf))
        return cdf, float(S)

    def verify_tree(self, logits, parent, token):
        """logits [B, N, V], parent [B, N], token [B, N]."""
        logits = np.ascontiguousarray(logits)
        B, N, V = logits.shape
        parent = _i32(parent).reshape(B, N)
        token = _i32(token).reshape(B, N)
        acc = np.zeros(B, np.int32)
        path = np.zeros((B, N), np.int32)
        emi = np.zeros((B, N), np.int32)
        amx = np.zeros((B, N), np.int32)
        flg = np.zeros(B, np.uint32)
        self.lib.orc_verify_tree(_ptr(logits), _dtype_code(logits), V, _ptr(parent), _ptr(token),
                                 B, N, V, _ptr(acc), _ptr(path), _ptr(emi), _ptr(amx), _ptr(flg))
        return dict(accepted=acc, path=path, emitted=emi, argmax=amx, flags=flg)

    def ngram_propose(self, tokens, lengths, n_min, n_max, K):
        """tokens [B, stride] int32, lengths [B] int32."""
        tokens = _i32(tokens)
        B, stride = tokens.shape
        lengths = _i32(lengths).reshape(B)
        prop = np.zeros((B, K), np.int32)
        plen = np.zeros(B, np.int32)
        mn = np.zeros(B, np.int32)
        mp = np.zeros(B, np.int32)
        flg = np.zeros(B, np.uint32)
        self.lib.orc_ngram_propose(_ptr(tokens), stride, _ptr(lengths), B, n_min, n_max, K,
                                   _ptr(prop), _ptr(plen), _ptr(mn), _ptr(mp), _ptr(flg))
        return dict(proposal=prop, proposal_len=plen, match_n=mn, match_pos=mp, flags=flg)


    def suffix_propose(self, tokens, lengths, history, m_min, m_max, K, min_prob,
                       occ_cap=SUFFIX_OCC_CAP):
        """tokens [B, stride] int32, lengths [B] int32, history [H] int32
        (None or empty for none)."""
        tokens = _i32(tokens)
        B, stride = tokens.shape
        lengths = _i32(lengths).reshape(B)
        hist = None if history is None else _i32(history).reshape(-1)
        H = 0 if hist is None else hist.size
        prop = np.zeros((B, K), np.int32)
        plen = np.zeros(B, np.int32)
        sco = np.zeros(B, np.float64)
        ml = np.zeros(B, np.int32)
        src = np.zeros(B, np.int32)
        flg = np.zeros(B, np.uint32)
        self.lib.orc_suffix_propose(_ptr(tokens), stride, _ptr(lengths), B,
                                    _ptr(hist) if H > 0 else None, H, m_min, m_max, K,
                                    float(min_prob), occ_cap, _ptr(prop), _ptr(plen), _ptr(sco),
                                    _ptr(ml), _ptr(src), _ptr(flg))
        return dict(proposal=prop, proposal_len=plen, score=sco, match_len=ml, source=src,
                    flags=flg)


_default = None


def default() -> Oracle:
    """The oracle built from oracle.c (compiled on first use if missing)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _default = Oracle(_LIB_PATH)
    return _default


def argmax(*a, **k):
    return default().argmax(*a, **k)


def verify_greedy(*a, **k):
    return default().verify_greedy(*a, **k)


def verify_rejection(*a, **k):
    return default().verify_rejection(*a, **k)


def sample_cdf(*a, **k):
    return default().sample_cdf(*a, **k)


def verify_tree(*a, **k):
    return default().verify_tree(*a, **k)


def ngram_propose(*a, **k):
    return default().ngram_propose(*a, **k)


def suffix_propose(*a, **k):
    return default().suffix_propose(*a, **k)


# ---------------------------------------------------------------- adaptive length

def adaptive_tier(ema, tiers):
    """The speculation length for an acceptance-length average `ema`: the
    smallest tier of at least 2 * ema, else the largest tier -- as much room
    above the usual accepted run as the run itself uses.  The average can
    never exceed the length in use, so the rule must move up before the
    average reaches the next tier (from length 1: once drafts are accepted
    more often than not) and back down before it reaches 0 (to length 1:
    once the average run is half a token)."""
    for t in tiers:
        if t >= 2.0 * ema:
            return t
    return tiers[-1]


def adaptive_lengths(accepted_means, tiers=(1, 3, 7), beta=0.2, ema0=0.0):
    """[Handbook] "adaptive" (SGLang's mechanism): after each verification
    round, an exponential moving average of the number of accepted draft
    tokens is updated, ema <- (1 - beta) * ema + beta * accepted, and the next
    round's speculation length is chosen among fixed tiers from it.  Returns
    the length used in each round (the first from ema0) and the averages
    after each round."""
    ema = float(ema0)
    ks, emas = [], []
    for a in accepted_means:
        ks.append(adaptive_tier(ema, tiers))
        ema = (1.0 - beta) * ema + beta * float(a)
        emas.append(ema)
    return ks, emas
