"""The library's adaptive speculation length (sv_adaptive_*, host code)
against the oracle's, on random rounds; and its argument checks.  Runs on
the CPU: the controller never touches the GPU."""
import ctypes

import numpy as np
import pytest

import oracle
import proposal_sv_verify_amd as sv


@pytest.mark.parametrize("seed", range(6))
def test_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    ntiers = int(rng.integers(1, 6))
    tiers = tuple(sorted(int(t) for t in rng.choice(np.arange(1, 40), size=ntiers, replace=False)))
    beta = float(rng.uniform(0.01, 1.0))
    ema0 = float(rng.uniform(0.0, 10.0))
    acc = list(rng.uniform(0.0, tiers[-1], size=200))
    ks, emas = oracle.adaptive_lengths(acc, tiers, beta, ema0)
    a = sv.Adaptive(tiers, beta, ema0)
    got_k, got_e = [a.k], []
    for x in acc:
        got_k.append(a.update(x))
        got_e.append(a.ema)
    assert got_k[:-1] == ks                        # the length each round used
    assert got_e == emas                           # bit-identical averages (fp64, same order)
    assert got_k[-1] == oracle.adaptive_tier(emas[-1], tiers)


def test_rejects_bad_arguments():
    L = sv.load()
    s = sv._AdaptiveState()
    def init(tiers, beta=0.2, ema0=0.0):
        arr = (ctypes.c_int32 * max(1, len(tiers)))(*tiers)
        return L.sv_adaptive_init(ctypes.byref(s), arr, len(tiers), beta, ema0)
    assert init([1, 3, 7]) == sv.SV_OK
    assert init([]) == sv.SV_ERR_INVALID_ARG
    assert init([3, 3]) == sv.SV_ERR_INVALID_ARG            # not strictly increasing
    assert init([0, 3]) == sv.SV_ERR_INVALID_ARG
    assert init([1, 5000]) == sv.SV_ERR_INVALID_ARG          # above SV_MAX_DRAFTS
    assert init(list(range(1, 18))) == sv.SV_ERR_INVALID_ARG # more than SV_MAX_TIERS
    assert init([1, 3], beta=0.0) == sv.SV_ERR_INVALID_ARG
    assert init([1, 3], beta=1.5) == sv.SV_ERR_INVALID_ARG
    assert init([1, 3], ema0=-1.0) == sv.SV_ERR_INVALID_ARG
    assert init([1, 3], ema0=float("nan")) == sv.SV_ERR_INVALID_ARG
    assert init([1, 3, 7]) == sv.SV_OK
    assert L.sv_adaptive_update(ctypes.byref(s), -0.5) == sv.SV_ERR_INVALID_ARG
    assert L.sv_adaptive_update(ctypes.byref(s), float("inf")) == sv.SV_ERR_INVALID_ARG
    assert L.sv_adaptive_update(None, 1.0) == sv.SV_ERR_INVALID_ARG
    assert L.sv_adaptive_update(ctypes.byref(s), 2.0) == sv.SV_OK and s.k == 1
