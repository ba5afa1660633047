"""The kernel's final-sample CDF against the oracle's.

Once a rejection-sampling call has completed, its workspace begins with the
masses of r (after a rejection) and of p over consecutive SV_SAMPLE_BLOCK-token
blocks of the row pair each sequence's final sample was drawn from: their
running sums are the CDF the kernel inverted, at every block end.  Their
distance from the oracle's fp64 CDF of the same row pair, both normalised by
their totals, is the error that decides which final samples can differ from
the oracle's.  The oracle flags a draw as a tie when u*S lies within
SAMPLE_BAND_SCALE * sqrt(sum p^2 + sum q^2) probability mass of an interval
end; the measured error must stay below half of that band everywhere, so
that every unflagged draw is decided the same way with room to spare."""
import numpy as np
import pytest
import torch
from scipy import special

import proposal_sv_verify_amd as sv
from proposal_sv_verify_amd import workloads as W
from gpu_util import dev, host, say, to_dev

pytestmark = pytest.mark.gpu

BLOCK = 1024


def _f64(rows):
    return (W.bf16_bits_to_f32(rows) if rows.dtype == np.uint16 else rows).astype(np.float64)


def _cdf_error(orc, wl):
    """Per sequence: (max |F_kernel - F_oracle| over block ends in probability
    mass, the sequence's tie band)."""
    B, K1, V = wl["target"].shape
    K, T = K1 - 1, wl["temperature"]
    L = sv.load()
    ws = torch.empty(L.sv_rejection_workspace_bytes(B, K, V), dtype=torch.uint8, device=dev())
    g = sv.verify_rejection(to_dev(wl["target"]), to_dev(wl["draft_logits"]), to_dev(wl["draft"]),
                            to_dev(wl["uniforms"]), T, ws=ws)
    acc = host(g["accepted"])
    nblk = (V + BLOCK - 1) // BLOCK
    masses = host(ws[:B * nblk * 16]).view(np.float64).reshape(B, nblk, 2)
    ends = np.minimum(np.arange(1, nblk + 1) * BLOCK, V) - 1
    err, band = np.zeros(B), np.zeros(B)
    for b in range(B):
        n = int(acc[b])
        residual = n < K
        trow = wl["target"][b, n]
        drow = wl["draft_logits"][b, n] if residual else None
        C, S = orc.sample_cdf(trow, drow, T)
        p = special.softmax(_f64(trow) / T)
        sq = (p * p).sum()
        col = 1
        if residual:
            q = special.softmax(_f64(drow) / T)
            sq += (q * q).sum()
            if masses[b, :, 0].sum() > 0.0:
                col = 0
        kc = np.cumsum(masses[b, :, col])
        err[b] = np.abs(kc / kc[-1] - C[ends] / S).max() * S
        band[b] = orc.SAMPLE_BAND_SCALE * np.sqrt(sq)
    return err, band


CASES = [("workload seed %d" % s, dict(W.REJECTION), s) for s in range(5)] + [
    ("bf16 top-50 masked", dict(B=24, K=4, V=50000, sigma=2.0, noise_sigma=0.7, temperature=1.0,
                                top_k=50), 11),
    ("f32 T 0.7", dict(B=24, K=4, V=60000, sigma=2.0, noise_sigma=0.7, temperature=0.7, dtype="f32"), 12),
    ("bf16 T 1.3", dict(B=24, K=4, V=60000, sigma=2.0, noise_sigma=0.7, temperature=1.3), 13),
    ("bf16 N(0, 1)", dict(B=24, K=4, V=151936, sigma=1.0, noise_sigma=0.3, temperature=1.0), 14),
    ("bf16 T 0.3", dict(B=24, K=4, V=32000, sigma=2.0, noise_sigma=0.7, temperature=0.3), 15),
    ("f32 T 1", dict(B=24, K=4, V=32000, sigma=1.0, noise_sigma=0.7, temperature=1.0, dtype="f32"), 16),
    ("f32 top-4000 T 0.7", dict(B=24, K=4, V=50000, sigma=2.0, noise_sigma=0.7, temperature=0.7,
                                dtype="f32", top_k=4000), 17),
    ("bf16 K 0", dict(B=48, K=0, V=128256, sigma=2.0, noise_sigma=0.5, temperature=1.0), 18),
    ("bf16 wide draft", dict(B=24, K=6, V=128256, sigma=3.0, noise_sigma=2.0, temperature=1.0), 19),
]


@pytest.mark.parametrize("label,kw,salt", CASES, ids=[c[0] for c in CASES])
def test_final_sample_cdf_error_within_half_band(orc, label, kw, salt):
    wl = W.rejection_workload(**kw, seed=W.seed_for(3, salt=500 + salt))
    say("sample cdf", label)
    err, band = _cdf_error(orc, wl)
    ratio = err / band
    say("sample cdf %s: max |dF| %.3g of mass, band %.3g..%.3g, dF/band median %.3g max %.3g"
        % (label, err.max(), band.min(), band.max(), np.median(ratio), ratio.max()))
    assert ratio.max() < 0.5, "CDF error %.3g of the band" % ratio.max()
