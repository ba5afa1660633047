"""Helpers shared by the GPU tests: host<->device moves and the tie-aware
comparison of rejection-sampling results."""
import sys

import numpy as np
import torch


def say(*a):
    """Name the case before each GPU step (flushed, so a crash still shows it)."""
    print("[gpu]", *a, file=sys.stderr, flush=True)


def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda:0")


def to_dev(a):
    """numpy -> device tensor; uint16 arrays are bf16 bit patterns."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev()).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def check_rejection(gpu, ref, label="", max_flagged=None):
    """Decisions agree except where the oracle flags a tie; reported
    probabilities agree within 1e-5 relative.  max_flagged bounds the
    sequences the oracle flags (skipped decisions must stay few for the
    comparison to mean anything).  Returns (#flagged, #mismatch)."""
    acc_g, acc_r = host(gpu["accepted"]), ref["accepted"]
    emi_g, emi_r = host(gpu["emitted"]), ref["emitted"]
    B = len(acc_r)
    mism = 0
    for b in range(B):
        if acc_g[b] != acc_r[b]:
            assert ref["accept_tie"][b], "%s seq %d: accepted %d vs oracle %d (no tie)" % (
                label, b, acc_g[b], acc_r[b])
            mism += 1
            continue
        n = acc_r[b]
        assert np.array_equal(emi_g[b, :n], emi_r[b, :n]), "%s seq %d drafts" % (label, b)
        assert (emi_g[b, n + 1:] == -1).all(), "%s seq %d padding" % (label, b)
        if emi_g[b, n] != emi_r[b, n]:
            assert ref["sample_tie"][b], "%s seq %d: sampled %d vs oracle %d (no tie)" % (
                label, b, emi_g[b, n], emi_r[b, n])
            mism += 1
    if "p_draft" in gpu:
        for k in ("p_draft", "q_draft"):
            g = host(gpu[k]).astype(np.float64)
            r = ref[k]
            np.testing.assert_allclose(g, r, rtol=1e-5, atol=0.0, err_msg="%s %s" % (label, k))
    flagged = int((ref["accept_tie"] | ref["sample_tie"]).sum())
    if max_flagged is not None:
        assert flagged <= max_flagged, "%s: %d of %d sequences flagged (at most %d allowed)" % (
            label, flagged, B, max_flagged)
    return flagged, mism
