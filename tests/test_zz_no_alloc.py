"""sv_verify_rejection_noalloc -- the rejection verifier on the library's own
per-GPU device array, for callers that cannot allocate -- gives exactly the
results of sv_verify_rejection with a caller workspace: the same kernels on
the same inputs.  Two calls in a row, the second on a smaller input, both
through the C ABI; the array keeps the first call's contents when the second
starts."""
import ctypes

import numpy as np
import pytest
import torch

import proposal_sv_verify_amd as sv
from proposal_sv_verify_amd import workloads as W
from gpu_util import check_rejection, dev, host, say, to_dev

pytestmark = pytest.mark.gpu

CASES = [("B64 K5 V128256 bf16", dict(W.REJECTION), 900),
         ("B7 K3 V5001 f32 T0.8 ragged", dict(B=7, K=3, V=5001, sigma=2.0, noise_sigma=0.7,
                                               temperature=0.8, dtype="f32"), 901)]


def _noalloc(L, t, d, x, dl, u, T, B, K, V, stats):
    acc = torch.full((B,), -9, dtype=torch.int32, device=dev())
    emi = torch.full((B, K + 1), -9, dtype=torch.int32, device=dev())
    pd = torch.full((B, K), -9.0, dtype=torch.float32, device=dev())
    qd = torch.full((B, K), -9.0, dtype=torch.float32, device=dev())
    fl = torch.full((B,), -9, dtype=torch.int32, device=dev())
    code = sv.SV_BF16 if t.dtype == torch.bfloat16 else sv.SV_F32
    st = L.sv_verify_rejection_noalloc(
        t.data_ptr(), d.data_ptr() if K > 0 else None, code, t.stride(1), x.data_ptr(),
        dl.data_ptr() if dl is not None else None, u.data_ptr(), ctypes.c_float(T), B, K, V,
        acc.data_ptr(), emi.data_ptr(), pd.data_ptr(), qd.data_ptr(), fl.data_ptr(),
        stats.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == sv.SV_OK, L.sv_last_error_message()
    return dict(accepted=acc, emitted=emi, p_draft=pd, q_draft=qd, flags=fl)


def test_noalloc_equals_workspace_call_twice_smaller_second(orc):
    L = sv.load()
    for label, kw, salt in CASES:
        wl = W.rejection_workload(**kw, seed=W.seed_for(3, salt=salt))
        B, K1, V = wl["target"].shape
        K, T = K1 - 1, wl["temperature"]
        dl = np.clip(np.arange(B) % (K + 2), 0, K).astype(np.int32) if B < 64 else None
        say("noalloc", label)
        t, d, x, u = to_dev(wl["target"]), to_dev(wl["draft_logits"]), to_dev(wl["draft"]), \
            to_dev(wl["uniforms"])
        dlg = to_dev(dl) if dl is not None else None
        s_ref = torch.zeros(3 + K, dtype=torch.int64, device=dev())
        s_na = torch.zeros(3 + K, dtype=torch.int64, device=dev())
        ref = sv.verify_rejection(t, d, x, u, T, dlg, stats=s_ref)
        got = _noalloc(L, t, d, x, dlg, u, T, B, K, V, s_na)
        for k in ("accepted", "emitted", "p_draft", "q_draft", "flags"):
            np.testing.assert_array_equal(host(got[k]), host(ref[k]), err_msg="%s %s" % (label, k))
        np.testing.assert_array_equal(host(s_na), host(s_ref), err_msg="%s stats" % label)
        r = orc.verify_rejection(wl["target"], wl["draft_logits"], wl["draft"], wl["uniforms"], T, dl)
        check_rejection(got, r, label, max_flagged=max(2, B // 16))


def test_noalloc_rejects_a_call_above_the_array():
    """B 4096, K 8, V 151936 needs more workspace than the array holds: the
    call fails on the host, before any launch, and writes nothing."""
    L = sv.load()
    B, K, V = 4096, 8, 151936
    assert L.sv_rejection_workspace_bytes(B, K, V) > sv.NOALLOC_WORKSPACE_BYTES
    acc = torch.full((B,), -9, dtype=torch.int32, device=dev())
    fake = torch.zeros(16, dtype=torch.int64, device=dev())
    st = L.sv_verify_rejection_noalloc(fake.data_ptr(), fake.data_ptr(), sv.SV_BF16, V,
                                       fake.data_ptr(), None, fake.data_ptr(), ctypes.c_float(1.0),
                                       B, K, V, acc.data_ptr(), acc.data_ptr(), None, None, None,
                                       None, torch.cuda.current_stream().cuda_stream)
    assert st == sv.SV_ERR_UNSUPPORTED
    assert b"device array" in L.sv_last_error_message()
    assert (host(acc) == -9).all()
