"""The C ABI library: it loads, exports every symbol the header declares, and
rejects invalid arguments on the host before any HIP call (no GPU needed:
none of these calls reaches a kernel launch or a device query)."""
import ctypes
import os
import re
import subprocess

import pytest

import proposal_sv_verify_amd as sv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specverify.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sv.LIB_PATH):
        from proposal_sv_verify_amd import build
        build.build()
    return sv.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sv_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert set(declared) == set(sv.EXPORTS)
    out = subprocess.check_output(["nm", "-D", "--defined-only", sv.LIB_PATH], text=True)
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    missing = [f for f in declared if f not in exported]
    assert not missing, missing
    for f in declared:
        assert getattr(lib, f) is not None


def test_version_and_status_strings(lib):
    assert lib.sv_abi_version() == 1
    assert lib.sv_status_string(0) == b"SV_OK"
    assert lib.sv_status_string(3) == b"SV_ERR_WORKSPACE"
    assert lib.sv_status_string(99) == b"SV_ERR_UNKNOWN"


FAKE = 0x10000          # a 64 KiB-aligned non-null address, never dereferenced
BIG = 1 << 40


def _greedy(lib, **kw):
    a = dict(logits=FAKE, dtype=1, row_stride=100, draft=FAKE, draft_len=None, B=2, K=3, V=100,
             acc=FAKE, emi=FAKE, amx=None, flags=None, stats=None, ws=FAKE, wsb=BIG, stream=None)
    a.update(kw)
    return lib.sv_verify_greedy(a["logits"], a["dtype"], a["row_stride"], a["draft"],
                                a["draft_len"], a["B"], a["K"], a["V"], a["acc"], a["emi"],
                                a["amx"], a["flags"], a["stats"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), sv.SV_ERR_INVALID_ARG),
    (dict(K=-1), sv.SV_ERR_INVALID_ARG),
    (dict(V=0), sv.SV_ERR_INVALID_ARG),
    (dict(K=5000), sv.SV_ERR_UNSUPPORTED),
    (dict(dtype=7), sv.SV_ERR_INVALID_ARG),
    (dict(logits=None), sv.SV_ERR_INVALID_ARG),
    (dict(logits=FAKE + 1), sv.SV_ERR_INVALID_ARG),     # bf16 needs 2-byte alignment
    (dict(row_stride=99), sv.SV_ERR_INVALID_ARG),
    (dict(draft=None), sv.SV_ERR_INVALID_ARG),
    (dict(acc=None), sv.SV_ERR_INVALID_ARG),
    (dict(ws=None), sv.SV_ERR_WORKSPACE),
    (dict(ws=FAKE + 8), sv.SV_ERR_WORKSPACE),
    (dict(wsb=16), sv.SV_ERR_WORKSPACE),
])
def test_greedy_rejects_bad_arguments(lib, kw, status):
    assert _greedy(lib, **kw) == status
    assert lib.sv_last_error_message()


def test_workspace_sizes(lib):
    assert lib.sv_greedy_workspace_bytes(0, 3, 10) == 0
    g = lib.sv_greedy_workspace_bytes(256, 8, 151936)
    assert g >= 4 * 256 * 9 and g % 256 == 0
    assert lib.sv_rejection_workspace_bytes(64, 5, 128256) > 0
    assert lib.sv_tree_workspace_bytes(32, 64, 128256) > 0
    # more rows than workgroups wanted -> one segment per row
    assert lib.sv_set_tuning(1, 64) == 0
    small = lib.sv_greedy_workspace_bytes(256, 8, 151936)
    assert lib.sv_set_tuning(1, 0) == 0
    assert small <= g
    assert lib.sv_set_tuning(42, 1) == sv.SV_ERR_INVALID_ARG


def test_rejection_rejects_bad_arguments(lib):
    def call(**kw):
        a = dict(t=FAKE, d=FAKE, dtype=1, rs=100, draft=FAKE, dl=None, u=FAKE, T=1.0, B=2, K=3,
                 V=100, acc=FAKE, emi=FAKE, pd=None, qd=None, fl=None, st=None, ws=FAKE, wsb=BIG)
        a.update(kw)
        return lib.sv_verify_rejection(a["t"], a["d"], a["dtype"], a["rs"], a["draft"], a["dl"],
                                       a["u"], a["T"], a["B"], a["K"], a["V"], a["acc"], a["emi"],
                                       a["pd"], a["qd"], a["fl"], a["st"], a["ws"], a["wsb"], None)
    assert call(T=0.0) == sv.SV_ERR_INVALID_ARG
    assert call(T=float("nan")) == sv.SV_ERR_INVALID_ARG
    assert call(T=float("inf")) == sv.SV_ERR_INVALID_ARG
    assert call(T=-1.0) == sv.SV_ERR_INVALID_ARG
    assert call(u=None) == sv.SV_ERR_INVALID_ARG
    assert call(d=None) == sv.SV_ERR_INVALID_ARG
    assert call(wsb=0) == sv.SV_ERR_WORKSPACE
    assert call(emi=None) == sv.SV_ERR_INVALID_ARG


def test_tree_rejects_bad_arguments(lib):
    def call(**kw):
        a = dict(l=FAKE, dtype=0, rs=100, par=FAKE, tok=FAKE, B=2, N=8, V=100, acc=FAKE,
                 path=FAKE, emi=FAKE, amx=None, fl=None, ws=FAKE, wsb=BIG)
        a.update(kw)
        return lib.sv_verify_tree(a["l"], a["dtype"], a["rs"], a["par"], a["tok"], a["B"], a["N"],
                                  a["V"], a["acc"], a["path"], a["emi"], a["amx"], a["fl"],
                                  a["ws"], a["wsb"], None)
    assert call(N=0) == sv.SV_ERR_INVALID_ARG
    assert call(N=2000) == sv.SV_ERR_UNSUPPORTED
    assert call(par=None) == sv.SV_ERR_INVALID_ARG
    assert call(path=None) == sv.SV_ERR_INVALID_ARG
    assert call(l=FAKE + 2) == sv.SV_ERR_INVALID_ARG       # fp32 needs 4-byte alignment
    assert call(wsb=1) == sv.SV_ERR_WORKSPACE


def test_ngram_rejects_bad_arguments(lib):
    def call(**kw):
        a = dict(tok=FAKE, stride=100, lens=FAKE, B=2, nmin=2, nmax=5, K=8, prop=FAKE,
                 plen=FAKE)
        a.update(kw)
        return lib.sv_ngram_propose(a["tok"], a["stride"], a["lens"], a["B"], a["nmin"],
                                    a["nmax"], a["K"], a["prop"], a["plen"], None, None, None,
                                    None)
    assert call(nmin=0) == sv.SV_ERR_INVALID_ARG
    assert call(nmin=6) == sv.SV_ERR_INVALID_ARG
    assert call(nmax=40) == sv.SV_ERR_UNSUPPORTED
    assert call(K=-1) == sv.SV_ERR_INVALID_ARG
    assert call(K=5000) == sv.SV_ERR_UNSUPPORTED
    assert call(stride=0) == sv.SV_ERR_INVALID_ARG
    assert call(stride=1 << 27) == sv.SV_ERR_UNSUPPORTED
    assert call(tok=FAKE + 2) == sv.SV_ERR_INVALID_ARG
    assert call(lens=None) == sv.SV_ERR_INVALID_ARG
    assert call(prop=None) == sv.SV_ERR_INVALID_ARG
    assert call(B=0) == sv.SV_ERR_INVALID_ARG


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(sv, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        sv.load(str(tmp_path / "nope.so"))


def test_shard_calls_reject_bad_arguments(lib):
    def shard(**kw):
        a = dict(l=FAKE, dtype=1, rs=100, rows=8, V=100, off=0, out=FAKE, ws=FAKE, wsb=BIG)
        a.update(kw)
        return lib.sv_argmax_shard(a["l"], a["dtype"], a["rs"], a["rows"], a["V"], a["off"],
                                   a["out"], a["ws"], a["wsb"], None)
    assert shard(rows=0) == sv.SV_ERR_INVALID_ARG
    assert shard(V=0) == sv.SV_ERR_INVALID_ARG
    assert shard(off=-1) == sv.SV_ERR_INVALID_ARG
    assert shard(off=(1 << 30) - 50) == sv.SV_ERR_UNSUPPORTED     # shard past SV_MAX_V
    assert shard(rs=99) == sv.SV_ERR_INVALID_ARG
    assert shard(out=None) == sv.SV_ERR_INVALID_ARG
    assert shard(out=FAKE + 4) == sv.SV_ERR_INVALID_ARG            # partials are 8-byte aligned
    assert shard(wsb=8) == sv.SV_ERR_WORKSPACE
    assert lib.sv_argmax_shard_workspace_bytes(0, 100) == 0
    assert lib.sv_argmax_shard_workspace_bytes(64, 32000) > 0

    def greedy(**kw):
        a = dict(parts=FAKE, P=4, draft=FAKE, dl=None, B=2, K=3, V=100, acc=FAKE, emi=FAKE)
        a.update(kw)
        return lib.sv_verify_greedy_partials(a["parts"], a["P"], a["draft"], a["dl"], a["B"],
                                             a["K"], a["V"], a["acc"], a["emi"], None, None,
                                             None, None)
    assert greedy(P=0) == sv.SV_ERR_INVALID_ARG
    assert greedy(P=5000) == sv.SV_ERR_UNSUPPORTED
    assert greedy(parts=None) == sv.SV_ERR_INVALID_ARG
    assert greedy(parts=FAKE + 4) == sv.SV_ERR_INVALID_ARG
    assert greedy(B=0) == sv.SV_ERR_INVALID_ARG
    assert greedy(draft=None) == sv.SV_ERR_INVALID_ARG
    assert greedy(emi=None) == sv.SV_ERR_INVALID_ARG

    def tree(**kw):
        a = dict(parts=FAKE, P=2, par=FAKE, tok=FAKE, B=2, N=8, V=100, acc=FAKE, path=FAKE,
                 emi=FAKE)
        a.update(kw)
        return lib.sv_verify_tree_partials(a["parts"], a["P"], a["par"], a["tok"], a["B"],
                                           a["N"], a["V"], a["acc"], a["path"], a["emi"], None,
                                           None, None)
    assert tree(P=0) == sv.SV_ERR_INVALID_ARG
    assert tree(N=2000) == sv.SV_ERR_UNSUPPORTED
    assert tree(tok=None) == sv.SV_ERR_INVALID_ARG
    assert tree(path=None) == sv.SV_ERR_INVALID_ARG
    for f in (shard, greedy, tree):
        assert lib.sv_last_error_message()


def test_rejection_shard_calls_reject_bad_arguments(lib):
    F = 1.0

    def stats(**kw):
        a = dict(t=FAKE, d=FAKE, dtype=1, rs=128, draft=FAKE, dl=None, T=F, B=2, K=3, V=100,
                 off=0, out=FAKE, ws=FAKE, wsb=BIG)
        a.update(kw)
        return lib.sv_rejection_shard_stats(a["t"], a["d"], a["dtype"], a["rs"], a["draft"],
                                            a["dl"], a["T"], a["B"], a["K"], a["V"], a["off"],
                                            a["out"], a["ws"], a["wsb"], None)
    assert stats(B=0) == sv.SV_ERR_INVALID_ARG
    assert stats(off=-1) == sv.SV_ERR_INVALID_ARG
    assert stats(off=(1 << 30) - 50) == sv.SV_ERR_UNSUPPORTED
    assert stats(rs=99) == sv.SV_ERR_INVALID_ARG
    assert stats(draft=None) == sv.SV_ERR_INVALID_ARG
    assert stats(T=0.0) == sv.SV_ERR_INVALID_ARG
    assert stats(T=float("inf")) == sv.SV_ERR_INVALID_ARG
    assert stats(out=FAKE + 4) == sv.SV_ERR_INVALID_ARG
    assert stats(wsb=8) == sv.SV_ERR_WORKSPACE
    assert lib.sv_rejection_shard_workspace_bytes(0, 3, 100) == 0
    assert lib.sv_rejection_shard_workspace_bytes(64, 5, 16032) > 0

    def decide(**kw):
        a = dict(parts=FAKE, P=4, draft=FAKE, dl=None, u=FAKE, T=F, B=2, K=3, V=100, acc=FAKE,
                 state=FAKE)
        a.update(kw)
        return lib.sv_verify_rejection_partials(a["parts"], a["P"], a["draft"], a["dl"], a["u"],
                                                a["T"], a["B"], a["K"], a["V"], a["acc"], None,
                                                None, None, None, a["state"], None)
    assert decide(P=0) == sv.SV_ERR_INVALID_ARG
    assert decide(P=sv.MAX_REJECT_SHARDS + 1) == sv.SV_ERR_UNSUPPORTED
    assert decide(parts=None) == sv.SV_ERR_INVALID_ARG
    assert decide(parts=FAKE + 4) == sv.SV_ERR_INVALID_ARG
    assert decide(u=None) == sv.SV_ERR_INVALID_ARG
    assert decide(T=-1.0) == sv.SV_ERR_INVALID_ARG
    assert decide(state=None) == sv.SV_ERR_INVALID_ARG
    assert decide(state=FAKE + 4) == sv.SV_ERR_INVALID_ARG
    assert decide(acc=None) == sv.SV_ERR_INVALID_ARG

    def mass(**kw):
        a = dict(t=FAKE, d=FAKE, dtype=1, rs=128, state=FAKE, T=F, B=2, K=3, V=100, out=FAKE,
                 ws=FAKE, wsb=BIG)
        a.update(kw)
        return lib.sv_rejection_shard_mass(a["t"], a["d"], a["dtype"], a["rs"], a["state"], a["T"],
                                           a["B"], a["K"], a["V"], a["out"], a["ws"], a["wsb"],
                                           None)
    assert mass(state=None) == sv.SV_ERR_INVALID_ARG
    assert mass(out=None) == sv.SV_ERR_INVALID_ARG
    assert mass(K=-1) == sv.SV_ERR_INVALID_ARG
    assert mass(wsb=8) == sv.SV_ERR_WORKSPACE

    def sample(**kw):
        a = dict(t=FAKE, d=FAKE, dtype=1, rs=128, draft=FAKE, u=FAKE, state=FAKE, masses=FAKE,
                 P=3, shard=1, T=F, B=2, K=3, V=100, off=0, emi=FAKE, ws=FAKE, wsb=BIG)
        a.update(kw)
        return lib.sv_rejection_shard_sample(a["t"], a["d"], a["dtype"], a["rs"], a["draft"],
                                             a["u"], a["state"], a["masses"], a["P"], a["shard"],
                                             a["T"], a["B"], a["K"], a["V"], a["off"], a["emi"],
                                             a["ws"], a["wsb"], None)
    assert sample(shard=3) == sv.SV_ERR_INVALID_ARG
    assert sample(shard=-1) == sv.SV_ERR_INVALID_ARG
    assert sample(P=17) == sv.SV_ERR_UNSUPPORTED
    assert sample(masses=FAKE + 4) == sv.SV_ERR_INVALID_ARG
    assert sample(emi=None) == sv.SV_ERR_INVALID_ARG
    assert sample(u=None) == sv.SV_ERR_INVALID_ARG
    assert sample(wsb=8) == sv.SV_ERR_WORKSPACE
    for f in (stats, decide, mass, sample):
        assert lib.sv_last_error_message()


def test_suffix_rejects_bad_arguments(lib):
    def call(**kw):
        a = dict(tok=FAKE, stride=64, lens=FAKE, B=2, hist=FAKE, H=100, mmin=1, mmax=8, K=4,
                 mp=0.1, prop=FAKE, plen=FAKE, score=FAKE, ws=FAKE, wsb=BIG)
        a.update(kw)
        return lib.sv_suffix_propose(a["tok"], a["stride"], a["lens"], a["B"], a["hist"], a["H"],
                                     a["mmin"], a["mmax"], a["K"], a["mp"], a["prop"], a["plen"],
                                     a["score"], None, None, None, a["ws"], a["wsb"], None)
    assert call(B=0) == sv.SV_ERR_INVALID_ARG
    assert call(mmin=0) == sv.SV_ERR_INVALID_ARG
    assert call(mmin=5, mmax=4) == sv.SV_ERR_INVALID_ARG
    assert call(mmax=33) == sv.SV_ERR_UNSUPPORTED
    assert call(K=-1) == sv.SV_ERR_INVALID_ARG
    assert call(K=33) == sv.SV_ERR_UNSUPPORTED
    assert call(mp=-0.1) == sv.SV_ERR_INVALID_ARG
    assert call(mp=1.5) == sv.SV_ERR_INVALID_ARG
    assert call(mp=float("nan")) == sv.SV_ERR_INVALID_ARG
    assert call(stride=0) == sv.SV_ERR_INVALID_ARG
    assert call(stride=(1 << 26) + 1) == sv.SV_ERR_UNSUPPORTED
    assert call(H=-1) == sv.SV_ERR_INVALID_ARG
    assert call(hist=None) == sv.SV_ERR_INVALID_ARG            # H > 0 needs a history
    assert call(prop=None) == sv.SV_ERR_INVALID_ARG
    assert call(plen=None) == sv.SV_ERR_INVALID_ARG
    assert call(score=FAKE + 4) == sv.SV_ERR_INVALID_ARG
    assert call(wsb=8) == sv.SV_ERR_WORKSPACE
    assert lib.sv_last_error_message()
    assert lib.sv_suffix_workspace_bytes(0, 64, 0) == 0
    assert lib.sv_suffix_workspace_bytes(64, 8192, 262144) > 64 * 17 * 1024


def test_rejection_probs_rejects_bad_arguments(lib):
    def call(**kw):
        a = dict(t=FAKE, d=FAKE, rs=128, draft=FAKE, dl=None, u=FAKE, B=2, K=3, V=100, acc=FAKE,
                 emi=FAKE, ws=FAKE, wsb=BIG)
        a.update(kw)
        return lib.sv_verify_rejection_probs(a["t"], a["d"], a["rs"], a["draft"], a["dl"], a["u"],
                                             a["B"], a["K"], a["V"], a["acc"], a["emi"], None, None,
                                             None, None, a["ws"], a["wsb"], None)
    assert call(B=0) == sv.SV_ERR_INVALID_ARG
    assert call(rs=99) == sv.SV_ERR_INVALID_ARG
    assert call(draft=None) == sv.SV_ERR_INVALID_ARG
    assert call(u=None) == sv.SV_ERR_INVALID_ARG
    assert call(emi=None) == sv.SV_ERR_INVALID_ARG
    assert call(wsb=8) == sv.SV_ERR_WORKSPACE
    assert lib.sv_last_error_message()


def test_read_probe_rejects_bad_arguments(lib):
    assert lib.sv_read_probe(None, 1024, FAKE, None) == sv.SV_ERR_INVALID_ARG
    assert lib.sv_read_probe(FAKE, 1024, None, None) == sv.SV_ERR_INVALID_ARG
    assert lib.sv_read_probe(FAKE, 1000, FAKE, None) == sv.SV_ERR_INVALID_ARG   # not a multiple of 16
    assert lib.sv_read_probe(FAKE + 4, 1024, FAKE, None) == sv.SV_ERR_INVALID_ARG
    assert lib.sv_read_probe(FAKE, 0, FAKE, None) == sv.SV_ERR_INVALID_ARG


def test_tuning_change_between_sizing_and_call(lib):
    """A call plans from one reading of the tuning: a workspace sized under
    one setting is either enough for the call under another (the call gets
    past the workspace check and stops only at the missing device) or
    rejected with SV_ERR_WORKSPACE -- never accepted and overrun.  The
    final-sample masses the shard calls hand over sit at the start of the
    workspace, whatever the setting."""
    B, K, V = 64, 5, 128256
    need_default = lib.sv_rejection_workspace_bytes(B, K, V)

    def call(wsb):
        return lib.sv_verify_rejection(FAKE, FAKE, 1, V, FAKE, None, FAKE, 1.0, B, K, V, FAKE, FAKE,
                                       None, None, None, None, FAKE, wsb, None)
    try:
        assert lib.sv_set_tuning(sv.TUNE_TARGET_WORKGROUPS, 1 << 16) == 0   # more pieces per row
        need_more = lib.sv_rejection_workspace_bytes(B, K, V)
        assert need_more > need_default
        assert call(need_default) == sv.SV_ERR_WORKSPACE
        assert call(need_more) not in (sv.SV_OK, sv.SV_ERR_WORKSPACE, sv.SV_ERR_INVALID_ARG)
        assert lib.sv_set_tuning(sv.TUNE_TARGET_WORKGROUPS, 64) == 0        # one piece per row
        need_less = lib.sv_rejection_workspace_bytes(B, K, V)
        assert need_less < need_default
        assert call(need_default) not in (sv.SV_OK, sv.SV_ERR_WORKSPACE, sv.SV_ERR_INVALID_ARG)
        assert call(need_less - 256) == sv.SV_ERR_WORKSPACE
        # the masses (B * ceil(V / 1024) records of 16 bytes) fit in every plan's workspace
        masses = B * ((V + 1023) // 1024) * 16
        assert need_less >= masses and need_more >= masses
    finally:
        lib.sv_set_tuning(sv.TUNE_TARGET_WORKGROUPS, 0)
    assert lib.sv_rejection_workspace_bytes(B, K, V) == need_default


def test_tuning_is_safe_to_change_from_threads(lib):
    """Setting the tuning while other threads size workspaces: every size
    returned is one of the sizes a single setting gives."""
    import threading
    B, K, V = 64, 5, 128256
    sizes = set()
    for w in (512, 2048):
        lib.sv_set_tuning(sv.TUNE_TARGET_WORKGROUPS, w)
        sizes.add(lib.sv_rejection_workspace_bytes(B, K, V))
    lib.sv_set_tuning(sv.TUNE_TARGET_WORKGROUPS, 0)
    seen = []
    stop = threading.Event()

    def reader():
        while not stop.is_set():
            seen.append(lib.sv_rejection_workspace_bytes(B, K, V))
    threads = [threading.Thread(target=reader) for _ in range(3)]
    for t in threads:
        t.start()
    try:
        for i in range(2000):
            lib.sv_set_tuning(sv.TUNE_TARGET_WORKGROUPS, 512 if i % 2 else 2048)
    finally:
        stop.set()
        for t in threads:
            t.join()
        lib.sv_set_tuning(sv.TUNE_TARGET_WORKGROUPS, 0)
    assert seen and set(seen) <= sizes


def test_noalloc_rejection_size_limit(lib):
    """The no-allocation rejection call rejects, on the host, a call whose
    workspace would not fit the library's device array, and validates its
    arguments like sv_verify_rejection."""
    B, K, V = 4096, 8, 151936
    assert lib.sv_rejection_workspace_bytes(B, K, V) > sv.NOALLOC_WORKSPACE_BYTES

    def call(**kw):
        a = dict(t=FAKE, d=FAKE, dtype=1, rs=V, draft=FAKE, dl=None, u=FAKE, T=1.0, B=B, K=K, V=V,
                 acc=FAKE, emi=FAKE)
        a.update(kw)
        return lib.sv_verify_rejection_noalloc(a["t"], a["d"], a["dtype"], a["rs"], a["draft"],
                                               a["dl"], a["u"], a["T"], a["B"], a["K"], a["V"],
                                               a["acc"], a["emi"], None, None, None, None, None)
    assert call() == sv.SV_ERR_UNSUPPORTED
    assert b"device array" in lib.sv_last_error_message()
    assert call(T=0.0) == sv.SV_ERR_INVALID_ARG
    assert call(u=None) == sv.SV_ERR_INVALID_ARG
    assert call(B=0) == sv.SV_ERR_INVALID_ARG
    # a call that fits gets past the size check (and stops at the missing device here)
    assert call(B=64, K=5, V=128256, rs=128256) not in (sv.SV_OK, sv.SV_ERR_INVALID_ARG,
                                                         sv.SV_ERR_WORKSPACE)


C_PROGRAM = r"""
#include "specverify.h"
#include <stdio.h>

int main(void)
{
    const int32_t tiers[3] = {1, 3, 7};
    sv_adaptive st;
    printf("%d %s\n", sv_abi_version(), sv_status_string(SV_ERR_INVALID_ARG));
    printf("%d\n", sv_greedy_workspace_bytes(4, 4, 32000) > 0);
    printf("%d\n", sv_rejection_workspace_bytes(64, 5, 128256) > 0);
    printf("%d\n", sv_verify_greedy(0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0) == SV_ERR_INVALID_ARG);
    if (sv_adaptive_init(&st, tiers, 3, 0.5, 0.0) != SV_OK)
        return 1;
    sv_adaptive_update(&st, 2.0);
    printf("%d %.2f\n", st.k, st.ema);
    return 0;
}
"""


def test_header_compiles_as_c99_and_links(lib, tmp_path):
    """The boundary is a C ABI: the header compiles as strict C99 with every
    warning an error, and a C program links against the library and calls
    the host-side entry points (version, status strings, workspace sizes,
    argument validation, the adaptive controller); nothing here needs a GPU."""
    import shutil
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "abi.c"
    src.write_text(C_PROGRAM)
    exe = tmp_path / "abi"
    # the library by path (a sanitizer build has another name, and its
    # runtime symbols come from a preloaded library)
    libdir = os.path.dirname(os.path.abspath(sv.LIB_PATH))
    subprocess.check_call([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I",
                           os.path.dirname(HEADER), str(src), os.path.abspath(sv.LIB_PATH),
                           "-Wl,-rpath," + libdir, "-Wl,--allow-shlib-undefined", "-o", str(exe)])
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    assert out[0] == "%d SV_ERR_INVALID_ARG" % lib.sv_abi_version()
    assert out[1:4] == ["1", "1", "1"]
    assert out[4] == "3 1.00"                  # ema 0.5 * 2 = 1; smallest tier >= 2 * 1 is 3
