"""libspecverify: speculative-decoding verification and n-gram proposal on
AMD Instinct MI355X (gfx950).

Thin ctypes binding over the C ABI in ``include/specverify.h``.  It only
marshals arguments: it allocates outputs (and a cached scratch
workspace) with torch on the tensors' device and passes raw device
pointers and torch's current HIP stream.  Every step of the computation
runs in the library's kernels.  If ``libspecverify.so`` has not been built
the calls raise; there is no fallback path.

    verify_greedy(logits, draft, draft_len=None)          -> dict
    verify_rejection(target, draft_logits, draft, uniforms, temperature=1.0, draft_len=None)
    verify_tree(logits, parent, token)
    ngram_propose(tokens, lengths, n_min, n_max, K)
    suffix_propose(tokens, lengths, history, m_min, m_max, K, min_prob)
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# The library this package loads: the in-tree build, or another build of the
# same sources named by SPECVERIFY_LIBRARY (e.g. one with sanitized host code).
LIB_PATH = os.environ.get("SPECVERIFY_LIBRARY") or os.path.join(HERE, "libspecverify.so")

SV_OK, SV_ERR_INVALID_ARG, SV_ERR_UNSUPPORTED, SV_ERR_WORKSPACE, SV_ERR_HIP = range(5)
SV_F32, SV_BF16 = 0, 1
NOALLOC_WORKSPACE_BYTES = 8 << 20
FLAG_DRAFT_OOR, FLAG_BAD_LEN, FLAG_BAD_PARENT = 1, 2, 4
TUNE_TARGET_WORKGROUPS, TUNE_MIN_SEGMENT_BYTES = 1, 2

# every symbol include/specverify.h declares
EXPORTS = ("sv_abi_version", "sv_status_string", "sv_last_error_message", "sv_set_tuning",
           "sv_greedy_workspace_bytes", "sv_verify_greedy",
           "sv_rejection_workspace_bytes", "sv_verify_rejection", "sv_verify_rejection_probs",
           "sv_verify_rejection_noalloc",
           "sv_tree_workspace_bytes", "sv_verify_tree", "sv_ngram_propose",
           "sv_argmax_shard_workspace_bytes", "sv_argmax_shard",
           "sv_verify_greedy_partials", "sv_verify_tree_partials",
           "sv_rejection_shard_workspace_bytes", "sv_rejection_shard_stats",
           "sv_verify_rejection_partials", "sv_rejection_shard_mass", "sv_rejection_shard_sample",
           "sv_suffix_workspace_bytes", "sv_suffix_propose",
           "sv_read_probe", "sv_adaptive_init", "sv_adaptive_update")

# One sv_argmax_partial: the row's largest value and the lowest global token
# id holding it (NO_INDEX when the shard's row is all -inf).  The binding
# keeps partials in int64 tensors, one element per partial.
PARTIAL_DTYPE = np.dtype([("value", "<f4"), ("index", "<i4")])
NO_INDEX = 0x7FFFFFFF

# Sharded rejection sampling: sv_softmax_partial, sv_rejection_state and
# sv_sample_mass records, kept in float64 tensors of 2, 4 and 2 elements per
# record.
SOFT_PARTIAL_DTYPE = np.dtype([("z", "<f8"), ("m", "<f4"), ("lx", "<f4")])
STATE_DTYPE = np.dtype([("zt", "<f8"), ("zd", "<f8"), ("mt", "<f4"), ("md", "<f4"),
                        ("n", "<i4"), ("len", "<i4")])
MASS_DTYPE = np.dtype([("r", "<f8"), ("p", "<f8")])
MAX_REJECT_SHARDS = 16


class SpecVerifyError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s: %s" % (_STATUS.get(status, status), message))
        self.status = status


_STATUS = {0: "SV_OK", 1: "SV_ERR_INVALID_ARG", 2: "SV_ERR_UNSUPPORTED", 3: "SV_ERR_WORKSPACE",
           4: "SV_ERR_HIP"}

_lib = None
_lock = threading.Lock()


def load(path: str = LIB_PATH):
    """Load the shared library and declare its C signatures."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError("libspecverify.so is not built (%s); run "
                               "proposal_sv_verify_amd.build.build() first" % path)
        L = ctypes.CDLL(path)
        P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.sv_abi_version.restype = ctypes.c_int
        L.sv_abi_version.argtypes = []
        L.sv_status_string.restype = ctypes.c_char_p
        L.sv_status_string.argtypes = [ctypes.c_int]
        L.sv_last_error_message.restype = ctypes.c_char_p
        L.sv_last_error_message.argtypes = []
        L.sv_set_tuning.restype = ctypes.c_int
        L.sv_set_tuning.argtypes = [i32, i64]
        for f in ("sv_greedy_workspace_bytes", "sv_rejection_workspace_bytes",
                  "sv_tree_workspace_bytes"):
            getattr(L, f).restype = sz
            getattr(L, f).argtypes = [i32, i32, i32]
        L.sv_verify_greedy.restype = ctypes.c_int
        L.sv_verify_greedy.argtypes = [P, i32, i64, P, P, i32, i32, i32, P, P, P, P, P, P, sz, P]
        L.sv_verify_rejection.restype = ctypes.c_int
        L.sv_verify_rejection.argtypes = [P, P, i32, i64, P, P, P, ctypes.c_float, i32, i32, i32,
                                          P, P, P, P, P, P, P, sz, P]
        L.sv_verify_rejection_noalloc.restype = ctypes.c_int
        L.sv_verify_rejection_noalloc.argtypes = [P, P, i32, i64, P, P, P, ctypes.c_float, i32, i32,
                                                  i32, P, P, P, P, P, P, P]
        L.sv_verify_rejection_probs.restype = ctypes.c_int
        L.sv_verify_rejection_probs.argtypes = [P, P, i64, P, P, P, i32, i32, i32, P, P, P, P, P, P,
                                                P, sz, P]
        L.sv_verify_tree.restype = ctypes.c_int
        L.sv_verify_tree.argtypes = [P, i32, i64, P, P, i32, i32, i32, P, P, P, P, P, P, sz, P]
        L.sv_ngram_propose.restype = ctypes.c_int
        L.sv_ngram_propose.argtypes = [P, i64, P, i32, i32, i32, i32, P, P, P, P, P, P]
        L.sv_argmax_shard_workspace_bytes.restype = sz
        L.sv_argmax_shard_workspace_bytes.argtypes = [i32, i32]
        L.sv_argmax_shard.restype = ctypes.c_int
        L.sv_argmax_shard.argtypes = [P, i32, i64, i32, i32, i32, P, P, sz, P]
        L.sv_verify_greedy_partials.restype = ctypes.c_int
        L.sv_verify_greedy_partials.argtypes = [P, i32, P, P, i32, i32, i32, P, P, P, P, P, P]
        L.sv_rejection_shard_workspace_bytes.restype = sz
        L.sv_rejection_shard_workspace_bytes.argtypes = [i32, i32, i32]
        L.sv_rejection_shard_stats.restype = ctypes.c_int
        L.sv_rejection_shard_stats.argtypes = [P, P, i32, i64, P, P, ctypes.c_float, i32, i32, i32,
                                               i32, P, P, sz, P]
        L.sv_verify_rejection_partials.restype = ctypes.c_int
        L.sv_verify_rejection_partials.argtypes = [P, i32, P, P, P, ctypes.c_float, i32, i32, i32,
                                                   P, P, P, P, P, P, P]
        L.sv_rejection_shard_mass.restype = ctypes.c_int
        L.sv_rejection_shard_mass.argtypes = [P, P, i32, i64, P, ctypes.c_float, i32, i32, i32, P,
                                              P, sz, P]
        L.sv_rejection_shard_sample.restype = ctypes.c_int
        L.sv_rejection_shard_sample.argtypes = [P, P, i32, i64, P, P, P, P, i32, i32, ctypes.c_float,
                                                i32, i32, i32, i32, P, P, sz, P]
        L.sv_suffix_workspace_bytes.restype = sz
        L.sv_suffix_workspace_bytes.argtypes = [i32, i64, i64]
        L.sv_suffix_propose.restype = ctypes.c_int
        L.sv_suffix_propose.argtypes = [P, i64, P, i32, P, i64, i32, i32, i32, ctypes.c_double,
                                        P, P, P, P, P, P, P, sz, P]
        L.sv_read_probe.restype = ctypes.c_int
        L.sv_read_probe.argtypes = [P, sz, P, P]
        L.sv_adaptive_init.restype = ctypes.c_int
        L.sv_adaptive_init.argtypes = [P, P, i32, ctypes.c_double, ctypes.c_double]
        L.sv_adaptive_update.restype = ctypes.c_int
        L.sv_adaptive_update.argtypes = [P, ctypes.c_double]
        L.sv_verify_tree_partials.restype = ctypes.c_int
        L.sv_verify_tree_partials.argtypes = [P, i32, P, P, i32, i32, i32, P, P, P, P, P, P]
        _lib = L
        return L


def _check(status):
    if status != SV_OK:
        msg = load().sv_last_error_message().decode(errors="replace")
        raise SpecVerifyError(status, msg)


def set_tuning(key: int, value: int):
    _check(load().sv_set_tuning(key, value))


# ---------------------------------------------------------------- helpers

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device):
    return _torch().cuda.current_stream(device).cuda_stream


_ws_cache = {}


def workspace(nbytes: int, device, stream=None):
    """A device scratch buffer of at least nbytes, cached per (device,
    stream).  Calls on one stream are ordered, so sharing it there is safe."""
    torch = _torch()
    dev = torch.device(device)
    key = (dev.index, stream)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
        _ws_cache[key] = buf
    return buf


def _row_stride(x, rows_dims, name, single=None):
    """Elements between consecutive rows of a [.., V] tensor whose first
    rows_dims dims index evenly spaced rows, and whose last dim has unit
    stride.  Dims of size 1 do not constrain it (torch leaves their stride
    arbitrary); a single row takes `single` (the stride of a tensor it is
    passed with), else V."""
    if x.dim() != rows_dims + 1 or (x.size(-1) > 1 and x.stride(-1) != 1):
        raise ValueError("%s must be [%s, V] with unit stride along V" % (name, "..." * rows_dims))
    rs = None
    span = 1                                      # rows one step of dim d moves over
    for d in range(rows_dims - 1, -1, -1):
        if x.size(d) > 1:
            if rs is None:
                rs = x.stride(d) // span if x.stride(d) % span == 0 else -1
            if rs < 0 or x.stride(d) != rs * span:
                raise ValueError("%s rows must be evenly spaced; call .contiguous()" % name)
        span *= x.size(d)
    if rs is None:
        return x.size(-1) if single is None else single
    return rs


def _logits_args(x, name, rows_dims, single=None):
    """Validate a [.., V] logits tensor whose leading dims are evenly spaced
    rows; returns (dtype code, row stride in elements)."""
    torch = _torch()
    if not x.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if x.dtype == torch.bfloat16:
        code = SV_BF16
    elif x.dtype == torch.float32:
        code = SV_F32
    else:
        raise TypeError("%s must be float32 or bfloat16, got %s" % (name, x.dtype))
    return code, _row_stride(x, rows_dims, name, single)


def _rows_readable(t, rows, stride, name):
    """The C calls may read every entry of every [stride] row: check that
    the tensor's storage holds rows * stride elements from its first one."""
    have = t.untyped_storage().nbytes() // t.element_size() - t.storage_offset()
    if have < rows * stride:
        raise ValueError("%s: rows of stride %d need %d elements of storage from the first one, "
                         "have %d; pass .contiguous()" % (name, stride, rows * stride, have))


def _i32(t, shape, name):
    torch = _torch()
    if t is None:
        return None
    if t.dtype != torch.int32 or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError("%s must be a contiguous int32 tensor of shape %s" % (name, tuple(shape)))
    return t


# ---------------------------------------------------------------- calls

class Prepared:
    """One library call with its arguments and output tensors bound.  Calling
    it enqueues the kernels again on the stream it was prepared for and
    returns the same output dict (overwritten in place)."""

    def __init__(self, fn, args, out, keep):
        self._fn = fn
        self._args = args
        self.out = out
        # the raw pointers in args stay valid only while these tensors live
        self._keep = keep

    def __call__(self):
        _check(self._fn(*self._args))
        return self.out


def prepare_greedy(logits, draft, draft_len=None, *, want_argmax=True, stats=None):
    """Greedy verification.  logits [B, K+1, V] (f32/bf16), draft [B, K]
    int32, draft_len [B] int32 or None, stats int64 [3+K] or None
    (accumulated in place).  Outputs: accepted [B], emitted [B, K+1],
    argmax [B, K+1] (if want_argmax), flags [B]."""
    torch = _torch()
    L = load()
    code, rs = _logits_args(logits, "logits", 2)
    B, K1, V = logits.shape
    K = K1 - 1
    dev = logits.device
    _i32(draft, (B, K), "draft")
    _i32(draft_len, (B,), "draft_len")
    if stats is not None and (stats.dtype != torch.int64 or stats.numel() < 3 + K):
        raise ValueError("stats must be an int64 tensor of at least 3+K entries")
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    emi = torch.empty(B, K1, dtype=torch.int32, device=dev)
    amx = torch.empty(B, K1, dtype=torch.int32, device=dev) if want_argmax else None
    flg = torch.empty(B, dtype=torch.int32, device=dev)
    s = _stream(dev)
    ws = workspace(L.sv_greedy_workspace_bytes(B, K, V), dev, s)
    args = (logits.data_ptr(), code, rs, _ptr(draft), _ptr(draft_len), B, K, V, acc.data_ptr(),
            emi.data_ptr(), _ptr(amx), flg.data_ptr(), _ptr(stats), ws.data_ptr(), ws.numel(), s)
    out = dict(accepted=acc, emitted=emi, flags=flg)
    if want_argmax:
        out["argmax"] = amx
    return Prepared(L.sv_verify_greedy, args, out, (logits, draft, draft_len, stats, ws))


def verify_greedy(*a, **k):
    return prepare_greedy(*a, **k)()


def prepare_rejection(target, draft_logits, draft, uniforms, temperature=1.0, draft_len=None, *,
                      want_probs=True, stats=None, ws=None):
    """Rejection-sampling verification.  target [B, K+1, V], draft_logits
    [B, K, V] (same dtype and row spacing), draft [B, K] int32, uniforms
    [B, K+1] float32, ws: a uint8 device tensor to use as the workspace
    (default: the cached one).  Outputs: accepted, emitted, p_draft,
    q_draft, flags."""
    torch = _torch()
    L = load()
    code, rs = _logits_args(target, "target", 2)
    B, K1, V = target.shape
    K = K1 - 1
    dev = target.device
    if K > 0:
        code2, rs2 = _logits_args(draft_logits, "draft_logits", 2, single=rs)
        if code2 != code or rs2 != rs or tuple(draft_logits.shape) != (B, K, V):
            raise ValueError("draft_logits must be [B, K, V] with the target's dtype and row stride")
    _i32(draft, (B, K), "draft")
    _i32(draft_len, (B,), "draft_len")
    if uniforms.dtype != torch.float32 or not uniforms.is_contiguous() or \
            tuple(uniforms.shape) != (B, K1):
        raise ValueError("uniforms must be a contiguous float32 tensor [B, K+1]")
    if stats is not None and (stats.dtype != torch.int64 or stats.numel() < 3 + K):
        raise ValueError("stats must be an int64 tensor of at least 3+K entries")
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    emi = torch.empty(B, K1, dtype=torch.int32, device=dev)
    pd = torch.empty(B, K, dtype=torch.float32, device=dev) if want_probs else None
    qd = torch.empty(B, K, dtype=torch.float32, device=dev) if want_probs else None
    flg = torch.empty(B, dtype=torch.int32, device=dev)
    s = _stream(dev)
    need = L.sv_rejection_workspace_bytes(B, K, V)
    if ws is None:
        ws = workspace(need, dev, s)
    elif ws.dtype != torch.uint8 or not ws.is_contiguous() or ws.device != dev:
        raise ValueError("ws must be a contiguous uint8 tensor on the logits' device")
    args = (target.data_ptr(), _ptr(draft_logits) if K > 0 else None, code, rs, _ptr(draft),
            _ptr(draft_len), uniforms.data_ptr(), float(temperature), B, K, V, acc.data_ptr(),
            emi.data_ptr(), _ptr(pd), _ptr(qd), flg.data_ptr(), _ptr(stats), ws.data_ptr(),
            ws.numel(), s)
    out = dict(accepted=acc, emitted=emi, flags=flg)
    if want_probs:
        out["p_draft"], out["q_draft"] = pd, qd
    return Prepared(L.sv_verify_rejection, args, out,
                    (target, draft_logits, draft, draft_len, uniforms, stats, ws))


def verify_rejection(*a, **k):
    return prepare_rejection(*a, **k)()


def prepare_rejection_probs(target_probs, draft_probs, draft, uniforms, draft_len=None, *,
                            want_probs=True, stats=None):
    """Rejection sampling on given probabilities: target_probs [B, K+1, V]
    and draft_probs [B, K, V] float32 (each row over its sum; no
    temperature).  Outputs as prepare_rejection."""
    torch = _torch()
    L = load()
    if target_probs.dtype != torch.float32:
        raise TypeError("probabilities must be float32")
    _, rs = _logits_args(target_probs, "target_probs", 2)
    B, K1, V = target_probs.shape
    K = K1 - 1
    dev = target_probs.device
    if K > 0:
        _, rs2 = _logits_args(draft_probs, "draft_probs", 2, single=rs)
        if draft_probs.dtype != torch.float32 or rs2 != rs or tuple(draft_probs.shape) != (B, K, V):
            raise ValueError("draft_probs must be float32 [B, K, V] with the target's row stride")
    _i32(draft, (B, K), "draft")
    _i32(draft_len, (B,), "draft_len")
    if uniforms.dtype != torch.float32 or not uniforms.is_contiguous() or \
            tuple(uniforms.shape) != (B, K1):
        raise ValueError("uniforms must be a contiguous float32 tensor [B, K+1]")
    if stats is not None and (stats.dtype != torch.int64 or stats.numel() < 3 + K):
        raise ValueError("stats must be an int64 tensor of at least 3+K entries")
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    emi = torch.empty(B, K1, dtype=torch.int32, device=dev)
    pd = torch.empty(B, K, dtype=torch.float32, device=dev) if want_probs else None
    qd = torch.empty(B, K, dtype=torch.float32, device=dev) if want_probs else None
    flg = torch.empty(B, dtype=torch.int32, device=dev)
    s = _stream(dev)
    ws = workspace(L.sv_rejection_workspace_bytes(B, K, V), dev, s)
    args = (target_probs.data_ptr(), _ptr(draft_probs) if K > 0 else None, rs, _ptr(draft),
            _ptr(draft_len), uniforms.data_ptr(), B, K, V, acc.data_ptr(), emi.data_ptr(), _ptr(pd),
            _ptr(qd), flg.data_ptr(), _ptr(stats), ws.data_ptr(), ws.numel(), s)
    out = dict(accepted=acc, emitted=emi, flags=flg)
    if want_probs:
        out["p_draft"], out["q_draft"] = pd, qd
    return Prepared(L.sv_verify_rejection_probs, args, out,
                    (target_probs, draft_probs, draft, draft_len, uniforms, stats, ws))


def verify_rejection_probs(*a, **k):
    return prepare_rejection_probs(*a, **k)()


def prepare_tree(logits, parent, token, *, want_argmax=True):
    """Tree verification.  logits [B, N, V], parent [B, N], token [B, N]
    int32.  Outputs: accepted [B], path [B, N], emitted [B, N], argmax, flags."""
    torch = _torch()
    L = load()
    code, rs = _logits_args(logits, "logits", 2)
    B, N, V = logits.shape
    dev = logits.device
    _i32(parent, (B, N), "parent")
    _i32(token, (B, N), "token")
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    path = torch.empty(B, N, dtype=torch.int32, device=dev)
    emi = torch.empty(B, N, dtype=torch.int32, device=dev)
    amx = torch.empty(B, N, dtype=torch.int32, device=dev) if want_argmax else None
    flg = torch.empty(B, dtype=torch.int32, device=dev)
    s = _stream(dev)
    ws = workspace(L.sv_tree_workspace_bytes(B, N, V), dev, s)
    args = (logits.data_ptr(), code, rs, parent.data_ptr(), token.data_ptr(), B, N, V,
            acc.data_ptr(), path.data_ptr(), emi.data_ptr(), _ptr(amx), flg.data_ptr(),
            ws.data_ptr(), ws.numel(), s)
    out = dict(accepted=acc, path=path, emitted=emi, flags=flg)
    if want_argmax:
        out["argmax"] = amx
    return Prepared(L.sv_verify_tree, args, out, (logits, parent, token, ws))


def verify_tree(*a, **k):
    return prepare_tree(*a, **k)()


def prepare_ngram(tokens, lengths, n_min, n_max, K):
    """N-gram prompt lookup.  tokens [B, stride] int32 (unit inner stride),
    lengths [B] int32.  Outputs: proposal [B, K], proposal_len [B],
    match_n [B], match_pos [B], flags [B]."""
    torch = _torch()
    L = load()
    if tokens.dtype != torch.int32:
        raise ValueError("tokens must be an int32 [B, stride] tensor with unit inner stride")
    B = tokens.shape[0]
    stride = _row_stride(tokens, 1, "tokens")
    dev = tokens.device
    _rows_readable(tokens, B, stride, "tokens")
    _i32(lengths, (B,), "lengths")
    prop = torch.empty(B, K, dtype=torch.int32, device=dev)
    plen = torch.empty(B, dtype=torch.int32, device=dev)
    mn = torch.empty(B, dtype=torch.int32, device=dev)
    mp = torch.empty(B, dtype=torch.int32, device=dev)
    flg = torch.empty(B, dtype=torch.int32, device=dev)
    args = (tokens.data_ptr(), stride, lengths.data_ptr(), B, n_min, n_max, K,
            prop.data_ptr() if K > 0 else None, plen.data_ptr(), mn.data_ptr(), mp.data_ptr(),
            flg.data_ptr(), _stream(dev))
    out = dict(proposal=prop, proposal_len=plen, match_n=mn, match_pos=mp, flags=flg)
    return Prepared(L.sv_ngram_propose, args, out, (tokens, lengths))


def ngram_propose(*a, **k):
    return prepare_ngram(*a, **k)()


def prepare_suffix(tokens, lengths, history, m_min, m_max, K, min_prob):
    """Suffix-decoding proposal.  tokens [B, stride] int32 (unit inner
    stride), lengths [B] int32, history [H] int32 (contiguous) or None.
    Outputs: proposal [B, K], proposal_len [B], score [B] float64,
    match_len [B], source [B] (0 context, 1 history, -1 none), flags [B]."""
    torch = _torch()
    L = load()
    if tokens.dtype != torch.int32:
        raise ValueError("tokens must be an int32 [B, stride] tensor with unit inner stride")
    B = tokens.shape[0]
    stride = _row_stride(tokens, 1, "tokens")
    dev = tokens.device
    _rows_readable(tokens, B, stride, "tokens")
    _i32(lengths, (B,), "lengths")
    H = 0
    if history is not None:
        if history.dtype != torch.int32 or history.dim() != 1 or not history.is_contiguous():
            raise ValueError("history must be a contiguous int32 [H] tensor")
        H = history.numel()
    prop = torch.empty(B, K, dtype=torch.int32, device=dev)
    plen = torch.empty(B, dtype=torch.int32, device=dev)
    sco = torch.empty(B, dtype=torch.float64, device=dev)
    ml = torch.empty(B, dtype=torch.int32, device=dev)
    src = torch.empty(B, dtype=torch.int32, device=dev)
    flg = torch.empty(B, dtype=torch.int32, device=dev)
    s = _stream(dev)
    ws = workspace(L.sv_suffix_workspace_bytes(B, stride, H), dev, s)
    args = (tokens.data_ptr(), stride, lengths.data_ptr(), B,
            history.data_ptr() if H > 0 else None, H, m_min, m_max, K, float(min_prob),
            prop.data_ptr() if K > 0 else None, plen.data_ptr(), sco.data_ptr(), ml.data_ptr(),
            src.data_ptr(), flg.data_ptr(), ws.data_ptr(), ws.numel(), s)
    out = dict(proposal=prop, proposal_len=plen, score=sco, match_len=ml, source=src, flags=flg)
    return Prepared(L.sv_suffix_propose, args, out, (tokens, lengths, history, ws))


def suffix_propose(*a, **k):
    return prepare_suffix(*a, **k)()


# ---------------------------------------------------------------- vocabulary shards

def prepare_argmax_shard(logits, v_offset, out=None):
    """Per-row partial of one vocabulary shard: logits [..., Vs] (evenly
    spaced rows, unit stride along the shard's columns, e.g. a column slice
    of the full logits), v_offset = the shard's first global token id.
    Output: partial, an int64 tensor [rows] of sv_argmax_partial (decode
    with PARTIAL_DTYPE); pass `out` (a contiguous int64 [rows] tensor, e.g.
    one row of a [P, rows] tensor) to write in place."""
    torch = _torch()
    L = load()
    code, rs = _logits_args(logits, "logits", logits.dim() - 1)
    V = logits.shape[-1]
    rows = logits.numel() // V
    dev = logits.device
    if out is None:
        out = torch.empty(rows, dtype=torch.int64, device=dev)
    elif out.dtype != torch.int64 or not out.is_contiguous() or out.numel() != rows:
        raise ValueError("out must be a contiguous int64 tensor of %d elements" % rows)
    s = _stream(dev)
    ws = workspace(L.sv_argmax_shard_workspace_bytes(rows, V), dev, s)
    args = (logits.data_ptr(), code, rs, rows, V, int(v_offset), out.data_ptr(), ws.data_ptr(),
            ws.numel(), s)
    return Prepared(L.sv_argmax_shard, args, dict(partial=out), (logits, out, ws))


def argmax_shard(*a, **k):
    return prepare_argmax_shard(*a, **k)()


def _partials(partials, rows):
    torch = _torch()
    if partials.dtype != torch.int64 or partials.dim() != 2 or not partials.is_contiguous() \
            or partials.shape[1] != rows:
        raise ValueError("partials must be a contiguous int64 [P, %d] tensor" % rows)
    return partials.shape[0]


def prepare_greedy_partials(partials, draft, V, draft_len=None, *, want_argmax=True, stats=None):
    """Greedy verification from vocabulary-shard partials [P, B*(K+1)]
    (shard p's partials in row p), draft [B, K] int32, V = the full
    vocabulary.  Outputs as prepare_greedy."""
    torch = _torch()
    L = load()
    B, K = draft.shape
    _i32(draft, (B, K), "draft")
    _i32(draft_len, (B,), "draft_len")
    Pn = _partials(partials, B * (K + 1))
    if stats is not None and (stats.dtype != torch.int64 or stats.numel() < 3 + K):
        raise ValueError("stats must be an int64 tensor of at least 3+K entries")
    dev = partials.device
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    emi = torch.empty(B, K + 1, dtype=torch.int32, device=dev)
    amx = torch.empty(B, K + 1, dtype=torch.int32, device=dev) if want_argmax else None
    flg = torch.empty(B, dtype=torch.int32, device=dev)
    args = (partials.data_ptr(), Pn, _ptr(draft), _ptr(draft_len), B, K, int(V), acc.data_ptr(),
            emi.data_ptr(), _ptr(amx), flg.data_ptr(), _ptr(stats), _stream(dev))
    out = dict(accepted=acc, emitted=emi, flags=flg)
    if want_argmax:
        out["argmax"] = amx
    return Prepared(L.sv_verify_greedy_partials, args, out, (partials, draft, draft_len, stats))


def verify_greedy_partials(*a, **k):
    return prepare_greedy_partials(*a, **k)()


def prepare_tree_partials(partials, parent, token, V, *, want_argmax=True):
    """Tree verification from vocabulary-shard partials [P, B*N], parent
    and token [B, N] int32, V = the full vocabulary.  Outputs as
    prepare_tree."""
    torch = _torch()
    L = load()
    B, N = parent.shape
    _i32(parent, (B, N), "parent")
    _i32(token, (B, N), "token")
    Pn = _partials(partials, B * N)
    dev = partials.device
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    path = torch.empty(B, N, dtype=torch.int32, device=dev)
    emi = torch.empty(B, N, dtype=torch.int32, device=dev)
    amx = torch.empty(B, N, dtype=torch.int32, device=dev) if want_argmax else None
    flg = torch.empty(B, dtype=torch.int32, device=dev)
    args = (partials.data_ptr(), Pn, parent.data_ptr(), token.data_ptr(), B, N, int(V),
            acc.data_ptr(), path.data_ptr(), emi.data_ptr(), _ptr(amx), flg.data_ptr(), _stream(dev))
    out = dict(accepted=acc, path=path, emitted=emi, flags=flg)
    if want_argmax:
        out["argmax"] = amx
    return Prepared(L.sv_verify_tree_partials, args, out, (partials, parent, token))


def verify_tree_partials(*a, **k):
    return prepare_tree_partials(*a, **k)()


def _shard_logits(target, draft_logits):
    """Validate a shard's target [B, K+1, Vs] and draft [B, K, Vs] column
    slices; returns (dtype code, row stride, B, K, Vs)."""
    code, rs = _logits_args(target, "target", 2)
    B, K1, Vs = target.shape
    K = K1 - 1
    if K > 0:
        code2, rs2 = _logits_args(draft_logits, "draft_logits", 2, single=rs)
        if code2 != code or rs2 != rs or tuple(draft_logits.shape) != (B, K, Vs):
            raise ValueError("draft_logits must be [B, K, Vs] with the target's dtype and row stride")
    return code, rs, B, K, Vs


def _f64_records(t, shape, name):
    torch = _torch()
    if t.dtype != torch.float64 or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError("%s must be a contiguous float64 tensor of shape %s" % (name, tuple(shape)))
    return t


def prepare_rejection_shard_stats(target, draft_logits, draft, v_offset, temperature=1.0,
                                  draft_len=None, out=None):
    """Step 1 of sharded rejection sampling, for one shard: target [B, K+1,
    Vs] and draft_logits [B, K, Vs] are the shard's column slices, v_offset
    its first global id.  Output: partial, float64 [B*(2K+1), 2] (one
    sv_softmax_partial per row; decode with SOFT_PARTIAL_DTYPE); pass `out`
    (e.g. one row of a [P, B*(2K+1), 2] tensor) to write in place."""
    torch = _torch()
    L = load()
    code, rs, B, K, Vs = _shard_logits(target, draft_logits)
    _i32(draft, (B, K), "draft")
    _i32(draft_len, (B,), "draft_len")
    rows = B * (2 * K + 1)
    dev = target.device
    if out is None:
        out = torch.empty(rows, 2, dtype=torch.float64, device=dev)
    _f64_records(out, (rows, 2), "out")
    s = _stream(dev)
    ws = workspace(L.sv_rejection_shard_workspace_bytes(B, K, Vs), dev, s)
    args = (target.data_ptr(), _ptr(draft_logits) if K > 0 else None, code, rs, _ptr(draft),
            _ptr(draft_len), float(temperature), B, K, Vs, int(v_offset), out.data_ptr(),
            ws.data_ptr(), ws.numel(), s)
    return Prepared(L.sv_rejection_shard_stats, args, dict(partial=out),
                    (target, draft_logits, draft, draft_len, out, ws))


def rejection_shard_stats(*a, **k):
    return prepare_rejection_shard_stats(*a, **k)()


def prepare_rejection_partials(partials, draft, uniforms, V, temperature=1.0, draft_len=None, *,
                               want_probs=True, stats=None):
    """Step 2: the accept test on every shard's partials [P, B*(2K+1), 2]
    (float64), draft [B, K], uniforms [B, K+1], V = the full vocabulary.
    Outputs: accepted, p_draft, q_draft, flags as prepare_rejection, and
    state, float64 [B, 4] (one sv_rejection_state per sequence; decode with
    STATE_DTYPE) for steps 3 and 4."""
    torch = _torch()
    L = load()
    B, K = draft.shape
    _i32(draft, (B, K), "draft")
    _i32(draft_len, (B,), "draft_len")
    if partials.dim() != 3:
        raise ValueError("partials must be [P, B*(2K+1), 2]")
    Pn = partials.shape[0]
    _f64_records(partials, (Pn, B * (2 * K + 1), 2), "partials")
    if uniforms.dtype != torch.float32 or not uniforms.is_contiguous() or \
            tuple(uniforms.shape) != (B, K + 1):
        raise ValueError("uniforms must be a contiguous float32 tensor [B, K+1]")
    if stats is not None and (stats.dtype != torch.int64 or stats.numel() < 3 + K):
        raise ValueError("stats must be an int64 tensor of at least 3+K entries")
    dev = partials.device
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    pd = torch.empty(B, K, dtype=torch.float32, device=dev) if want_probs else None
    qd = torch.empty(B, K, dtype=torch.float32, device=dev) if want_probs else None
    flg = torch.empty(B, dtype=torch.int32, device=dev)
    state = torch.empty(B, 4, dtype=torch.float64, device=dev)
    args = (partials.data_ptr(), Pn, _ptr(draft), _ptr(draft_len), uniforms.data_ptr(),
            float(temperature), B, K, int(V), acc.data_ptr(), _ptr(pd), _ptr(qd), flg.data_ptr(),
            _ptr(stats), state.data_ptr(), _stream(dev))
    out = dict(accepted=acc, flags=flg, state=state)
    if want_probs:
        out["p_draft"], out["q_draft"] = pd, qd
    return Prepared(L.sv_verify_rejection_partials, args, out,
                    (partials, draft, draft_len, uniforms, stats))


def verify_rejection_partials(*a, **k):
    return prepare_rejection_partials(*a, **k)()


def prepare_rejection_shard_mass(target, draft_logits, state, temperature=1.0, out=None):
    """Step 3, for one shard: the shard's final-sample masses out [B, 2]
    (float64; one sv_sample_mass per sequence, decode with MASS_DTYPE).
    The call gets a workspace of its own, returned as `workspace`: step 4
    of the same shard takes it back."""
    torch = _torch()
    L = load()
    code, rs, B, K, Vs = _shard_logits(target, draft_logits)
    _f64_records(state, (B, 4), "state")
    dev = target.device
    if out is None:
        out = torch.empty(B, 2, dtype=torch.float64, device=dev)
    _f64_records(out, (B, 2), "out")
    ws = torch.empty(max(256, L.sv_rejection_shard_workspace_bytes(B, K, Vs)), dtype=torch.uint8,
                     device=dev)
    args = (target.data_ptr(), _ptr(draft_logits) if K > 0 else None, code, rs, state.data_ptr(),
            float(temperature), B, K, Vs, out.data_ptr(), ws.data_ptr(), ws.numel(), _stream(dev))
    return Prepared(L.sv_rejection_shard_mass, args, dict(mass=out, workspace=ws),
                    (target, draft_logits, state, out, ws))


def rejection_shard_mass(*a, **k):
    return prepare_rejection_shard_mass(*a, **k)()


def prepare_rejection_shard_sample(target, draft_logits, draft, uniforms, state, masses, shard,
                                   v_offset, workspace, emitted, temperature=1.0):
    """Step 4, for one shard: masses [P, B, 2] float64 of every shard,
    `workspace` the one step 3 returned for this shard, emitted [B, K+1]
    int32 written in place for the sequences whose sample this shard owns."""
    torch = _torch()
    L = load()
    code, rs, B, K, Vs = _shard_logits(target, draft_logits)
    _i32(draft, (B, K), "draft")
    _i32(emitted, (B, K + 1), "emitted")
    _f64_records(state, (B, 4), "state")
    if masses.dim() != 3:
        raise ValueError("masses must be [P, B, 2]")
    Pn = masses.shape[0]
    _f64_records(masses, (Pn, B, 2), "masses")
    if uniforms.dtype != torch.float32 or not uniforms.is_contiguous() or \
            tuple(uniforms.shape) != (B, K + 1):
        raise ValueError("uniforms must be a contiguous float32 tensor [B, K+1]")
    dev = target.device
    args = (target.data_ptr(), _ptr(draft_logits) if K > 0 else None, code, rs, _ptr(draft),
            uniforms.data_ptr(), state.data_ptr(), masses.data_ptr(), Pn, int(shard),
            float(temperature), B, K, Vs, int(v_offset), emitted.data_ptr(), workspace.data_ptr(),
            workspace.numel(), _stream(dev))
    return Prepared(L.sv_rejection_shard_sample, args, dict(emitted=emitted),
                    (target, draft_logits, draft, uniforms, state, masses, workspace, emitted))


def rejection_shard_sample(*a, **k):
    return prepare_rejection_shard_sample(*a, **k)()


# ---------------------------------------------------------------- measurement

def prepare_read_probe(buf):
    """One streaming read of a device tensor (16-byte aligned, a multiple
    of 16 bytes) with the verifiers' loads: the reference rate."""
    torch = _torch()
    L = load()
    out = torch.zeros(1, dtype=torch.int32, device=buf.device)
    nbytes = buf.numel() * buf.element_size()
    args = (buf.data_ptr(), nbytes, out.data_ptr(), _stream(buf.device))
    return Prepared(L.sv_read_probe, args, dict(out=out), (buf, out))


# ---------------------------------------------------------------- adaptive length

class _AdaptiveState(ctypes.Structure):
    _fields_ = [("ema", ctypes.c_double), ("beta", ctypes.c_double), ("ntiers", ctypes.c_int32),
                ("tiers", ctypes.c_int32 * 16), ("k", ctypes.c_int32)]


class Adaptive:
    """Adaptive speculation length (sv_adaptive_*): `k` is the length for
    the next round; call update(accepted_mean) after each round."""

    def __init__(self, tiers=(1, 3, 7), beta=0.2, ema0=0.0):
        L = load()
        self._s = _AdaptiveState()
        arr = (ctypes.c_int32 * len(tiers))(*[int(t) for t in tiers])
        _check(L.sv_adaptive_init(ctypes.byref(self._s), arr, len(tiers), float(beta), float(ema0)))

    @property
    def k(self) -> int:
        return int(self._s.k)

    @property
    def ema(self) -> float:
        return float(self._s.ema)

    def update(self, accepted_mean) -> int:
        _check(load().sv_adaptive_update(ctypes.byref(self._s), float(accepted_mean)))
        return self.k
