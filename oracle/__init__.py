"""ctypes wrapper around the scalar fp64 oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
CPU-baseline leg of bench.py.  The GPU library never imports this package and
this package never imports the GPU library.

Every wrapper takes numpy arrays for ONE sequence and ONE KV head:
K, V: float32 [T, d] (exact stored values), q: float32 [G, d].
Results are float64.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64 = ctypes.c_int64
_int = ctypes.c_int


def lib():
    """Load liboracle.so, compiling it first if it is missing or stale."""
    global _LIB
    if _LIB is not None:
        return _LIB
    so = os.path.join(_HERE, "liboracle.so")
    src = os.path.join(_HERE, "oracle.c")
    if not os.path.exists(so) or os.path.getmtime(so) < os.path.getmtime(src):
        _build.build()
    L = ctypes.CDLL(so)
    L.orc_desc_minmax.argtypes = [_f32p, _i64, _int, _int, _f64p, _f64p]
    L.orc_desc_mean.argtypes = [_f32p, _i64, _int, _int, _f64p]
    L.orc_score_quest.argtypes = [_f32p, _int, _int, _f64p, _f64p, _i64, _f64p]
    L.orc_score_gate.argtypes = [_f32p, _int, _int, _f32p, _f64p, _i64, _f64p]
    L.orc_block_count.argtypes = [_i64, _int, _i64, _int, _int, _int]
    L.orc_block_count.restype = _i64
    L.orc_select.argtypes = [_f64p, _i64, _i64, _int, _i32p, _i64]
    L.orc_select.restype = _i64
    L.orc_attend.argtypes = [_f32p, _f32p, _f32p, _i64, _int, _int, _i32p, _i64,
                             ctypes.c_double, _f64p, _f64p]
    L.orc_dense_attend.argtypes = [_f32p, _f32p, _f32p, _i64, _int,
                                   ctypes.c_double, _f64p, _f64p]
    L.orc_rectify.argtypes = [_f32p, _int, _int, _f32p, _f32p, _i64, _int,
                              _f32p, _f32p, ctypes.c_double, _f64p, _f64p]
    L.orc_decode_group.argtypes = [_f32p, _int, _f32p, _f32p, _i64, _int, _int,
                                   _int, _f32p, _i64, _int, _int, _int,
                                   ctypes.c_double, _i32p, _i64, _f64p, _f64p,
                                   _f64p]
    L.orc_decode_group.restype = _i64
    L.orc_gate_bias.argtypes = [_f64p, _i64, _int, ctypes.c_double, _i32p, _i64,
                                _f64p]
    L.orc_attend_biased.argtypes = [_f32p, _f32p, _f32p, _i64, _int, _int, _i32p,
                                    _i64, _f64p, ctypes.c_double, _f64p, _f64p]
    L.orc_decode_group_gated.argtypes = [_f32p, _int, _f32p, _f32p, _i64, _int,
                                         _int, _int, _f32p, _i64, _int, _int, _int,
                                         _int, ctypes.c_double, ctypes.c_double, _i32p,
                                         _i64, _f64p, _f64p, _f64p]
    L.orc_decode_group_gated.restype = _i64
    _LIB = L
    return L


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a, a.ctypes.data_as(_f32p)


def _f64(a):
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a, a.ctypes.data_as(_f64p)


def nblocks(T, b):
    return (T + b - 1) // b


def desc_minmax(K, b):
    K, pK = _f32(K)
    T, d = K.shape
    NB = nblocks(T, b)
    mn = np.empty((NB, d), np.float64)
    mx = np.empty((NB, d), np.float64)
    lib().orc_desc_minmax(pK, T, d, b, mn.ctypes.data_as(_f64p), mx.ctypes.data_as(_f64p))
    return mn, mx


def desc_mean(K, b):
    K, pK = _f32(K)
    T, d = K.shape
    NB = nblocks(T, b)
    mean = np.empty((NB, d), np.float64)
    lib().orc_desc_mean(pK, T, d, b, mean.ctypes.data_as(_f64p))
    return mean


def score_quest(q, mn, mx, nblk=None):
    q, pq = _f32(q)
    G, d = q.shape
    mn, pmn = _f64(mn)
    mx, pmx = _f64(mx)
    nblk = mn.shape[0] if nblk is None else nblk
    s = np.empty(max(nblk, 0), np.float64)
    lib().orc_score_quest(pq, G, d, pmn, pmx, nblk, s.ctypes.data_as(_f64p))
    return s


def score_gate(q, W, mean, nblk=None):
    q, pq = _f32(q)
    G, d = q.shape
    W, pW = _f32(W)
    mean, pm = _f64(mean)
    nblk = mean.shape[0] if nblk is None else nblk
    s = np.empty(max(nblk, 0), np.float64)
    lib().orc_score_gate(pq, G, d, pW, pm, nblk, s.ctypes.data_as(_f64p))
    return s


def block_count(NB, b, budget_tokens=0, sparsity_bp=0, n_local=1, n_min=0):
    return int(lib().orc_block_count(NB, b, budget_tokens, sparsity_bp, n_local, n_min))


def select(scores, NB, n, n_local, idx_cap=None):
    """scores: [>= NB - n_local'] candidate scores.  Returns ascending idx."""
    full = np.full(max(NB, 1), np.nan, np.float64)
    sc = np.asarray(scores, np.float64)
    full[: sc.shape[0]] = sc[: NB]
    cap = NB if idx_cap is None else idx_cap
    idx = np.empty(max(cap, 1), np.int32)
    c = lib().orc_select(full.ctypes.data_as(_f64p), NB, n, n_local,
                         idx.ctypes.data_as(_i32p), cap)
    return idx[:c].copy() if idx_cap is None else idx


def attend(q, K, V, b, idx, scale):
    q, pq = _f32(q)
    K, pK = _f32(K)
    V, pV = _f32(V)
    T, d = K.shape
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    o = np.empty(d, np.float64)
    lse = ctypes.c_double()
    lib().orc_attend(pq, pK, pV, T, d, b, idx.ctypes.data_as(_i32p), idx.shape[0],
                     scale, o.ctypes.data_as(_f64p), ctypes.byref(lse))
    return o, lse.value


def dense_attend(q, K, V, n_tok, scale):
    q, pq = _f32(q)
    K, pK = _f32(K)
    V, pV = _f32(V)
    d = K.shape[1]
    o = np.empty(d, np.float64)
    lse = ctypes.c_double()
    lib().orc_dense_attend(pq, pK, pV, n_tok, d, scale, o.ctypes.data_as(_f64p),
                           ctypes.byref(lse))
    return o, lse.value


def rectify(q, K, V, k_new, v_new, scale):
    """q: [G, f, d]; K, V: float32 [T, d] (MODIFIED IN PLACE: they must be
    C-contiguous float32); k_new, v_new: [f, d].  Returns o [G, f, d],
    lse [G, f]."""
    assert K.dtype == np.float32 and K.flags.c_contiguous
    assert V.dtype == np.float32 and V.flags.c_contiguous
    q, pq = _f32(q)
    G, f, d = q.shape
    T = K.shape[0]
    kn, pkn = _f32(k_new)
    vn, pvn = _f32(v_new)
    o = np.empty((G, f, d), np.float64)
    lse = np.empty((G, f), np.float64)
    lib().orc_rectify(pq, G, f, K.ctypes.data_as(_f32p), V.ctypes.data_as(_f32p),
                      T, d, pkn, pvn, scale, o.ctypes.data_as(_f64p),
                      lse.ctypes.data_as(_f64p))
    return o, lse


def decode_group(q, K, V, b, desc_kind, W=None, budget_tokens=0, sparsity_bp=0,
                 n_local=1, n_min=0, scale=None, idx_cap=None, want_scores=False):
    """One full sparse decode step for one (sequence, KV head) group.
    desc_kind: 0 = min/max (Quest), 1 = mean-pooled keys + gate W.
    Returns (idx ascending [cnt], o [G, d], lse [G]) and optionally the
    candidate scores [NB] (NaN for the local blocks)."""
    q, pq = _f32(q)
    G, d = q.shape
    K, pK = _f32(K)
    V, pV = _f32(V)
    T = K.shape[0]
    NB = nblocks(T, b)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if W is None:
        Wc, pW = None, None
    else:
        Wc, pW = _f32(W)
    cap = NB if idx_cap is None else idx_cap
    idx = np.empty(max(cap, 1), np.int32)
    o = np.empty((G, d), np.float64)
    lse = np.empty(G, np.float64)
    s = np.empty(NB, np.float64) if want_scores else None
    c = lib().orc_decode_group(pq, G, pK, pV, T, d, b, desc_kind, pW, budget_tokens,
                               sparsity_bp, n_local, n_min, scale,
                               idx.ctypes.data_as(_i32p), cap, o.ctypes.data_as(_f64p),
                               lse.ctypes.data_as(_f64p),
                               s.ctypes.data_as(_f64p) if want_scores else None)
    out = (idx[:c].copy(), o, lse)
    if want_scores:
        out = out + (s,)
    return out


def gate_bias(scores, NB, n_current, tau, idx):
    """Log-gate bias (SAS) of the selected blocks idx: log softmax(tau * s)
    over the NB - n_current historical blocks, 0 for the n_current trailing
    (current) blocks.  scores: [>= NB - n_current] historical-block scores."""
    full = np.full(max(NB, 1), np.nan, np.float64)
    sc = np.asarray(scores, np.float64)
    full[: min(sc.shape[0], NB)] = sc[: NB]
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    bias = np.empty(max(idx.shape[0], 1), np.float64)
    lib().orc_gate_bias(full.ctypes.data_as(_f64p), NB, n_current, tau,
                        idx.ctypes.data_as(_i32p), idx.shape[0],
                        bias.ctypes.data_as(_f64p))
    return bias[: idx.shape[0]].copy()


def attend_biased(q, K, V, b, idx, bias, scale):
    """Attention over the kept blocks with an additive logit bias per block."""
    q, pq = _f32(q)
    K, pK = _f32(K)
    V, pV = _f32(V)
    T, d = K.shape
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    bias, pb = _f64(bias)
    assert bias.shape[0] == idx.shape[0]
    o = np.empty(d, np.float64)
    lse = ctypes.c_double()
    lib().orc_attend_biased(pq, pK, pV, T, d, b, idx.ctypes.data_as(_i32p),
                            idx.shape[0], pb, scale, o.ctypes.data_as(_f64p),
                            ctypes.byref(lse))
    return o, lse.value


def decode_group_gated(q, K, V, b, desc_kind, tau, W=None, budget_tokens=0,
                       sparsity_bp=0, n_local=1, n_min=0, scale=None, n_current=1):
    """decode_group with the SAS log-gate bias; n_current trailing blocks keep
    the unit gate (1: the page's single current block).  Returns (idx [cnt],
    o [G, d], lse [G], bias [cnt])."""
    q, pq = _f32(q)
    G, d = q.shape
    K, pK = _f32(K)
    V, pV = _f32(V)
    T = K.shape[0]
    NB = nblocks(T, b)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if W is None:
        Wk, pW = None, None
    else:
        Wk, pW = _f32(W)
    idx = np.empty(max(NB, 1), np.int32)
    o = np.empty((G, d), np.float64)
    lse = np.empty(G, np.float64)
    bias = np.empty(max(NB, 1), np.float64)
    c = lib().orc_decode_group_gated(pq, G, pK, pV, T, d, b, desc_kind, pW,
                                     budget_tokens, sparsity_bp, n_local, n_min,
                                     n_current, scale, tau, idx.ctypes.data_as(_i32p), NB,
                                     o.ctypes.data_as(_f64p), lse.ctypes.data_as(_f64p),
                                     bias.ctypes.data_as(_f64p))
    return idx[:c].copy(), o, lse, bias[:c].copy()
