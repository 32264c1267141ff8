"""fp64 CPU oracle for Kimi Delta Attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library in
``gated_delta_rule_chunkwise_amd``) never imports, links or calls it, and the two
share no code.

The arithmetic lives in ``kda_oracle.c`` (plain C, fp64, per-token recurrence of
the KimiLinear article, section 2.3, with the read-out o_t = S_t^T q_t).  This
module only marshals numpy arrays into it.

``bwd`` is the gradient of ``fwd`` (reverse-mode differentiation of the same
recurrence), pinned by central finite differences of ``fwd``, by PyTorch fp64
autograd through an independently written recurrence, and by the closed form
of the frozen-state case.

Pins: every function here is pinned by ``tests/test_oracle_pins.py`` against
special cases that the pages' own equations fix (sections 2.1-2.3 of the
KimiLinear article), a brute-force product of explicit transition matrices, a
hand-worked scalar example and invariants.  No function is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math",
                               "-ffp-contract=off", "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int64)
        i64 = ctypes.c_int64
        lib.kda_oracle_gen_fwd.argtypes = [dp, dp, dp, dp, dp, dp, dp, ip, i64, i64, i64, i64,
                                           dp, dp, ctypes.c_int]
        lib.kda_oracle_gen_fwd.restype = ctypes.c_int
        lib.kda_oracle_fwd.argtypes = [dp, dp, dp, dp, dp, dp, ip, i64, i64, i64, i64, dp, dp,
                                       ctypes.c_int]
        lib.kda_oracle_fwd.restype = ctypes.c_int
        lib.kda_oracle_decode.argtypes = [dp, dp, dp, dp, dp, dp, i64, i64, i64, i64, dp,
                                          ctypes.c_int]
        lib.kda_oracle_decode.restype = ctypes.c_int
        lib.kda_oracle_prologue.argtypes = [dp, dp, dp, dp, i64, i64, ctypes.c_double,
                                             ctypes.c_double, dp, dp, dp, dp]
        lib.kda_oracle_prologue.restype = ctypes.c_int
        lib.kda_oracle_bwd.argtypes = [dp, dp, dp, dp, dp, dp, ip, i64, i64, i64, i64, dp, dp,
                                       dp, dp, dp, dp, dp, dp, ctypes.c_int]
        lib.kda_oracle_bwd.restype = ctypes.c_int
        lib.kda_oracle_gen_bwd.argtypes = [dp, dp, dp, dp, dp, dp, dp, ip, i64, i64, i64, i64, dp, dp,
                                           dp, dp, dp, dp, dp, dp, dp, ctypes.c_int]
        lib.kda_oracle_gen_bwd.restype = ctypes.c_int
        lib.kda_oracle_prologue_bwd.argtypes = [dp, dp, dp, dp, i64, i64, ctypes.c_double, ctypes.c_double,
                                                dp, dp, dp, dp, dp, dp, dp, dp]
        lib.kda_oracle_prologue_bwd.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _f64(x, shape=None):
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    if shape is not None and a.shape != tuple(shape):
        raise ValueError("expected shape %s, got %s" % (tuple(shape), a.shape))
    return a


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double if a.dtype == np.float64
                                           else ctypes.c_int64))


def _cu(cu_seqlens, T_total):
    if cu_seqlens is None:
        cu = np.array([0, T_total], dtype=np.int64)
    else:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    if cu.ndim != 1 or cu.size < 1 or cu[0] != 0 or cu[-1] != T_total or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at T_total")
    return cu


def gen_fwd(q, k, v, log_alpha, b_erase, w_write, h0=None, cu_seqlens=None, nthreads=None):
    """Generalised recurrence with separate erase (b) and write (w) strengths.

    q, k, log_alpha: [T, H, dk]; v: [T, H, dv]; b_erase, w_write: [T, H];
    h0: [N, H, dk, dv] or None; cu_seqlens: [N+1] or None (one sequence).
    Returns (o [T, H, dv], h_T [N, H, dk, dv]) in fp64.
    """
    q = _f64(q)
    if q.ndim != 3:
        raise ValueError("q must be [T, H, dk]")
    T, H, dk = q.shape
    k = _f64(k, (T, H, dk))
    la = _f64(log_alpha, (T, H, dk))
    v = _f64(v)
    if v.ndim != 3 or v.shape[:2] != (T, H):
        raise ValueError("v must be [T, H, dv]")
    dv = v.shape[2]
    b = _f64(b_erase, (T, H))
    w = _f64(w_write, (T, H))
    cu = _cu(cu_seqlens, T)
    N = cu.size - 1
    h0a = None if h0 is None else _f64(h0, (N, H, dk, dv))
    o = np.zeros((T, H, dv), dtype=np.float64)
    hT = np.zeros((N, H, dk, dv), dtype=np.float64)
    rc = _load().kda_oracle_gen_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(b), _ptr(w),
                                    _ptr(h0a), _ptr(cu), N, H, dk, dv, _ptr(o), _ptr(hT),
                                    int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError("kda_oracle_gen_fwd failed with code %d" % rc)
    return o, hT


def fwd(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, nthreads=None):
    """KDA forward (b = w = beta) over a packed batch; see ``gen_fwd``."""
    q = _f64(q)
    if q.ndim != 3:
        raise ValueError("q must be [T, H, dk]")
    T, H, dk = q.shape
    k = _f64(k, (T, H, dk))
    la = _f64(log_alpha, (T, H, dk))
    v = _f64(v)
    if v.ndim != 3 or v.shape[:2] != (T, H):
        raise ValueError("v must be [T, H, dv]")
    dv = v.shape[2]
    be = _f64(beta, (T, H))
    cu = _cu(cu_seqlens, T)
    N = cu.size - 1
    h0a = None if h0 is None else _f64(h0, (N, H, dk, dv))
    o = np.zeros((T, H, dv), dtype=np.float64)
    hT = np.zeros((N, H, dk, dv), dtype=np.float64)
    rc = _load().kda_oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(be), _ptr(h0a),
                                _ptr(cu), N, H, dk, dv, _ptr(o), _ptr(hT),
                                int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError("kda_oracle_fwd failed with code %d" % rc)
    return o, hT


def decode(q, k, v, log_alpha, beta, S, nthreads=None):
    """One decode step for B sequences.  q, k, log_alpha: [B, H, dk];
    v: [B, H, dv]; beta: [B, H]; S: [B, H, dk, dv].  Returns (o, S_new)."""
    q = _f64(q)
    B, H, dk = q.shape
    k = _f64(k, (B, H, dk))
    la = _f64(log_alpha, (B, H, dk))
    v = _f64(v)
    dv = v.shape[2]
    be = _f64(beta, (B, H))
    S_new = np.array(_f64(S, (B, H, dk, dv)), copy=True)
    o = np.zeros((B, H, dv), dtype=np.float64)
    rc = _load().kda_oracle_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(be), _ptr(S_new),
                                   B, H, dk, dv, _ptr(o), int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError("kda_oracle_decode failed with code %d" % rc)
    return o, S_new


def bwd(q, k, v, log_alpha, beta, d_o, h0=None, d_hT=None, cu_seqlens=None, nthreads=None):
    """Gradient of the KDA forward (reverse-mode differentiation of the per-token
    recurrence; ``kda_oracle_bwd`` in kda_oracle.c) for a loss whose gradients
    with respect to o and h_T are d_o [T, H, dv] and d_hT [N, H, dk, dv] (None:
    zero).  Returns (dq, dk, dv, dlog_alpha, dbeta, dh0) in fp64 with the input
    shapes; dh0 is returned whether or not h0 was given."""
    q = _f64(q)
    if q.ndim != 3:
        raise ValueError("q must be [T, H, dk]")
    T, H, dk = q.shape
    k = _f64(k, (T, H, dk))
    la = _f64(log_alpha, (T, H, dk))
    v = _f64(v)
    if v.ndim != 3 or v.shape[:2] != (T, H):
        raise ValueError("v must be [T, H, dv]")
    dv = v.shape[2]
    be = _f64(beta, (T, H))
    do = _f64(d_o, (T, H, dv))
    cu = _cu(cu_seqlens, T)
    N = cu.size - 1
    h0a = None if h0 is None else _f64(h0, (N, H, dk, dv))
    dhT = None if d_hT is None else _f64(d_hT, (N, H, dk, dv))
    dq = np.zeros((T, H, dk))
    dk_ = np.zeros((T, H, dk))
    dv_ = np.zeros((T, H, dv))
    dla = np.zeros((T, H, dk))
    db = np.zeros((T, H))
    dh0 = np.zeros((N, H, dk, dv))
    rc = _load().kda_oracle_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(be), _ptr(h0a),
                                _ptr(cu), N, H, dk, dv, _ptr(do), _ptr(dhT), _ptr(dq), _ptr(dk_),
                                _ptr(dv_), _ptr(dla), _ptr(db), _ptr(dh0),
                                int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError("kda_oracle_bwd failed with code %d" % rc)
    return dq, dk_, dv_, dla, db, dh0


def gen_bwd(q, k, v, log_alpha, b_erase, w_write, d_o, h0=None, d_hT=None, cu_seqlens=None, nthreads=None):
    """Gradient of the generalised recurrence (``gen_fwd``: separate erase and
    write strengths; ``kda_oracle_gen_bwd`` in kda_oracle.c).  Returns (dq, dk,
    dv, dlog_alpha, db_erase, dw_write, dh0) in fp64 with the input shapes."""
    q = _f64(q)
    if q.ndim != 3:
        raise ValueError("q must be [T, H, dk]")
    T, H, dk = q.shape
    k = _f64(k, (T, H, dk))
    la = _f64(log_alpha, (T, H, dk))
    v = _f64(v)
    if v.ndim != 3 or v.shape[:2] != (T, H):
        raise ValueError("v must be [T, H, dv]")
    dv = v.shape[2]
    be = _f64(b_erase, (T, H))
    wr = _f64(w_write, (T, H))
    do = _f64(d_o, (T, H, dv))
    cu = _cu(cu_seqlens, T)
    N = cu.size - 1
    h0a = None if h0 is None else _f64(h0, (N, H, dk, dv))
    dhT = None if d_hT is None else _f64(d_hT, (N, H, dk, dv))
    dq = np.zeros((T, H, dk))
    dk_ = np.zeros((T, H, dk))
    dv_ = np.zeros((T, H, dv))
    dla = np.zeros((T, H, dk))
    db = np.zeros((T, H))
    dw = np.zeros((T, H))
    dh0 = np.zeros((N, H, dk, dv))
    rc = _load().kda_oracle_gen_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(be), _ptr(wr), _ptr(h0a),
                                    _ptr(cu), N, H, dk, dv, _ptr(do), _ptr(dhT), _ptr(dq), _ptr(dk_),
                                    _ptr(dv_), _ptr(dla), _ptr(db), _ptr(dw), _ptr(dh0),
                                    int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError("kda_oracle_gen_bwd failed with code %d" % rc)
    return dq, dk_, dv_, dla, db, dw, dh0


# Default eps of the L2 normalisation (the GPU entry points use the same value).
PROLOGUE_EPS = 1e-6


def prologue(q_raw, k_raw, gate_pre, beta_pre, log_alpha_min, eps=PROLOGUE_EPS):
    """Input prologue (see ``kda_oracle_prologue`` in kda_oracle.c): per row,
    q / max(||q||, eps), k / max(||k||, eps), max(-softplus(gate_pre), log_alpha_min)
    and sigmoid(beta_pre).  q_raw, k_raw, gate_pre: [..., dk]; beta_pre: [...].
    Returns (q_hat, k_hat, log_alpha, beta) in fp64 with the input shapes."""
    q = _f64(q_raw)
    dk = q.shape[-1]
    lead = q.shape[:-1]
    k = _f64(k_raw, q.shape)
    a = _f64(gate_pre, q.shape)
    b = _f64(beta_pre, lead)
    rows = int(np.prod(lead)) if lead else 1
    qh = np.zeros_like(q)
    kh = np.zeros_like(k)
    la = np.zeros_like(a)
    be = np.zeros_like(b)
    rc = _load().kda_oracle_prologue(_ptr(q), _ptr(k), _ptr(a), _ptr(b), rows, dk,
                                     float(log_alpha_min), float(eps), _ptr(qh), _ptr(kh),
                                     _ptr(la), _ptr(be))
    if rc != 0:
        raise RuntimeError("kda_oracle_prologue failed with code %d" % rc)
    return qh, kh, la, be


def fwd_prologue(q_raw, k_raw, v, gate_pre, beta_pre, log_alpha_min, h0=None,
                 cu_seqlens=None, nthreads=None, eps=PROLOGUE_EPS):
    """KDA forward on raw projections: ``prologue`` then ``fwd``."""
    qh, kh, la, be = prologue(q_raw, k_raw, gate_pre, beta_pre, log_alpha_min, eps)
    return fwd(qh, kh, v, la, be, h0=h0, cu_seqlens=cu_seqlens, nthreads=nthreads)


def bwd_prologue(q_raw, k_raw, v, gate_pre, beta_pre, log_alpha_min, d_o, h0=None, d_hT=None,
                 cu_seqlens=None, nthreads=None, eps=PROLOGUE_EPS):
    """Gradient of ``fwd_prologue``: ``bwd`` at the mapped inputs, then the chain
    rule through the prologue maps (``kda_oracle_prologue_bwd`` in kda_oracle.c).
    Returns (dq_raw, dk_raw, dv, dgate_pre, dbeta_pre, dh0) in fp64."""
    qh, kh, la, be = prologue(q_raw, k_raw, gate_pre, beta_pre, log_alpha_min, eps)
    dqh, dkh, dv, dla, dbe, dh0 = bwd(qh, kh, v, la, be, d_o, h0=h0, d_hT=d_hT, cu_seqlens=cu_seqlens,
                                      nthreads=nthreads)
    q = _f64(q_raw)
    dk = q.shape[-1]
    lead = q.shape[:-1]
    k = _f64(k_raw, q.shape)
    a = _f64(gate_pre, q.shape)
    b = _f64(beta_pre, lead)
    rows = int(np.prod(lead)) if lead else 1
    dq, dk_, da, db = np.zeros_like(q), np.zeros_like(k), np.zeros_like(a), np.zeros_like(b)
    rc = _load().kda_oracle_prologue_bwd(_ptr(q), _ptr(k), _ptr(a), _ptr(b), rows, dk, float(log_alpha_min),
                                         float(eps), _ptr(dqh), _ptr(dkh), _ptr(dla), _ptr(dbe), _ptr(dq),
                                         _ptr(dk_), _ptr(da), _ptr(db))
    if rc != 0:
        raise RuntimeError("kda_oracle_prologue_bwd failed with code %d" % rc)
    return dq, dk_, dv, da, db, dh0


def decode_prologue(q_raw, k_raw, v, gate_pre, beta_pre, log_alpha_min, S, nthreads=None,
                    eps=PROLOGUE_EPS):
    """One decode step on raw projections: ``prologue`` then ``decode``."""
    qh, kh, la, be = prologue(q_raw, k_raw, gate_pre, beta_pre, log_alpha_min, eps)
    return decode(qh, kh, v, la, be, S, nthreads=nthreads)
