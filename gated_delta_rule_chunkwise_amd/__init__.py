"""libkda Python binding: Kimi Delta Attention forward on MI355X (gfx950).

A thin ctypes layer over the C ABI declared in ``include/kda.h``.  It only
marshals torch tensors (device memory and the current HIP stream) into the C
calls; every step of the computation runs in the HIP kernels of ``libkda.so``.
There is no fallback: if the library is missing or fails to load, every entry
point raises.

Entry points (same names as the C ABI):
    kda_chunk_fwd(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, ...)
    kda_chunk_fwd_noalloc(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, o=..., h_T=...)
    kda_decode_step(q, k, v, log_alpha, beta, S, o=None)
    kda_chunk_fwd_prologue(q_raw, k_raw, v, gate_pre, beta_pre, log_alpha_min, ...)
    kda_decode_step_prologue(q_raw, k_raw, v, gate_pre, beta_pre, log_alpha_min, S, o=None)
    kda_gdn_chunk_fwd(q, k, v, log_alpha_or_None, beta, ...)   (scalar gate [.., H], or none)
    kda_gdn_decode_step(q, k, v, log_alpha_or_None, beta, S, o=None)
    kda_chunk_fwd_decoupled(q, k, v, log_alpha, b_erase, w_write, ...)
    kda_decode_step_decoupled(q, k, v, log_alpha, b_erase, w_write, S, o=None)
    kda_chunk_bwd(q, k, v, log_alpha, beta, grad_o, h0=None, grad_hT=None, cu_seqlens=None, ...)
    kda_gdn_chunk_bwd(q, k, v, log_alpha_or_None, beta, grad_o, ...)
    kda_chunk_bwd_decoupled(q, k, v, log_alpha, b_erase, w_write, grad_o, ...)
    kda_chunk_bwd_prologue(q_raw, k_raw, v, gate_pre, beta_pre, log_alpha_min, grad_o, ...)
    chunk_kda(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None)        (autograd: fwd + bwd)
    chunk_gated_delta_rule(q, k, v, log_alpha_or_None, beta, ...)       (autograd, scalar gate)
    kda_chunk_fwd_workspace_size(...), kda_chunk_bwd_workspace_size(...),
    kda_gdn_chunk_bwd_workspace_size(...),
    kda_status_string(code), kda_abi_version()
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_OK, KDA_ERR_INVALID_ARGUMENT, KDA_ERR_UNSUPPORTED, KDA_ERR_WORKSPACE, KDA_ERR_HIP = range(5)
KDA_F32, KDA_BF16 = 0, 1
EXPORTED_SYMBOLS = ("kda_abi_version", "kda_status_string", "kda_last_hip_error",
                    "kda_chunk_fwd_workspace_size", "kda_chunk_fwd", "kda_decode_step",
                    "kda_chunk_fwd_prologue", "kda_decode_step_prologue", "kda_gdn_chunk_fwd",
                    "kda_gdn_decode_step", "kda_chunk_fwd_decoupled", "kda_decode_step_decoupled",
                    "kda_chunk_bwd_workspace_size", "kda_chunk_bwd",
                    "kda_gdn_chunk_bwd_workspace_size", "kda_gdn_chunk_bwd", "kda_chunk_bwd_decoupled",
                    "kda_chunk_bwd_prologue_workspace_size", "kda_chunk_bwd_prologue",
                    "kda_chunk_fwd_noalloc")

_lib = None


class KDAError(RuntimeError):
    def __init__(self, code: int, where: str, detail: str = ""):
        self.code = code
        msg = "%s failed: %s" % (where, kda_status_string(code))
        if detail:
            msg += " (%s)" % detail
        super().__init__(msg)


def load_library(path: str = LIB_PATH):
    """Loads libkda.so and declares the C signatures.  Raises OSError if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise OSError("libkda.so is not built (%s); run "
                      "`python -m gated_delta_rule_chunkwise_amd.build`" % path)
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.kda_abi_version.argtypes = []
    lib.kda_abi_version.restype = i32
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_last_hip_error.argtypes = []
    lib.kda_last_hip_error.restype = ctypes.c_char_p
    lib.kda_chunk_fwd_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.c_int]
    lib.kda_chunk_fwd_workspace_size.restype = sz
    lib.kda_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32,
                                  ctypes.c_int, ctypes.c_int, vp, sz, vp]
    lib.kda_chunk_fwd.restype = ctypes.c_int
    lib.kda_chunk_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32,
                                          ctypes.c_int, ctypes.c_int, vp]
    lib.kda_chunk_fwd_noalloc.restype = ctypes.c_int
    lib.kda_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, ctypes.c_int,
                                    ctypes.c_int, vp]
    lib.kda_decode_step.restype = ctypes.c_int
    lib.kda_chunk_fwd_prologue.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, i32, vp, vp, i32,
                                           i32, i32, i32, i32, ctypes.c_int, ctypes.c_int, vp, sz, vp]
    lib.kda_chunk_fwd_prologue.restype = ctypes.c_int
    lib.kda_decode_step_prologue.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, i32, i32, i32,
                                             i32, ctypes.c_int, ctypes.c_int, vp]
    lib.kda_decode_step_prologue.restype = ctypes.c_int
    lib.kda_gdn_chunk_fwd.argtypes = list(lib.kda_chunk_fwd.argtypes)
    lib.kda_gdn_chunk_fwd.restype = ctypes.c_int
    lib.kda_gdn_decode_step.argtypes = list(lib.kda_decode_step.argtypes)
    lib.kda_gdn_decode_step.restype = ctypes.c_int
    lib.kda_chunk_fwd_decoupled.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32,
                                            ctypes.c_int, ctypes.c_int, vp, sz, vp]
    lib.kda_chunk_fwd_decoupled.restype = ctypes.c_int
    lib.kda_decode_step_decoupled.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, ctypes.c_int,
                                              ctypes.c_int, vp]
    lib.kda_decode_step_decoupled.restype = ctypes.c_int
    lib.kda_chunk_bwd_workspace_size.argtypes = list(lib.kda_chunk_fwd_workspace_size.argtypes)
    lib.kda_chunk_bwd_workspace_size.restype = sz
    lib.kda_chunk_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                  i32, i32, i32, i32, i32, ctypes.c_int, ctypes.c_int, vp, sz, vp]
    lib.kda_chunk_bwd.restype = ctypes.c_int
    lib.kda_gdn_chunk_bwd_workspace_size.argtypes = list(lib.kda_chunk_fwd_workspace_size.argtypes)
    lib.kda_gdn_chunk_bwd_workspace_size.restype = sz
    lib.kda_gdn_chunk_bwd.argtypes = list(lib.kda_chunk_bwd.argtypes)
    lib.kda_gdn_chunk_bwd.restype = ctypes.c_int
    lib.kda_chunk_bwd_decoupled.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                            vp, i32, i32, i32, i32, i32, ctypes.c_int, ctypes.c_int, vp, sz, vp]
    lib.kda_chunk_bwd_decoupled.restype = ctypes.c_int
    lib.kda_chunk_bwd_prologue_workspace_size.argtypes = list(lib.kda_chunk_fwd_workspace_size.argtypes)
    lib.kda_chunk_bwd_prologue_workspace_size.restype = sz
    lib.kda_chunk_bwd_prologue.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, i32, vp, vp, vp, vp, vp, vp,
                                           vp, vp, i32, i32, i32, i32, i32, ctypes.c_int, ctypes.c_int, vp, sz, vp]
    lib.kda_chunk_bwd_prologue.restype = ctypes.c_int
    _lib = lib
    return lib


def kda_abi_version() -> int:
    return int(load_library().kda_abi_version())


def kda_status_string(code: int) -> str:
    return load_library().kda_status_string(int(code)).decode()


def kda_last_hip_error() -> str:
    return load_library().kda_last_hip_error().decode()


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError("unsupported dtype %s (bfloat16 or float32)" % t.dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_of(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check_dev(name, t, device):
    if not t.is_cuda or t.device != device:
        raise ValueError("%s must be on %s" % (name, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _check_out(name, t, device, shape=None, dtype=None):
    """A caller-supplied output or workspace: on the device, contiguous, and of
    exactly the shape and dtype the call writes (workspace: any shape; its
    byte length is checked by the library)."""
    _check_dev(name, t, device)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, not %s" % (name, tuple(shape), tuple(t.shape)))
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, not %s" % (name, dtype, t.dtype))


def kda_chunk_fwd_workspace_size(B, T, H, d_k, d_v, num_seqs=0, io_dtype=KDA_BF16) -> int:
    return int(load_library().kda_chunk_fwd_workspace_size(B, T, H, d_k, d_v, num_seqs, io_dtype))


def kda_chunk_fwd(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, *, o=None, h_T=None,
                  output_final_state=True, workspace=None):
    """Chunkwise KDA forward.

    q, k, log_alpha: [B, T, H, d_k] (or [T, H, d_k] for B = 1); v: [B, T, H, d_v];
    beta: [B, T, H]; h0: [N, H, d_k, d_v] fp32 or None; cu_seqlens: int32 [N+1]
    on the device (B must be 1) or None.  Returns (o, h_T) with h_T None when
    output_final_state is False.  Runs asynchronously on the current stream.
    """
    return _chunk_fwd(q, k, v, log_alpha, beta, h0, cu_seqlens, o, h_T, output_final_state, workspace,
                      None)


def kda_chunk_fwd_noalloc(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, *, o, h_T=None):
    """kda_chunk_fwd through the C entry point that allocates nothing: its
    workspace is a scratch array the library holds on each device (80 MiB),
    shared by every such call on the device, so calls that overlap in time on
    one device race.  The caller passes the outputs o (and h_T, or None when
    the final state is not wanted); this function allocates no device memory.
    Raises KDAError (KDA_ERR_WORKSPACE) for calls that need more scratch
    (bf16 at d_k or d_v = 64 with a large batch)."""
    return _chunk_fwd(q, k, v, log_alpha, beta, h0, cu_seqlens, o, h_T, h_T is not None, None, None,
                      noalloc=True)


def kda_gdn_chunk_fwd(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, *, o=None, h_T=None,
                      output_final_state=True, workspace=None):
    """Gated DeltaNet (log_alpha [B, T, H], one decay per token and head) or
    DeltaNet (log_alpha None) through the chunkwise path; otherwise as
    kda_chunk_fwd."""
    return _chunk_fwd(q, k, v, log_alpha, beta, h0, cu_seqlens, o, h_T, output_final_state, workspace,
                      None, gdn=True)


def kda_chunk_fwd_decoupled(q, k, v, log_alpha, b_erase, w_write, h0=None, cu_seqlens=None, *, o=None,
                            h_T=None, output_final_state=True, workspace=None):
    """KDA with separate erase (b_erase) and write (w_write) strengths, both
    [B, T, H] in log_alpha's dtype; otherwise as kda_chunk_fwd."""
    return _chunk_fwd(q, k, v, log_alpha, b_erase, h0, cu_seqlens, o, h_T, output_final_state, workspace,
                      None, w_write=w_write)


def kda_chunk_fwd_prologue(q_raw, k_raw, v, gate_pre, beta_pre, log_alpha_min, h0=None,
                           cu_seqlens=None, *, o=None, h_T=None, output_final_state=True,
                           workspace=None):
    """kda_chunk_fwd on raw projections: the kernels apply q/|q|, k/|k|,
    log_alpha = max(-softplus(gate_pre), log_alpha_min) and beta = sigmoid(beta_pre)
    as they read the inputs.  Shapes and dtypes as for kda_chunk_fwd."""
    return _chunk_fwd(q_raw, k_raw, v, gate_pre, beta_pre, h0, cu_seqlens, o, h_T, output_final_state,
                      workspace, float(log_alpha_min))


def _chunk_fwd(q, k, v, log_alpha, beta, h0, cu_seqlens, o, h_T, output_final_state, workspace,
               log_alpha_min, gdn=False, w_write=None, noalloc=False):
    import torch
    lib = load_library()
    squeeze = q.dim() == 3
    if squeeze:
        q, k, v, beta = (x.unsqueeze(0) for x in (q, k, v, beta))
        if w_write is not None:
            w_write = w_write.unsqueeze(0)
        if log_alpha is not None:
            log_alpha = log_alpha.unsqueeze(0)
        if o is not None and o.dim() == 3:
            o = o.unsqueeze(0)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("log_alpha", log_alpha), ("beta", beta)):
        if t is not None or not gdn:
            _check_dev(name, t, dev)
    gshape = (B, T, H) if gdn else q.shape
    if k.shape != q.shape or (log_alpha is not None and log_alpha.shape != gshape) \
            or v.shape[:3] != (B, T, H) or beta.shape != (B, T, H):
        raise ValueError("shape mismatch among q, k, v, log_alpha, beta")
    if k.dtype != q.dtype or v.dtype != q.dtype or (log_alpha is not None and beta.dtype != log_alpha.dtype):
        raise TypeError("q, k, v share one dtype; log_alpha and beta share one dtype")
    if w_write is not None:
        _check_dev("w_write", w_write, dev)
        if w_write.shape != beta.shape or w_write.dtype != beta.dtype:
            raise ValueError("w_write must match beta in shape and dtype")
    if cu_seqlens is not None:
        _check_dev("cu_seqlens", cu_seqlens, dev)
        if cu_seqlens.dtype != torch.int32:
            raise TypeError("cu_seqlens must be int32")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if h0 is not None:
        _check_dev("h0", h0, dev)
        if h0.dtype != torch.float32 or tuple(h0.shape) != (N, H, dk, dv):
            raise ValueError("h0 must be fp32 [N, H, d_k, d_v]")
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    else:
        _check_out("o", o, dev, (B, T, H, dv), q.dtype)
    if h_T is None and output_final_state:
        h_T = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    elif h_T is not None:
        _check_out("h_T", h_T, dev, (N, H, dk, dv), torch.float32)
    io, gt = _dtype_code(q), _dtype_code(beta)
    nseq = N if cu_seqlens is not None else 0
    if noalloc:
        rc = lib.kda_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(h0),
                                       _ptr(cu_seqlens), nseq, _ptr(o), _ptr(h_T), B, T, H, dk, dv, io, gt,
                                       _stream_of(q))
        if rc != KDA_OK:
            raise KDAError(rc, "kda_chunk_fwd_noalloc", kda_last_hip_error())
        return (o.squeeze(0) if squeeze else o), h_T
    ws_bytes = kda_chunk_fwd_workspace_size(B, T, H, dk, dv, nseq, io)
    if workspace is not None:
        _check_out("workspace", workspace, dev)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if w_write is not None:
        name = "kda_chunk_fwd_decoupled"
        rc = lib.kda_chunk_fwd_decoupled(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(w_write),
                                         _ptr(h0), _ptr(cu_seqlens), nseq, _ptr(o), _ptr(h_T), B, T, H, dk, dv,
                                         io, gt, _ptr(workspace), ws_len, _stream_of(q))
    elif gdn:
        name = "kda_gdn_chunk_fwd"
        rc = lib.kda_gdn_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(h0),
                                   _ptr(cu_seqlens), nseq, _ptr(o), _ptr(h_T), B, T, H, dk, dv, io, gt,
                                   _ptr(workspace), ws_len, _stream_of(q))
    elif log_alpha_min is None:
        name = "kda_chunk_fwd"
        rc = lib.kda_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(h0),
                               _ptr(cu_seqlens), nseq, _ptr(o), _ptr(h_T), B, T, H, dk, dv, io, gt,
                               _ptr(workspace), ws_len, _stream_of(q))
    else:
        name = "kda_chunk_fwd_prologue"
        rc = lib.kda_chunk_fwd_prologue(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                        log_alpha_min, _ptr(h0), _ptr(cu_seqlens), nseq, _ptr(o),
                                        _ptr(h_T), B, T, H, dk, dv, io, gt, _ptr(workspace), ws_len,
                                        _stream_of(q))
    if rc != KDA_OK:
        raise KDAError(rc, name, kda_last_hip_error())
    if squeeze:
        o = o.squeeze(0)
    return o, h_T


def kda_chunk_bwd_workspace_size(B, T, H, d_k, d_v, num_seqs=0, io_dtype=KDA_BF16) -> int:
    return int(load_library().kda_chunk_bwd_workspace_size(B, T, H, d_k, d_v, num_seqs, io_dtype))


def kda_gdn_chunk_bwd_workspace_size(B, T, H, d_k, d_v, num_seqs=0, io_dtype=KDA_BF16) -> int:
    return int(load_library().kda_gdn_chunk_bwd_workspace_size(B, T, H, d_k, d_v, num_seqs, io_dtype))


def kda_chunk_bwd(q, k, v, log_alpha, beta, grad_o, h0=None, grad_hT=None, cu_seqlens=None, *,
                  want_grad_h0=True, workspace=None):
    """Gradients of kda_chunk_fwd (see kda_chunk_bwd in include/kda.h).

    Inputs as for kda_chunk_fwd plus grad_o (like o) and grad_hT (like h_T, or
    None).  Returns (dq, dk, dv, dlog_alpha, dbeta, dh0); dh0 is None when
    want_grad_h0 is False."""
    return _chunk_bwd(q, k, v, log_alpha, beta, grad_o, h0, grad_hT, cu_seqlens, want_grad_h0, workspace,
                      gdn=False)


def kda_gdn_chunk_bwd(q, k, v, log_alpha, beta, grad_o, h0=None, grad_hT=None, cu_seqlens=None, *,
                      want_grad_h0=True, workspace=None):
    """Gradients of kda_gdn_chunk_fwd: log_alpha is [B, T, H] or None (no
    decay).  Returns (dq, dk, dv, dlog_alpha, dbeta, dh0); dlog_alpha is None
    when log_alpha is None, dh0 when want_grad_h0 is False."""
    return _chunk_bwd(q, k, v, log_alpha, beta, grad_o, h0, grad_hT, cu_seqlens, want_grad_h0, workspace,
                      gdn=True)


def kda_chunk_bwd_prologue_workspace_size(B, T, H, d_k, d_v, num_seqs=0, io_dtype=KDA_BF16) -> int:
    return int(load_library().kda_chunk_bwd_prologue_workspace_size(B, T, H, d_k, d_v, num_seqs, io_dtype))


def kda_chunk_bwd_prologue(q_raw, k_raw, v, gate_pre, beta_pre, log_alpha_min, grad_o, h0=None, grad_hT=None,
                           cu_seqlens=None, *, want_grad_h0=True, workspace=None):
    """Gradients of kda_chunk_fwd_prologue with respect to its raw inputs.
    Returns (dq_raw, dk_raw, dv, dgate_pre, dbeta_pre, dh0); dh0 is None when
    want_grad_h0 is False."""
    return _chunk_bwd(q_raw, k_raw, v, gate_pre, beta_pre, grad_o, h0, grad_hT, cu_seqlens, want_grad_h0,
                      workspace, gdn=False, log_alpha_min=float(log_alpha_min))


def kda_chunk_bwd_decoupled(q, k, v, log_alpha, b_erase, w_write, grad_o, h0=None, grad_hT=None, cu_seqlens=None,
                            *, want_grad_h0=True, workspace=None):
    """Gradients of kda_chunk_fwd_decoupled: b_erase and w_write [B, T, H] in
    log_alpha's dtype.  Returns (dq, dk, dv, dlog_alpha, db_erase, dw_write, dh0);
    dh0 is None when want_grad_h0 is False."""
    return _chunk_bwd(q, k, v, log_alpha, b_erase, grad_o, h0, grad_hT, cu_seqlens, want_grad_h0, workspace,
                      gdn=False, w_write=w_write)


def _chunk_bwd(q, k, v, log_alpha, beta, grad_o, h0, grad_hT, cu_seqlens, want_grad_h0, workspace, gdn,
               w_write=None, log_alpha_min=None):
    import torch
    lib = load_library()
    squeeze = q.dim() == 3
    if squeeze:
        q, k, v, beta, grad_o = (x.unsqueeze(0) for x in (q, k, v, beta, grad_o))
        if log_alpha is not None:
            log_alpha = log_alpha.unsqueeze(0)
        if w_write is not None:
            w_write = w_write.unsqueeze(0)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if log_alpha is None and not gdn:
        raise ValueError("log_alpha is required")
    for name, t in (("q", q), ("k", k), ("v", v), ("log_alpha", log_alpha), ("beta", beta),
                    ("grad_o", grad_o)):
        if t is not None:
            _check_dev(name, t, dev)
    gshape = (B, T, H) if gdn else q.shape
    if k.shape != q.shape or (log_alpha is not None and log_alpha.shape != gshape) \
            or v.shape[:3] != (B, T, H) or beta.shape != (B, T, H) or grad_o.shape != v.shape:
        raise ValueError("shape mismatch among q, k, v, log_alpha, beta, grad_o")
    if k.dtype != q.dtype or v.dtype != q.dtype or grad_o.dtype != q.dtype \
            or (log_alpha is not None and beta.dtype != log_alpha.dtype):
        raise TypeError("q, k, v, grad_o share one dtype; log_alpha and beta share one dtype")
    if w_write is not None:
        _check_dev("w_write", w_write, dev)
        if w_write.shape != beta.shape or w_write.dtype != beta.dtype:
            raise ValueError("w_write must match b_erase in shape and dtype")
    if cu_seqlens is not None:
        _check_dev("cu_seqlens", cu_seqlens, dev)
        if cu_seqlens.dtype != torch.int32:
            raise TypeError("cu_seqlens must be int32")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    for name, t in (("h0", h0), ("grad_hT", grad_hT)):
        if t is not None:
            _check_dev(name, t, dev)
            if t.dtype != torch.float32 or tuple(t.shape) != (N, H, dk, dv):
                raise ValueError("%s must be fp32 [N, H, d_k, d_v]" % name)
    dq = torch.empty_like(q)
    dk_ = torch.empty_like(k)
    dv_ = torch.empty_like(v)
    dla = torch.empty_like(log_alpha) if log_alpha is not None else None
    db = torch.empty_like(beta)
    dh0 = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev) if want_grad_h0 else None
    io, gt = _dtype_code(q), _dtype_code(beta)
    nseq = N if cu_seqlens is not None else 0
    size_fn = kda_gdn_chunk_bwd_workspace_size if gdn else (
        kda_chunk_bwd_prologue_workspace_size if log_alpha_min is not None else kda_chunk_bwd_workspace_size)
    ws_bytes = size_fn(B, T, H, dk, dv, nseq, io)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    else:
        _check_out("workspace", workspace, dev)
    ws_len = workspace.numel() * workspace.element_size()
    if log_alpha_min is not None:
        name = "kda_chunk_bwd_prologue"
        rc = lib.kda_chunk_bwd_prologue(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), log_alpha_min,
                                        _ptr(h0), _ptr(cu_seqlens), nseq, _ptr(grad_o), _ptr(grad_hT), _ptr(dq),
                                        _ptr(dk_), _ptr(dv_), _ptr(dla), _ptr(db), _ptr(dh0), B, T, H, dk, dv, io,
                                        gt, _ptr(workspace), ws_len, _stream_of(q))
    elif w_write is not None:
        name = "kda_chunk_bwd_decoupled"
        dw = torch.empty_like(w_write)
        rc = lib.kda_chunk_bwd_decoupled(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(w_write),
                                         _ptr(h0), _ptr(cu_seqlens), nseq, _ptr(grad_o), _ptr(grad_hT), _ptr(dq),
                                         _ptr(dk_), _ptr(dv_), _ptr(dla), _ptr(db), _ptr(dw), _ptr(dh0), B, T, H,
                                         dk, dv, io, gt, _ptr(workspace), ws_len, _stream_of(q))
    else:
        name = "kda_gdn_chunk_bwd" if gdn else "kda_chunk_bwd"
        rc = getattr(lib, name)(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(h0),
                                _ptr(cu_seqlens), nseq, _ptr(grad_o), _ptr(grad_hT), _ptr(dq), _ptr(dk_),
                                _ptr(dv_), _ptr(dla), _ptr(db), _ptr(dh0), B, T, H, dk, dv, io, gt,
                                _ptr(workspace), ws_len, _stream_of(q))
    if rc != KDA_OK:
        raise KDAError(rc, name, kda_last_hip_error())
    if squeeze:
        dq, dk_, dv_, db = (x.squeeze(0) for x in (dq, dk_, dv_, db))
        if dla is not None:
            dla = dla.squeeze(0)
        if w_write is not None:
            dw = dw.squeeze(0)
    if w_write is not None:
        return dq, dk_, dv_, dla, db, dw, dh0
    return dq, dk_, dv_, dla, db, dh0


def kda_decode_step(q, k, v, log_alpha, beta, S, o=None):
    """One decode step.  q, k, log_alpha: [B, H, d_k]; v: [B, H, d_v];
    beta: [B, H]; S: [B, H, d_k, d_v] fp32, updated in place.  Returns o."""
    return _decode_step(q, k, v, log_alpha, beta, S, o, None)


def kda_gdn_decode_step(q, k, v, log_alpha, beta, S, o=None):
    """Decode step with a scalar gate: log_alpha [B, H] or None (no decay)."""
    return _decode_step(q, k, v, log_alpha, beta, S, o, None, gdn=True)


def kda_decode_step_decoupled(q, k, v, log_alpha, b_erase, w_write, S, o=None):
    """Decode step with separate erase and write strengths ([B, H] each)."""
    return _decode_step(q, k, v, log_alpha, b_erase, S, o, None, w_write=w_write)


def kda_decode_step_prologue(q_raw, k_raw, v, gate_pre, beta_pre, log_alpha_min, S, o=None):
    """kda_decode_step on raw projections (the maps of kda_chunk_fwd_prologue)."""
    return _decode_step(q_raw, k_raw, v, gate_pre, beta_pre, S, o, float(log_alpha_min))


def _decode_step(q, k, v, log_alpha, beta, S, o, log_alpha_min, gdn=False, w_write=None):
    import torch
    lib = load_library()
    B, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("log_alpha", log_alpha), ("beta", beta),
                    ("S", S)):
        if t is not None or not gdn:
            _check_dev(name, t, dev)
    if log_alpha is not None and tuple(log_alpha.shape) != ((B, H) if gdn else (B, H, dk)):
        raise ValueError("log_alpha has the wrong shape")
    if k.shape != q.shape or v.dim() != 3 or tuple(v.shape[:2]) != (B, H) or tuple(beta.shape) != (B, H):
        raise ValueError("shape mismatch among q, k, v, beta")
    if k.dtype != q.dtype or v.dtype != q.dtype or (log_alpha is not None and log_alpha.dtype != beta.dtype):
        raise TypeError("q, k, v share one dtype; log_alpha and beta share one dtype")
    if w_write is not None:
        _check_dev("w_write", w_write, dev)
        if w_write.shape != beta.shape or w_write.dtype != beta.dtype:
            raise ValueError("w_write must match beta in shape and dtype")
    if S.dtype != torch.float32 or tuple(S.shape) != (B, H, dk, dv):
        raise ValueError("S must be fp32 [B, H, d_k, d_v]")
    if o is None:
        o = torch.empty((B, H, dv), dtype=q.dtype, device=dev)
    else:
        _check_out("o", o, dev, (B, H, dv), q.dtype)
    if w_write is not None:
        name = "kda_decode_step_decoupled"
        rc = lib.kda_decode_step_decoupled(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                           _ptr(w_write), _ptr(S), _ptr(o), B, H, dk, dv, _dtype_code(q),
                                           _dtype_code(beta), _stream_of(q))
    elif gdn:
        name = "kda_gdn_decode_step"
        rc = lib.kda_gdn_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S),
                                     _ptr(o), B, H, dk, dv, _dtype_code(q), _dtype_code(beta),
                                     _stream_of(q))
    elif log_alpha_min is None:
        name = "kda_decode_step"
        rc = lib.kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S),
                                 _ptr(o), B, H, dk, dv, _dtype_code(q), _dtype_code(log_alpha),
                                 _stream_of(q))
    else:
        name = "kda_decode_step_prologue"
        rc = lib.kda_decode_step_prologue(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                          log_alpha_min, _ptr(S), _ptr(o), B, H, dk, dv,
                                          _dtype_code(q), _dtype_code(log_alpha), _stream_of(q))
    if rc != KDA_OK:
        raise KDAError(rc, name, kda_last_hip_error())
    return o


chunk_fwd = kda_chunk_fwd
decode_step = kda_decode_step
chunk_fwd_prologue = kda_chunk_fwd_prologue
decode_step_prologue = kda_decode_step_prologue
gdn_chunk_fwd = kda_gdn_chunk_fwd
gdn_decode_step = kda_gdn_decode_step
chunk_fwd_decoupled = kda_chunk_fwd_decoupled
decode_step_decoupled = kda_decode_step_decoupled


# ---------------------------------------------------------------- autograd
# Training use from PyTorch: the forward is kda_chunk_fwd (or kda_gdn_chunk_fwd)
# and the backward kda_chunk_bwd (or kda_gdn_chunk_bwd); these wrappers only
# connect the two to torch.autograd.
def _autograd_function():
    import torch

    class _ChunkKDA(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, log_alpha, beta, h0, cu_seqlens, gdn):
            fwd = kda_gdn_chunk_fwd if gdn else kda_chunk_fwd
            o, h_T = fwd(q, k, v, log_alpha, beta, h0=h0, cu_seqlens=cu_seqlens)
            ctx.save_for_backward(q, k, v, log_alpha, beta, h0, cu_seqlens)
            ctx.gdn = gdn
            return o, h_T

        @staticmethod
        def backward(ctx, grad_o, grad_hT):
            q, k, v, log_alpha, beta, h0, cu_seqlens = ctx.saved_tensors
            if grad_o is None:
                grad_o = torch.zeros(v.shape, dtype=v.dtype, device=v.device)
            bwd = kda_gdn_chunk_bwd if ctx.gdn else kda_chunk_bwd
            dq, dk, dv, dla, db, dh0 = bwd(q, k, v, log_alpha, beta, grad_o.contiguous(), h0=h0,
                                           grad_hT=None if grad_hT is None else grad_hT.contiguous(),
                                           cu_seqlens=cu_seqlens, want_grad_h0=h0 is not None and ctx.needs_input_grad[5])
            return dq, dk, dv, dla, db, dh0, None, None

    return _ChunkKDA


_CHUNK_KDA = None


def chunk_kda(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None):
    """KDA prefill with autograd: returns (o, h_T) as kda_chunk_fwd does, and
    gradients flow to q, k, v, log_alpha, beta and h0 through kda_chunk_bwd."""
    global _CHUNK_KDA
    if _CHUNK_KDA is None:
        _CHUNK_KDA = _autograd_function()
    return _CHUNK_KDA.apply(q, k, v, log_alpha, beta, h0, cu_seqlens, False)


def chunk_gated_delta_rule(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None):
    """Gated DeltaNet (log_alpha [.., H]) or DeltaNet (log_alpha None) prefill
    with autograd, through kda_gdn_chunk_fwd and kda_gdn_chunk_bwd."""
    global _CHUNK_KDA
    if _CHUNK_KDA is None:
        _CHUNK_KDA = _autograd_function()
    return _CHUNK_KDA.apply(q, k, v, log_alpha, beta, h0, cu_seqlens, True)
