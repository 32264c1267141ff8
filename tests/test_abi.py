"""CPU tests of the C-ABI boundary: the library loads, exports every symbol its
header declares, and rejects invalid arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def kda():
    import gated_delta_rule_chunkwise_amd as kda
    if not os.path.exists(kda.LIB_PATH):
        from gated_delta_rule_chunkwise_amd import build
        build.build()
    kda.load_library()
    return kda


def header_functions():
    src = open(os.path.join(ROOT, "include", "kda.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol(kda):
    names = header_functions()
    assert "kda_chunk_fwd" in names and "kda_decode_step" in names
    lib = ctypes.CDLL(kda.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(kda.EXPORTED_SYMBOLS)


def test_version_and_status_strings(kda):
    assert kda.kda_abi_version() == 1
    assert kda.kda_status_string(0) == "KDA_OK"
    assert kda.kda_status_string(2) == "KDA_ERR_UNSUPPORTED"
    assert kda.kda_status_string(99) == "KDA_ERR_UNKNOWN"
    assert kda.kda_last_hip_error() == ""


def seg_state_bytes(chains, nseg, dk=128, dv=128):
    """Per (chain, segment): start state, end state from zero (fp32 d_k x d_v) and
    the segment's transition (fp32 d_k x d_k)."""
    return chains * nseg * (2 * dk * dv + dk * dk) * 4


def test_workspace_size(kda):
    # bf16 I/O at d_k = d_v = 128: the query covers both forward paths (the input
    # variants run the fused kernel, plain KDA the two-kernel path), so it is at
    # least the fused kernel's segment states (chains split into segments to fill
    # the GPU: about 256 workgroups, segments of at least 4 chunks, at least 3 of
    # them) and at least the two-kernel records (below)
    W = lambda *a: kda.kda_chunk_fwd_workspace_size(*a)
    assert W(1, 1000, 2, 128, 128, 5, kda.KDA_BF16) == 256   # packed: the fused kernel's sequence order
    assert W(1, 65536, 32, 128, 128, 0, kda.KDA_BF16) >= seg_state_bytes(32, 8)
    assert W(2, 65536, 32, 128, 128, 0, kda.KDA_BF16) >= seg_state_bytes(64, 4)
    assert W(1, 4096, 16, 128, 128, 0, kda.KDA_BF16) >= seg_state_bytes(16, 16)
    # bf16 I/O at other dimensions (two-kernel path): one per-chunk record per
    # (chunk, head), at least the decayed keys, queries and transposed keys
    # (3 x 64 x d_k bf16) and at most ~96 KiB per chunk-head, plus a small header
    two = W(2, 65536, 32, 64, 64, 0, kda.KDA_BF16)
    assert 2 * 1024 * 32 * (3 * 64 * 64 * 2) <= two <= 2 * 1024 * 32 * 96 * 1024 + 4096
    # one long sequence runs in segments of at most 2048 chunk-heads of records,
    # plus the fp32 state carried between them
    big = W(1, 65536, 32, 64, 64, 0, kda.KDA_BF16)
    carry = 32 * 64 * 64 * 4
    assert 2048 * (3 * 64 * 64 * 2) + carry <= big <= 2048 * 96 * 1024 + carry + 4096
    # fp32 I/O: none at d_k = 64 (one fused kernel); at d_k = 128 the chunkwise
    # fp32 path keeps per chunk-head its fp32 record (3 x 64 x d_k + 3 x 64 x 64
    # + 3 x d_k floats), the chunk's start state and U, and per token-head the
    # input prologue's mapped q, k, log alpha and beta
    assert W(1, 65536, 32, 64, 64, 0, kda.KDA_F32) == 0
    per = 4 * (3 * 64 * 128 + 3 * 64 * 64 + 3 * 128 + 128 * 128 + 64 * 128) + 64 * 4 * (3 * 128 + 3)
    f32 = W(1, 4096, 16, 128, 128, 0, kda.KDA_F32)
    assert 64 * 16 * per <= f32 <= 64 * 16 * (per + 1024) + 4096
    assert W(1, 0, 16, 128, 128, 0, kda.KDA_F32) == 0     # no tokens: h_T = h0 only
    assert W(1, 100, 2, 96, 128, 0, kda.KDA_BF16) == 0
    # varlen: room for one partial chunk per sequence
    v1 = W(1, 1000, 2, 64, 64, 5, kda.KDA_BF16)
    v0 = W(1, 1000, 2, 64, 64, 0, kda.KDA_BF16)
    assert v1 > v0 > 0


def test_chunk_fwd_requires_workspace(kda):
    lib = kda.load_library()
    # a single sequence of 64 chunks at H = 2 runs in segments: it needs workspace
    need = kda.kda_chunk_fwd_workspace_size(1, 4096, 2, 128, 128, 0, kda.KDA_BF16)
    assert need > 0
    assert chunk(lib, T=4096, ws=None, wsb=0) == 3
    assert chunk(lib, T=4096, ws=P, wsb=need - 1) == 3
    assert chunk(lib, T=4096, ws=P + 8, wsb=need) == 1   # misaligned workspace


P = 1 << 20   # a fake, 16-byte aligned "device" address; never dereferenced


def chunk(lib, **kw):
    a = dict(q=P, k=P, v=P, la=P, beta=P, h0=None, cu=None, N=0, o=P, hT=P, B=1, T=4096, H=2,
             dk=128, dv=128, io=1, gt=1, ws=None, wsb=0)
    a.update(kw)
    return lib.kda_chunk_fwd(a["q"], a["k"], a["v"], a["la"], a["beta"], a["h0"], a["cu"], a["N"],
                             a["o"], a["hT"], a["B"], a["T"], a["H"], a["dk"], a["dv"], a["io"],
                             a["gt"], a["ws"], a["wsb"], None)


def decode(lib, **kw):
    a = dict(q=P, k=P, v=P, la=P, beta=P, S=P, o=P, B=4, H=2, dk=128, dv=128, io=1, gt=1)
    a.update(kw)
    return lib.kda_decode_step(a["q"], a["k"], a["v"], a["la"], a["beta"], a["S"], a["o"], a["B"],
                               a["H"], a["dk"], a["dv"], a["io"], a["gt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dk=96), 2), (dict(dv=32), 2), (dict(dk=0), 1), (dict(io=5), 2), (dict(gt=-1), 2),
    (dict(B=0), 1), (dict(T=-1), 1), (dict(H=0), 1),
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(la=None), 1),
    (dict(beta=None), 1), (dict(o=None), 1),
    (dict(q=P + 4), 1), (dict(o=P + 8), 1), (dict(h0=P + 2), 1), (dict(hT=P + 4), 1),
    (dict(beta=P + 1), 1), (dict(beta=P + 2, gt=0), 1),
    (dict(cu=P, N=2, B=2), 1), (dict(cu=P, N=0), 1), (dict(cu=P + 2, N=2), 1),
    (dict(N=3), 1), (dict(B=2, N=3), 1),
    (dict(T=1 << 30, H=1 << 20), 1),
])
def test_chunk_fwd_rejects(kda, kw, code):
    lib = kda.load_library()
    assert chunk(lib, **kw) == code


def test_chunk_fwd_empty_without_state_is_noop(kda):
    lib = kda.load_library()
    assert chunk(lib, T=0, q=None, k=None, v=None, la=None, beta=None, o=None, hT=None) == 0


def test_calls_beyond_the_launch_limits_are_refused(kda):
    """HIP launches at most 2^32 work-items per grid: at N * H = 2^19 chains of
    d_v = 128 the forward's state kernel (1024 threads over 8 value-column
    blocks per chain) would need 2^32, so the call is refused with
    KDA_ERR_UNSUPPORTED before anything is enqueued (the fake pointers are
    never touched).  Likewise the decode step at B * H = 2^24 (256 threads per
    chain) and the backward at N * H = 2^20."""
    lib = kda.load_library()
    assert chunk(lib, B=1 << 14, H=32, T=64, ws=P, wsb=1 << 62) == 2
    assert chunk(lib, B=(1 << 14) - 8, H=32, T=64, ws=None, wsb=0) == 3   # just below: only the workspace is missing
    assert decode(lib, B=1 << 19, H=32) == 2
    assert bwd(lib, B=1 << 15, H=32, T=64, ws=P, wsb=1 << 62) == 2
    assert bwd(lib, B=(1 << 15) - 8, H=32, T=64, ws=None, wsb=0) == 3


def chunk_noalloc(lib, **kw):
    a = dict(q=P, k=P, v=P, la=P, beta=P, h0=None, cu=None, N=0, o=P, hT=P, B=1, T=4096, H=2,
             dk=128, dv=128, io=1, gt=1)
    a.update(kw)
    return lib.kda_chunk_fwd_noalloc(a["q"], a["k"], a["v"], a["la"], a["beta"], a["h0"], a["cu"], a["N"],
                                     a["o"], a["hT"], a["B"], a["T"], a["H"], a["dk"], a["dv"], a["io"],
                                     a["gt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dk=96), 2), (dict(io=5), 2), (dict(B=0), 1), (dict(T=-1), 1), (dict(q=None), 1),
    (dict(o=P + 8), 1), (dict(h0=P + 2), 1), (dict(beta=P + 1), 1), (dict(cu=P, N=2, B=2), 1),
    (dict(N=3), 1), (dict(T=1 << 30, H=1 << 20), 1),
])
def test_chunk_fwd_noalloc_validates_like_chunk_fwd(kda, kw, code):
    lib = kda.load_library()
    assert chunk_noalloc(lib, **kw) == code == chunk(lib, **kw)


def test_chunk_fwd_noalloc_rejects_calls_beyond_its_scratch(kda):
    """bf16 at d = 64 runs the two-pass forward, whose per-chunk records for a
    long batch exceed the 80 MiB scratch: KDA_ERR_WORKSPACE before any launch."""
    lib = kda.load_library()
    need = kda.kda_chunk_fwd_workspace_size(8, 8192, 32, 64, 64, 0, kda.KDA_BF16)
    assert need > 80 << 20
    assert chunk_noalloc(lib, B=8, T=8192, H=32, dk=64, dv=64) == 3
    assert chunk_noalloc(lib, B=8, T=8192, H=32, dk=128, dv=64) == 3


def test_chunk_fwd_noalloc_empty_without_state_is_noop(kda):
    lib = kda.load_library()
    assert chunk_noalloc(lib, T=0, q=None, k=None, v=None, la=None, beta=None, o=None, hT=None) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(dk=32), 2), (dict(dv=256), 2), (dict(B=0), 1), (dict(H=-1), 1), (dict(io=3), 2),
    (dict(S=None), 1), (dict(q=None), 1), (dict(o=None), 1), (dict(beta=None), 1),
    (dict(S=P + 4), 1), (dict(k=P + 2), 1), (dict(beta=P + 1), 1),
])
def test_decode_rejects(kda, kw, code):
    lib = kda.load_library()
    assert decode(lib, **kw) == code


def test_binding_raises_without_gpu_tensors(kda):
    import torch
    x = torch.zeros(1, 64, 2, 64)
    b = torch.zeros(1, 64, 2)
    with pytest.raises(ValueError):
        kda.kda_chunk_fwd(x, x, x, x, b)
    with pytest.raises(ValueError):
        kda.kda_chunk_bwd(x, x, x, x, b, x)
    with pytest.raises(ValueError):
        kda.chunk_kda(x, x, x, x, b)
    s = torch.zeros(3, 2, 64)
    with pytest.raises(ValueError):
        kda.kda_decode_step(s, s, s, s, torch.zeros(3, 2), torch.zeros(3, 2, 64, 64))


def chunk_pro(lib, lo=-20.0, **kw):
    a = dict(q=P, k=P, v=P, la=P, beta=P, h0=None, cu=None, N=0, o=P, hT=P, B=1, T=4096, H=2,
             dk=128, dv=128, io=1, gt=1, ws=None, wsb=0)
    a.update(kw)
    return lib.kda_chunk_fwd_prologue(a["q"], a["k"], a["v"], a["la"], a["beta"], lo, a["h0"], a["cu"],
                                      a["N"], a["o"], a["hT"], a["B"], a["T"], a["H"], a["dk"], a["dv"],
                                      a["io"], a["gt"], a["ws"], a["wsb"], None)


def decode_pro(lib, lo=-20.0, **kw):
    a = dict(q=P, k=P, v=P, la=P, beta=P, S=P, o=P, B=4, H=2, dk=128, dv=128, io=1, gt=1)
    a.update(kw)
    return lib.kda_decode_step_prologue(a["q"], a["k"], a["v"], a["la"], a["beta"], lo, a["S"], a["o"],
                                        a["B"], a["H"], a["dk"], a["dv"], a["io"], a["gt"], None)


@pytest.mark.parametrize("lo", [float("nan"), float("inf"), float("-inf"), 0.5, 1e-30])
def test_prologue_rejects_bad_floor(kda, lo):
    lib = kda.load_library()
    need = kda.kda_chunk_fwd_workspace_size(1, 4096, 2, 128, 128, 0, kda.KDA_BF16)
    assert chunk_pro(lib, lo=lo, ws=P, wsb=need) == 1
    assert decode_pro(lib, lo=lo) == 1


@pytest.mark.parametrize("kw,code", [
    (dict(dk=96), 2), (dict(io=5), 2), (dict(B=0), 1), (dict(q=None), 1), (dict(la=None), 1),
    (dict(beta=P + 1), 1), (dict(cu=P, N=2, B=2), 1), (dict(ws=None, wsb=0), 3),
])
def test_chunk_fwd_prologue_validates_like_chunk_fwd(kda, kw, code):
    lib = kda.load_library()
    need = kda.kda_chunk_fwd_workspace_size(1, 4096, 2, 128, 128, 0, kda.KDA_BF16)
    a = dict(ws=P, wsb=need)
    a.update(kw)
    assert chunk_pro(lib, lo=0.0, **a) == code
    assert chunk(lib, **a) == code


@pytest.mark.parametrize("kw,code", [
    (dict(dk=32), 2), (dict(B=0), 1), (dict(S=None), 1), (dict(k=P + 2), 1),
])
def test_decode_prologue_validates_like_decode(kda, kw, code):
    lib = kda.load_library()
    assert decode_pro(lib, **kw) == code
    assert decode(lib, **kw) == code


def chunk_gdn(lib, **kw):
    a = dict(q=P, k=P, v=P, la=P, beta=P, h0=None, cu=None, N=0, o=P, hT=P, B=1, T=4096, H=2,
             dk=128, dv=128, io=1, gt=1, ws=None, wsb=0)
    a.update(kw)
    return lib.kda_gdn_chunk_fwd(a["q"], a["k"], a["v"], a["la"], a["beta"], a["h0"], a["cu"], a["N"],
                                 a["o"], a["hT"], a["B"], a["T"], a["H"], a["dk"], a["dv"], a["io"],
                                 a["gt"], a["ws"], a["wsb"], None)


def decode_gdn(lib, **kw):
    a = dict(q=P, k=P, v=P, la=P, beta=P, S=P, o=P, B=4, H=2, dk=128, dv=128, io=1, gt=1)
    a.update(kw)
    return lib.kda_gdn_decode_step(a["q"], a["k"], a["v"], a["la"], a["beta"], a["S"], a["o"], a["B"],
                                   a["H"], a["dk"], a["dv"], a["io"], a["gt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dk=96), 2), (dict(B=0), 1), (dict(q=None), 1), (dict(beta=None), 1),
    (dict(la=P + 1), 1), (dict(la=P + 2, gt=0), 1), (dict(cu=P, N=2, B=2), 1), (dict(ws=None, wsb=0), 3),
])
def test_gdn_chunk_fwd_validates(kda, kw, code):
    lib = kda.load_library()
    need = kda.kda_chunk_fwd_workspace_size(1, 4096, 2, 128, 128, 0, kda.KDA_BF16)
    a = dict(ws=P, wsb=need)
    a.update(kw)
    assert chunk_gdn(lib, **a) == code


def test_gdn_gate_alignment_is_element_size(kda):
    # a scalar gate is [B, T, H]: aligned to its element, not to 16 bytes; the
    # per-channel entry point still needs 16 bytes
    lib = kda.load_library()
    assert decode_gdn(lib, la=P + 2, S=None) == 1      # rejected for the missing state only
    assert decode_gdn(lib, la=P + 1, gt=1) == 1
    assert decode_gdn(lib, la=P + 2, gt=0) == 1
    assert decode(lib, la=P + 2, S=None) == 1


@pytest.mark.parametrize("kw,code", [
    (dict(dk=32), 2), (dict(B=0), 1), (dict(S=None), 1), (dict(k=P + 2), 1), (dict(beta=P + 1), 1),
])
def test_gdn_decode_validates(kda, kw, code):
    lib = kda.load_library()
    assert decode_gdn(lib, **kw) == code


def chunk_dec(lib, wwr=P, **kw):
    a = dict(q=P, k=P, v=P, la=P, beta=P, h0=None, cu=None, N=0, o=P, hT=P, B=1, T=4096, H=2,
             dk=128, dv=128, io=1, gt=1, ws=None, wsb=0)
    a.update(kw)
    return lib.kda_chunk_fwd_decoupled(a["q"], a["k"], a["v"], a["la"], a["beta"], wwr, a["h0"], a["cu"],
                                       a["N"], a["o"], a["hT"], a["B"], a["T"], a["H"], a["dk"], a["dv"],
                                       a["io"], a["gt"], a["ws"], a["wsb"], None)


def decode_dec(lib, wwr=P, **kw):
    a = dict(q=P, k=P, v=P, la=P, beta=P, S=P, o=P, B=4, H=2, dk=128, dv=128, io=1, gt=1)
    a.update(kw)
    return lib.kda_decode_step_decoupled(a["q"], a["k"], a["v"], a["la"], a["beta"], wwr, a["S"], a["o"],
                                         a["B"], a["H"], a["dk"], a["dv"], a["io"], a["gt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(wwr=None), 1), (dict(wwr=P + 1), 1), (dict(wwr=P + 2, gt=0), 1),
    (dict(dk=96), 2), (dict(B=0), 1), (dict(la=None), 1), (dict(la=P + 4), 1), (dict(beta=P + 1), 1),
    (dict(ws=None, wsb=0), 3),
])
def test_decoupled_chunk_fwd_validates(kda, kw, code):
    lib = kda.load_library()
    need = kda.kda_chunk_fwd_workspace_size(1, 4096, 2, 128, 128, 0, kda.KDA_BF16)
    a = dict(ws=P, wsb=need)
    a.update(kw)
    assert chunk_dec(lib, **a) == code


@pytest.mark.parametrize("kw,code", [
    (dict(wwr=None), 1), (dict(wwr=P + 1), 1), (dict(dk=32), 2), (dict(S=None), 1), (dict(la=P + 2), 1),
])
def test_decoupled_decode_validates(kda, kw, code):
    lib = kda.load_library()
    assert decode_dec(lib, **kw) == code


def bwd(lib, **kw):
    a = dict(q=P, k=P, v=P, la=P, beta=P, h0=None, cu=None, N=0, go=P, ghT=None, dq=P, dk=P, dv=P,
             dla=P, db=P, dh0=P, B=1, T=128, H=2, dk_=128, dv_=128, io=1, gt=1, ws=P, wsb=1 << 40)
    a.update(kw)
    return lib.kda_chunk_bwd(a["q"], a["k"], a["v"], a["la"], a["beta"], a["h0"], a["cu"], a["N"],
                             a["go"], a["ghT"], a["dq"], a["dk"], a["dv"], a["dla"], a["db"], a["dh0"],
                             a["B"], a["T"], a["H"], a["dk_"], a["dv_"], a["io"], a["gt"], a["ws"],
                             a["wsb"], None)


def test_bwd_workspace_size(kda):
    # per chunk-head: the fp32 record (3 x 64 x d_k + 3 x 64 x 64 + 3 x d_k floats),
    # the state and state gradient (2 x d_k x d_v) and U, dU (2 x 64 x d_v), fp32
    per = 4 * (3 * 64 * 128 + 3 * 64 * 64 + 3 * 128 + 2 * 128 * 128 + 2 * 64 * 128)
    w = kda.kda_chunk_bwd_workspace_size(1, 65536, 32, 128, 128, 0, kda.KDA_BF16)
    assert 1024 * 32 * per <= w <= 1024 * 32 * (per + 1024) + 65536
    assert kda.kda_chunk_bwd_workspace_size(1, 65536, 32, 128, 128, 0, kda.KDA_F32) == w
    assert kda.kda_chunk_bwd_workspace_size(1, 100, 2, 96, 128, 0, kda.KDA_BF16) == 0
    assert kda.kda_chunk_bwd_workspace_size(2, 100, 2, 64, 64, 3, kda.KDA_BF16) == 0
    v1 = kda.kda_chunk_bwd_workspace_size(1, 1000, 2, 64, 64, 5, kda.KDA_BF16)
    v0 = kda.kda_chunk_bwd_workspace_size(1, 1000, 2, 64, 64, 0, kda.KDA_BF16)
    assert v1 > v0 > 0


@pytest.mark.parametrize("kw,code", [
    (dict(dk_=96), 2), (dict(dv_=32), 2), (dict(io=4), 2), (dict(gt=9), 2),
    (dict(B=0), 1), (dict(T=-1), 1), (dict(H=0), 1),
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(la=None), 1), (dict(beta=None), 1),
    (dict(go=None), 1), (dict(dq=None), 1), (dict(dk=None), 1), (dict(dv=None), 1), (dict(dla=None), 1),
    (dict(db=None), 1),
    (dict(q=P + 4), 1), (dict(go=P + 8), 1), (dict(dv=P + 2), 1), (dict(dla=P + 4), 1),
    (dict(h0=P + 4), 1), (dict(ghT=P + 8), 1), (dict(dh0=P + 2), 1), (dict(beta=P + 1), 1),
    (dict(db=P + 2, gt=0), 1),
    (dict(cu=P, N=2, B=2), 1), (dict(cu=P, N=0), 1), (dict(cu=P + 2, N=2), 1), (dict(N=3), 1),
    (dict(ws=None), 3), (dict(wsb=0), 3), (dict(ws=P + 8), 1),
    (dict(T=1 << 30, H=1 << 20), 2), (dict(H=65536, T=1), 2),
])
def test_bwd_rejects(kda, kw, code):
    lib = kda.load_library()
    assert bwd(lib, **kw) == code


def test_bwd_empty_without_state_is_noop(kda):
    lib = kda.load_library()
    assert bwd(lib, T=0, q=None, k=None, v=None, la=None, beta=None, go=None, dq=None, dk=None, dv=None,
               dla=None, db=None, dh0=None) == 0


def bwd_gdn(lib, **kw):
    a = dict(q=P, k=P, v=P, la=P, beta=P, h0=None, cu=None, N=0, go=P, ghT=None, dq=P, dk=P, dv=P,
             dla=P, db=P, dh0=P, B=1, T=128, H=2, dk_=128, dv_=128, io=1, gt=1, ws=P, wsb=1 << 40)
    a.update(kw)
    return lib.kda_gdn_chunk_bwd(a["q"], a["k"], a["v"], a["la"], a["beta"], a["h0"], a["cu"], a["N"],
                                 a["go"], a["ghT"], a["dq"], a["dk"], a["dv"], a["dla"], a["db"], a["dh0"],
                                 a["B"], a["T"], a["H"], a["dk_"], a["dv_"], a["io"], a["gt"], a["ws"],
                                 a["wsb"], None)


def test_gdn_bwd_workspace_size(kda):
    # the scalar-gate backward runs the per-channel backward's kernels with the
    # gate read per (token, head): the same workspace
    for d_k in (64, 128):
        assert kda.kda_gdn_chunk_bwd_workspace_size(1, 1000, 2, d_k, 64, 0, kda.KDA_BF16) == \
            kda.kda_chunk_bwd_workspace_size(1, 1000, 2, d_k, 64, 0, kda.KDA_BF16)
    assert kda.kda_gdn_chunk_bwd_workspace_size(1, 100, 2, 96, 128, 0, kda.KDA_BF16) == 0
    assert kda.kda_gdn_chunk_bwd_workspace_size(1, 100, 65536, 64, 64, 0, kda.KDA_BF16) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(dk_=96), 2), (dict(B=0), 1), (dict(H=65536, T=1), 2), (dict(q=None), 1), (dict(go=None), 1),
    (dict(beta=None), 1), (dict(db=None), 1),
    (dict(la=P + 1), 1), (dict(la=P + 2, gt=0), 1), (dict(dla=None), 1), (dict(dla=P + 1), 1),
    (dict(dla=P + 2, gt=0), 1), (dict(cu=P, N=2, B=2), 1), (dict(ws=None), 3),
])
def test_gdn_bwd_rejects(kda, kw, code):
    lib = kda.load_library()
    assert bwd_gdn(lib, **kw) == code


def test_gdn_bwd_gate_alignment_is_element_size(kda):
    # a [B, T, H] gate and its gradient are accepted at element alignment: with
    # both at P + 2 (bf16) the call gets as far as the workspace check
    lib = kda.load_library()
    need = kda.kda_gdn_chunk_bwd_workspace_size(1, 128, 2, 128, 128, 0, kda.KDA_BF16)
    assert bwd_gdn(lib, la=P + 2, dla=P + 2, wsb=need - 1) == 3
    assert bwd_gdn(lib, la=P + 4, dla=P + 4, gt=0, wsb=need - 1) == 3
    assert bwd(lib, la=P + 2, dla=P + 2) == 1          # the per-channel entry point needs 16 bytes


def bwd_dec(lib, wr=P, dwr=P, **kw):
    a = dict(q=P, k=P, v=P, la=P, beta=P, h0=None, cu=None, N=0, go=P, ghT=None, dq=P, dk=P, dv=P,
             dla=P, db=P, dh0=P, B=1, T=128, H=2, dk_=128, dv_=128, io=1, gt=1, ws=P, wsb=1 << 40)
    a.update(kw)
    return lib.kda_chunk_bwd_decoupled(a["q"], a["k"], a["v"], a["la"], a["beta"], wr, a["h0"], a["cu"],
                                       a["N"], a["go"], a["ghT"], a["dq"], a["dk"], a["dv"], a["dla"], a["db"],
                                       dwr, a["dh0"], a["B"], a["T"], a["H"], a["dk_"], a["dv_"], a["io"],
                                       a["gt"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(wr=None), 1), (dict(dwr=None), 1), (dict(wr=P + 1), 1), (dict(dwr=P + 2, gt=0), 1),
    (dict(dk_=96), 2), (dict(H=65536, T=1), 2), (dict(la=P + 4), 1), (dict(beta=None), 1), (dict(db=None), 1),
    (dict(ws=None), 3), (dict(wsb=0), 3),
])
def test_decoupled_bwd_rejects(kda, kw, code):
    lib = kda.load_library()
    assert bwd_dec(lib, **kw) == code


def test_decoupled_bwd_empty_without_state_is_noop(kda):
    lib = kda.load_library()
    assert bwd_dec(lib, T=0, q=None, k=None, v=None, la=None, beta=None, wr=None, dwr=None, go=None, dq=None,
                   dk=None, dv=None, dla=None, db=None, dh0=None) == 0


def bwd_pro(lib, lo=-20.0, **kw):
    a = dict(q=P, k=P, v=P, la=P, beta=P, h0=None, cu=None, N=0, go=P, ghT=None, dq=P, dk=P, dv=P,
             dla=P, db=P, dh0=P, B=1, T=128, H=2, dk_=128, dv_=128, io=1, gt=1, ws=P, wsb=1 << 40)
    a.update(kw)
    return lib.kda_chunk_bwd_prologue(a["q"], a["k"], a["v"], a["la"], a["beta"], lo, a["h0"], a["cu"], a["N"],
                                      a["go"], a["ghT"], a["dq"], a["dk"], a["dv"], a["dla"], a["db"], a["dh0"],
                                      a["B"], a["T"], a["H"], a["dk_"], a["dv_"], a["io"], a["gt"], a["ws"],
                                      a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(lo=float("nan")), 1), (dict(lo=float("-inf")), 1), (dict(lo=0.5), 1),
    (dict(dk_=96), 2), (dict(H=65536, T=1), 2), (dict(q=None), 1), (dict(la=P + 4), 1), (dict(dla=P + 8), 1),
    (dict(beta=P + 1), 1), (dict(cu=P, N=2, B=2), 1), (dict(ws=None), 3),
])
def test_prologue_bwd_rejects(kda, kw, code):
    lib = kda.load_library()
    assert bwd_pro(lib, **kw) == code


def test_prologue_bwd_workspace_size(kda):
    # the backward's workspace plus six fp32 [rows, d_k] and four fp32 [rows] buffers
    rows = 1000 * 2
    base = kda.kda_chunk_bwd_workspace_size(1, 1000, 2, 128, 64, 0, kda.KDA_BF16)
    w = kda.kda_chunk_bwd_prologue_workspace_size(1, 1000, 2, 128, 64, 0, kda.KDA_BF16)
    assert base + 6 * rows * 128 * 4 + 4 * rows * 4 <= w <= base + 6 * rows * 128 * 4 + 4 * rows * 4 + 2560
    assert kda.kda_chunk_bwd_prologue_workspace_size(1, 100, 2, 96, 128, 0, kda.KDA_BF16) == 0
    need = kda.kda_chunk_bwd_prologue_workspace_size(1, 128, 2, 128, 128, 0, kda.KDA_BF16)
    assert bwd_pro(kda.load_library(), wsb=need - 1) == 3


@pytest.mark.parametrize("lang,std", [("c", "-std=c99"), ("c++", "-std=c++17")])
def test_header_is_plain_c(tmp_path, lang, std):
    """include/kda.h compiles as C99 and as C++ with warnings on: callers need
    no torch, HIP or C++ types to use the ABI."""
    import shutil
    import subprocess
    cc = shutil.which("gcc" if lang == "c" else "g++")
    if cc is None:
        pytest.skip("no host compiler")
    src = tmp_path / "use.c"
    src.write_text('#include "kda.h"\nint main(void) { return (int)kda_abi_version(); }\n')
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([cc, std, "-Wall", "-Wextra", "-Werror", "-fsyntax-only", "-I", os.path.join(root, "include"),
                        "-x", lang, str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
