"""GPU parity of kda_chunk_bwd (through the C ABI) against the fp64 oracle's
backward (oracle.bwd) on the same seeded inputs and upstream gradients.

Tolerance, derived from the arithmetic: the backward computes every product
and accumulation in fp32, and rounds each output once to its dtype.  A bf16
output is then off by at most 2^-9 of its own size plus the fp32 error, so bf16
outputs must meet max|d| <= 2^-8 max|ref| and ||d||_F <= 2^-8 ||ref||_F (twice
the rounding bound); fp32 outputs (everything with fp32 I/O, and grad_h0 always)
must meet 1e-4 relative in both norms, the forward's fp32 bound.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from kda_testutil import errors, f64, to_oracle

from gated_delta_rule_chunkwise_amd import inputs as I

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF16_REL = 2.0 ** -8
F32_REL = 1e-4
NAMES = ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dh0")


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_chunkwise_amd as kda
    kda.load_library()
    return kda


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_bwd(kda, d, go, ghT, with_h0=True, want_dh0=True):
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    cu = g["cu_seqlens"] if len(d["lengths"]) > 1 else None
    out = kda.kda_chunk_bwd(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], go.to(DEV),
                            h0=g["h0"] if with_h0 else None,
                            grad_hT=None if ghT is None else ghT.to(DEV), cu_seqlens=cu,
                            want_grad_h0=want_dh0)
    torch.cuda.synchronize()
    return [None if x is None else x.cpu() for x in out]


def oracle_bwd(d, go, ghT, seqs=None, heads=None, with_h0=True):
    ref = to_oracle(d, seqs, heads)
    hs = slice(None) if heads is None else list(heads)
    sq = list(range(len(d["lengths"]))) if seqs is None else list(seqs)
    rows = torch.from_numpy(ref["rows"])
    dO = f64(go[rows][:, hs])
    dhT = None if ghT is None else f64(ghT[sq][:, hs])
    res = oracle.bwd(ref["q"], ref["k"], ref["v"], ref["log_alpha"], ref["beta"], dO,
                     h0=ref["h0"] if with_h0 else None, d_hT=dhT, cu_seqlens=ref["cu_seqlens"])
    return res, rows, hs, sq


def check(kda, d, io, go, ghT, seqs=None, heads=None, with_h0=True, what=""):
    out = run_bwd(kda, d, go, ghT, with_h0=with_h0)
    ref, rows, hs, sq = oracle_bwd(d, go, ghT, seqs, heads, with_h0)
    errs = {}
    for name, g, r in zip(NAMES, out, ref):
        g = g[sq][:, hs] if name == "dh0" else g[rows][:, hs]
        e = errors(g, r)
        tol = F32_REL if (io == "f32" or name == "dh0") else BF16_REL
        assert e["rel_max"] <= tol and e["rel_fro"] <= tol, "%s %s: %s (tol %g)" % (what, name, e, tol)
        errs[name] = "%.1e/%.1e" % (e["rel_max"], e["rel_fro"])
    log(what, errs)
    return out


def test_bwd_c0_shape_fp32(kda):
    d = I.make_chunk_inputs(I.C0, h0=True)
    go, ghT = I.make_upstream_grads(d, 3000)
    check(kda, d, "f32", go, ghT, what="c0")


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_bwd_ragged_varlen_dims(kda, io, dk, dv):
    """Lengths span partial, exact and multi-chunk sequences and an empty one."""
    cfg = I.ChunkConfig("ragged", io, io, H=3, dk=dk, dv=dv, h0=True, seed=3100 + dk + dv)
    d = I.make_chunk_inputs(cfg, lengths=[1, 63, 64, 65, 200, 0, 130])
    go, ghT = I.make_upstream_grads(d, 3101)
    check(kda, d, io, go, ghT, what="ragged %s %dx%d" % (io, dk, dv))


def test_bwd_bf16_io_fp32_gates(kda):
    cfg = I.ChunkConfig("mixed", "bf16", "f32", H=2, dk=128, dv=128, h0=True, seed=3200)
    d = I.make_chunk_inputs(cfg, lengths=[300, 77])
    go, ghT = I.make_upstream_grads(d, 3201)
    check(kda, d, "bf16", go, ghT, what="bf16 io, f32 gates")


def test_bwd_c1_shape_bf16(kda):
    d = I.make_chunk_inputs(I.C1)
    go, ghT = I.make_upstream_grads(d, 3300)
    check(kda, d, "bf16", go, ghT, what="c1")


def test_bwd_c3_full(kda):
    """Full long-context shape (T = 65,536, H = 32) in the launch the benchmark
    times; every gradient of every head against the oracle's backward."""
    d = I.make_chunk_inputs(I.C3)
    go, ghT = I.make_upstream_grads(d, 3400, with_state=False)
    check(kda, d, "bf16", go, None, what="c3 all heads")


def test_bwd_max_heads(kda):
    """H = 65,535, the largest head count the backward accepts (heads are a grid
    dimension): workspace offsets past 2^32 bytes, a full chunk plus a one-token
    tail, h0 and grad_hT given."""
    cfg = I.ChunkConfig("maxh", "bf16", "bf16", H=65535, dk=64, dv=64, h0=True, seed=3460)
    d = I.make_chunk_inputs(cfg, lengths=[65])
    go, ghT = I.make_upstream_grads(d, 3461)
    heads = [0, 1, 32767, 65534]
    check(kda, d, "bf16", go, ghT, heads=heads, what="H=65535 heads %s" % heads)


def test_bwd_c2_varlen_full(kda):
    """Full-size packed batch (32 sequences of 512-8192 tokens, h0 != 0, with
    grad_hT) in one call; every sequence and head against the oracle."""
    d = I.make_chunk_inputs(I.C2)
    go, ghT = I.make_upstream_grads(d, 3450)
    check(kda, d, "bf16", go, ghT, what="c2 all sequences")


def test_bwd_without_state_inputs(kda):
    """h0 = NULL, grad_hT = NULL; grad_h0 not requested, then requested."""
    cfg = I.ChunkConfig("nostate", "bf16", "bf16", H=2, dk=128, dv=64, h0=False, seed=3500)
    d = I.make_chunk_inputs(cfg, lengths=[150, 40])
    go, _ = I.make_upstream_grads(d, 3501, with_state=False)
    out = run_bwd(kda, d, go, None, with_h0=False, want_dh0=False)
    assert out[5] is None
    check(kda, d, "bf16", go, None, with_h0=False, what="no h0, no grad_hT")


@pytest.mark.parametrize("lengths", [[1], [1, 2, 3, 1, 64, 65, 1], [127, 0, 0, 129]])
def test_bwd_tiny_and_empty_sequences(kda, lengths):
    """Single tokens, runs of one-token sequences, and empty sequences between
    others (grad_h0 of an empty sequence is grad_hT)."""
    cfg = I.ChunkConfig("tiny", "bf16", "bf16", H=2, dk=64, dv=128, h0=True, seed=3900 + len(lengths))
    d = I.make_chunk_inputs(cfg, lengths=lengths)
    go, ghT = I.make_upstream_grads(d, 3901)
    check(kda, d, "bf16", go, ghT, what="lengths %s" % lengths)


def test_bwd_empty_batch_passes_state_gradient(kda):
    """T = 0: only grad_h0 = grad_hT is written."""
    dev = DEV
    H, dk, dv = 2, 64, 64
    z = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device=dev)
    ghT = torch.randn((1, H, dk, dv), generator=torch.Generator().manual_seed(3950)).to(dev)
    out = kda.kda_chunk_bwd(z(1, 0, H, dk), z(1, 0, H, dk), z(1, 0, H, dv), z(1, 0, H, dk), z(1, 0, H),
                            z(1, 0, H, dv), grad_hT=ghT)
    torch.cuda.synchronize()
    assert torch.equal(out[5], ghT)


def test_bwd_bitwise_determinism(kda):
    cfg = I.ChunkConfig("det", "bf16", "bf16", H=4, dk=128, dv=128, h0=True, seed=3600)
    d = I.make_chunk_inputs(cfg, lengths=[500, 129])
    go, ghT = I.make_upstream_grads(d, 3601)
    a = run_bwd(kda, d, go, ghT)
    b = run_bwd(kda, d, go, ghT)
    for name, x, y in zip(NAMES, a, b):
        assert torch.equal(x, y), name


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("case", ["one channel -3", "one channel -30", "all channels -30", "single tokens -30"])
def test_bwd_strong_decay_chunks(kda, case, io):
    """Chunks whose decay leaves the fp32 range of the anchored factors (a key
    channel decaying by more than about e^-159 within 64 tokens) run exact:
    pairwise decay factors e^{G_r - G_i} <= 1 and state-side operands without
    anchor.  Every gradient still matches the oracle, for log alpha down to
    -30 per token: on one channel over a whole chunk (-3: e^-192 in total;
    -30: e^-1920), on every channel of a head over a chunk, and at single
    tokens on every channel and head."""
    cfg = I.ChunkConfig("strong-bwd", io, io, H=2, dk=64, dv=64, h0=True, seed=3700)
    d = I.make_chunk_inputs(cfg, lengths=[192, 100])
    la = d["log_alpha"].clone()
    if case == "one channel -3":
        la[64:128, 0, 0] = -3.0
    elif case == "one channel -30":
        la[64:128, 0, 0] = -30.0
    elif case == "all channels -30":
        la[64:128, 1, :] = -30.0
    else:
        la[[5, 70, 200, 250]] = -30.0
    d["log_alpha"] = la.to(d["log_alpha"].dtype)
    go, ghT = I.make_upstream_grads(d, 3701)
    out = run_bwd(kda, d, go, ghT)
    for name, g in zip(NAMES, out):
        assert torch.isfinite(g.float()).all(), name
    check(kda, d, io, go, ghT, what="strong decay (%s) %s" % (case, io))


def test_bwd_strong_decay_d128_varlen(kda):
    """The same at d_k = d_v = 128 in a ragged packed batch: log alpha = -30 on
    a quarter of the key channels over a whole chunk of one sequence, and -5 on
    one channel over most of another."""
    cfg = I.ChunkConfig("strong-bwd-128", "bf16", "bf16", H=2, dk=128, dv=128, h0=True, seed=3710)
    d = I.make_chunk_inputs(cfg, lengths=[130, 64, 1, 260])
    la = d["log_alpha"].clone()
    la[0:64, 1, 0:32] = -30.0
    la[200:380, 0, 77] = -5.0
    d["log_alpha"] = la
    go, ghT = I.make_upstream_grads(d, 3711)
    check(kda, d, "bf16", go, ghT, what="strong decay d128 varlen")


def test_bwd_matches_forward_directional_derivative(kda):
    """Cross-check of the two GPU paths: for a random direction x' of all
    inputs, <grad, x'> from kda_chunk_bwd equals the central difference of
    <grad_o, o> + <grad_hT, h_T> computed with kda_chunk_fwd (fp32 I/O)."""
    cfg = I.ChunkConfig("dir", "f32", "f32", H=2, dk=64, dv=64, h0=True, seed=3800)
    d = I.make_chunk_inputs(cfg, lengths=[130, 70])
    go, ghT = I.make_upstream_grads(d, 3801)
    grads = run_bwd(kda, d, go, ghT)
    gen = torch.Generator().manual_seed(3802)
    keys = ("q", "k", "v", "log_alpha", "beta", "h0")
    dirs = {k: torch.randn(d[k].shape, generator=gen, dtype=torch.float64) for k in keys}
    dirs["log_alpha"] *= 0.1
    cu = d["cu_seqlens"].to(DEV)

    def loss(eps):
        x = {k: (d[k].double() + eps * dirs[k]).float().to(DEV) for k in keys}
        o, hT = kda.kda_chunk_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], h0=x["h0"],
                                  cu_seqlens=cu)
        return float((o.double().cpu() * go.double()).sum() + (hT.double().cpu() * ghT.double()).sum())

    # The forward's own rounding (about 1e-5 relative per output) over ~3e4
    # outputs puts about 2e-3 of noise on each loss; divided by 2 eps = 2e-2 that
    # is about 0.1 on the difference quotient, against |<grad, x'>| ~ 1e2.
    eps = 1e-2
    fd = (loss(eps) - loss(-eps)) / (2 * eps)
    an = sum(float((g.double() * dirs[k]).sum()) for g, k in zip(grads, keys))
    log("directional derivative: fd %.6f analytic %.6f" % (fd, an))
    assert abs(fd - an) <= 1e-2 * max(1.0, abs(an))


# ------------------------------------------------------------------ scalar gates
# kda_gdn_chunk_bwd: Gated DeltaNet (one log decay per token and head) or
# DeltaNet (none), against the oracle's backward with that value on every key
# channel; the scalar gate's gradient is the oracle's channel gradients summed
# (the chain rule, pinned on the CPU by finite differences of a scalar-gate
# recurrence).
def gdn_check(kda, d, g, io, go, ghT, seqs=None, heads=None, what=""):
    dev = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    cu = dev["cu_seqlens"] if len(d["lengths"]) > 1 else None
    out = kda.kda_gdn_chunk_bwd(dev["q"], dev["k"], dev["v"], None if g is None else g.to(DEV), dev["beta"],
                                go.to(DEV), h0=dev["h0"], grad_hT=None if ghT is None else ghT.to(DEV),
                                cu_seqlens=cu)
    torch.cuda.synchronize()
    out = [None if x is None else x.cpu() for x in out]
    assert (out[3] is None) == (g is None)
    T, H, dk = d["q"].shape
    dd = dict(d)
    dd["log_alpha"] = torch.zeros((T, H, dk), dtype=torch.float64) if g is None else \
        g.to(torch.float64)[:, :, None].expand(T, H, dk).contiguous()
    ref, rows, hs, sq = oracle_bwd(dd, go, ghT, seqs, heads)
    ref = list(ref)
    ref[3] = ref[3].sum(-1)
    errs = {}
    for name, x, r in zip(NAMES, out, ref):
        if x is None:
            continue
        x = x[sq][:, hs] if name == "dh0" else x[rows][:, hs]
        e = errors(x, r)
        tol = F32_REL if (io == "f32" or name == "dh0") else BF16_REL
        assert e["rel_max"] <= tol and e["rel_fro"] <= tol, "%s %s: %s (tol %g)" % (what, name, e, tol)
        errs[name] = "%.1e/%.1e" % (e["rel_max"], e["rel_fro"])
    log(what, errs)


@pytest.mark.parametrize("gate", ["scalar", "none"])
@pytest.mark.parametrize("io,dk,dv", [("bf16", 128, 128), ("bf16", 64, 128), ("f32", 128, 64), ("f32", 64, 64)])
def test_gdn_bwd_ragged_varlen(kda, gate, io, dk, dv):
    """Ragged packed sequences with h0 and grad_hT; the scalar gate includes a
    near-reset (log a = -30) and a chunk that decays by e^-128 in total."""
    cfg = I.ChunkConfig("gdn-bwd", io, io, H=3, dk=dk, dv=dv, h0=True, seed=4000 + dk + dv)
    d = I.make_chunk_inputs(cfg, lengths=[300, 64, 130, 1, 200, 0])
    g = None
    if gate == "none":
        # no decay: keep the growing state's outputs, and so the gradients,
        # of order one (they are linear in v and h0)
        d["v"] = (d["v"].float() * 0.35).to(d["v"].dtype)
        d["h0"] = d["h0"] * 0.35
    else:
        g = d["log_alpha"][:, :, 0].float().clone()
        g[10] = -30.0
        g[300:364, 1] = -2.0
        g = g.to(d["log_alpha"].dtype).contiguous()
    go, ghT = I.make_upstream_grads(d, 4001)
    gdn_check(kda, d, g, io, go, ghT, what="gdn bwd %s %s %dx%d" % (gate, io, dk, dv))


def test_gdn_bwd_c3_full(kda):
    """Full long-context size (T = 65,536, H = 32) with one decay per token
    and head; every head against the oracle."""
    d = I.make_chunk_inputs(I.C3)
    g = d["log_alpha"][:, :, 0].contiguous()
    go, _ = I.make_upstream_grads(d, 4100, with_state=False)
    gdn_check(kda, d, g, "bf16", go, None, what="gdn bwd c3 all heads")


# ------------------------------------------------------------------ separate strengths
# kda_chunk_bwd_decoupled: erase strength b and write strength w, against the
# oracle's generalised backward (oracle.gen_bwd).
NAMES_DEC = ("dq", "dk", "dv", "dlog_alpha", "db_erase", "dw_write", "dh0")


def dec_check(kda, d, w, io, go, ghT, seqs=None, heads=None, what=""):
    dev = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    cu = dev["cu_seqlens"] if len(d["lengths"]) > 1 else None
    out = kda.kda_chunk_bwd_decoupled(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], w.to(DEV),
                                      go.to(DEV), h0=dev["h0"], grad_hT=None if ghT is None else ghT.to(DEV),
                                      cu_seqlens=cu)
    torch.cuda.synchronize()
    out = [x.cpu() for x in out]
    ref = to_oracle(d, seqs, heads)
    hs = slice(None) if heads is None else list(heads)
    sq = list(range(len(d["lengths"]))) if seqs is None else list(seqs)
    rows = torch.from_numpy(ref["rows"])
    res = oracle.gen_bwd(ref["q"], ref["k"], ref["v"], ref["log_alpha"], ref["beta"], f64(w[rows][:, hs]),
                         f64(go[rows][:, hs]), h0=ref["h0"], d_hT=None if ghT is None else f64(ghT[sq][:, hs]),
                         cu_seqlens=ref["cu_seqlens"])
    errs = {}
    for name, x, r in zip(NAMES_DEC, out, res):
        x = x[sq][:, hs] if name == "dh0" else x[rows][:, hs]
        e = errors(x, r)
        tol = F32_REL if (io == "f32" or name == "dh0") else BF16_REL
        assert e["rel_max"] <= tol and e["rel_fro"] <= tol, "%s %s: %s (tol %g)" % (what, name, e, tol)
        errs[name] = "%.1e/%.1e" % (e["rel_max"], e["rel_fro"])
    log(what, errs)
    return out


@pytest.mark.parametrize("io,dk,dv", [("bf16", 128, 128), ("bf16", 64, 128), ("f32", 128, 64), ("f32", 64, 64)])
def test_decoupled_bwd_ragged(kda, io, dk, dv):
    cfg = I.ChunkConfig("dec-bwd", io, io, H=3, dk=dk, dv=dv, h0=True, seed=4200 + dk + dv)
    d = I.make_chunk_inputs(cfg, lengths=[300, 64, 1, 0, 130])
    w = I.draw_strength(d["beta"].shape, 4201, d["beta"].dtype)
    go, ghT = I.make_upstream_grads(d, 4202)
    dec_check(kda, d, w, io, go, ghT, what="decoupled bwd %s %dx%d" % (io, dk, dv))


def test_decoupled_bwd_tied_is_kda_bwd(kda):
    """w = b: the same gradients as kda_chunk_bwd, and db + dw = dbeta (each part
    rounded on its own)."""
    cfg = I.ChunkConfig("dec-tied", "f32", "f32", H=2, dk=128, dv=128, h0=True, seed=4300)
    d = I.make_chunk_inputs(cfg, lengths=[200, 77])
    go, ghT = I.make_upstream_grads(d, 4301)
    a = run_bwd(kda, d, go, ghT)
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    b = kda.kda_chunk_bwd_decoupled(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["beta"], go.to(DEV),
                                    h0=g["h0"], grad_hT=ghT.to(DEV), cu_seqlens=g["cu_seqlens"])
    torch.cuda.synchronize()
    b = [x.cpu() for x in b]
    for i, name in ((0, "dq"), (1, "dk"), (2, "dv"), (3, "dlog_alpha")):
        assert torch.equal(a[i], b[i]), name
    assert torch.equal(a[5], b[6]), "dh0"
    e = errors(b[4] + b[5], f64(a[4]))
    assert e["rel_max"] <= 1e-5, e


def test_decoupled_bwd_c1_shape(kda):
    d = I.make_chunk_inputs(I.C1)
    w = I.draw_strength(d["beta"].shape, 4400, d["beta"].dtype)
    go, ghT = I.make_upstream_grads(d, 4401)
    dec_check(kda, d, w, "bf16", go, ghT, what="decoupled bwd c1")


# ------------------------------------------------------------------ input prologue
# kda_chunk_bwd_prologue: gradients with respect to the raw projections,
# against the oracle's backward of the forward on raw inputs (oracle.bwd_prologue).
NAMES_PRO = ("dq_raw", "dk_raw", "dv", "dgate_pre", "dbeta_pre", "dh0")


def pro_bwd_check(kda, d, io, lo, go, ghT, eps_rows=(), heads=None, what=""):
    dev = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    cu = dev["cu_seqlens"] if len(d["lengths"]) > 1 else None
    out = kda.kda_chunk_bwd_prologue(dev["q_raw"], dev["k_raw"], dev["v"], dev["gate_pre"], dev["beta_pre"], lo,
                                     go.to(DEV), h0=dev["h0"], grad_hT=None if ghT is None else ghT.to(DEV),
                                     cu_seqlens=cu)
    torch.cuda.synchronize()
    out = [x.cpu() for x in out]
    plain = dict(q=d["q_raw"], k=d["k_raw"], v=d["v"], log_alpha=d["gate_pre"], beta=d["beta_pre"], h0=d["h0"],
                 lengths=d["lengths"], cu_seqlens=d["cu_seqlens"])
    ref = to_oracle(plain, None, heads)
    hs = slice(None) if heads is None else list(heads)
    rows = torch.from_numpy(ref["rows"])
    res = oracle.bwd_prologue(ref["q"], ref["k"], ref["v"], ref["log_alpha"], ref["beta"], lo,
                              f64(go[rows][:, hs]), h0=ref["h0"],
                              d_hT=None if ghT is None else f64(ghT[:, hs]), cu_seqlens=ref["cu_seqlens"])
    T = rows.numel()
    keep = np.ones(T, bool)
    for t, _ in eps_rows:
        keep[t] = False
    errs = {}
    for name, x, r in zip(NAMES_PRO, out, res):
        x = f64(x[:, hs] if name == "dh0" else x[rows][:, hs])
        tol = F32_REL if (io == "f32" or name == "dh0") else BF16_REL
        if name in ("dq_raw", "dk_raw"):
            # rows in the eps branch are (dq_hat / eps): compare them on their own
            for t, hh in eps_rows:
                e = errors(x[t, hh], r[t, hh])
                assert e["rel_max"] <= tol, "%s %s eps row %d: %s" % (what, name, t, e)
            x, r = x[keep], r[keep]
        elif name != "dh0":
            x, r = x[keep], r[keep]
        e = errors(x, r)
        assert e["rel_max"] <= tol and e["rel_fro"] <= tol, "%s %s: %s (tol %g)" % (what, name, e, tol)
        errs[name] = "%.1e/%.1e" % (e["rel_max"], e["rel_fro"])
    log(what, errs)


@pytest.mark.parametrize("io,dk,dv", [("bf16", 128, 128), ("bf16", 64, 128), ("f32", 128, 64), ("f32", 64, 64)])
def test_prologue_bwd_ragged(kda, io, dk, dv):
    """Ragged packed sequences with h0 and grad_hT, gate pre-activations N(0, 2^2),
    the floor at -20 with gates driven onto it over whole chunks (as the
    forward's prologue tests do: those chunks run exact), a zero query row and
    a zero key row (the eps branch)."""
    cfg = I.ChunkConfig("pro-bwd", io, io, H=3, dk=dk, dv=dv, h0=True, seed=4500 + dk + dv)
    d = I.make_chunk_raw_inputs(cfg, lengths=[300, 64, 130, 1, 200, 0], gate_scale=2.0)
    q, k, a = d["q_raw"].clone(), d["k_raw"].clone(), d["gate_pre"].clone()
    q[5, 0] = 0.0
    k[7, 1] = 0.0
    a[10] = 60.0                  # -softplus(60) = -60, floored to -20 on every channel
    a[70:75] = 40.0
    a[300:364, 1, :3] = 25.0      # sequence 1, head 1: a whole chunk on the floor
    d["q_raw"], d["k_raw"], d["gate_pre"] = q, k, a.to(d["gate_pre"].dtype)
    go, ghT = I.make_upstream_grads(dict(d, q=d["q_raw"]), 4501)
    pro_bwd_check(kda, d, io, -20.0, go, ghT, eps_rows=[(5, 0), (7, 1)],
                  what="prologue bwd %s %dx%d" % (io, dk, dv))


def test_prologue_bwd_c1_shape(kda):
    d = I.make_chunk_raw_inputs(I.C1, gate_scale=2.0)
    go, ghT = I.make_upstream_grads(dict(d, q=d["q_raw"]), 4600)
    pro_bwd_check(kda, d, "bf16", -3.0, go, ghT, what="prologue bwd c1")


def test_decoupled_bwd_c3_full(kda):
    """Full long-context size with a write strength drawn like beta (as the
    benchmark times it); every head against the oracle."""
    d = I.make_chunk_inputs(I.C3)
    w = I.draw_strength(d["beta"].shape, 5200, d["beta"].dtype)
    go, _ = I.make_upstream_grads(d, 3400, with_state=False)
    dec_check(kda, d, w, "bf16", go, None, what="decoupled bwd c3 all heads")


def test_prologue_bwd_c3_full(kda):
    """Full long-context size on raw projections, floor -30 (as the benchmark
    times it); every head against the oracle."""
    d = I.make_chunk_raw_inputs(I.C3, gate="uniform")
    go, _ = I.make_upstream_grads(dict(d, q=d["q_raw"]), 3400, with_state=False)
    pro_bwd_check(kda, d, "bf16", -30.0, go, None, what="prologue bwd c3 all heads")


@pytest.mark.parametrize("gdn", [False, True])
def test_autograd_wrapper_is_the_direct_calls(kda, gdn):
    """chunk_kda / chunk_gated_delta_rule: loss.backward() gives exactly the
    gradients of the direct backward call with grad_o, grad_hT = dL/do, dL/dh_T."""
    cfg = I.ChunkConfig("autograd", "bf16", "f32", H=2, dk=128, dv=64, h0=True, seed=4700)
    d = I.make_chunk_inputs(cfg, lengths=[150, 90])
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    la = g["log_alpha"][:, :, 0].contiguous() if gdn else g["log_alpha"]
    leaves = [x.detach().clone().requires_grad_(True) for x in (g["q"], g["k"], g["v"], la, g["beta"], g["h0"])]
    go, ghT = I.make_upstream_grads(d, 4701)
    go, ghT = go.to(DEV), ghT.to(DEV)
    fn = kda.chunk_gated_delta_rule if gdn else kda.chunk_kda
    o, hT = fn(*leaves, cu_seqlens=g["cu_seqlens"])
    ((o.float() * go.float()).sum() + (hT * ghT).sum()).backward()
    bwd = kda.kda_gdn_chunk_bwd if gdn else kda.kda_chunk_bwd
    ref = bwd(g["q"], g["k"], g["v"], la, g["beta"], go, h0=g["h0"], grad_hT=ghT, cu_seqlens=g["cu_seqlens"])
    torch.cuda.synchronize()
    for leaf, r, name in zip(leaves, ref, NAMES):
        assert leaf.grad is not None and torch.equal(leaf.grad, r), name


def test_bwd_c3_linear_in_upstream_gradients(kda):
    """At the long-context size: every gradient is linear in (grad_o, grad_hT)
    for fixed inputs, and scaling by 2 is exact, so doubling both doubles every
    output bitwise."""
    d = I.make_chunk_inputs(I.C3)
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    go, _ = I.make_upstream_grads(d, 3400, with_state=False)
    go = go.to(DEV)
    ghT = 0.1 * torch.randn((1, 32, 128, 128), generator=torch.Generator().manual_seed(5000)).to(DEV)
    a = kda.kda_chunk_bwd(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], go, grad_hT=ghT)
    b = kda.kda_chunk_bwd(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], 2 * go, grad_hT=2 * ghT)
    torch.cuda.synchronize()
    for name, x, y in zip(NAMES, a, b):
        assert torch.equal(y, 2 * x), name


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_bwd_near_range_limit(kda, io):
    """A chunk in which key channel 0 decays by e^-150 in total (log_alpha =
    -150/64 per token), just inside the fp32 range of the anchored factors
    (about e^-160): the gradients still meet the tolerance there, and the other
    chunks and heads are unaffected."""
    cfg = I.ChunkConfig("near-limit", io, io, H=2, dk=64, dv=64, h0=True, seed=5100)
    d = I.make_chunk_inputs(cfg, lengths=[192, 100])
    la = d["log_alpha"].clone()
    la[64:128, 0, 0] = -150.0 / 64
    d["log_alpha"] = la.to(d["log_alpha"].dtype)
    go, ghT = I.make_upstream_grads(d, 5101)
    out = run_bwd(kda, d, go, ghT)
    for g in out:
        assert torch.isfinite(g.float()).all()
    check(kda, d, io, go, ghT, what="near range limit %s" % io)
