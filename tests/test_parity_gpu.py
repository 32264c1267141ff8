"""GPU parity: libkda (through the C ABI) against the fp64 oracle on the same
seeded inputs.  Tolerances: bf16 I/O max-abs 5e-3 and relative Frobenius 1e-2;
fp32 I/O 1e-4 relative; on o and on the final state."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from kda_testutil import assert_close, bf16_rounding_stats, errors, f64, to_oracle

from gated_delta_rule_chunkwise_amd import inputs as I

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


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


def run_gpu(kda, d, with_h0=True, packed=False):
    dev = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    cu = dev["cu_seqlens"] if len(d["lengths"]) > 1 or packed else None
    o, hT = kda.kda_chunk_fwd(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"],
                              h0=dev["h0"] if with_h0 else None, cu_seqlens=cu)
    torch.cuda.synchronize()
    return o.cpu(), hT.cpu()


def check_against_oracle(kda, d, io, seqs=None, heads=None, what=""):
    o, hT = run_gpu(kda, d)
    ref = to_oracle(d, seqs, heads)
    ro, rh = oracle.fwd(ref["q"], ref["k"], ref["v"], ref["log_alpha"], ref["beta"], h0=ref["h0"],
                        cu_seqlens=ref["cu_seqlens"])
    hs = slice(None) if heads is None else list(heads)
    rows = torch.from_numpy(ref["rows"])
    go = o.reshape(-1, *o.shape[-2:])[rows][:, hs]
    sq = list(range(len(d["lengths"]))) if seqs is None else list(seqs)
    gh = hT[sq][:, hs]
    eo = assert_close(go, ro, io, what + " o")
    eh = assert_close(gh, rh, io, what + " h_T")
    if io == "bf16":
        log(what, "o", eo, "h_T", eh, "o against the oracle rounded to bf16:", bf16_rounding_stats(go, ro))
    else:
        log(what, "o", eo, "h_T", eh)
    return eo, eh


# ------------------------------------------------------------------ the workloads
def test_c0_fp32_full(kda):
    d = I.make_chunk_inputs(I.C0)
    check_against_oracle(kda, d, "f32", what="c0")


def test_c1_bf16_full(kda):
    d = I.make_chunk_inputs(I.C1)
    check_against_oracle(kda, d, "bf16", what="c1")


def test_c2_varlen_full(kda):
    """Full-size varlen batch (32 sequences of 512-8192 tokens, h0 != 0) in the
    launch the benchmark times; the oracle checks every sequence and head."""
    d = I.make_chunk_inputs(I.C2)
    check_against_oracle(kda, d, "bf16", what="c2 all %d sequences" % len(d["lengths"]))


@pytest.mark.parametrize("bv", [16, 32])
def test_block_width_variants(kda, bv):
    """Both value-column block widths of the paths that have two (fp32 I/O, and
    bf16 at d_k = 64): a workgroup takes 32 value columns once the chains times
    d_v / 32 reach 512, else 16, so the head count picks the width."""
    for io, dk, dv, lens, seed in (("f32", 64, 128, [300, 17], 20), ("bf16", 64, 128, [5, 700, 64, 129], 19),
                                   ("f32", 128, 128, [130, 3], 21)):
        H = 128 // len(lens) if bv == 32 else 2
        assert (len(lens) * H * (dv // 32) >= 512) == (bv == 32)
        cfg = I.ChunkConfig("bv", io, io, H=H, dk=dk, dv=dv, h0=True, seed=seed)
        d = I.make_chunk_inputs(cfg, lengths=lens)
        check_against_oracle(kda, d, io, what="%s d_k=%d BV=%d" % (io, dk, bv))


def test_c3_long_full(kda):
    """Full-size T = 65536 prefill; the oracle checks all 32 heads end to end."""
    d = I.make_chunk_inputs(I.C3)
    check_against_oracle(kda, d, "bf16", what="c3 all heads")


def test_c3_constant_decay_full(kda):
    """Long-memory variant at full size (T = 65536, H = 32): one decay per
    (head, channel), drawn in [0.5, 0.9999] and held over time; all heads."""
    d = I.make_chunk_inputs(I.C3, gate="uniform_const")
    check_against_oracle(kda, d, "bf16", what="c3 uniform_const all heads")


def test_c3_strong_decay_full(kda):
    """The strong-decay case the benchmark times, at full size: the long-context
    workload with key channel 0 of every head at log alpha = -3 on every token
    (192 nats per chunk on that channel, which leaves the Gram products and has
    its pairs summed exactly); the oracle checks all 32 heads."""
    d = I.make_chunk_inputs(I.C3)
    la = d["log_alpha"].clone()
    la[:, :, 0] = -3.0
    d["log_alpha"] = la
    check_against_oracle(kda, d, "bf16", what="c3 strong decay all heads")


def test_max_heads(kda):
    """H = 65,535, the largest head count the backward's grid admits: record
    and state offsets past 2^32 bytes, a full chunk plus a one-token tail."""
    cfg = I.ChunkConfig("maxh", "bf16", "bf16", H=65535, dk=64, dv=64, h0=True, seed=61)
    d = I.make_chunk_inputs(cfg, lengths=[65])
    heads = [0, 1, 32767, 65534]
    check_against_oracle(kda, d, "bf16", heads=heads, what="H=65535 heads %s" % heads)


def test_segments_of_one_chunk(kda):
    """A long single sequence with 1,024 < H <= 2,048 runs in segments of one
    chunk each (the record budget is 2,048 chunk-heads): three segments, the
    last one ragged, with the state carried across both boundaries."""
    cfg = I.ChunkConfig("seg1", "bf16", "bf16", H=1500, dk=128, dv=128, h0=True, seed=62)
    d = I.make_chunk_inputs(cfg, lengths=[130])
    heads = [0, 749, 1499]
    check_against_oracle(kda, d, "bf16", heads=heads, what="H=1500 one-chunk segments heads %s" % heads)


def test_long_sequence_past_2_32_elements(kda):
    """One sequence of 1,050,000 tokens at H = 32, d = 128: q, k, v, log alpha
    and o each hold 4.3e9 elements, past 2^32, so every token offset needs 64
    bits.  It runs as 257 segments and ends in a 16-token chunk.  Inputs are
    drawn on the device; the oracle checks two whole heads."""
    T, heads = 1_050_000, [0, 31]
    cfg = I.ChunkConfig("long", "bf16", "bf16", H=32, dk=128, dv=128, h0=True, seed=63)
    d = I.make_chunk_inputs(cfg, device=DEV, lengths=[T])
    assert d["q"].numel() > 2 ** 32
    o, hT = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], h0=d["h0"])
    torch.cuda.synchronize()
    go, gh = o[:, heads].cpu(), hT[:, heads].cpu()
    sub = {key: d[key][:, heads].cpu() for key in ("q", "k", "v", "log_alpha", "beta", "h0")}
    sub["lengths"] = d["lengths"]
    del d, o, hT
    torch.cuda.empty_cache()
    ref = to_oracle(sub)
    ro, rh = oracle.fwd(ref["q"], ref["k"], ref["v"], ref["log_alpha"], ref["beta"], h0=ref["h0"],
                        cu_seqlens=ref["cu_seqlens"])
    eo = assert_close(go, ro, "bf16", "T=1,050,000 o")
    eh = assert_close(gh, rh, "bf16", "T=1,050,000 h_T")
    log("T=1,050,000 heads %s" % heads, "o", eo, "h_T", eh)


# ------------------------------------------------------------------ shapes / edge cases
@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_ragged_varlen_dims(kda, dk, dv, io):
    cfg = I.ChunkConfig("edge", io, io, H=3, dk=dk, dv=dv, h0=True, seed=11)
    lens = [1, 63, 64, 65, 0, 130, 200, 7]
    d = I.make_chunk_inputs(cfg, lengths=lens)
    check_against_oracle(kda, d, io, what="ragged dk=%d dv=%d %s" % (dk, dv, io))


def test_bf16_io_fp32_gates(kda):
    cfg = I.ChunkConfig("mixed", "bf16", "f32", H=4, dk=128, dv=128, T=333, seed=12, h0=True)
    d = I.make_chunk_inputs(cfg)
    check_against_oracle(kda, d, "bf16", what="bf16 io f32 gates")


def test_strong_decay_takes_exact_path(kda):
    """Gates so strong that a chunk's total decay exceeds the matrix-core range
    (near-resets): those chunks run token by token; results still match."""
    cfg = I.ChunkConfig("strong", "f32", "f32", H=2, dk=64, dv=64, T=300, seed=13, h0=True)
    d = I.make_chunk_inputs(cfg)
    la = d["log_alpha"].clone()
    la[10] = -30.0
    la[70:75] = -28.0
    la[200:264, 0, :5] = -3.0
    d["log_alpha"] = la
    check_against_oracle(kda, d, "f32", what="strong decay")


@pytest.mark.parametrize("gate_io", ["bf16", "f32"])
def test_strong_decay_bf16_two_pass(kda, gate_io):
    """bf16 I/O (prep + state kernels) with chunks whose decay exceeds the
    matrix-core range mixed with ordinary ones, across packed sequences: the
    flagged chunks run token by token in the state kernel."""
    cfg = I.ChunkConfig("strong16", "bf16", gate_io, H=3, dk=128, dv=128, h0=True, seed=18)
    lens = [300, 64, 130, 1, 200]
    d = I.make_chunk_inputs(cfg, lengths=lens)
    la = d["log_alpha"].clone()
    la[10] = -30.0                 # a reset inside the first chunk of sequence 0
    la[70:75] = -28.0              # second chunk of sequence 0
    la[300:364, 1, :3] = -2.0      # the whole of sequence 1 for head 1 (sum -128 on 3 channels)
    la[400:430, :, 7] = -4.0       # partial chunk of sequence 2
    d["log_alpha"] = la.to(d["log_alpha"].dtype)
    check_against_oracle(kda, d, "bf16", what="strong decay bf16 gates=%s" % gate_io)


@pytest.mark.parametrize("gate_io", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128)])
def test_strong_decay_two_kernel_single_sequence(kda, gate_io, dk, dv):
    """One sequence (no cu_seqlens: the prep + state kernels at any d_k) whose
    chunks mix ordinary decay with channels beyond the matrix-core range: a reset
    of every channel (more than 16 such channels, staged from the inputs), a few
    channels over a whole chunk (staged from registers) and one channel inside the
    partial last chunk."""
    cfg = I.ChunkConfig("strong2k", "bf16", gate_io, H=3, dk=dk, dv=dv, T=300, h0=True, seed=19)
    d = I.make_chunk_inputs(cfg)
    la = d["log_alpha"].clone()
    la[10] = -30.0                 # every channel of every head: a reset in chunk 0
    la[70:75] = -28.0              # chunk 1
    la[130:194, 1, :3] = -2.0      # chunk 2 of head 1, three channels (sum -128)
    la[200:230, :, 7] = -4.0       # chunk 3, one channel
    la[260:290, 2, 9] = -4.0       # the partial chunk 4 of head 2
    d["log_alpha"] = la.to(d["log_alpha"].dtype)
    check_against_oracle(kda, d, "bf16", what="strong decay, one sequence, d=%d/%d gates=%s" % (dk, dv, gate_io))


def test_strong_decay_prologue_single_sequence(kda):
    """The same on raw projections at d_k = 64 (prep + state kernels with the
    input prologue): gate pre-activations whose floored log decay leaves some
    channels beyond the matrix-core range."""
    cfg = I.ChunkConfig("strongpro", "bf16", "bf16", H=2, dk=64, dv=64, T=200, h0=True, seed=21)
    d = I.make_chunk_raw_inputs(cfg)
    ga = d["gate_pre"].clone()
    ga[64:128, :, :4] = -40.0      # -softplus(-40) ~ 0: no decay ...
    ga[64:128, 1, 5] = 6.0         # ... and one channel at log alpha ~ -6 per token
    ga[150:180, 0, 2] = 8.0
    d["gate_pre"] = ga.to(d["gate_pre"].dtype)
    check_prologue_against_oracle(kda, d, "bf16", -20.0, what="strong decay prologue d=64")


def test_beta_negative_eigenvalue_range(kda):
    cfg = I.ChunkConfig("beta2", "f32", "f32", H=2, dk=128, dv=128, T=257, seed=14)
    d = I.make_chunk_inputs(cfg)
    d["beta"] = (d["beta"] * 1.9).contiguous()
    check_against_oracle(kda, d, "f32", what="beta in (0,1.9)")


def test_zero_decay_and_tiny_sequences(kda):
    cfg = I.ChunkConfig("nodecay", "bf16", "bf16", H=2, dk=128, dv=128, h0=True, seed=15)
    d = I.make_chunk_inputs(cfg, lengths=[1, 2, 3, 64])
    d["log_alpha"] = torch.zeros_like(d["log_alpha"])
    check_against_oracle(kda, d, "bf16", what="alpha=1")


# ------------------------------------------------------------------ invariants on the GPU
def test_split_chaining_and_alias(kda):
    cfg = I.ChunkConfig("chain", "f32", "f32", H=2, dk=128, dv=128, T=500, seed=16, h0=True)
    d = I.make_chunk_inputs(cfg)
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    o, hT = kda.kda_chunk_fwd(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], h0=g["h0"])
    s = 190
    o1, h1 = kda.kda_chunk_fwd(*(g[x][:s] for x in ("q", "k", "v", "log_alpha", "beta")), h0=g["h0"])
    # h_T aliasing h0: the second half writes its final state over its own h0.
    h1c = h1.clone()
    o2, h2 = kda.kda_chunk_fwd(*(g[x][s:].contiguous() for x in ("q", "k", "v", "log_alpha", "beta")),
                               h0=h1c, h_T=h1c)
    torch.cuda.synchronize()
    assert_close(torch.cat([o1, o2]), o, "f32", "split o")
    assert_close(h1c, hT, "f32", "split h_T")


def test_bitwise_determinism(kda):
    d = I.make_chunk_inputs(I.C1, lengths=[1000])
    a = run_gpu(kda, d)
    b = run_gpu(kda, d)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_varlen_equals_separate_calls(kda):
    cfg = I.ChunkConfig("sep", "bf16", "bf16", H=2, dk=128, dv=128, h0=True, seed=17)
    lens = [100, 64, 1, 250]
    d = I.make_chunk_inputs(cfg, lengths=lens)
    o, hT = run_gpu(kda, d)
    cu = np.concatenate([[0], np.cumsum(lens)])
    for n in range(len(lens)):
        sub = dict(d)
        for x in ("q", "k", "v", "log_alpha", "beta"):
            sub[x] = d[x][cu[n]:cu[n + 1]].contiguous()
        sub["h0"] = d["h0"][n:n + 1].contiguous()
        sub["lengths"] = [lens[n]]
        sub["cu_seqlens"] = torch.tensor([0, lens[n]], dtype=d["cu_seqlens"].dtype)
        on, hn = run_gpu(kda, sub, packed=True)
        assert torch.equal(on.reshape(-1, *on.shape[-2:]), o.reshape(-1, *o.shape[-2:])[cu[n]:cu[n + 1]])
        assert torch.equal(hn[0], hT[n])


# ------------------------------------------------------------------ decode
def _decode_block_as_fwd(x):
    """A block of decode-step inputs [steps, B, H, d] as one packed prefill of B
    sequences of `steps` tokens each ([B*steps, H, d], cu_seqlens): T decode
    steps from a state equal a T-token forward from it (the oracle's pinned
    decode-equals-forward invariant), so the oracle walks each (sequence, head)
    chain through the whole block in one call, carrying its fp64 state."""
    steps, B = x["q"].shape[0], x["q"].shape[1]
    seq = lambda t: np.ascontiguousarray(f64(t).swapaxes(0, 1).reshape((B * steps,) + tuple(t.shape[2:])))
    cu = np.arange(B + 1, dtype=np.int64) * steps
    return {n: seq(x[n]) for n in ("q", "k", "v", "log_alpha", "beta")}, cu


@pytest.mark.timeout(900)
def test_decode_full_size_all_steps(kda):
    """The decode workload at full size: B = 256, H = 32, d = 128, fp32 states
    N(0, 0.1^2), 1000 steps with fresh seeded inputs (drawn on the device, as
    the benchmark does).  Every step's o and the final S against the oracle, in
    blocks of 100 steps with the oracle's fp64 state carried between blocks."""
    cfg = I.C4
    S = I.make_decode_state(cfg, device=DEV)
    Sref = f64(S)
    names = ("q", "k", "v", "log_alpha", "beta")
    block, worst = 100, dict(max_abs=0.0, rel_fro=0.0)
    od = torch.empty((cfg.B, cfg.H, cfg.dv), dtype=torch.bfloat16, device=DEV)
    for s0 in range(0, cfg.steps, block):
        n = min(block, cfg.steps - s0)
        x = I.make_decode_step_inputs(cfg, s0, device=DEV, steps=n)
        outs = torch.empty((n, cfg.B, cfg.H, cfg.dv), dtype=torch.bfloat16, device=DEV)
        for s in range(n):
            kda.kda_decode_step(*(x[nm][s] for nm in names), S, o=od)
            outs[s].copy_(od)
        torch.cuda.synchronize()
        go = outs.cpu()
        xin, cu = _decode_block_as_fwd({nm: x[nm].cpu() for nm in names})
        del x, outs
        ro, Sref = oracle.fwd(xin["q"], xin["k"], xin["v"], xin["log_alpha"], xin["beta"], h0=Sref,
                              cu_seqlens=cu)
        ro = ro.reshape(cfg.B, n, cfg.H, cfg.dv).swapaxes(0, 1)
        for s in range(n):
            e = assert_close(go[s], ro[s], "bf16", "decode step %d o" % (s0 + s))
            worst = {k: max(worst[k], e[k]) for k in worst}
        log("decode steps %d-%d: worst so far %s" % (s0, s0 + n - 1, worst))
    eS = errors(S.cpu(), Sref)
    assert eS["rel_fro"] < 1e-5, eS
    log("decode all %d steps: worst o %s; final S %s" % (cfg.steps, worst, eS))


def test_binding_rejects_bad_buffers(kda):
    """Caller-supplied outputs and workspaces of the wrong shape, dtype or
    device, and mismatched decode inputs, raise before anything is launched."""
    cfg = I.ChunkConfig("rej", "bf16", "bf16", H=2, dk=64, dv=64, T=70, seed=64, h0=True)
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in I.make_chunk_inputs(cfg).items()}
    args = [d[n].unsqueeze(0) for n in ("q", "k", "v", "log_alpha", "beta")]
    good, _ = kda.kda_chunk_fwd(*args)
    bad = [dict(o=torch.empty(1, 70, 2, 32, dtype=torch.bfloat16, device=DEV)),
           dict(o=torch.empty(1, 70, 2, 64, dtype=torch.float32, device=DEV)),
           dict(h_T=torch.empty(1, 2, 64, 64)),
           dict(workspace=torch.empty(1 << 20, dtype=torch.uint8))]
    for kw in bad:
        with pytest.raises((ValueError, TypeError)):
            kda.kda_chunk_fwd(*args, **kw)
    dc = I.DecodeConfig("rej", "bf16", "bf16", B=3, H=2, dk=64, dv=64, steps=1, seed=2401)
    S = I.make_decode_state(dc, device=DEV)
    x = {n: t[0] for n, t in I.make_decode_step_inputs(dc, 0, device=DEV).items()}
    S0 = S.clone()
    with pytest.raises(ValueError):
        kda.kda_decode_step(x["q"], x["k"][:2], x["v"][:2], x["log_alpha"], x["beta"], S)
    with pytest.raises(ValueError):
        kda.kda_decode_step(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], S,
                            o=torch.empty(3, 2, 32, dtype=torch.bfloat16, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(S, S0)
    assert torch.equal(kda.kda_chunk_fwd(*args)[0], good)


def test_decode_past_2_32_state_elements(kda):
    """B = 4,100 sequences x H = 64 heads at d = 128: the fp32 state holds 4.3e9
    elements (17 GB), past 2^32.  Drawn on the device; the oracle checks the
    output and the updated state of the first, a middle and the last
    (sequence, head) pair."""
    cfg = I.DecodeConfig("decode past 2^32", "bf16", "bf16", B=4100, H=64, dk=128, dv=128, steps=1, seed=2400)
    S = I.make_decode_state(cfg, device=DEV)
    assert S.numel() > 2 ** 32
    x = {n: t[0] for n, t in I.make_decode_step_inputs(cfg, 0, device=DEV).items()}
    names = ("q", "k", "v", "log_alpha", "beta")
    bs, hs = [0, 2049, 4099], [0, 31, 63]
    S0 = S[bs, hs].cpu()
    o = kda.kda_decode_step(*(x[n] for n in names), S)
    torch.cuda.synchronize()
    go, gS = o[bs, hs].cpu()[:, None], S[bs, hs].cpu()[:, None]
    # the sampled pairs as a batch of 3 sequences with one head each
    ro, rS = oracle.decode(*(f64(x[n][bs, hs].cpu()[:, None]) for n in names), f64(S0[:, None]))
    eo = assert_close(go, ro, "bf16", "decode past 2^32 o")
    eS = errors(gS, rS)
    assert eS["rel_fro"] < 1e-5, eS
    log("decode past 2^32", "o", eo, "S", eS)


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64)])
def test_decode_dims_fp32(kda, dk, dv):
    cfg = I.DecodeConfig("d", "f32", "f32", B=5, H=3, dk=dk, dv=dv, steps=4, seed=2100)
    S = I.make_decode_state(cfg)
    Sg, Sref = S.to(DEV), f64(S)
    steps = I.make_decode_step_inputs(cfg, 0, steps=4)
    for s in range(4):
        x = {n: t[s] for n, t in steps.items()}
        o = kda.kda_decode_step(*(x[n].to(DEV) for n in ("q", "k", "v", "log_alpha", "beta")), Sg)
        ro, Sref = oracle.decode(*(f64(x[n]) for n in ("q", "k", "v", "log_alpha", "beta")), Sref)
        assert_close(o.cpu(), ro, "f32", "decode o")
    assert_close(Sg.cpu(), Sref, "f32", "decode S")


def test_decode_steps_equal_chunk_fwd(kda):
    """T decode steps from h0 give the chunkwise forward's outputs and state."""
    cfg = I.ChunkConfig("dec-vs-fwd", "f32", "f32", H=2, dk=128, dv=128, B=3, T=70, seed=18, h0=True)
    B, T = 3, 70
    d = I.make_chunk_inputs(cfg)
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    q, k, v, la, be = (g[x].reshape(B, T, *g[x].shape[1:]) for x in ("q", "k", "v", "log_alpha", "beta"))
    o, hT = kda.kda_chunk_fwd(q, k, v, la, be, h0=g["h0"])
    S = g["h0"].clone()
    outs = []
    for t in range(T):
        outs.append(kda.kda_decode_step(q[:, t].contiguous(), k[:, t].contiguous(), v[:, t].contiguous(),
                                        la[:, t].contiguous(), be[:, t].contiguous(), S))
    torch.cuda.synchronize()
    assert_close(torch.stack(outs, 1), o, "f32", "decode vs fwd o")
    assert_close(S, hT, "f32", "decode vs fwd state")


# ------------------------------------------------------------------ input prologue
# kda_chunk_fwd_prologue / kda_decode_step_prologue on raw projections against
# the oracle's prologue (q/|q|, k/|k|, max(-softplus(a), lo), sigmoid(b)) followed
# by the recurrence.
def _raw_as_plain(d):
    return dict(q=d["q_raw"], k=d["k_raw"], v=d["v"], log_alpha=d["gate_pre"], beta=d["beta_pre"],
                h0=d["h0"], lengths=d["lengths"], cu_seqlens=d["cu_seqlens"])


def check_prologue_against_oracle(kda, d, io, lo, seqs=None, heads=None, what=""):
    dev = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    cu = dev["cu_seqlens"] if len(d["lengths"]) > 1 else None
    o, hT = kda.kda_chunk_fwd_prologue(dev["q_raw"], dev["k_raw"], dev["v"], dev["gate_pre"],
                                       dev["beta_pre"], lo, h0=dev["h0"], cu_seqlens=cu)
    torch.cuda.synchronize()
    o, hT = o.cpu(), hT.cpu()
    ref = to_oracle(_raw_as_plain(d), seqs, heads)
    ro, rh = oracle.fwd_prologue(ref["q"], ref["k"], ref["v"], ref["log_alpha"], ref["beta"], lo,
                                 h0=ref["h0"], cu_seqlens=ref["cu_seqlens"])
    hs = slice(None) if heads is None else list(heads)
    rows = torch.from_numpy(ref["rows"])
    go = o.reshape(-1, *o.shape[-2:])[rows][:, hs]
    sq = list(range(len(d["lengths"]))) if seqs is None else list(seqs)
    eo = assert_close(go, ro, io, what + " o")
    eh = assert_close(hT[sq][:, hs], rh, io, what + " h_T")
    log(what, "o", eo, "h_T", eh)
    return eo, eh


def test_prologue_c3_full(kda):
    """The benchmarked prologue call: c3's full size (T = 65536, H = 32) on raw
    projections, gate pre-activations spanning decays 0.5-0.9999, floor -30;
    the oracle checks every head end to end."""
    d = I.make_chunk_raw_inputs(I.C3, gate="uniform")
    check_prologue_against_oracle(kda, d, "bf16", -30.0, what="prologue c3 all heads")


@pytest.mark.parametrize("B,H,T", [(4, 32, 1024), (2, 43, 768), (1, 85, 1024), (3, 43, 512), (1, 2, 4096)])
def test_fused_segment_plans(kda, B, H, T):
    """Equal-length batches on raw projections (the fused kernel) across its
    segment plans, h0 given: 128 chains (3 segments), 86 (3), 85 (4), 129 (one
    pass) and 2 chains of 64 chunks (16 segments of 4 chunks).  A segmented
    call runs each chain's first segment exactly from h0 beside the
    transitions of the middle segments, then the rest from the scanned start
    states."""
    cfg = I.ChunkConfig("segplan", "bf16", "bf16", H=H, dk=128, dv=128, h0=True, seed=7100 + B * H)
    d = I.make_chunk_raw_inputs(cfg, lengths=[T] * B)
    lo = -30.0
    as4 = lambda x: x.reshape(B, T, *x.shape[1:]).to(DEV)
    o, hT = kda.kda_chunk_fwd_prologue(as4(d["q_raw"]), as4(d["k_raw"]), as4(d["v"]), as4(d["gate_pre"]),
                                       as4(d["beta_pre"]), lo, h0=d["h0"].to(DEV))
    torch.cuda.synchronize()
    ref = to_oracle(_raw_as_plain(d))
    ro, rh = oracle.fwd_prologue(ref["q"], ref["k"], ref["v"], ref["log_alpha"], ref["beta"], lo,
                                 h0=ref["h0"], cu_seqlens=ref["cu_seqlens"])
    eo = assert_close(o.cpu().reshape(B * T, H, 128), ro, "bf16", "segment plan %dx%dx%d o" % (B, H, T))
    eh = assert_close(hT.cpu(), rh, "bf16", "segment plan %dx%dx%d h_T" % (B, H, T))
    log("segment plan B=%d H=%d T=%d" % (B, H, T), "o", eo, "h_T", eh)


def test_prologue_c1_shape_bf16(kda):
    """c1's shape (bf16, H=16, T=4096, d=128) on raw projections; gate
    pre-activations N(0, 2^2) with floor -3, so about 7% of gates sit on it."""
    d = I.make_chunk_raw_inputs(I.C1, gate_scale=2.0)
    check_prologue_against_oracle(kda, d, "bf16", -3.0, what="prologue c1")


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_prologue_ragged_varlen(kda, dk, dv, io):
    """Ragged packed sequences with h0, zero-norm rows (the eps branch) and gates
    driven to the floor -20 over whole chunks (decay beyond the matrix-core
    range: those chunks run token by token, also under the prologue)."""
    cfg = I.ChunkConfig("pro-ragged", io, io, H=3, dk=dk, dv=dv, h0=True, seed=31)
    lens = [300, 64, 130, 1, 200]
    d = I.make_chunk_raw_inputs(cfg, lengths=lens, gate_scale=2.0)
    q, k, a = d["q_raw"].clone(), d["k_raw"].clone(), d["gate_pre"].clone()
    q[5] = 0.0                    # zero query: no read-out from the state
    k[7, 1] = 0.0                 # zero key: no erase or write for head 1
    a[10] = 60.0                  # -softplus(60) = -60, floored to -20 on every channel
    a[70:75] = 40.0
    a[300:364, 1, :3] = 25.0      # sequence 1, head 1: a whole chunk on the floor
    d["q_raw"], d["k_raw"], d["gate_pre"] = q, k, a.to(d["gate_pre"].dtype)
    check_prologue_against_oracle(kda, d, io, -20.0, what="prologue ragged dk=%d dv=%d %s" % (dk, dv, io))


def test_prologue_decode_c4_shape(kda):
    cfg = I.C4
    S = I.make_decode_state(cfg)
    Sg, Sref = S.to(DEV), f64(S)
    steps = I.make_decode_raw_step_inputs(cfg, 0, steps=2)
    names = ("q_raw", "k_raw", "v", "gate_pre", "beta_pre")
    for s in range(2):
        x = {n: t[s] for n, t in steps.items()}
        o = kda.kda_decode_step_prologue(*(x[n].to(DEV) for n in names[:5]), -6.0, Sg)
        ro, Sref = oracle.decode_prologue(*(f64(x[n]) for n in names), -6.0, Sref)
        torch.cuda.synchronize()
        log("prologue decode step", s, assert_close(o.cpu(), ro, "bf16", "prologue decode o"))
    eS = errors(Sg.cpu(), Sref)
    assert eS["rel_fro"] < 1e-5, eS
    log("prologue decode S", eS)


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_prologue_decode_dims_fp32(kda, dk, dv):
    cfg = I.DecodeConfig("dp", "f32", "f32", B=5, H=3, dk=dk, dv=dv, steps=3, seed=2200)
    S = I.make_decode_state(cfg)
    Sg, Sref = S.to(DEV), f64(S)
    steps = I.make_decode_raw_step_inputs(cfg, 0, steps=3)
    names = ("q_raw", "k_raw", "v", "gate_pre", "beta_pre")
    for s in range(3):
        x = {n: t[s] for n, t in steps.items()}
        if s == 1:
            x["q_raw"] = x["q_raw"].clone()
            x["q_raw"][0, 0] = 0.0
            x["gate_pre"] = x["gate_pre"] * 8.0
        o = kda.kda_decode_step_prologue(*(x[n].to(DEV) for n in names), -2.5, Sg)
        ro, Sref = oracle.decode_prologue(*(f64(x[n]) for n in names), -2.5, Sref)
        assert_close(o.cpu(), ro, "f32", "prologue decode o")
    assert_close(Sg.cpu(), Sref, "f32", "prologue decode S")


# ------------------------------------------------------------------ scalar gates
# kda_gdn_chunk_fwd / kda_gdn_decode_step: one log decay per (token, head)
# (Gated DeltaNet) or none (DeltaNet), against the oracle with that value on
# every key channel (the oracle's channel-constant case is pinned to a scalar
# Gated DeltaNet recurrence).
def _gdn_check(kda, d, g, io, what, seqs=None, heads=None):
    dev = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    cu = dev["cu_seqlens"] if len(d["lengths"]) > 1 else None
    o, hT = kda.kda_gdn_chunk_fwd(dev["q"], dev["k"], dev["v"], None if g is None else g.to(DEV), dev["beta"],
                                  h0=dev["h0"], cu_seqlens=cu)
    torch.cuda.synchronize()
    o, hT = o.cpu(), hT.cpu()
    T, H, dk = d["q"].shape
    la_full = torch.zeros((T, H, dk), dtype=torch.float64) if g is None else \
        g.to(torch.float64)[:, :, None].expand(T, H, dk).contiguous()
    dd = dict(d)
    dd["log_alpha"] = la_full
    ref = to_oracle(dd, seqs, heads)
    ro, rh = oracle.fwd(ref["q"], ref["k"], ref["v"], ref["log_alpha"], ref["beta"], h0=ref["h0"],
                        cu_seqlens=ref["cu_seqlens"])
    hs = slice(None) if heads is None else list(heads)
    rows = torch.from_numpy(ref["rows"])
    go = o.reshape(-1, *o.shape[-2:])[rows][:, hs]
    sq = list(range(len(d["lengths"]))) if seqs is None else list(seqs)
    eo = assert_close(go, ro, io, what + " o")
    eh = assert_close(hT[sq][:, hs], rh, io, what + " h_T")
    log(what, "o", eo, "h_T", eh)


@pytest.mark.parametrize("gate", ["scalar", "none"])
@pytest.mark.parametrize("io,dk,dv", [("bf16", 128, 128), ("bf16", 64, 128), ("f32", 128, 64), ("f32", 64, 64)])
def test_gdn_ragged_varlen(kda, gate, io, dk, dv):
    """Ragged packed sequences with h0; the scalar gate includes near-resets and
    a chunk whose decay exceeds the matrix-core range (token path)."""
    cfg = I.ChunkConfig("gdn", io, io, H=3, dk=dk, dv=dv, h0=True, seed=41)
    d = I.make_chunk_inputs(cfg, lengths=[300, 64, 130, 1, 200])
    g = None
    if gate == "none":
        # With no decay the state keeps growing (|o| reaches ~2.7 here), and a
        # bf16 output in [2, 4) alone rounds by up to 7.8e-3, above the 5e-3
        # max-abs bound.  o is linear in (v, h0): scale both so |o| stays below 1.
        d["v"] = (d["v"].float() * 0.35).to(d["v"].dtype)
        d["h0"] = d["h0"] * 0.35
    if gate == "scalar":
        g = d["log_alpha"][:, :, 0].float().clone()
        g[10] = -30.0
        g[300:364, 1] = -2.0          # sequence 1, head 1: -128 over one chunk
        g = g.to(d["log_alpha"].dtype).contiguous()
    _gdn_check(kda, d, g, io, "gdn %s %s dk=%d dv=%d" % (gate, io, dk, dv))


@pytest.mark.parametrize("gate", ["scalar", "none"])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128)])
def test_gdn_single_sequence_strong(kda, gate, dk, dv):
    """One sequence (prep + state kernels, where the scalar gate makes the Gram
    blocks plain products of the raw keys and queries under a pairwise decay
    mask): a reset, a whole chunk at log alpha = -6 per token (384 nats), and a
    partial last chunk; with no gate, values scaled so that |o| stays below 1."""
    cfg = I.ChunkConfig("gdn1", "bf16", "bf16", H=3, dk=dk, dv=dv, T=300, h0=True, seed=43)
    d = I.make_chunk_inputs(cfg)
    g = None
    if gate == "scalar":
        g = d["log_alpha"][:, :, 0].float().clone()
        g[10] = -30.0
        g[64:128, 1] = -6.0
        g[270:280, 2] = -5.0
        g = g.to(d["log_alpha"].dtype).contiguous()
    else:
        d["v"] = (d["v"].float() * 0.35).to(d["v"].dtype)
        d["h0"] = d["h0"] * 0.35
    _gdn_check(kda, d, g, "bf16", "gdn one sequence %s dk=%d" % (gate, dk))


def test_gdn_c3_full(kda):
    """c3's full size with one decay per token and head (c3's per-channel draw,
    first channel); the oracle checks every head."""
    d = I.make_chunk_inputs(I.C3)
    g = d["log_alpha"][:, :, 0].contiguous()
    _gdn_check(kda, d, g, "bf16", "gdn c3 all heads")


@pytest.mark.parametrize("gate", ["scalar", "none"])
def test_gdn_decode(kda, gate):
    cfg = I.DecodeConfig("gdn-dec", "f32", "f32", B=5, H=3, dk=128, dv=64, steps=3, seed=2300)
    S = I.make_decode_state(cfg)
    Sg, Sref = S.to(DEV), f64(S)
    steps = I.make_decode_step_inputs(cfg, 0, steps=3)
    for s in range(3):
        x = {n: t[s] for n, t in steps.items()}
        g = x["log_alpha"][:, :, 0].contiguous() if gate == "scalar" else None
        o = kda.kda_gdn_decode_step(x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV),
                                    None if g is None else g.to(DEV), x["beta"].to(DEV), Sg)
        la = np.zeros(tuple(x["q"].shape)) if g is None else np.repeat(f64(g)[:, :, None], 128, axis=2)
        ro, Sref = oracle.decode(f64(x["q"]), f64(x["k"]), f64(x["v"]), la, f64(x["beta"]), Sref)
        assert_close(o.cpu(), ro, "f32", "gdn decode o")
    assert_close(Sg.cpu(), Sref, "f32", "gdn decode S")


# ------------------------------------------------------------------ decoupled strengths
# kda_chunk_fwd_decoupled / kda_decode_step_decoupled against the oracle's
# generalised recurrence S <- (I - b k k^T) Diag(alpha) S + w k v^T (pinned: b = w
# is KDA, b = 0, w = 1, alpha = 1 is linear attention).
def _dec_check(kda, d, wv, io, what, heads=None):
    dev = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    cu = dev["cu_seqlens"] if len(d["lengths"]) > 1 else None
    o, hT = kda.kda_chunk_fwd_decoupled(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], wv.to(DEV),
                                        h0=dev["h0"], cu_seqlens=cu)
    torch.cuda.synchronize()
    o, hT = o.cpu(), hT.cpu()
    dd = dict(d)
    dd["w"] = wv
    ref = to_oracle(dd, None, heads)
    hs = slice(None) if heads is None else list(heads)
    wref = f64(wv)[ref["rows"]][:, hs]
    ro, rh = oracle.gen_fwd(ref["q"], ref["k"], ref["v"], ref["log_alpha"], ref["beta"], wref, h0=ref["h0"],
                            cu_seqlens=ref["cu_seqlens"])
    go = o.reshape(-1, *o.shape[-2:])[torch.from_numpy(ref["rows"])][:, hs]
    eo = assert_close(go, ro, io, what + " o")
    eh = assert_close(hT[:, hs], rh, io, what + " h_T")
    log(what, "o", eo, "h_T", eh)


@pytest.mark.parametrize("case", ["independent", "erase_only", "write_only"])
@pytest.mark.parametrize("io,dk,dv", [("bf16", 128, 128), ("bf16", 64, 64), ("f32", 128, 128), ("f32", 64, 128)])
def test_decoupled_ragged_varlen(kda, case, io, dk, dv):
    """Ragged packed sequences with h0 and a flagged chunk (token path); write
    strengths drawn independently of beta, or one of the two strengths zero."""
    cfg = I.ChunkConfig("dec", io, io, H=3, dk=dk, dv=dv, h0=True, seed=51)
    d = I.make_chunk_inputs(cfg, lengths=[300, 64, 130, 1, 200])
    la = d["log_alpha"].clone()
    la[300:364, 1, :3] = -2.0      # sequence 1, head 1: a chunk beyond the matrix-core range
    d["log_alpha"] = la
    wv = I.draw_strength(d["beta"].shape, 5100, d["beta"].dtype)
    if case == "erase_only":
        wv = torch.zeros_like(wv)
    elif case == "write_only":
        d["beta"] = torch.zeros_like(d["beta"])
    _dec_check(kda, d, wv, io, "decoupled %s %s dk=%d dv=%d" % (case, io, dk, dv))


def test_decoupled_c3_full(kda):
    """c3's full size with the write strength drawn independently of beta; the
    oracle checks every head."""
    d = I.make_chunk_inputs(I.C3)
    wv = I.draw_strength(d["beta"].shape, 5200, d["beta"].dtype)
    _dec_check(kda, d, wv, "bf16", "decoupled c3 all heads")


def test_decoupled_decode(kda):
    cfg = I.DecodeConfig("dec-dec", "f32", "f32", B=5, H=3, dk=128, dv=128, steps=3, seed=2400)
    S = I.make_decode_state(cfg)
    Sg, Sref = S.to(DEV), f64(S)
    steps = I.make_decode_step_inputs(cfg, 0, steps=3)
    for s in range(3):
        x = {n: t[s] for n, t in steps.items()}
        wv = I.draw_strength(x["beta"].shape, 5300 + s, torch.float32)
        o = kda.kda_decode_step_decoupled(x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV), x["log_alpha"].to(DEV),
                                          x["beta"].to(DEV), wv.to(DEV), Sg)
        Sn = np.zeros_like(Sref)
        ro = np.zeros((cfg.B, cfg.H, cfg.dv))
        # one step per (b, h) chain: the generalised recurrence with h0 = S
        cu = np.arange(cfg.B + 1)
        ro, Sn = oracle.gen_fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["log_alpha"]), f64(x["beta"]), f64(wv),
                                h0=Sref, cu_seqlens=cu)
        Sref = Sn
        assert_close(o.cpu(), ro, "f32", "decoupled decode o")
    assert_close(Sg.cpu(), Sref, "f32", "decoupled decode S")


# ------------------------------------------------------------------ long-sequence segments
def test_long_sequence_segments(kda):
    """A single long sequence runs as segments of 64 chunks at H = 32 (records
    kept in the last-level cache): three segments, the last partial, with h0, a
    near-reset across the first segment boundary (token path), and h_T aliasing
    h0 on a second call."""
    cfg = I.ChunkConfig("seg", "bf16", "bf16", H=32, dk=128, dv=128, T=2 * 4096 + 77, seed=61, h0=True)
    d = I.make_chunk_inputs(cfg)
    la = d["log_alpha"].clone()
    la[4090:4100] = -30.0
    d["log_alpha"] = la
    heads = [0, 13, 31]
    check_against_oracle(kda, d, "bf16", heads=heads, what="segments T=%d" % cfg.T)
    # h_T written over h0 in place
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    o1, h1 = kda.kda_chunk_fwd(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], h0=g["h0"])
    hh = g["h0"].clone()
    o2, h2 = kda.kda_chunk_fwd(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], h0=hh, h_T=hh)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2) and h2.data_ptr() == hh.data_ptr()


# ------------------------------------------------------------------ pipelined segments
# A single sequence at d_k = 128 whose state pass has at most 128 workgroups
# (one per compute unit, half the chip) runs as two or more segments of at most
# 1,024 chunk-heads, each launch running the state pass of one segment beside
# the prep pass of the next.
def test_pipelined_segments(kda):
    """H = 16, d = 128, T = 8333 (131 chunks: segments of 64, 64 and 3
    chunks, the last with a 13-token tail), h0 given; a near-reset across the
    first segment boundary and one fast-forgetting channel inside the second
    segment, whose records a combined launch prepares; then h_T written over
    h0 in place."""
    cfg = I.ChunkConfig("pipe", "bf16", "bf16", H=16, dk=128, dv=128, T=8333, seed=71, h0=True)
    d = I.make_chunk_inputs(cfg)
    la = d["log_alpha"].clone()
    la[4090:4100] = -30.0          # tokens on both sides of the first boundary (4096)
    la[5000:5064, 5, 11] = -3.0    # one channel of head 5 over a chunk of segment 2
    d["log_alpha"] = la
    check_against_oracle(kda, d, "bf16", what="pipelined segments H=16 T=%d" % cfg.T)
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    o1, h1 = kda.kda_chunk_fwd(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], h0=g["h0"])
    hh = g["h0"].clone()
    o2, h2 = kda.kda_chunk_fwd(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], h0=hh, h_T=hh)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2) and h2.data_ptr() == hh.data_ptr()


def test_pipelined_paired_prep_strong_decay(kda):
    """The combined launch prepares two chunk-heads per workgroup (chunk-heads
    2i and 2i + 1: consecutive heads of a chunk, or the last head of one chunk
    and the first of the next), which must agree on the Gram path and the
    number of exact-pair groups.  H = 5, T = 1940 (31 chunks: segments of 16 and
    15 chunks, the second with a 20-token tail and an odd 75 chunk-heads, so
    its last workgroup prepares one).  In chunk 2 of the second segment: head 1
    past the anchored range on every channel (128 big channels, staged from
    the inputs) beside head 0 with none; head 2 with three big channels
    (staged from registers) beside head 3 with none; head 4 with three beside
    head 0 of chunk 3 with twenty.  In the partial last chunk head 4, the lone chunk-head, has one;
    segment 0 (the prep kernel alone) has a near-reset too."""
    cfg = I.ChunkConfig("pipepair", "bf16", "bf16", H=5, dk=128, dv=128, T=1940, seed=73, h0=True)
    d = I.make_chunk_inputs(cfg)
    la = d["log_alpha"].clone()
    c2 = 1024 + 128                  # chunk 2 of the second segment
    la[300, 2] = -30.0               # segment 0, head 2: a reset
    la[c2 + 5:c2 + 8, 1] = -30.0     # head 1: every channel, over 80 nats
    la[c2:c2 + 64, 2, 4:7] = -2.0    # head 2: three channels, -128 each
    la[c2:c2 + 64, 4, 0:3] = -2.0    # head 4: three channels
    la[c2 + 64:c2 + 128, 0, 20:40] = -2.0   # head 0 of chunk 3: twenty channels
    la[1920:1940, 4, 9] = -5.0       # head 4, partial last chunk: -100 on one channel
    d["log_alpha"] = la
    check_against_oracle(kda, d, "bf16", what="pipelined paired prep, strong decay")


@pytest.mark.parametrize("gate", ["channel", "scalar", "none"])
@pytest.mark.parametrize("H,dv,T", [(5, 128, 2000), (32, 64, 1100)])
def test_pipelined_segments_variants(kda, gate, H, dv, T):
    """The pipelined launches with per-channel, per-head and no gates; H = 5
    (state blocks padded to 8 chains, the padding blocks ending at once; two
    segments of 16 chunks, the second ragged) and H = 32 at d_v = 64 (exactly
    128 state blocks; segments of 9 and 9 chunks, the second ragged)."""
    cfg = I.ChunkConfig("pipev", "bf16", "bf16", H=H, dk=128, dv=dv, T=T, seed=72, h0=True)
    d = I.make_chunk_inputs(cfg)
    if gate == "channel":
        check_against_oracle(kda, d, "bf16", what="pipelined H=%d dv=%d T=%d" % (H, dv, T))
        return
    g = None
    if gate == "scalar":
        g = d["log_alpha"][:, :, 0].float().clone()
        g[600:610] = -30.0
        g = g.to(d["log_alpha"].dtype).contiguous()
    else:
        d["v"] = (d["v"].float() * 0.35).to(d["v"].dtype)
        d["h0"] = d["h0"] * 0.35
    _gdn_check(kda, d, g, "bf16", "pipelined gdn %s H=%d dv=%d T=%d" % (gate, H, dv, T))


# ------------------------------------------------------------------ invariants at full size
# Properties of the recurrence that hold at any size, checked on the GPU at the
# long-context shape the benchmark times (no oracle needed): the value columns
# of S evolve independently, and o, h_T are homogeneous in q and linear in
# (v, h0) jointly.  Each value column's arithmetic is the same whichever block
# it lands in, and scaling by 2 is exact, so both hold bitwise.
def test_c3_value_column_permutation(kda):
    d = I.make_chunk_inputs(I.C3)
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    H, dv = g["v"].shape[1], g["v"].shape[2]
    h0 = 0.1 * torch.randn((1, H, 128, dv), generator=torch.Generator().manual_seed(4800)).to(DEV)
    perm = torch.randperm(dv, generator=torch.Generator().manual_seed(4801)).to(DEV)
    o, hT = kda.kda_chunk_fwd(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], h0=h0)
    op, hp = kda.kda_chunk_fwd(g["q"], g["k"], g["v"][..., perm].contiguous(), g["log_alpha"], g["beta"],
                               h0=h0[..., perm].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(op, o[..., perm]) and torch.equal(hp, hT[..., perm])


def test_c3_homogeneity_and_linearity(kda):
    d = I.make_chunk_inputs(I.C3)
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    H, dv = g["v"].shape[1], g["v"].shape[2]
    h0 = 0.1 * torch.randn((1, H, 128, dv), generator=torch.Generator().manual_seed(4900)).to(DEV)
    o, hT = kda.kda_chunk_fwd(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], h0=h0)
    oq, hq = kda.kda_chunk_fwd(2 * g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], h0=h0)
    ov, hv = kda.kda_chunk_fwd(g["q"], g["k"], 2 * g["v"], g["log_alpha"], g["beta"], h0=2 * h0)
    torch.cuda.synchronize()
    assert torch.equal(oq, 2 * o) and torch.equal(hq, hT)        # o is linear in q; h_T does not see q
    assert torch.equal(ov, 2 * o) and torch.equal(hv, 2 * hT)
