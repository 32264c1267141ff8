"""Seeded synthetic inputs for the KDA forward and decode workloads.

This module only draws random numbers and rounds them to the I/O dtype; it holds
none of the method's arithmetic.  The tests feed the very same tensors to the
HIP library and to the fp64 oracle, and the benchmark uses the same recipes.

Recipe (per token and head unless stated):
  * q, k ~ N(0, 1), L2-normalised over d_k, then rounded to the I/O dtype (RNE);
  * v ~ N(0, 1);
  * beta = sigmoid(N(0, 1));
  * log_alpha = -softplus(N(0, 1)) per channel ("softplus" gate), or
    log(U(0.5, 0.9999)) per channel ("uniform" gate: per-channel decay between
    0.5 and 0.9999), or the same uniform draw held constant over time per
    (head, channel) ("uniform_const", the long-memory variant);
  * h0 = N(0, 0.1^2) per sequence when requested, else absent (zeros);
  * varlen lengths are integers drawn uniformly from [lo, hi] inclusive, always
    by the host's generator (seeded like the call), so that a batch drawn on
    the GPU has the same lengths as the same batch drawn on the host; the
    call's own generator takes the same draw too and discards it, so the
    values that follow keep their stream.  (The host's and the GPU's
    generators give different numbers for one seed: the same recipe drawn on
    the two devices gives equally distributed but different values.)
Draw order for one call: lengths, q, k, v, beta, log_alpha, h0.

Raw projections (for the entry points with the input prologue) are the same
draws before those maps: q_raw, k_raw ~ N(0, 1) (not normalised), beta_pre ~
N(0, 1), gate_pre ~ N(0, gate_scale^2), rounded to their dtypes; with the same
seed they are the pre-images of the recipe above ("softplus" gate).  The
"uniform" raw gate draws gate_pre ~ U(a_lo, 0), the interval that -softplus maps
onto decays between 0.5 and 0.9999.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class ChunkConfig:
    name: str
    io: str            # "f32" or "bf16": dtype of q, k, v, o
    gate_io: str       # dtype of log_alpha and beta
    H: int
    dk: int
    dv: int
    T: int = 0         # tokens per sequence when lengths is None
    B: int = 1         # equal-length sequences (packed into one batch)
    lengths: Optional[tuple] = None   # (count, lo, hi): varlen batch
    gate: str = "softplus"
    h0: bool = False
    seed: int = 1000


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    io: str
    gate_io: str
    B: int
    H: int
    dk: int
    dv: int
    steps: int
    seed: int = 2000


# The five workloads of the path.
C0 = ChunkConfig("fp32 B=1 H=2 T=256 d=64", "f32", "f32", H=2, dk=64, dv=64, T=256, seed=1000)
C1 = ChunkConfig("bf16 B=1 H=16 T=4096 d=128", "bf16", "bf16", H=16, dk=128, dv=128, T=4096,
                 seed=1001)
C2 = ChunkConfig("bf16 varlen N=32 L~U[512,8192] H=32 d=128 h0~N(0,0.1)", "bf16", "bf16", H=32,
                 dk=128, dv=128, lengths=(32, 512, 8192), h0=True, seed=1002)
C3 = ChunkConfig("bf16 B=1 H=32 T=65536 d=128 decay U(0.5,0.9999)", "bf16", "bf16", H=32,
                 dk=128, dv=128, T=65536, gate="uniform", seed=1003)
C4 = DecodeConfig("decode bf16 B=256 H=32 d=128 fp32 S~N(0,0.1)", "bf16", "bf16", B=256, H=32,
                  dk=128, dv=128, steps=1000, seed=2000)
CHUNK_CONFIGS = {"c0": C0, "c1": C1, "c2": C2, "c3": C3}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, g, device):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def _unit_rows(x):
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-30)


def draw_gate(shape, gate: str, g, device):
    """log_alpha draws (fp32, all <= 0)."""
    if gate == "softplus":
        return -torch.nn.functional.softplus(_randn(shape, g, device))
    if gate == "uniform":
        u = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
        return torch.log(0.5 + u * (0.9999 - 0.5))
    if gate == "uniform_const":
        T = shape[0]
        u = torch.rand((1,) + tuple(shape[1:]), generator=g, device=device, dtype=torch.float32)
        return torch.log(0.5 + u * (0.9999 - 0.5)).expand((T,) + tuple(shape[1:])).contiguous()
    raise ValueError("unknown gate " + gate)


def seq_lengths(cfg: ChunkConfig, g=None, device="cpu", seed: Optional[int] = None):
    if cfg.lengths is None:
        return [cfg.T] * cfg.B
    n, lo, hi = cfg.lengths
    seed = cfg.seed if seed is None else seed
    if g is None:
        g = _gen(seed, device)
    torch.randint(lo, hi + 1, (n,), generator=g, device=device)   # the call's stream moves on
    return torch.randint(lo, hi + 1, (n,), generator=_gen(seed, "cpu")).tolist()


def make_chunk_inputs(cfg: ChunkConfig, device="cpu", seed: Optional[int] = None,
                      lengths: Optional[list] = None, gate: Optional[str] = None,
                      h0: Optional[bool] = None):
    """Returns a dict with q, k, v, log_alpha, beta, h0 (or None), cu_seqlens
    (int32, on `device`), lengths (list) -- all contiguous, packed as [T_total, H, d]."""
    seed = cfg.seed if seed is None else seed
    g = _gen(seed, device)
    if lengths is None:
        lengths = seq_lengths(cfg, g, device, seed)
    gate = cfg.gate if gate is None else gate
    want_h0 = cfg.h0 if h0 is None else h0
    T = int(sum(lengths))
    H, dk, dv = cfg.H, cfg.dk, cfg.dv
    io, gio = _DT[cfg.io], _DT[cfg.gate_io]
    q = _unit_rows(_randn((T, H, dk), g, device)).to(io)
    k = _unit_rows(_randn((T, H, dk), g, device)).to(io)
    v = _randn((T, H, dv), g, device).to(io)
    beta = torch.sigmoid(_randn((T, H), g, device)).to(gio)
    la = draw_gate((T, H, dk), gate, g, device).to(gio)
    h0_t = None
    if want_h0:
        h0_t = (0.1 * _randn((len(lengths), H, dk, dv), g, device)).contiguous()
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0)
    return dict(q=q, k=k, v=v, log_alpha=la, beta=beta, h0=h0_t,
                cu_seqlens=cu.to(torch.int32).to(device), lengths=list(lengths))


def make_decode_state(cfg: DecodeConfig, device="cpu", seed: Optional[int] = None):
    g = _gen(cfg.seed if seed is None else seed, device)
    return (0.1 * _randn((cfg.B, cfg.H, cfg.dk, cfg.dv), g, device)).contiguous()


def make_decode_step_inputs(cfg: DecodeConfig, step: int, device="cpu", steps: int = 1):
    """Inputs of `steps` consecutive decode steps starting at `step`, stacked on a
    leading axis: q, k, log_alpha [steps, B, H, dk]; v [steps, B, H, dv];
    beta [steps, B, H].  Each step s is drawn from its own seed (cfg.seed + 1 + s)."""
    io, gio = _DT[cfg.io], _DT[cfg.gate_io]
    B, H, dk, dv = cfg.B, cfg.H, cfg.dk, cfg.dv
    out = {n: [] for n in ("q", "k", "v", "beta", "log_alpha")}
    for s in range(step, step + steps):
        g = _gen(cfg.seed + 1 + s, device)
        out["q"].append(_unit_rows(_randn((B, H, dk), g, device)).to(io))
        out["k"].append(_unit_rows(_randn((B, H, dk), g, device)).to(io))
        out["v"].append(_randn((B, H, dv), g, device).to(io))
        out["beta"].append(torch.sigmoid(_randn((B, H), g, device)).to(gio))
        out["log_alpha"].append(draw_gate((B, H, dk), "softplus", g, device).to(gio))
    return {n: torch.stack(xs).contiguous() for n, xs in out.items()}


# gate pre-activation interval whose -softplus image is log alpha in
# [log 0.5, log 0.9999]: softplus(a) = -log(alpha)  <=>  a = log(expm1(-log(alpha)))
RAW_GATE_LO = math.log(math.expm1(-math.log(0.9999)))
RAW_GATE_HI = math.log(math.expm1(-math.log(0.5)))


def make_chunk_raw_inputs(cfg: ChunkConfig, device="cpu", seed: Optional[int] = None,
                          lengths: Optional[list] = None, h0: Optional[bool] = None,
                          gate_scale: float = 1.0, gate: str = "softplus"):
    """Raw projections for kda_chunk_fwd_prologue: q_raw, k_raw, v, gate_pre,
    beta_pre, h0 (or None), cu_seqlens, lengths (same draw order as
    make_chunk_inputs)."""
    seed = cfg.seed if seed is None else seed
    g = _gen(seed, device)
    if lengths is None:
        lengths = seq_lengths(cfg, g, device, seed)
    want_h0 = cfg.h0 if h0 is None else h0
    T = int(sum(lengths))
    H, dk, dv = cfg.H, cfg.dk, cfg.dv
    io, gio = _DT[cfg.io], _DT[cfg.gate_io]
    q = _randn((T, H, dk), g, device).to(io)
    k = _randn((T, H, dk), g, device).to(io)
    v = _randn((T, H, dv), g, device).to(io)
    beta_pre = _randn((T, H), g, device).to(gio)
    if gate == "uniform":
        u = torch.rand((T, H, dk), generator=g, device=device, dtype=torch.float32)
        gate_pre = (RAW_GATE_LO + u * (RAW_GATE_HI - RAW_GATE_LO)).to(gio)
    elif gate == "softplus":
        gate_pre = (gate_scale * _randn((T, H, dk), g, device)).to(gio)
    else:
        raise ValueError("unknown raw gate " + gate)
    h0_t = None
    if want_h0:
        h0_t = (0.1 * _randn((len(lengths), H, dk, dv), g, device)).contiguous()
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0)
    return dict(q_raw=q, k_raw=k, v=v, gate_pre=gate_pre, beta_pre=beta_pre, h0=h0_t,
                cu_seqlens=cu.to(torch.int32).to(device), lengths=list(lengths))


def make_decode_raw_step_inputs(cfg: DecodeConfig, step: int, device="cpu", steps: int = 1):
    """Raw projections of `steps` decode steps from `step` (same seeds and draw
    order as make_decode_step_inputs): q_raw, k_raw, gate_pre [steps, B, H, dk];
    v [steps, B, H, dv]; beta_pre [steps, B, H]."""
    io, gio = _DT[cfg.io], _DT[cfg.gate_io]
    B, H, dk, dv = cfg.B, cfg.H, cfg.dk, cfg.dv
    out = {n: [] for n in ("q_raw", "k_raw", "v", "beta_pre", "gate_pre")}
    for s in range(step, step + steps):
        g = _gen(cfg.seed + 1 + s, device)
        out["q_raw"].append(_randn((B, H, dk), g, device).to(io))
        out["k_raw"].append(_randn((B, H, dk), g, device).to(io))
        out["v"].append(_randn((B, H, dv), g, device).to(io))
        out["beta_pre"].append(_randn((B, H), g, device).to(gio))
        out["gate_pre"].append(_randn((B, H, dk), g, device).to(gio))
    return {n: torch.stack(xs).contiguous() for n, xs in out.items()}


def draw_strength(shape, seed: int, dtype=torch.bfloat16, device="cpu"):
    """Update strengths drawn like beta, sigmoid(N(0, 1)), from their own seed
    (the separate write strength of the decoupled entry points)."""
    g = _gen(seed, device)
    return torch.sigmoid(_randn(tuple(shape), g, device)).to(dtype)


def make_upstream_grads(d: dict, seed: int, device="cpu", with_state=True):
    """Gradients of a training loss with respect to o and h_T, for the backward:
    grad_o ~ N(0, 1) in the dtype of v, [T_total, H, d_v]; grad_hT ~ N(0, 0.1^2)
    fp32 [N, H, d_k, d_v] (None when with_state is False).  Own seed."""
    g = _gen(seed, device)
    T, H, dv = d["v"].shape
    dk = d["q"].shape[-1]
    N = len(d["lengths"])
    grad_o = _randn((T, H, dv), g, device).to(d["v"].dtype)
    grad_hT = (0.1 * _randn((N, H, dk, dv), g, device)).contiguous() if with_state else None
    return grad_o, grad_hT
