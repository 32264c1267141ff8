"""Shared helpers for the GPU parity tests: tolerance checks and oracle calls."""
import numpy as np
import torch

# Tolerances of the path: bf16 I/O -- max-abs 5e-3 and relative Frobenius 1e-2;
# fp32 I/O -- 1e-4 relative (Frobenius and max-norm).  Applied to o and h_T.
BF16_MAX_ABS = 5e-3
BF16_REL_FRO = 1e-2
F32_REL = 1e-4


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy() if isinstance(t, torch.Tensor) else np.asarray(t, np.float64)


def errors(out, ref):
    out, ref = f64(out), f64(ref)
    d = out - ref
    nref = np.linalg.norm(ref)
    return dict(max_abs=float(np.abs(d).max()) if d.size else 0.0,
                rel_fro=float(np.linalg.norm(d) / nref) if nref > 0 else float(np.linalg.norm(d)),
                rel_max=float(np.abs(d).max() / np.abs(ref).max()) if d.size and np.abs(ref).max() > 0 else 0.0)


def bf16_rounding_stats(out, ref):
    """How bf16 outputs compare with the oracle rounded to bf16 (diagnostic
    only; the tolerance is the one above): the share of elements equal to the
    rounded oracle value, the largest error that rounding alone makes
    (|rn(ref) - ref|, up to 3.9e-3 for |o| in [1, 2)), and the largest excess
    of an element's error over that rounding error (|out - ref| - |rn(ref) - ref|),
    i.e. the path's own arithmetic at its worst element."""
    ref = f64(ref)
    o = f64(out)
    r = torch.as_tensor(ref).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    if o.size == 0:
        return dict(exact=1.0, max_rounding=0.0, max_excess=0.0)
    rnd = np.abs(r - ref)
    exc = np.abs(o - ref) - rnd
    return dict(exact=float((o == r).mean()), max_rounding=float(rnd.max()), max_excess=float(exc.max()))


def assert_close(out, ref, io, what=""):
    e = errors(out, ref)
    if io == "bf16":
        ok = e["max_abs"] <= BF16_MAX_ABS and e["rel_fro"] <= BF16_REL_FRO
    else:
        ok = e["rel_fro"] <= F32_REL and e["rel_max"] <= F32_REL
    assert ok, "%s: %s (io=%s)" % (what, e, io)
    return e


def to_oracle(d, seqs=None, heads=None):
    """Slices the packed inputs dict to the given sequences/heads and returns
    fp64 numpy arrays plus cu_seqlens for the oracle."""
    lengths = d["lengths"]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    seqs = list(range(len(lengths))) if seqs is None else list(seqs)
    hs = slice(None) if heads is None else list(heads)
    idx = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in seqs]) if seqs else np.zeros(0, np.int64)
    idx_t = torch.from_numpy(idx)
    pick = lambda t: f64(t.detach().cpu()[idx_t][:, hs])
    out = dict(q=pick(d["q"]), k=pick(d["k"]), v=pick(d["v"]), log_alpha=pick(d["log_alpha"]),
               beta=pick(d["beta"]))
    sub_len = [lengths[s] for s in seqs]
    out["cu_seqlens"] = np.concatenate([[0], np.cumsum(sub_len)]).astype(np.int64)
    out["h0"] = None if d["h0"] is None else f64(d["h0"].cpu()[seqs][:, hs])
    out["rows"] = idx
    return out
