#!/usr/bin/env python3
"""Benchmark of the KDA hot path on one MI355X.

One "step" is one kda_chunk_fwd call over the long-context prefill workload
(bf16, B=1, H=32, T=65536, d_k=d_v=128, chunk 64, per-channel decay in
[0.5, 0.9999]); inputs are seeded, synthetic and resident in HBM before timing.
The decode step (B=256 resident fp32 states, H=32, d=128, 1000 steps with fresh
inputs) is timed in the same run and reported under "decode"; the same prefill
on raw projections through the fused input prologue (kda_chunk_fwd_prologue)
under "prologue"; the same shape with one decay per token and head (Gated
DeltaNet) and with none (DeltaNet), through kda_gdn_chunk_fwd, under "gdn"; and
with separate erase and write strengths (kda_chunk_fwd_decoupled) under
"decoupled"; the gradients of the same prefill (kda_chunk_bwd, and the
scalar-gate, separate-strength and raw-projection backwards) under "backward"; kda_chunk_fwd on the small fp32 (H=2, T=256, d=64), short (H=16, T=4096) and
packed variable-length (32 sequences of 512-8192 tokens, h0 given) workloads
under "other_workloads"; and the long-context prefill with one fast-forgetting
key channel per head (log alpha = -3 per token) under "strong_decay".

Prints ONE JSON line.  Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0 # MI355X dense bf16 matrix peak, published
FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix peak, published
METRIC = "KDA chunk_fwd tokens/s + % MFMA peak; decode step HBM GB/s (1×MI355X)"


def chunk_alg_bytes(tok_heads, n_states, dk, dv, io_b=2, gate_b=2, gate_per_th=None):
    """Algorithmic HBM bytes of one chunk_fwd launch: q, k, log_alpha (d_k each,
    or gate_per_th values for the scalar-gate forms), v and o (d_v each), beta
    (1) per token-head, plus h_T (and h0) per state."""
    ng = dk if gate_per_th is None else gate_per_th
    per = 2 * dk * io_b + ng * gate_b + 2 * dv * io_b + gate_b
    return tok_heads * per + n_states * dk * dv * 4


def chunk_alg_flops(tok_heads, dk, dv, C=64):
    """Algorithmic flops per token-head (triangles counted as triangles):
    A and P Gram blocks, the UT transform, U, the three state products and P.U."""
    per = 2 * ((C - 1) / 2 * dk + (C + 1) / 2 * dk + C * C / 6 + (C - 1) / 2 * (dk + dv)
               + 3 * dk * dv + (C + 1) / 2 * dv)
    return tok_heads * per


def bwd_alg_flops(tok_heads, dk, dv, C=64):
    """Algorithmic flops per token-head of the chunkwise backward (triangles as
    triangles): the prep (the two Gram blocks, the UT transform, W), the state
    replay (U, the state update), the reverse pass (dU, the state gradient) and
    the per-chunk gradients (X, dY, dP, dA, dQA, dKA, dKB, dKI)."""
    prep = C * dk + C * C / 6 + (C - 1) / 2 * dk
    replay = (C - 1) / 2 * dv + 2 * dk * dv
    reverse = (C + 1) / 2 * dv + 3 * dk * dv
    grads = 4 * dk * dv + 3 * C / 2 * dv + C * dk + C * dk
    return tok_heads * 2 * (prep + replay + reverse + grads)


def bwd_alg_bytes(tok_heads, dk, dv, io_b=2, gate_b=2):
    """Algorithmic HBM bytes of one backward call: q, k, v, log_alpha, beta and
    grad_o read, grad_q, grad_k, grad_v, grad_log_alpha and grad_beta written,
    per token-head."""
    reads = (2 * dk + 2 * dv) * io_b + dk * gate_b + gate_b
    writes = (2 * dk + dv) * io_b + dk * gate_b + gate_b
    return tok_heads * (reads + writes)


def decode_alg_bytes(B, H, dk, dv, io_b=2, gate_b=2):
    per_state = 2 * dk * dv * 4 + (2 * dk + 2 * dv) * io_b + dk * gate_b + gate_b
    return B * H * per_state


CHUNK_SOURCES = ("kda_chunk.hip", "kda_chunk2.hip", "kda_fused.hip", "kda_chunk_common.h", "kda_plan.h", "kda_device.h")
DECODE_SOURCES = ("kda_decode.hip", "kda_device.h")
BWD_SOURCES = ("kda_bwd.hip", "kda_plan.h", "kda_device.h")


def source_digest(files):
    """Digest of the kernel sources a counter profile was taken with."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "gated_delta_rule_chunkwise_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(name, digest):
    """Counter-measured HBM bytes per call, from a committed rocprofv3 summary;
    None when absent or when the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", name)
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_digest") != digest:
        return None
    return rec.get("hbm_bytes_per_call")


def load_mfma_counters(name, digest):
    """Counter-measured matrix-core busy share and matrix flops per call, from the
    same committed summary; None when absent or stale."""
    try:
        with open(os.path.join(ROOT, "profiles", name)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_digest") != digest or rec.get("mfma_busy_pct") is None:
        return None
    return {"busy_pct": rec["mfma_busy_pct"], "flops_per_call": rec.get("mfma_flops_per_call")}


def copy_calibration():
    """A plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE
    counters to bytes: 1 GiB read + 1 GiB written per launch, three launches."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read_per_launch": n, "bytes_written_per_launch": n,
                                           "launches": 3}}), flush=True)


def time_launches(fn, steps, warmup, stream):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return per, wall


def cpu_baseline_chunk(d, heads, T_sample, H_total):
    """Times the fp64 oracle (as it stands) on host cores on a bounded sample of
    the same workload: `heads` whole chains over the first T_sample tokens."""
    import oracle
    oracle.build(force=False)
    sl = slice(0, T_sample)
    f = lambda x: x[sl][:, :heads].to("cpu", torch.float64).numpy()
    q, k, v, la, be = (np.ascontiguousarray(f(d[x])) for x in ("q", "k", "v", "log_alpha", "beta"))
    nthreads = min(heads, oracle.default_threads())
    t0 = time.perf_counter()
    oracle.fwd(q, k, v, la, be, nthreads=nthreads)
    dt = time.perf_counter() - t0
    tok_heads = heads * T_sample
    return {"value": tok_heads / H_total / dt, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "sample": "fp64 per-token recurrence, %d heads x first %d tokens of the same inputs "
                      "(%d token-heads, %.1f s); tokens/s = token-heads/s / %d heads"
                      % (heads, T_sample, tok_heads, dt, H_total)}


def cpu_baseline_bwd(d, go, heads, T_sample, H_total):
    """Times the oracle's backward (as it stands) on a bounded sample: `heads`
    whole chains over the first T_sample tokens of the same inputs."""
    import oracle
    oracle.build(force=False)
    sl = slice(0, T_sample)
    f = lambda x: np.ascontiguousarray(x[sl][:, :heads].to("cpu", torch.float64).numpy())
    q, k, v, la, be, do = (f(x) for x in (d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], go))
    nthreads = min(heads, oracle.default_threads())
    t0 = time.perf_counter()
    oracle.bwd(q, k, v, la, be, do, nthreads=nthreads)
    dt = time.perf_counter() - t0
    tok_heads = heads * T_sample
    return {"value": tok_heads / H_total / dt, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "sample": "fp64 reverse-mode per-token recurrence, %d heads x first %d tokens (%d token-heads, "
                      "%.1f s); tokens/s = token-heads/s / %d heads" % (heads, T_sample, tok_heads, dt, H_total)}


# Workloads that --only can select, each timed by one section of main().
ONLY = ("c3", "prologue", "gdn_gated", "gdn_deltanet", "decoupled", "strong", "c0", "c1", "c2", "c1_fp32",
        "bwd", "bwd_prologue", "bwd_decoupled", "bwd_gdn", "bwd_c2", "decode")


def time_pipelined(fn, calls, stream):
    """Mean time per call of `calls` back-to-back calls between one event pair:
    the device time per call once the host's per-call marshalling overlaps the
    previous call (for calls too short to hide it one at a time)."""
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(calls):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / calls


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-prologue", action="store_true")
    ap.add_argument("--no-gdn", action="store_true")
    ap.add_argument("--no-decoupled", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-other", action="store_true")
    ap.add_argument("--no-strong", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=32)
    ap.add_argument("--cpu-tokens", type=int, default=65536)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a 1 GiB device copy (counter calibration) and exit")
    ap.add_argument("--only", choices=ONLY, default=None,
                    help="time one workload alone (for per-workload profiler runs); the JSON line then "
                         "holds that entry and the number of entry-point calls made")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import gated_delta_rule_chunkwise_amd as kda
    from gated_delta_rule_chunkwise_amd import inputs as I
    kda.load_library()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    calls = {}   # entry-point calls made per workload (for profiler runs)

    def want(name, skip_flag=False):
        return (args.only is None and not skip_flag) or args.only == name

    # ---------------- chunk_fwd on the long-context prefill workload
    cfg = I.C3
    d = I.make_chunk_inputs(cfg, device=dev)
    T, H, dk, dv = sum(d["lengths"]), cfg.H, cfg.dk, cfg.dv
    o = torch.empty((T, H, dv), dtype=torch.bfloat16, device=dev)
    hT = torch.empty((1, H, dk, dv), dtype=torch.float32, device=dev)
    args_c = (d["q"], d["k"], d["v"], d["log_alpha"], d["beta"])
    fn = lambda: kda.kda_chunk_fwd(*args_c, o=o, h_T=hT)
    if want("c3"):
        per, wall = time_launches(fn, args.steps, args.warmup, stream)
        calls["c3"] = args.steps + args.warmup
        ms = float(np.mean(per))
        print("chunk_fwd per-launch ms: mean %.4f median %.4f min %.4f" % (ms, np.median(per), min(per)),
              file=sys.stderr, flush=True)
    else:
        ms = float("nan")
    tok_heads = T * H
    alg_b = chunk_alg_bytes(tok_heads, H, dk, dv)
    alg_f = chunk_alg_flops(tok_heads, dk, dv)
    digest = source_digest(CHUNK_SOURCES)
    traffic = load_traffic("chunk_fwd_prefill_h32_t65536_traffic.json", digest)
    counters = load_mfma_counters("chunk_fwd_prefill_h32_t65536_traffic.json", digest)
    # one kda_chunk_fwd call = chunk_prep_kernel + chunk_state_kernel on one stream.
    # Roofline: the call's arithmetic intensity (algorithmic flops over
    # algorithmic bytes, about 110 flop/B) lies below the chip's ridge point
    # (2,500 TFLOP/s over 8 TB/s = 312 flop/B), so the bytes bind first and the
    # roofline is HBM's; at that intensity the matrix cores can be at most
    # 110/312 = 35% busy.  The metric's matrix-core share (algorithmic, and
    # counter-measured) is reported under "mfma".  "traffic" is FETCH_SIZE +
    # WRITE_SIZE per call (bytes leaving L2, Infinity Cache hits included)
    # scaled by a plain copy.
    roof = {"bound": "hbm", "achieved": alg_b / (ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": alg_b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "traffic": traffic,
            "traffic_counted": "FETCH_SIZE + WRITE_SIZE (L2 misses, Infinity Cache hits included), bytes per call",
            "kernel": "kda_chunk_fwd = chunk_prep_kernel<128,128,bf16,bf16,false,0> + "
                      "chunk_state_kernel<128,128,16,bf16,bf16,false,0>",
            "alg_bytes_per_launch": alg_b, "alg_flops_per_launch": alg_f,
            "arith_intensity_flop_per_byte": alg_f / alg_b,
            "ridge_flop_per_byte": BF16_MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)}
    hbm = {"bound": "hbm", "achieved": alg_b / (ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": alg_b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "alg_bytes_per_launch": alg_b,
           "floor_ms": alg_b / (HBM_PEAK_GBS * 1e9) * 1e3}
    mfma = {"alg_flops_per_launch": alg_f, "achieved_tflops": alg_f / (ms * 1e-3) / 1e12,
            "peak_tflops": BF16_MFMA_PEAK_TFLOPS,
            "frac": alg_f / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
            "frac_attainable_at_intensity": alg_f / alg_b / (BF16_MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)),
            "counter_busy_frac": None if counters is None else counters["busy_pct"] / 100.0,
            "counters": counters}

    out = {} if not want("c3") else {"metric": METRIC, "value": T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "kda_chunk_fwd bf16 B=1 H=32 T=65536 d_k=d_v=128 chunk=64, "
                                  "log_alpha=log U(0.5,0.9999)",
                      "B": 1, "T": T, "H": H, "d_k": dk, "d_v": dv, "chunk": 64,
                      "parallelism": "single GPU"},
           "roofline": roof, "hbm": hbm, "mfma": mfma, "source_digest": digest}

    # ---------------- the same prefill on raw projections (fused input prologue)
    if want("prologue", args.no_prologue):
        dr = I.make_chunk_raw_inputs(cfg, device=dev, gate="uniform")
        args_p = (dr["q_raw"], dr["k_raw"], dr["v"], dr["gate_pre"], dr["beta_pre"])
        lo = -30.0
        fnp = lambda: kda.kda_chunk_fwd_prologue(*args_p, lo, o=o, h_T=hT)
        per_p, _ = time_launches(fnp, args.steps, args.warmup, stream)
        calls["prologue"] = args.steps + args.warmup
        pms = float(np.mean(per_p))
        # a separate prologue pass would read q, k, the gate and beta raw and write
        # them back mapped: twice their bytes per token-head
        sep_b = tok_heads * 2 * (2 * dk * 2 + dk * 2 + 2)
        out["prologue"] = {
            "workload": "kda_chunk_fwd_prologue bf16 B=1 H=32 T=65536 d_k=d_v=128 chunk=64 on raw "
                        "projections (q, k ~ N(0,1) unnormalised; beta_pre ~ N(0,1); gate_pre ~ "
                        "U(%.3f, 0), i.e. decay in [0.5, 0.9999]; floor -30)" % I.RAW_GATE_LO,
            "ms_per_step": pms, "tokens_per_s": T / (pms * 1e-3), "vs_plain_ms": pms / ms,
            "roofline": {"bound": "hbm", "achieved": alg_b / (pms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": alg_b / (pms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "traffic": load_traffic("chunk_fwd_prologue_prefill_h32_t65536_traffic.json", digest),
                         "kernel": "kda_chunk_fwd_prologue = chunk_prep_kernel<128,128,bf16,bf16,true,0> + "
                                   "chunk_state_kernel<128,128,16,bf16,bf16,true,0>",
                         "alg_bytes_per_launch": alg_b},
            "separate_pass_alg_bytes": sep_b,
            "separate_pass_floor_ms": sep_b / (HBM_PEAK_GBS * 1e9) * 1e3}
        del dr, args_p

    # ---------------- scalar gates: Gated DeltaNet and DeltaNet on the same shape
    if want("gdn_gated", args.no_gdn) or want("gdn_deltanet", args.no_gdn):
        g = d["log_alpha"][:, :, 0].contiguous()   # c3's draw, one decay per (token, head)
        gdn = {"workload": "kda_gdn_chunk_fwd bf16 B=1 H=32 T=65536 d_k=d_v=128 chunk=64, log_alpha "
                           "[T, H] = the first channel of the same per-channel draw; and with "
                           "log_alpha = NULL (DeltaNet)"}
        for key, gate, ng in (("gated", g, 1), ("deltanet", None, 0)):
            if not want("gdn_" + key, args.no_gdn):
                continue
            fng = lambda: kda.kda_gdn_chunk_fwd(d["q"], d["k"], d["v"], gate, d["beta"], o=o, h_T=hT)
            per_g, _ = time_launches(fng, args.steps, args.warmup, stream)
            calls["gdn_" + key] = args.steps + args.warmup
            gms = float(np.mean(per_g))
            gb = chunk_alg_bytes(tok_heads, H, dk, dv, gate_per_th=ng)
            gdn[key] = {"ms_per_step": gms, "tokens_per_s": T / (gms * 1e-3), "vs_plain_ms": gms / ms,
                        "roofline": {"bound": "hbm", "achieved": gb / (gms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                                     "unit": "GB/s", "frac": gb / (gms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                     "traffic": load_traffic("chunk_gdn_%s_prefill_h32_t65536_traffic.json" % key,
                                                             digest),
                                     "alg_bytes_per_launch": gb}}
        out["gdn"] = gdn
        del g

    # ---------------- separate erase and write strengths on the same inputs
    if want("decoupled", args.no_decoupled):
        wv = I.draw_strength(d["beta"].shape, 5200, d["beta"].dtype, device=dev)
        fnd = lambda: kda.kda_chunk_fwd_decoupled(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], wv,
                                                  o=o, h_T=hT)
        per_d, _ = time_launches(fnd, args.steps, args.warmup, stream)
        calls["decoupled"] = args.steps + args.warmup
        dms_ = float(np.mean(per_d))
        db_ = alg_b + tok_heads * 2       # plus the write strength, 2 B per token-head
        out["decoupled"] = {
            "workload": "kda_chunk_fwd_decoupled on the same inputs, beta as the erase strength and a "
                        "write strength drawn like beta from its own seed",
            "ms_per_step": dms_, "tokens_per_s": T / (dms_ * 1e-3), "vs_plain_ms": dms_ / ms,
            "roofline": {"bound": "hbm", "achieved": db_ / (dms_ * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": db_ / (dms_ * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "traffic": load_traffic("chunk_fwd_decoupled_prefill_h32_t65536_traffic.json", digest),
                         "alg_bytes_per_launch": db_}}
        del wv

    # ---------------- strong decay: one fast-forgetting key channel per head
    if want("strong", args.no_strong):
        la_s = d["log_alpha"].clone()
        la_s[:, :, 0] = -3.0   # channel 0 of every head: log alpha = -3 on every token
        fns = lambda: kda.kda_chunk_fwd(d["q"], d["k"], d["v"], la_s, d["beta"], o=o, h_T=hT)
        per_s, _ = time_launches(fns, max(2, args.steps // 4), 1, stream)
        calls["strong"] = max(2, args.steps // 4) + 1
        sms = float(np.mean(per_s))
        out["strong_decay"] = {
            "workload": "kda_chunk_fwd on the same inputs with key channel 0 of every head at log alpha = -3 "
                        "per token (a 192-nat decay per chunk on that channel)",
            "ms_per_step": sms, "tokens_per_s": T / (sms * 1e-3), "vs_plain_ms": sms / ms,
            "traffic": load_traffic("chunk_fwd_strong_decay_prefill_h32_t65536_traffic.json", digest)}
        del la_s

    # ---------------- the other prefill workloads: short sequence and packed batch
    other_keys = ("c0", "c1", "c2", "c1_fp32")
    if any(want(k, args.no_other) for k in other_keys) or want("bwd_c2", args.no_other or args.no_backward):
        other = {}
        # fp32 I/O at d = 128 runs on the backward's kernels (kda_bwd.hip)
        f32_digest = source_digest(CHUNK_SOURCES + ("kda_bwd.hip",))
        profile_name = {"c0": "chunk_fwd_fp32_h2_t256_d64", "c1": "chunk_fwd_h16_t4096",
                        "c2": "chunk_fwd_varlen_n32_h32", "c1_fp32": "chunk_fwd_fp32_h16_t4096_d128"}
        # c1's shape with fp32 I/O at d = 128: the chunkwise fp32 forward
        c1_f32 = I.ChunkConfig("fp32 B=1 H=16 T=4096 d=128 (c1's shape and draws in fp32)", "f32", "f32",
                               H=16, dk=128, dv=128, T=4096, seed=I.C1.seed)
        for key, ocfg in (("c0", I.C0), ("c1", I.C1), ("c2", I.C2), ("c1_fp32", c1_f32)):
            fwd_on = want(key, args.no_other)
            bwd_on = key == "c2" and want("bwd_c2", args.no_other or args.no_backward)
            if not (fwd_on or bwd_on):
                continue
            dd = I.make_chunk_inputs(ocfg, device=dev)
            Tt, Hh = dd["q"].shape[0], dd["q"].shape[1]
            odk, odv = dd["q"].shape[2], dd["v"].shape[2]
            nseq = len(dd["lengths"])
            cu = dd["cu_seqlens"].to(dev) if nseq > 1 else None
            h_T = torch.empty((nseq, Hh, odk, odv), dtype=torch.float32, device=dev)
            o2 = torch.empty_like(dd["v"])
            fno = lambda: kda.kda_chunk_fwd(dd["q"], dd["k"], dd["v"], dd["log_alpha"], dd["beta"], h0=dd["h0"],
                                            cu_seqlens=cu, o=o2, h_T=h_T)
            ob = chunk_alg_bytes(Tt * Hh, nseq * Hh * (2 if dd["h0"] is not None else 1), odk, odv,
                                 io_b=dd["q"].element_size(), gate_b=dd["log_alpha"].element_size())
            of = chunk_alg_flops(Tt * Hh, odk, odv)
            other[key] = {}
            if fwd_on:
                per_o, _ = time_launches(fno, args.steps, args.warmup, stream)
                oms = float(np.mean(per_o))
                # the same calls back to back: the device time per call once the
                # host's marshalling of one call overlaps the previous one
                npipe = 4 * args.steps
                pipe = time_pipelined(fno, npipe, stream)
                calls[key] = args.steps + args.warmup + 1 + npipe
                other[key] = {"workload": "kda_chunk_fwd, " + ocfg.name + (" (%d sequences, %d tokens)" % (nseq, Tt)),
                              "ms_per_step": oms, "tokens_per_s_per_call_events": Tt / (oms * 1e-3),
                              "ms_per_call_pipelined": pipe, "tokens_per_s": Tt / (pipe * 1e-3),
                              "timing": "ms_per_step: one event pair around each call (host marshalling "
                                        "included when the call is shorter than it); tokens_per_s: %d calls "
                                        "back to back between one event pair" % npipe,
                              "hbm_frac": ob / (pipe * 1e-3) / 1e9 / HBM_PEAK_GBS, "alg_bytes_per_launch": ob,
                              "alg_flops_per_launch": of,
                              "mfma_frac": of / (pipe * 1e-3) / 1e12 /
                              (BF16_MFMA_PEAK_TFLOPS if dd["q"].dtype == torch.bfloat16 else FP32_MFMA_PEAK_TFLOPS),
                              "traffic": load_traffic(profile_name[key] + "_traffic.json",
                                                      f32_digest if key == "c1_fp32" else digest)}
            if bwd_on:
                # the packed batch's gradients (grad_o ~ N(0,1), grad_hT ~ N(0, 0.1^2))
                go2, ghT2 = I.make_upstream_grads(dd, 3450, device=dev)
                fnb2 = lambda: kda.kda_chunk_bwd(dd["q"], dd["k"], dd["v"], dd["log_alpha"], dd["beta"], go2,
                                                 h0=dd["h0"], grad_hT=ghT2, cu_seqlens=cu)
                per_b2, _ = time_launches(fnb2, args.steps, args.warmup, stream)
                calls["bwd_c2"] = args.steps + args.warmup
                b2 = float(np.mean(per_b2))
                other[key]["backward"] = {"ms_per_step": b2, "tokens_per_s": Tt / (b2 * 1e-3),
                                          "alg_flops_frac_fp32": bwd_alg_flops(Tt * Hh, dk, dv) / (b2 * 1e-3) / 1e12
                                          / FP32_MFMA_PEAK_TFLOPS}
                del go2, ghT2
            del dd, o2, h_T, cu
        out["other_workloads"] = other

    # ---------------- backward of the same prefill
    if any(want(k, args.no_backward) for k in ("bwd", "bwd_prologue", "bwd_decoupled", "bwd_gdn")):
        go, _ = I.make_upstream_grads(d, 3400, device=dev, with_state=False)
        ws = torch.empty(kda.kda_chunk_bwd_workspace_size(1, T, H, dk, dv, 0, kda.KDA_BF16),
                         dtype=torch.uint8, device=dev)
        a4 = [x.unsqueeze(0) for x in args_c]
        fnb = lambda: kda.kda_chunk_bwd(*a4, go.unsqueeze(0), want_grad_h0=False, workspace=ws)
        bms = float("nan")
        out["backward"] = {}
    if want("bwd", args.no_backward):
        per_b, _ = time_launches(fnb, args.steps, args.warmup, stream)
        calls["bwd"] = args.steps + args.warmup
        bms = float(np.mean(per_b))
        bf = bwd_alg_flops(tok_heads, dk, dv)
        bb = bwd_alg_bytes(tok_heads, dk, dv)
        out["backward"] = {
            "workload": "kda_chunk_bwd on the same inputs, grad_o ~ N(0,1) bf16 (seed 3400), no grad_hT, "
                        "no h0; fp32 arithmetic on the fp32 matrix cores",
            "ms_per_step": bms, "tokens_per_s": T / (bms * 1e-3), "vs_forward_ms": bms / ms,
            "roofline": {"bound": "mfma", "achieved": bf / (bms * 1e-3) / 1e12, "peak": FP32_MFMA_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": bf / (bms * 1e-3) / 1e12 / FP32_MFMA_PEAK_TFLOPS,
                         "traffic": load_traffic("chunk_bwd_prefill_h32_t65536_traffic.json",
                                                 source_digest(BWD_SOURCES)),
                         "kernel": "kda_chunk_bwd = bwd_prep_kernel + bwd_state_kernel (replay and reverse "
                                   "passes in one launch) + bwd_grad_kernel <128,128,bf16,bf16>",
                         "alg_flops_per_launch": bf,
                         "counters": load_mfma_counters("chunk_bwd_prefill_h32_t65536_traffic.json",
                                                        source_digest(BWD_SOURCES))},
            "hbm": {"alg_bytes_per_launch": bb, "achieved_gbs": bb / (bms * 1e-3) / 1e9,
                    "frac": bb / (bms * 1e-3) / 1e9 / HBM_PEAK_GBS},
            "workspace_bytes": ws.numel()}
    if "backward" in out:
        if want("bwd_prologue", args.no_backward or args.no_prologue):
            # the same gradients taken through the input prologue, on raw projections
            del ws
            dr = I.make_chunk_raw_inputs(cfg, device=dev, gate="uniform")
            ws = torch.empty(kda.kda_chunk_bwd_prologue_workspace_size(1, T, H, dk, dv, 0, kda.KDA_BF16),
                             dtype=torch.uint8, device=dev)
            r4 = [dr[n].unsqueeze(0) for n in ("q_raw", "k_raw", "v", "gate_pre", "beta_pre")]
            fnp = lambda: kda.kda_chunk_bwd_prologue(*r4, -30.0, go.unsqueeze(0), want_grad_h0=False, workspace=ws)
            per_pb, _ = time_launches(fnp, args.steps, args.warmup, stream)
            calls["bwd_prologue"] = args.steps + args.warmup
            pbms = float(np.mean(per_pb))
            out["backward"]["prologue"] = {
                "workload": "kda_chunk_bwd_prologue on raw projections of the same shape (as the forward's "
                            "prologue line), floor -30",
                "ms_per_step": pbms, "tokens_per_s": T / (pbms * 1e-3), "vs_kda_backward_ms": pbms / bms,
                "workspace_bytes": ws.numel()}
            del dr, r4, ws
            ws = torch.empty(kda.kda_chunk_bwd_workspace_size(1, T, H, dk, dv, 0, kda.KDA_BF16),
                             dtype=torch.uint8, device=dev)
        if want("bwd_decoupled", args.no_backward or args.no_decoupled):
            # separate erase and write strengths: beta erases, a write strength
            # drawn like beta from its own seed writes
            wv4 = I.draw_strength(d["beta"].shape, 5200, d["beta"].dtype, device=dev).unsqueeze(0)
            fnd = lambda: kda.kda_chunk_bwd_decoupled(*a4, wv4, go.unsqueeze(0), want_grad_h0=False, workspace=ws)
            per_db, _ = time_launches(fnd, args.steps, args.warmup, stream)
            calls["bwd_decoupled"] = args.steps + args.warmup
            dbms = float(np.mean(per_db))
            out["backward"]["decoupled"] = {
                "workload": "kda_chunk_bwd_decoupled on the same inputs, beta as the erase strength",
                "ms_per_step": dbms, "tokens_per_s": T / (dbms * 1e-3), "vs_kda_backward_ms": dbms / bms}
            del wv4
        if want("bwd_gdn", args.no_backward or args.no_gdn):
            # the scalar-gate backward (Gated DeltaNet) on the same inputs, the
            # gate being the first channel of the per-channel draw
            del ws
            g4 = d["log_alpha"][:, :, 0].contiguous().unsqueeze(0)
            ws = torch.empty(kda.kda_gdn_chunk_bwd_workspace_size(1, T, H, dk, dv, 0, kda.KDA_BF16),
                             dtype=torch.uint8, device=dev)
            fng = lambda: kda.kda_gdn_chunk_bwd(a4[0], a4[1], a4[2], g4, a4[4], go.unsqueeze(0),
                                                want_grad_h0=False, workspace=ws)
            per_gb, _ = time_launches(fng, args.steps, args.warmup, stream)
            calls["bwd_gdn"] = args.steps + args.warmup
            gbms = float(np.mean(per_gb))
            out["backward"]["gdn"] = {
                "workload": "kda_gdn_chunk_bwd, log_alpha [T, H] = the first channel of the same draw",
                "ms_per_step": gbms, "tokens_per_s": T / (gbms * 1e-3), "vs_kda_backward_ms": gbms / bms,
                "workspace_bytes": ws.numel()}
            del g4
        if args.only is None and not args.no_cpu_baseline:
            out["backward"]["cpu_baseline"] = cpu_baseline_bwd(d, go, 2, 16384, H)
        del go, ws, a4

    # ---------------- decode step
    if want("decode", args.no_decode):
        dcfg = I.C4
        S = I.make_decode_state(dcfg, device=dev)
        nst = args.decode_steps
        xs = I.make_decode_step_inputs(dcfg, 0, device=dev, steps=nst)
        od = torch.empty((dcfg.B, dcfg.H, dcfg.dv), dtype=torch.bfloat16, device=dev)
        names = ("q", "k", "v", "log_alpha", "beta")
        for s in range(min(3, nst)):
            kda.kda_decode_step(*(xs[n][s] for n in names), S, o=od)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for s in range(nst):
            kda.kda_decode_step(*(xs[n][s] for n in names), S, o=od)
        e1.record(stream)
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1) / nst
        calls["decode"] = min(3, nst) + nst
        db = decode_alg_bytes(dcfg.B, dcfg.H, dcfg.dk, dcfg.dv)
        gbs = db / (dms * 1e-3) / 1e9
        out["decode"] = {"workload": "kda_decode_step bf16 B=256 H=32 d=128 fp32 S (512 MiB), "
                                     "%d steps with fresh inputs" % nst,
                         "ms_per_step": dms, "tokens_per_s": dcfg.B / (dms * 1e-3),
                         "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS,
                                      "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                                      "traffic": load_traffic("decode_step_b256_h32_traffic.json",
                                                              source_digest(DECODE_SOURCES)),
                                      "alg_bytes_per_launch": db}}
        del xs, S

    # ---------------- CPU baseline: the oracle on a bounded sample
    if args.only is None and not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_chunk(d, args.cpu_heads, args.cpu_tokens, H)
    if args.only is not None:
        out = {"only": args.only, "calls": calls.get(args.only), "entries": out}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
