"""Pins of the oracle's backward (``oracle.bwd``) against what does not depend
on its own reverse-mode code.

The backward is the gradient of the KDA forward (the per-token recurrence of
the KimiLinear article, section 2.3; the pages motivate the chunkwise form by
training throughput, sections 3 and 4.1).  It is pinned by
  * central finite differences of the forward oracle, on every input;
  * PyTorch fp64 autograd through a separately written recurrence;
  * closed forms: the frozen state (alpha = 1, beta = 0) and linear attention
    with orthonormal keys (alpha = 1, beta = 1, h0 = 0, section 2.1).
A dropped term (the erase path into dk, the decay into dlog_alpha, the write
into dbeta), a wrong sign or a missing d_hT/dh0 link fails at least one.
"""
import numpy as np
import pytest
import torch

rng0 = np.random.default_rng


def _case(T, H, dk, dv, N, seed, la_scale=1.0):
    r = rng0(seed)
    q = r.standard_normal((T, H, dk))
    k = r.standard_normal((T, H, dk)) / np.sqrt(dk)
    v = r.standard_normal((T, H, dv))
    la = -la_scale * r.uniform(0.01, 1.0, (T, H, dk))
    b = r.uniform(0.0, 1.0, (T, H))
    h0 = r.standard_normal((N, H, dk, dv))
    return q, k, v, la, b, h0


def test_bwd_matches_central_finite_differences(oracle_mod):
    """Every gradient, element by element, against (L(x+e) - L(x-e)) / 2e of
    the forward oracle, with an empty sequence in the batch."""
    T, H, dk, dv = 9, 2, 3, 2
    cu = np.array([0, 5, 5, 9])
    N = 3
    x = list(_case(T, H, dk, dv, N, 11))
    r = rng0(12)
    Wo = r.standard_normal((T, H, dv))
    Wh = r.standard_normal((N, H, dk, dv))

    def loss(a):
        o, hT = oracle_mod.fwd(*a[:5], h0=a[5], cu_seqlens=cu)
        return float((o * Wo).sum() + (hT * Wh).sum())

    g = oracle_mod.bwd(*x[:5], Wo, h0=x[5], d_hT=Wh, cu_seqlens=cu)
    eps = 1e-6
    for ai in range(6):
        fd = np.zeros_like(x[ai])
        for idx in np.ndindex(x[ai].shape):
            a = [y.copy() for y in x]
            a[ai][idx] += eps
            lp = loss(a)
            a[ai][idx] -= 2 * eps
            fd[idx] = (lp - loss(a)) / (2 * eps)
        np.testing.assert_allclose(g[ai], fd, rtol=1e-6, atol=1e-7, err_msg="input %d" % ai)


def _torch_recurrence(q, k, v, la, b, h0, cu):
    """The forward written again with torch ops, vectorised over heads."""
    outs, hts = [], []
    for n in range(len(cu) - 1):
        S = h0[n]
        for t in range(int(cu[n]), int(cu[n + 1])):
            S = torch.exp(la[t]).unsqueeze(-1) * S
            r = torch.einsum("hc,hcj->hj", k[t], S)
            u = b[t].unsqueeze(-1) * (v[t] - r)
            S = S + k[t].unsqueeze(-1) * u.unsqueeze(-2)
            outs.append(torch.einsum("hc,hcj->hj", q[t], S))
        hts.append(S)
    return torch.stack(outs), torch.stack(hts)


@pytest.mark.parametrize("la_scale", [1.0, 4.0])
def test_bwd_matches_torch_autograd(oracle_mod, la_scale):
    T, H, dk, dv = 40, 2, 8, 6
    cu = np.array([0, 17, 40])
    N = 2
    x = _case(T, H, dk, dv, N, 21, la_scale)
    r = rng0(22)
    Wo = r.standard_normal((T, H, dv))
    Wh = r.standard_normal((N, H, dk, dv))
    tx = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in x]
    o, hT = _torch_recurrence(*tx, cu)
    ((o * torch.tensor(Wo)).sum() + (hT * torch.tensor(Wh)).sum()).backward()
    g = oracle_mod.bwd(*x[:5], Wo, h0=x[5], d_hT=Wh, cu_seqlens=cu)
    for ai in range(6):
        ref = tx[ai].grad.numpy()
        np.testing.assert_allclose(g[ai], ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max(),
                                   err_msg="input %d" % ai)


def test_bwd_frozen_state_closed_form(oracle_mod):
    """alpha = 1, beta = 0: S_t = h0 for all t and o_t = h0^T q_t.  With
    G_t = d_hT + sum_{s >= t} q_s do_s^T (the state gradient seen by token t):
    dq_t = h0 do_t, dk = dv = 0, dh0 = G_0, dlog_alpha_t[c] = sum_j G_t[c,j] h0[c,j],
    dbeta_t = (G_t^T k_t) . (v_t - h0^T k_t)."""
    T, H, dk, dv = 12, 2, 5, 4
    q, k, v, _, _, h0 = _case(T, H, dk, dv, 1, 31)
    la = np.zeros((T, H, dk))
    b = np.zeros((T, H))
    r = rng0(32)
    do = r.standard_normal((T, H, dv))
    dhT = r.standard_normal((1, H, dk, dv))
    dq, dk_, dv_, dla, db, dh0 = oracle_mod.bwd(q, k, v, la, b, do, h0=h0, d_hT=dhT)
    G = dhT[0].copy()
    for t in range(T - 1, -1, -1):
        G = G + np.einsum("hc,hj->hcj", q[t], do[t])
        np.testing.assert_allclose(dq[t], np.einsum("hcj,hj->hc", h0[0], do[t]), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dla[t], np.einsum("hcj,hcj->hc", G, h0[0]), rtol=1e-12, atol=1e-12)
        du = np.einsum("hcj,hc->hj", G, k[t])
        rr = np.einsum("hcj,hc->hj", h0[0], k[t])
        np.testing.assert_allclose(db[t], np.einsum("hj,hj->h", du, v[t] - rr), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dh0[0], G, rtol=1e-12, atol=1e-12)
    assert np.all(dk_ == 0.0) and np.all(dv_ == 0.0)


def test_bwd_linear_attention_closed_form(oracle_mod):
    """alpha = 1, beta = 1, orthonormal keys, h0 = 0 (section 2.1's linear
    attention): o_t = sum_{i <= t} (q_t . k_i) v_i, so
    dq_t = sum_{i <= t} k_i (v_i . do_t) and dv_i = sum_{t >= i} (q_t . k_i) do_t."""
    T, H, dk, dv = 8, 2, 8, 5
    r = rng0(41)
    k = np.zeros((T, H, dk))
    for h in range(H):
        Qm, _ = np.linalg.qr(r.standard_normal((dk, dk)))
        k[:, h, :] = Qm[:, :T].T
    q = r.standard_normal((T, H, dk))
    v = r.standard_normal((T, H, dv))
    do = r.standard_normal((T, H, dv))
    dq, _, dv_, _, _, _ = oracle_mod.bwd(q, k, v, np.zeros((T, H, dk)), np.ones((T, H)), do)
    qk = np.einsum("thc,ihc->hti", q, k)            # [H, t, i] = q_t . k_i
    mask = np.tril(np.ones((T, T)))
    ref_dq = np.einsum("ti,ihc,ihj,thj->thc", mask, k, v, do)
    ref_dv = np.einsum("hti,thj->ihj", qk * mask, do)
    np.testing.assert_allclose(dq, ref_dq, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv_, ref_dv, rtol=1e-10, atol=1e-12)


def test_bwd_zero_length_sequence_passes_state_gradient(oracle_mod):
    """A zero-length sequence has h_T = h0, so dh0 = d_hT."""
    H, dk, dv = 2, 4, 3
    x = _case(3, H, dk, dv, 2, 51)
    dhT = rng0(52).standard_normal((2, H, dk, dv))
    do = rng0(53).standard_normal((3, H, dv))
    g = oracle_mod.bwd(*x[:5], do, h0=x[5], d_hT=dhT, cu_seqlens=[0, 0, 3])
    np.testing.assert_array_equal(g[5][0], dhT[0])


@pytest.mark.parametrize("T,chunk", [(150, 64), (64, 64), (37, 16)])
def test_bwd_chunkwise_algebra_agrees(oracle_mod, T, chunk):
    """The gradient taken through the chunk form (tests/chunk_ref.py, the
    algebra the GPU backward evaluates) equals the oracle's token-by-token
    reverse mode, with ragged last chunks and decays in [0.5, 0.9999]."""
    import chunk_ref
    r = rng0(61)
    H, dk, dv = 2, 16, 12
    q = r.standard_normal((T, H, dk))
    k = r.standard_normal((T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((T, H, dv))
    la = np.log(r.uniform(0.5, 0.9999, (T, H, dk)))
    b = 1.0 / (1.0 + np.exp(-r.standard_normal((T, H))))
    h0 = 0.1 * r.standard_normal((H, dk, dv))
    do = r.standard_normal((T, H, dv))
    dhT = r.standard_normal((H, dk, dv))
    got = chunk_ref.chunk_bwd(q, k, v, la, b, do, h0=h0, d_hT=dhT, chunk=chunk)
    ref = oracle_mod.bwd(q, k, v, la, b, do, h0=h0[None], d_hT=dhT[None])
    for name, g, rr in zip(("dq", "dk", "dv", "dlog_alpha", "dbeta", "dh0"), got, ref):
        rr = rr.reshape(g.shape)
        assert np.abs(g - rr).max() <= 1e-11 * max(1.0, np.abs(rr).max()), name


def test_bwd_scalar_gate_is_channel_sum(oracle_mod):
    """Gated DeltaNet (section 2.2: one decay a_t per token and head) is KDA
    with every key channel's log_alpha equal to log a_t, so dL/dlog a_t is the
    sum over channels of the oracle's dlog_alpha.  Pinned by central finite
    differences of a separately written scalar-gate recurrence in log a_t; the
    other gradients against the same differences on beta."""
    T, H, dk, dv = 11, 2, 4, 3
    r = rng0(71)
    q = r.standard_normal((T, H, dk))
    k = r.standard_normal((T, H, dk)) / np.sqrt(dk)
    v = r.standard_normal((T, H, dv))
    g = np.log(r.uniform(0.4, 1.0, (T, H)))
    b = r.uniform(0.0, 1.0, (T, H))
    h0 = r.standard_normal((H, dk, dv))
    Wo = r.standard_normal((T, H, dv))
    Wh = r.standard_normal((H, dk, dv))

    def loss(gg, bb):
        o = np.zeros((T, H, dv))
        S = h0.copy()
        for t in range(T):
            for h in range(H):
                kk = k[t, h]
                S[h] = np.exp(gg[t, h]) * S[h]
                S[h] = S[h] + bb[t, h] * np.outer(kk, v[t, h] - kk @ S[h])
                o[t, h] = S[h].T @ q[t, h]
        return float((o * Wo).sum() + (S * Wh).sum())

    la = np.repeat(g[:, :, None], dk, axis=2)
    res = oracle_mod.bwd(q, k, v, la, b, Wo, h0=h0[None], d_hT=Wh[None])
    eps = 1e-6
    for x, got in ((g, res[3].sum(-1)), (b, res[4])):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            fd[idx] = ((loss(xp, b) - loss(xm, b)) if x is g else (loss(g, xp) - loss(g, xm))) / (2 * eps)
        np.testing.assert_allclose(got, fd, rtol=1e-6, atol=1e-7)


def test_gen_bwd_matches_central_finite_differences(oracle_mod):
    """Separate erase and write strengths: every element of all seven
    gradients of the generalised recurrence against central differences of
    oracle.gen_fwd, with an empty sequence in the batch."""
    T, H, dk, dv = 8, 2, 3, 2
    cu = np.array([0, 5, 5, 8])
    N = 3
    q, k, v, la, b, h0 = _case(T, H, dk, dv, N, 81)
    w = rng0(82).uniform(-0.5, 1.5, (T, H))
    x = [q, k, v, la, b, w, h0]
    r = rng0(83)
    Wo = r.standard_normal((T, H, dv))
    Wh = r.standard_normal((N, H, dk, dv))

    def loss(a):
        o, hT = oracle_mod.gen_fwd(*a[:6], h0=a[6], cu_seqlens=cu)
        return float((o * Wo).sum() + (hT * Wh).sum())

    g = oracle_mod.gen_bwd(*x[:6], Wo, h0=x[6], d_hT=Wh, cu_seqlens=cu)
    order = (0, 1, 2, 3, 4, 5, 6)     # gen_bwd returns dq, dk, dv, dla, db, dw, dh0
    eps = 1e-6
    for ai, gi in zip(range(7), order):
        fd = np.zeros_like(x[ai])
        for idx in np.ndindex(x[ai].shape):
            a = [y.copy() for y in x]
            a[ai][idx] += eps
            lp = loss(a)
            a[ai][idx] -= 2 * eps
            fd[idx] = (lp - loss(a)) / (2 * eps)
        np.testing.assert_allclose(g[gi], fd, rtol=1e-6, atol=1e-7, err_msg="input %d" % ai)


def test_gen_bwd_tied_strengths_is_kda_bwd(oracle_mod):
    """w = b = beta is KDA: the generalised gradient equals oracle.bwd, with
    db + dw = dbeta."""
    T, H, dk, dv = 30, 2, 6, 5
    cu = np.array([0, 13, 30])
    x = _case(T, H, dk, dv, 2, 91)
    do = rng0(92).standard_normal((T, H, dv))
    dhT = rng0(93).standard_normal((2, H, dk, dv))
    a = oracle_mod.bwd(*x[:5], do, h0=x[5], d_hT=dhT, cu_seqlens=cu)
    g = oracle_mod.gen_bwd(*x[:5], x[4], do, h0=x[5], d_hT=dhT, cu_seqlens=cu)
    for name, u, ref in (("dq", g[0], a[0]), ("dk", g[1], a[1]), ("dv", g[2], a[2]), ("dla", g[3], a[3]),
                         ("dbeta", g[4] + g[5], a[4]), ("dh0", g[6], a[5])):
        np.testing.assert_allclose(u, ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max(), err_msg=name)


def test_gen_bwd_write_only_linear_attention(oracle_mod):
    """b = 0, w = 1, alpha = 1, h0 = 0: S_t = sum_{i<=t} k_i v_i^T for ANY keys
    (section 2.1's linear attention), o_t = sum_{i<=t} (q_t . k_i) v_i.  So
    dq_t = sum_{i<=t} k_i (v_i . do_t), dk_i = sum_{t>=i} q_t (v_i . do_t),
    dv_i = sum_{t>=i} (q_t . k_i) do_t, dw_i = v_i . dv_i, and
    db_i = -(sum_{t>=i} (q_t . k_i) do_t) . (sum_{m<i} (k_m . k_i) v_m)."""
    T, H, dk, dv = 9, 2, 4, 3
    r = rng0(101)
    q = r.standard_normal((T, H, dk))
    k = r.standard_normal((T, H, dk))
    v = r.standard_normal((T, H, dv))
    do = r.standard_normal((T, H, dv))
    la = np.zeros((T, H, dk))
    g = oracle_mod.gen_bwd(q, k, v, la, np.zeros((T, H)), np.ones((T, H)), do)
    qk = np.einsum("thc,ihc->hti", q, k)                 # [H, t, i] = q_t . k_i
    kk = np.einsum("mhc,ihc->hmi", k, k)                 # [H, m, i] = k_m . k_i
    vd = np.einsum("ihj,thj->hit", v, do)                # [H, i, t] = v_i . do_t
    low = np.tril(np.ones((T, T)))                       # [t, i]: i <= t
    ref_dq = np.einsum("ti,hit,ihc->thc", low, vd, k)
    ref_dk = np.einsum("ti,hit,thc->ihc", low, vd, q)
    ref_dv = np.einsum("ti,hti,thj->ihj", low, qk, do)
    ref_dw = np.einsum("ihj,ihj->ih", v, ref_dv)
    strict = np.tril(np.ones((T, T)), -1)                # [i, m]: m < i
    rvec = np.einsum("im,hmi,mhj->ihj", strict, kk, v)   # sum_{m<i} (k_m . k_i) v_m
    ref_db = -np.einsum("ihj,ihj->ih", ref_dv, rvec)
    for name, u, ref in (("dq", g[0], ref_dq), ("dk", g[1], ref_dk), ("dv", g[2], ref_dv),
                         ("dw", g[5], ref_dw), ("db", g[4], ref_db)):
        np.testing.assert_allclose(u, ref, rtol=1e-10, atol=1e-12, err_msg=name)


def test_bwd_prologue_matches_central_finite_differences(oracle_mod):
    """The forward on raw projections (oracle.fwd_prologue): every gradient of
    oracle.bwd_prologue against central differences, with rows whose norm is
    below eps (the eps branch), gates where the floor binds and where it does
    not, and an empty sequence.  eps = 0.5 and the floor at -2 keep every
    difference away from a branch point."""
    T, H, dk, dv = 8, 2, 3, 2
    cu = np.array([0, 5, 5, 8])
    N = 3
    r = rng0(111)
    q = r.standard_normal((T, H, dk))
    k = r.standard_normal((T, H, dk))
    q[2, 0] *= 0.05 / np.linalg.norm(q[2, 0])       # below eps
    k[6, 1] *= 0.1 / np.linalg.norm(k[6, 1])
    v = r.standard_normal((T, H, dv))
    a = r.uniform(-3.0, 1.0, (T, H, dk))
    a[1, 0, 0], a[4, 1, 2] = 4.0, 6.0                # -softplus below the floor -2
    b = r.standard_normal((T, H))
    h0 = r.standard_normal((N, H, dk, dv))
    lo, eps = -2.0, 0.5
    Wo = r.standard_normal((T, H, dv))
    Wh = r.standard_normal((N, H, dk, dv))
    x = [q, k, v, a, b, h0]

    def loss(z):
        o, hT = oracle_mod.fwd_prologue(z[0], z[1], z[2], z[3], z[4], lo, h0=z[5], cu_seqlens=cu, eps=eps)
        return float((o * Wo).sum() + (hT * Wh).sum())

    g = oracle_mod.bwd_prologue(q, k, v, a, b, lo, Wo, h0=h0, d_hT=Wh, cu_seqlens=cu, eps=eps)
    assert np.all(g[3][1, 0, 0] == 0.0) and np.all(g[3][4, 1, 2] == 0.0)
    step = 1e-6
    for ai in range(6):
        fd = np.zeros_like(x[ai])
        for idx in np.ndindex(x[ai].shape):
            z = [y.copy() for y in x]
            z[ai][idx] += step
            lp = loss(z)
            z[ai][idx] -= 2 * step
            fd[idx] = (lp - loss(z)) / (2 * step)
        np.testing.assert_allclose(g[ai], fd, rtol=1e-6, atol=1e-7, err_msg="input %d" % ai)
