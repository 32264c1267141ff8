"""Staged fp64 chunkwise reference (numpy) -- a test aid, not the oracle.

It evaluates the chunkwise form of the KDA recurrence: within a chunk of n
tokens with start state S0 (d_k x d_v) and inclusive per-channel log-decay
cumsum G (rows g_r),

    A[r, i] = beta_r * sum_c K[r,c] K[i,c] exp(G[r,c] - G[i,c])     (i < r)
    P[r, i] = sum_c Q[r,c] K[i,c] exp(G[r,c] - G[i,c])               (i <= r)
    (I + A) U = diag(beta) (V - (K * exp(G)) S0)
    O = (Q * exp(G)) S0 + P U
    S_n = Diag(exp(g_n)) S0 + (K * exp(g_n - G))^T U

which follows from unrolling the per-token update within the chunk (the
chunkwise strategy of section 3.1 of the KimiLinear article: an intra-chunk part
by matrix products and an inter-chunk part carried by the state).  Exponents are
formed as differences, so nothing overflows.  Because it is a different
algorithm from the token-by-token oracle that reaches the same result in exact
arithmetic, agreement at ~1e-12 pins both; it also exposes the per-chunk
intermediates to localise a GPU discrepancy to one stage.
"""
from __future__ import annotations

import numpy as np


def chunk_fwd(q, k, v, log_alpha, beta, h0=None, chunk=64, return_stages=False):
    """One sequence: q, k, log_alpha [T, H, dk]; v [T, H, dv]; beta [T, H];
    h0 [H, dk, dv] or None.  Returns (o [T, H, dv], hT [H, dk, dv])."""
    q, k, v, la, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, log_alpha, beta))
    T, H, dk = q.shape
    dv = v.shape[2]
    o = np.zeros((T, H, dv))
    hT = np.zeros((H, dk, dv))
    stages = []
    for h in range(H):
        S = np.zeros((dk, dv)) if h0 is None else np.array(h0[h], dtype=np.float64)
        for s in range(0, T, chunk):
            e = min(s + chunk, T)
            n = e - s
            Q, K, V, L, b = q[s:e, h], k[s:e, h], v[s:e, h], la[s:e, h], beta[s:e, h]
            G = np.cumsum(L, axis=0)                       # [n, dk], inclusive
            D = G[:, None, :] - G[None, :, :]              # [r, i, c] = G_r - G_i
            mask_lo = np.tril(np.ones((n, n)), -1)[:, :, None]
            mask_le = np.tril(np.ones((n, n)), 0)[:, :, None]
            Wd = np.exp(np.where(mask_le > 0, D, -np.inf))  # exp(G_r - G_i) for i <= r
            A = b[:, None] * np.einsum("rc,ic,ric->ri", K, K, Wd * mask_lo)
            P = np.einsum("rc,ic,ric->ri", Q, K, Wd * mask_le)
            E = np.exp(G)
            rhs = b[:, None] * (V - (K * E) @ S)
            U = np.linalg.solve(np.eye(n) + A, rhs)
            O = (Q * E) @ S + P @ U
            gn = G[-1]
            S_new = np.exp(gn)[:, None] * S + (K * np.exp(gn[None, :] - G)).T @ U
            if return_stages:
                stages.append(dict(h=h, start=s, G=G, A=A, P=P, U=U, O=O, S0=S, S1=S_new))
            o[s:e, h] = O
            S = S_new
        hT[h] = S
    if return_stages:
        return o, hT, stages
    return o, hT


def chunk_bwd(q, k, v, log_alpha, beta, d_o, h0=None, d_hT=None, chunk=64):
    """Gradients through the chunkwise form above, one sequence, per head.

    The chunk form is differentiated stage by stage with the anchored operands
    QA = Q e^{G-m}, KA = K e^{G-m}, KI = K e^{m-G} (m = g_n / 2, held fixed: it
    cancels from every result), T = (I + A)^{-1}, W = T diag(beta) KA and
    S' = Diag(e^m) S:
        forward passes store S and U per chunk; a reverse pass carries
        dS <- Diag(e^m)(QA^T dO - W^T dU) + Diag(e^{g_n}) dS with
        dU = P^T dO + KI Diag(e^{g_n - m}) dS;
        then per chunk dY = T^T dU, dP = lower(dO U^T), dA = -strict(dY U^T),
        dQA = dO S'^T + dP KI, dKA = -diag(beta) dY S'^T + diag(beta) dA KI,
        dKI = dP^T QA + (diag(beta) dA)^T KA + (U dS^T) Diag(e^{g_n - m}),
        dbeta = rowsum(dY X) + rowsum(dA M), dV = diag(beta) dY,
        dlog_alpha = reverse cumsum of dQA.QA + dKA.KA - dKI.KI plus dg_n.
    A different algorithm from the oracle's token-by-token reverse mode, so
    agreement pins both.  Inputs as chunk_fwd plus d_o [T, H, dv] and d_hT
    [H, dk, dv]; returns (dq, dk, dv, dlog_alpha, dbeta, dh0)."""
    q, k, v, la, beta, d_o = (np.asarray(x, dtype=np.float64) for x in (q, k, v, log_alpha, beta, d_o))
    T, H, dk = q.shape
    dv = v.shape[2]
    C = chunk
    out = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros_like(la), np.zeros_like(beta),
           np.zeros((H, dk, dv))]
    for h in range(H):
        recs, Ss, Us = [], [], []
        S = np.zeros((dk, dv)) if h0 is None else np.array(h0[h], dtype=np.float64)
        for t0 in range(0, T, C):
            n = min(C, T - t0)
            sl = slice(t0, t0 + n)
            G = np.cumsum(la[sl, h], axis=0)
            gn = G[-1]
            m = gn / 2
            QA, KA, KI = q[sl, h] * np.exp(G - m), k[sl, h] * np.exp(G - m), k[sl, h] * np.exp(m - G)
            b = beta[sl, h]
            M = np.tril(KA @ KI.T, -1)
            P = np.tril(QA @ KI.T)
            Tm = np.linalg.inv(np.eye(n) + b[:, None] * M)
            W = Tm @ (b[:, None] * KA)
            Sp = np.exp(m)[:, None] * S
            X = v[sl, h] - KA @ Sp
            U = Tm @ (b[:, None] * X)
            recs.append((sl, G, m, gn, QA, KA, KI, b, M, P, Tm, W, X))
            Ss.append(S)
            Us.append(U)
            S = np.exp(gn)[:, None] * S + (np.exp(gn - m)[None, :] * KI).T @ U
        dS = np.zeros((dk, dv)) if d_hT is None else np.array(d_hT[h], dtype=np.float64)
        for ci in range(len(recs) - 1, -1, -1):
            sl, G, m, gn, QA, KA, KI, b, M, P, Tm, W, X = recs[ci]
            S0, U = Ss[ci], Us[ci]
            Sp = np.exp(m)[:, None] * S0
            dO = d_o[sl, h]
            dU = P.T @ dO + KI @ (np.exp(gn - m)[:, None] * dS)
            dY = Tm.T @ dU
            dP = np.tril(dO @ U.T)
            dA = -np.tril(dY @ U.T, -1)
            dM = b[:, None] * dA
            dQA = dO @ Sp.T + dP @ KI
            dKA = -b[:, None] * (dY @ Sp.T) + dM @ KI
            dKB = U @ dS.T
            dKI = dP.T @ QA + dM.T @ KA + np.exp(gn - m)[None, :] * dKB
            ea, ei = np.exp(G - m), np.exp(m - G)
            dG = dQA * QA + dKA * KA - dKI * KI
            dgn = np.exp(gn - m) * ((dS * Sp).sum(axis=1) + (dKB * KI).sum(axis=0))
            out[0][sl, h] = dQA * ea
            out[1][sl, h] = dKA * ea + dKI * ei
            out[2][sl, h] = b[:, None] * dY
            out[3][sl, h] = np.cumsum(dG[::-1], axis=0)[::-1] + dgn
            out[4][sl, h] = (dY * X).sum(axis=1) + (dA * M).sum(axis=1)
            dS = np.exp(m)[:, None] * (QA.T @ dO - W.T @ dU) + np.exp(gn)[:, None] * dS
        out[5][h] = dS
    return tuple(out)
