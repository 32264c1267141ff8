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
