"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Every check here is independent of the oracle's own code path: closed forms of
the special cases that the pages' equations reduce to (KimiLinear article,
sections 2.1-2.3), hand-worked examples (tests/golden), a brute-force product of
explicit transition matrices, a different (chunkwise) algorithm, and invariants.
Each is chosen so that a plausible slip in the oracle fails at least one: a
dropped term, a wrong sign, decay applied after the update instead of before,
gating columns instead of rows, an S q read-out instead of S^T q, or an
exclusive read-out.
"""
import json
import os

import numpy as np
import pytest

import chunk_ref

HERE = os.path.dirname(os.path.abspath(__file__))
rng0 = np.random.default_rng


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rand_case(T, H, dk, dv, seed, gate_scale=1.0, beta=None):
    r = rng0(seed)
    q = _unit(r.standard_normal((T, H, dk)))
    k = _unit(r.standard_normal((T, H, dk)))
    v = r.standard_normal((T, H, dv))
    la = -gate_scale * np.log1p(np.exp(r.standard_normal((T, H, dk))))
    b = 1.0 / (1.0 + np.exp(-r.standard_normal((T, H)))) if beta is None else beta
    return q, k, v, la, b


def _orthonormal_keys(T, H, dk, seed):
    r = rng0(seed)
    out = np.zeros((T, H, dk))
    for h in range(H):
        Qm, _ = np.linalg.qr(r.standard_normal((dk, dk)))
        out[:, h] = Qm[:, :T].T
    return out


# ---------------------------------------------------------------- worked examples
def test_golden_worked_examples(oracle_mod):
    with open(os.path.join(HERE, "golden", "worked_examples.json")) as f:
        gold = json.load(f)
    for ex in gold["examples"]:
        T = len(ex["k"])
        k = np.array(ex["k"])[:, None, :]
        q = np.array(ex["q"])[:, None, :]
        v = np.array(ex["v"])[:, None, :]
        la = np.log(np.array(ex["alpha"]))[:, None, :]
        b = np.array(ex["beta"])[:, None]
        h0 = np.array(ex["h0"])[None, None]
        o, hT = oracle_mod.fwd(q, k, v, la, b, h0=h0)
        np.testing.assert_allclose(o[:, 0], np.array(ex["o"]), rtol=0, atol=1e-14, err_msg=ex["name"])
        np.testing.assert_allclose(hT[0, 0], np.array(ex["hT"]), rtol=0, atol=1e-14,
                                   err_msg=ex["name"])
        assert T == o.shape[0]


# ---------------------------------------------------------------- P1: frozen state
def test_p1_beta_zero_alpha_one_freezes_state(oracle_mod):
    """alpha = 1, beta = 0: the update of section 2.3 is the identity, so
    S_t = h0 and o_t = h0^T q_t (non-square state to pin the orientation)."""
    T, H, dk, dv = 17, 2, 6, 5
    q, k, v, _, _ = _rand_case(T, H, dk, dv, 1)
    h0 = rng0(2).standard_normal((1, H, dk, dv))
    o, hT = oracle_mod.fwd(q, k, v, np.zeros((T, H, dk)), np.zeros((T, H)), h0=h0)
    np.testing.assert_array_equal(hT, h0)
    np.testing.assert_allclose(o, np.einsum("hcj,thc->thj", h0[0], q), rtol=0, atol=1e-14)


# ---------------------------------------------------------------- P2: linear attention
def test_p2a_orthonormal_keys_beta_one_is_linear_attention(oracle_mod):
    """Section 2.1: with alpha = 1, beta = 1 and orthonormal keys the erase term
    vanishes (k_t^T S_{t-1} = 0), leaving pure linear attention
    S_t = sum_{i<=t} k_i v_i^T and o_t = sum_{i<=t} (q_t . k_i) v_i (inclusive)."""
    T, H, dk, dv = 12, 3, 16, 7
    k = _orthonormal_keys(T, H, dk, 3)
    r = rng0(4)
    q = r.standard_normal((T, H, dk))
    v = r.standard_normal((T, H, dv))
    o, hT = oracle_mod.fwd(q, k, v, np.zeros((T, H, dk)), np.ones((T, H)))
    scores = np.einsum("thc,ihc->hti", q, k) * np.tril(np.ones((T, T)))[None]
    ref_o = np.einsum("hti,ihj->thj", scores, v)
    np.testing.assert_allclose(o, ref_o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(hT[0], np.einsum("thc,thj->hcj", k, v), rtol=0, atol=1e-13)


def test_p2b_orthonormal_keys_general_beta(oracle_mod):
    """Section 2.1 with general beta and orthonormal keys: S_t = sum beta_i k_i v_i^T."""
    T, H, dk, dv = 10, 2, 12, 9
    k = _orthonormal_keys(T, H, dk, 5)
    r = rng0(6)
    q = r.standard_normal((T, H, dk))
    v = r.standard_normal((T, H, dv))
    b = r.uniform(0.05, 1.9, (T, H))
    o, hT = oracle_mod.fwd(q, k, v, np.zeros((T, H, dk)), b)
    scores = np.einsum("thc,ihc->hti", q, k) * np.tril(np.ones((T, T)))[None]
    ref_o = np.einsum("hti,ihj->thj", scores * b.T[:, None, :], v)
    np.testing.assert_allclose(o, ref_o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(hT[0], np.einsum("th,thc,thj->hcj", b, k, v), rtol=0, atol=1e-13)


def test_p2c_decoupled_write_only_is_linear_attention_any_keys(oracle_mod):
    """Generalised form (separate erase b and write w): b = 0, w = 1, alpha = 1
    is exactly the linear-attention accumulation of section 2.1 for any keys."""
    T, H, dk, dv = 9, 2, 5, 4
    q, k, v, _, _ = _rand_case(T, H, dk, dv, 7)
    k = k * rng0(8).uniform(0.5, 2.0, (T, H, 1))   # not unit, not orthogonal
    o, hT = oracle_mod.gen_fwd(q, k, v, np.zeros((T, H, dk)), np.zeros((T, H)), np.ones((T, H)))
    S = np.cumsum(np.einsum("thc,thj->thcj", k, v), axis=0)
    np.testing.assert_allclose(o, np.einsum("thcj,thc->thj", S, q), rtol=0, atol=1e-13)
    np.testing.assert_allclose(hT[0], S[-1], rtol=0, atol=1e-13)


def test_kda_is_generalised_form_with_tied_strengths(oracle_mod):
    T, H, dk, dv = 20, 2, 8, 6
    q, k, v, la, b = _rand_case(T, H, dk, dv, 9)
    o1, h1 = oracle_mod.fwd(q, k, v, la, b)
    o2, h2 = oracle_mod.gen_fwd(q, k, v, la, b, b)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(h1, h2)


# ---------------------------------------------------------------- P3: Gated DeltaNet
def _gdn_scalar_gate(q, k, v, a, b, h0):
    """Section 2.2 written out independently: S_t = a_t (I - b_t k k^T) S_{t-1} + b_t k v^T."""
    T, H, dk = q.shape
    dv = v.shape[2]
    o = np.zeros((T, H, dv))
    S = np.array(h0, dtype=np.float64)
    for h in range(H):
        for t in range(T):
            kk = k[t, h]
            M = a[t, h] * (np.eye(dk) - b[t, h] * np.outer(kk, kk))
            S[h] = M @ S[h] + b[t, h] * np.outer(kk, v[t, h])
            o[t, h] = S[h].T @ q[t, h]
    return o, S


def test_p3_channel_constant_gate_is_gated_deltanet(oracle_mod):
    T, H, dk, dv = 30, 2, 7, 5
    q, k, v, _, b = _rand_case(T, H, dk, dv, 10)
    a = rng0(11).uniform(0.3, 1.0, (T, H))
    h0 = rng0(12).standard_normal((H, dk, dv))
    la = np.repeat(np.log(a)[:, :, None], dk, axis=2)
    o, hT = oracle_mod.fwd(q, k, v, la, b, h0=h0[None])
    ro, rS = _gdn_scalar_gate(q, k, v, a, b, h0)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-13)
    np.testing.assert_allclose(hT[0], rS, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- P4: overwrite
def test_p4_beta_one_unit_key_overwrites(oracle_mod):
    """Section 2.1 (beta -> 1 overwrites): with beta = 1 and |k_t| = 1,
    k_t^T S_t = v_t^T exactly, for any gate and start state.  Fails if the decay
    were applied after the delta-rule correction."""
    T, H, dk, dv = 25, 2, 8, 6
    q, k, v, la, _ = _rand_case(T, H, dk, dv, 13)
    h0 = rng0(14).standard_normal((1, H, dk, dv))
    for t_end in (1, 7, T):
        _, hT = oracle_mod.fwd(q[:t_end], k[:t_end], v[:t_end], la[:t_end], np.ones((t_end, H)),
                               h0=h0)
        np.testing.assert_allclose(np.einsum("hc,hcj->hj", k[t_end - 1], hT[0]), v[t_end - 1],
                                   rtol=0, atol=1e-13)


def test_p4b_orthonormal_overwrite_leaves_other_keys(oracle_mod):
    """alpha = 1, beta = 1, orthonormal keys: writing v_t under k_t leaves what is
    stored under every other (orthogonal) key untouched."""
    T, H, dk, dv = 6, 1, 8, 3
    k = _orthonormal_keys(T, H, dk, 15)
    r = rng0(16)
    v = r.standard_normal((T, H, dv))
    h0 = r.standard_normal((1, H, dk, dv))
    q = r.standard_normal((T, H, dk))
    _, hT = oracle_mod.fwd(q, k, v, np.zeros((T, H, dk)), np.ones((T, H)), h0=h0)
    basis, _ = np.linalg.qr(np.concatenate([k[:, 0].T, r.standard_normal((dk, dk - T))], axis=1))
    others = basis[:, T:]
    np.testing.assert_allclose(others.T @ hT[0, 0], others.T @ h0[0, 0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(k[:, 0] @ hT[0, 0], v[:, 0], rtol=0, atol=1e-13)


# ---------------------------------------------------------------- P5: basis keys
def test_p5_basis_keys_per_row_gated_ema(oracle_mod):
    """k_t = e_{c_t}: row c_t becomes (1 - beta_t) a_t[c_t] S[c_t] + beta_t v_t and
    every other row c is scaled by its own gate a_t[c] (gate on rows, section 2.3)."""
    T, H, dk, dv = 40, 2, 6, 4
    r = rng0(17)
    cidx = r.integers(0, dk, (T, H))
    k = np.zeros((T, H, dk))
    for t in range(T):
        for h in range(H):
            k[t, h, cidx[t, h]] = 1.0
    q = r.standard_normal((T, H, dk))
    v = r.standard_normal((T, H, dv))
    a = r.uniform(0.2, 1.0, (T, H, dk))
    b = r.uniform(0.0, 1.0, (T, H))
    h0 = r.standard_normal((H, dk, dv))
    o, hT = oracle_mod.fwd(q, k, v, np.log(a), b, h0=h0[None])
    S = h0.copy()
    for t in range(T):
        for h in range(H):
            S[h] *= a[t, h][:, None]
            c = cidx[t, h]
            S[h, c] = (1.0 - b[t, h]) * S[h, c] + b[t, h] * v[t, h]
            np.testing.assert_allclose(o[t, h], q[t, h] @ S[h], rtol=0, atol=1e-12)
    np.testing.assert_allclose(hT[0], S, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- P7: brute force
def test_p7_brute_force_transition_products(oracle_mod):
    """Explicit d_k x d_k transitions M_t = (I - b k k^T) Diag(a_t): the unrolled
    S_t = M_t..M_1 h0 + sum_j M_t..M_{j+1} b_j k_j v_j^T for T <= 8."""
    for seed, (T, dk, dv) in enumerate([(8, 6, 5), (5, 3, 7), (1, 4, 4), (8, 1, 1)]):
        q, k, v, la, b = _rand_case(T, 1, dk, dv, 100 + seed)
        k = k * rng0(200 + seed).uniform(0.5, 1.5, (T, 1, 1))
        h0 = rng0(300 + seed).standard_normal((1, 1, dk, dv))
        o, hT = oracle_mod.fwd(q, k, v, la, b, h0=h0)
        Ms = [(np.eye(dk) - b[t, 0] * np.outer(k[t, 0], k[t, 0])) @ np.diag(np.exp(la[t, 0]))
              for t in range(T)]
        for t in range(T):
            prod = np.eye(dk)
            for m in Ms[: t + 1]:
                prod = m @ prod
            St = prod @ h0[0, 0]
            for j in range(t + 1):
                tail = np.eye(dk)
                for m in Ms[j + 1: t + 1]:
                    tail = m @ tail
                St = St + tail @ (b[j, 0] * np.outer(k[j, 0], v[j, 0]))
            np.testing.assert_allclose(o[t, 0], St.T @ q[t, 0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(hT[0, 0], St, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- P8: reset
def test_p8_strong_decay_resets(oracle_mod):
    """A gate of exp(-30) on every channel at token t0 wipes the state (the forget
    gate of section 2.2 forgetting rapidly): outputs from t0 on match a fresh run
    from zero state started at t0, to within exp(-30) times the state size."""
    T, H, dk, dv, t0 = 50, 2, 8, 8, 21
    q, k, v, la, b = _rand_case(T, H, dk, dv, 18)
    la[t0] = -30.0
    h0 = rng0(19).standard_normal((1, H, dk, dv))
    o, hT = oracle_mod.fwd(q, k, v, la, b, h0=h0)
    la_fresh = la[t0:].copy()
    la_fresh[0] = 0.0
    o2, hT2 = oracle_mod.fwd(q[t0:], k[t0:], v[t0:], la_fresh, b[t0:])
    np.testing.assert_allclose(o[t0:], o2, rtol=0, atol=1e-11)
    np.testing.assert_allclose(hT, hT2, rtol=0, atol=1e-11)


# ---------------------------------------------------------------- chunkwise algebra
@pytest.mark.parametrize("T,dk,dv,chunk,with_h0", [(200, 16, 12, 64, True), (256, 8, 8, 64, False),
                                                  (130, 16, 16, 32, True), (3, 4, 5, 64, True)])
def test_chunkwise_algebra_agrees_with_recurrence(oracle_mod, T, dk, dv, chunk, with_h0):
    """The chunkwise form (section 3.1: intra-chunk by matrix products, inter-chunk
    by the carried state) is a different algorithm that must reach the oracle's
    result; a partial last chunk is included."""
    H = 2
    q, k, v, la, b = _rand_case(T, H, dk, dv, 20 + T)
    h0 = rng0(21).standard_normal((H, dk, dv)) * 0.1 if with_h0 else None
    o, hT = oracle_mod.fwd(q, k, v, la, b, h0=None if h0 is None else h0[None])
    ro, rh = chunk_ref.chunk_fwd(q, k, v, la, b, h0=h0, chunk=chunk)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(hT[0], rh, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- invariants
def test_i1_split_chaining(oracle_mod):
    T, H, dk, dv = 70, 2, 8, 6
    q, k, v, la, b = _rand_case(T, H, dk, dv, 22)
    h0 = rng0(23).standard_normal((1, H, dk, dv))
    o, hT = oracle_mod.fwd(q, k, v, la, b, h0=h0)
    s = 33
    o1, h1 = oracle_mod.fwd(q[:s], k[:s], v[:s], la[:s], b[:s], h0=h0)
    o2, h2 = oracle_mod.fwd(q[s:], k[s:], v[s:], la[s:], b[s:], h0=h1)
    np.testing.assert_allclose(np.concatenate([o1, o2]), o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(h2, hT, rtol=0, atol=1e-13)


def test_i2_varlen_equals_separate_calls(oracle_mod):
    lens = [5, 0, 17, 1, 9]
    T, H, dk, dv = sum(lens), 2, 6, 4
    q, k, v, la, b = _rand_case(T, H, dk, dv, 24)
    h0 = rng0(25).standard_normal((len(lens), H, dk, dv))
    cu = np.concatenate([[0], np.cumsum(lens)])
    o, hT = oracle_mod.fwd(q, k, v, la, b, h0=h0, cu_seqlens=cu)
    for n in range(len(lens)):
        s, e = cu[n], cu[n + 1]
        on, hn = oracle_mod.fwd(q[s:e], k[s:e], v[s:e], la[s:e], b[s:e], h0=h0[n:n + 1])
        np.testing.assert_array_equal(o[s:e], on)
        np.testing.assert_array_equal(hT[n], hn[0])
    np.testing.assert_array_equal(hT[1], h0[1])   # empty sequence: h_T = h0


def test_i3_decode_steps_equal_forward(oracle_mod):
    B, H, dk, dv, T = 3, 2, 6, 5, 8
    r = rng0(26)
    S = r.standard_normal((B, H, dk, dv))
    S0 = S.copy()
    os_ = []
    cases = [_rand_case(B, H, dk, dv, 27 + t) for t in range(T)]
    for (q, k, v, la, b) in cases:
        o, S = oracle_mod.decode(q, k, v, la, b, S)
        os_.append(o)
    for bi in range(B):
        qs = np.stack([c[0][bi] for c in cases])
        ks = np.stack([c[1][bi] for c in cases])
        vs = np.stack([c[2][bi] for c in cases])
        las = np.stack([c[3][bi] for c in cases])
        bs = np.stack([c[4][bi] for c in cases])
        of, hf = oracle_mod.fwd(qs, ks, vs, las, bs, h0=S0[bi:bi + 1])
        np.testing.assert_allclose(np.stack([x[bi] for x in os_]), of, rtol=0, atol=1e-13)
        np.testing.assert_allclose(S[bi], hf[0], rtol=0, atol=1e-13)


def test_i4_value_column_permutation(oracle_mod):
    T, H, dk, dv = 40, 2, 6, 7
    q, k, v, la, b = _rand_case(T, H, dk, dv, 28)
    h0 = rng0(29).standard_normal((1, H, dk, dv))
    perm = rng0(30).permutation(dv)
    o, hT = oracle_mod.fwd(q, k, v, la, b, h0=h0)
    o2, h2 = oracle_mod.fwd(q, k, v[:, :, perm], la, b, h0=h0[..., perm])
    np.testing.assert_allclose(o2, o[:, :, perm], rtol=0, atol=1e-14)
    np.testing.assert_allclose(h2, hT[..., perm], rtol=0, atol=1e-14)


def test_i5_homogeneity_and_linearity(oracle_mod):
    T, H, dk, dv = 40, 2, 6, 5
    q, k, v, la, b = _rand_case(T, H, dk, dv, 31)
    r = rng0(32)
    h0a, h0b = r.standard_normal((2, 1, H, dk, dv))
    va, vb = v, r.standard_normal(v.shape)
    oa, ha = oracle_mod.fwd(q, k, va, la, b, h0=h0a)
    ob, hb = oracle_mod.fwd(q, k, vb, la, b, h0=h0b)
    c1, c2 = 0.7, -1.3
    oc, hc = oracle_mod.fwd(q, k, c1 * va + c2 * vb, la, b, h0=c1 * h0a + c2 * h0b)
    np.testing.assert_allclose(oc, c1 * oa + c2 * ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(hc, c1 * ha + c2 * hb, rtol=0, atol=1e-12)
    o3, _ = oracle_mod.fwd(2.5 * q, k, va, la, b, h0=h0a)
    np.testing.assert_allclose(o3, 2.5 * oa, rtol=0, atol=1e-12)


def test_i7_thread_count_does_not_change_result(oracle_mod):
    T, H, dk, dv = 64, 5, 8, 8
    q, k, v, la, b = _rand_case(T, H, dk, dv, 33)
    o1, h1 = oracle_mod.fwd(q, k, v, la, b, nthreads=1)
    o4, h4 = oracle_mod.fwd(q, k, v, la, b, nthreads=4)
    np.testing.assert_array_equal(o1, o4)
    np.testing.assert_array_equal(h1, h4)


def test_bad_arguments_raise(oracle_mod):
    q, k, v, la, b = _rand_case(4, 1, 3, 3, 34)
    with pytest.raises(ValueError):
        oracle_mod.fwd(q, k, v, la, b, cu_seqlens=[0, 3])      # does not end at T
    with pytest.raises(ValueError):
        oracle_mod.fwd(q, k, v, la, b, cu_seqlens=[0, 3, 2, 4])  # decreasing


# ---------------------------------------------------------------- input prologue
# KimiLinear article, section 3.2: inputs normalised, gate values constrained and
# reparameterised (reading: L2 norm, max(-softplus, floor), sigmoid).  Each map is
# pinned by closed forms, library routines and invariances, and the composition
# by a hand-worked example.
def test_prologue_golden_example(oracle_mod):
    with open(os.path.join(HERE, "golden", "prologue_examples.json")) as f:
        gold = json.load(f)
    for ex in gold["examples"]:
        T, dk = len(ex["q_raw"]), ex["dk"]
        sh = lambda a: np.asarray(a, dtype=np.float64).reshape(T, 1, -1)
        qh, kh, la, be = oracle_mod.prologue(sh(ex["q_raw"]), sh(ex["k_raw"]), sh(ex["gate_pre"]),
                                             np.asarray(ex["beta_pre"]).reshape(T, 1), ex["lo"])
        np.testing.assert_allclose(qh[:, 0], ex["q_hat"], rtol=0, atol=1e-15)
        np.testing.assert_allclose(kh[:, 0], ex["k_hat"], rtol=0, atol=1e-15)
        np.testing.assert_allclose(la[:, 0], ex["log_alpha"], rtol=0, atol=1e-15)
        np.testing.assert_allclose(be[:, 0], ex["beta"], rtol=0, atol=1e-15)
        o, hT = oracle_mod.fwd_prologue(sh(ex["q_raw"]), sh(ex["k_raw"]), sh(ex["v"]), sh(ex["gate_pre"]),
                                        np.asarray(ex["beta_pre"]).reshape(T, 1), ex["lo"])
        np.testing.assert_allclose(o[:, 0], ex["o"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(hT[0, 0], ex["hT"], rtol=0, atol=1e-14)


def test_prologue_normalisation(oracle_mod):
    r = rng0(71)
    q = r.standard_normal((9, 3, 16)) * r.uniform(0.01, 50.0, (9, 3, 1))
    k = r.standard_normal((9, 3, 16))
    a = r.standard_normal((9, 3, 16))
    b = r.standard_normal((9, 3))
    qh, kh, _, _ = oracle_mod.prologue(q, k, a, b, -30.0)
    np.testing.assert_allclose(np.linalg.norm(qh, axis=-1), 1.0, rtol=1e-15)
    np.testing.assert_allclose(np.linalg.norm(kh, axis=-1), 1.0, rtol=1e-15)
    # same direction: the cosine with the raw vector is 1
    cos = np.sum(qh * q, axis=-1) / np.linalg.norm(q, axis=-1)
    np.testing.assert_allclose(cos, 1.0, rtol=1e-14)
    # scale invariance per row (positive scales)
    qh2, kh2, _, _ = oracle_mod.prologue(q * 7.25, k * 1e-3, a, b, -30.0)
    np.testing.assert_allclose(qh2, qh, rtol=0, atol=1e-15)
    np.testing.assert_allclose(kh2, kh, rtol=0, atol=1e-15)
    # eps: a zero row stays zero; a row shorter than eps is divided by eps
    z = np.zeros((1, 1, 4))
    tiny = np.array([[[1e-9, 0.0, 0.0, 0.0]]])
    qz, kt, _, _ = oracle_mod.prologue(z, tiny, np.zeros((1, 1, 4)), np.zeros((1, 1)), -30.0, eps=1e-6)
    assert np.all(qz == 0.0)
    np.testing.assert_allclose(kt[0, 0], [1e-3, 0.0, 0.0, 0.0], rtol=1e-15)


def test_prologue_gate_softplus_and_floor(oracle_mod):
    a = np.array([0.0, np.log(np.e - 1.0), -50.0, 50.0, 3.0, -3.0])
    x = a.reshape(1, 1, -1)
    one = np.ones_like(x)
    _, _, la, _ = oracle_mod.prologue(one, one, x, np.zeros((1, 1)), -100.0)
    la = la[0, 0]
    assert la[0] == pytest.approx(-np.log(2.0), rel=1e-15)        # softplus(0) = ln 2
    assert la[1] == pytest.approx(-1.0, rel=1e-15)                # softplus(ln(e-1)) = 1
    assert la[2] == pytest.approx(-np.exp(-50.0), rel=1e-12)      # alpha -> 1
    assert la[3] == pytest.approx(-50.0, rel=1e-15)               # softplus(a) -> a
    # softplus(a) - softplus(-a) = a, and the library's log(1 + e^a)
    r = rng0(72)
    aa = r.uniform(-40, 40, (1, 1, 64))
    ones = np.ones_like(aa)
    _, _, lp, _ = oracle_mod.prologue(ones, ones, aa, np.zeros((1, 1)), -1e3)
    _, _, lm, _ = oracle_mod.prologue(ones, ones, -aa, np.zeros((1, 1)), -1e3)
    np.testing.assert_allclose(-lp + lm, aa, rtol=0, atol=1e-13)
    np.testing.assert_allclose(-lp, np.logaddexp(0.0, aa), rtol=1e-15, atol=0)
    # the floor: exactly lo where -softplus falls below it, untouched elsewhere
    lo = -0.75
    _, _, lf, _ = oracle_mod.prologue(ones, ones, aa, np.zeros((1, 1)), lo)
    below = -np.logaddexp(0.0, aa) < lo
    assert below.any() and (~below).any()
    assert np.all(lf[below] == lo)
    np.testing.assert_allclose(lf[~below], lp[~below], rtol=0, atol=0)


def test_prologue_beta_sigmoid(oracle_mod):
    from scipy.special import expit
    r = rng0(73)
    b = np.concatenate([[0.0, 40.0, -40.0, 1e-9], r.uniform(-30, 30, 60)]).reshape(64, 1)
    one = np.ones((64, 1, 2))
    _, _, _, bp = oracle_mod.prologue(one, one, one, b, -30.0)
    _, _, _, bm = oracle_mod.prologue(one, one, one, -b, -30.0)
    assert bp[0, 0] == 0.5
    np.testing.assert_allclose(bp + bm, 1.0, rtol=0, atol=1e-15)   # sigmoid(b) + sigmoid(-b) = 1
    np.testing.assert_allclose(bp, expit(b), rtol=1e-15, atol=0)
    assert bp[2, 0] == pytest.approx(np.exp(-40.0), rel=1e-12)


def test_prologue_forward_scale_invariance(oracle_mod):
    # o and h_T depend on q and k only through their directions
    r = rng0(74)
    T, H, dk, dv = 40, 2, 8, 5
    q = r.standard_normal((T, H, dk))
    k = r.standard_normal((T, H, dk))
    v = r.standard_normal((T, H, dv))
    a = r.standard_normal((T, H, dk))
    b = r.standard_normal((T, H))
    o1, h1 = oracle_mod.fwd_prologue(q, k, v, a, b, -20.0)
    s = r.uniform(0.1, 10.0, (T, H, 1))
    o2, h2 = oracle_mod.fwd_prologue(q * s, k / s, v, a, b, -20.0)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(h2, h1, rtol=0, atol=1e-12)
    # and decode on raw inputs equals one forward step
    S0 = r.standard_normal((T, H, dk, dv)) * 0.1
    od, Sd = oracle_mod.decode_prologue(q, k, v, a, b, -20.0, S0)
    cu = np.arange(T + 1)
    of, hf = oracle_mod.fwd_prologue(q, k, v, a, b, -20.0, h0=S0, cu_seqlens=cu)
    np.testing.assert_allclose(od, of, rtol=0, atol=1e-15)
    np.testing.assert_allclose(Sd, hf, rtol=0, atol=1e-15)
