"""Pins for the fp64 oracle, each against something other than the oracle itself.

The recurrence is the one on the page "Why NVIDIA Gated DeltaNet-2 separates
erase and write gates" (axbrief.com), section "Gated Delta Rule-2: channel-wise
separation of erase and write".  The pages print no worked numerical example, so
the pins are: the equation itself as explicit dk x dk transition matrices (also
in exact rational arithmetic), the two special cases the same section names
(both gates equal to one scalar -> KDA; decay also scalar -> Gated DeltaNet),
exact retrieval along a unit key (page "Why Qwen3.5 chose Gated DeltaNet",
laonpeople.com, section on the delta rule as a precise eraser), closed-form
decay, the parallel (attention) form of gated linear attention, linearity,
resume, decode equivalence and finite differences for the VJP.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle

RTOL = 1e-12


def rand_inputs(rng, B, T, H, dk, dv, g_lo=-0.5, g_hi=0.0, s0=True):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    g = rng.uniform(g_lo, g_hi, (B, T, H, dk))
    b = rng.uniform(0, 1, (B, T, H, dk))
    w = rng.uniform(0, 1, (B, T, H, dv))
    S0 = rng.standard_normal((B, H, dk, dv)) * 0.3 if s0 else None
    return q, k, v, g, b, w, S0


def dense_transition_reference(q, k, v, g, b, w, S0):
    """Literal equation: M_t = (I - k (b.k)^T) Diag(alpha_t) as explicit matrices.

    S_t is built from the unrolled sum  S_t = (M_t ... M_1) S_0
    + sum_{s<=t} (M_t ... M_{s+1}) k_s (w_s.v_s)^T, and o_t = S_t^T q_t."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    ST = np.zeros((B, H, dk, dv))
    for bi in range(B):
        for h in range(H):
            Ms = []
            for t in range(T):
                kk, bb = k[bi, t, h], b[bi, t, h]
                Ms.append((np.eye(dk) - np.outer(kk, bb * kk)) @ np.diag(np.exp(g[bi, t, h])))
            S0h = S0[bi, h] if S0 is not None else np.zeros((dk, dv))
            for t in range(T):
                # (M_t ... M_1) S_0
                P = np.eye(dk)
                for s in range(t + 1):
                    P = Ms[s] @ P
                S = P @ S0h
                for s in range(t + 1):
                    Q = np.eye(dk)
                    for r in range(s + 1, t + 1):
                        Q = Ms[r] @ Q
                    S = S + Q @ np.outer(k[bi, s, h], w[bi, s, h] * v[bi, s, h])
                o[bi, t, h] = S.T @ q[bi, t, h]
                if t == T - 1:
                    ST[bi, h] = S
    return o, ST


def test_dense_transition_products():
    rng = np.random.default_rng(11)
    q, k, v, g, b, w, S0 = rand_inputs(rng, 1, 9, 2, 5, 4)
    o_ref, s_ref = dense_transition_reference(q, k, v, g, b, w, S0)
    o, s = oracle.fwd(q, k, v, g, b, w, S0)
    np.testing.assert_allclose(o, o_ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(s, s_ref, rtol=1e-11, atol=1e-12)


def test_dense_transition_zero_init_and_multibatch():
    rng = np.random.default_rng(12)
    q, k, v, g, b, w, _ = rand_inputs(rng, 2, 7, 3, 4, 6, s0=False)
    o_ref, s_ref = dense_transition_reference(q, k, v, g, b, w, None)
    o, s = oracle.fwd(q, k, v, g, b, w, None)
    np.testing.assert_allclose(o, o_ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(s, s_ref, rtol=1e-11, atol=1e-12)


def test_exact_rational_worked_example():
    """Tiny case in exact rational arithmetic of the literal equation.

    alpha is chosen rational (g = log alpha), so the only rounding on the
    oracle side is fp64 arithmetic; the expected values here are exact."""
    F = Fraction
    dk, dv, T = 2, 2, 3
    alpha = [[F(1, 2), F(3, 4)], [F(1, 1), F(1, 3)], [F(2, 3), F(1, 1)]]
    kk = [[F(3, 5), F(4, 5)], [F(1, 1), F(0)], [F(-4, 5), F(3, 5)]]
    bb = [[F(1, 2), F(1)], [F(1, 4), F(3, 4)], [F(1), F(0)]]
    vv = [[F(2), F(-1)], [F(1, 2), F(3)], [F(-1), F(1, 3)]]
    ww = [[F(1), F(1, 2)], [F(1, 3), F(1)], [F(0), F(1)]]
    qq = [[F(1), F(2)], [F(-1), F(1, 2)], [F(1, 2), F(1, 2)]]
    S = [[F(1, 10), F(0)], [F(-1, 5), F(3, 10)]]

    def matmul(A, Bm):
        return [[sum(A[i][m] * Bm[m][j] for m in range(len(Bm))) for j in range(len(Bm[0]))]
                for i in range(len(A))]

    outs = []
    for t in range(T):
        M = [[(1 if i == j else 0) - kk[t][i] * bb[t][j] * kk[t][j] for j in range(dk)]
             for i in range(dk)]
        D = [[alpha[t][i] if i == j else 0 for j in range(dk)] for i in range(dk)]
        W = [[kk[t][i] * ww[t][j] * vv[t][j] for j in range(dv)] for i in range(dk)]
        MD = matmul(M, D)
        S = [[x + y for x, y in zip(r1, r2)] for r1, r2 in zip(matmul(MD, S), W)]
        outs.append([sum(S[c][j] * qq[t][c] for c in range(dk)) for j in range(dv)])

    def arr(x):
        return np.array([[float(e) for e in row] for row in x])

    q = arr(qq)[None, :, None, :]
    k = arr(kk)[None, :, None, :]
    v = arr(vv)[None, :, None, :]
    w = arr(ww)[None, :, None, :]
    b = arr(bb)[None, :, None, :]
    g = np.log(arr(alpha))[None, :, None, :]
    S0 = arr([[F(1, 10), F(0)], [F(-1, 5), F(3, 10)]])[None, None]
    o, s = oracle.fwd(q, k, v, g, b, w, S0)
    np.testing.assert_allclose(o[0, :, 0], arr(outs), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(s[0, 0], arr(S), rtol=1e-14, atol=1e-15)


def kda_reference(q, k, v, g, beta, S0):
    """Kimi Delta Attention: S = (I - beta k k^T) Diag(alpha) S + beta k v^T."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    ST = np.zeros((B, H, dk, dv))
    for bi in range(B):
        for h in range(H):
            S = S0[bi, h].copy()
            for t in range(T):
                kk, bt = k[bi, t, h], beta[bi, t, h]
                S = (np.eye(dk) - bt * np.outer(kk, kk)) @ (np.exp(g[bi, t, h])[:, None] * S) \
                    + bt * np.outer(kk, v[bi, t, h])
                o[bi, t, h] = S.T @ q[bi, t, h]
            ST[bi, h] = S
    return o, ST


def gated_deltanet_reference(q, k, v, a, beta, S0):
    """Gated DeltaNet: S = alpha (I - beta k k^T) S + beta k v^T, scalar alpha."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    ST = np.zeros((B, H, dk, dv))
    for bi in range(B):
        for h in range(H):
            S = S0[bi, h].copy()
            for t in range(T):
                kk, bt = k[bi, t, h], beta[bi, t, h]
                S = math.exp(a[bi, t, h]) * (np.eye(dk) - bt * np.outer(kk, kk)) @ S \
                    + bt * np.outer(kk, v[bi, t, h])
                o[bi, t, h] = S.T @ q[bi, t, h]
            ST[bi, h] = S
    return o, ST


def test_reduces_to_kda_when_gates_equal_scalar():
    rng = np.random.default_rng(13)
    B, T, H, dk, dv = 2, 12, 2, 6, 5
    q, k, v, g, _, _, S0 = rand_inputs(rng, B, T, H, dk, dv)
    beta = rng.uniform(0, 1, (B, T, H))
    b = np.repeat(beta[..., None], dk, axis=-1)
    w = np.repeat(beta[..., None], dv, axis=-1)
    o, s = oracle.fwd(q, k, v, g, b, w, S0)
    o_ref, s_ref = kda_reference(q, k, v, g, beta, S0)
    np.testing.assert_allclose(o, o_ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(s, s_ref, rtol=1e-11, atol=1e-12)


def test_reduces_to_gated_deltanet_when_decay_also_scalar():
    rng = np.random.default_rng(14)
    B, T, H, dk, dv = 1, 15, 3, 7, 4
    q, k, v, _, _, _, S0 = rand_inputs(rng, B, T, H, dk, dv)
    beta = rng.uniform(0, 1, (B, T, H))
    a = rng.uniform(-0.5, 0, (B, T, H))
    g = np.repeat(a[..., None], dk, axis=-1)
    b = np.repeat(beta[..., None], dk, axis=-1)
    w = np.repeat(beta[..., None], dv, axis=-1)
    o, s = oracle.fwd(q, k, v, g, b, w, S0)
    o_ref, s_ref = gated_deltanet_reference(q, k, v, a, beta, S0)
    np.testing.assert_allclose(o, o_ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(s, s_ref, rtol=1e-11, atol=1e-12)


def test_exact_retrieval_along_unit_key():
    """q = k, |k| = 1, b = 1  =>  o_t = S_t^T k_t = w_t . v_t for any decay and state."""
    rng = np.random.default_rng(15)
    B, T, H, dk, dv = 2, 20, 2, 8, 6
    _, k, v, g, _, w, S0 = rand_inputs(rng, B, T, H, dk, dv, g_lo=-3.0)
    k = k / np.linalg.norm(k, axis=-1, keepdims=True)
    b = np.ones_like(k)
    o, _ = oracle.fwd(k, k, v, g, b, w, S0)
    np.testing.assert_allclose(o, w * v, rtol=1e-12, atol=1e-12)


def test_single_write_retrieval():
    """One write with alpha = b = w = 1, S_0 = 0, |k| = 1, q = k  =>  o = v."""
    rng = np.random.default_rng(16)
    k = rng.standard_normal((1, 1, 1, 16))
    k /= np.linalg.norm(k)
    v = rng.standard_normal((1, 1, 1, 16))
    o, s = oracle.fwd(k, k, v, np.zeros_like(k), np.ones_like(k), np.ones_like(v))
    np.testing.assert_allclose(o, v, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(s[0, 0], np.outer(k[0, 0, 0], v[0, 0, 0]), rtol=1e-13, atol=1e-14)


def test_closed_form_geometric_decay():
    """b = w = 0: S_T = Diag(exp(sum g)) S_0 and o_t = S_0^T (exp(G_t) . q_t)."""
    rng = np.random.default_rng(17)
    B, T, H, dk, dv = 2, 30, 2, 6, 5
    q, k, v, g, _, _, S0 = rand_inputs(rng, B, T, H, dk, dv, g_lo=-0.3)
    b = np.zeros_like(k)
    w = np.zeros_like(v)
    o, s = oracle.fwd(q, k, v, g, b, w, S0)
    G = np.cumsum(g, axis=1)
    o_ref = np.einsum("bhcj,bthc->bthj", S0, np.exp(G) * q)
    s_ref = np.exp(G[:, -1])[..., None] * S0
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(s, s_ref, rtol=1e-12, atol=1e-13)


def test_gated_linear_attention_parallel_form():
    """b = 0, w = 1: o_t = S_0^T(e^{G_t}.q_t) + sum_{j<=t} (sum_c q_tc e^{G_tc-G_jc} k_jc) v_j."""
    rng = np.random.default_rng(18)
    B, T, H, dk, dv = 1, 40, 2, 8, 6
    q, k, v, g, _, _, S0 = rand_inputs(rng, B, T, H, dk, dv, g_lo=-0.2)
    b = np.zeros_like(k)
    w = np.ones_like(v)
    o, s = oracle.fwd(q, k, v, g, b, w, S0)
    G = np.cumsum(g, axis=1)
    for h in range(H):
        Gh, qh, kh, vh = G[0, :, h], q[0, :, h], k[0, :, h], v[0, :, h]
        att = np.einsum("tc,jc,tjc->tj", qh, kh, np.exp(Gh[:, None, :] - Gh[None, :, :]))
        att = np.tril(att)
        o_ref = att @ vh + (np.exp(Gh) * qh) @ S0[0, h]
        np.testing.assert_allclose(o[0, :, h], o_ref, rtol=1e-11, atol=1e-12)
        s_ref = np.exp(Gh[-1])[:, None] * S0[0, h] + (kh * np.exp(Gh[-1] - Gh)).T @ vh
        np.testing.assert_allclose(s[0, h], s_ref, rtol=1e-11, atol=1e-12)


def test_causal_linear_attention_without_decay():
    """b = 0, w = 1, alpha = 1, S_0 = 0: o = tril(Q K^T) V (a plain matmul)."""
    rng = np.random.default_rng(19)
    B, T, H, dk, dv = 1, 33, 1, 5, 7
    q, k, v, _, _, _, _ = rand_inputs(rng, B, T, H, dk, dv)
    o, s = oracle.fwd(q, k, v, np.zeros_like(q), np.zeros_like(k), np.ones_like(v))
    Q, K, V = q[0, :, 0], k[0, :, 0], v[0, :, 0]
    np.testing.assert_allclose(o[0, :, 0], np.tril(Q @ K.T) @ V, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(s[0, 0], K.T @ V, rtol=1e-11, atol=1e-12)


def test_linearity_in_initial_state_and_written_value():
    rng = np.random.default_rng(20)
    B, T, H, dk, dv = 1, 25, 2, 6, 5
    q, k, v1, g, b, _, S1 = rand_inputs(rng, B, T, H, dk, dv)
    v2 = rng.standard_normal(v1.shape)
    S2 = rng.standard_normal(S1.shape)
    w = np.ones_like(v1)
    a1, a2 = 0.7, -1.3
    o1, s1 = oracle.fwd(q, k, v1, g, b, w, S1)
    o2, s2 = oracle.fwd(q, k, v2, g, b, w, S2)
    o12, s12 = oracle.fwd(q, k, a1 * v1 + a2 * v2, g, b, w, a1 * S1 + a2 * S2)
    np.testing.assert_allclose(o12, a1 * o1 + a2 * o2, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(s12, a1 * s1 + a2 * s2, rtol=1e-10, atol=1e-11)


@pytest.mark.parametrize("split", [1, 17, 64])
def test_resume_equals_one_call(split):
    rng = np.random.default_rng(21)
    B, T, H, dk, dv = 2, 80, 2, 6, 5
    q, k, v, g, b, w, S0 = rand_inputs(rng, B, T, H, dk, dv)
    o, s = oracle.fwd(q, k, v, g, b, w, S0)
    sl1, sl2 = slice(0, split), slice(split, T)
    oa, sa = oracle.fwd(q[:, sl1], k[:, sl1], v[:, sl1], g[:, sl1], b[:, sl1], w[:, sl1], S0)
    ob, sb = oracle.fwd(q[:, sl2], k[:, sl2], v[:, sl2], g[:, sl2], b[:, sl2], w[:, sl2], sa)
    np.testing.assert_allclose(np.concatenate([oa, ob], axis=1), o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(sb, s, rtol=1e-13, atol=1e-14)


def test_decode_steps_equal_forward():
    rng = np.random.default_rng(22)
    B, T, H, dk, dv = 3, 11, 2, 6, 4
    q, k, v, g, b, w, S0 = rand_inputs(rng, B, T, H, dk, dv)
    o, s = oracle.fwd(q, k, v, g, b, w, S0)
    st = S0.copy()
    for t in range(T):
        ot, st = oracle.decode(q[:, t], k[:, t], v[:, t], g[:, t], b[:, t], w[:, t], st)
        np.testing.assert_allclose(ot, o[:, t], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(st, s, rtol=1e-13, atol=1e-14)


def test_thread_count_does_not_change_results():
    rng = np.random.default_rng(23)
    q, k, v, g, b, w, S0 = rand_inputs(rng, 3, 20, 3, 8, 8)
    o1, s1 = oracle.fwd(q, k, v, g, b, w, S0, nthreads=1)
    o4, s4 = oracle.fwd(q, k, v, g, b, w, S0, nthreads=4)
    assert np.array_equal(o1, o4) and np.array_equal(s1, s4)


def test_strong_decay_stays_finite():
    """log alpha down to -200 per step: exp underflows to 0, results stay finite."""
    rng = np.random.default_rng(24)
    q, k, v, g, b, w, S0 = rand_inputs(rng, 1, 50, 1, 6, 5, g_lo=-200.0, g_hi=-50.0)
    o, s = oracle.fwd(q, k, v, g, b, w, S0)
    assert np.isfinite(o).all() and np.isfinite(s).all()
    # alpha ~ 0: S_t = k_t (w_t.v_t)^T exactly (the erase reads an all-zero state)
    kk = k[0, -1, 0]
    np.testing.assert_allclose(s[0, 0], np.outer(kk, w[0, -1, 0] * v[0, -1, 0]), rtol=1e-13,
                               atol=1e-14)


# ---------------------------------------------------------------- VJP ------

def _loss(q, k, v, g, b, w, S0, do, dsT):
    o, s = oracle.fwd(q, k, v, g, b, w, S0, nthreads=1)
    return float(np.sum(o * do) + np.sum(s * dsT))


def test_vjp_matches_central_finite_differences():
    """Every input element of a T=64, dk=dv=16 case (two heads), h = 1e-6."""
    rng = np.random.default_rng(25)
    B, T, H, dk, dv = 1, 64, 2, 16, 16
    q, k, v, g, b, w, S0 = rand_inputs(rng, B, T, H, dk, dv, g_lo=-0.3)
    S0 = S0 * 0.1
    do = rng.standard_normal((B, T, H, dv))
    dsT = rng.standard_normal((B, H, dk, dv))
    grads = oracle.vjp(q, k, v, g, b, w, do, S0, dsT)
    args = dict(q=q, k=k, v=v, g=g, b=b, w=w, S0=S0)
    names = dict(q="dq", k="dk", v="dv", g="dlog_alpha", b="db", w="dw", S0="ds0")
    h = 1e-6
    worst = 0.0
    for name, x in args.items():
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + h
            lp = _loss(**args, do=do, dsT=dsT)
            x[idx] = old - h
            lm = _loss(**args, do=do, dsT=dsT)
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        an = grads[names[name]]
        scale = max(1.0, np.abs(fd).max())
        err = np.abs(an - fd).max() / scale
        worst = max(worst, err)
        assert err < 1e-7, (name, err)
    assert worst < 1e-7


def test_vjp_zero_length_passes_state_gradient_through():
    rng = np.random.default_rng(26)
    dsT = rng.standard_normal((1, 1, 3, 2))
    z = np.zeros((1, 0, 1, 3))
    zv = np.zeros((1, 0, 1, 2))
    gr = oracle.vjp(z, z, zv, z, z, zv, zv, np.zeros((1, 1, 3, 2)), dsT)
    np.testing.assert_array_equal(gr["ds0"], dsT)


def test_oracle_matches_its_regression_fixture():
    """Drift guard (not a pin): sampled outputs stored by tests/golden/make_oracle_regression.py."""
    import importlib.util
    import os

    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    spec = importlib.util.spec_from_file_location("make_oracle_regression",
                                                  os.path.join(here, "make_oracle_regression.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    _, o, s = mod.compute()
    n = 0
    for line in open(os.path.join(here, "oracle_regression_tiny.txt")):
        if line.startswith("#"):
            continue
        kind, a, b_, c, d, val = line.split()
        x = (o if kind == "o" else s)[int(a), int(b_), int(c), int(d)]
        assert abs(x - float(val)) <= 1e-13 * max(1.0, abs(float(val))), line
        n += 1
    assert n == 60
