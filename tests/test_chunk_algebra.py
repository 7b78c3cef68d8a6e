"""The closed forms the matrix-core kernels evaluate, checked against the oracle.

The GPU's chunk form does not step through the tokens: for one (entry, value head) with
row decays d_t = exp(g_t) exp(gk_t), decay products c_t = d_0 ... d_t and
g(t,s) = d_{s+1} ... d_t, it forms

    M[t,s] = sum_i g(t,s)_i k_s,i k_t,i   (s < t),   N[t,s] = sum_i g(t,s)_i k_s,i (scale q_t)_i   (s <= t)
    u_t  = beta_t (v_t - S0^T (c_t k_t) - sum_{s<t} M[t,s] u_s)
    o_t  = S0^T (c_t scale q_t) + sum_{s<=t} N[t,s] u_s
    S_n  = diag(c_{n-1}) S0 + sum_{s<n} (g(n-1,s) k_s) (x) u_s

(MindSpore Lite API page "lite_boost.ops.recurrent_gated_delta_rule", algorithm section,
unrolled). This file evaluates exactly that, in plain fp64 numpy with no rounding, and
requires it to equal the oracle's token-by-token recurrence to 1e-12: the derivation the
kernel rests on is then exact, and only the kernel's rounding separates it from the oracle.
"""
import numpy as np
import pytest

import oracle


def closed_form(S0, q, k, v, beta, g, gk, scale, L, n):
    """One (entry, value head): S0 [D_k, D_v]; q, k [T, D_k]; v [T, D_v]; beta, g [T];
    gk [T, D_k]. Returns (out [L, D_v], committed state [D_k, D_v])."""
    d = np.exp(g)[:, None] * np.exp(gk)                  # [T, D_k] row decays
    c = np.cumprod(d[:L], axis=0)                        # c_t
    def gts(t, s):                                        # g(t, s) = d_{s+1} ... d_t
        return np.prod(d[s + 1:t + 1], axis=0) if t > s else np.ones(S0.shape[0])
    qs = scale * q
    M = np.zeros((L, L))
    N = np.zeros((L, L))
    for t in range(L):
        for s in range(t + 1):
            w = gts(t, s) * k[s]
            if s < t:
                M[t, s] = w @ k[t]
            N[t, s] = w @ qs[t]
    A = (c * k[:L]) @ S0                                  # [L, D_v]: S0^T (c_t k_t)
    Bq = (c * qs[:L]) @ S0                                # [L, D_v]: S0^T (c_t scale q_t)
    u = np.zeros((L, S0.shape[1]))
    out = np.zeros((L, S0.shape[1]))
    for t in range(L):
        u[t] = beta[t] * (v[t] - A[t] - M[t, :t] @ u[:t])
        out[t] = Bq[t] + N[t, :t + 1] @ u[:t + 1]
    if n == 0:
        return out, S0.copy()
    S = c[n - 1][:, None] * S0
    for s in range(n):
        S += np.outer(gts(n - 1, s) * k[s], u[s])
    return out, S


@pytest.mark.parametrize("seed", range(6))
def test_closed_form_equals_the_recurrence(seed):
    rng = np.random.default_rng(500 + seed)
    B, Hq, Hv, T, Dk, Dv = 3, 1, 2, 8, 12, 7
    q = rng.standard_normal((B, Hq, T, Dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((B, Hq, T, Dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, Hv, T, Dv))
    beta = 1 / (1 + np.exp(-rng.standard_normal((B, Hv, T))))
    if seed == 5:
        beta[0, 0, :] = 0.0                               # pure decay entry
    g = -np.log1p(np.exp(rng.standard_normal((B, Hv, T)) * (1 + 3 * seed)))  # up to strong decay
    gk = -rng.uniform(1e-3, 0.1 * (1 + seed), (B, Hv, T, Dk))
    pool = 0.3 * rng.standard_normal((B, Hv, Dk, Dv))
    lens = np.array([8, 1 + seed % 7, 5], np.int32)
    nacc = np.array([8 - seed % 3, lens[1], 0 if seed % 2 else 3], np.int32)
    idx = np.arange(B, dtype=np.int32)
    scale = 1 / np.sqrt(Dk)
    out_ref, pool_ref = oracle.rgdr_f64(q, k, v, beta, pool, lens, idx, g, gk, nacc, scale)
    for b in range(B):
        for h in range(Hv):
            out, S = closed_form(pool[b, h], q[b, 0], k[b, 0], v[b, h], beta[b, h], g[b, h],
                                 gk[b, h], scale, lens[b], nacc[b])
            np.testing.assert_allclose(out, out_ref[b, h, :lens[b]], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(S, pool_ref[b, h], rtol=1e-12, atol=1e-12)


def test_closed_form_detects_a_wrong_decay_product():
    """The check has teeth: using c_t instead of g(t, s) in M (a plausible slip in the
    derivation) is far outside the bound."""
    rng = np.random.default_rng(9)
    T, Dk, Dv = 6, 10, 5
    q = rng.standard_normal((1, 1, T, Dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((1, 1, T, Dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((1, 1, T, Dv))
    beta = np.full((1, 1, T), 0.7)
    g = np.full((1, 1, T), -0.5)
    gk = -rng.uniform(0.01, 0.3, (1, 1, T, Dk))
    pool = 0.3 * rng.standard_normal((1, 1, Dk, Dv))
    lens = np.array([T], np.int32)
    out_ref, _ = oracle.rgdr_f64(q, k, v, beta, pool, lens, np.zeros(1, np.int32), g, gk, lens, 1.0)
    d = np.exp(g[0, 0])[:, None] * np.exp(gk[0, 0])
    c = np.cumprod(d, axis=0)
    kk, qq = k[0, 0], q[0, 0]
    Mwrong = np.array([[(c[t] * kk[s]) @ kk[t] if s < t else 0.0 for s in range(T)] for t in range(T)])
    A = (c * kk) @ pool[0, 0]
    u = np.zeros((T, Dv))
    for t in range(T):
        u[t] = beta[0, 0, t] * (v[0, 0, t] - A[t] - Mwrong[t, :t] @ u[:t])
    out, _ = closed_form(pool[0, 0], qq, kk, v[0, 0], beta[0, 0], g[0, 0], gk[0, 0], 1.0, T, T)
    np.testing.assert_allclose(out, out_ref[0, 0], rtol=1e-12, atol=1e-12)
    # the slip changes u (and so the outputs) by far more than the bound
    u_right = np.zeros((T, Dv))
    M = np.zeros((T, T))
    for t in range(T):
        for s in range(t):
            M[t, s] = (np.prod(d[s + 1:t + 1], axis=0) * kk[s]) @ kk[t]
    for t in range(T):
        u_right[t] = beta[0, 0, t] * (v[0, 0, t] - A[t] - M[t, :t] @ u_right[:t])
    assert np.abs(u - u_right).max() > 1e-3


# ---------------------------------------------------------------------------------------
# The long-sequence kernel's steps: chunks of up to 32 tokens in the factored closed form,
# decay products measured from each row's middle of the chunk, the state carried with a
# pending per-row factor, the triangular system solved in 16-token blocks.
# ---------------------------------------------------------------------------------------


def long_sequence_form(S0, q, k, v, beta, g, gk, scale, L, n, chunk=32, span=96.0, mid=True):
    """One (entry, value head) through the long-sequence kernel's steps in fp64. Returns
    (out [L, D_v], committed state [D_k, D_v], chunk lengths). mid=False measures the decay
    products from the chunk's start instead of each row's middle."""
    Dk, Dv = S0.shape
    log2d = (g[:, None] + gk) / np.log(2.0)          # log2 of each row's decay, [T, D_k]
    out = np.zeros((L, Dv))
    keep, pend = S0.copy(), np.ones(Dk)              # the true state is diag(pend) keep
    committed = S0.copy() if n == 0 else None
    lengths = []
    t0 = 0
    while t0 < L:
        t1 = min(t0 + chunk, L)
        if t0 < n < t1:
            t1 = n                                   # the chunk holding n - 1 ends there
        while True:                                  # cut by the decay range
            Lt = np.zeros((t1 - t0, Dk))            # L_t = log2 c_t, token 0's decay excluded
            Lt[1:] = np.cumsum(log2d[t0 + 1:t1], axis=0)
            lref = 0.5 * Lt[-1] if mid else np.zeros(Dk)   # each row's reference
            with np.errstate(invalid="ignore"):      # a zero decay gives -inf - -inf here
                x = Lt - lref
                if np.all(np.abs(x) <= span):
                    break
                cuts = []
                for i in np.nonzero(~(np.abs(x) <= span).all(axis=0))[0]:
                    wide = mid and abs(Lt[-1, i]) > 2 * span
                    y, lim = (Lt[:, i], 2 * span) if wide else (x[:, i], span)
                    cuts.append(int(np.nonzero(~(np.abs(y) <= lim))[0][0]))
            t1 = t0 + min(cuts)
        Lc = t1 - t0
        lengths.append(Lc)
        cp = 2.0 ** x                                # c'_t
        S2 = (pend * 2.0 ** (log2d[t0] + lref))[:, None] * keep   # S'' = diag(r) diag(d_0) S
        kk, qs, bt = k[t0:t1], scale * q[t0:t1], beta[t0:t1]
        Xk, Xq, Kd = cp * kk, cp * qs, kk / cp
        YK, YQ = Xk @ S2, Xq @ S2
        M = np.tril(Xk @ Kd.T, -1)                   # M[t][s] = sum_i (c_t / c_s) k_t k_s, s < t
        N = np.tril(Xq @ Kd.T)                       # N[t][s], s <= t
        R = v[t0:t1] - YK
        U = np.zeros((Lc, Dv))
        for a in range(0, Lc, 16):                   # U_b = A_bb (R_b - M_b,<b U_<b)
            b = min(a + 16, Lc)
            Abb = np.linalg.inv(np.eye(b - a) + bt[a:b, None] * M[a:b, a:b]) * bt[None, a:b]
            U[a:b] = Abb @ (R[a:b] - M[a:b, :a] @ U[:a])
        out[t0:t1] = YQ + N @ U
        keep = S2 + Kd.T @ U                         # S'' + K'^T U
        pend = 2.0 ** (Lt[-1] - lref)                # c'_last
        t0 = t1
        if t0 == n:
            committed = pend[:, None] * keep
    return out, committed, lengths


def _long_case(rng, T, Dk, Dv, g, gk):
    q = rng.standard_normal((1, 1, T, Dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((1, 1, T, Dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((1, 1, T, Dv))
    beta = 1 / (1 + np.exp(-rng.standard_normal((1, 1, T))))
    pool = 0.3 * rng.standard_normal((1, 1, Dk, Dv))
    return q, k, v, beta, pool, g.reshape(1, 1, T), gk.reshape(1, 1, T, Dk)


@pytest.mark.parametrize("case", ["mild", "strong", "very_strong", "mixed_rows", "zero_decay"])
def test_long_sequence_form_equals_the_recurrence(case):
    """The steps agree with the oracle's token-by-token recurrence to 1e-10 (relative to the
    largest value): mild decays (chunks of 32, then a ragged end, the accepted count inside a
    chunk); decays of 4.5 and 12 nats per token (chunks cut around the middle, and rows whose
    whole chunk spans more than 2^192); rows decaying at different rates; and a decay of
    exactly zero (the state wiped)."""
    rng = np.random.default_rng({"mild": 1, "strong": 2, "very_strong": 3, "mixed_rows": 4,
                                 "zero_decay": 5}[case])
    T, Dk, Dv = 90, 12, 7
    g = -np.log1p(np.exp(rng.standard_normal(T)))
    gk = -rng.uniform(1e-3, 0.1, (T, Dk))
    if case == "strong":
        g[:] = -4.5
    elif case == "very_strong":
        g[:] = -12.0
    elif case == "mixed_rows":
        gk[:, : Dk // 2] = -rng.uniform(3.0, 9.0, (T, Dk // 2))
    elif case == "zero_decay":
        g[40] = -np.inf
    q, k, v, beta, pool, g3, gk4 = _long_case(rng, T, Dk, Dv, g, gk)
    L, n = 90, 50
    lens, nacc = np.array([L], np.int32), np.array([n], np.int32)
    out_ref, pool_ref = oracle.rgdr_f64(q, k, v, beta, pool, lens, np.zeros(1, np.int32), g3,
                                        gk4, nacc, 1.0 / np.sqrt(Dk))
    out, S, lengths = long_sequence_form(pool[0, 0], q[0, 0], k[0, 0], v[0, 0], beta[0, 0], g,
                                         gk, 1.0 / np.sqrt(Dk), L, n)
    assert sum(lengths) == L
    if case == "mild":
        assert lengths == [32, 18, 32, 8]            # split at n = 50, then the ragged end
    if case in ("strong", "very_strong", "mixed_rows"):
        assert max(lengths) < 32                     # the range cut the chunks
    scale_o = np.abs(out_ref[0, 0, :L]).max()
    np.testing.assert_allclose(out, out_ref[0, 0, :L], rtol=1e-10, atol=1e-10 * scale_o)
    np.testing.assert_allclose(S, pool_ref[0, 0], rtol=1e-10,
                               atol=1e-10 * np.abs(pool_ref[0, 0]).max())


@pytest.mark.parametrize("g_val", [-0.3, -4.5])
def test_long_sequence_form_reference_is_free(g_val):
    """The per-row reference cancels: measuring the decay products from the chunk's start
    (so a chunk may span only 2^96, and strong decays cut it earlier) gives the same outputs
    and state as the middle reference, to 1e-12 relative."""
    rng = np.random.default_rng(6)
    T, Dk, Dv = 70, 8, 5
    g = np.full(T, g_val)
    gk = -rng.uniform(1e-3, 0.1, (T, Dk))
    q, k, v, beta, pool, _, _ = _long_case(rng, T, Dk, Dv, g, gk)
    args = (pool[0, 0], q[0, 0], k[0, 0], v[0, 0], beta[0, 0], g, gk, 0.5, T, 45)
    o_mid, s_mid, l_mid = long_sequence_form(*args)
    o_start, s_start, l_start = long_sequence_form(*args, mid=False)
    if g_val < -1:
        assert max(l_start) < max(l_mid) < 32      # the two references cut differently
    else:
        assert l_start == l_mid == [32, 13, 25]
    np.testing.assert_allclose(o_start, o_mid, rtol=1e-12, atol=1e-12 * np.abs(o_mid).max())
    np.testing.assert_allclose(s_start, s_mid, rtol=1e-12, atol=1e-12 * np.abs(s_mid).max())
