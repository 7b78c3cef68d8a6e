"""The closed form the matrix-core decode evaluates for T > 1, checked against the oracle.

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
