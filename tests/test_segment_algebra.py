"""The decomposition the segmented long-sequence form rests on, checked with the oracle alone.

Steps 1 and 3 of the recurrence (MindSpore Lite API page
"lite_boost.ops.recurrent_gated_delta_rule", algorithm section) map the state as
S -> (I - beta_t k_t k_t^T) diag(exp(g_t) exp(gk_t)) S + beta_t k_t v_t^T: affine in S,
with v only in the constant term, and every state column evolves with its own column of v.
So a run of tokens maps its incoming state S to Phi S + Psi, where

    Psi = the end state from a zero state (with the tokens' v),
    Phi = the end states of the identity's columns with v = 0 (D_k x D_k),

and each token's output is o_t = S^T P_t + O0_t, with O0_t the output from the zero state and
P_t the identity run's output (q_t through Phi's partial products). This file obtains Psi,
Phi, P and O0 from the oracle's own token-by-token recurrence run on each segment, composes
them in fp64 numpy (S_{j+1} = Phi_j S_j + Psi_j), and requires the result to equal the
oracle's single run over the whole sequence: states and outputs to 1e-10 relative. Two
planted slips (v kept in the identity run; Psi added without Phi) must fail it.
"""
import numpy as np
import pytest

import oracle


def case(seed, T, Dk, Dv, decay=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, 1, T, Dk))
    k = rng.standard_normal((1, 1, T, Dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((1, 1, T, Dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((1, 1, T))))
    g = -decay * np.log1p(np.exp(rng.standard_normal((1, 1, T))))
    gk = -rng.uniform(1e-3, 0.1, (1, 1, T, Dk))
    S0 = 0.05 * rng.standard_normal((1, 1, Dk, Dv))
    return q, k, v, beta, g, gk, S0


def run(q, k, v, beta, g, gk, S, scale, t0, t1):
    """The oracle over tokens t0 .. t1 - 1 from state S (one entry, one head, fp64)."""
    T = t1 - t0
    sl = slice(t0, t1)
    one = np.array([T], np.int32)
    out, pool = oracle.rgdr_f64(q[:, :, sl], k[:, :, sl], v[:, :, sl], beta[:, :, sl], S,
                                one, np.zeros(1, np.int32), g[:, :, sl], gk[:, :, sl], one,
                                scale)
    return out[0, 0], pool[0, 0]


def segmented(q, k, v, beta, g, gk, S0, scale, bounds, slip=None):
    Dk = q.shape[-1]
    S = S0[0, 0].copy()
    outs = []
    for t0, t1 in zip(bounds[:-1], bounds[1:]):
        zero = np.zeros_like(S0)
        O0, Psi = run(q, k, v, beta, g, gk, zero, scale, t0, t1)
        vz = v.copy() if slip == "v_in_phi" else np.zeros_like(v)
        vz = vz[..., :Dk] if vz.shape[-1] >= Dk else np.zeros(v.shape[:-1] + (Dk,))
        P, Phi = run(q, k, vz, beta, g, gk, np.eye(Dk)[None, None], scale, t0, t1)
        outs.append(P @ S + O0)
        S = Psi + S if slip == "no_phi" else Phi @ S + Psi
    return np.concatenate(outs), S


@pytest.mark.parametrize("T,Dk,Dv,bounds,decay", [
    (96, 16, 24, [0, 32, 64, 96], 1.0),
    (100, 8, 8, [0, 7, 40, 41, 100], 1.0),        # ragged segments, one of a single token
    (64, 16, 16, [0, 16, 32, 48, 64], 0.05),      # weak decays: the state carries far
    (80, 16, 8, [0, 20, 80], 6.0),                 # strong decays
])
def test_segments_compose_to_the_whole_run(T, Dk, Dv, bounds, decay):
    q, k, v, beta, g, gk, S0 = case(1000 + T + Dk, T, Dk, Dv, decay)
    scale = 1.0 / np.sqrt(Dk)
    out_ref, S_ref = run(q, k, v, beta, g, gk, S0, scale, 0, T)
    out, S = segmented(q, k, v, beta, g, gk, S0, scale, bounds)
    tol = 1e-10 * max(1.0, np.abs(out_ref).max())
    assert np.abs(out - out_ref).max() <= tol
    assert np.abs(S - S_ref).max() <= 1e-10 * max(1.0, np.abs(S_ref).max())


@pytest.mark.parametrize("slip", ["v_in_phi", "no_phi"])
def test_planted_slips_fail(slip):
    T, Dk, Dv = 96, 16, 16
    q, k, v, beta, g, gk, S0 = case(2000, T, Dk, Dv, 0.05)
    scale = 1.0 / np.sqrt(Dk)
    out_ref, S_ref = run(q, k, v, beta, g, gk, S0, scale, 0, T)
    out, S = segmented(q, k, v, beta, g, gk, S0, scale, [0, 32, 64, 96], slip=slip)
    assert np.abs(S - S_ref).max() > 1e-6 or np.abs(out - out_ref).max() > 1e-6
