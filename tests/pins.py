"""Pins for the CPU oracle: checks against facts the pages and the mathematics fix.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises ``AssertionError`` when the
oracle disagrees with the fact it checks. ``tests/test_oracle_pins.py`` runs them on the
oracle; ``tests/test_oracle_mutants.py`` runs them on copies of the oracle with a planted
mistake and requires that some pin fails for each.

Sources: MindSpore Lite page "lite_boost.ops.recurrent_gated_delta_rule" (algorithm
section; parameters; returns; example) and the "com.microsoft.LinearAttentionGate" README
(Description; Inputs/Outputs; Type constraints). None of the pages prints a numeric
result, so the pins are closed forms, special cases that reduce to textbook operations,
brute force in exact rational arithmetic, invariants, and library conversions.
"""
import math
from fractions import Fraction

import numpy as np
import torch
from scipy.special import expit

# ------------------------------------------------------------------------------------
# fp64 case generator for the unrounded core (inputs only; no method arithmetic)
# ------------------------------------------------------------------------------------


def unit(rng, shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def f64_case(rng, B, Hq, Hv, T, Dk, Dv, N_slots, lens=None, idx=None, zero_state=False):
    c = dict(
        query=unit(rng, (B, Hq, T, Dk)),
        key=unit(rng, (B, Hq, T, Dk)),
        value=rng.standard_normal((B, Hv, T, Dv)),
        beta=rng.uniform(0.05, 0.95, (B, Hv, T)),
        state_pool=(np.zeros((N_slots, Hv, Dk, Dv)) if zero_state
                    else 0.3 * rng.standard_normal((N_slots, Hv, Dk, Dv))),
        actual_seq_lengths=np.full(B, T, np.int32) if lens is None else np.asarray(lens, np.int32),
        ssm_state_indices=(rng.permutation(N_slots)[:B].astype(np.int32) if idx is None
                           else np.asarray(idx, np.int32)),
        g=-rng.uniform(0.01, 1.0, (B, Hv, T)),
        gk=-rng.uniform(0.001, 0.3, (B, Hv, T, Dk)),
    )
    c["num_accepted_tokens"] = c["actual_seq_lengths"].copy()
    c["scale_value"] = 1.0 / math.sqrt(Dk)
    return c


def call_f64(o, c):
    return o.rgdr_f64(c["query"], c["key"], c["value"], c["beta"], c["state_pool"],
                      c["actual_seq_lengths"], c["ssm_state_indices"], c["g"], c["gk"],
                      c["num_accepted_tokens"], c["scale_value"])


def close(a, b, rtol, atol):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    assert np.all(np.isfinite(a)), "non-finite values"
    err = np.abs(a - b)
    bound = atol + rtol * np.abs(b)
    assert np.all(err <= bound), f"max err {err.max():.3e}, worst excess {(err - bound).max():.3e}"


def bits_equal(a, b):
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape
    assert a.view(np.uint64 if a.dtype == np.float64 else a.dtype).tobytes() == \
        b.view(np.uint64 if b.dtype == np.float64 else b.dtype).tobytes(), "not bit-identical"


# ------------------------------------------------------------------------------------
# Codec pins (bf16 and fp16) against torch/numpy conversions and hand-computed ties
# ------------------------------------------------------------------------------------


def pin_bf16_decode_all_patterns(o):
    """Every bf16 pattern decodes to what torch's bf16 -> fp32 widening gives."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    got = o.bf16_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan].astype(np.float64))
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def pin_bf16_encode_vs_torch(o):
    """fp32 -> bf16 by the oracle (from the exact fp64 value) equals torch's RNE cast."""
    rng = np.random.default_rng(7)
    raw = rng.integers(0, 2**32, 200000, dtype=np.uint64).astype(np.uint32)
    # ties: exact bf16 midpoints, and values next to them
    hi = rng.integers(0, 2**16, 20000, dtype=np.uint64).astype(np.uint32) << 16
    ties = np.concatenate([hi | 0x8000, hi | 0x7FFF, hi | 0x8001])
    x = np.concatenate([raw, ties]).view(np.float32)
    x = x[~np.isnan(x)]
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = o.f64_to_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref), f"{np.count_nonzero(got != ref)} mismatches"
    nanbits = o.f64_to_bf16(np.array([np.nan]))
    assert np.isnan(o.bf16_to_f64(nanbits))[0]


def pin_bf16_encode_single_rounding(o):
    """Rounding from fp64 is one rounding to nearest, ties to even (hand-computed cases)."""
    cases = [
        (1 + 2**-8 + 2**-40, 0x3F81),  # just above the midpoint: up (fp32 detour would tie)
        (1 + 2**-8, 0x3F80),           # exact midpoint, 1.0 has even mantissa: stays
        (1 + 3 * 2**-8, 0x3F82),       # midpoint above an odd mantissa: up to even
        (1 + 2**-8 - 2**-40, 0x3F80),  # just below the midpoint: down
        (-(1 + 2**-8 + 2**-40), 0xBF81),
        (2.0**-134, 0x0000),           # half the smallest subnormal: tie to even zero
        (2.0**-134 + 2.0**-160, 0x0001),
        (3 * 2.0**-134, 0x0002),       # 1.5 quanta: tie, odd 1 -> even 2
        (2.0**-126, 0x0080),           # smallest normal
        ((2 - 2**-8) * 2.0**127, 0x7F80),          # midpoint above the max: infinity
        ((2 - 2**-8 - 2**-30) * 2.0**127, 0x7F7F),  # below it: the max finite
        (1e300, 0x7F80),
        (-0.0, 0x8000),
        (0.0, 0x0000),
        (math.inf, 0x7F80),
        (-math.inf, 0xFF80),
    ]
    x = np.array([c[0] for c in cases])
    want = np.array([c[1] for c in cases], np.uint16)
    got = o.f64_to_bf16(x)
    assert np.array_equal(got, want), [(hex(a), hex(b)) for a, b in zip(got, want) if a != b]


def pin_f16_decode_all_patterns(o):
    """Every fp16 pattern decodes to what numpy's float16 widening gives."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = o.f16_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# ------------------------------------------------------------------------------------
# Recurrence pins
# ------------------------------------------------------------------------------------


def pin_zero_state_closed_form(o):
    """S0 = 0, one token: out = scale*beta*(q.k)*v and the state is beta * k (x) v."""
    rng = np.random.default_rng(11)
    B, H, T, Dk, Dv, N = 3, 3, 1, 7, 5, 4
    c = f64_case(rng, B, H, H, T, Dk, Dv, N, zero_state=True)
    out, pool = call_f64(o, c)
    q, k, v, beta, idx = c["query"], c["key"], c["value"], c["beta"], c["ssm_state_indices"]
    s = c["scale_value"]
    for b in range(B):
        for h in range(H):
            qk = float(np.dot(q[b, h, 0], k[b, h, 0]))
            close(out[b, h, 0], s * beta[b, h, 0] * qk * v[b, h, 0], 1e-12, 1e-15)
            close(pool[idx[b], h], beta[b, h, 0] * np.outer(k[b, h, 0], v[b, h, 0]),
                  1e-13, 1e-16)


def pin_recall(o):
    """beta = 1, unit-norm k, no decay: after the update S^T k = v exactly (delta rule).

    With q = k and scale 1 the output therefore equals v as well.
    """
    rng = np.random.default_rng(12)
    B, H, T, Dk, Dv, N = 2, 2, 1, 6, 9, 2
    c = f64_case(rng, B, H, H, T, Dk, Dv, N)
    c["beta"][:] = 1.0
    c["g"][:] = 0.0
    c["gk"][:] = 0.0
    c["query"] = c["key"].copy()
    c["scale_value"] = 1.0
    out, pool = call_f64(o, c)
    for b in range(B):
        for h in range(H):
            S1 = pool[c["ssm_state_indices"][b], h]
            close(S1.T @ c["key"][b, h, 0], c["value"][b, h, 0], 1e-12, 1e-12)
            close(out[b, h, 0], c["value"][b, h, 0], 1e-12, 1e-12)


def pin_chaining(o):
    """Two calls of 4 tokens equal one call of 8 tokens, bit for bit (the state is the
    resumable context: the returned state feeds the next call)."""
    rng = np.random.default_rng(13)
    B, Hq, Hv, T, Dk, Dv, N = 3, 1, 2, 8, 5, 6, 5
    lens = np.array([8, 6, 3], np.int32)
    c = f64_case(rng, B, Hq, Hv, T, Dk, Dv, N, lens=lens)
    out8, pool8 = call_f64(o, c)
    first = dict(c)
    second = dict(c)
    for key_, ax in (("query", 2), ("key", 2), ("value", 2), ("beta", 2), ("g", 2), ("gk", 2)):
        first[key_] = np.ascontiguousarray(np.take(c[key_], range(0, 4), axis=ax))
        second[key_] = np.ascontiguousarray(np.take(c[key_], range(4, 8), axis=ax))
    first["actual_seq_lengths"] = np.minimum(lens, 4).astype(np.int32)
    first["num_accepted_tokens"] = first["actual_seq_lengths"].copy()
    second["actual_seq_lengths"] = np.maximum(lens - 4, 0).astype(np.int32)
    second["num_accepted_tokens"] = second["actual_seq_lengths"].copy()
    out_a, pool_a = call_f64(o, first)
    second["state_pool"] = pool_a
    out_b, pool_b = call_f64(o, second)
    bits_equal(np.concatenate([out_a, out_b], axis=2), out8)
    bits_equal(pool_b, pool8)


def _frac_matrix_form(S0, q, k, v, beta, g, gk, scale, L, n):
    """Exact rational recurrence in matrix form:
    S_t = (I - beta_t k_t k_t^T) D_t S_{t-1} + beta_t k_t v_t^T,  D_t = e^{g_t} diag(e^{gk_t}),
    o_t = S_t^T (scale q_t). The exponentials are the fp64 values of exp, taken exactly."""
    Dk, Dv = len(S0), len(S0[0])
    S = [[Fraction(x) for x in row] for row in S0]
    outs, commit = [], [row[:] for row in S]
    for t in range(L):
        eg = Fraction(math.exp(g[t]))
        d = [eg * Fraction(math.exp(gk[t][i])) for i in range(Dk)]
        DS = [[d[i] * S[i][j] for j in range(Dv)] for i in range(Dk)]
        kf = [Fraction(x) for x in k[t]]
        bt = Fraction(beta[t])
        P = [[(1 if i == r else 0) - bt * kf[i] * kf[r] for r in range(Dk)] for i in range(Dk)]
        S = [[sum(P[i][r] * DS[r][j] for r in range(Dk)) + bt * kf[i] * Fraction(v[t][j])
              for j in range(Dv)] for i in range(Dk)]
        qs = [Fraction(x) * Fraction(scale) for x in q[t]]
        outs.append([sum(S[i][j] * qs[i] for i in range(Dk)) for j in range(Dv)])
        if t + 1 == n:
            commit = [row[:] for row in S]
    return outs, commit


def pin_bruteforce_rational(o):
    """Tiny sizes (D_k=4, D_v=3), up to 8 tokens, varlen, head sharing, an early commit:
    the oracle agrees with an exact rational evaluation of the matrix form."""
    rng = np.random.default_rng(14)
    B, Hq, Hv, T, Dk, Dv, N = 3, 1, 2, 8, 4, 3, 4
    lens = np.array([8, 5, 2], np.int32)
    c = f64_case(rng, B, Hq, Hv, T, Dk, Dv, N, lens=lens)
    c["num_accepted_tokens"] = np.array([8, 3, 0], np.int32)
    out, pool = call_f64(o, c)
    for b in range(B):
        L = int(lens[b])
        n = int(c["num_accepted_tokens"][b])
        slot = int(c["ssm_state_indices"][b])
        for h in range(Hv):
            hq = (h * Hq) // Hv
            outs, commit = _frac_matrix_form(
                c["state_pool"][slot, h].tolist(), c["query"][b, hq].tolist(),
                c["key"][b, hq].tolist(), c["value"][b, h].tolist(), c["beta"][b, h].tolist(),
                c["g"][b, h].tolist(), c["gk"][b, h].tolist(), c["scale_value"], L, n)
            for t in range(L):
                close(out[b, h, t], [float(x) for x in outs[t]], 1e-12, 1e-14)
            assert np.all(out[b, h, L:] == 0.0)
            close(pool[slot, h], [[float(x) for x in row] for row in commit], 1e-12, 1e-14)


def pin_numpy_matrix_form(o):
    """Medium sizes: the oracle agrees with an independent vectorised numpy evaluation of
    the matrix form (projection (I - beta k k^T) applied to the decayed state)."""
    rng = np.random.default_rng(15)
    B, Hq, Hv, T, Dk, Dv, N = 4, 2, 4, 8, 24, 40, 6
    lens = np.array([8, 1, 5, 7], np.int32)
    c = f64_case(rng, B, Hq, Hv, T, Dk, Dv, N, lens=lens)
    out, pool = call_f64(o, c)
    idx = c["ssm_state_indices"]
    rep = Hv // Hq
    q = np.repeat(c["query"], rep, axis=1)
    k = np.repeat(c["key"], rep, axis=1)
    S = c["state_pool"][idx].copy()                      # [B,Hv,Dk,Dv]
    ref = np.zeros((B, Hv, T, Dv))
    eye = np.eye(Dk)
    for t in range(T):
        active = t < lens                                # [B]
        D = np.exp(c["g"][:, :, t])[..., None] * np.exp(c["gk"][:, :, t])   # [B,Hv,Dk]
        kt = k[:, :, t]                                  # [B,Hv,Dk]
        P = eye - c["beta"][:, :, t, None, None] * kt[..., :, None] * kt[..., None, :]
        Snew = P @ (D[..., None] * S) + \
            c["beta"][:, :, t, None, None] * kt[..., :, None] * c["value"][:, :, t, None, :]
        S = np.where(active[:, None, None, None], Snew, S)
        o_t = np.einsum("bhij,bhi->bhj", S, q[:, :, t] * c["scale_value"])
        ref[:, :, t] = np.where(active[:, None, None], o_t, 0.0)
    close(out, ref, 1e-11, 1e-13)
    close(pool[idx], S, 1e-11, 1e-13)


def pin_pure_decay(o):
    """beta = 0: the state only decays, S_t = e^{sum g} diag(e^{sum gk}) S_0 row-wise, and
    o_t = S_t^T (scale q_t) is a plain matrix-vector product (non-square, D_k != D_v)."""
    rng = np.random.default_rng(16)
    B, H, T, Dk, Dv, N = 2, 3, 6, 5, 8, 2
    c = f64_case(rng, B, H, H, T, Dk, Dv, N)
    c["beta"][:] = 0.0
    out, pool = call_f64(o, c)
    for b in range(B):
        slot = c["ssm_state_indices"][b]
        for h in range(H):
            S0 = c["state_pool"][slot, h]
            for t in range(T):
                tot = np.exp(np.sum(c["g"][b, h, :t + 1])) * np.exp(np.sum(c["gk"][b, h, :t + 1], axis=0))
                St = tot[:, None] * S0
                close(out[b, h, t], St.T @ (c["query"][b, h, t] * c["scale_value"]), 1e-12, 1e-14)
            close(pool[slot, h], St, 1e-12, 1e-15)


def pin_linear_attention(o):
    """Zero state, mutually orthogonal one-hot keys, beta = 1, no decay: the memory read is
    always zero and the output is causal linear attention, o_t = scale sum_{s<=t} (q_t.k_s) v_s."""
    rng = np.random.default_rng(17)
    B, H, T, Dk, Dv, N = 2, 2, 6, 8, 5, 2
    c = f64_case(rng, B, H, H, T, Dk, Dv, N, zero_state=True)
    c["beta"][:] = 1.0
    c["g"][:] = 0.0
    c["gk"][:] = 0.0
    for b in range(B):
        for h in range(H):
            perm = rng.permutation(Dk)[:T]
            c["key"][b, h] = np.eye(Dk)[perm]
    out, _ = call_f64(o, c)
    mask = np.tril(np.ones((T, T)))
    for b in range(B):
        for h in range(H):
            Q, K, V = c["query"][b, h], c["key"][b, h], c["value"][b, h]
            ref = c["scale_value"] * ((Q @ K.T) * mask) @ V
            close(out[b, h], ref, 1e-12, 1e-14)


def pin_gqa_expansion(o):
    """Value head h reads query/key head floor(h H_q / H_v): repeating each shared head
    H_v/H_q times and calling with H_q = H_v gives bit-identical results."""
    rng = np.random.default_rng(18)
    B, Hq, Hv, T, Dk, Dv, N = 2, 2, 6, 3, 4, 5, 3
    c = f64_case(rng, B, Hq, Hv, T, Dk, Dv, N)
    out, pool = call_f64(o, c)
    e = dict(c)
    e["query"] = np.repeat(c["query"], Hv // Hq, axis=1)
    e["key"] = np.repeat(c["key"], Hv // Hq, axis=1)
    out2, pool2 = call_f64(o, e)
    bits_equal(out, out2)
    bits_equal(pool, pool2)


def pin_index_semantics(o):
    """Pool gather/scatter and varlen masking, bit for bit:
    untouched slots keep their bytes; permuting batch rows with their indices permutes
    the outputs; NaN in padded tokens never leaks; padded output rows are +0.0; an
    out-of-range slot index skips its row; L = 0 writes the state back unchanged."""
    rng = np.random.default_rng(19)
    B, Hq, Hv, T, Dk, Dv, N = 4, 2, 4, 5, 6, 4, 9
    lens = np.array([5, 2, 0, 3], np.int32)
    c = f64_case(rng, B, Hq, Hv, T, Dk, Dv, N, lens=lens)
    c["state_pool"][:] = 12345.0  # sentinel everywhere
    base = rng.standard_normal((B, Hv, Dk, Dv)) * 0.3
    c["state_pool"][c["ssm_state_indices"]] = base
    out, pool = call_f64(o, c)
    untouched = np.setdiff1d(np.arange(N), c["ssm_state_indices"])
    assert np.all(pool[untouched] == 12345.0)
    for b in range(B):
        assert np.all(out[b, :, lens[b]:] == 0.0) and not np.any(np.signbit(out[b, :, lens[b]:]))
    # L = 0 row: state unchanged
    b0 = 2
    bits_equal(pool[c["ssm_state_indices"][b0]], base[b0])
    # NaN in padding
    d = {kk: (vv.copy() if isinstance(vv, np.ndarray) else vv) for kk, vv in c.items()}
    for b in range(B):
        L = lens[b]
        hq_pad = slice(L, None)
        d["query"][b, :, hq_pad] = np.nan
        d["key"][b, :, hq_pad] = np.nan
        d["value"][b, :, hq_pad] = np.nan
        d["beta"][b, :, hq_pad] = np.nan
        d["g"][b, :, hq_pad] = np.nan
        d["gk"][b, :, hq_pad] = np.nan
    out_n, pool_n = call_f64(o, d)
    bits_equal(out_n, out)
    bits_equal(pool_n, pool)
    # permutation of batch rows
    perm = np.array([2, 0, 3, 1])
    p = {kk: (vv[perm] if isinstance(vv, np.ndarray) and kk != "state_pool" else vv)
         for kk, vv in c.items()}
    out_p, pool_p = call_f64(o, p)
    bits_equal(out_p, out[perm])
    bits_equal(pool_p, pool)
    # out-of-range slot: row skipped, nothing written anywhere
    s = {kk: (vv.copy() if isinstance(vv, np.ndarray) else vv) for kk, vv in c.items()}
    s["ssm_state_indices"][1] = N + 3
    s["ssm_state_indices"][3] = -1
    out_s, pool_s = call_f64(o, s)
    assert np.all(out_s[1] == 0.0) and np.all(out_s[3] == 0.0)
    bits_equal(out_s[[0, 2]], out[[0, 2]])
    for b in (1, 3):
        bits_equal(pool_s[c["ssm_state_indices"][b]], c["state_pool"][c["ssm_state_indices"][b]])


def pin_length_clamp(o):
    """Lengths outside [0, T] act as clamped: a negative length is 0 (nothing read, state
    written back unchanged, zero output), a length above T is T; an accepted count above
    L is L and a negative one is 0."""
    rng = np.random.default_rng(24)
    B, H, T, Dk, Dv, N = 4, 2, 3, 4, 5, 4
    c = f64_case(rng, B, H, H, T, Dk, Dv, N, idx=[0, 1, 2, 3])
    c["actual_seq_lengths"] = np.array([-2, 7, 2, 3], np.int32)
    c["num_accepted_tokens"] = np.array([1, 9, 5, -4], np.int32)
    out, pool = call_f64(o, c)
    ref = dict(c)
    ref["actual_seq_lengths"] = np.array([0, 3, 2, 3], np.int32)
    ref["num_accepted_tokens"] = np.array([0, 3, 2, 0], np.int32)
    out_r, pool_r = call_f64(o, ref)
    bits_equal(out, out_r)
    bits_equal(pool, pool_r)
    assert np.all(out[0] == 0.0)
    bits_equal(pool[0], c["state_pool"][0])
    bits_equal(pool[3], c["state_pool"][3])


def pin_accept_prefix(o):
    """num_accepted_tokens n < L: outputs equal the n = L call, and the committed state
    equals that of a call that stops after n tokens."""
    rng = np.random.default_rng(20)
    B, H, T, Dk, Dv, N = 3, 2, 6, 4, 5, 3
    lens = np.array([6, 4, 5], np.int32)
    c = f64_case(rng, B, H, H, T, Dk, Dv, N, lens=lens)
    out_full, _ = call_f64(o, c)
    a = dict(c)
    a["num_accepted_tokens"] = np.array([2, 0, 5], np.int32)
    out_a, pool_a = call_f64(o, a)
    bits_equal(out_a, out_full)
    s = dict(c)
    s["actual_seq_lengths"] = a["num_accepted_tokens"].copy()
    s["num_accepted_tokens"] = a["num_accepted_tokens"].copy()
    _, pool_s = call_f64(o, s)
    bits_equal(pool_a, pool_s)


def pin_bf16_api_matches_core(o):
    """The bf16-storage entry point is the fp64 core applied to the decoded inputs; its
    state output is the core's state rounded once to bf16."""
    rng = np.random.default_rng(21)
    B, Hq, Hv, T, Dk, Dv, N = 2, 2, 4, 3, 8, 6, 3
    c = f64_case(rng, B, Hq, Hv, T, Dk, Dv, N, lens=[3, 2])
    to_bits = lambda x: torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16).copy()
    qb, kb, vb, bb, sb = (to_bits(c[x]) for x in ("query", "key", "value", "beta", "state_pool"))
    g32 = c["g"].astype(np.float32)
    gk32 = c["gk"].astype(np.float32)
    scale = float(np.float32(c["scale_value"]))
    out_b, pool_b, rows = o.rgdr_bf16(qb, kb, vb, bb, sb, c["actual_seq_lengths"],
                                      c["ssm_state_indices"], g32, gk32,
                                      c["num_accepted_tokens"], scale, want_rows=True)
    dec = lambda x: torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    out_f, pool_f = o.rgdr_f64(dec(qb), dec(kb), dec(vb), dec(bb), dec(sb),
                               c["actual_seq_lengths"], c["ssm_state_indices"],
                               g32.astype(np.float64), gk32.astype(np.float64),
                               c["num_accepted_tokens"], scale)
    bits_equal(out_b, out_f)
    bits_equal(rows, pool_f[c["ssm_state_indices"]])
    assert np.array_equal(pool_b, o.f64_to_bf16(pool_f))


def _bf16_case(rng, B, Hq, Hv, T, Dk, Dv, N, lens, nacc, zero_state=False):
    """An f64 case rounded to bf16 storage (the bf16 entry point's inputs)."""
    c = f64_case(rng, B, Hq, Hv, T, Dk, Dv, N, lens=lens, zero_state=zero_state)
    to_bits = lambda x: torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16).copy()
    return dict(query=to_bits(c["query"]), key=to_bits(c["key"]), value=to_bits(c["value"]),
                beta=to_bits(c["beta"]), state_pool=to_bits(c["state_pool"]),
                actual_seq_lengths=c["actual_seq_lengths"],
                ssm_state_indices=c["ssm_state_indices"], g=c["g"].astype(np.float32),
                gk=c["gk"].astype(np.float32), num_accepted_tokens=np.asarray(nacc, np.int32),
                scale_value=float(np.float32(c["scale_value"])))


def pin_snapshots_prefix(o):
    """The state after token t is the state a call commits when it accepts t + 1 tokens
    (num_accepted_tokens marks the accepted prefix): snapshot (b, t) equals, bit for bit,
    the committed state of the same call with num_accepted_tokens = t + 1, for every t below
    the clamped length; snapshot (b, n - 1) is the call's own committed state; entries past
    the length or of a skipped slot are left unwritten; out and state_out are those of the
    call without snapshots."""
    rng = np.random.default_rng(22)
    B, Hq, Hv, T, Dk, Dv, N = 4, 2, 4, 6, 5, 3, 5
    c = _bf16_case(rng, B, Hq, Hv, T, Dk, Dv, N, lens=[6, 4, 9, 0], nacc=[2, 4, 5, 0])
    c["ssm_state_indices"] = np.array([3, 0, 1, -1], np.int32)
    out, st, rows, snaps = o.rgdr_bf16_snapshots(**c)
    out2, st2, rows2 = o.rgdr_bf16(**c, want_rows=True)
    bits_equal(out, out2)
    assert np.array_equal(st, st2)
    lens = np.clip(c["actual_seq_lengths"], 0, T)
    for b in range(3):
        bits_equal(snaps[b, c["num_accepted_tokens"][b] - 1], rows2[b])
        for t in range(T):
            if t < lens[b]:
                a = dict(c)
                a["num_accepted_tokens"] = np.array([min(t + 1, L) for L in lens], np.int32)
                _, _, r = o.rgdr_bf16(**a, want_rows=True)
                bits_equal(snaps[b, t], r[b])
            else:
                assert np.isnan(snaps[b, t]).all()
    assert np.isnan(snaps[3]).all()  # skipped slot, zero length


def pin_snapshots_zero_state_closed_form(o):
    """S0 = 0, two tokens: the state after token 0 is beta_0 k_0 (x) v_0 whatever the
    decay; after token 1 it is D S_1 + k_1 (x) beta_1 (v_1 - (D S_1)^T k_1) with
    D = diag(exp(g_1) exp(gk_1))."""
    rng = np.random.default_rng(23)
    B, H, T, Dk, Dv, N = 2, 2, 2, 6, 4, 2
    c = _bf16_case(rng, B, H, H, T, Dk, Dv, N, lens=[2, 2], nacc=[2, 2], zero_state=True)
    _, _, _, snaps = o.rgdr_bf16_snapshots(**c)
    dec = lambda x: torch.from_numpy(np.asarray(x).view(np.int16).copy()).view(
        torch.bfloat16).double().numpy()
    k, v, beta = dec(c["key"]), dec(c["value"]), dec(c["beta"])
    g, gk = c["g"].astype(np.float64), c["gk"].astype(np.float64)
    for b in range(B):
        for h in range(H):
            s1 = beta[b, h, 0] * np.outer(k[b, h, 0], v[b, h, 0])
            close(snaps[b, 0, h], s1, 1e-13, 1e-16)
            d = np.exp(g[b, h, 1]) * np.exp(gk[b, h, 1])
            s1d = d[:, None] * s1
            u = beta[b, h, 1] * (v[b, h, 1] - s1d.T @ k[b, h, 1])
            close(snaps[b, 1, h], s1d + np.outer(k[b, h, 1], u), 1e-12, 1e-15)


# ------------------------------------------------------------------------------------
# Gate pins
# ------------------------------------------------------------------------------------


def pin_gate_special_values(o):
    """sigmoid(0) = 1/2 exactly; softplus(0) = ln 2, so decay = decay_scale * ln 2."""
    H = 4
    dt = np.array([0.5, -1.25, 3.0, 0.0], np.float32)
    ds = np.array([-1.0, -2.5, 0.75, 1.0], np.float32)
    a = (-dt)[None, :].copy()                 # a + dt_bias = 0 exactly
    b = np.zeros((1, H), np.float32)
    decay, beta = o.la_gate(a, dt, ds, b)
    assert np.all(beta == 0.5)
    close(decay[0], ds.astype(np.float64) * math.log(2.0), 4e-16, 0.0)


def pin_gate_vs_library(o):
    """decay and beta agree with scipy's logistic function and numpy's log-add-exp
    (softplus(x) = logaddexp(0, x)), broadcasting dt_bias/decay_scale over the last axis."""
    rng = np.random.default_rng(22)
    a = rng.standard_normal((3, 4, 6)).astype(np.float32) * 6
    b = rng.standard_normal((3, 4, 6)).astype(np.float32) * 6
    dt = rng.standard_normal(6).astype(np.float32)
    ds = (-np.exp(rng.uniform(0, np.log(16), 6))).astype(np.float32)
    decay, beta = o.la_gate(a, dt, ds, b)
    x = a.astype(np.float64) + dt.astype(np.float64)
    close(decay, ds.astype(np.float64) * np.logaddexp(0.0, x), 1e-15, 0.0)
    close(beta, expit(b.astype(np.float64)), 1e-15, 0.0)
    assert np.all(np.sign(decay) == np.sign(ds))


def pin_gate_identities(o):
    """softplus(x) - softplus(-x) = x, sigmoid(x) + sigmoid(-x) = 1, and the asymptotes
    softplus(x) -> x (x >> 0), softplus(x) -> e^x (x << 0)."""
    x = np.concatenate([np.linspace(-30, 30, 241), [-40.0, 40.0, 1e-6, -1e-6]]).astype(np.float32)
    one = np.ones(1, np.float32)
    zero = np.zeros(1, np.float32)
    dp, bp = o.la_gate(x[:, None], zero, one, x[:, None])
    dn, bn = o.la_gate(-x[:, None], zero, one, -x[:, None])
    xd = x.astype(np.float64)
    close(dp[:, 0] - dn[:, 0], xd, 1e-14, 1e-15)
    close(bp[:, 0] + bn[:, 0], np.ones_like(xd), 0.0, 4.5e-16)
    big = np.array([[40.0], [-40.0]], np.float32)
    d, _ = o.la_gate(big, zero, one)
    close(d[:, 0], [40.0 + math.exp(-40.0), math.exp(-40.0)], 1e-15, 0.0)


def pin_gate_types_and_shapes(o):
    """T may be fp16 (decoded exactly); rank >= 1 with leading axes folded; beta requires b,
    an unconsumed b is allowed."""
    rng = np.random.default_rng(23)
    a16 = (rng.standard_normal((2, 3, 5)) * 3).astype(np.float16)
    b16 = (rng.standard_normal((2, 3, 5)) * 3).astype(np.float16)
    dt = rng.standard_normal(5).astype(np.float32)
    ds = -np.ones(5, np.float32)
    d16, be16 = o.la_gate(a16, dt, ds, b16)
    d32, be32 = o.la_gate(a16.astype(np.float32), dt, ds, b16.astype(np.float32))
    bits_equal(d16, d32)
    bits_equal(be16, be32)
    d_flat, _ = o.la_gate(a16.reshape(6, 5), dt, ds)
    bits_equal(d_flat.reshape(2, 3, 5), d16)
    d1, _ = o.la_gate(a16[0, 0], dt, ds)     # rank 1
    bits_equal(d1, d16[0, 0])
    d_nb, be_nb = o.la_gate(a16, dt, ds, b16, want_beta=False)
    assert be_nb is None
    bits_equal(d_nb, d16)
    try:
        o.la_gate(a16, dt, ds, None, want_beta=True)
    except RuntimeError:
        pass
    else:
        raise AssertionError("beta without b must fail")


# ------------------------------------------------------------------------------------
# q/k normalisation (the operator's unit-norm precondition on query and key, established
# by the oracle on request)
# ------------------------------------------------------------------------------------


def _raw_qk_case(rng, B, Hq, Hv, T, Dk, Dv, N):
    c = f64_case(rng, B, Hq, Hv, T, Dk, Dv, N)
    # raw projections: magnitudes far from 1, different per token and head
    c["query"] = c["query"] * rng.uniform(0.2, 7.0, (B, Hq, T, 1))
    c["key"] = c["key"] * rng.uniform(0.2, 7.0, (B, Hq, T, 1))
    return c


def pin_normalize_matches_prenormalized(o):
    """normalize_qk on raw q, k equals the plain call on q / ||q||, k / ||k|| computed by
    numpy (its own norm routine), with head sharing, varlen and a scale != 1."""
    rng = np.random.default_rng(24)
    c = _raw_qk_case(rng, 3, 2, 4, 3, 9, 5, 5)
    c["actual_seq_lengths"] = np.array([3, 1, 2], np.int32)
    c["num_accepted_tokens"] = c["actual_seq_lengths"].copy()
    c["scale_value"] = 0.37
    args = (c["value"], c["beta"], c["state_pool"], c["actual_seq_lengths"],
            c["ssm_state_indices"], c["g"], c["gk"], c["num_accepted_tokens"], c["scale_value"])
    out_n, pool_n = o.rgdr_f64(c["query"], c["key"], *args, normalize_qk=True)
    qn = c["query"] / np.linalg.norm(c["query"], axis=-1, keepdims=True)
    kn = c["key"] / np.linalg.norm(c["key"], axis=-1, keepdims=True)
    out_p, pool_p = o.rgdr_f64(qn, kn, *args)
    close(out_n, out_p, 1e-12, 1e-14)
    close(pool_n, pool_p, 1e-12, 1e-14)
    # and the flag matters: without it the raw magnitudes change the result
    out_raw, _ = o.rgdr_f64(c["query"], c["key"], *args)
    assert np.abs(out_raw - out_p).max() > 1e-3


def pin_normalize_scale_invariance(o):
    """With normalize_qk, multiplying each q and k head vector by its own positive power of
    two changes nothing, bit for bit (the norm scales by exactly that factor)."""
    rng = np.random.default_rng(25)
    c = _raw_qk_case(rng, 2, 2, 2, 2, 8, 6, 3)
    base = o.rgdr_f64(c["query"], c["key"], c["value"], c["beta"], c["state_pool"],
                      c["actual_seq_lengths"], c["ssm_state_indices"], c["g"], c["gk"],
                      c["num_accepted_tokens"], c["scale_value"], normalize_qk=True)
    fq = 2.0 ** rng.integers(-6, 7, (2, 2, 2, 1))
    fk = 2.0 ** rng.integers(-6, 7, (2, 2, 2, 1))
    scaled = o.rgdr_f64(c["query"] * fq, c["key"] * fk, c["value"], c["beta"],
                        c["state_pool"], c["actual_seq_lengths"], c["ssm_state_indices"],
                        c["g"], c["gk"], c["num_accepted_tokens"], c["scale_value"],
                        normalize_qk=True)
    bits_equal(base[0], scaled[0])
    bits_equal(base[1], scaled[1])


def pin_normalize_zero_vectors(o):
    """A zero query gives a zero output row; a zero key leaves the state at its decayed
    value (no update). Both without NaN, and equal to the call without normalisation,
    which sees the same zero vectors."""
    rng = np.random.default_rng(26)
    c = _raw_qk_case(rng, 2, 1, 1, 2, 6, 4, 2)
    c["query"][0, 0, 1] = 0.0
    c["key"][1, 0, 0] = 0.0
    c["query"][1, 0, 0] = 0.0
    out_n, pool_n = o.rgdr_f64(c["query"], c["key"], c["value"], c["beta"], c["state_pool"],
                               c["actual_seq_lengths"], c["ssm_state_indices"], c["g"],
                               c["gk"], c["num_accepted_tokens"], c["scale_value"],
                               normalize_qk=True)
    assert np.all(np.isfinite(out_n)) and np.all(np.isfinite(pool_n))
    assert np.all(out_n[0, 0, 1] == 0.0) and np.all(out_n[1, 0, 0] == 0.0)
    qn = c["query"].copy()
    kn = c["key"].copy()
    for arr in (qn, kn):
        nrm = np.linalg.norm(arr, axis=-1, keepdims=True)
        np.divide(arr, nrm, out=arr, where=nrm > 0)
    out_p, pool_p = o.rgdr_f64(qn, kn, c["value"], c["beta"], c["state_pool"],
                               c["actual_seq_lengths"], c["ssm_state_indices"], c["g"],
                               c["gk"], c["num_accepted_tokens"], c["scale_value"])
    close(out_n, out_p, 1e-12, 1e-14)
    close(pool_n, pool_p, 1e-12, 1e-14)


def pin_normalize_bf16_api(o):
    """The bf16 entry point with normalize_qk is the fp64 core with normalize_qk on the
    decoded inputs (unrounded out, state rounded once)."""
    rng = np.random.default_rng(27)
    B, Hq, Hv, T, Dk, Dv, N = 2, 1, 2, 2, 8, 8, 3
    c = _raw_qk_case(rng, B, Hq, Hv, T, Dk, Dv, N)
    enc = lambda x: o.f64_to_bf16(x)
    q16, k16, v16 = enc(c["query"]), enc(c["key"]), enc(c["value"])
    b16, p16 = enc(c["beta"]), enc(c["state_pool"])
    g32 = c["g"].astype(np.float32)
    gk32 = c["gk"].astype(np.float32)
    scale = float(np.float32(c["scale_value"]))
    out, pool, _ = o.rgdr_bf16(q16, k16, v16, b16, p16, c["actual_seq_lengths"],
                               c["ssm_state_indices"], g32, gk32, c["num_accepted_tokens"],
                               scale, normalize_qk=True)
    dec = o.bf16_to_f64
    out_c, pool_c = o.rgdr_f64(dec(q16), dec(k16), dec(v16), dec(b16), dec(p16),
                               c["actual_seq_lengths"], c["ssm_state_indices"],
                               g32.astype(np.float64), gk32.astype(np.float64),
                               c["num_accepted_tokens"], scale, normalize_qk=True)
    bits_equal(out, out_c)
    bits_equal(pool, enc(pool_c))


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
