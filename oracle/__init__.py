"""fp64 CPU oracle for the recurrent gated-delta-rule decode step and its gate front end.

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import this package. The GPU library never imports it and shares
no code with it; this package never imports the GPU library.

It wraps ``rgdr_oracle.c`` (plain C, fp64, built by ``oracle/build.py``), which follows:

* MindSpore Lite API page "lite_boost.ops.recurrent_gated_delta_rule": the algorithm
  section (decay, memory read, delta update, output; token by token), the parameter
  list and the returns;
* kernel README "com.microsoft.LinearAttentionGate": Description, Inputs, Outputs and
  Type constraints.

Every function is pinned by ``tests/test_oracle_pins.py`` (closed forms, invariants,
special cases that reduce to textbook operations, brute force in exact rationals).

Arrays are numpy: bf16 tensors are ``uint16`` bit patterns, fp16 gate inputs are
``float16``, index arrays ``int32``.
"""
import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "librgdr_oracle.so")
TY_F32 = 1
TY_F16 = 3

_u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")


def _bind(lib):
    lib.oracle_bf16_to_f64.restype = C.c_double
    lib.oracle_bf16_to_f64.argtypes = [C.c_uint16]
    lib.oracle_f16_to_f64.restype = C.c_double
    lib.oracle_f16_to_f64.argtypes = [C.c_uint16]
    lib.oracle_f64_to_bf16.restype = C.c_uint16
    lib.oracle_f64_to_bf16.argtypes = [C.c_double]
    for name, (ti, to) in {"oracle_bf16_to_f64_array": (_u16p, _f64p),
                           "oracle_f16_to_f64_array": (_u16p, _f64p),
                           "oracle_f64_to_bf16_array": (_f64p, _u16p)}.items():
        fn = getattr(lib, name)
        fn.restype = None
        fn.argtypes = [ti, to, C.c_longlong]
    ints = [C.c_int] * 7
    lib.oracle_rgdr_bf16.restype = C.c_int
    lib.oracle_rgdr_bf16.argtypes = (
        [_u16p, _u16p, _u16p, _u16p, _u16p, _i32p, _i32p, _f32p, _f32p, _i32p, C.c_float]
        + ints + [_f64p, _u16p, C.c_void_p, C.c_int])
    lib.oracle_rgdr_bf16_snapshots.restype = C.c_int
    lib.oracle_rgdr_bf16_snapshots.argtypes = (
        [_u16p, _u16p, _u16p, _u16p, _u16p, _i32p, _i32p, _f32p, _f32p, _i32p, C.c_float]
        + ints + [_f64p, _u16p, C.c_void_p, _f64p])
    lib.oracle_rgdr_f64.restype = C.c_int
    lib.oracle_rgdr_f64.argtypes = (
        [_f64p, _f64p, _f64p, _f64p, _f64p, _i32p, _i32p, _f64p, _f64p, _i32p, C.c_double]
        + ints + [_f64p, _f64p, C.c_int])
    lib.oracle_la_gate.restype = C.c_int
    lib.oracle_la_gate.argtypes = [C.c_void_p, _f32p, _f32p, C.c_void_p, C.c_int,
                                   C.c_longlong, C.c_int, _f64p, C.c_void_p]
    return lib


def _dims(query, value, state_pool):
    B, Hq, T, Dk = query.shape
    Bv, Hv, Tv, Dv = value.shape
    N_slots = state_pool.shape[0]
    assert Bv == B and Tv == T, "value must be [B, H_v, T, D_v]"
    assert state_pool.shape == (N_slots, Hv, Dk, Dv), "state must be [N_slots, H_v, D_k, D_v]"
    return B, Hq, Hv, T, Dk, Dv, N_slots


class Oracle:
    """The oracle's functions bound to one build of ``rgdr_oracle.c``.

    The module-level functions use the default build (``librgdr_oracle.so``); tests may
    bind another build of the same source with ``Oracle(path)``.
    """

    def __init__(self, path=None):
        path = path or _LIB_PATH
        if path == _LIB_PATH and not os.path.exists(path):
            from . import build as _build
            _build.build()
        self.path = path
        self.lib = _bind(C.CDLL(path))

    # --- bf16 / fp16 codec (the oracle's own; pinned against library conversions) ---

    def bf16_to_f64(self, bits):
        """Exact decode of bf16 bit patterns (uint16 array) to fp64."""
        bits = np.ascontiguousarray(bits, dtype=np.uint16)
        out = np.empty(bits.shape, np.float64)
        self.lib.oracle_bf16_to_f64_array(bits.reshape(-1), out.reshape(-1), bits.size)
        return out

    def f16_to_f64(self, bits):
        """Exact decode of fp16 bit patterns (uint16 array) to fp64."""
        bits = np.ascontiguousarray(bits, dtype=np.uint16)
        out = np.empty(bits.shape, np.float64)
        self.lib.oracle_f16_to_f64_array(bits.reshape(-1), out.reshape(-1), bits.size)
        return out

    def f64_to_bf16(self, x):
        """Round fp64 values to bf16 (nearest, ties to even, one rounding); uint16 bits."""
        x = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty(x.shape, np.uint16)
        self.lib.oracle_f64_to_bf16_array(x.reshape(-1), out.reshape(-1), x.size)
        return out

    # --- the recurrence ---

    def rgdr_bf16(self, query, key, value, beta, state_pool, actual_seq_lengths,
                  ssm_state_indices, g, gk, num_accepted_tokens, scale_value=1.0, *,
                  want_rows=False, normalize_qk=False):
        """The decode operator with bf16 storage: returns ``(out, state_out, rows)``.

        With ``normalize_qk`` each token's query and key head vector is first divided by
        its L2 norm (the operator's unit-norm precondition established by the oracle).

        ``out`` is fp64 ``[B, H_v, T, D_v]`` (unrounded); ``state_out`` a bf16 copy of the
        pool in which every named slot holds its committed state (others unchanged);
        ``rows`` (if ``want_rows``) the unrounded committed state of each batch entry,
        fp64 ``[B, H_v, D_k, D_v]`` (NaN for a skipped entry).
        """
        B, Hq, Hv, T, Dk, Dv, N_slots = _dims(query, value, state_pool)
        out = np.full((B, Hv, T, Dv), np.nan)
        state_out = np.array(state_pool, dtype=np.uint16, copy=True, order="C")
        rows = np.full((B, Hv, Dk, Dv), np.nan) if want_rows else None
        rc = self.lib.oracle_rgdr_bf16(
            np.ascontiguousarray(query, np.uint16), np.ascontiguousarray(key, np.uint16),
            np.ascontiguousarray(value, np.uint16), np.ascontiguousarray(beta, np.uint16),
            np.ascontiguousarray(state_pool, np.uint16),
            np.ascontiguousarray(actual_seq_lengths, np.int32),
            np.ascontiguousarray(ssm_state_indices, np.int32),
            np.ascontiguousarray(g, np.float32), np.ascontiguousarray(gk, np.float32),
            np.ascontiguousarray(num_accepted_tokens, np.int32),
            float(np.float32(scale_value)), B, Hq, Hv, T, Dk, Dv, N_slots, out, state_out,
            rows.ctypes.data if rows is not None else None, int(bool(normalize_qk)))
        if rc != 0:
            raise RuntimeError(f"oracle_rgdr_bf16 failed with code {rc}")
        return out, state_out, rows

    def rgdr_bf16_snapshots(self, query, key, value, beta, state_pool, actual_seq_lengths,
                            ssm_state_indices, g, gk, num_accepted_tokens, scale_value=1.0):
        """``rgdr_bf16`` plus the state after every token: returns
        ``(out, state_out, rows, snaps)`` with ``snaps`` fp64 ``[B, T, H_v, D_k, D_v]``, entry
        (b, t) the unrounded state after the first t + 1 tokens of entry b, for t below its
        clamped length and a valid slot (NaN elsewhere)."""
        B, Hq, Hv, T, Dk, Dv, N_slots = _dims(query, value, state_pool)
        out = np.full((B, Hv, T, Dv), np.nan)
        state_out = np.array(state_pool, dtype=np.uint16, copy=True, order="C")
        rows = np.full((B, Hv, Dk, Dv), np.nan)
        snaps = np.full((B, T, Hv, Dk, Dv), np.nan)
        rc = self.lib.oracle_rgdr_bf16_snapshots(
            np.ascontiguousarray(query, np.uint16), np.ascontiguousarray(key, np.uint16),
            np.ascontiguousarray(value, np.uint16), np.ascontiguousarray(beta, np.uint16),
            np.ascontiguousarray(state_pool, np.uint16),
            np.ascontiguousarray(actual_seq_lengths, np.int32),
            np.ascontiguousarray(ssm_state_indices, np.int32),
            np.ascontiguousarray(g, np.float32), np.ascontiguousarray(gk, np.float32),
            np.ascontiguousarray(num_accepted_tokens, np.int32),
            float(np.float32(scale_value)), B, Hq, Hv, T, Dk, Dv, N_slots, out, state_out,
            rows.ctypes.data, snaps)
        if rc != 0:
            raise RuntimeError(f"oracle_rgdr_bf16_snapshots failed with code {rc}")
        return out, state_out, rows, snaps

    def rgdr_f64(self, query, key, value, beta, state_pool, actual_seq_lengths,
                 ssm_state_indices, g, gk, num_accepted_tokens, scale_value=1.0, *,
                 normalize_qk=False):
        """The same recurrence with fp64 inputs and an fp64 pool, no rounding at all.

        Returns ``(out, state_out)``: fp64 ``[B, H_v, T, D_v]`` and the fp64 pool.
        """
        B, Hq, Hv, T, Dk, Dv, N_slots = _dims(query, value, state_pool)
        out = np.full((B, Hv, T, Dv), np.nan)
        state_out = np.array(state_pool, dtype=np.float64, copy=True, order="C")
        f = lambda x: np.ascontiguousarray(x, np.float64)
        i = lambda x: np.ascontiguousarray(x, np.int32)
        rc = self.lib.oracle_rgdr_f64(f(query), f(key), f(value), f(beta), f(state_pool),
                                      i(actual_seq_lengths), i(ssm_state_indices), f(g),
                                      f(gk), i(num_accepted_tokens), float(scale_value),
                                      B, Hq, Hv, T, Dk, Dv, N_slots, out, state_out,
                                      int(bool(normalize_qk)))
        if rc != 0:
            raise RuntimeError(f"oracle_rgdr_f64 failed with code {rc}")
        return out, state_out

    # --- gate front end ---

    def la_gate(self, a, dt_bias, decay_scale, b=None, want_beta=None):
        """``decay = decay_scale * softplus(a + dt_bias)``, ``beta = sigmoid(b)``, fp64.

        ``a`` (and ``b``) are float32 or float16 arrays of any rank >= 1 whose last axis
        is the head axis; ``dt_bias`` and ``decay_scale`` are float32 ``[H]``. ``beta`` is
        computed when ``want_beta`` (default: ``b is not None``); it requires ``b``.
        """
        a = np.asarray(a)
        if a.dtype not in (np.float32, np.float16):
            raise TypeError("a must be float32 or float16")
        ty = TY_F32 if a.dtype == np.float32 else TY_F16
        H = a.shape[-1]
        n_rows = a.size // H if H else 0
        if want_beta is None:
            want_beta = b is not None
        a_c = np.ascontiguousarray(a)
        b_c = None
        if b is not None:
            b_c = np.ascontiguousarray(b, dtype=a.dtype)
            assert b_c.shape == a.shape
        decay = np.full(a.shape, np.nan)
        beta = np.full(a.shape, np.nan) if want_beta else None
        rc = self.lib.oracle_la_gate(
            a_c.ctypes.data, np.ascontiguousarray(dt_bias, np.float32),
            np.ascontiguousarray(decay_scale, np.float32),
            b_c.ctypes.data if b_c is not None else None, ty, n_rows, H, decay,
            beta.ctypes.data if beta is not None else None)
        if rc != 0:
            raise RuntimeError(f"oracle_la_gate failed with code {rc}")
        return decay, beta


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def bf16_to_f64(bits):
    return default().bf16_to_f64(bits)


def f16_to_f64(bits):
    return default().f16_to_f64(bits)


def f64_to_bf16(x):
    return default().f64_to_bf16(x)


def rgdr_bf16(*args, **kw):
    return default().rgdr_bf16(*args, **kw)


def rgdr_bf16_snapshots(*args, **kw):
    return default().rgdr_bf16_snapshots(*args, **kw)


def rgdr_f64(*args, **kw):
    return default().rgdr_f64(*args, **kw)


def la_gate(*args, **kw):
    return default().la_gate(*args, **kw)
