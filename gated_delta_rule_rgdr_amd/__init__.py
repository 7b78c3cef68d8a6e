"""Gated-delta-rule decode for AMD MI355X (gfx950): Python binding of ``include/rgdr.h``.

Argument marshalling only: every step of the computation runs in the HIP kernels of
``librgdr.so``; PyTorch supplies device memory and the current stream. There is no CPU
fallback: if the library is missing, the first call of any binding function raises
``ImportError``.

* ``rgdr_decode``  -- the recurrent gated-delta-rule decode step (MindSpore Lite API page
  "lite_boost.ops.recurrent_gated_delta_rule"), in place on a bf16 state pool.
* ``recurrent_gated_delta_rule`` -- the page's functional form: returns ``(out, state_out)``
  and leaves ``state`` untouched.
* ``rgdr_decode_snapshots`` -- ``rgdr_decode`` that also returns the state after every
  token (speculative decoding: the state of each candidate accepted prefix).
* ``rgdr_decode_gated`` -- the decode step with the gate front end fused in: takes the raw
  gate projections instead of g and beta.
* ``rgdr_prefill`` / ``rgdr_prefill_gated`` -- the same recurrence over long sequences
  (T up to 65536; the page's notes hand prefill to a chunk-level operator), same arguments.
* ``la_gate`` -- the gate front end (README "com.microsoft.LinearAttentionGate").
* ``rgdr_validate`` -- synchronous check of the index arrays.

A non-OK status from the library raises ``RuntimeError`` (the page's error behaviour).

With ``RGDR_VALIDATE=1`` in the environment (read at import; ``VALIDATE`` holds it), every
decode call first checks its index arrays with ``rgdr_validate``: a synchronous copy to the
host, for debugging only (it cannot run under graph capture). A bad length, count or slot
then raises ``RuntimeError`` instead of being clamped or skipped by the kernel.
"""
import ctypes as C
import os

import torch

__all__ = ["rgdr_decode", "rgdr_decode_snapshots", "rgdr_decode_gated",
           "rgdr_decode_gated_snapshots", "rgdr_prefill", "rgdr_prefill_gated",
           "rgdr_prefill_ws", "rgdr_prefill_gated_ws", "rgdr_prefill_workspace_size",
           "rgdr_prefill_noalloc",
           "recurrent_gated_delta_rule", "la_gate",
           "rgdr_validate", "VALIDATE",
           "rgdr_validate_host", "status_string", "library", "LIB_PATH", "RGDR_F32",
           "RGDR_F16", "RGDR_BF16"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librgdr.so")

RGDR_F32, RGDR_F16, RGDR_BF16 = 0, 1, 2
RGDR_NORMALIZE_QK = 1  # option bit of rgdr_decode_gated
NORMALIZE_QK = RGDR_NORMALIZE_QK
_DTYPE_CODE = {torch.float32: RGDR_F32, torch.float16: RGDR_F16, torch.bfloat16: RGDR_BF16}

_lib = None
VALIDATE = os.environ.get("RGDR_VALIDATE", "") == "1"


def library():
    """Load ``librgdr.so`` (built by ``gated_delta_rule_rgdr_amd/build.py``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m gated_delta_rule_rgdr_amd.build` "
            "(there is no fallback path)")
    lib = C.CDLL(LIB_PATH)
    vp, i32, i64, f32 = C.c_void_p, C.c_int32, C.c_int64, C.c_float
    lib.rgdr_decode.restype = C.c_int
    lib.rgdr_decode.argtypes = [vp] * 10 + [f32] + [i32] * 7 + [vp, vp, vp]
    lib.rgdr_decode_snapshots.restype = C.c_int
    lib.rgdr_decode_snapshots.argtypes = [vp] * 10 + [f32] + [i32] * 7 + [vp, vp, vp, vp]
    lib.rgdr_decode_gated.restype = C.c_int
    lib.rgdr_decode_gated.argtypes = ([vp] * 7 + [C.c_int] + [vp] * 5 + [f32] + [i32] * 7
                                      + [vp] * 2 + [C.c_uint32, vp])
    lib.rgdr_decode_gated_snapshots.restype = C.c_int
    lib.rgdr_decode_gated_snapshots.argtypes = ([vp] * 7 + [C.c_int] + [vp] * 5 + [f32]
                                                + [i32] * 7 + [vp] * 3 + [C.c_uint32, vp])
    lib.rgdr_prefill.restype = C.c_int
    lib.rgdr_prefill.argtypes = lib.rgdr_decode.argtypes
    lib.rgdr_prefill_gated.restype = C.c_int
    lib.rgdr_prefill_gated.argtypes = lib.rgdr_decode_gated.argtypes
    lib.rgdr_prefill_noalloc.restype = C.c_int
    lib.rgdr_prefill_noalloc.argtypes = lib.rgdr_decode.argtypes
    lib.rgdr_prefill_workspace_size.restype = C.c_int
    lib.rgdr_prefill_workspace_size.argtypes = [i32] * 5 + [C.POINTER(C.c_size_t)]
    lib.rgdr_prefill_ws.restype = C.c_int
    lib.rgdr_prefill_ws.argtypes = [vp] * 10 + [f32] + [i32] * 7 + [vp, vp, vp, C.c_size_t, vp]
    lib.rgdr_prefill_gated_ws.restype = C.c_int
    lib.rgdr_prefill_gated_ws.argtypes = ([vp] * 7 + [C.c_int] + [vp] * 5 + [f32] + [i32] * 7
                                          + [vp] * 2 + [C.c_uint32, vp, C.c_size_t, vp])
    lib.la_gate.restype = C.c_int
    lib.la_gate.argtypes = [vp, vp, vp, vp, C.c_int, i64, i32, vp, C.c_int, vp, C.c_int, vp]
    lib.rgdr_validate.restype = C.c_int
    lib.rgdr_validate.argtypes = [vp, vp, vp, i32, i32, i32, vp]
    lib.rgdr_validate_host.restype = C.c_int
    lib.rgdr_validate_host.argtypes = [vp, vp, vp, i32, i32, i32]
    lib.rgdr_status_string.restype = C.c_char_p
    lib.rgdr_status_string.argtypes = [C.c_int]
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return library().rgdr_status_string(code).decode()


def _check(code: int, what: str):
    if code != 0:
        raise RuntimeError(f"{what}: {status_string(code)}")


def _stream_handle(stream, device):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return s.cuda_stream


def _same_device(ref, **tensors):
    """Every tensor on ref's GPU: the library launches on the current device and takes the
    pointers as that device's addresses."""
    for name, t in tensors.items():
        if t is not None and t.device != ref.device:
            raise RuntimeError(f"{name} is on {t.device}, expected {ref.device}")


def _validate_indices(lens, idx, nacc, T, N):
    code = rgdr_validate(lens, idx, nacc, T, N)
    _check(code, "index arrays (RGDR_VALIDATE)")


def _dtype_code(dtype, name):
    if dtype not in _DTYPE_CODE:
        raise RuntimeError(f"{name}: unsupported dtype {dtype}")
    return _DTYPE_CODE[dtype]


def _dev(t, name, dtype, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise RuntimeError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise RuntimeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise RuntimeError(f"{name} must have {ndim} dimensions, got {t.dim()}")
    if not t.is_contiguous():
        raise RuntimeError(f"{name} must be contiguous")
    return t


def rgdr_decode(query, key, value, beta, state_pool, actual_seq_lengths, ssm_state_indices,
                g, gk, num_accepted_tokens, scale=1.0, *, out=None, state_out=None,
                stream=None):
    """One decode step (T <= 8); returns ``(out, state_out)``.

    Shapes (page parameter list; the state is a slot pool): query/key bf16
    ``[B,H_q,T,D_k]``, value bf16 ``[B,H_v,T,D_v]``, beta bf16 ``[B,H_v,T]``, state_pool bf16
    ``[N_slots,H_v,D_k,D_v]``, g fp32 ``[B,H_v,T]``, gk fp32 ``[B,H_v,T,D_k]``, the three index
    arrays int32 ``[B]``. ``state_out`` defaults to ``state_pool`` (in-place update of the
    named slots); ``out`` is allocated if not given.
    """
    return _plain_call("rgdr_decode", query, key, value, beta, state_pool, actual_seq_lengths,
                       ssm_state_indices, g, gk, num_accepted_tokens, scale, out, state_out,
                       stream)


def rgdr_decode_snapshots(query, key, value, beta, state_pool, actual_seq_lengths,
                          ssm_state_indices, g, gk, num_accepted_tokens, scale=1.0, *,
                          out=None, state_out=None, state_snapshots=None, stream=None):
    """``rgdr_decode`` that also stores the state after every token; returns
    ``(out, state_out, state_snapshots)``.

    ``state_snapshots``: bf16 ``[B, T, H_v, D_k, D_v]``, allocated (uninitialised) if not
    given. Entry ``[b, t]`` is written for ``t`` below the clamped length of entry ``b`` when
    its slot is valid, and holds the state after its first ``t + 1`` tokens; other entries
    keep what the buffer held.
    """
    state_snapshots = _snapshot_buffer(query, value, state_pool, state_snapshots)
    out, state_out = _plain_call("rgdr_decode_snapshots", query, key, value, beta, state_pool,
                                 actual_seq_lengths, ssm_state_indices, g, gk,
                                 num_accepted_tokens, scale, out, state_out, stream,
                                 extra={"state_snapshots": state_snapshots})
    return out, state_out, state_snapshots


def _snapshot_buffer(query, value, state_pool, state_snapshots):
    """The per-token state buffer of a snapshot call: checked, or allocated uninitialised."""
    if not isinstance(query, torch.Tensor) or not isinstance(value, torch.Tensor) \
            or not isinstance(state_pool, torch.Tensor):
        raise TypeError("query, value and state_pool must be torch.Tensor")
    if query.dim() != 4 or value.dim() != 4 or state_pool.dim() != 4:
        raise RuntimeError("query, value and state_pool must have 4 dimensions")
    B, _, T, Dk = query.shape
    Hv, Dv = value.shape[1], value.shape[3]
    if state_snapshots is None:
        return torch.empty((B, T, Hv, Dk, Dv), dtype=torch.bfloat16, device=query.device)
    _dev(state_snapshots, "state_snapshots", torch.bfloat16, 5)
    if tuple(state_snapshots.shape) != (B, T, Hv, Dk, Dv):
        raise RuntimeError("state_snapshots must be [B, T, H_v, D_k, D_v]")
    return state_snapshots


def rgdr_prefill(query, key, value, beta, state_pool, actual_seq_lengths, ssm_state_indices,
                 g, gk, num_accepted_tokens, scale=1.0, *, out=None, state_out=None,
                 stream=None):
    """The same recurrence over long sequences (T up to 65536, the prefill counterpart the
    page's notes name); arguments and results as ``rgdr_decode``."""
    return _plain_call("rgdr_prefill", query, key, value, beta, state_pool, actual_seq_lengths,
                       ssm_state_indices, g, gk, num_accepted_tokens, scale, out, state_out,
                       stream)


def rgdr_prefill_workspace_size(B, H_v, T, D_k, D_v, device=None):
    """Bytes of workspace ``rgdr_prefill_ws`` uses for a call of these sizes on ``device``
    (0: such a call runs in one pass and needs none)."""
    lib = library()
    n = C.c_size_t(0)
    with torch.cuda.device(device if device is not None else torch.cuda.current_device()):
        rc = lib.rgdr_prefill_workspace_size(B, H_v, T, D_k, D_v, C.byref(n))
    _check(rc, "rgdr_prefill_workspace_size")
    return n.value


def _workspace(query, value, state_pool, workspace):
    """The caller's workspace (a uint8 CUDA tensor), or one allocated for the call."""
    if workspace is None:
        B, _, T, Dk = query.shape
        Hv, Dv = value.shape[1], value.shape[3]
        nbytes = rgdr_prefill_workspace_size(B, Hv, T, Dk, Dv, query.device)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=query.device)
    if workspace.dtype != torch.uint8 or not workspace.is_cuda or not workspace.is_contiguous():
        raise RuntimeError("workspace must be a contiguous uint8 CUDA tensor")
    return workspace


def rgdr_prefill_ws(query, key, value, beta, state_pool, actual_seq_lengths, ssm_state_indices,
                    g, gk, num_accepted_tokens, scale=1.0, *, workspace=None, out=None,
                    state_out=None, stream=None):
    """``rgdr_prefill`` with a workspace (a uint8 CUDA tensor of at least
    ``rgdr_prefill_workspace_size`` bytes; allocated for the call when None). Calls of few
    sequences then evaluate all segments of a sequence at once."""
    workspace = _workspace(query, value, state_pool, workspace)
    return _plain_call("rgdr_prefill_ws", query, key, value, beta, state_pool,
                       actual_seq_lengths, ssm_state_indices, g, gk, num_accepted_tokens, scale,
                       out, state_out, stream, workspace=workspace)


def rgdr_prefill_noalloc(query, key, value, beta, state_pool, actual_seq_lengths,
                         ssm_state_indices, g, gk, num_accepted_tokens, scale=1.0, *, out=None,
                         state_out=None, stream=None):
    """``rgdr_prefill_ws`` whose workspace is the library's fixed 128 MiB device array: the
    call allocates no device memory itself (``out`` and ``state_out`` are still allocated
    here when not given). Calls that overlap on one device race on that array."""
    return _plain_call("rgdr_prefill_noalloc", query, key, value, beta, state_pool,
                       actual_seq_lengths, ssm_state_indices, g, gk, num_accepted_tokens, scale,
                       out, state_out, stream)


def _plain_call(fn, query, key, value, beta, state_pool, actual_seq_lengths, ssm_state_indices,
                g, gk, num_accepted_tokens, scale, out, state_out, stream, extra=None,
                workspace=None):
    extra = extra or {}  # further output buffers, passed after state_out in this order
    lib = library()
    _dev(query, "query", torch.bfloat16, 4)
    B, Hq, T, Dk = query.shape
    _dev(key, "key", torch.bfloat16, 4)
    _dev(value, "value", torch.bfloat16, 4)
    _dev(beta, "beta", torch.bfloat16, 3)
    _dev(state_pool, "state_pool", torch.bfloat16, 4)
    _dev(g, "g", torch.float32, 3)
    _dev(gk, "gk", torch.float32, 4)
    for nm, t in (("actual_seq_lengths", actual_seq_lengths),
                  ("ssm_state_indices", ssm_state_indices),
                  ("num_accepted_tokens", num_accepted_tokens)):
        _dev(t, nm, torch.int32, 1)
        if t.shape[0] != B:
            raise RuntimeError(f"{nm} must have shape [{B}]")
    Hv, Dv = value.shape[1], value.shape[3]
    N = state_pool.shape[0]
    if tuple(key.shape) != (B, Hq, T, Dk) or tuple(value.shape) != (B, Hv, T, Dv) \
            or tuple(beta.shape) != (B, Hv, T) or tuple(g.shape) != (B, Hv, T) \
            or tuple(gk.shape) != (B, Hv, T, Dk) or tuple(state_pool.shape) != (N, Hv, Dk, Dv):
        raise RuntimeError(f"{fn}: inconsistent shapes")
    if out is None:
        out = torch.empty((B, Hv, T, Dv), dtype=torch.bfloat16, device=query.device)
    else:
        _dev(out, "out", torch.bfloat16, 4)
        if tuple(out.shape) != (B, Hv, T, Dv):
            raise RuntimeError("out must be [B, H_v, T, D_v]")
    if state_out is None:
        state_out = state_pool
    else:
        _dev(state_out, "state_out", torch.bfloat16, 4)
        if state_out.shape != state_pool.shape:
            raise RuntimeError("state_out must have the pool's shape")
    _same_device(query, key=key, value=value, beta=beta, state_pool=state_pool,
                 actual_seq_lengths=actual_seq_lengths, ssm_state_indices=ssm_state_indices,
                 g=g, gk=gk, num_accepted_tokens=num_accepted_tokens, out=out,
                 state_out=state_out, **extra)
    if VALIDATE:
        _validate_indices(actual_seq_lengths, ssm_state_indices, num_accepted_tokens, T, N)
    with torch.cuda.device(query.device):
        rc = getattr(lib, fn)(query.data_ptr(), key.data_ptr(), value.data_ptr(),
                              beta.data_ptr(), state_pool.data_ptr(),
                              actual_seq_lengths.data_ptr(), ssm_state_indices.data_ptr(),
                              g.data_ptr(), gk.data_ptr(), num_accepted_tokens.data_ptr(),
                              float(scale), B, Hq, Hv, T, Dk, Dv, N, out.data_ptr(),
                              state_out.data_ptr(), *[t.data_ptr() for t in extra.values()],
                              *_ws_args(workspace, query), _stream_handle(stream, query.device))
    _check(rc, fn)
    return out, state_out


def _ws_args(workspace, ref):
    if workspace is None:
        return ()
    _same_device(ref, workspace=workspace)
    return (workspace.data_ptr(), workspace.numel())


def rgdr_decode_gated(query, key, value, a, b, dt_bias, decay_scale, state_pool,
                      actual_seq_lengths, ssm_state_indices, gk, num_accepted_tokens, scale=1.0,
                      *, normalize_qk=False, out=None, state_out=None, stream=None):
    """One decode step with the gate fused in; returns ``(out, state_out)``.

    ``a``, ``b``: raw gate projections ``[B, T, H_v]`` (float32 or float16, head axis last);
    ``dt_bias``, ``decay_scale``: float32 ``[H_v]``. ``g = decay_scale * softplus(a + dt_bias)``
    and ``beta = sigmoid(b)`` are computed in the kernel in fp32. With ``normalize_qk`` the
    kernel also divides each token's query and key head vector by its L2 norm (the
    operator's unit-norm precondition), so raw projections may be passed. Other arguments as
    ``rgdr_decode`` (which takes g and beta instead).
    """
    return _gated_call("rgdr_decode_gated", query, key, value, a, b, dt_bias, decay_scale,
                       state_pool, actual_seq_lengths, ssm_state_indices, gk,
                       num_accepted_tokens, scale, normalize_qk, out, state_out, stream)


def rgdr_decode_gated_snapshots(query, key, value, a, b, dt_bias, decay_scale, state_pool,
                                actual_seq_lengths, ssm_state_indices, gk, num_accepted_tokens,
                                scale=1.0, *, normalize_qk=False, out=None, state_out=None,
                                state_snapshots=None, stream=None):
    """``rgdr_decode_gated`` that also stores the state after every token, as
    ``rgdr_decode_snapshots`` extends ``rgdr_decode``; returns
    ``(out, state_out, state_snapshots)`` with the buffer as described there."""
    state_snapshots = _snapshot_buffer(query, value, state_pool, state_snapshots)
    out, state_out = _gated_call("rgdr_decode_gated_snapshots", query, key, value, a, b,
                                 dt_bias, decay_scale, state_pool, actual_seq_lengths,
                                 ssm_state_indices, gk, num_accepted_tokens, scale,
                                 normalize_qk, out, state_out, stream,
                                 extra={"state_snapshots": state_snapshots})
    return out, state_out, state_snapshots


def rgdr_prefill_gated(query, key, value, a, b, dt_bias, decay_scale, state_pool,
                       actual_seq_lengths, ssm_state_indices, gk, num_accepted_tokens,
                       scale=1.0, *, normalize_qk=False, out=None, state_out=None,
                       stream=None):
    """``rgdr_prefill`` with the gate fused in, as ``rgdr_decode_gated`` extends
    ``rgdr_decode``."""
    return _gated_call("rgdr_prefill_gated", query, key, value, a, b, dt_bias, decay_scale,
                       state_pool, actual_seq_lengths, ssm_state_indices, gk,
                       num_accepted_tokens, scale, normalize_qk, out, state_out, stream)


def rgdr_prefill_gated_ws(query, key, value, a, b, dt_bias, decay_scale, state_pool,
                          actual_seq_lengths, ssm_state_indices, gk, num_accepted_tokens,
                          scale=1.0, *, normalize_qk=False, workspace=None, out=None,
                          state_out=None, stream=None):
    """``rgdr_prefill_gated`` with a workspace, as ``rgdr_prefill_ws`` extends
    ``rgdr_prefill``."""
    workspace = _workspace(query, value, state_pool, workspace)
    return _gated_call("rgdr_prefill_gated_ws", query, key, value, a, b, dt_bias, decay_scale,
                       state_pool, actual_seq_lengths, ssm_state_indices, gk,
                       num_accepted_tokens, scale, normalize_qk, out, state_out, stream,
                       workspace=workspace)


def _gated_call(fn, query, key, value, a, b, dt_bias, decay_scale, state_pool,
                actual_seq_lengths, ssm_state_indices, gk, num_accepted_tokens, scale,
                normalize_qk, out, state_out, stream, extra=None, workspace=None):
    extra = extra or {}  # further output buffers, passed after state_out in this order
    lib = library()
    _dev(query, "query", torch.bfloat16, 4)
    B, Hq, T, Dk = query.shape
    _dev(key, "key", torch.bfloat16, 4)
    _dev(value, "value", torch.bfloat16, 4)
    _dev(state_pool, "state_pool", torch.bfloat16, 4)
    _dev(gk, "gk", torch.float32, 4)
    if a.dtype not in (torch.float32, torch.float16):
        raise RuntimeError("gate projections must be float32 or float16")
    _dev(a, "a", a.dtype, 3)
    _dev(b, "b", a.dtype, 3)
    _dev(dt_bias, "dt_bias", torch.float32, 1)
    _dev(decay_scale, "decay_scale", torch.float32, 1)
    for nm, t in (("actual_seq_lengths", actual_seq_lengths),
                  ("ssm_state_indices", ssm_state_indices),
                  ("num_accepted_tokens", num_accepted_tokens)):
        _dev(t, nm, torch.int32, 1)
        if t.shape[0] != B:
            raise RuntimeError(f"{nm} must have shape [{B}]")
    Hv, Dv = value.shape[1], value.shape[3]
    N = state_pool.shape[0]
    if tuple(key.shape) != (B, Hq, T, Dk) or tuple(value.shape) != (B, Hv, T, Dv) \
            or tuple(a.shape) != (B, T, Hv) or tuple(b.shape) != (B, T, Hv) \
            or tuple(gk.shape) != (B, Hv, T, Dk) or tuple(state_pool.shape) != (N, Hv, Dk, Dv) \
            or dt_bias.shape[0] != Hv or decay_scale.shape[0] != Hv:
        raise RuntimeError(f"{fn}: inconsistent shapes")
    if out is None:
        out = torch.empty((B, Hv, T, Dv), dtype=torch.bfloat16, device=query.device)
    else:
        _dev(out, "out", torch.bfloat16, 4)
        if tuple(out.shape) != (B, Hv, T, Dv):
            raise RuntimeError("out must be [B, H_v, T, D_v]")
    if state_out is None:
        state_out = state_pool
    else:
        _dev(state_out, "state_out", torch.bfloat16, 4)
        if state_out.shape != state_pool.shape:
            raise RuntimeError("state_out must have the pool's shape")
    _same_device(query, key=key, value=value, a=a, b=b, dt_bias=dt_bias,
                 decay_scale=decay_scale, state_pool=state_pool,
                 actual_seq_lengths=actual_seq_lengths, ssm_state_indices=ssm_state_indices,
                 gk=gk, num_accepted_tokens=num_accepted_tokens, out=out, state_out=state_out,
                 **extra)
    if VALIDATE:
        _validate_indices(actual_seq_lengths, ssm_state_indices, num_accepted_tokens, T, N)
    with torch.cuda.device(query.device):
        rc = getattr(lib, fn)(query.data_ptr(), key.data_ptr(), value.data_ptr(),
                              a.data_ptr(), b.data_ptr(), dt_bias.data_ptr(),
                              decay_scale.data_ptr(), _DTYPE_CODE[a.dtype],
                              state_pool.data_ptr(), actual_seq_lengths.data_ptr(),
                              ssm_state_indices.data_ptr(), gk.data_ptr(),
                              num_accepted_tokens.data_ptr(), float(scale), B, Hq, Hv, T,
                              Dk, Dv, N, out.data_ptr(), state_out.data_ptr(),
                              *[t.data_ptr() for t in extra.values()],
                              NORMALIZE_QK if normalize_qk else 0,
                              *_ws_args(workspace, query), _stream_handle(stream, query.device))
    _check(rc, fn)
    return out, state_out


def recurrent_gated_delta_rule(query, key, value, beta, state, actual_seq_lengths,
                               ssm_state_indices, g, gk, num_accepted_tokens, scale_value=1.0):
    """The page's functional signature: ``(out, state_out)`` with ``state`` left unchanged.

    ``state_out`` starts as a device copy of ``state``; the kernel then writes every slot a
    batch entry names. Feed it back as ``state`` for the next step.
    """
    state_out = torch.empty_like(state)
    state_out.copy_(state)
    return rgdr_decode(query, key, value, beta, state_out, actual_seq_lengths,
                       ssm_state_indices, g, gk, num_accepted_tokens, scale_value)


def la_gate(a, dt_bias, decay_scale, b=None, *, want_beta=None, decay_dtype=None,
            beta_dtype=None, decay_out=None, beta_out=None, stream=None):
    """``decay = decay_scale * softplus(a + dt_bias)``, ``beta = sigmoid(b)`` (fp32 math).

    ``a``/``b``: float32 or float16, any rank >= 1, head axis last. ``dt_bias`` and
    ``decay_scale``: float32 ``[H]``. ``decay`` has ``decay_dtype`` (default: a's dtype);
    ``beta`` (computed when ``want_beta``, default ``b is not None``) has ``beta_dtype``
    (default a's dtype; ``torch.bfloat16`` feeds ``rgdr_decode`` directly).
    """
    lib = library()
    if a.dtype not in (torch.float32, torch.float16):
        raise RuntimeError("a must be float32 or float16")
    _dev(a, "a", a.dtype)
    if a.dim() < 1:
        raise RuntimeError("a must have rank >= 1")
    H = a.shape[-1]
    _dev(dt_bias, "dt_bias", torch.float32, 1)
    _dev(decay_scale, "decay_scale", torch.float32, 1)
    if dt_bias.shape[0] != H or decay_scale.shape[0] != H:
        raise RuntimeError("dt_bias and decay_scale must be [H]")
    if want_beta is None:
        want_beta = b is not None
    if b is not None:
        _dev(b, "b", a.dtype)
        if b.shape != a.shape:
            raise RuntimeError("b must have a's shape")
    decay_dtype = decay_dtype or a.dtype
    if decay_out is None:
        decay_out = torch.empty(a.shape, dtype=decay_dtype, device=a.device)
    _dev(decay_out, "decay_out", decay_dtype)
    beta_t = None
    if want_beta:
        beta_dtype = beta_dtype or a.dtype
        beta_t = beta_out if beta_out is not None else torch.empty(a.shape, dtype=beta_dtype,
                                                                   device=a.device)
        _dev(beta_t, "beta_out", beta_dtype)
    n_rows = a.numel() // H if H else 0
    _same_device(a, dt_bias=dt_bias, decay_scale=decay_scale, b=b, decay_out=decay_out,
                 beta_out=beta_t)
    with torch.cuda.device(a.device):
        rc = lib.la_gate(a.data_ptr(), dt_bias.data_ptr(), decay_scale.data_ptr(),
                         b.data_ptr() if b is not None else None, _DTYPE_CODE[a.dtype], n_rows,
                         H, decay_out.data_ptr(), _dtype_code(decay_dtype, "decay_out"),
                         beta_t.data_ptr() if beta_t is not None else None,
                         _dtype_code(beta_dtype, "beta_out") if beta_t is not None else 0,
                         _stream_handle(stream, a.device))
    _check(rc, "la_gate")
    return decay_out, beta_t


def rgdr_validate(actual_seq_lengths, ssm_state_indices, num_accepted_tokens, T, N_slots,
                  stream=None):
    """Synchronous check of device index arrays; returns the status code (0 = valid)."""
    lib = library()
    B = actual_seq_lengths.shape[0]
    for nm, t in (("actual_seq_lengths", actual_seq_lengths),
                  ("ssm_state_indices", ssm_state_indices),
                  ("num_accepted_tokens", num_accepted_tokens)):
        _dev(t, nm, torch.int32, 1)
        if t.shape[0] != B:
            raise RuntimeError(f"{nm} must have shape [{B}]")
    _same_device(actual_seq_lengths, ssm_state_indices=ssm_state_indices,
                 num_accepted_tokens=num_accepted_tokens)
    with torch.cuda.device(actual_seq_lengths.device):
        return lib.rgdr_validate(actual_seq_lengths.data_ptr(), ssm_state_indices.data_ptr(),
                                 num_accepted_tokens.data_ptr(), B, T, N_slots,
                                 _stream_handle(stream, actual_seq_lengths.device))


def rgdr_validate_host(actual_seq_lengths, ssm_state_indices, num_accepted_tokens, T, N_slots):
    """The same checks on host (CPU) int32 tensors; returns the status code."""
    lib = library()
    ts = [torch.as_tensor(x, dtype=torch.int32).contiguous()
          for x in (actual_seq_lengths, ssm_state_indices, num_accepted_tokens)]
    B = ts[0].shape[0]
    return lib.rgdr_validate_host(ts[0].data_ptr(), ts[1].data_ptr(), ts[2].data_ptr(),
                                  B, T, N_slots)
