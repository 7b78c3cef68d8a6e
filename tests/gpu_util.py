"""Helpers for the GPU parity tests: upload seeded inputs, run the HIP path through the
C ABI binding, run the oracle on the same bytes, compare.

Tolerance for bf16 outputs produced from fp32 arithmetic, against the UNROUNDED fp64
oracle value: |gpu - ref| <= 2e-2 + 2e-2 |ref| per element. Indexing, padding and
untouched slots are compared bit for bit.
"""
import copy
import sys

import numpy as np
import torch

import oracle
import workloads

ATOL = 2e-2
RTOL = 2e-2


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bits_to_dev(x: np.ndarray) -> torch.Tensor:
    """uint16 bf16 patterns -> a bf16 CUDA tensor holding the same bytes."""
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()


def dev_to_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_dev_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def upload(inp):
    """Device tensors for one ``workloads.Inputs``."""
    d = dict(
        query=bits_to_dev(inp.query), key=bits_to_dev(inp.key), value=bits_to_dev(inp.value),
        beta=bits_to_dev(inp.beta), state=bits_to_dev(inp.state),
        actual_seq_lengths=torch.from_numpy(inp.actual_seq_lengths).cuda(),
        ssm_state_indices=torch.from_numpy(inp.ssm_state_indices).cuda(),
        g=torch.from_numpy(inp.g).cuda(), gk=torch.from_numpy(inp.gk).cuda(),
        num_accepted_tokens=torch.from_numpy(inp.num_accepted_tokens).cuda(),
    )
    return d


def gpu_decode(inp, d=None, *, inplace=False, fn="rgdr_decode"):
    """Run rgdr_decode (or another entry with its arguments, such as rgdr_prefill) on the
    GPU; returns (out bf16 tensor, state_out bf16 tensor)."""
    import gated_delta_rule_rgdr_amd as rg
    d = d or upload(inp)
    pool = d["state"] if inplace else d["state"].clone()
    out, st = getattr(rg, fn)(d["query"], d["key"], d["value"], d["beta"], pool,
                              d["actual_seq_lengths"], d["ssm_state_indices"], d["g"], d["gk"],
                              d["num_accepted_tokens"], inp.scale)
    torch.cuda.synchronize()
    return out, st


def gpu_prefill(inp, d=None, *, inplace=False):
    """Run rgdr_prefill on the GPU; returns (out, state_out) as gpu_decode."""
    return gpu_decode(inp, d, inplace=inplace, fn="rgdr_prefill")


def oracle_decode(inp, **over):
    a = dict(query=inp.query, key=inp.key, value=inp.value, beta=inp.beta,
             state_pool=inp.state, actual_seq_lengths=inp.actual_seq_lengths,
             ssm_state_indices=inp.ssm_state_indices, g=inp.g, gk=inp.gk,
             num_accepted_tokens=inp.num_accepted_tokens, scale_value=inp.scale)
    a.update(over)
    return oracle.rgdr_bf16(**a, want_rows=True)


def assert_tol(got: np.ndarray, ref: np.ndarray, what: str, atol=ATOL, rtol=RTOL):
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if ref.size == 0:  # nothing served (every length 0, or every slot skipped)
        say(f"  {what}: n=0")
        return
    fin = np.isfinite(got)
    assert fin.all(), f"{what}: {np.count_nonzero(~fin)} non-finite values"
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref)
    bad = err > bound
    rel = err / np.maximum(np.abs(ref), 1e-30)
    say(f"  {what}: n={ref.size} max_abs_err={err.max():.3e} "
        f"max_rel_err(|ref|>1e-3)={rel[np.abs(ref) > 1e-3].max() if (np.abs(ref) > 1e-3).any() else 0:.3e}")
    assert not bad.any(), (f"{what}: {np.count_nonzero(bad)} of {ref.size} elements beyond "
                           f"{atol} + {rtol}|ref|; worst err {err[bad].max():.3e}")


def check_decode(inp, out_t, state_t, ref, label):
    """Compare one GPU decode against the oracle's (out, state_out, rows)."""
    out_ref, pool_ref_bits, rows = ref
    out = bf16_dev_to_f64(out_t)
    B, Hv, T = inp.B, inp.Hv, inp.T
    lens = np.clip(inp.actual_seq_lengths, 0, T)
    valid = (inp.ssm_state_indices >= 0) & (inp.ssm_state_indices < inp.N_slots)
    mask = np.zeros((B, Hv, T), bool)
    for b in range(B):
        if valid[b]:
            mask[b, :, :lens[b]] = True
    assert_tol(out[mask], out_ref[mask], f"{label} out")
    # padded rows and skipped entries: exactly +0.0 (bit pattern 0)
    out_bits = dev_to_bits(out_t)
    assert np.all(out_bits[~mask] == 0), f"{label}: padded output rows are not +0.0"
    pool = bf16_dev_to_f64(state_t)
    pool_bits = dev_to_bits(state_t)
    named = inp.ssm_state_indices[valid]
    assert_tol(pool[named], rows[valid], f"{label} state_out")
    untouched = np.setdiff1d(np.arange(inp.N_slots), named)
    assert np.array_equal(pool_bits[untouched], inp.state[untouched]), \
        f"{label}: slots no entry names were modified"
    assert np.array_equal(pool_ref_bits[untouched], inp.state[untouched])


# ---- the fused gate: oracle chain (fp64 gate, then the fp64 core, no rounding between) ----


def gate_tensors(inp, dtype=np.float32):
    return (torch.from_numpy(inp.gate_a.astype(dtype)).cuda(),
            torch.from_numpy(inp.gate_b.astype(dtype)).cuda(),
            torch.from_numpy(inp.dt_bias).cuda(), torch.from_numpy(inp.decay_scale).cuda())


def gpu_gated(rg, inp, dtype=np.float32, d=None, normalize_qk=False, fn="rgdr_decode_gated"):
    """Run a fused-gate entry (rgdr_decode_gated or rgdr_prefill_gated) out of place."""
    d = d or upload(inp)
    a, b, dt, ds = gate_tensors(inp, dtype)
    pool = d["state"].clone()
    out, st = getattr(rg, fn)(d["query"], d["key"], d["value"], a, b, dt, ds, pool,
                              d["actual_seq_lengths"], d["ssm_state_indices"], d["gk"],
                              d["num_accepted_tokens"], inp.scale, normalize_qk=normalize_qk)
    torch.cuda.synchronize()
    return out, st


def oracle_gated(inp, entries=None, dtype=np.float32, normalize_qk=False):
    """Oracle chain for the batch entries `entries` (all when None): returns fp64 out
    [n, H_v, T, D_v] and each entry's committed state [n, H_v, D_k, D_v] (NaN if skipped)."""
    sel = np.arange(inp.B) if entries is None else np.asarray(entries)
    g64, b64 = oracle.la_gate(inp.gate_a[sel].astype(dtype), inp.dt_bias, inp.decay_scale,
                              inp.gate_b[sel].astype(dtype))
    g64 = np.ascontiguousarray(g64.transpose(0, 2, 1))  # [n, H_v, T]
    b64 = np.ascontiguousarray(b64.transpose(0, 2, 1))
    idx = inp.ssm_state_indices[sel]
    valid = (idx >= 0) & (idx < inp.N_slots)
    pool_small = oracle.bf16_to_f64(inp.state[idx[valid]])
    idx_small = np.full(len(sel), -1, np.int32)
    idx_small[valid] = np.arange(int(valid.sum()), dtype=np.int32)
    if pool_small.shape[0] == 0:
        pool_small = np.zeros((1, inp.Hv, inp.Dk, inp.Dv))
    out, pool_out = oracle.rgdr_f64(
        oracle.bf16_to_f64(inp.query[sel]), oracle.bf16_to_f64(inp.key[sel]),
        oracle.bf16_to_f64(inp.value[sel]), b64, pool_small, inp.actual_seq_lengths[sel],
        idx_small, g64, inp.gk[sel].astype(np.float64), inp.num_accepted_tokens[sel],
        float(np.float32(inp.scale)), normalize_qk=normalize_qk)
    rows = np.full((len(sel), inp.Hv, inp.Dk, inp.Dv), np.nan)
    rows[valid] = pool_out[idx_small[valid]]
    return out, rows


def check_gated(inp, out_t, st_t, ref, label, entries=None):
    out_ref, rows = ref
    sel = np.arange(inp.B) if entries is None else np.asarray(entries)
    out = bf16_dev_to_f64(out_t)[sel]
    lens = np.clip(inp.actual_seq_lengths[sel], 0, inp.T)
    idx = inp.ssm_state_indices[sel]
    valid = (idx >= 0) & (idx < inp.N_slots)
    mask = np.zeros((len(sel), inp.Hv, inp.T), bool)
    for i in range(len(sel)):
        if valid[i]:
            mask[i, :, :lens[i]] = True
    assert_tol(out[mask], out_ref[mask], f"{label} out")
    assert np.all(dev_to_bits(out_t)[sel][~mask] == 0), f"{label}: padded rows not +0.0"
    pool = bf16_dev_to_f64(st_t)
    assert_tol(pool[idx[valid]], rows[valid], f"{label} state_out")
    if entries is None:
        untouched = np.setdiff1d(np.arange(inp.N_slots), idx[valid])
        assert np.array_equal(dev_to_bits(st_t)[untouched], inp.state[untouched])


def raw_qk(inp, seed):
    """Replace the case's unit-norm q and k by raw projections: each head vector scaled by
    its own factor in [0.05, 20] (bf16 again), so the unit-norm precondition does not hold."""
    rng = np.random.default_rng(seed)
    for name in ("query", "key"):
        x = oracle.bf16_to_f64(getattr(inp, name))
        f = rng.uniform(0.05, 20.0, x.shape[:-1] + (1,))
        setattr(inp, name, workloads.to_bf16_bits(x * f))
    return inp


# ---- per-token state snapshots ----

SENTINEL = np.uint16(0xFFED)  # a quiet NaN whose payload no rounding produces


def _sentinel_buffer(inp):
    return torch.full((inp.B, inp.T, inp.Hv, inp.Dk, inp.Dv), int(SENTINEL.view(np.int16)),
                      dtype=torch.int16, device="cuda").view(torch.bfloat16)


def _check_snapshot_buffer(inp, snap, st, o_snaps, label):
    """Every written entry within the bar of the oracle's state after that token, every other
    entry still the sentinel, and the entry after the accepted prefix equal to the committed
    slot's bytes."""
    got = bf16_dev_to_f64(snap)
    bits = dev_to_bits(snap)
    pool_bits = dev_to_bits(st)
    lens = np.clip(inp.actual_seq_lengths, 0, inp.T)
    valid = (inp.ssm_state_indices >= 0) & (inp.ssm_state_indices < inp.N_slots)
    written = np.zeros((inp.B, inp.T), bool)
    for b in range(inp.B):
        if valid[b]:
            written[b, :lens[b]] = True
    assert np.isfinite(o_snaps[written]).all()
    assert_tol(got[written], o_snaps[written], f"{label} snapshots")
    assert np.all(bits[~written] == SENTINEL), f"{label}: unwritten snapshot entries changed"
    n_acc = np.clip(inp.num_accepted_tokens, 0, lens)
    for b in range(inp.B):
        if valid[b] and n_acc[b] >= 1:
            assert np.array_equal(bits[b, n_acc[b] - 1], pool_bits[inp.ssm_state_indices[b]]), \
                f"{label}: entry {b}: snapshot {n_acc[b] - 1} is not the committed state"
    say(f"  {label}: {int(written.sum())} snapshot entries written")


def check_snapshots(rg, inp, label):
    """Run rgdr_decode_snapshots on a sentinel-filled buffer and compare out, the committed
    slots and every snapshot entry with the oracle; unwritten entries must keep the
    sentinel, and the snapshot after the accepted prefix must be the committed slot's bytes."""
    d = upload(inp)
    pool = d["state"].clone()
    snap = _sentinel_buffer(inp)
    out, st, snap_r = rg.rgdr_decode_snapshots(
        d["query"], d["key"], d["value"], d["beta"], pool, d["actual_seq_lengths"],
        d["ssm_state_indices"], d["g"], d["gk"], d["num_accepted_tokens"], inp.scale,
        state_snapshots=snap)
    torch.cuda.synchronize()
    assert snap_r.data_ptr() == snap.data_ptr()
    o_out, o_pool, o_rows, o_snaps = oracle.rgdr_bf16_snapshots(
        inp.query, inp.key, inp.value, inp.beta, inp.state, inp.actual_seq_lengths,
        inp.ssm_state_indices, inp.g, inp.gk, inp.num_accepted_tokens, inp.scale)
    check_decode(inp, out, st, (o_out, o_pool, o_rows), label)
    lens = np.clip(inp.actual_seq_lengths, 0, inp.T)
    valid = (inp.ssm_state_indices >= 0) & (inp.ssm_state_indices < inp.N_slots)
    written = np.zeros((inp.B, inp.T), bool)
    for b in range(inp.B):
        if valid[b]:
            written[b, :lens[b]] = True
    assert np.array_equal(np.isfinite(o_snaps).all(axis=(2, 3, 4)), written)
    _check_snapshot_buffer(inp, snap, st, o_snaps, label)


def check_gated_snapshots(rg, inp, label, dtype=np.float32, normalize_qk=False):
    """Run rgdr_decode_gated_snapshots on a sentinel-filled buffer. out and the committed
    slots are compared with the oracle chain (la_gate, then the recurrence) as for
    rgdr_decode_gated. Snapshot t of an entry is compared with the state that the same chain
    commits when t + 1 tokens are accepted, which is that snapshot's definition. Buffer
    checks as check_snapshots."""
    d = upload(inp)
    a, b, dt, ds = gate_tensors(inp, dtype)
    pool = d["state"].clone()
    snap = _sentinel_buffer(inp)
    out, st, snap_r = rg.rgdr_decode_gated_snapshots(
        d["query"], d["key"], d["value"], a, b, dt, ds, pool, d["actual_seq_lengths"],
        d["ssm_state_indices"], d["gk"], d["num_accepted_tokens"], inp.scale,
        normalize_qk=normalize_qk, state_snapshots=snap)
    torch.cuda.synchronize()
    assert snap_r.data_ptr() == snap.data_ptr()
    check_gated(inp, out, st, oracle_gated(inp, dtype=dtype, normalize_qk=normalize_qk), label)
    o_snaps = np.full((inp.B, inp.T, inp.Hv, inp.Dk, inp.Dv), np.nan)
    for t in range(inp.T):
        prefix = copy.copy(inp)
        prefix.num_accepted_tokens = np.full(inp.B, t + 1, np.int32)
        o_snaps[:, t] = oracle_gated(prefix, dtype=dtype, normalize_qk=normalize_qk)[1]
    _check_snapshot_buffer(inp, snap, st, o_snaps, label)
