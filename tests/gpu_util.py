"""Helpers for the GPU parity tests: upload seeded inputs, run the HIP path through the
C ABI binding, run the oracle on the same bytes, compare.

Tolerance for bf16 outputs produced from fp32 arithmetic, against the UNROUNDED fp64
oracle value: |gpu - ref| <= 2e-2 + 2e-2 |ref| per element. Indexing, padding and
untouched slots are compared bit for bit.
"""
import sys

import numpy as np
import torch

import oracle

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


def gpu_decode(inp, d=None, *, inplace=False):
    """Run rgdr_decode on the GPU; returns (out bf16 tensor, state_out bf16 tensor)."""
    import gated_delta_rule_rgdr_amd as rg
    d = d or upload(inp)
    pool = d["state"] if inplace else d["state"].clone()
    out, st = rg.rgdr_decode(d["query"], d["key"], d["value"], d["beta"], pool,
                             d["actual_seq_lengths"], d["ssm_state_indices"], d["g"], d["gk"],
                             d["num_accepted_tokens"], inp.scale)
    torch.cuda.synchronize()
    return out, st


def oracle_decode(inp, **over):
    a = dict(query=inp.query, key=inp.key, value=inp.value, beta=inp.beta,
             state_pool=inp.state, actual_seq_lengths=inp.actual_seq_lengths,
             ssm_state_indices=inp.ssm_state_indices, g=inp.g, gk=inp.gk,
             num_accepted_tokens=inp.num_accepted_tokens, scale_value=inp.scale)
    a.update(over)
    return oracle.rgdr_bf16(**a, want_rows=True)


def assert_tol(got: np.ndarray, ref: np.ndarray, what: str, atol=ATOL, rtol=RTOL):
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
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
