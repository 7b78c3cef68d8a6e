"""Seeded synthetic inputs for the gated-delta-rule decode and long-sequence workloads.

This module only draws inputs. It holds none of the method's arithmetic, and both the
GPU tests/bench and the CPU oracle receive the identical bytes it returns.

Workloads (shapes from the MindSpore Lite page "lite_boost.ops.recurrent_gated_delta_rule",
parameter list and example; gate inputs from the "com.microsoft.LinearAttentionGate"
README, Inputs table):

  0  tiny decode:            B=1,  H_q=H_v=4,  T=1, D_k=D_v=64,  1 zero slot
  1  single sequence:        B=1,  H_q=H_v=64, T=1, D_k=64, D_v=512 (the page example shape)
  2  batched GQA decode:     B=64, H_q=16, H_v=32, T=1, D=128, 256 slots, 64 distinct used
  3  speculative / varlen:   B=32, H_q=H_v=32, T=8, D=128, lengths U{1..8}, 64 slots
  4  gate + recurrence:      B=256, H_q=16, H_v=32, T=1, D=128, 512 slots, raw gate inputs
  5  chunked prefill:        B=16, H_q=16, H_v=32, T=1024, D=128, 32 slots, 16 distinct used
                             (the long-sequence counterpart the page's notes name; the pages
                             give no prefill shape, so this takes workload 2's heads and head
                             size with 1024-token prompts)
  6  chunked prefill:        B=4, H_q=H_v=64, T=1024, D_k=64, D_v=512, 8 slots, 4 distinct
                             (the same reading at the page example's head size, with the
                             step bytes of workload 5)
  7  single-prompt prefill:  B=1, H_q=16, H_v=32, T=8192, D=128, 2 slots, 1 used (workload
                             5's heads with one long prompt: too few (entry, head) pairs to
                             fill the device, the case the segmented form serves)

Recipe (one numpy ``default_rng(1000 + id)`` stream, drawn in this order):
  q, k ~ N(0,1) fp64, L2-normalised along D_k per (b, head, t), stored as bf16;
  v ~ N(0,1) -> bf16; beta = sigmoid(N(0,1)) -> bf16; g = -softplus(N(0,1)) fp32;
  gk = -U(1e-3, gk_hi) fp32 (gk_hi = 0.1, 0.05 for workload 4);
  state ~ 0.05 * N(0,1) (fp32 draws) -> bf16 (workload 0: zeros, no draw);
  slot indices; lengths (workload 3 only); then the gate inputs (workload 4 only):
  a, b ~ N(0,1) fp32 [B,T,H_v]; dt_bias ~ N(0,1) fp32 [H_v]; A_log ~ U(0, ln 16) fp32
  [H_v]; decay_scale = -exp(A_log) in fp32 (the gated-DeltaNet choice the README names).

With ``gate_inputs=True`` a workload without its own gate inputs (0-3, 5-7) also gets raw gate
projections, drawn after everything else: a, b ~ N(0,1) fp32 [B,T,H_v], dt_bias = 0 and
decay_scale = -1. The gate then yields g = -softplus(a) and beta = sigmoid(b), the same
distributions the recipe draws g and beta from, so the whole path (gate, then decode)
runs at that workload's shape.

bf16 values are stored as uint16 bit patterns. The conversion to bf16 uses torch's CPU
cast (round to nearest even); it only shapes the inputs.
"""
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch
from scipy.special import expit

WORKLOADS = {
    0: dict(B=1, Hq=4, Hv=4, T=1, Dk=64, Dv=64, N_slots=1),
    1: dict(B=1, Hq=64, Hv=64, T=1, Dk=64, Dv=512, N_slots=1),
    2: dict(B=64, Hq=16, Hv=32, T=1, Dk=128, Dv=128, N_slots=256),
    3: dict(B=32, Hq=32, Hv=32, T=8, Dk=128, Dv=128, N_slots=64),
    4: dict(B=256, Hq=16, Hv=32, T=1, Dk=128, Dv=128, N_slots=512),
    5: dict(B=16, Hq=16, Hv=32, T=1024, Dk=128, Dv=128, N_slots=32),
    6: dict(B=4, Hq=64, Hv=64, T=1024, Dk=64, Dv=512, N_slots=8),
    7: dict(B=1, Hq=16, Hv=32, T=8192, Dk=128, Dv=128, N_slots=2),
}

WORKLOAD_NAMES = {
    0: "tiny decode B=1 H=4 T=1 D=64",
    1: "single-sequence decode B=1 H=64 T=1 Dk=64 Dv=512",
    2: "batched GQA decode B=64 Hq=16 Hv=32 T=1 D=128",
    3: "varlen speculative decode B=32 H=32 T=8 D=128",
    4: "gate + decode B=256 Hq=16 Hv=32 T=1 D=128",
    5: "chunked prefill B=16 Hq=16 Hv=32 T=1024 D=128",
    6: "chunked prefill B=4 H=64 T=1024 Dk=64 Dv=512",
    7: "single-prompt prefill B=1 Hq=16 Hv=32 T=8192 D=128",
}


def to_bf16_bits(x) -> np.ndarray:
    """float array -> bf16 bit patterns (uint16), via torch's round-to-nearest-even cast."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _unit_rows(rng, shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


@dataclass
class Inputs:
    B: int
    Hq: int
    Hv: int
    T: int
    Dk: int
    Dv: int
    N_slots: int
    query: np.ndarray        # bf16 bits [B,Hq,T,Dk]
    key: np.ndarray          # bf16 bits [B,Hq,T,Dk]
    value: np.ndarray        # bf16 bits [B,Hv,T,Dv]
    beta: np.ndarray         # bf16 bits [B,Hv,T]
    g: np.ndarray            # fp32 [B,Hv,T]
    gk: np.ndarray           # fp32 [B,Hv,T,Dk]
    state: np.ndarray        # bf16 bits [N_slots,Hv,Dk,Dv]
    ssm_state_indices: np.ndarray   # int32 [B]
    actual_seq_lengths: np.ndarray  # int32 [B]
    num_accepted_tokens: np.ndarray  # int32 [B]
    scale: float
    # gate inputs (workload 4 / gated cases)
    gate_a: Optional[np.ndarray] = None        # fp32 [B,T,Hv]
    gate_b: Optional[np.ndarray] = None        # fp32 [B,T,Hv]
    dt_bias: Optional[np.ndarray] = None       # fp32 [Hv]
    decay_scale: Optional[np.ndarray] = None   # fp32 [Hv]
    extra: dict = field(default_factory=dict)

    def decode_args(self):
        """Positional arguments in the operator's order (page parameter list)."""
        return (self.query, self.key, self.value, self.beta, self.state,
                self.actual_seq_lengths, self.ssm_state_indices, self.g, self.gk,
                self.num_accepted_tokens, self.scale)


def make_case(B, Hq, Hv, T, Dk, Dv, N_slots, seed, *, zero_state=False, gk_hi=0.1,
              indices="choice", lengths=None, gate=False, state_std=0.05) -> Inputs:
    """Draw one seeded case following the recipe in the module docstring.

    ``indices``: "identity" (0..B-1), "choice" (B distinct slots drawn with
    ``rng.choice(N_slots, B, replace=False)``) or "permutation" (the first B entries of
    ``rng.permutation(N_slots)``). ``lengths``: None (all T), "uniform" (U{1..T}) or an
    explicit int array.
    """
    rng = np.random.default_rng(seed)
    q = to_bf16_bits(_unit_rows(rng, (B, Hq, T, Dk)))
    k = to_bf16_bits(_unit_rows(rng, (B, Hq, T, Dk)))
    v = to_bf16_bits(rng.standard_normal((B, Hv, T, Dv)))
    beta = to_bf16_bits(expit(rng.standard_normal((B, Hv, T))))
    g = (-np.logaddexp(0.0, rng.standard_normal((B, Hv, T)))).astype(np.float32)
    gk = (-rng.uniform(1e-3, gk_hi, (B, Hv, T, Dk))).astype(np.float32)
    if zero_state:
        state = np.zeros((N_slots, Hv, Dk, Dv), np.uint16)
    else:
        s = rng.standard_normal((N_slots, Hv, Dk, Dv), dtype=np.float32)
        s *= np.float32(state_std)
        state = to_bf16_bits(s)
        del s
    if indices == "identity":
        idx = np.arange(B, dtype=np.int32)
    elif indices == "choice":
        idx = rng.choice(N_slots, B, replace=False).astype(np.int32)
    elif indices == "permutation":
        idx = rng.permutation(N_slots)[:B].astype(np.int32)
    else:
        raise ValueError(indices)
    if lengths is None:
        lens = np.full(B, T, np.int32)
    elif isinstance(lengths, str) and lengths == "uniform":
        lens = rng.integers(1, T + 1, B).astype(np.int32)
    else:
        lens = np.asarray(lengths, np.int32)
    inp = Inputs(B, Hq, Hv, T, Dk, Dv, N_slots, q, k, v, beta, g, gk, state, idx, lens,
                 lens.copy(), float(np.float32(1.0 / np.sqrt(Dk))))
    if gate:
        inp.gate_a = rng.standard_normal((B, T, Hv)).astype(np.float32)
        inp.gate_b = rng.standard_normal((B, T, Hv)).astype(np.float32)
        inp.dt_bias = rng.standard_normal(Hv).astype(np.float32)
        a_log = rng.uniform(0.0, np.log(16.0), Hv).astype(np.float32)
        inp.decay_scale = (-np.exp(a_log)).astype(np.float32)
    return inp


def make_workload(wid: int, gate_inputs: bool = False, batch: Optional[int] = None) -> Inputs:
    """The eight workloads, seeded with 1000 + id (see the module docstring). ``batch``
    replaces the batch size B (the recipe is otherwise unchanged; the pool keeps its slots,
    at least B)."""
    w = dict(WORKLOADS[wid])
    if batch is not None:
        w["B"] = int(batch)
        w["N_slots"] = max(w["N_slots"], w["B"])
    seed = 1000 + wid
    if wid == 0:
        inp = make_case(**w, seed=seed, zero_state=True, indices="identity")
    elif wid == 1:
        inp = make_case(**w, seed=seed, indices="identity")
    elif wid == 2:
        inp = make_case(**w, seed=seed, indices="choice")
    elif wid == 3:
        inp = make_case(**w, seed=seed, indices="permutation", lengths="uniform")
    elif wid == 4:
        return make_case(**w, seed=seed, indices="choice", gk_hi=0.05, gate=True)
    elif wid in (5, 6, 7):
        inp = make_case(**w, seed=seed, indices="choice")
    else:
        raise KeyError(wid)
    if gate_inputs:
        rng = np.random.default_rng(seed + 100000)
        inp.gate_a = rng.standard_normal((inp.B, inp.T, inp.Hv)).astype(np.float32)
        inp.gate_b = rng.standard_normal((inp.B, inp.T, inp.Hv)).astype(np.float32)
        inp.dt_bias = np.zeros(inp.Hv, np.float32)
        inp.decay_scale = np.full(inp.Hv, -1.0, np.float32)
    return inp
