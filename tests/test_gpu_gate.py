"""GPU parity of la_gate against the fp64 oracle.

Bars (fp32 arithmetic on the GPU, narrowed once on store):
  decay fp32: |d| <= 1e-6 + 1e-5 |ref| (expf/log1pf are within a few ulp; the sum a + dt_bias
              is one fp32 rounding, amplified at most by softplus' slope <= 1);
  beta fp32: |d| <= 4 ulp(ref); fp16/bf16 outputs: |d| <= 1 ulp of the output type
  (round-to-nearest of a value already within a few fp32 ulp).
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

FRAC_BITS = {torch.float32: 23, torch.float16: 10, torch.bfloat16: 7}


@pytest.fixture(scope="module")
def rg():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gated_delta_rule_rgdr_amd as m
    m.library()
    return m


def ulp(ref, dtype):
    e = np.floor(np.log2(np.maximum(np.abs(ref), 1e-300)))
    if dtype == torch.float16:
        e = np.maximum(e, -14)
    return np.exp2(e - FRAC_BITS[dtype])


def make(shape, H, dtype, seed):
    rng = np.random.default_rng(seed)
    a = (rng.standard_normal(shape + (H,)) * 4).astype(np.float32)
    b = (rng.standard_normal(shape + (H,)) * 4).astype(np.float32)
    dt = rng.standard_normal(H).astype(np.float32)
    ds = (-np.exp(rng.uniform(0, np.log(16), H))).astype(np.float32)
    npdt = np.float16 if dtype == torch.float16 else np.float32
    return a.astype(npdt), b.astype(npdt), dt, ds


CASES = [
    # leading shape, H, input dtype, decay dtype, beta dtype
    ((256, 1), 32, torch.float32, torch.float32, torch.bfloat16),   # feeds the decode
    ((3, 7), 5, torch.float32, torch.float32, torch.float32),
    ((11,), 1, torch.float16, torch.float16, torch.float16),
    ((2, 3, 4), 6, torch.float16, torch.float32, torch.bfloat16),
    ((2049, 257), 2, torch.float32, torch.float32, torch.float32),   # > one pass of the grid
    ((), 9, torch.float32, torch.float16, torch.float16),             # rank 1
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}x{c[1]}_{c[2]}_{c[3]}_{c[4]}")
def test_gate_parity(rg, case):
    shape, H, in_dt, dec_dt, beta_dt = case
    a, b, dt, ds = make(shape, H, in_dt, seed=H + len(shape))
    dec, bet = rg.la_gate(torch.from_numpy(a).cuda(), torch.from_numpy(dt).cuda(),
                          torch.from_numpy(ds).cuda(), torch.from_numpy(b).cuda(),
                          decay_dtype=dec_dt, beta_dtype=beta_dt)
    torch.cuda.synchronize()
    d64, b64 = oracle.la_gate(a, dt, ds, b)
    got_d = dec.float().cpu().numpy().astype(np.float64)
    got_b = bet.float().cpu().numpy().astype(np.float64)
    assert got_d.shape == d64.shape and got_b.shape == b64.shape
    if dec_dt == torch.float32:
        assert np.all(np.abs(got_d - d64) <= 1e-6 + 1e-5 * np.abs(d64))
    else:
        assert np.all(np.abs(got_d - d64) <= ulp(d64, dec_dt))
    k = 4 if beta_dt == torch.float32 else 1
    assert np.all(np.abs(got_b - b64) <= k * ulp(b64, beta_dt))


def test_gate_without_beta(rg):
    a, b, dt, ds = make((4,), 3, torch.float32, 1)
    dec, bet = rg.la_gate(torch.from_numpy(a).cuda(), torch.from_numpy(dt).cuda(),
                          torch.from_numpy(ds).cuda(), torch.from_numpy(b).cuda(),
                          want_beta=False)
    assert bet is None
    d64, _ = oracle.la_gate(a, dt, ds)
    got = dec.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - d64) <= 1e-6 + 1e-5 * np.abs(d64))


def test_gate_special_values(rg):
    """a + dt_bias = 0 gives decay = decay_scale ln 2; b = 0 gives beta = 1/2 exactly."""
    dt = torch.tensor([0.5, -1.25, 3.0], device="cuda")
    ds = torch.tensor([-1.0, -2.5, 0.75], device="cuda")
    a = (-dt)[None, :].contiguous()
    b = torch.zeros_like(a)
    dec, bet = rg.la_gate(a, dt, ds, b)
    ref = ds.double().cpu().numpy() * np.log(2.0)
    assert np.all(np.abs(dec.cpu().numpy()[0] - ref) <= 2e-7 * np.abs(ref))
    assert torch.all(bet == 0.5)


def test_gate_empty(rg):
    a = torch.empty((0, 4), device="cuda")
    dt = torch.zeros(4, device="cuda")
    dec, bet = rg.la_gate(a, dt, dt, a.clone())
    assert dec.shape == (0, 4) and bet.shape == (0, 4)
