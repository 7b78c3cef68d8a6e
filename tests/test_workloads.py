"""The seeded input generator follows its stated recipe (CPU only): shapes, value ranges
and distributions, slot indices, lengths and determinism. The GPU tests, the bench and the
oracle all draw their inputs from it, so a silent change here would change every figure."""
import numpy as np
import pytest

import workloads


def f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.fixture(scope="module")
def wl():
    return {w: workloads.make_workload(w, gate_inputs=True) for w in (0, 1, 2, 3, 4)}


@pytest.mark.parametrize("wid", [0, 1, 2, 3, 4])
def test_shapes_and_dtypes(wl, wid):
    inp = wl[wid]
    s = workloads.WORKLOADS[wid]
    B, Hq, Hv, T, Dk, Dv, N = (s[k] for k in ("B", "Hq", "Hv", "T", "Dk", "Dv", "N_slots"))
    assert (inp.B, inp.Hq, inp.Hv, inp.T, inp.Dk, inp.Dv, inp.N_slots) == (B, Hq, Hv, T, Dk, Dv, N)
    for name, shape in (("query", (B, Hq, T, Dk)), ("key", (B, Hq, T, Dk)),
                        ("value", (B, Hv, T, Dv)), ("beta", (B, Hv, T)),
                        ("state", (N, Hv, Dk, Dv))):
        a = getattr(inp, name)
        assert a.shape == shape and a.dtype == np.uint16, name
    assert inp.g.shape == (B, Hv, T) and inp.g.dtype == np.float32
    assert inp.gk.shape == (B, Hv, T, Dk) and inp.gk.dtype == np.float32
    assert inp.gate_a.shape == (B, T, Hv) and inp.gate_b.shape == (B, T, Hv)
    assert np.float32(inp.scale) == np.float32(1.0 / np.sqrt(Dk))


@pytest.mark.parametrize("wid", [0, 1, 2, 3, 4])
def test_value_ranges(wl, wid):
    inp = wl[wid]
    for name in ("query", "key"):  # unit-norm head vectors, up to their bf16 rounding
        n = np.linalg.norm(f64(getattr(inp, name)), axis=-1)
        assert np.all(np.abs(n - 1.0) < 1e-2), name
    beta = f64(inp.beta)
    assert np.all((beta > 0) & (beta < 1))
    assert np.all(inp.g < 0)  # -softplus(x) < 0
    gk_hi = 0.05 if wid == 4 else 0.1
    assert np.all((inp.gk <= -1e-3) & (inp.gk >= -gk_hi))
    if wid == 0:
        assert np.all(inp.state == 0)
    else:  # the first slots (at least 1 M values where the pool has them)
        st = f64(inp.state[:4])
        assert abs(st.mean()) < 2e-3 and abs(st.std() - 0.05) < 2e-3


@pytest.mark.parametrize("wid", [0, 1, 2, 3, 4])
def test_indices_and_lengths(wl, wid):
    inp = wl[wid]
    idx = inp.ssm_state_indices
    assert idx.dtype == np.int32 and len(np.unique(idx)) == inp.B
    assert np.all((idx >= 0) & (idx < inp.N_slots))
    if wid in (0, 1):
        assert np.array_equal(idx, np.arange(inp.B))
    lens = inp.actual_seq_lengths
    if wid == 3:
        assert lens.min() >= 1 and lens.max() <= inp.T and len(np.unique(lens)) > 1
    else:
        assert np.all(lens == inp.T)
    assert np.array_equal(inp.num_accepted_tokens, lens)


def test_gate_inputs_of_the_fused_workload(wl):
    inp = wl[4]
    ds = inp.decay_scale
    assert ds.shape == (inp.Hv,) and np.all((ds <= -1.0) & (ds >= -16.0))
    assert inp.dt_bias.shape == (inp.Hv,) and np.std(inp.dt_bias) > 0.3
    for wid in (0, 1, 2, 3):  # the stand-in gate of the other workloads
        assert np.all(wl[wid].dt_bias == 0) and np.all(wl[wid].decay_scale == -1)


def test_deterministic(wl):
    again = workloads.make_workload(3, gate_inputs=True)
    first = wl[3]
    for name in ("query", "key", "value", "beta", "g", "gk", "state", "ssm_state_indices",
                 "actual_seq_lengths", "gate_a", "gate_b"):
        assert np.array_equal(getattr(again, name), getattr(first, name)), name
