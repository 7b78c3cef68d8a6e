"""GPU parity of rgdr_decode_gated (gate front end fused into the decode) against the oracle
chain: the fp64 gate, then the fp64 recurrence core on the decoded inputs (no rounding of g
or beta in between, as in the fused kernel).

Bars as for rgdr_decode: 2e-2 + 2e-2 |ref| on bf16 out/state_out against unrounded fp64
values; padding, untouched slots and absent tokens bit for bit.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import (assert_tol, bf16_dev_to_f64, check_gated, dev_to_bits, gate_tensors,
                      gpu_gated, oracle_gated, raw_qk, say, upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rg():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gated_delta_rule_rgdr_amd as m
    m.library()
    return m


def test_gated_bench_workload_full(rg):
    """The bench's step at full size: workload 2 with gate inputs, one fused launch."""
    inp = workloads.make_workload(2, gate_inputs=True)
    say(f"gated: {workloads.WORKLOAD_NAMES[2]}")
    out, st = gpu_gated(rg, inp)
    check_gated(inp, out, st, oracle_gated(inp), "gated workload 2")


def test_gated_workload4_all_entries(rg):
    """Workload 4 at full size (B=256, 512 slots: four launches of the resident grid); the
    oracle recomputes every entry, in slices of 64 entries to bound its memory."""
    inp = workloads.make_workload(4)
    out, st = gpu_gated(rg, inp)
    for lo in range(0, inp.B, 64):
        entries = np.arange(lo, min(lo + 64, inp.B))
        say(f"gated workload 4: entries {lo}..{entries[-1]}")
        check_gated(inp, out, st, oracle_gated(inp, entries), f"gated workload 4 [{lo}:]",
                    entries)
    # slots no entry names are untouched, bit for bit
    untouched = np.setdiff1d(np.arange(inp.N_slots), inp.ssm_state_indices)
    assert np.array_equal(dev_to_bits(st)[untouched], inp.state[untouched])


def test_gated_varlen_T8_nan_padding(rg):
    """Multi-token form with the fused gate: varlen, T = 8; NaN in the padded gate entries
    changes nothing (they are never read)."""
    inp = workloads.make_workload(3, gate_inputs=True)
    out0, st0 = gpu_gated(rg, inp)
    check_gated(inp, out0, st0, oracle_gated(inp), "gated workload 3")
    for b in range(inp.B):
        L = inp.actual_seq_lengths[b]
        inp.gate_a[b, L:] = np.nan
        inp.gate_b[b, L:] = np.nan
    out1, st1 = gpu_gated(rg, inp)
    assert np.array_equal(dev_to_bits(out0), dev_to_bits(out1))
    assert np.array_equal(dev_to_bits(st0), dev_to_bits(st1))


def test_gated_fp16_projections(rg):
    # wave form (T = 1), chunk form at D_k = 128 and 64, per-token form (D_v = 64, T = 3)
    for shape in [(5, 2, 4, 1, 128, 128, 8), (4, 2, 4, 5, 128, 256, 8), (2, 2, 2, 5, 64, 128, 4),
                  (3, 2, 2, 3, 64, 64, 4)]:
        B, Hq, Hv, T, Dk, Dv, N = shape
        inp = workloads.make_case(B, Hq, Hv, T, Dk, Dv, N, seed=77, indices="choice",
                                  lengths="uniform", gate=True)
        out, st = gpu_gated(rg, inp, np.float16)
        check_gated(inp, out, st, oracle_gated(inp, dtype=np.float16), f"gated fp16 {shape}")


def test_gated_absent_and_rejected_token(rg):
    """T = 1: an absent token (L = 0) leaves the state bit-exact and writes +0.0; a rejected
    token (n = 0) still produces its output and commits the incoming state bit-exact."""
    inp = workloads.make_case(4, 2, 4, 1, 128, 128, 6, seed=31, indices="choice",
                              lengths=[1, 0, 1, 0], gate=True)
    inp.num_accepted_tokens = np.array([1, 0, 0, 0], np.int32)
    out, st = gpu_gated(rg, inp)
    bits = dev_to_bits(st)
    for b in (1, 2, 3):
        s = inp.ssm_state_indices[b]
        assert np.array_equal(bits[s], inp.state[s]), f"entry {b}: state changed"
    ob = dev_to_bits(out)
    assert np.all(ob[[1, 3]] == 0)
    check_gated(inp, out, st, oracle_gated(inp), "gated absent/rejected")


def test_gated_matches_unfused_chain(rg):
    """Fused and unfused (la_gate storing bf16 beta, then rgdr_decode) agree within the bar."""
    inp = workloads.make_workload(2, gate_inputs=True)
    out_f, st_f = gpu_gated(rg, inp)
    d = upload(inp)
    a, b, dt, ds = gate_tensors(inp)
    g, beta = rg.la_gate(a, dt, ds, b, decay_dtype=torch.float32, beta_dtype=torch.bfloat16)
    pool = d["state"].clone()
    out_u, st_u = rg.rgdr_decode(d["query"], d["key"], d["value"],
                                 beta.view(inp.B, inp.Hv, 1), pool, d["actual_seq_lengths"],
                                 d["ssm_state_indices"], g.view(inp.B, inp.Hv, 1), d["gk"],
                                 d["num_accepted_tokens"], inp.scale)
    torch.cuda.synchronize()
    assert_tol(bf16_dev_to_f64(out_f), bf16_dev_to_f64(out_u), "fused vs unfused out")
    idx = inp.ssm_state_indices
    assert_tol(bf16_dev_to_f64(st_f)[idx], bf16_dev_to_f64(st_u)[idx], "fused vs unfused state")


@pytest.mark.parametrize("shape", [
    (4, 2, 4, 1, 128, 128, 6),   # wave form, D_k = 128 (64-column tiles: a small call)
    (3, 2, 2, 1, 64, 128, 4),    # wave form, D_k = 64
    (3, 1, 2, 1, 128, 192, 5),   # wave form, 64-column tiles
    (4, 2, 4, 6, 128, 128, 6),   # chunk form (T > 1, D_k = 128), varlen
    (3, 2, 2, 8, 64, 192, 4),    # chunk form with a last half tile, D_k = 64
    (3, 2, 2, 3, 64, 64, 4),     # per-token multi-token form, D_k = 64, 64-column tiles
    (3, 2, 2, 5, 64, 256, 4),    # chunk form at D_k = 64
    (40, 4, 16, 1, 64, 512, 48),  # wave form, 128-column tiles at D_k = 64 (large call)
])
def test_gated_normalize_qk(rg, shape):
    """RGDR_NORMALIZE_QK: raw q, k in, the oracle normalises them per token and head (fp64);
    the kernel's fp32 normalisation must meet the same bar."""
    B, Hq, Hv, T, Dk, Dv, N = shape
    say(f"normalize_qk {shape}")
    inp = raw_qk(workloads.make_case(B, Hq, Hv, T, Dk, Dv, N, seed=91, indices="choice",
                                     lengths="uniform", gate=True), 92)
    out, st = gpu_gated(rg, inp, normalize_qk=True)
    check_gated(inp, out, st, oracle_gated(inp, normalize_qk=True), f"normalize {shape}")
    # the flag matters: without it the raw magnitudes give a different result
    out0, _ = gpu_gated(rg, inp)
    assert not torch.equal(out0, out)


def test_gated_normalize_qk_bench_shape_and_zero_vectors(rg):
    """The bench shape with raw q, k, some of them all-zero (those stay zero: no NaN)."""
    inp = raw_qk(workloads.make_workload(2, gate_inputs=True), 93)
    inp.query[3, 5, 0] = 0
    inp.key[7, 2, 0] = 0
    inp.key[11, 9, 0] = 0
    inp.query[11, 9, 0] = 0
    out, st = gpu_gated(rg, inp, normalize_qk=True)
    assert torch.isfinite(out.float()).all() and torch.isfinite(st.float()).all()
    check_gated(inp, out, st, oracle_gated(inp, normalize_qk=True), "normalize bench shape")


def test_gated_normalize_qk_is_noop_on_unit_inputs(rg):
    """On inputs that already have unit-norm q, k (up to their bf16 rounding), the flag
    changes the result by no more than the bar."""
    inp = workloads.make_case(4, 2, 4, 3, 128, 128, 6, seed=94, indices="choice",
                              lengths="uniform", gate=True)
    out1, st1 = gpu_gated(rg, inp, normalize_qk=True)
    out0, st0 = gpu_gated(rg, inp)
    assert_tol(bf16_dev_to_f64(out1), bf16_dev_to_f64(out0), "unit inputs out")
    idx = inp.ssm_state_indices
    assert_tol(bf16_dev_to_f64(st1)[idx], bf16_dev_to_f64(st0)[idx], "unit inputs state")


@pytest.mark.parametrize("case", ["workload3", "workload4", "chunk_half", "per_token"])
def test_gated_graph_replay_matches_eager(rg, case):
    """The fused call captured in a HIP graph gives the eager bytes on every replay: the chunk
    form (varlen T = 8), the wave form over several launches of the resident grid (B = 256),
    the chunk form with a last half tile (D_v = 192) and the per-token multi-token form
    (D_v = 64, T = 3). Out-of-place, so every replay starts from
    the same state; the output and state buffers are reset eagerly between replays."""
    if case == "workload3":
        inp = workloads.make_workload(3, gate_inputs=True)
    elif case == "workload4":
        inp = workloads.make_workload(4, gate_inputs=True)
    else:
        Dv = 192 if case == "chunk_half" else 64
        inp = workloads.make_case(6, 2, 4, 3, 128, Dv, 8, seed=41, indices="choice",
                                  lengths="uniform", gate=True)
    say(f"gated graph replay: {case}")
    d = upload(inp)
    a, b, dt, ds = gate_tensors(inp)
    out = torch.empty((inp.B, inp.Hv, inp.T, inp.Dv), dtype=torch.bfloat16, device="cuda")
    st = torch.empty_like(d["state"])

    def step():
        rg.rgdr_decode_gated(d["query"], d["key"], d["value"], a, b, dt, ds, d["state"],
                             d["actual_seq_lengths"], d["ssm_state_indices"], d["gk"],
                             d["num_accepted_tokens"], inp.scale, out=out, state_out=st)

    st.copy_(d["state"])
    step()
    torch.cuda.synchronize()
    want_out, want_st = dev_to_bits(out), dev_to_bits(st)
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        out.fill_(1.0)
        st.copy_(d["state"])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(dev_to_bits(out), want_out), f"{case} replay {rep}: out differs"
        assert np.array_equal(dev_to_bits(st), want_st), f"{case} replay {rep}: state differs"


_HOLD_CHILD = r"""
import sys
import numpy as np
sys.path[:0] = [sys.argv[1], sys.argv[1] + "/tests"]
import gated_delta_rule_rgdr_amd as rg
import workloads
from gpu_util import dev_to_bits
from gpu_util import gpu_gated
inp = workloads.make_workload(2, gate_inputs=True)
out, st = gpu_gated(rg, inp)
np.savez(sys.argv[2], out=dev_to_bits(out), st=dev_to_bits(st))
print("child done", flush=True)
"""


@pytest.mark.parametrize("rate", ["0", "100"])
def test_commit_hold_never_changes_results(rg, tmp_path, rate):
    """The T = 1 commit hold only delays the stores: with it off (rate 0) or very long (an
    assumed read rate of 100 GB/s, so the poll cap ends it) the fused call at the bench
    shape writes the same bytes as with the default hold. The library reads the rate once
    per process, so the other rate runs in a child process (one at a time, after this
    process's call has finished)."""
    import os
    import subprocess
    import sys
    inp = workloads.make_workload(2, gate_inputs=True)
    out0, st0 = gpu_gated(rg, inp)
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    dst = str(tmp_path / "hold.npz")
    env = dict(os.environ, RGDR_HOLD_READ_GBPS=rate)
    say(f"child process with RGDR_HOLD_READ_GBPS={rate}")
    r = subprocess.run([sys.executable, "-c", _HOLD_CHILD, root, dst], env=env, timeout=100,
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    got = np.load(dst)
    assert np.array_equal(dev_to_bits(out0), got["out"])
    assert np.array_equal(dev_to_bits(st0), got["st"])


def test_gated_wide_tiles_absent_and_rejected(rg):
    """The fused T = 1 call with 128-column tiles (a call too large for 64-column tiles in
    one launch): absent (L = 0) and rejected (n = 0) tokens commit the incoming state bit for
    bit and write +0.0 where absent; the rest meets the bar."""
    B = 40
    lens = np.ones(B, np.int32)
    lens[2::5] = 0
    inp = workloads.make_case(B, 16, 32, 1, 128, 128, 44, seed=83, indices="choice",
                              lengths=lens, gate=True)
    inp.num_accepted_tokens = lens.copy()
    inp.num_accepted_tokens[1::4] = 0
    out, st = gpu_gated(rg, inp)
    bits = dev_to_bits(st)
    for b in range(B):
        if lens[b] == 0 or inp.num_accepted_tokens[b] == 0:
            s = inp.ssm_state_indices[b]
            assert np.array_equal(bits[s], inp.state[s]), f"entry {b}: state changed"
    assert np.all(dev_to_bits(out)[lens == 0] == 0)
    check_gated(inp, out, st, oracle_gated(inp), "gated wide tiles absent/rejected")
