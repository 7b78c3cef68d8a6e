"""GPU parity of the segmented long-sequence form (rgdr_prefill_ws, rgdr_prefill_gated_ws)
against the fp64 oracle.

The form rests on the recurrence of the MindSpore Lite page
"lite_boost.ops.recurrent_gated_delta_rule" (algorithm section) being affine in the state:
steps 1 and 3 map S to (I - beta k k^T) diag(decays) S + beta k v^T, so a segment of tokens
maps its incoming state S to Phi S + Psi. The oracle knows nothing of segments: it runs the
four steps token by token over the whole sequence.

Values: bf16 out/state_out within 2e-2 + 2e-2 |ref| of the unrounded oracle value. Indexing
(untouched slots, padded +0.0 rows, skipped entries, the commit after the accepted prefix,
n = 0 committing the incoming bytes) bit for bit.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import (check_decode, check_gated, dev_to_bits, gpu_prefill, oracle_decode,
                      oracle_gated, raw_qk, say, upload, gate_tensors)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rg():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gated_delta_rule_rgdr_amd as m
    m.library()
    return m


def run_ws(rg, inp, *, inplace=False, workspace=None):
    d = upload(inp)
    pool = d["state"] if inplace else d["state"].clone()
    out, st = rg.rgdr_prefill_ws(d["query"], d["key"], d["value"], d["beta"], pool,
                                 d["actual_seq_lengths"], d["ssm_state_indices"], d["g"],
                                 d["gk"], d["num_accepted_tokens"], inp.scale,
                                 workspace=workspace)
    torch.cuda.synchronize()
    return out, st


def segmented(rg, inp):
    """The call takes the segmented form (its workspace query is not 0)."""
    n = rg.rgdr_prefill_workspace_size(inp.B, inp.Hv, inp.T, inp.Dk, inp.Dv)
    say(f"  workspace {n} bytes")
    return n > 0


# B, Hq, Hv, T, Dk, Dv, N_slots
SHAPES = [
    (1, 2, 4, 1024, 128, 128, 2),   # one prompt: 16 segments of 64 tokens
    (3, 2, 4, 700, 128, 256, 5),    # two tiles per head, ragged lengths
    (1, 1, 2, 600, 64, 256, 2),     # D_k = 64
    (2, 2, 2, 1333, 128, 64, 3),    # D_v = 64: half tiles, a segment length not dividing T
    (1, 1, 1, 2048, 64, 512, 2),    # the example page's head size, one head
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%d_Hq%d_Hv%d_T%d_Dk%d_Dv%d" % s[:6])
def test_segmented_shapes(rg, shape):
    """Ragged lengths, an accepted prefix inside a segment, against the oracle."""
    B, Hq, Hv, T, Dk, Dv, N = shape
    inp = workloads.make_case(B, Hq, Hv, T, Dk, Dv, N, seed=8100 + T + Dv, indices="choice",
                              lengths="uniform")
    rng = np.random.default_rng(8101 + T)
    inp.actual_seq_lengths[0] = T
    inp.num_accepted_tokens = rng.integers(1, inp.actual_seq_lengths + 1).astype(np.int32)
    say(f"segmented {shape}, lengths {inp.actual_seq_lengths.tolist()}, "
        f"accepted {inp.num_accepted_tokens.tolist()}")
    assert segmented(rg, inp)
    out, st = run_ws(rg, inp)
    check_decode(inp, out, st, oracle_decode(inp), f"segmented {shape}")


def test_segmented_edge_entries(rg):
    """Entries with n = 0 (the incoming bytes committed bit for bit), n = L, L = 0, a skipped
    slot, and an accepted count on a segment boundary, in one call; in place."""
    B, T = 6, 640
    inp = workloads.make_case(B, 2, 4, T, 128, 128, 8, seed=8200, indices="choice",
                              lengths="uniform")
    inp.actual_seq_lengths[:] = [640, 500, 0, 640, 311, 640]
    inp.num_accepted_tokens[:] = [0, 500, 0, 640, 64, 200]
    inp.ssm_state_indices[5] = 8  # skipped: no state read or written, zero outputs
    say("segmented edge entries")
    assert segmented(rg, inp)
    out, st = run_ws(rg, inp, inplace=True)
    check_decode(inp, out, st, oracle_decode(inp), "segmented edges")
    slots = inp.ssm_state_indices
    got = dev_to_bits(st)
    assert np.array_equal(got[slots[0]], inp.state[slots[0]]), "n = 0 must commit the input"
    assert np.array_equal(got[slots[2]], inp.state[slots[2]]), "L = 0 must commit the input"


def test_segmented_strong_decays(rg):
    """Chunks cut inside segments (decays of 6 to 12 nats per token in one entry, rows at
    different rates in another)."""
    inp = workloads.make_case(2, 2, 4, 900, 128, 128, 3, seed=8300, indices="permutation",
                              lengths="uniform")
    inp.actual_seq_lengths[:] = [900, 777]
    inp.num_accepted_tokens[:] = [850, 777]
    inp.g[0] *= 8.0
    inp.gk[1, :, :, ::2] *= 40.0
    say("segmented strong decays")
    assert segmented(rg, inp)
    out, st = run_ws(rg, inp)
    check_decode(inp, out, st, oracle_decode(inp), "segmented strong decays")


def test_segmented_small_workspace_is_single_pass(rg):
    """A workspace smaller than the size query: the call runs the single pass, the same bits
    as rgdr_prefill."""
    inp = workloads.make_case(1, 2, 4, 1024, 128, 128, 2, seed=8400, indices="choice",
                              lengths="uniform")
    assert segmented(rg, inp)
    small = torch.empty(1024, dtype=torch.uint8, device="cuda")
    out_w, st_w = run_ws(rg, inp, workspace=small)
    out_p, st_p = gpu_prefill(inp)
    assert np.array_equal(dev_to_bits(out_w), dev_to_bits(out_p))
    assert np.array_equal(dev_to_bits(st_w), dev_to_bits(st_p))


def test_segmented_reused_workspace(rg):
    """One workspace for two calls in a row, the second with fewer tokens and other entries:
    nothing of the first call leaks into the second."""
    a = workloads.make_case(2, 2, 4, 1600, 128, 128, 3, seed=8500, indices="choice",
                            lengths="uniform")
    b = workloads.make_case(1, 2, 4, 1100, 128, 128, 2, seed=8501, indices="choice",
                            lengths="uniform")
    b.num_accepted_tokens = np.minimum(b.num_accepted_tokens, 100).astype(np.int32)
    need = max(rg.rgdr_prefill_workspace_size(x.B, x.Hv, x.T, x.Dk, x.Dv) for x in (a, b))
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
    for x, tag in ((a, "first"), (b, "second")):
        assert segmented(rg, x)
        out, st = run_ws(rg, x, workspace=ws)
        check_decode(x, out, st, oracle_decode(x), f"reused workspace, {tag} call")


def test_segmented_single_pass_for_large_batches(rg):
    """Calls that fill the device run in one pass: the size query gives 0."""
    assert rg.rgdr_prefill_workspace_size(16, 32, 1024, 128, 128) == 0
    assert rg.rgdr_prefill_workspace_size(4, 64, 1024, 64, 512) == 0
    assert rg.rgdr_prefill_workspace_size(1, 32, 8192, 128, 128) > 0


@pytest.mark.parametrize("normalize_qk", [False, True])
def test_segmented_gated(rg, normalize_qk):
    """rgdr_prefill_gated_ws against the oracle's gate-then-recurrence chain (fp16 gate
    projections with normalisation: raw q/k projections)."""
    inp = workloads.make_case(2, 2, 4, 520, 128, 128, 3, seed=8600 + normalize_qk,
                              indices="choice", lengths="uniform", gate=True)
    inp.actual_seq_lengths[0] = 520
    inp.num_accepted_tokens[:] = [400, inp.actual_seq_lengths[1]]
    dtype = np.float16 if normalize_qk else np.float32
    if normalize_qk:
        raw_qk(inp, 8602)
    say(f"segmented gated, normalize_qk={normalize_qk}")
    assert segmented(rg, inp)
    d = upload(inp)
    a, b, dt, ds = gate_tensors(inp, dtype)
    pool = d["state"].clone()
    out, st = rg.rgdr_prefill_gated_ws(d["query"], d["key"], d["value"], a, b, dt, ds, pool,
                                       d["actual_seq_lengths"], d["ssm_state_indices"],
                                       d["gk"], d["num_accepted_tokens"], inp.scale,
                                       normalize_qk=normalize_qk)
    torch.cuda.synchronize()
    check_gated(inp, out, st, oracle_gated(inp, dtype=dtype, normalize_qk=normalize_qk),
                f"segmented gated nqk={normalize_qk}")


def test_segmented_noalloc_graph_replays(rg):
    """rgdr_prefill_noalloc captured in a HIP graph (the segmented form's three launches on
    the library's fixed array, out of place) gives the eager call's bytes of out and the
    committed slots on each of four replays, with eager work on the device between them."""
    inp = workloads.make_case(2, 2, 4, 900, 128, 128, 3, seed=8800, indices="choice",
                              lengths="uniform")
    inp.actual_seq_lengths[0] = 900
    inp.num_accepted_tokens[:] = [700, inp.actual_seq_lengths[1]]
    assert segmented(rg, inp)
    d = upload(inp)
    out = torch.empty((inp.B, inp.Hv, inp.T, inp.Dv), dtype=torch.bfloat16, device="cuda")
    st = torch.empty_like(d["state"])

    def step():
        rg.rgdr_prefill_noalloc(d["query"], d["key"], d["value"], d["beta"], d["state"],
                                d["actual_seq_lengths"], d["ssm_state_indices"], d["g"],
                                d["gk"], d["num_accepted_tokens"], inp.scale, out=out,
                                state_out=st)

    st.copy_(d["state"])
    step()  # eager: also fills the library's per-device lookups before the capture
    torch.cuda.synchronize()
    want = (dev_to_bits(out), dev_to_bits(st))
    check_decode(inp, out, st, oracle_decode(inp), "segmented noalloc, eager")
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        out.zero_()
        st.copy_(d["state"])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(dev_to_bits(out), want[0]), f"replay {rep}: out differs"
        assert np.array_equal(dev_to_bits(st), want[1]), f"replay {rep}: state differs"
