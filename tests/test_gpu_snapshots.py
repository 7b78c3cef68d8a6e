"""GPU parity of rgdr_decode_snapshots and rgdr_decode_gated_snapshots: the decode step
(plain, or with the gate fused in) that also stores the state after every token (the
per-prefix states a speculative-decoding caller needs when it learns the accepted count,
the page's num_accepted_tokens, only after the step).

Against the fp64 oracle on the same seeded bytes:
  - out and the committed slots: as rgdr_decode (2e-2 + 2e-2 |ref|, indexing bit for bit);
  - every written snapshot entry: within the same bound of the oracle's unrounded state
    after that token;
  - entries past an entry's length, and all entries of a skipped slot: untouched (the
    sentinel bytes the buffer held, bit for bit);
  - the snapshot after the accepted prefix: the committed slot's bytes, bit for bit.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import (bf16_dev_to_f64, check_gated_snapshots,
                      check_snapshots as run_and_check, dev_to_bits, say, upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rg():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gated_delta_rule_rgdr_amd as m
    m.library()
    return m


CASES = [
    # B, Hq, Hv, T, Dk, Dv, N, seed, lengths, n_acc
    (4, 2, 4, 8, 128, 128, 8, 11, None, None),           # full length, D_k = 128
    (6, 2, 4, 5, 128, 256, 9, 12, "uniform", "draw"),    # varlen, accepted n < L, 2 tiles
    (3, 4, 4, 8, 64, 128, 3, 13, [8, 1, 6], [3, 1, 0]),  # D_k = 64, 128-column tiles, n = 0
    (5, 1, 2, 3, 64, 64, 7, 14, "uniform", "draw"),      # D_k = 64, 64-column tiles
    (4, 2, 4, 1, 128, 128, 4, 15, [1, 0, 1, 1], None),   # T = 1, an empty entry
    (8, 16, 32, 8, 128, 128, 16, 16, "uniform", "draw"), # the varlen speculative shape
    (1, 1, 2, 8, 128, 4096, 2, 18, [7], [5]),            # D_v = 4096: 32 tiles per head
    (3, 2, 2, 8, 128, 320, 4, 19, "uniform", "draw"),    # chunk form, last tile 64 columns
    (4, 2, 4, 6, 64, 192, 5, 20, "uniform", "draw"),     # chunk form at D_k = 64, half tile
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_snapshots_parity(rg, case):
    B, Hq, Hv, T, Dk, Dv, N, seed, lengths, nacc = CASES[case]
    inp = workloads.make_case(B, Hq, Hv, T, Dk, Dv, N, seed, indices="choice",
                              lengths=lengths)
    if nacc == "draw":
        rng = np.random.default_rng(seed + 100)
        inp.num_accepted_tokens = rng.integers(0, inp.actual_seq_lengths + 1).astype(np.int32)
    elif nacc is not None:
        inp.num_accepted_tokens = np.asarray(nacc, np.int32)
    say(f"snapshots case {case}: B={B} Hq={Hq} Hv={Hv} T={T} Dk={Dk} Dv={Dv} "
        f"L={inp.actual_seq_lengths.tolist()} n={inp.num_accepted_tokens.tolist()}")
    run_and_check(rg, inp, f"snapshots case {case}")


def test_snapshots_skipped_slot_and_clamps(rg):
    """A slot outside the pool skips its entry (no snapshot written); lengths above T and
    accepted counts above L are clamped as in rgdr_decode."""
    inp = workloads.make_case(4, 2, 4, 6, 128, 128, 6, 17, indices="choice",
                              lengths=[6, 9, 3, 6])
    inp.ssm_state_indices[2] = 6  # == N_slots: skipped
    inp.num_accepted_tokens = np.asarray([2, 9, 3, 7], np.int32)
    say("snapshots: skipped slot, clamped length and count")
    run_and_check(rg, inp, "snapshots skipped/clamped")


def test_snapshots_workload3(rg):
    """The varlen speculative workload at full size (B = 32, T = 8, H_v = 32, D = 128)."""
    inp = workloads.make_workload(3)
    say(f"snapshots: {workloads.WORKLOAD_NAMES[3]}")
    run_and_check(rg, inp, "snapshots workload 3")


def test_snapshots_out_of_place(rg):
    """state_out a separate buffer: the pool is left as it was, state_out receives the
    committed slots (and keeps its other bytes), and the snapshots are those of the
    in-place call, bit for bit."""
    inp = workloads.make_case(4, 2, 4, 5, 128, 128, 6, 21, indices="choice", lengths="uniform")
    d = upload(inp)
    pool = d["state"].clone()
    fill = torch.full_like(pool.view(torch.int16), 0x1234).view(torch.bfloat16)
    st_out = fill.clone()
    args = (d["query"], d["key"], d["value"], d["beta"], pool, d["actual_seq_lengths"],
            d["ssm_state_indices"], d["g"], d["gk"], d["num_accepted_tokens"], inp.scale)
    out1, st1, sn1 = rg.rgdr_decode_snapshots(*args, state_out=st_out)
    torch.cuda.synchronize()
    assert np.array_equal(dev_to_bits(pool), inp.state), "the pool was modified"
    named = inp.ssm_state_indices
    others = np.setdiff1d(np.arange(inp.N_slots), named)
    assert np.all(dev_to_bits(st1)[others] == 0x1234), "state_out slots no entry names changed"
    pool2 = d["state"].clone()
    out2, st2, sn2 = rg.rgdr_decode_snapshots(*args[:4], pool2, *args[5:])
    torch.cuda.synchronize()
    lens = np.clip(inp.actual_seq_lengths, 0, inp.T)
    for b in range(inp.B):
        assert np.array_equal(dev_to_bits(sn1)[b, :lens[b]], dev_to_bits(sn2)[b, :lens[b]])
    assert np.array_equal(dev_to_bits(out1), dev_to_bits(out2))
    assert np.array_equal(dev_to_bits(st1)[named], dev_to_bits(st2)[named])
    say("  out-of-place snapshots: equal to the in-place call")


def test_snapshots_graph_replay_matches_eager(rg):
    """rgdr_decode_snapshots captured in a HIP graph (the chunk form at the varlen
    speculative shape) gives the eager bytes of out, the committed slots and every written
    snapshot on each of four replays, with eager work on the device between them."""
    inp = workloads.make_workload(3)
    d = upload(inp)
    out = torch.empty((inp.B, inp.Hv, inp.T, inp.Dv), dtype=torch.bfloat16, device="cuda")
    st = torch.empty_like(d["state"])
    snap = torch.empty((inp.B, inp.T, inp.Hv, inp.Dk, inp.Dv), dtype=torch.bfloat16,
                       device="cuda")

    def step():
        rg.rgdr_decode_snapshots(d["query"], d["key"], d["value"], d["beta"], d["state"],
                                 d["actual_seq_lengths"], d["ssm_state_indices"], d["g"],
                                 d["gk"], d["num_accepted_tokens"], inp.scale, out=out,
                                 state_out=st, state_snapshots=snap)

    lens = np.clip(inp.actual_seq_lengths, 0, inp.T)
    st.copy_(d["state"])
    step()
    torch.cuda.synchronize()
    want = (dev_to_bits(out), dev_to_bits(st), dev_to_bits(snap))
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        out.zero_()
        snap.zero_()
        st.copy_(d["state"])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (dev_to_bits(out), dev_to_bits(st), dev_to_bits(snap))
        assert np.array_equal(got[0], want[0]), f"replay {rep}: out differs"
        assert np.array_equal(got[1], want[1]), f"replay {rep}: state differs"
        for b in range(inp.B):
            assert np.array_equal(got[2][b, :lens[b]], want[2][b, :lens[b]]), \
                f"replay {rep}: snapshots of entry {b} differ"
    say("  snapshot graph replays equal the eager call")


GATED_CASES = [
    # B, Hq, Hv, T, Dk, Dv, N, seed, lengths, n_acc, gate dtype, normalize q/k
    (6, 2, 4, 5, 128, 256, 9, 31, "uniform", "draw", np.float32, False),  # chunk form
    (4, 2, 4, 8, 128, 128, 6, 32, "uniform", "draw", np.float16, True),   # fp16 gate, norm
    (5, 1, 2, 3, 64, 64, 7, 33, "uniform", "draw", np.float32, True),     # per-token form
    (3, 4, 4, 8, 64, 128, 3, 34, [8, 1, 6], [3, 1, 0], np.float16, False),  # D_k = 64
    (4, 2, 4, 1, 128, 128, 4, 35, [1, 0, 1, 1], None, np.float32, False),  # T = 1
    (3, 2, 2, 8, 128, 320, 4, 36, "uniform", "draw", np.float32, True),   # half last tile
]


@pytest.mark.parametrize("case", range(len(GATED_CASES)))
def test_gated_snapshots_parity(rg, case):
    B, Hq, Hv, T, Dk, Dv, N, seed, lengths, nacc, dtype, norm = GATED_CASES[case]
    inp = workloads.make_case(B, Hq, Hv, T, Dk, Dv, N, seed, indices="choice",
                              lengths=lengths, gate=True)
    if nacc == "draw":
        rng = np.random.default_rng(seed + 100)
        inp.num_accepted_tokens = rng.integers(0, inp.actual_seq_lengths + 1).astype(np.int32)
    elif nacc is not None:
        inp.num_accepted_tokens = np.asarray(nacc, np.int32)
    say(f"gated snapshots case {case}: B={B} Hq={Hq} Hv={Hv} T={T} Dk={Dk} Dv={Dv} "
        f"gate {np.dtype(dtype).name} norm={norm} L={inp.actual_seq_lengths.tolist()} "
        f"n={inp.num_accepted_tokens.tolist()}")
    check_gated_snapshots(rg, inp, f"gated snapshots case {case}", dtype=dtype,
                          normalize_qk=norm)


def test_gated_snapshots_skipped_slot_and_clamps(rg):
    """With the gate fused in: a skipped slot writes no snapshot; lengths above T and
    accepted counts above L are clamped."""
    inp = workloads.make_case(4, 2, 4, 6, 128, 128, 6, 37, indices="choice",
                              lengths=[6, 9, 3, 6], gate=True)
    inp.ssm_state_indices[2] = 6  # == N_slots: skipped
    inp.num_accepted_tokens = np.asarray([2, 9, 3, 7], np.int32)
    say("gated snapshots: skipped slot, clamped length and count")
    check_gated_snapshots(rg, inp, "gated snapshots skipped/clamped")


def test_gated_snapshots_workload3(rg):
    """The varlen speculative workload at full size with raw gate projections."""
    inp = workloads.make_workload(3, gate_inputs=True)
    say(f"gated snapshots: {workloads.WORKLOAD_NAMES[3]}")
    check_gated_snapshots(rg, inp, "gated snapshots workload 3")


@pytest.mark.parametrize("gated", [False, True], ids=["plain", "gated"])
def test_snapshot_calls_match_their_plain_calls(rg, gated):
    """A snapshot call's out and committed slots against the same call without snapshots,
    on the same inputs. out is bit for bit in both kernel forms, and so are the committed
    slots in the per-token form. The chunk form's snapshot loop forms each row's key
    weights g(t, s) k_s in another order (decay products first), so its committed slots may
    differ by one bf16 unit in the last place."""
    for Dk, Dv, T, form in ((128, 128, 8, "chunk"), (64, 64, 3, "per-token")):
        inp = workloads.make_case(4, 2, 4, T, Dk, Dv, 6, 38 + T, indices="choice",
                                  lengths="uniform", gate=gated)
        rng = np.random.default_rng(39)
        inp.num_accepted_tokens = rng.integers(0, inp.actual_seq_lengths + 1).astype(np.int32)
        d = upload(inp)
        tail = (d["actual_seq_lengths"], d["ssm_state_indices"], d["gk"],
                d["num_accepted_tokens"], inp.scale)
        p1, p2 = d["state"].clone(), d["state"].clone()
        if gated:
            gate = tuple(torch.from_numpy(x).cuda()
                         for x in (inp.gate_a, inp.gate_b, inp.dt_bias, inp.decay_scale))
            head = (d["query"], d["key"], d["value"]) + gate
            o1, s1 = rg.rgdr_decode_gated(*head, p1, *tail)
            o2, s2, _ = rg.rgdr_decode_gated_snapshots(*head, p2, *tail)
        else:
            head = (d["query"], d["key"], d["value"], d["beta"])
            plain_tail = (d["actual_seq_lengths"], d["ssm_state_indices"], d["g"], d["gk"],
                          d["num_accepted_tokens"], inp.scale)
            o1, s1 = rg.rgdr_decode(*head, p1, *plain_tail)
            o2, s2, _ = rg.rgdr_decode_snapshots(*head, p2, *plain_tail)
        torch.cuda.synchronize()
        assert np.array_equal(dev_to_bits(o1), dev_to_bits(o2)), f"{form}: out differs"
        if form == "per-token":
            assert np.array_equal(dev_to_bits(s1), dev_to_bits(s2)), f"{form}: state differs"
        else:
            a1, a2 = bf16_dev_to_f64(s1), bf16_dev_to_f64(s2)
            ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(a1), 1e-30))) - 7)
            assert np.all(np.abs(a1 - a2) <= ulp), f"{form}: state differs by more than 1 ulp"
            say(f"  {form}: {int((a1 != a2).sum())} of {a1.size} state values differ by 1 ulp")
