"""GPU parity of rgdr_decode_snapshots: the decode step that also stores the state after
every token (the per-prefix states a speculative-decoding caller needs when it learns the
accepted count, the page's num_accepted_tokens, only after the step).

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

import oracle
import workloads
from gpu_util import assert_tol, bf16_dev_to_f64, check_decode, dev_to_bits, say, upload

pytestmark = pytest.mark.gpu

SENTINEL = np.uint16(0xFFED)  # a quiet NaN whose payload no rounding produces


@pytest.fixture(scope="module")
def rg():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gated_delta_rule_rgdr_amd as m
    m.library()
    return m


def run_and_check(rg, inp, label):
    d = upload(inp)
    pool = d["state"].clone()
    snap = torch.full((inp.B, inp.T, inp.Hv, inp.Dk, inp.Dv), int(SENTINEL.view(np.int16)),
                      dtype=torch.int16, device="cuda").view(torch.bfloat16)
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

    got = bf16_dev_to_f64(snap)
    bits = dev_to_bits(snap)
    pool_bits = dev_to_bits(st)
    lens = np.clip(inp.actual_seq_lengths, 0, inp.T)
    valid = (inp.ssm_state_indices >= 0) & (inp.ssm_state_indices < inp.N_slots)
    written = np.zeros((inp.B, inp.T), bool)
    for b in range(inp.B):
        if valid[b]:
            written[b, :lens[b]] = True
    assert np.array_equal(np.isfinite(o_snaps).all(axis=(2, 3, 4)), written)
    assert_tol(got[written], o_snaps[written], f"{label} snapshots")
    assert np.all(bits[~written] == SENTINEL), f"{label}: unwritten snapshot entries changed"
    n_acc = np.clip(inp.num_accepted_tokens, 0, lens)
    for b in range(inp.B):
        if valid[b] and n_acc[b] >= 1:
            assert np.array_equal(bits[b, n_acc[b] - 1], pool_bits[inp.ssm_state_indices[b]]), \
                f"{label}: entry {b}: snapshot {n_acc[b] - 1} is not the committed state"
    say(f"  {label}: {int(written.sum())} snapshot entries written")


CASES = [
    # B, Hq, Hv, T, Dk, Dv, N, seed, lengths, n_acc
    (4, 2, 4, 8, 128, 128, 8, 11, None, None),           # full length, D_k = 128
    (6, 2, 4, 5, 128, 256, 9, 12, "uniform", "draw"),    # varlen, accepted n < L, 2 tiles
    (3, 4, 4, 8, 64, 128, 3, 13, [8, 1, 6], [3, 1, 0]),  # D_k = 64, 128-column tiles, n = 0
    (5, 1, 2, 3, 64, 64, 7, 14, "uniform", "draw"),      # D_k = 64, 64-column tiles
    (4, 2, 4, 1, 128, 128, 4, 15, [1, 0, 1, 1], None),   # T = 1, an empty entry
    (8, 16, 32, 8, 128, 128, 16, 16, "uniform", "draw"), # the varlen speculative shape
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
