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

import workloads
from gpu_util import check_snapshots as run_and_check, say

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
