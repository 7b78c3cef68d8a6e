"""Seeded random shapes through every entry of the recurrence, against the fp64 oracle.

Each case draws its sizes, lengths, accepted counts and slot indices from one seed, so a
failure names a reproducible case. Decode calls (T <= 8) cover every kernel form; the
long-sequence entry covers chunks split at the accepted prefix; the snapshot entry covers
the per-token states (unwritten entries and the committed prefix bit for bit). Values within
2e-2 + 2e-2 |ref| of the unrounded oracle; padding and untouched slots bit for bit.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import check_decode, check_snapshots, gpu_decode, gpu_prefill, oracle_decode, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rg():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gated_delta_rule_rgdr_amd as m
    m.library()
    return m


def draw(seed, t_max):
    rng = np.random.default_rng(seed)
    Hq = int(rng.choice([1, 2, 4]))
    Hv = Hq * int(rng.choice([1, 2, 4]))
    Dk = int(rng.choice([64, 128]))
    Dv = 64 * int(rng.integers(1, 9))
    T = int(rng.integers(1, t_max + 1))
    B = int(rng.integers(1, 7))
    N = B + int(rng.integers(0, 4))
    lens = rng.integers(0, T + 1, B).astype(np.int32)
    inp = workloads.make_case(B, Hq, Hv, T, Dk, Dv, N, seed=seed + 1, indices="choice",
                              lengths=lens)
    nacc = np.array([rng.integers(0, L + 1) for L in lens], np.int32)
    inp.num_accepted_tokens = nacc
    if B > 1 and rng.random() < 0.3:
        inp.ssm_state_indices[int(rng.integers(0, B))] = -1  # a skipped entry
    return inp


@pytest.mark.parametrize("seed", range(16))
def test_random_decode(rg, seed):
    inp = draw(900 + seed, 8)
    say(f"decode case {seed}: B={inp.B} Hq={inp.Hq} Hv={inp.Hv} T={inp.T} Dk={inp.Dk} "
        f"Dv={inp.Dv} L={inp.actual_seq_lengths.tolist()} n={inp.num_accepted_tokens.tolist()}")
    out, st = gpu_decode(inp)
    check_decode(inp, out, st, oracle_decode(inp), f"random decode {seed}")


@pytest.mark.parametrize("seed", range(20))
def test_random_prefill(rg, seed):
    inp = draw(1900 + seed, 48)
    say(f"prefill case {seed}: B={inp.B} Hq={inp.Hq} Hv={inp.Hv} T={inp.T} Dk={inp.Dk} "
        f"Dv={inp.Dv} L={inp.actual_seq_lengths.tolist()} n={inp.num_accepted_tokens.tolist()}")
    out, st = gpu_prefill(inp)
    check_decode(inp, out, st, oracle_decode(inp), f"random prefill {seed}")


@pytest.mark.parametrize("seed", range(4))
def test_random_prefill_wide_tiles(rg, seed):
    """Random D_k = 64 calls with more 128-column items than the device holds at once (512 on
    MI355X), so that D_v a multiple of 256 takes 256-column tiles and other D_v keep 128."""
    rng = np.random.default_rng(2900 + seed)
    Hq = int(rng.choice([8, 16, 32]))
    Hv = 64
    Dv = int(rng.choice([256, 320, 512, 768]))
    B = int(-(-513 * 128 // (Hv * Dv))) + int(rng.integers(0, 3))
    T = int(rng.integers(2, 25))
    lens = rng.integers(0, T + 1, B).astype(np.int32)
    inp = workloads.make_case(B, Hq, Hv, T, 64, Dv, B + 1, seed=2950 + seed, indices="choice",
                              lengths=lens)
    inp.num_accepted_tokens = np.array([rng.integers(0, L + 1) for L in lens], np.int32)
    assert B * Hv * -(-Dv // 128) > 512
    say(f"wide prefill case {seed}: B={B} Hq={Hq} Dv={Dv} T={T} L={lens.tolist()}")
    out, st = gpu_prefill(inp)
    check_decode(inp, out, st, oracle_decode(inp), f"random wide prefill {seed}")


@pytest.mark.parametrize("seed", range(10))
def test_random_snapshots(rg, seed):
    inp = draw(2900 + seed, 8)
    say(f"snapshot case {seed}: B={inp.B} Hq={inp.Hq} Hv={inp.Hv} T={inp.T} Dk={inp.Dk} "
        f"Dv={inp.Dv} L={inp.actual_seq_lengths.tolist()} n={inp.num_accepted_tokens.tolist()}")
    check_snapshots(rg, inp, f"random snapshots {seed}")


@pytest.mark.parametrize("seed", range(8))
def test_random_segmented(rg, seed):
    """Random calls of one or two long entries through rgdr_prefill_ws, sized so that the
    segmented form serves them: ragged lengths, accepted counts anywhere (0 and L included),
    a skipped slot now and then."""
    rng = np.random.default_rng(3900 + seed)
    Hq = int(rng.choice([1, 2]))
    Hv = Hq * int(rng.choice([1, 2]))
    Dk = int(rng.choice([64, 128]))
    Dv = 64 * int(rng.integers(1, 5))
    B = int(rng.integers(1, 3))
    T = int(rng.integers(520, 1201))
    lens = rng.integers(0, T + 1, B).astype(np.int32)
    lens[0] = max(lens[0], 520)
    inp = workloads.make_case(B, Hq, Hv, T, Dk, Dv, B + 1, seed=3950 + seed, indices="choice",
                              lengths=lens)
    inp.num_accepted_tokens = np.array([rng.integers(0, L + 1) for L in lens], np.int32)
    if B > 1 and rng.random() < 0.3:
        inp.ssm_state_indices[1] = -1
    assert rg.rgdr_prefill_workspace_size(B, Hv, T, Dk, Dv) > 0
    say(f"segmented case {seed}: B={B} Hq={Hq} Hv={Hv} T={T} Dk={Dk} Dv={Dv} "
        f"L={lens.tolist()} n={inp.num_accepted_tokens.tolist()}")
    out, st = gpu_decode(inp, fn="rgdr_prefill_ws")
    check_decode(inp, out, st, oracle_decode(inp), f"random segmented {seed}")
