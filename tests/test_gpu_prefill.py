"""GPU parity of rgdr_prefill / rgdr_prefill_gated (the recurrence over long sequences, the
prefill counterpart named in the notes of the MindSpore Lite page
"lite_boost.ops.recurrent_gated_delta_rule") against the fp64 oracle, whose token-by-token
recurrence has no bound on T.

Values: bf16 out/state_out within 2e-2 + 2e-2 |ref| of the unrounded oracle value. Indexing
(pool gather/scatter, untouched slots, varlen masking, padded +0.0 rows, skipped entries,
head sharing, the accepted prefix) bit for bit.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import (assert_tol, bf16_dev_to_f64, check_decode, check_gated, dev_to_bits,
                      gpu_decode, gpu_gated, gpu_prefill, oracle_decode, oracle_gated, raw_qk,
                      say, upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rg():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gated_delta_rule_rgdr_amd as m
    m.library()
    return m


# B, Hq, Hv, T, Dk, Dv, N_slots; lengths U{1..T}
SHAPES = [
    (3, 2, 4, 16, 128, 128, 5),     # half a chunk
    (4, 2, 4, 64, 128, 256, 6),     # two tiles per head
    (2, 1, 2, 512, 128, 128, 3),    # 16 chunks
    (3, 1, 3, 40, 64, 192, 4),      # D_k = 64, a last tile of 64 columns
    (2, 4, 4, 33, 64, 512, 3),      # the example page's head size
    (5, 4, 8, 9, 128, 64, 7),       # T = 9; every tile half
    (2, 1, 1, 3, 128, 128, 2),      # T < 8 is accepted too
    (2, 2, 2, 20, 128, 4096, 3),    # the largest D_v
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%d_Hq%d_Hv%d_T%d_Dk%d_Dv%d" % s[:6])
def test_prefill_shapes(rg, shape):
    B, Hq, Hv, T, Dk, Dv, N = shape
    inp = workloads.make_case(B, Hq, Hv, T, Dk, Dv, N, seed=7000 + T + Dv, indices="choice",
                              lengths="uniform")
    say(f"prefill {shape}, lengths {inp.actual_seq_lengths.tolist()}")
    out, st = gpu_prefill(inp)
    check_decode(inp, out, st, oracle_decode(inp), f"prefill {shape}")


# D_k = 64 calls with more 128-column items than the device holds at once (two per compute
# unit: 512 on MI355X) take 256-column tiles when D_v allows; B, Hq, Hv, T, Dv, N_slots
WIDE = [
    (4, 16, 64, 40, 512, 6),     # the example page's head size, 1024 narrow items
    (5, 8, 64, 35, 256, 7),      # one wide tile per head, 640 narrow items
    (2, 4, 16, 20, 4096, 3),     # the largest D_v: 16 wide tiles per head
    (3, 16, 64, 18, 768, 4),     # three wide tiles per head
    (4, 16, 64, 18, 320, 6),     # D_v not a multiple of 256: 128-column tiles at any size
]


@pytest.mark.parametrize("shape", WIDE, ids=lambda s: "B%d_Hq%d_Hv%d_T%d_Dv%d" % s[:5])
def test_prefill_wide_tiles(rg, shape):
    """256-column tiles at D_k = 64: ragged lengths, accepted prefixes inside and at the end
    of chunks, head sharing, a skipped slot, against the oracle (values) and bit for bit
    (padded rows, untouched slots)."""
    B, Hq, Hv, T, Dv, N = shape
    inp = workloads.make_case(B, Hq, Hv, T, 64, Dv, N, seed=7300 + Dv, indices="choice",
                              lengths="uniform")
    rng = np.random.default_rng(7301 + Dv)
    inp.num_accepted_tokens = rng.integers(0, inp.actual_seq_lengths + 1).astype(np.int32)
    inp.ssm_state_indices[1] = N  # skipped entry
    assert B * Hv * -(-Dv // 128) > 512
    say(f"prefill wide tiles {shape}, lengths {inp.actual_seq_lengths.tolist()}")
    out, st = gpu_prefill(inp)
    check_decode(inp, out, st, oracle_decode(inp), f"prefill wide {shape}")


def test_prefill_wide_tiles_equal_narrow_tiles(rg):
    """The same entries through 256-column tiles (one call of 4 entries: 1024 narrow items)
    and through 128-column tiles (two calls of 2 entries: 512 narrow items each, which the
    device holds at once) give the same bits: a column's arithmetic and an item's chunk cuts
    do not depend on the tile width."""
    inp = workloads.make_case(4, 16, 64, 70, 64, 512, 4, seed=7320, indices="permutation",
                              lengths="uniform")
    rng = np.random.default_rng(7321)
    inp.num_accepted_tokens = rng.integers(0, inp.actual_seq_lengths + 1).astype(np.int32)
    inp.g[2] *= 6.0  # strong decays in one entry: its chunks are cut
    out_w, st_w = gpu_prefill(inp)
    d = upload(inp)
    pool = d["state"].clone()
    outs = []
    for half in (slice(0, 2), slice(2, 4)):
        o, pool = rg.rgdr_prefill(d["query"][half], d["key"][half], d["value"][half],
                                  d["beta"][half], pool, d["actual_seq_lengths"][half],
                                  d["ssm_state_indices"][half], d["g"][half], d["gk"][half],
                                  d["num_accepted_tokens"][half], inp.scale)
        outs.append(o)
    torch.cuda.synchronize()
    assert np.array_equal(dev_to_bits(out_w), dev_to_bits(torch.cat(outs))), "out differs"
    assert np.array_equal(dev_to_bits(st_w), dev_to_bits(pool)), "state differs"


def test_prefill_four_wave_tiles_at_d128(rg):
    """More 128-column items than half the compute units (144 here): the call keeps
    128-column tiles, against the oracle, with ragged lengths and accepted prefixes."""
    inp = workloads.make_case(9, 8, 16, 40, 128, 128, 12, seed=7330, indices="choice",
                              lengths="uniform")
    rng = np.random.default_rng(7331)
    inp.num_accepted_tokens = rng.integers(0, inp.actual_seq_lengths + 1).astype(np.int32)
    assert 2 * inp.B * inp.Hv > 256
    out, st = gpu_prefill(inp)
    check_decode(inp, out, st, oracle_decode(inp), "prefill 128-column tiles at D_k = 128")


def test_prefill_narrow_tiles_equal_wide_tiles(rg):
    """At D_k = 128 a call with few items takes 64-column tiles. The same entries as one call
    (144 items, 128-column tiles) and as one call per entry (16 items each, 64-column tiles)
    give the same bits: a column's arithmetic and an item's chunk cuts do not depend on the
    tile width."""
    inp = workloads.make_case(9, 8, 16, 70, 128, 192, 9, seed=7340, indices="permutation",
                              lengths="uniform")
    rng = np.random.default_rng(7341)
    inp.num_accepted_tokens = rng.integers(0, inp.actual_seq_lengths + 1).astype(np.int32)
    inp.g[4] *= 6.0  # strong decays in one entry: its chunks are cut
    out_w, st_w = gpu_prefill(inp)
    d = upload(inp)
    pool = d["state"].clone()
    outs = []
    for b in range(inp.B):
        e = slice(b, b + 1)
        o, pool = rg.rgdr_prefill(d["query"][e], d["key"][e], d["value"][e], d["beta"][e], pool,
                                  d["actual_seq_lengths"][e], d["ssm_state_indices"][e],
                                  d["g"][e], d["gk"][e], d["num_accepted_tokens"][e], inp.scale)
        outs.append(o)
    torch.cuda.synchronize()
    assert np.array_equal(dev_to_bits(out_w), dev_to_bits(torch.cat(outs))), "out differs"
    assert np.array_equal(dev_to_bits(st_w), dev_to_bits(pool)), "state differs"


def test_prefill_gated_wide_tiles(rg):
    """The fused gate (fp16 projections) with in-kernel q/k normalisation of raw q and k on
    256-column tiles."""
    inp = workloads.make_case(4, 16, 64, 24, 64, 512, 5, seed=7310, indices="choice",
                              lengths="uniform", gate=True)
    inp = raw_qk(inp, 7311)
    out, st = gpu_gated(rg, inp, np.float16, normalize_qk=True, fn="rgdr_prefill_gated")
    check_gated(inp, out, st, oracle_gated(inp, dtype=np.float16, normalize_qk=True),
                "prefill gated wide tiles")


@pytest.mark.parametrize("T", [16, 64, 512])
def test_prefill_full_lengths(rg, T):
    """Every entry runs all T tokens (GQA, D = 128)."""
    inp = workloads.make_case(3, 2, 4, T, 128, 128, 5, seed=7100 + T, indices="choice")
    out, st = gpu_prefill(inp)
    check_decode(inp, out, st, oracle_decode(inp), f"prefill T={T}")


def test_prefill_nan_padding_bitexact(rg):
    """Padded tokens filled with NaN change no valid output or state, bit for bit."""
    inp = workloads.make_case(4, 2, 4, 40, 128, 128, 6, seed=7201, indices="choice",
                              lengths=[40, 17, 8, 1])
    out0, st0 = gpu_prefill(inp)
    nan = np.uint16(0x7FC0)
    for b in range(inp.B):
        L = inp.actual_seq_lengths[b]
        inp.query[b, :, L:] = nan
        inp.key[b, :, L:] = nan
        inp.value[b, :, L:] = nan
        inp.beta[b, :, L:] = nan
        inp.g[b, :, L:] = np.nan
        inp.gk[b, :, L:] = np.nan
    out1, st1 = gpu_prefill(inp)
    assert np.array_equal(dev_to_bits(out0), dev_to_bits(out1))
    assert np.array_equal(dev_to_bits(st0), dev_to_bits(st1))
    check_decode(inp, out1, st1, oracle_decode(inp), "prefill NaN padding")


def test_prefill_accepted_prefix(rg):
    """n < L: the committed state equals that of a call that stops after n tokens, bit for
    bit; outputs of tokens before n equal those of the n = L call within the bar (the chunk
    that ends at n measures its decays from its own middle, so they may differ in rounding);
    everything meets the bar against the oracle. Counts inside the first chunk of 32 (8, 13,
    16, 20 of 21), zero and the full length."""
    lens = [30, 30, 30, 30, 30, 21]
    nacc = [8, 16, 13, 0, 30, 20]
    full = workloads.make_case(6, 2, 4, 32, 128, 128, 8, seed=7301, indices="choice",
                               lengths=lens)
    out_f, _ = gpu_prefill(full)
    acc = workloads.make_case(6, 2, 4, 32, 128, 128, 8, seed=7301, indices="choice",
                              lengths=lens)
    acc.num_accepted_tokens = np.array(nacc, np.int32)
    out_a, st_a = gpu_prefill(acc)
    of, oa = bf16_dev_to_f64(out_f), bf16_dev_to_f64(out_a)
    for b, n in enumerate(nacc):
        assert_tol(oa[b, :, :n], of[b, :, :n], f"entry {b}: outputs before {n}")
    short = workloads.make_case(6, 2, 4, 32, 128, 128, 8, seed=7301, indices="choice",
                                lengths=lens)
    short.actual_seq_lengths = acc.num_accepted_tokens.copy()
    short.num_accepted_tokens = acc.num_accepted_tokens.copy()
    _, st_s = gpu_prefill(short)
    assert np.array_equal(dev_to_bits(st_a), dev_to_bits(st_s))
    check_decode(acc, out_a, st_a, oracle_decode(acc), "prefill accepted prefix")


def test_prefill_zero_lengths_and_skipped_entries(rg):
    """L = 0 writes the state back unchanged and +0.0 rows; an out-of-range slot skips its
    entry (+0.0 rows, no state access)."""
    inp = workloads.make_case(4, 2, 4, 24, 128, 128, 6, seed=7401, indices="choice",
                              lengths=[0, 24, 0, 11])
    inp.ssm_state_indices[1] = -3
    out, st = gpu_prefill(inp)
    ob, sb = dev_to_bits(out), dev_to_bits(st)
    assert np.all(ob[[0, 1, 2]] == 0)
    for b in (0, 2):
        s = inp.ssm_state_indices[b]
        assert np.array_equal(sb[s], inp.state[s])
    check_decode(inp, out, st, oracle_decode(inp), "prefill zero lengths")


def test_prefill_permutation_equivariance(rg):
    inp = workloads.make_case(5, 2, 4, 24, 128, 128, 8, seed=7501, indices="choice",
                              lengths="uniform")
    out, st = gpu_prefill(inp)
    perm = np.array([3, 0, 4, 1, 2])
    p = workloads.make_case(5, 2, 4, 24, 128, 128, 8, seed=7501, indices="choice",
                            lengths="uniform")
    for name in ("query", "key", "value", "beta", "g", "gk", "ssm_state_indices",
                 "actual_seq_lengths", "num_accepted_tokens"):
        setattr(p, name, np.ascontiguousarray(getattr(inp, name)[perm]))
    out_p, st_p = gpu_prefill(p)
    assert np.array_equal(dev_to_bits(out_p), dev_to_bits(out)[perm])
    assert np.array_equal(dev_to_bits(st_p), dev_to_bits(st))


def test_prefill_gqa_expansion_bitexact(rg):
    inp = workloads.make_case(2, 4, 16, 20, 128, 128, 3, seed=7601, indices="choice",
                              lengths="uniform")
    out, st = gpu_prefill(inp)
    e = workloads.make_case(2, 4, 16, 20, 128, 128, 3, seed=7601, indices="choice",
                            lengths="uniform")
    e.query = np.ascontiguousarray(np.repeat(inp.query, 4, axis=1))
    e.key = np.ascontiguousarray(np.repeat(inp.key, 4, axis=1))
    e.Hq = 16
    out_e, st_e = gpu_prefill(e)
    assert np.array_equal(dev_to_bits(out), dev_to_bits(out_e))
    assert np.array_equal(dev_to_bits(st), dev_to_bits(st_e))


def test_prefill_inplace_equals_out_of_place(rg):
    inp = workloads.make_case(3, 2, 4, 24, 128, 256, 5, seed=7701, indices="choice",
                              lengths="uniform")
    out1, st1 = gpu_prefill(inp)
    out2, st2 = gpu_prefill(inp, inplace=True)
    assert np.array_equal(dev_to_bits(out1), dev_to_bits(out2))
    assert np.array_equal(dev_to_bits(st1), dev_to_bits(st2))


def _slice_call(rg, d, inp, lo, hi, fn):
    sl = slice(lo, hi)
    n = hi - lo
    return getattr(rg, fn)(
        d["query"][:, :, sl].contiguous(), d["key"][:, :, sl].contiguous(),
        d["value"][:, :, sl].contiguous(), d["beta"][:, :, sl].contiguous(), d["pool"],
        torch.full((inp.B,), n, dtype=torch.int32, device="cuda"), d["ssm_state_indices"],
        d["g"][:, :, sl].contiguous(), d["gk"][:, :, sl].contiguous(),
        torch.full((inp.B,), n, dtype=torch.int32, device="cuda"), inp.scale)[0]


def test_prefill_chaining(rg):
    """Resuming from a committed state: two prefill calls of 32 tokens (state fed back), and
    eight decode calls of 8 tokens, each match one 64-token oracle call within the bar (the
    state is rounded to bf16 between calls), and one 64-token prefill call too."""
    inp = workloads.make_case(3, 2, 4, 64, 128, 128, 5, seed=7801, indices="choice")
    ref = oracle_decode(inp)
    out1, st1 = gpu_prefill(inp)
    check_decode(inp, out1, st1, ref, "one prefill call of 64")
    for fn, step in (("rgdr_prefill", 32), ("rgdr_decode", 8)):
        d = upload(inp)
        d["pool"] = d["state"].clone()
        outs = [_slice_call(rg, d, inp, lo, lo + step, fn) for lo in range(0, 64, step)]
        torch.cuda.synchronize()
        check_decode(inp, torch.cat(outs, dim=2), d["pool"], ref, f"{64 // step} calls ({fn})")


EXTREMES = ["strong_decay", "zero_decay", "mixed_rows", "split_rows", "growth"]


@pytest.mark.parametrize("case", EXTREMES)
def test_prefill_extreme_decays(rg, case):
    rng = np.random.default_rng(79)
    inp = workloads.make_case(4, 2, 4, 24, 128, 128, 6, seed=7901, indices="choice",
                              lengths=[24, 19, 24, 9])
    inp.num_accepted_tokens = np.array([24, 13, 16, 9], np.int32)
    if case == "strong_decay":
        inp.g[:] = -30.0
    elif case == "zero_decay":    # exp(g) is exactly 0 at token 11: the state is wiped
        inp.g[:] = -1.0
        inp.g[:, :, 11] = -1000.0
    elif case == "mixed_rows":
        inp.g[:] = rng.uniform(-25.0, 3.0, inp.g.shape).astype(np.float32)
        inp.gk[:] = -rng.uniform(0.0, 12.0, inp.gk.shape).astype(np.float32)
    elif case == "split_rows":   # rows 64.. decay by e^-10 per token, rows 0..63 mildly:
        inp.gk[:, :, :, 64:] = -10.0  # those rows alone shorten the chunks
    else:                         # exp(g) > 1 throughout: outside the operator's domain
        inp.g[:] = 2.5
    out, st = gpu_prefill(inp)
    ref = oracle_decode(inp)
    if case != "growth":
        check_decode(inp, out, st, ref, f"prefill extreme {case}")
        return
    # As for the decode's matrix-core form: finite, and within the bar plus 1e-4 of the
    # largest |value| of each (entry, head) (operands carry about 2^-17 of each value).
    out_ref, _, rows = ref
    got = bf16_dev_to_f64(out)
    assert np.all(np.isfinite(got))
    for b in range(inp.B):
        L = int(inp.actual_seq_lengths[b])
        for h in range(inp.Hv):
            r = out_ref[b, h, :L]
            assert_tol(got[b, h, :L], r, f"growth out b{b} h{h}", atol=2e-2 + 1e-4 * np.abs(r).max())
    pool = bf16_dev_to_f64(st)
    for b in range(inp.B):
        for h in range(inp.Hv):
            r = rows[b, h]
            assert_tol(pool[inp.ssm_state_indices[b], h], r, f"growth state b{b} h{h}",
                       atol=2e-2 + 1e-4 * np.abs(r).max())


def test_prefill_long_sequence(rg):
    """4096 tokens (128 chunks of 32) with ragged lengths and an accepted prefix deep in the
    sequence: errors do not accumulate past the bar over a long walk."""
    inp = workloads.make_case(2, 1, 2, 4096, 128, 128, 3, seed=7921, indices="choice",
                              lengths=[4096, 3001])
    inp.num_accepted_tokens = np.array([4096, 2777], np.int32)
    out, st = gpu_prefill(inp)
    check_decode(inp, out, st, oracle_decode(inp), "prefill T=4096")


def test_prefill_max_length(rg):
    """The longest sequence the call accepts, 65536 tokens (2048 chunks), two value heads
    sharing one query head: a full entry and a ragged one whose accepted prefix ends
    mid-chunk, deep in the sequence."""
    inp = workloads.make_case(2, 1, 2, 65536, 128, 128, 3, seed=7925, indices="choice",
                              lengths=[65536, 60001])
    inp.num_accepted_tokens = np.array([65536, 41234], np.int32)
    out, st = gpu_prefill(inp)
    check_decode(inp, out, st, oracle_decode(inp), "prefill T=65536")


@pytest.mark.parametrize("g_val", [-12.0, -7.0, -4.5])
def test_prefill_many_short_chunks(rg, g_val):
    """Decays strong enough that a chunk's decay products span more than 2^192 (the factored
    range around the chunk's middle) after about 11 (g = -12), 19 (g = -7) or 29 (g = -4.5)
    tokens: chunks are cut at many different positions relative to the 32-token grid, the
    accepted prefix and the ragged ends."""
    inp = workloads.make_case(3, 1, 2, 160, 128, 128, 4, seed=7911, indices="choice",
                              lengths=[160, 131, 70])
    inp.num_accepted_tokens = np.array([160, 77, 5], np.int32)
    inp.g[:] = g_val
    out, st = gpu_prefill(inp)
    check_decode(inp, out, st, oracle_decode(inp), f"prefill short chunks g={g_val}")


@pytest.mark.parametrize("dtype,norm,Dk", [(np.float32, False, 128), (np.float16, False, 128),
                                           (np.float32, True, 128), (np.float32, True, 64)])
def test_prefill_gated(rg, dtype, norm, Dk):
    """The fused gate (fp32 or fp16 projections) and the in-kernel q/k normalisation."""
    inp = workloads.make_case(3, 2, 4, 40, Dk, 192, 5, seed=8001 + Dk, indices="choice",
                              lengths="uniform", gate=True)
    if norm:  # raw projections: each head vector scaled by its own factor
        rng = np.random.default_rng(8002)
        for name in ("query", "key"):
            x = workloads.to_bf16_bits(
                (getattr(inp, name).astype(np.uint32) << 16).view(np.float32)
                * rng.uniform(0.05, 20.0, getattr(inp, name).shape[:-1] + (1,)).astype(np.float32))
            setattr(inp, name, x)
    out, st = gpu_gated(rg, inp, dtype, normalize_qk=norm, fn="rgdr_prefill_gated")
    check_gated(inp, out, st, oracle_gated(inp, dtype=dtype, normalize_qk=norm),
                f"prefill gated {dtype.__name__} norm={norm} Dk={Dk}")


def test_prefill_gated_nan_padding(rg):
    inp = workloads.make_case(3, 2, 4, 30, 128, 128, 5, seed=8101, indices="choice",
                              lengths=[30, 9, 17], gate=True)
    out0, st0 = gpu_gated(rg, inp, fn="rgdr_prefill_gated")
    for b in range(inp.B):
        L = inp.actual_seq_lengths[b]
        inp.gate_a[b, L:] = np.nan
        inp.gate_b[b, L:] = np.nan
    out1, st1 = gpu_gated(rg, inp, fn="rgdr_prefill_gated")
    assert np.array_equal(dev_to_bits(out0), dev_to_bits(out1))
    assert np.array_equal(dev_to_bits(st0), dev_to_bits(st1))
    check_gated(inp, out1, st1, oracle_gated(inp), "prefill gated NaN padding")


def test_prefill_workload5_sampled(rg):
    """The prefill workload at full size (B=16, H_q=16, H_v=32, T=1024, D=128), fused gate,
    in the launch the bench times; the oracle recomputes two sampled entries, and every
    slot no entry names is untouched."""
    inp = workloads.make_workload(5, gate_inputs=True)
    say(f"prefill workload 5: {workloads.WORKLOAD_NAMES[5]}")
    out, st = gpu_gated(rg, inp, fn="rgdr_prefill_gated")
    entries = np.array([0, 15])
    check_gated(inp, out, st, oracle_gated(inp, entries), "prefill workload 5", entries)
    untouched = np.setdiff1d(np.arange(inp.N_slots), inp.ssm_state_indices)
    assert np.array_equal(dev_to_bits(st)[untouched], inp.state[untouched])


def test_prefill_graph_replay(rg):
    """The prefill captured in a HIP graph writes the eager bytes on every replay."""
    inp = workloads.make_case(4, 2, 4, 48, 128, 128, 6, seed=8201, indices="choice",
                              lengths="uniform")
    d = upload(inp)
    out = torch.empty((inp.B, inp.Hv, inp.T, inp.Dv), dtype=torch.bfloat16, device="cuda")
    st = torch.empty_like(d["state"])

    def step():
        rg.rgdr_prefill(d["query"], d["key"], d["value"], d["beta"], d["state"],
                        d["actual_seq_lengths"], d["ssm_state_indices"], d["g"], d["gk"],
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
        assert np.array_equal(dev_to_bits(out), want_out), f"replay {rep}: out differs"
        assert np.array_equal(dev_to_bits(st), want_st), f"replay {rep}: state differs"


def test_prefill_deterministic(rg):
    inp = workloads.make_case(4, 2, 4, 40, 128, 128, 6, seed=8301, indices="choice",
                              lengths="uniform")
    a = gpu_prefill(inp)
    b = gpu_prefill(inp)
    assert np.array_equal(dev_to_bits(a[0]), dev_to_bits(b[0]))
    assert np.array_equal(dev_to_bits(a[1]), dev_to_bits(b[1]))


def test_prefill_bad_arguments_raise(rg):
    inp = workloads.make_case(2, 1, 2, 4, 128, 128, 3, seed=8401, indices="choice")
    d = upload(inp)
    with pytest.raises(RuntimeError):  # D_k = 96 is not built
        z = torch.zeros((2, 1, 4, 96), dtype=torch.bfloat16, device="cuda")
        rg.rgdr_prefill(z, z, d["value"], d["beta"],
                        torch.zeros((3, 2, 96, 128), dtype=torch.bfloat16, device="cuda"),
                        d["actual_seq_lengths"], d["ssm_state_indices"], d["g"],
                        torch.zeros((2, 2, 4, 96), device="cuda"), d["num_accepted_tokens"])


def test_prefill_decode_agree_at_T8(rg):
    """Up to 8 tokens the prefill and the decode's matrix-core form evaluate the same closed
    form; both meet the bar against the oracle, and each other within it."""
    inp = workloads.make_case(6, 2, 4, 8, 128, 128, 8, seed=8501, indices="choice",
                              lengths="uniform")
    ref = oracle_decode(inp)
    out_p, st_p = gpu_prefill(inp)
    out_d, st_d = gpu_decode(inp)
    check_decode(inp, out_p, st_p, ref, "prefill at T = 8")
    check_decode(inp, out_d, st_d, ref, "decode at T = 8")
    assert_tol(bf16_dev_to_f64(out_p), bf16_dev_to_f64(out_d), "prefill vs decode out")
