"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the same seeded
bytes, at the five workloads' full sizes and on edge cases.

Values: bf16 out/state_out within 2e-2 + 2e-2 |ref| of the unrounded oracle value.
Indexing (pool gather/scatter, untouched slots, varlen masking, padded +0.0 rows,
skipped entries) bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import (assert_tol, bf16_dev_to_f64, check_decode, dev_to_bits,
                      gpu_decode, oracle_decode, say, upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rg():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gated_delta_rule_rgdr_amd as m
    m.library()
    return m


# ---------------------------------------------------------------------------------------
# The five workloads at full size
# ---------------------------------------------------------------------------------------


@pytest.mark.parametrize("wid", [0, 1, 2, 3])
def test_workload_parity(rg, wid):
    say(f"workload {wid}: {workloads.WORKLOAD_NAMES[wid]}")
    inp = workloads.make_workload(wid)
    out, st = gpu_decode(inp)
    ref = oracle_decode(inp)
    check_decode(inp, out, st, ref, f"workload {wid}")


def test_workload3_nan_padding_bitexact(rg):
    """Padded tokens filled with NaN change no valid output or state, bit for bit."""
    inp = workloads.make_workload(3)
    out0, st0 = gpu_decode(inp)
    nan_bf16 = np.uint16(0x7FC0)
    for b in range(inp.B):
        L = inp.actual_seq_lengths[b]
        inp.query[b, :, L:] = nan_bf16
        inp.key[b, :, L:] = nan_bf16
        inp.value[b, :, L:] = nan_bf16
        inp.beta[b, :, L:] = nan_bf16
        inp.g[b, :, L:] = np.nan
        inp.gk[b, :, L:] = np.nan
    out1, st1 = gpu_decode(inp)
    assert np.array_equal(dev_to_bits(out0), dev_to_bits(out1))
    assert np.array_equal(dev_to_bits(st0), dev_to_bits(st1))
    ref = oracle_decode(inp)
    check_decode(inp, out1, st1, ref, "workload 3 NaN padding")


def test_chunk_form_more_items_than_resident(rg):
    """The matrix-core form with more items than the device holds at once (48 x 32 =
    1536 tiles against four per compute unit): later items start as earlier ones finish.
    Every entry is checked against the oracle."""
    inp = workloads.make_case(48, 32, 32, 8, 128, 128, 96, seed=47, indices="permutation",
                              lengths="uniform")
    say(f"chunk form, {inp.B * inp.Hv} items")
    out, st = gpu_decode(inp)
    check_decode(inp, out, st, oracle_decode(inp), "chunk form, 1536 items")


@pytest.mark.parametrize("case", ["varlen", "one_extra_round", "skips_and_half_tiles"])
def test_chunk_form_dk64_more_items_than_resident(rg, case):
    """The matrix-core form at D_k = 64 with more items than the device holds at once (six
    per compute unit): later items start as earlier ones finish. Every entry is checked
    against the oracle: the example page's head size at B = 16, H = 64, D_v = 512, T = 8
    varlen (4096 items, about 2.7 rounds); a call just past one round (1728 items); and
    skipped slots, entries with nothing accepted and half tiles (D_v = 320) among 2304
    items."""
    if case == "varlen":
        inp = workloads.make_case(16, 16, 64, 8, 64, 512, 24, seed=48, indices="choice",
                                  lengths="uniform")
    elif case == "one_extra_round":
        inp = workloads.make_case(9, 8, 64, 6, 64, 384, 9, seed=49, indices="permutation",
                                  lengths="uniform")
    else:
        inp = workloads.make_case(12, 8, 64, 8, 64, 320, 14, seed=50, indices="choice",
                                  lengths="uniform")
        inp.ssm_state_indices[[2, 7]] = [-1, 14]  # skipped entries
        inp.num_accepted_tokens[[0, 5]] = 0       # nothing accepted
        inp.num_accepted_tokens[3] = max(1, inp.actual_seq_lengths[3] - 2)
    items = inp.B * inp.Hv * ((inp.Dv + 127) // 128)
    say(f"chunk form D_k=64 ({case}): {items} items")
    out, st = gpu_decode(inp)
    check_decode(inp, out, st, oracle_decode(inp), f"chunk form D_k=64 {case}")


def test_workload4_gate_then_decode(rg):
    """la_gate feeds rgdr_decode (g fp32, beta bf16); the oracle chain uses its own gate."""
    inp = workloads.make_workload(4)
    B, Hv = inp.B, inp.Hv
    say(f"workload 4: {workloads.WORKLOAD_NAMES[4]}")
    d = upload(inp)
    a = torch.from_numpy(inp.gate_a).cuda()
    b = torch.from_numpy(inp.gate_b).cuda()
    dt = torch.from_numpy(inp.dt_bias).cuda()
    ds = torch.from_numpy(inp.decay_scale).cuda()
    g_dev, beta_dev = rg.la_gate(a, dt, ds, b, decay_dtype=torch.float32,
                                 beta_dtype=torch.bfloat16)
    pool = d["state"].clone()
    # T = 1: the gate's [B, 1, H] buffers are the [B, H, 1] layout the decode reads
    out, st = rg.rgdr_decode(d["query"], d["key"], d["value"], beta_dev.view(B, Hv, 1), pool,
                             d["actual_seq_lengths"], d["ssm_state_indices"],
                             g_dev.view(B, Hv, 1), d["gk"], d["num_accepted_tokens"], inp.scale)
    torch.cuda.synchronize()
    dec64, beta64 = oracle.la_gate(inp.gate_a, inp.dt_bias, inp.decay_scale, inp.gate_b)
    assert_tol(g_dev.cpu().numpy().astype(np.float64), dec64, "workload 4 decay", 1e-6, 1e-5)
    beta_gpu = bf16_dev_to_f64(beta_dev)
    ulp = np.exp2(np.floor(np.log2(np.abs(beta64))) - 7)
    assert np.all(np.abs(beta_gpu - beta64) <= ulp), "beta not within 1 bf16 ulp"
    g32 = dec64.astype(np.float32).reshape(B, Hv, 1)
    beta_bits = oracle.f64_to_bf16(beta64).reshape(B, Hv, 1)
    ref = oracle_decode(inp, g=g32, beta=beta_bits)
    inp.g, inp.beta = g32, beta_bits
    check_decode(inp, out, st, ref, "workload 4")


def test_page_example_shapes(rg):
    """The page's example decode shape (workload 1) returns out [1,64,1,512] and a state
    [1,64,64,512] through the functional form; the input state is left unchanged."""
    inp = workloads.make_workload(1)
    d = upload(inp)
    before = dev_to_bits(d["state"])
    out, st = rg.recurrent_gated_delta_rule(
        d["query"], d["key"], d["value"], d["beta"], d["state"], d["actual_seq_lengths"],
        d["ssm_state_indices"], d["g"], d["gk"], d["num_accepted_tokens"], scale_value=inp.scale)
    torch.cuda.synchronize()
    assert list(out.shape) == [1, 64, 1, 512]
    assert list(st.shape) == [1, 64, 64, 512]
    assert np.array_equal(dev_to_bits(d["state"]), before)
    check_decode(inp, out, st, oracle_decode(inp), "functional form")


# ---------------------------------------------------------------------------------------
# Shapes: several tiles, ragged tile counts, both D_k, T up to 8
# ---------------------------------------------------------------------------------------

SHAPES = [
    # B, Hq, Hv, T, Dk, Dv, N_slots
    (3, 2, 4, 1, 64, 64, 5),
    (2, 1, 3, 3, 64, 192, 4),     # D_k = 64 with T < 5: the per-token form, 64-wide tiles
    (2, 1, 3, 5, 64, 192, 4),     # chunk form at D_k = 64, the second tile half
    (4, 2, 2, 8, 128, 320, 6),    # chunk form, 3 tiles per row, the last one half
    (2, 4, 8, 5, 128, 384, 3),    # 128-wide tiles, 3 per row
    (5, 5, 5, 2, 128, 64, 9),
    (1, 1, 8, 8, 64, 512, 2),     # MQA; chunk form at D_k = 64
    (7, 2, 6, 4, 128, 128, 11),
    (6, 2, 4, 3, 128, 256, 8),    # T = 3 at D_k = 128: the chunk form, ragged items
    (4, 2, 4, 3, 128, 192, 7),    # T = 3 at D_k = 128, D_v = 192: chunk form, half last tile
    (9, 3, 6, 6, 128, 256, 12),   # the chunk form, 2 tiles per row
    (2, 1, 2, 1, 128, 4096, 3),   # the largest D_v: wave form, 64 tiles per row
    (2, 2, 2, 3, 128, 4096, 3),   # the largest D_v: chunk form
    (2, 1, 1, 5, 64, 4096, 2),    # the largest D_v at D_k = 64: chunk form, four row blocks
    (2, 1, 1, 4, 64, 4096, 2),    # the largest D_v at D_k = 64, T < 5: the per-token form
    (3, 1, 2, 6, 64, 576, 4),     # chunk form at D_k = 64 with a last half tile
    (3, 2, 4, 4, 128, 64, 5),     # D_v = 64 with T < 5: the per-token form
    (3, 2, 4, 6, 64, 64, 5),      # D_v = 64 with T >= 5: the chunk form, one half tile
    (40, 4, 16, 1, 64, 512, 48),  # T = 1 with more 64-column items than resident waves:
                                  # 128-column tiles at D_k = 64, two launches
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%d_Hq%d_Hv%d_T%d_Dk%d_Dv%d" % s[:6])
def test_shapes(rg, shape):
    B, Hq, Hv, T, Dk, Dv, N = shape
    inp = workloads.make_case(B, Hq, Hv, T, Dk, Dv, N, seed=hash(shape) % 2**31,
                              indices="choice", lengths="uniform")
    out, st = gpu_decode(inp)
    check_decode(inp, out, st, oracle_decode(inp), "shape %s" % (shape,))


# ---------------------------------------------------------------------------------------
# Decays far from 1 over several tokens. The multi-token kernel keeps each tile as
# diag(c) St with c the decay not yet applied, and folds c into St when c would leave
# [2^-64, 2^64]; the oracle applies every decay directly in fp64.
# ---------------------------------------------------------------------------------------


# The chunk form (T = 8, D_v = 128) and the per-token form (T = 4, D_v = 64), whose scaled
# state folds its running decay into the tile when it would leave [2^-64, 2^64].
EXTREME_FORMS = {"chunk": (8, 128, [8, 5, 8, 3], [8, 5, 6, 3], 8.0),
                 "per_token": (4, 64, [4, 3, 4, 2], [4, 3, 2, 2], 12.0)}


@pytest.mark.parametrize("form", sorted(EXTREME_FORMS))
@pytest.mark.parametrize("Dk", [128, 64])
@pytest.mark.parametrize("case", ["strong_decay", "growth", "zero_decay", "mixed_rows"])
def test_extreme_decays(rg, case, Dk, form):
    T, Dv, lens, nacc, growth = EXTREME_FORMS[form]
    rng = np.random.default_rng(61)
    inp = workloads.make_case(4, 2, 4, T, Dk, Dv, 6, seed=62, indices="choice", lengths=lens)
    inp.num_accepted_tokens = np.array(nacc, np.int32)  # one early commit
    if case == "strong_decay":    # c falls below 2^-64 every other token
        inp.g[:] = -30.0
    elif case == "growth":        # c passes 2^64 before the last token
        inp.g[:] = growth
    elif case == "zero_decay":    # exp(g) is exactly 0 at token 3: the state is wiped
        inp.g[:] = -1.0
        inp.g[:, :, 3] = -1000.0
    else:                         # every row on its own path
        inp.g[:] = rng.uniform(-25.0, 5.0, inp.g.shape).astype(np.float32)
        inp.gk[:] = -rng.uniform(0.0, 12.0, inp.gk.shape).astype(np.float32)
    say(f"extreme decays: {case}, D_k {Dk}, {form} form")
    out, st = gpu_decode(inp)
    ref = oracle_decode(inp)
    if case != "growth" or form == "per_token":
        # The per-token form computes in plain fp32 on the VALU: held to the decode bar even
        # outside the operator's domain.
        check_decode(inp, out, st, ref, f"extreme {case} Dk{Dk} {form}")
        return
    # Growth (exp(g) > 1) is outside the operator's domain (g and gk negative): states and
    # outputs grow by e^8 per token and a few outputs are near-total cancellations of terms
    # ~1e5 times larger. The chunk form's matrix-core operands carry about 2^-17 of each
    # value (bf16 high part and remainder), so its error is bounded relative to the item's
    # largest values, not to each small one. Checked here: everything finite, and each
    # output and each committed state element within the bar plus 1e-4 of the largest
    # |value| of its (entry, head).
    out_ref, _, rows = ref
    got = bf16_dev_to_f64(out)
    assert np.all(np.isfinite(got)), "non-finite output"
    for b in range(inp.B):
        L = int(inp.actual_seq_lengths[b])
        for h in range(inp.Hv):
            r = out_ref[b, h, :L]
            slack = 1e-4 * np.abs(r).max()
            assert_tol(got[b, h, :L], r, f"growth out b{b} h{h}", atol=2e-2 + slack)
    pool = bf16_dev_to_f64(st)
    assert np.all(np.isfinite(pool)), "non-finite state"
    for b in range(inp.B):
        for h in range(inp.Hv):
            r = rows[b, h]
            assert_tol(pool[inp.ssm_state_indices[b], h], r, f"growth state b{b} h{h}",
                       atol=2e-2 + 1e-4 * np.abs(r).max())


# ---------------------------------------------------------------------------------------
# Indexing semantics, bit for bit
# ---------------------------------------------------------------------------------------


def small_case(seed=5, B=6, T=4, lengths="uniform", Dv=128, **kw):
    return workloads.make_case(B, 2, 4, T, 128, Dv, 10, seed=seed, indices="choice",
                               lengths=lengths, **kw)


# (T, D_v) that select each kernel form: the wave form (T = 1), the chunk form (T > 1, D_v a
# multiple of 128), the chunk form with a last half tile (D_v = 192) and the per-token
# multi-token form (D_v = 64 with T < 5)
FORMS = {"wave": (1, 128), "chunk": (4, 128), "chunk_half": (3, 192), "per_token": (3, 64)}


@pytest.mark.parametrize("form", sorted(FORMS))
def test_permutation_equivariance(rg, form):
    T, Dv = FORMS[form]
    inp = small_case(T=T, Dv=Dv)
    out, st = gpu_decode(inp)
    perm = np.array([3, 0, 5, 1, 4, 2])
    p = small_case(T=T, Dv=Dv)
    for name in ("query", "key", "value", "beta", "g", "gk", "ssm_state_indices",
                 "actual_seq_lengths", "num_accepted_tokens"):
        setattr(p, name, np.ascontiguousarray(getattr(inp, name)[perm]))
    out_p, st_p = gpu_decode(p)
    assert np.array_equal(dev_to_bits(out_p), dev_to_bits(out)[perm])
    assert np.array_equal(dev_to_bits(st_p), dev_to_bits(st))


@pytest.mark.parametrize("form", sorted(FORMS))
def test_out_of_range_slot_skips_row(rg, form):
    T, Dv = FORMS[form]
    inp = small_case(T=T, Dv=Dv)
    out, st = gpu_decode(inp)
    bad = small_case(T=T, Dv=Dv)
    bad.ssm_state_indices = inp.ssm_state_indices.copy()
    bad.ssm_state_indices[1] = -1
    bad.ssm_state_indices[4] = inp.N_slots + 5
    out_b, st_b = gpu_decode(bad)
    ob = dev_to_bits(out_b)
    assert np.all(ob[[1, 4]] == 0)
    keep = [0, 2, 3, 5]
    assert np.array_equal(ob[keep], dev_to_bits(out)[keep])
    sb = dev_to_bits(st_b)
    for b in (1, 4):
        s = inp.ssm_state_indices[b]
        assert np.array_equal(sb[s], inp.state[s])  # the row's own slot was not written
    for b in keep:
        s = inp.ssm_state_indices[b]
        assert np.array_equal(sb[s], dev_to_bits(st)[s])
    check_decode(bad, out_b, st_b, oracle_decode(bad), f"out-of-range slots ({form})")


@pytest.mark.parametrize("form", sorted(FORMS))
def test_gqa_expansion_bitexact(rg, form):
    """Value head h reads query/key head floor(h H_q / H_v): expanding the shared heads
    and calling with H_q = H_v gives identical bytes."""
    T, Dv = FORMS[form]
    inp = workloads.make_case(3, 4, 16, T, 128, Dv, 4, seed=9, indices="choice")
    out, st = gpu_decode(inp)
    e = workloads.make_case(3, 4, 16, T, 128, Dv, 4, seed=9, indices="choice")
    e.query = np.ascontiguousarray(np.repeat(inp.query, 4, axis=1))
    e.key = np.ascontiguousarray(np.repeat(inp.key, 4, axis=1))
    e.Hq = 16
    out_e, st_e = gpu_decode(e)
    assert np.array_equal(dev_to_bits(out), dev_to_bits(out_e))
    assert np.array_equal(dev_to_bits(st), dev_to_bits(st_e))


def test_length_and_count_clamping(rg):
    inp = small_case(B=4, lengths=[-3, 11, 2, 4])
    inp.num_accepted_tokens = np.array([2, 9, -1, 4], np.int32)
    out, st = gpu_decode(inp)
    ref = small_case(B=4, lengths=[0, 4, 2, 4])
    ref.num_accepted_tokens = np.array([0, 4, 0, 4], np.int32)
    out_r, st_r = gpu_decode(ref)
    assert np.array_equal(dev_to_bits(out), dev_to_bits(out_r))
    assert np.array_equal(dev_to_bits(st), dev_to_bits(st_r))


def test_accepted_prefix_commit(rg):
    """n < L: outputs equal the n = L call; the committed state equals a call that stops
    after n tokens; both against the oracle too."""
    full = small_case(B=5, T=8, lengths=[8, 6, 5, 8, 3])
    out_f, _ = gpu_decode(full)
    acc = small_case(B=5, T=8, lengths=[8, 6, 5, 8, 3])
    acc.num_accepted_tokens = np.array([3, 6, 0, 1, 2], np.int32)
    out_a, st_a = gpu_decode(acc)
    assert np.array_equal(dev_to_bits(out_a), dev_to_bits(out_f))
    short = small_case(B=5, T=8, lengths=[8, 6, 5, 8, 3])
    short.actual_seq_lengths = acc.num_accepted_tokens.copy()
    short.num_accepted_tokens = acc.num_accepted_tokens.copy()
    _, st_s = gpu_decode(short)
    assert np.array_equal(dev_to_bits(st_a), dev_to_bits(st_s))
    check_decode(acc, out_a, st_a, oracle_decode(acc), "accepted prefix")


def test_zero_lengths_write_state_back(rg):
    inp = small_case(B=3, lengths=[0, 0, 0])
    out, st = gpu_decode(inp)
    assert np.all(dev_to_bits(out) == 0)
    assert np.array_equal(dev_to_bits(st), inp.state)


@pytest.mark.parametrize("form", sorted(FORMS))
def test_inplace_equals_out_of_place(rg, form):
    T, Dv = FORMS[form]
    inp = small_case(T=T, Dv=Dv)
    out1, st1 = gpu_decode(inp)
    out2, st2 = gpu_decode(inp, inplace=True)
    assert np.array_equal(dev_to_bits(out1), dev_to_bits(out2))
    assert np.array_equal(dev_to_bits(st1), dev_to_bits(st2))


def test_deterministic(rg):
    inp = workloads.make_workload(3)
    a = gpu_decode(inp)
    b = gpu_decode(inp)
    assert np.array_equal(dev_to_bits(a[0]), dev_to_bits(b[0]))
    assert np.array_equal(dev_to_bits(a[1]), dev_to_bits(b[1]))


def test_chaining_two_calls_of_four(rg):
    """Two T=4 calls (state fed back) match one T=8 oracle call within tolerance."""
    inp = workloads.make_case(4, 2, 4, 8, 128, 128, 6, seed=33, indices="choice",
                              lengths=[8, 8, 8, 8])
    ref = oracle_decode(inp)
    d = upload(inp)
    pool = d["state"].clone()
    outs = []
    for lo in (0, 4):
        sl = slice(lo, lo + 4)
        o, _ = rg.rgdr_decode(d["query"][:, :, sl].contiguous(), d["key"][:, :, sl].contiguous(),
                              d["value"][:, :, sl].contiguous(), d["beta"][:, :, sl].contiguous(),
                              pool, torch.full((4,), 4, dtype=torch.int32, device="cuda"),
                              d["ssm_state_indices"], d["g"][:, :, sl].contiguous(),
                              d["gk"][:, :, sl].contiguous(),
                              torch.full((4,), 4, dtype=torch.int32, device="cuda"), inp.scale)
        outs.append(o)
    torch.cuda.synchronize()
    out = torch.cat(outs, dim=2)
    check_decode(inp, out, pool, ref, "two calls of four")


def test_empty_batch_is_noop(rg):
    z = torch.empty((0, 2, 1, 128), dtype=torch.bfloat16, device="cuda")
    v = torch.empty((0, 4, 1, 128), dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros((3, 4, 128, 128), dtype=torch.bfloat16, device="cuda")
    i = torch.empty((0,), dtype=torch.int32, device="cuda")
    out, st = rg.rgdr_decode(z, z, v, v[..., 0], pool, i, i,
                             torch.empty((0, 4, 1), device="cuda"),
                             torch.empty((0, 4, 1, 128), device="cuda"), i, 1.0)
    assert out.shape == (0, 4, 1, 128)


def test_bad_arguments_raise(rg):
    inp = small_case(T=4)
    d = upload(inp)
    q9 = torch.zeros((inp.B, 2, 9, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError):
        rg.rgdr_decode(q9, q9, torch.zeros((inp.B, 4, 9, 128), dtype=torch.bfloat16, device="cuda"),
                       torch.zeros((inp.B, 4, 9), dtype=torch.bfloat16, device="cuda"), d["state"],
                       d["actual_seq_lengths"], d["ssm_state_indices"],
                       torch.zeros((inp.B, 4, 9), device="cuda"),
                       torch.zeros((inp.B, 4, 9, 128), device="cuda"), d["num_accepted_tokens"])


def test_validate_on_device(rg):
    lens = torch.tensor([3, 8, 0], dtype=torch.int32, device="cuda")
    idx = torch.tensor([5, 0, 2], dtype=torch.int32, device="cuda")
    assert rg.rgdr_validate(lens, idx, lens, 8, 6) == 0
    idx_dup = torch.tensor([5, 0, 5], dtype=torch.int32, device="cuda")
    assert rg.rgdr_validate(lens, idx_dup, lens, 8, 6) == 5
    idx_bad = torch.tensor([5, 0, 6], dtype=torch.int32, device="cuda")
    assert rg.rgdr_validate(lens, idx_bad, lens, 8, 6) == 4


def test_validate_switch_checks_each_call(rg, monkeypatch):
    """With the RGDR_VALIDATE switch on, a call whose index arrays name one slot twice
    raises before launching; valid arrays go through and match the unchecked call."""
    inp = small_case(seed=21)
    d = upload(inp)
    ref_out, ref_st = gpu_decode(inp, d)
    monkeypatch.setattr(rg, "VALIDATE", True)
    out, st = gpu_decode(inp, d)
    assert np.array_equal(dev_to_bits(out), dev_to_bits(ref_out))
    assert np.array_equal(dev_to_bits(st), dev_to_bits(ref_st))
    dup = d["ssm_state_indices"].clone()
    dup[1] = dup[0]
    with pytest.raises(RuntimeError, match="RGDR_ERR_DUPLICATE"):
        rg.rgdr_decode(d["query"], d["key"], d["value"], d["beta"], d["state"].clone(),
                       d["actual_seq_lengths"], dup, d["g"], d["gk"],
                       d["num_accepted_tokens"], inp.scale)


def test_graph_replay_matches_eager(rg):
    """The gate and the decode captured in a HIP graph give the eager bytes on every replay
    (out-of-place, so each replay starts from the same state)."""
    inp = workloads.make_workload(2, gate_inputs=True)
    B, Hv = inp.B, inp.Hv
    d = upload(inp)
    a = torch.from_numpy(inp.gate_a).cuda()
    b = torch.from_numpy(inp.gate_b).cuda()
    dt = torch.from_numpy(inp.dt_bias).cuda()
    ds = torch.from_numpy(inp.decay_scale).cuda()
    g_buf = torch.empty((B, 1, Hv), device="cuda")
    beta_buf = torch.empty((B, 1, Hv), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((B, Hv, 1, inp.Dv), dtype=torch.bfloat16, device="cuda")
    st = torch.empty_like(d["state"])

    def step():
        rg.la_gate(a, dt, ds, b, decay_dtype=torch.float32, beta_dtype=torch.bfloat16,
                   decay_out=g_buf, beta_out=beta_buf)
        rg.rgdr_decode(d["query"], d["key"], d["value"], beta_buf.view(B, Hv, 1), d["state"],
                       d["actual_seq_lengths"], d["ssm_state_indices"], g_buf.view(B, Hv, 1),
                       d["gk"], d["num_accepted_tokens"], inp.scale, out=out, state_out=st)

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
        out.zero_()
        st.copy_(d["state"])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(dev_to_bits(out), want_out), f"replay {rep}: out differs"
        assert np.array_equal(dev_to_bits(st), want_st), f"replay {rep}: state differs"


def test_concurrent_streams_and_host_threads(rg):
    """Calls on two streams at once, issued from two host threads, give the bytes of the same
    calls made one after another: a wave-form call (T = 1, several launches of the resident
    grid) and a chunk-form call (T = 8) on separate pools."""
    import threading

    cases = [workloads.make_case(96, 16, 32, 1, 128, 128, 128, seed=71, indices="choice"),
             workloads.make_case(24, 8, 16, 8, 128, 256, 30, seed=72, indices="choice",
                                 lengths="uniform")]
    devs = [upload(c) for c in cases]
    want = [gpu_decode(c, d) for c, d in zip(cases, devs)]
    got = [None, None]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    start = threading.Barrier(2)

    def run(i):
        c, d = cases[i], devs[i]
        with torch.cuda.stream(streams[i]):
            pool = d["state"].clone()
            start.wait()
            got[i] = rg.rgdr_decode(d["query"], d["key"], d["value"], d["beta"], pool,
                                    d["actual_seq_lengths"], d["ssm_state_indices"], d["g"],
                                    d["gk"], d["num_accepted_tokens"], c.scale,
                                    stream=streams[i])
            streams[i].synchronize()

    threads = [threading.Thread(target=run, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    for i in range(2):
        assert np.array_equal(dev_to_bits(got[i][0]), dev_to_bits(want[i][0])), f"case {i}: out"
        assert np.array_equal(dev_to_bits(got[i][1]), dev_to_bits(want[i][1])), f"case {i}: state"


@pytest.mark.parametrize("shape", [(40, 16, 32, 128, 128, 48), (40, 4, 16, 64, 512, 48)],
                         ids=["Dk128", "Dk64_Dv512"])
def test_single_token_wide_tiles_absent_and_rejected(rg, shape):
    """T = 1 calls large enough for 128-column tiles (more 64-column items than resident
    waves): absent tokens (L = 0) and rejected ones (n = 0) commit the incoming state bit
    for bit, out-of-range slots are skipped, and everything else meets the bar."""
    B, Hq, Hv, Dk, Dv, N = shape
    lens = np.ones(B, np.int32)
    lens[3::7] = 0
    inp = workloads.make_case(B, Hq, Hv, 1, Dk, Dv, N, seed=81, indices="choice",
                              lengths=lens)
    inp.num_accepted_tokens = lens.copy()
    inp.num_accepted_tokens[5::6] = 0
    inp.ssm_state_indices[11] = -1
    out, st = gpu_decode(inp)
    bits = dev_to_bits(st)
    for b in range(B):
        s = inp.ssm_state_indices[b]
        if 0 <= s < inp.N_slots and (lens[b] == 0 or inp.num_accepted_tokens[b] == 0):
            assert np.array_equal(bits[s], inp.state[s]), f"entry {b}: state changed"
    check_decode(inp, out, st, oracle_decode(inp), f"wide tiles {shape}")


@pytest.mark.parametrize("B", [24, 25, 33])
def test_single_token_load_order_and_tile_width_boundaries(rg, B):
    """T = 1 at H_v = 32, D = 128 around the launch-size boundaries: B = 24 reads 24 MiB of
    64-column tiles (operands first), B = 25 a little more (tile first), B = 33 no longer
    fits one launch with 64-column tiles (128-column tiles). All meet the bar."""
    inp = workloads.make_case(B, 16, 32, 1, 128, 128, B + 8, seed=90 + B, indices="choice")
    out, st = gpu_decode(inp)
    check_decode(inp, out, st, oracle_decode(inp), f"T = 1 boundaries, B = {B}")
