"""rgdr_prefill_noalloc (the allocation-free entry: the segmented form's workspace is the
library's fixed device array) against the entry it varies, rgdr_prefill_ws with a
caller's workspace, and against the fp64 oracle, on calls in a row that reuse the array.

Values: bf16 out/state_out within 2e-2 + 2e-2 |ref| of the unrounded oracle value, and the
same bits as rgdr_prefill_ws (the two run the same kernels with the same segments).
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import check_decode, dev_to_bits, oracle_decode, say, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rg():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gated_delta_rule_rgdr_amd as m
    m.library()
    return m


def call(rg, fn, inp, **kw):
    d = upload(inp)
    pool = d["state"].clone()
    out, st = getattr(rg, fn)(d["query"], d["key"], d["value"], d["beta"], pool,
                              d["actual_seq_lengths"], d["ssm_state_indices"], d["g"], d["gk"],
                              d["num_accepted_tokens"], inp.scale, **kw)
    torch.cuda.synchronize()
    return out, st


def test_noalloc_matches_workspace_entry(rg):
    """Two segmented calls in a row through the fixed array, the second smaller, then a
    call that runs in one pass; each equals rgdr_prefill_ws (or rgdr_prefill) bit for bit
    and the oracle within the bar."""
    big = workloads.make_case(2, 2, 4, 1600, 128, 128, 3, seed=8700, indices="choice",
                              lengths="uniform")
    big.actual_seq_lengths[0] = 1600
    big.num_accepted_tokens[:] = [1200, big.actual_seq_lengths[1]]
    small = workloads.make_case(1, 1, 2, 700, 128, 256, 2, seed=8701, indices="choice",
                                lengths="uniform")
    small.num_accepted_tokens[:] = [small.actual_seq_lengths[0] // 2]
    for inp, tag in ((big, "first call"), (small, "second call, smaller")):
        need = rg.rgdr_prefill_workspace_size(inp.B, inp.Hv, inp.T, inp.Dk, inp.Dv)
        say(f"noalloc {tag}: B={inp.B} H_v={inp.Hv} T={inp.T} D_v={inp.Dv}, workspace {need}")
        assert 0 < need <= 128 << 20
        out_n, st_n = call(rg, "rgdr_prefill_noalloc", inp)
        out_w, st_w = call(rg, "rgdr_prefill_ws", inp)
        assert np.array_equal(dev_to_bits(out_n), dev_to_bits(out_w)), f"{tag}: out differs"
        assert np.array_equal(dev_to_bits(st_n), dev_to_bits(st_w)), f"{tag}: state differs"
        check_decode(inp, out_n, st_n, oracle_decode(inp), f"noalloc {tag}")
    # a batch that fills the device: one pass, no scratch use
    one = workloads.make_case(20, 8, 16, 40, 128, 128, 24, seed=8702, indices="choice",
                              lengths="uniform")
    assert rg.rgdr_prefill_workspace_size(one.B, one.Hv, one.T, one.Dk, one.Dv) == 0
    out_n, st_n = call(rg, "rgdr_prefill_noalloc", one)
    out_p, st_p = call(rg, "rgdr_prefill", one)
    assert np.array_equal(dev_to_bits(out_n), dev_to_bits(out_p))
    assert np.array_equal(dev_to_bits(st_n), dev_to_bits(st_p))


def test_noalloc_allocates_nothing(rg):
    """The call leaves torch's allocator untouched when given its outputs (the library's
    own array is fixed at load time)."""
    inp = workloads.make_case(1, 2, 4, 1024, 128, 128, 2, seed=8710, indices="choice",
                              lengths="uniform")
    d = upload(inp)
    pool = d["state"].clone()
    out = torch.empty((1, 4, 1024, 128), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    before = torch.cuda.memory_stats()["allocation.all.allocated"]
    rg.rgdr_prefill_noalloc(d["query"], d["key"], d["value"], d["beta"], pool,
                            d["actual_seq_lengths"], d["ssm_state_indices"], d["g"], d["gk"],
                            d["num_accepted_tokens"], inp.scale, out=out)
    torch.cuda.synchronize()
    assert torch.cuda.memory_stats()["allocation.all.allocated"] == before
    check_decode(inp, out, pool, oracle_decode(inp), "noalloc, caller's outputs")
