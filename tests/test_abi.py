"""The C ABI without a GPU: the library loads, exports every function include/rgdr.h
declares, and rejects bad arguments on the host before launching anything.

The argument checks return before any HIP call, so the fake (never dereferenced) device
addresses used here are safe.
"""
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rgdr.h")

OK, NULL, SHAPE, UNSUP, RANGE, DUP, DTYPE, HIP, ALIGN, SCRATCH = range(10)
F32, F16, BF16 = 0, 1, 2


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    import gated_delta_rule_rgdr_amd as g
    return g.library()


def test_header_declares_the_operations():
    names = declared_functions()
    for want in ("rgdr_decode", "rgdr_decode_snapshots", "rgdr_decode_gated",
                 "rgdr_decode_gated_snapshots", "rgdr_prefill", "rgdr_prefill_gated",
                 "rgdr_prefill_ws", "rgdr_prefill_gated_ws", "rgdr_prefill_workspace_size",
                 "la_gate", "rgdr_validate", "rgdr_validate_host", "rgdr_status_string"):
        assert want in names, names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"librgdr.so does not export {name}"


def test_status_strings(lib):
    import gated_delta_rule_rgdr_amd as g
    for code in range(10):
        s = g.status_string(code)
        assert s.startswith("RGDR_")
    assert g.status_string(99) == "unknown rgdr_status"


def _decode(lib, ptrs=None, **kw):
    dims = dict(B=2, Hq=2, Hv=4, T=1, Dk=128, Dv=128, N=4)
    dims.update(kw)
    p = [0x10000] * 10 if ptrs is None else ptrs
    out = kw.get("out", 0x20000)
    so = kw.get("state_out", 0x30000)
    return lib.rgdr_decode(*p[:10], 1.0, dims["B"], dims["Hq"], dims["Hv"], dims["T"],
                           dims["Dk"], dims["Dv"], dims["N"], out, so, None)


def test_decode_argument_checks(lib):
    assert _decode(lib, ptrs=[None] + [0x10000] * 9) == NULL
    assert _decode(lib, out=None) == NULL
    assert _decode(lib, state_out=None) == NULL
    assert _decode(lib, T=9) == SHAPE          # decode only: T <= 8
    assert _decode(lib, T=0) == SHAPE
    assert _decode(lib, B=-1) == SHAPE
    assert _decode(lib, ptrs=[None] * 10, B=0, out=None, state_out=None) == OK  # empty batch
    assert _decode(lib, Hq=3, Hv=4) == SHAPE   # H_v must be a multiple of H_q
    assert _decode(lib, Hq=8, Hv=4) == SHAPE   # more query heads than value heads
    assert _decode(lib, N=0) == SHAPE
    assert _decode(lib, Dk=96) == UNSUP
    assert _decode(lib, Dk=256) == UNSUP
    assert _decode(lib, Dv=96) == UNSUP
    assert _decode(lib, Dv=4160) == UNSUP     # above the 4096 bound
    bad = [0x10000] * 10
    bad[2] = 0x10002  # value not 16-byte aligned
    assert _decode(lib, ptrs=bad) == ALIGN
    bad = [0x10000] * 10
    bad[4] = 0x10008  # state pool not 16-byte aligned
    assert _decode(lib, ptrs=bad) == ALIGN
    bad = [0x10000] * 10
    bad[7] = 0x10002  # g not 4-byte aligned
    assert _decode(lib, ptrs=bad) == ALIGN
    assert _decode(lib, out=0x20004) == ALIGN


def _snapshots(lib, ptrs=None, **kw):
    dims = dict(B=2, Hq=2, Hv=4, T=4, Dk=128, Dv=128, N=4)
    dims.update(kw)
    p = [0x10000] * 10 if ptrs is None else ptrs
    return lib.rgdr_decode_snapshots(*p[:10], 1.0, dims["B"], dims["Hq"], dims["Hv"],
                                     dims["T"], dims["Dk"], dims["Dv"], dims["N"],
                                     kw.get("out", 0x20000), kw.get("state_out", 0x30000),
                                     kw.get("snap", 0x40000), None)


def test_snapshots_argument_checks(lib):
    assert _snapshots(lib, ptrs=[None] * 10, B=0, out=None, state_out=None, snap=None) == OK
    for i in range(10):
        p = [0x10000] * 10
        p[i] = None
        assert _snapshots(lib, ptrs=p) == NULL, i
    assert _snapshots(lib, snap=None) == NULL
    assert _snapshots(lib, snap=0x40008) == ALIGN  # snapshots not 16-byte aligned
    assert _snapshots(lib, T=9) == SHAPE
    assert _snapshots(lib, Hq=3, Hv=4) == SHAPE
    assert _snapshots(lib, Dk=96) == UNSUP
    assert _snapshots(lib, Dv=96) == UNSUP
    bad = [0x10000] * 10
    bad[3] = 0x10001  # beta not 2-byte aligned
    assert _snapshots(lib, ptrs=bad) == ALIGN


def _prefill(lib, ptrs=None, **kw):
    dims = dict(B=2, Hq=2, Hv=4, T=64, Dk=128, Dv=128, N=4)
    dims.update(kw)
    p = [0x10000] * 10 if ptrs is None else ptrs
    return lib.rgdr_prefill(*p[:10], 1.0, dims["B"], dims["Hq"], dims["Hv"], dims["T"],
                            dims["Dk"], dims["Dv"], dims["N"], kw.get("out", 0x20000),
                            kw.get("state_out", 0x30000), None)


def test_prefill_argument_checks(lib):
    assert _prefill(lib, ptrs=[None] * 10, B=0, out=None, state_out=None) == OK
    for i in range(10):
        p = [0x10000] * 10
        p[i] = None
        assert _prefill(lib, ptrs=p) == NULL, i
    assert _prefill(lib, out=None) == NULL
    assert _prefill(lib, T=65537) == SHAPE        # at most 65536 tokens
    assert _prefill(lib, T=0) == SHAPE
    assert _prefill(lib, T=65536, Hv=16384, Hq=16384) == SHAPE  # T * H_v > 2^29
    assert _prefill(lib, Hq=3) == SHAPE
    assert _prefill(lib, N=0) == SHAPE
    assert _prefill(lib, Dk=96) == UNSUP
    assert _prefill(lib, Dv=96) == UNSUP
    assert _prefill(lib, Dv=4160) == UNSUP
    bad = [0x10000] * 10
    bad[0] = 0x10008  # query not 16-byte aligned
    assert _prefill(lib, ptrs=bad) == ALIGN
    bad = [0x10000] * 10
    bad[3] = 0x10001  # beta not 2-byte aligned
    assert _prefill(lib, ptrs=bad) == ALIGN
    assert _prefill(lib, state_out=0x30004) == ALIGN


def test_prefill_gated_argument_checks(lib):
    def call(ptrs=None, gdt=F32, flags=0, **kw):
        dims = dict(B=2, Hq=2, Hv=4, T=64, Dk=128, Dv=128, N=4)
        dims.update(kw)
        p = [0x10000] * 12 if ptrs is None else ptrs
        return lib.rgdr_prefill_gated(*p[:7], gdt, *p[7:12], 1.0, dims["B"], dims["Hq"],
                                      dims["Hv"], dims["T"], dims["Dk"], dims["Dv"], dims["N"],
                                      kw.get("out", 0x20000), kw.get("state_out", 0x30000),
                                      flags, None)
    assert call(ptrs=[None] * 12, B=0, out=None, state_out=None) == OK
    for i in range(12):
        p = [0x10000] * 12
        p[i] = None
        assert call(ptrs=p) == NULL, i
    assert call(gdt=BF16) == DTYPE
    assert call(T=70000) == SHAPE
    assert call(Dk=256) == UNSUP
    assert call(flags=4) == UNSUP
    p = [0x10000] * 12
    p[4] = 0x10002  # fp32 projection b not 4-byte aligned
    assert call(ptrs=p) == ALIGN


def _gated(lib, ptrs=None, gdt=F32, **kw):
    dims = dict(B=2, Hq=2, Hv=4, T=1, Dk=128, Dv=128, N=4)
    dims.update(kw)
    p = [0x10000] * 12 if ptrs is None else ptrs
    return lib.rgdr_decode_gated(*p[:7], gdt, *p[7:12], 1.0, dims["B"], dims["Hq"], dims["Hv"],
                                 dims["T"], dims["Dk"], dims["Dv"], dims["N"],
                                 kw.get("out", 0x20000), kw.get("state_out", 0x30000),
                                 kw.get("flags", 0), None)


def test_gated_decode_argument_checks(lib):
    assert _gated(lib, ptrs=[None] * 12, B=0, out=None, state_out=None) == OK  # empty batch
    for i in range(12):
        p = [0x10000] * 12
        p[i] = None
        assert _gated(lib, ptrs=p) == NULL, i
    assert _gated(lib, gdt=BF16) == DTYPE
    assert _gated(lib, T=9) == SHAPE
    assert _gated(lib, Hq=3) == SHAPE
    assert _gated(lib, Dk=32) == UNSUP
    p = [0x10000] * 12
    p[3] = 0x10002  # fp32 gate projection a not 4-byte aligned
    assert _gated(lib, ptrs=p) == ALIGN
    # fp16 needs only 2-byte alignment: the call passes the alignment check and stops at the
    # next host check (more than 2^31 items), so nothing is launched on any machine
    assert _gated(lib, ptrs=p, gdt=F16, T=2, B=1 << 20, Hq=1 << 10, Hv=1 << 10, Dv=4096) == SHAPE
    # option bits: RGDR_NORMALIZE_QK (1) is known, any other bit is refused before launch
    assert _gated(lib, flags=2) == UNSUP
    assert _gated(lib, flags=0x80000001) == UNSUP
    assert _gated(lib, ptrs=[None] * 12, B=0, out=None, state_out=None, flags=1) == OK


def _gated_snapshots(lib, ptrs=None, gdt=F32, **kw):
    dims = dict(B=2, Hq=2, Hv=4, T=4, Dk=128, Dv=128, N=4)
    dims.update(kw)
    p = [0x10000] * 12 if ptrs is None else ptrs
    return lib.rgdr_decode_gated_snapshots(
        *p[:7], gdt, *p[7:12], 1.0, dims["B"], dims["Hq"], dims["Hv"], dims["T"], dims["Dk"],
        dims["Dv"], dims["N"], kw.get("out", 0x20000), kw.get("state_out", 0x30000),
        kw.get("snap", 0x40000), kw.get("flags", 0), None)


def test_gated_snapshots_argument_checks(lib):
    assert _gated_snapshots(lib, ptrs=[None] * 12, B=0, out=None, state_out=None,
                            snap=None) == OK
    for i in range(12):
        p = [0x10000] * 12
        p[i] = None
        assert _gated_snapshots(lib, ptrs=p) == NULL, i
    assert _gated_snapshots(lib, snap=None) == NULL
    assert _gated_snapshots(lib, snap=0x40008) == ALIGN  # snapshots not 16-byte aligned
    assert _gated_snapshots(lib, gdt=BF16) == DTYPE
    assert _gated_snapshots(lib, flags=2) == UNSUP
    assert _gated_snapshots(lib, snap=None, flags=2) == UNSUP  # flags are checked first
    assert _gated_snapshots(lib, T=9) == SHAPE
    assert _gated_snapshots(lib, Hq=3) == SHAPE
    assert _gated_snapshots(lib, Dk=96) == UNSUP
    assert _gated_snapshots(lib, Dv=96) == UNSUP
    p = [0x10000] * 12
    p[4] = 0x10002  # fp32 gate projection b not 4-byte aligned
    assert _gated_snapshots(lib, ptrs=p) == ALIGN


def test_gate_argument_checks(lib):
    P = 0x10000
    assert lib.la_gate(None, P, P, P, F32, 4, 2, P, F32, P, F32, None) == NULL
    assert lib.la_gate(P, None, P, P, F32, 4, 2, P, F32, P, F32, None) == NULL
    assert lib.la_gate(P, P, P, P, F32, 4, 2, None, F32, P, F32, None) == NULL
    assert lib.la_gate(P, P, P, None, F32, 4, 2, P, F32, P, F32, None) == SHAPE  # beta needs b
    assert lib.la_gate(P, P, P, P, F32, -1, 2, P, F32, None, F32, None) == SHAPE
    assert lib.la_gate(P, P, P, P, F32, 4, 0, P, F32, None, F32, None) == SHAPE
    assert lib.la_gate(P, P, P, P, BF16, 4, 2, P, F32, None, F32, None) == DTYPE
    assert lib.la_gate(P, P, P, P, F32, 4, 2, P, BF16, None, F32, None) == DTYPE
    assert lib.la_gate(P, P, P, P, F32, 4, 2, P, F32, P, 7, None) == DTYPE
    assert lib.la_gate(P + 2, P, P, P, F32, 4, 2, P, F32, None, F32, None) == ALIGN
    # zero rows: nothing to do, nothing read or launched
    assert lib.la_gate(P, P, P, P, F32, 0, 2, P, F32, P, BF16, None) == OK
    assert lib.la_gate(None, None, None, None, F32, 0, 2, None, F32, None, F32, None) == OK
    # an unconsumed b is allowed when beta is not requested (checked before launch via n=0)
    assert lib.la_gate(P, P, P, P, F16, 0, 3, P, F16, None, F32, None) == OK


def test_validate_host():
    import gated_delta_rule_rgdr_amd as g
    T, N = 8, 6
    assert g.rgdr_validate_host([3, 8, 0], [5, 0, 2], [3, 8, 0], T, N) == OK
    assert g.rgdr_validate_host([3, 9, 0], [5, 0, 2], [3, 8, 0], T, N) == RANGE   # L > T
    assert g.rgdr_validate_host([3, -1, 0], [5, 0, 2], [3, 0, 0], T, N) == RANGE  # L < 0
    assert g.rgdr_validate_host([3, 8, 0], [5, 0, 2], [4, 8, 0], T, N) == RANGE   # n > L
    assert g.rgdr_validate_host([3, 8, 0], [5, 6, 2], [3, 8, 0], T, N) == RANGE   # slot >= N
    assert g.rgdr_validate_host([3, 8, 0], [5, -1, 2], [3, 8, 0], T, N) == RANGE  # slot < 0
    assert g.rgdr_validate_host([3, 8, 0], [5, 0, 5], [3, 8, 0], T, N) == DUP
    lib = g.library()
    assert lib.rgdr_validate_host(None, None, None, 3, T, N) == NULL
    z = np.zeros(3, np.int32)
    assert lib.rgdr_validate_host(z.ctypes.data, z.ctypes.data, z.ctypes.data, 0, T, N) == SHAPE


def test_binding_refuses_cpu_tensors():
    import torch
    import gated_delta_rule_rgdr_amd as g
    q = torch.zeros(1, 1, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(RuntimeError, match="GPU"):
        g.rgdr_decode(q, q, q, q[..., 0], q, *([torch.zeros(1, dtype=torch.int32)] * 2),
                      q.float()[..., 0], q.float(), torch.zeros(1, dtype=torch.int32))


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """With no librgdr.so the binding raises on its first call; nothing falls back to the
    CPU (the call never reaches an argument check or a computation)."""
    import torch

    import gated_delta_rule_rgdr_amd as g
    monkeypatch.setattr(g, "LIB_PATH", str(tmp_path / "librgdr.so"))
    monkeypatch.setattr(g, "_lib", None)
    with pytest.raises(ImportError, match="no fallback"):
        g.library()
    x = torch.zeros(1)
    with pytest.raises(ImportError):
        g.rgdr_decode(x, x, x, x, x, x, x, x, x, x)
    with pytest.raises(ImportError):
        g.la_gate(x, x, x)


def test_prefill_workspace_entries_argument_checks(lib):
    """The workspace size query and the workspace entries reject bad arguments before any
    HIP call (the size query needs the device only for sizes it accepts)."""
    import ctypes as C
    n = C.c_size_t(123)
    assert lib.rgdr_prefill_workspace_size(1, 4, 1024, 128, 128, None) == NULL
    assert lib.rgdr_prefill_workspace_size(1, 4, 0, 128, 128, C.byref(n)) == SHAPE
    assert n.value == 0
    assert lib.rgdr_prefill_workspace_size(1, 4, 65537, 128, 128, C.byref(n)) == SHAPE
    assert lib.rgdr_prefill_workspace_size(-1, 4, 64, 128, 128, C.byref(n)) == SHAPE
    assert lib.rgdr_prefill_workspace_size(1, 4, 64, 96, 128, C.byref(n)) == UNSUP
    assert lib.rgdr_prefill_workspace_size(1, 4, 64, 128, 96, C.byref(n)) == UNSUP
    assert lib.rgdr_prefill_workspace_size(0, 4, 64, 128, 128, C.byref(n)) == OK
    assert n.value == 0

    def call(ptrs=None, **kw):
        dims = dict(B=2, Hq=2, Hv=4, T=64, Dk=128, Dv=128, N=4)
        dims.update(kw)
        p = [0x10000] * 10 if ptrs is None else ptrs
        return lib.rgdr_prefill_ws(*p[:10], 1.0, dims["B"], dims["Hq"], dims["Hv"], dims["T"],
                                   dims["Dk"], dims["Dv"], dims["N"], kw.get("out", 0x20000),
                                   kw.get("state_out", 0x30000), 0x40000, 1 << 20, None)
    assert call(ptrs=[None] * 10, B=0, out=None, state_out=None) == OK
    for i in range(10):
        p = [0x10000] * 10
        p[i] = None
        assert call(ptrs=p) == NULL, i
    assert call(T=65537) == SHAPE
    assert call(Dk=64, Dv=100) == UNSUP
    bad = [0x10000] * 10
    bad[2] = 0x10004  # value not 16-byte aligned
    assert call(ptrs=bad) == ALIGN

    def gcall(ptrs=None, gdt=F32, flags=0, **kw):
        dims = dict(B=2, Hq=2, Hv=4, T=64, Dk=128, Dv=128, N=4)
        dims.update(kw)
        p = [0x10000] * 12 if ptrs is None else ptrs
        return lib.rgdr_prefill_gated_ws(*p[:7], gdt, *p[7:12], 1.0, dims["B"], dims["Hq"],
                                         dims["Hv"], dims["T"], dims["Dk"], dims["Dv"],
                                         dims["N"], 0x20000, 0x30000, flags, 0x40000, 1 << 20,
                                         None)
    assert gcall(ptrs=[None] * 12, B=0) == OK
    assert gcall(ptrs=[None] + [0x10000] * 11) == NULL
    assert gcall(gdt=BF16) == DTYPE
    assert gcall(flags=4) == UNSUP
    assert gcall(Hq=3) == SHAPE
