"""Host-side checks of libapmoe that need no GPU: every symbol declared in
include/apmoe.h is exported, and the weight page table's staging/validation
logic (PagedWeight, Section 3.1: q_i may only name GPU-resident planes; offload
lowers q_i before planes leave, reload raises it after they return)."""
import ctypes
import json
import os
import re

import pytest

import any_precision_weight_amd as apw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "apmoe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(apmoe_[a-z_0-9]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert _declared() == sorted(apw.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(apw.LIB_PATH)
    for name in _declared():
        assert hasattr(L, name), name


def test_status_strings_and_version():
    L = apw.lib()
    assert L.apmoe_status_string(apw.OK) == b"ok"
    assert L.apmoe_status_string(apw.NOT_RESIDENT) == b"not resident"
    assert apw.version() >= 100


def test_block_bytes_eq3():
    for (n, k) in [(28672, 4096), (4096, 14336), (1024, 256)]:
        for b in range(3, 9):
            assert apw.block_bytes(n, k, b) == n * b * k // 8 + n * (1 << b) * 2
    assert apw.block_bytes(-1, 128, 3) == -1
    assert apw.block_bytes(8, 128, 9) == -1


# fake, 16-byte aligned "device" addresses: the host logic never dereferences them
def _addr(i):
    return 0x10000000 + 256 * i


def _stage(tbl, layer, expert, kind, q, n=64, k=256, resident=0xFF, lut_levels=range(3, 9)):
    planes = [_addr(10 * (expert * 2 + kind) + p) if (resident >> p) & 1 else None for p in range(8)]
    luts = {b: _addr(1000 + 10 * (expert * 2 + kind) + b) for b in lut_levels}
    tbl.set_block(layer, expert, kind, n, k, q, planes, luts, resident_mask=resident)


def test_table_validation_rules():
    t = apw.Table(1, 2)
    for e in range(2):
        for u in range(2):
            _stage(t, 0, e, u, 5)
    assert t.validate() == apw.OK
    for bad in (9, 2):
        with pytest.raises(apw.ApmoeError) as ex:
            t.set_bits(0, 1, 0, bad)
        assert ex.value.status == apw.UNSUPPORTED
    t.set_bits(0, 1, 0, 8)
    assert t.validate() == apw.OK
    # offload plane 6: q = 8 may no longer be committed, q = 6 may
    t.set_plane(0, 1, 0, 6, None, False)
    assert t.validate() == apw.NOT_RESIDENT
    t.set_bits(0, 1, 0, 6)
    assert t.validate() == apw.OK
    # a resident bit without a pointer is not resident
    t.set_plane(0, 1, 0, 5, None, True)
    assert t.validate() == apw.NOT_RESIDENT
    t.set_plane(0, 1, 0, 5, _addr(77), True)
    assert t.validate() == apw.OK
    # misaligned plane
    t.set_plane(0, 1, 0, 2, _addr(5) + 4, True)
    assert t.validate() == apw.INVALID_ARG
    t.set_plane(0, 1, 0, 2, _addr(5), True)
    # experts of one (layer, kind) must agree on the shape
    _stage(t, 0, 0, 1, 4, n=128)
    assert t.validate() == apw.INVALID_ARG
    _stage(t, 0, 0, 1, 4)
    assert t.validate() == apw.OK
    # k must be a multiple of 128
    _stage(t, 0, 0, 0, 4, k=96)
    assert t.validate() == apw.INVALID_ARG
    # the LUT of the committed level must exist
    _stage(t, 0, 0, 0, 4, lut_levels=[3, 5, 6])
    assert t.validate() == apw.NOT_RESIDENT
    t.close()


def test_table_index_errors():
    t = apw.Table(2, 3)
    with pytest.raises(apw.ApmoeError):
        t.set_bits(2, 0, 0, 4)
    with pytest.raises(apw.ApmoeError):
        t.set_bits(0, 3, 0, 4)
    with pytest.raises(apw.ApmoeError):
        t.set_bits(0, 0, 2, 4)
    with pytest.raises(apw.ApmoeError):  # never staged
        t.set_bits(0, 0, 0, 4)
    assert t.committed_bits(1, 2, 1) == 0
    t.close()
    with pytest.raises(apw.ApmoeError):
        apw.Table(0, 4)
    with pytest.raises(apw.ApmoeError):
        apw.Table(1, 257)


def test_figure3_page_table_example():
    """Figure 3 lists page-table rows (q_i, d_i) = (5, 6) for E1 gate_up, (4, 6) for
    E1 down and (7, 8) for En gate_up, each block drawn with 8 planes b7..b0.
    Committing q_i requires planes 0..q_i-1 resident; planes at or above q_i may be
    CPU-resident, and the desired d_i is carried but not used by the kernels."""
    fx = json.load(open(os.path.join(ROOT, "tests", "golden", "fig3_page_table.json")))
    rows = fx["rows"]
    t = apw.Table(1, 2)
    for r in rows:
        e, u, q, d = r["expert"], r["kind"], r["q"], r["d"]
        # resident: exactly the planes the committed bitwidth needs
        _stage(t, 0, e, u, q, resident=(1 << q) - 1)
        assert t.validate() in (apw.OK, apw.NOT_RESIDENT)
    # the fourth block of the two experts (E2 down) is staged at q = 3 to complete the layer
    _stage(t, 0, 1, 1, 3, resident=0x07)
    assert t.validate() == apw.OK
    # raising q to d before the planes are resident must be refused (reload order)
    for r in rows:
        t.set_bits(0, r["expert"], r["kind"], r["d"])
        assert t.validate() == apw.NOT_RESIDENT
        t.set_bits(0, r["expert"], r["kind"], r["q"])
    assert t.validate() == apw.OK
    t.close()
