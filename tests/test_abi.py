"""The C-ABI library without a GPU: it loads, exports every symbol the header
declares, and rejects bad arguments on the host before any HIP call."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import trellis_coded_row_amd as cp
from trellis_coded_row_amd import build as cpbuild

HEADER = os.path.join(cpbuild.ROOT, "include", "cp.h")


def declared_functions() -> list[str]:
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cp_\w+)\s*\(", text)))


def test_library_is_built_in_tree_and_loaded():
    assert os.path.exists(cpbuild.LIB)
    assert cp.load_library()._name == cpbuild.LIB


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 11
    lib = ctypes.CDLL(cpbuild.LIB)
    for name in names:
        assert hasattr(lib, name), name


def test_record_bytes_and_supported_shapes():
    for d in (64, 128, 256, 512):
        for kv in (3, 4, 5, 6):
            assert cp.cp_record_bytes(d, kv) == kv * d // 16 + 2
            assert cp.cp_supported(d, kv)
    assert cp.cp_record_bytes(10, 4) == 0  # 20 code bits: not whole bytes
    assert cp.cp_record_bytes(6, 4) == 0   # shorter than one window
    assert not cp.cp_supported(96, 4)      # a valid record shape without a kernel
    assert cp.cp_record_bytes(96, 4) == 26
    assert not cp.cp_supported(512, 7)


def test_status_strings():
    for s in range(6):
        assert cp.cp_status_string(s)
    assert cp.cp_status_string(99) == "unknown status"


def _desc(**kw):
    base = dict(struct_size=ctypes.sizeof(cp.cp_table_desc), d=64, bits_per_step=4,
                residency=0, rows=16, flags=0, reserved=0)
    base.update(kw)
    return cp.cp_table_desc(**base)


def test_create_rejects_bad_descriptors_before_touching_the_device():
    lut = (ctypes.c_uint16 * 1024)()
    lut_p = ctypes.addressof(lut)
    cases = [
        (_desc(struct_size=8), cp.CP_ERR_INVALID_ARGUMENT),
        (_desc(rows=0), cp.CP_ERR_INVALID_ARGUMENT),
        (_desc(residency=7), cp.CP_ERR_INVALID_ARGUMENT),
        (_desc(flags=2), cp.CP_ERR_INVALID_ARGUMENT),
        (_desc(reserved=1), cp.CP_ERR_INVALID_ARGUMENT),
        (_desc(d=10), cp.CP_ERR_INVALID_ARGUMENT),
        (_desc(d=96), cp.CP_ERR_UNSUPPORTED),
        (_desc(bits_per_step=7), cp.CP_ERR_UNSUPPORTED),
        (_desc(rows=2**63), cp.CP_ERR_INVALID_ARGUMENT),
    ]
    for desc, want in cases:
        st, h = cp.cp_table_create(desc, lut_p)
        assert (st, h) == (want, 0), (desc.d, desc.rows, desc.flags)
    st, h = cp.cp_table_create(_desc(), 0)
    assert st == cp.CP_ERR_INVALID_ARGUMENT and h == 0


def test_null_table_and_pointer_checks():
    assert cp.cp_table_destroy(0) == cp.CP_OK
    assert cp.cp_lookup_decode(0, 8, 1, 16, None) == cp.CP_ERR_INVALID_ARGUMENT
    assert cp.cp_lookup_decode_raw(0, 8, 1, 16, None) == cp.CP_ERR_INVALID_ARGUMENT
    assert cp.cp_table_upload(0, 0, 1, 8) == cp.CP_ERR_INVALID_ARGUMENT
    assert cp.cp_table_check(0, None) == cp.CP_ERR_INVALID_ARGUMENT
    st, _ = cp.cp_table_describe(0)
    assert st == cp.CP_ERR_INVALID_ARGUMENT


def test_binding_exposes_the_c_names():
    for name in declared_functions():
        assert callable(getattr(cp, name)), name


def test_product_code_does_not_reach_the_oracle():
    # the library and its binding neither import nor link the CPU oracle
    pkg = os.path.dirname(cp.__file__)
    for root, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(root, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "cp_oracle" not in text and "cpo_" not in text, f


def test_dedup_workspace_query_without_a_table():
    assert cp.cp_dedup_workspace_bytes(0, 1000) == 0
    assert cp.cp_lookup_decode_dedup(0, 8, 1, 16, 256, 1 << 20, None) == cp.CP_ERR_INVALID_ARGUMENT


def test_encode_and_download_without_a_table():
    assert cp.cp_encode_workspace_bytes(0, 1000) == 0
    assert cp.cp_table_encode(0, 0, 1, 16, 256, 1 << 20, None) == cp.CP_ERR_INVALID_ARGUMENT
    assert cp.cp_table_download(0, 0, 1, 16) == cp.CP_ERR_INVALID_ARGUMENT
