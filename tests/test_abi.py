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


def test_probe_library_exports_its_header():
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(cpbuild.ROOT, "include", "cp_probe.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(cpp_\w+)\s*\(", text)))
    assert names == ["cpp_gather_records", "cpp_lds_pair", "cpp_read_stream", "cpp_store_rows"]
    lib = ctypes.CDLL(cpbuild.PROBE_LIB)
    for name in names:
        assert hasattr(lib, name), name
    # argument checks come before any HIP call: hipErrorInvalidValue (1)
    f = lib.cpp_lds_pair
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_uint32] * 5 + [ctypes.c_void_p] * 2
    sink = ctypes.c_uint32(0)
    assert f(16, 0, 3, 3, 1, ctypes.addressof(sink), None) == 1   # the same lane twice
    assert f(16, 0, 3, 64, 1, ctypes.addressof(sink), None) == 1  # lane 64 of a 64-lane wave
    assert f(16, 0, 3, 4, 1, None, None) == 1                     # no sink


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
        (_desc(flags=4), cp.CP_ERR_INVALID_ARGUMENT),
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


def _mdesc(**kw):
    base = dict(struct_size=ctypes.sizeof(cp.cp_mixed_desc), d=64, nclass=2,
                bits_per_step=(ctypes.c_uint32 * 4)(4, 3, 0, 0), residency=0, rows=8, flags=0, reserved=0)
    base.update(kw)
    return cp.cp_mixed_desc(**base)


def test_mixed_create_rejects_bad_descriptors_before_touching_the_device():
    lut = (ctypes.c_uint16 * 1024)()
    cls = (ctypes.c_uint8 * 8)(0, 1, 0, 1, 1, 1, 0, 0)
    bad_cls = (ctypes.c_uint8 * 8)(0, 1, 2, 1, 1, 1, 0, 0)
    lp, cp_ = ctypes.addressof(lut), ctypes.addressof(cls)
    u4 = lambda *v: (ctypes.c_uint32 * 4)(*v)
    cases = [
        (_mdesc(struct_size=40), cp_, cp.CP_ERR_INVALID_ARGUMENT),
        (_mdesc(nclass=0), cp_, cp.CP_ERR_INVALID_ARGUMENT),
        (_mdesc(nclass=5), cp_, cp.CP_ERR_INVALID_ARGUMENT),
        (_mdesc(bits_per_step=u4(4, 3, 5, 0)), cp_, cp.CP_ERR_INVALID_ARGUMENT),  # unused class set
        (_mdesc(bits_per_step=u4(4, 7, 0, 0)), cp_, cp.CP_ERR_UNSUPPORTED),
        (_mdesc(d=96), cp_, cp.CP_ERR_UNSUPPORTED),
        (_mdesc(d=10), cp_, cp.CP_ERR_INVALID_ARGUMENT),
        (_mdesc(rows=0), cp_, cp.CP_ERR_INVALID_ARGUMENT),
        (_mdesc(residency=3), cp_, cp.CP_ERR_INVALID_ARGUMENT),
        (_mdesc(), ctypes.addressof(bad_cls), cp.CP_ERR_INVALID_ARGUMENT),  # class 2 of 2
        (_mdesc(), 0, cp.CP_ERR_INVALID_ARGUMENT),
    ]
    for desc, cls_p, want in cases:
        st, h = cp.cp_table_create_mixed(desc, lp, cls_p)
        assert (st, h) == (want, 0), (desc.d, desc.nclass, list(desc.bits_per_step))


def test_descriptor_layouts_match_the_header(tmp_path):
    # the ctypes mirrors must have the C layout (compiled with the host compiler)
    src = tmp_path / "layout.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "cp.h"\n'
                   'int main(void) { printf("%zu %zu %zu %zu %zu\\n", sizeof(cp_table_desc), '
                   'offsetof(cp_table_desc, rows), sizeof(cp_mixed_desc), offsetof(cp_mixed_desc, rows), '
                   'offsetof(cp_mixed_desc, residency)); return 0; }\n')
    exe = tmp_path / "layout"
    import subprocess
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(cpbuild.ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    got = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()
    want = [ctypes.sizeof(cp.cp_table_desc), cp.cp_table_desc.rows.offset, ctypes.sizeof(cp.cp_mixed_desc),
            cp.cp_mixed_desc.rows.offset, cp.cp_mixed_desc.residency.offset]
    assert [int(x) for x in got] == want


def test_record_range_without_a_table():
    st, _, _ = cp.cp_table_record_range(0, 0)
    assert st == cp.CP_ERR_INVALID_ARGUMENT
    st, _ = cp.cp_table_describe_mixed(0)
    assert st == cp.CP_ERR_INVALID_ARGUMENT


def test_one_hip_runtime_in_the_process():
    # the binding loads torch's HIP runtime before the library, so importing
    # the package alone (torch not yet imported) maps a single libamdhip64
    import subprocess
    import sys

    code = ("import trellis_coded_row_amd\n"
            "maps = open('/proc/self/maps').read().splitlines()\n"
            "print(len({l.split()[-1] for l in maps if 'libamdhip64' in l}))\n")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, check=True,
                         cwd=cpbuild.ROOT).stdout.split()
    assert out[-1] == "1"


def test_hot_rows_without_a_table():
    assert cp.cp_table_set_hot_rows(0, 0, 0) == cp.CP_ERR_INVALID_ARGUMENT
    assert cp.cp_table_hot_rows(0) == 0


@pytest.mark.parametrize("bad", [0x7C00, 0xFC00, 0x7E00, 0xFFFF])
def test_create_rejects_a_codebook_entry_that_is_not_finite(bad):
    # the shared codebook of a Gaussian trellis holds finite values; +-inf and
    # NaN entries are refused before any device memory is touched
    lut = (ctypes.c_uint16 * 1024)()
    lut[517] = bad
    st, h = cp.cp_table_create(_desc(), ctypes.addressof(lut))
    assert (st, h) == (cp.CP_ERR_INVALID_ARGUMENT, 0)
    cls = (ctypes.c_uint8 * 8)(0, 1, 0, 1, 1, 1, 0, 0)
    st, h = cp.cp_table_create_mixed(_mdesc(), ctypes.addressof(lut), ctypes.addressof(cls))
    assert (st, h) == (cp.CP_ERR_INVALID_ARGUMENT, 0)


def test_noalloc_limit_matches_the_header_and_null_table_is_refused():
    text = open(HEADER).read()
    m = re.search(r"#define CP_DEDUP_NOALLOC_MAX_IDS (\d+)u", text)
    assert m and int(m.group(1)) == cp.CP_DEDUP_NOALLOC_MAX_IDS
    assert cp.cp_lookup_decode_dedup_noalloc(0, 8, 1, 16, None) == cp.CP_ERR_INVALID_ARGUMENT


def test_touch_ahead_is_for_single_rate_device_tables():
    lut = (ctypes.c_uint16 * 1024)()
    st, h = cp.cp_table_create(_desc(residency=cp.CP_RESIDENCY_HOST_MAPPED, flags=cp.CP_FLAG_TOUCH_AHEAD),
                               ctypes.addressof(lut))
    assert (st, h) == (cp.CP_ERR_INVALID_ARGUMENT, 0)
    cls = (ctypes.c_uint8 * 8)(0, 1, 0, 1, 1, 1, 0, 0)
    st, h = cp.cp_table_create_mixed(_mdesc(flags=cp.CP_FLAG_TOUCH_AHEAD), ctypes.addressof(lut),
                                     ctypes.addressof(cls))
    assert (st, h) == (cp.CP_ERR_INVALID_ARGUMENT, 0)


def test_shard_entry_points_check_arguments_on_the_host():
    assert cp.cp_shard_plan_workspace_bytes(0, 4) == 0
    assert cp.cp_shard_plan_workspace_bytes(1000, 0) == 0
    assert cp.cp_shard_plan_workspace_bytes(1000, cp.CP_MAX_SHARDS + 1) == 0
    # tiles of 512 ids: 4-byte counts and 8-byte starts per tile and shard, each array padded to 256 bytes
    assert cp.cp_shard_plan_workspace_bytes(1000, 4) == 512
    assert cp.cp_shard_plan_workspace_bytes(393_216, 4) == 12_288 + 24_576
    E = cp.CP_ERR_INVALID_ARGUMENT
    ws = 1 << 20  # a stand-in address, never dereferenced: every call below fails its checks first
    plan = lambda n=8, rps=10, shards=4, ids=256, loc=256, pos=256, cnt=256, w=ws, wb=1 << 16: \
        cp.cp_shard_plan(ids, n, rps, shards, loc, pos, cnt, w, wb, None)
    assert plan(shards=0) == E
    assert plan(shards=cp.CP_MAX_SHARDS + 1) == E
    assert plan(rps=0) == E
    assert plan(rps=2**63, shards=2) == E          # shards * rows_per_shard overflows
    assert plan(n=2**31) == E
    assert plan(cnt=0) == E and plan(cnt=260) == E
    assert plan(ids=0) == E and plan(ids=260) == E
    assert plan(loc=0) == E and plan(pos=4) == E
    assert plan(w=0) == E and plan(w=ws + 16) == E
    assert plan(wb=511) == E                        # 8 ids over 4 shards need 512 bytes
    assert cp.cp_table_gather_records(0, 256, 1, 256, None) == E
    assert cp.cp_lookup_decode_staged(0, 256, 1, 256, 1, 256, None) == E
