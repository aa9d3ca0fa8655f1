"""The allocation-free dedup lookup (cp_lookup_decode_dedup_noalloc), called
through the C ABI, against the dedup lookup with a caller workspace
(cp_lookup_decode_dedup): identical rows, bit for bit, on two calls in a
row, the second with a smaller batch, so the fixed scratch keeps the first
call's contents when the second starts; batches above the limit are refused.
Both entry points decode the same records; the workspace path is itself
checked against the oracle in the other GPU tests, and so is this one here."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import trellis_coded_row_amd as cp
import workload
from parity import assert_bit_exact, assert_scaled_matches, make_table, say

pytestmark = pytest.mark.gpu

LUT = workload.lut_fp16(0)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    torch.cuda.init()


def noalloc(table: cp.Table, ids: np.ndarray) -> np.ndarray:
    dev = torch.from_numpy(ids).cuda()
    out = torch.empty((ids.size, table.d), dtype=torch.bfloat16, device="cuda")
    st = cp.cp_lookup_decode_dedup_noalloc(table.handle, dev.data_ptr(), ids.size, out.data_ptr(),
                                           torch.cuda.current_stream().cuda_stream)
    assert st == cp.CP_OK, cp.cp_status_string(st)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16)


def with_workspace(table: cp.Table, ids: np.ndarray) -> np.ndarray:
    dev = torch.from_numpy(ids).cuda()
    out = table.lookup_decode_dedup(dev)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("d,kv,residency", [(512, 4, cp.CP_RESIDENCY_DEVICE), (512, 6, cp.CP_RESIDENCY_DEVICE),
                                            (256, 3, cp.CP_RESIDENCY_DEVICE), (512, 4, cp.CP_RESIDENCY_HOST_MAPPED)])
def test_noalloc_dedup_matches_the_workspace_dedup(d, kv, residency):
    rows = 30011
    recs = workload.random_records(rows, d, kv, seed=1300 + d + kv)
    t = make_table(LUT, recs, d, kv, residency=residency)
    try:
        big = workload.zipf_ids(rows, cp.CP_DEDUP_NOALLOC_MAX_IDS, seed=d + kv)  # the largest batch allowed
        big[17], big[-1] = rows, -2                                               # two ids outside the table
        small = workload.uniform_ids(rows, 4099, seed=kv)
        for label, ids, bad in (("largest batch", big, 2), ("smaller batch after it", small, 0)):
            say(f"no-alloc dedup d={d} kv={kv} residency={residency}: {label}, n={ids.size}")
            got = noalloc(t, ids)
            assert t.check() == (bad == 0)
            ref = with_workspace(t, ids)
            assert t.check() == (bad == 0)
            assert_bit_exact(got, ref, f"no-alloc vs workspace dedup, {label}")
            exp, nbad = oracle.lookup_decode(LUT, recs, rows, d, kv, ids)
            assert nbad == bad
            assert_scaled_matches(got, exp, f"no-alloc vs oracle, {label}")
    finally:
        t.close()


@pytest.mark.parametrize("d,kvs", [(512, (6, 5, 4, 3)), (128, (3, 6))])
def test_noalloc_dedup_of_a_mixed_rate_table(d, kvs):
    rows = 30011
    cls = np.random.default_rng(d).integers(0, len(kvs), size=rows).astype(np.uint8)
    packed = workload.random_mixed_records(d, kvs, cls, seed=1400 + d)
    t = cp.MixedTable(d, kvs, cls, LUT)
    try:
        t.upload_bytes(packed, 0, rows)
        big = workload.zipf_ids(rows, cp.CP_DEDUP_NOALLOC_MAX_IDS, seed=d + 1)
        big[5] = -1
        small = workload.uniform_ids(rows, 3001, seed=d + 2)
        for label, ids, bad in (("largest batch", big, 1), ("smaller batch after it", small, 0)):
            say(f"no-alloc dedup, mixed d={d} rates={kvs}: {label}, n={ids.size}")
            got = noalloc(t, ids)
            assert t.check() == (bad == 0)
            ref = with_workspace(t, ids)
            assert t.check() == (bad == 0)
            assert_bit_exact(got, ref, f"no-alloc vs workspace dedup (mixed), {label}")
            exp, nbad = oracle.lookup_decode_mixed(LUT, packed, d, kvs, cls, ids)
            assert nbad == bad
            assert_scaled_matches(got, exp, f"no-alloc vs oracle (mixed), {label}")
    finally:
        t.close()


def test_noalloc_dedup_refuses_batches_above_the_limit():
    d, kv, rows = 64, 4, 100
    t = make_table(LUT, workload.random_records(rows, d, kv, seed=3), d, kv)
    try:
        n = cp.CP_DEDUP_NOALLOC_MAX_IDS + 1
        ids = torch.zeros(n, dtype=torch.int64, device="cuda")
        out = torch.empty((n, d), dtype=torch.bfloat16, device="cuda")
        st = cp.cp_lookup_decode_dedup_noalloc(t.handle, ids.data_ptr(), n, out.data_ptr(), None)
        assert st == cp.CP_ERR_INVALID_ARGUMENT
        assert cp.cp_lookup_decode_dedup_noalloc(t.handle, ids.data_ptr(), 0, out.data_ptr(), None) == cp.CP_OK
        torch.cuda.synchronize()
    finally:
        t.close()
