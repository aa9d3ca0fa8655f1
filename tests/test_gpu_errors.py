"""The boundary's error contract on a GPU: a table too large for device
memory reports CP_ERR_OUT_OF_MEMORY without a fault, and the library keeps
working afterwards. (The host-only checks are in test_abi.py.)"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import trellis_coded_row_amd as cp
import workload
from parity import check_lookup, make_table, say

pytestmark = pytest.mark.gpu

LUT = workload.lut_fp16(0)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    torch.cuda.init()


def test_device_table_larger_than_memory_reports_out_of_memory():
    d, kv = 512, 4
    R = cp.cp_record_bytes(d, kv)
    _, total = torch.cuda.mem_get_info()
    rows = 2 * total // R  # twice the device's memory
    say(f"create a {rows * R / 2**30:.0f} GiB device table (device memory {total / 2**30:.0f} GiB)")
    lut = np.ascontiguousarray(LUT).reshape(-1)
    desc = cp.cp_table_desc(ctypes.sizeof(cp.cp_table_desc), d, kv, cp.CP_RESIDENCY_DEVICE, rows, 0, 0)
    st, h = cp.cp_table_create(desc, lut.ctypes.data)
    assert (st, h) == (cp.CP_ERR_OUT_OF_MEMORY, 0), cp.cp_status_string(st)
    assert cp.cp_last_hip_error() != 0
    with pytest.raises(cp.CPError):
        cp.Table(rows, d, kv, LUT)
    # the failure is not left pending for the caller's own error checks:
    # torch's next kernel launch and synchronisation succeed
    x = torch.arange(8, device="cuda", dtype=torch.float32) * 2
    torch.cuda.synchronize()
    assert float(x.sum()) == 56.0
    # the library and the device are still usable
    recs = workload.random_records(1000, d, kv, seed=31)
    t = make_table(LUT, recs, d, kv)
    try:
        ids = np.random.default_rng(3).integers(0, 1000, 5000, dtype=np.int64)
        check_lookup(t, LUT, recs, d, kv, ids, "after an out-of-memory create")
    finally:
        t.close()
