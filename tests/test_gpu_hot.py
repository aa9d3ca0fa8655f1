"""Hot-row copies in device memory for a table in pinned host memory
(cp_table_set_hot_rows): lookups give exactly the rows of the oracle, whether
a row is served from its device copy or from host memory."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import trellis_coded_row_amd as cp
import workload
from parity import check_lookup, make_table, say, shape_change_sizes

pytestmark = pytest.mark.gpu

LUT = workload.lut_fp16()


@pytest.mark.parametrize("d,kv", [(64, 3), (128, 4), (256, 6), (512, 4), (512, 5)])
def test_hot_rows_give_the_same_rows(d, kv):
    rows = 20_000
    recs = workload.random_records(rows, d, kv, seed=d + kv)
    t = make_table(LUT, recs, d, kv, residency=cp.CP_RESIDENCY_HOST_MAPPED)
    rng = np.random.default_rng(kv)
    hot = np.concatenate([rng.choice(rows, size=2_000, replace=False), [0, rows - 1, 0, 31, 32]])
    n_hot = t.set_hot_rows(hot)
    assert n_hot == np.unique(hot).size
    ids = np.concatenate([rng.choice(hot, size=3_000), rng.integers(0, rows, size=3_000),
                          np.arange(rows - 70, rows)]).astype(np.int64)
    rng.shuffle(ids)
    check_lookup(t, LUT, recs, d, kv, ids, f"hot rows d{d} kv{kv}")
    bad = ids[:1001].copy()
    bad[::97] = rows + 3
    bad[5] = -2
    check_lookup(t, LUT, recs, d, kv, bad, f"hot rows, bad ids d{d} kv{kv}",
                 expect_bad=int(((bad < 0) | (bad >= rows)).sum()))
    # an upload over hot and cold rows refreshes the device copies
    new = workload.random_records(rows, d, kv, seed=999, first=5_000, count=6_000)
    t.upload(new, first_row=5_000)
    recs[5_000:11_000] = new
    check_lookup(t, LUT, recs, d, kv, ids, f"hot rows after upload d{d} kv{kv}")
    # dropping the copies changes nothing either
    assert t.set_hot_rows([]) == 0
    check_lookup(t, LUT, recs, d, kv, ids[:2000], f"hot rows dropped d{d} kv{kv}")
    t.close()


@pytest.mark.parametrize("d,kv", [(256, 4), (512, 4)])
def test_hot_rows_at_every_launch_shape(d, kv):
    rows = 9_001
    recs = workload.random_records(rows, d, kv, seed=40 + d)
    t = make_table(LUT, recs, d, kv, residency=cp.CP_RESIDENCY_HOST_MAPPED)
    rng = np.random.default_rng(d)
    assert t.set_hot_rows(rng.choice(rows, size=1_500, replace=False)) == 1_500
    for n in shape_change_sizes():
        ids = rng.integers(0, rows, n, dtype=np.int64)
        ids[n // 2] = rows + 1
        check_lookup(t, LUT, recs, d, kv, ids, f"hot rows d{d} kv{kv} n{n}", expect_bad=1)
    t.close()


def test_every_row_hot_and_one_row_tables():
    d, kv, rows = 512, 4, 777
    recs = workload.random_records(rows, d, kv, seed=4)
    t = make_table(LUT, recs, d, kv, residency=cp.CP_RESIDENCY_HOST_MAPPED)
    assert t.set_hot_rows(np.arange(rows)) == rows
    check_lookup(t, LUT, recs, d, kv, np.random.default_rng(1).integers(0, rows, 999), "all rows hot")
    t.close()
    recs1 = workload.random_records(1, d, kv, seed=5)
    t = make_table(LUT, recs1, d, kv, residency=cp.CP_RESIDENCY_HOST_MAPPED)
    assert t.set_hot_rows([0]) == 1
    check_lookup(t, LUT, recs1, d, kv, np.array([0, 0, 1], dtype=np.int64), "one-row table", expect_bad=1)
    t.close()


def test_hot_rows_rejected_where_they_do_not_apply():
    d, kv = 64, 4
    t = cp.Table(64, d, kv, LUT)  # device-resident
    with pytest.raises(cp.CPError) as ei:
        t.set_hot_rows([1, 2])
    assert ei.value.status == cp.CP_ERR_UNSUPPORTED
    t.close()
    t = cp.Table(64, d, kv, LUT, residency=cp.CP_RESIDENCY_HOST_MAPPED)
    with pytest.raises(cp.CPError) as ei:
        t.set_hot_rows([1, 64])
    assert ei.value.status == cp.CP_ERR_INVALID_ARGUMENT
    assert t.set_hot_rows([3]) == 1
    rows = torch.zeros((4, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(1 << 24, dtype=torch.uint8, device="cuda")
    assert cp.cp_table_encode(t.handle, 0, 4, rows.data_ptr(), ws.data_ptr(), 1 << 24, None) == \
        cp.CP_ERR_UNSUPPORTED
    t.close()
