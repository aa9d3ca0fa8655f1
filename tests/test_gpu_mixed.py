"""Mixed-rate tables on the GPU (cp_table_create_mixed + cp_lookup_decode)
against the oracle's mixed-rate lookup: f(c) bit-exact, scaled rows within
1 bf16 ulp, record ranges equal to the oracle's offsets."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import trellis_coded_row_amd as cp
import workload
from parity import assert_scaled_matches, assert_bit_exact, device_lookup, say, shape_change_sizes

pytestmark = pytest.mark.gpu

LUT = workload.lut_fp16()


def make_mixed(d, kvs, cls, packed, residency=cp.CP_RESIDENCY_DEVICE, chunk=1 << 20):
    t = cp.MixedTable(d, kvs, cls, LUT, residency=residency)
    off = workload.mixed_layout(d, kvs, cls)
    for r0 in range(0, cls.size, chunk):
        r1 = min(cls.size, r0 + chunk)
        t.upload_bytes(packed[int(off[r0]):int(off[r1])], r0, r1 - r0)
    return t


def check_mixed(t, d, kvs, cls, packed, ids, label, offsets=None, expect_bad=0):
    say(f"{label}: n={ids.shape[0]} d={d} rates={kvs} rows={cls.size}")
    exp_raw, bad = oracle.lookup_decode_mixed(LUT, packed, d, kvs, cls, ids, raw=True, offsets=offsets)
    exp, _ = oracle.lookup_decode_mixed(LUT, packed, d, kvs, cls, ids, offsets=offsets)
    assert bad == expect_bad
    got_raw = device_lookup(t, ids, raw=True)
    assert t.check() == (expect_bad == 0)
    assert_bit_exact(got_raw, exp_raw, label + " f(c)")
    got = device_lookup(t, ids)
    assert t.check() == (expect_bad == 0)
    assert_scaled_matches(got, exp, label + " rows")
    ndiff = int((got != exp).sum())
    say(f"{label}: ok (scaled rows differing from the oracle: {ndiff})")


@pytest.mark.parametrize("d", [64, 128, 256, 512])
@pytest.mark.parametrize("kvs", [(6, 5, 4, 3), (3, 6), (5,)])
def test_mixed_lookup_matches_oracle(d, kvs):
    rows = 3001
    rng = np.random.default_rng(d * 7 + len(kvs))
    cls = rng.integers(0, len(kvs), size=rows).astype(np.uint8)
    packed = workload.random_mixed_records(d, kvs, cls, seed=d + 11)
    t = make_mixed(d, kvs, cls, packed)
    # record ranges: the library's index against the oracle's running sum
    off = oracle.mixed_offsets(d, kvs, cls)
    for r in (0, 1, 31, 32, 33, 1000, rows - 1):
        assert t.record_range(r) == (int(off[r]), int(off[r + 1] - off[r])), r
    ids = np.concatenate([rng.integers(0, rows, size=2000), np.arange(rows - 40, rows), [0, 0, rows - 1]])
    check_mixed(t, d, kvs, cls, packed, ids.astype(np.int64), f"mixed d{d} {kvs}")
    # ragged batch with ids outside the table
    bad = ids[:517].copy()
    bad[::50] = rows + 5
    bad[7] = -1
    check_mixed(t, d, kvs, cls, packed, bad.astype(np.int64), f"mixed bad ids d{d} {kvs}",
                expect_bad=int(((bad < 0) | (bad >= rows)).sum()))
    st, desc = cp.cp_table_describe_mixed(t.handle)
    assert st == cp.CP_OK and desc.nclass == len(kvs) and list(desc.bits_per_step)[:len(kvs)] == list(kvs)
    t.close()


@pytest.mark.parametrize("d", [128, 512])
def test_mixed_at_every_launch_shape(d):
    kvs = (6, 4, 3)
    rows = 6007
    rng = np.random.default_rng(d + 1)
    cls = rng.integers(0, len(kvs), size=rows).astype(np.uint8)
    packed = workload.random_mixed_records(d, kvs, cls, seed=d + 21)
    t = make_mixed(d, kvs, cls, packed)
    for n in shape_change_sizes():
        ids = rng.integers(0, rows, n).astype(np.int64)
        ids[1] = -1
        check_mixed(t, d, kvs, cls, packed, ids, f"mixed d{d} n{n}", expect_bad=1)
    t.close()


def test_mixed_one_row_table_and_empty_batch():
    d, kvs = 512, (3, 6)
    cls = np.array([1], dtype=np.uint8)
    packed = workload.random_mixed_records(d, kvs, cls, seed=5)
    t = make_mixed(d, kvs, cls, packed)
    check_mixed(t, d, kvs, cls, packed, np.array([0, 0, 1, 0], dtype=np.int64), "one row", expect_bad=1)
    out = t.lookup_decode(torch.empty(0, dtype=torch.int64, device="cuda"))
    torch.cuda.synchronize()
    assert out.shape == (0, d)
    t.close()


def test_mixed_host_resident():
    d, kvs = 256, (6, 4, 3)
    rows = 5000
    cls = np.random.default_rng(3).integers(0, 3, size=rows).astype(np.uint8)
    packed = workload.random_mixed_records(d, kvs, cls, seed=12)
    t = make_mixed(d, kvs, cls, packed, residency=cp.CP_RESIDENCY_HOST_MAPPED)
    ids = workload.zipf_ids(rows, 3000, seed=4)
    check_mixed(t, d, kvs, cls, packed, ids, "mixed host-resident")
    assert (t.download(100, 50) == packed[int(t.record_range(100)[0]):int(sum(t.record_range(149)))]).all()
    t.close()


@pytest.mark.parametrize("d,kvs,host", [(64, (4, 3), False), (128, (6, 5, 4, 3), True), (256, (3, 6), False),
                                         (512, (6, 4, 3), False), (512, (5,), True)])
def test_mixed_dedup_matches_oracle(d, kvs, host):
    """Each distinct record fetched once (cp_lookup_decode_dedup on a
    mixed-rate table): rows against the oracle and bit-identical to the
    direct lookup, for batches whose distinct rows span several blocks of 32
    and several tiles of 8,192 staged rows, heavy repeats, one id, all ids the
    same, ids outside the table; each batch twice."""
    rows = 40_009
    rng = np.random.default_rng(d + 31 * len(kvs) + host)
    cls = rng.integers(0, len(kvs), size=rows).astype(np.uint8)
    packed = workload.random_mixed_records(d, kvs, cls, seed=d + 41)
    t = make_mixed(d, kvs, cls, packed, residency=cp.CP_RESIDENCY_HOST_MAPPED if host else cp.CP_RESIDENCY_DEVICE)
    try:
        off = oracle.mixed_offsets(d, kvs, cls)
        cases = {
            "zipf": workload.zipf_ids(rows, 30_000, seed=d),
            "uniform (18,000 distinct)": rng.integers(0, rows, 30_000).astype(np.int64),
            "one id": np.array([rows - 1], dtype=np.int64),
            "one row repeated": np.full(777, 12345, dtype=np.int64),
            "ragged with bad ids": rng.integers(-3, rows + 3, 5_003).astype(np.int64),
            "all bad": np.array([-1, rows, 2**40], dtype=np.int64),
        }
        for label, ids in cases.items():
            exp, nbad = oracle.lookup_decode_mixed(LUT, packed, d, kvs, cls, ids, offsets=off)
            direct = device_lookup(t, ids)
            assert t.check() == (nbad == 0)
            for rep in range(2):
                say(f"mixed dedup d{d} {kvs} {'host' if host else 'hbm'}: {label}, n={ids.size}, run {rep}")
                got = device_lookup(t, ids, dedup=True)
                assert t.check() == (nbad == 0), label
                assert_scaled_matches(got, exp, f"mixed dedup {label}")
                assert_bit_exact(got, direct, f"mixed dedup vs direct {label}")
        assert t.dedup_workspace_bytes(30_000) > 0
        # a workspace one byte short is refused
        ids = torch.zeros(4, dtype=torch.int64, device="cuda")
        out = torch.empty((4, d), dtype=torch.bfloat16, device="cuda")
        need = t.dedup_workspace_bytes(4)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        assert cp.cp_lookup_decode_dedup(t.handle, ids.data_ptr(), 4, out.data_ptr(), ws.data_ptr(), need - 1,
                                         None) == cp.CP_ERR_INVALID_ARGUMENT
    finally:
        t.close()


def test_mixed_dedup_beyond_one_pass_of_the_staging_grid():
    """More distinct rows than one pass of the staging copy's capped grid
    (32 workgroups of 4 waves per CU, 16 records a wave: 524,288 on 256 CUs)
    and than one round of the tile scan cover (d = 64, four rates)."""
    d, kvs, rows = 64, (6, 5, 4, 3), 2_000_003
    rng = np.random.default_rng(77)
    cls = rng.integers(0, len(kvs), size=rows).astype(np.uint8)
    packed = workload.random_mixed_records(d, kvs, cls, seed=78)
    t = make_mixed(d, kvs, cls, packed, chunk=1 << 22)
    try:
        ids = workload.uniform_ids(rows, 700_001, seed=79)
        assert np.unique(ids).size > 524_288
        exp, nbad = oracle.lookup_decode_mixed(LUT, packed, d, kvs, cls, ids)
        say(f"mixed dedup, {np.unique(ids).size} distinct rows")
        got = device_lookup(t, ids, dedup=True)
        assert t.check() and nbad == 0
        assert_scaled_matches(got, exp, "mixed dedup, 590 K distinct rows")
    finally:
        t.close()


@pytest.mark.parametrize("d,kvs", [(64, (6, 5, 4, 3)), (128, (3, 5)), (512, (6, 4, 3))])
def test_mixed_encode_matches_oracle(d, kvs):
    """Rows encoded on the GPU into a mixed-rate table: each row's record equals
    the oracle's heuristic encoding of that row at its own class's rate."""
    rows = 301 if d < 512 else 37
    rng = np.random.default_rng(d)
    cls = rng.integers(0, len(kvs), size=rows).astype(np.uint8)
    e = workload.gaussian_rows(rows, d, seed=500 + d).astype(np.float32)
    e[3] = 0.0                                     # a zero row
    say(f"mixed encode d={d} rates={kvs} rows={rows}")
    exp_parts = [None] * rows
    for c, kv in enumerate(kvs):
        sel = np.nonzero(cls == c)[0]
        if sel.size:
            recs, _ = oracle.encode_rows(e[sel].astype(np.float64), d, kv, LUT, mode=oracle.ENC_HEURISTIC)
            for k, r in enumerate(sel):
                exp_parts[r] = recs[k]
    exp = np.concatenate(exp_parts)
    t = cp.MixedTable(d, kvs, cls, LUT)
    t.upload_bytes(np.zeros(exp.size, dtype=np.uint8), 0, rows)
    # two calls: rows [0, 120) then the rest, the second into a sub-range
    dev = torch.from_numpy(e).cuda()
    k = min(120, rows)
    t.encode(dev[:k].contiguous(), first_row=0)
    if k < rows:
        t.encode(dev[k:].contiguous(), first_row=k)
    got = t.download()
    assert got.size == exp.size
    if not (got == exp).all():
        off = oracle.mixed_offsets(d, kvs, cls)
        bad = [r for r in range(rows) if not (got[off[r]:off[r + 1]] == exp[off[r]:off[r + 1]]).all()]
        raise AssertionError(f"{len(bad)} of {rows} records differ, first row {bad[0]} (class {cls[bad[0]]})")
    # and the table decodes them like the oracle decodes its own encoding
    check_mixed(t, d, kvs, cls, exp, np.arange(rows, dtype=np.int64)[::-1].copy(), f"decode of encoded d{d}")
    t.close()
