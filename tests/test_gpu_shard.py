"""The per-GPU steps of a lookup into a row-sharded table against the
oracle: the requester's plan (cp_shard_plan), the owner's record gather
(cp_table_gather_records), the requester's decode of received records
(cp_lookup_decode_staged), and all three chained over shards held on one
GPU, with the exchanges replaced by placing each owner's records in the
received buffer directly. Integer outputs and records bit for bit, rows bit
for bit."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import trellis_coded_row_amd as cp
import workload
from parity import assert_scaled_matches, make_table, say

pytestmark = pytest.mark.gpu

LUT = workload.lut_fp16(0)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    torch.cuda.init()


def check_plan(ids: np.ndarray, rps: int, shards: int, label: str) -> None:
    say(f"plan {label}: n={ids.size} shards={shards} rows/shard={rps}")
    loc, pos, cnt = cp.shard_plan(torch.from_numpy(ids).cuda(), rps, shards)
    torch.cuda.synchronize()
    e_loc, e_pos, e_cnt = oracle.shard_plan(ids, rps, shards)
    assert (cnt.cpu().numpy() == e_cnt).all(), label
    assert (pos.cpu().numpy() == e_pos).all(), label
    assert (loc.cpu().numpy()[: e_loc.size] == e_loc).all(), label


@pytest.mark.parametrize("shards", [1, 2, 3, 8, 64])
def test_shard_plan_matches_the_oracle(shards):
    rng = np.random.default_rng(5000 + shards)
    rps = 1_000_003
    for n in (1, 63, 1023, 1024, 1025, 3001, 70_001):
        ids = workload.zipf_ids(shards * rps, n, seed=n + shards)
        bad = rng.choice(n, size=min(3, n), replace=False)
        ids[bad] = rng.choice(np.array([-1, shards * rps, 2**62], dtype=np.int64), size=bad.size)
        check_plan(ids, rps, shards, f"zipf n{n}")
    # every id in one shard, and ids in descending order
    check_plan(np.full(5000, 2 * rps // 3, dtype=np.int64) if shards == 1 else
               np.full(5000, rps + 7, dtype=np.int64), rps, shards, "one shard")
    check_plan(np.arange(shards * rps - 1, shards * rps - 1 - 20_000, -1, dtype=np.int64).clip(0), rps, shards,
               "descending")


@pytest.mark.parametrize("shards", [3, 64])
def test_shard_plan_of_a_batch_above_a_million_ids(shards):
    # more tiles than one thread run per scan thread covers: the chunked scan
    rps = 50_000_017
    ids = workload.uniform_ids(shards * rps + 10, 1_300_003, seed=5050 + shards)  # a few ids past the last shard
    check_plan(ids, rps, shards, "1.3 M ids")


def test_shard_plan_of_an_empty_batch_zeroes_the_counts():
    counts = torch.full((8,), 77, dtype=torch.int64, device="cuda")
    st = cp.cp_shard_plan(0, 0, 10, 8, 0, 0, counts.data_ptr(), 0, 0, None)
    assert st == cp.CP_OK
    torch.cuda.synchronize()
    assert (counts.cpu().numpy() == 0).all()
    assert cp.cp_shard_plan(0, 0, 10, cp.CP_MAX_SHARDS + 1, 0, 0, counts.data_ptr(), 0, 0, None) == \
        cp.CP_ERR_INVALID_ARGUMENT
    assert cp.cp_shard_plan(0, 0, 0, 8, 0, 0, counts.data_ptr(), 0, 0, None) == cp.CP_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("d,kv,host", [(512, 4, False), (64, 5, False), (256, 3, True)])
def test_gather_records_matches_the_oracle(d, kv, host):
    rows = 20_011
    recs = workload.random_records(rows, d, kv, seed=5100 + d + kv)
    t = make_table(LUT, recs, d, kv, residency=cp.CP_RESIDENCY_HOST_MAPPED if host else cp.CP_RESIDENCY_DEVICE)
    try:
        ids = workload.zipf_ids(rows, 9_999, seed=5101)
        ids[[5, 77]] = [-3, rows]
        R = t.record_bytes
        exp = oracle.gather_records(recs, rows, ids)
        for shift in (0, 2, 6):
            # a destination starting mid-dword, and mid-line
            say(f"gather records d{d} kv{kv} {'host' if host else 'hbm'} dst+{shift}")
            buf = torch.full((ids.size * R + 64,), 0xEE, dtype=torch.uint8, device="cuda")
            t.gather_records(torch.from_numpy(ids).cuda(), dst=buf[shift:])
            torch.cuda.synchronize()
            got = buf.cpu().numpy()
            assert (got[shift:shift + ids.size * R].reshape(ids.size, R) == exp).all()
            assert (got[:shift] == 0xEE).all() and (got[shift + ids.size * R:] == 0xEE).all()  # nothing else written
            assert not t.check()  # the two bad ids raised the flag
            assert t.check()
        for n in (1, 15, 16, 17, 33):
            got = t.gather_records(torch.from_numpy(ids[:n].copy()).cuda())
            torch.cuda.synchronize()
            assert (got.cpu().numpy()[: n * R].reshape(n, R) == exp[:n]).all(), n
        t.check()
    finally:
        t.close()


def test_gather_records_beyond_one_pass_of_the_grid():
    # more records than one pass of the capped grid covers (32 workgroups of 4
    # waves per CU, 16 records a wave): the group loop strides over the rest
    d, kv, rows = 64, 3, 1_000_003
    recs = workload.random_records(rows, d, kv, seed=5150)
    t = make_table(LUT, recs, d, kv)
    try:
        ids = workload.uniform_ids(rows, 700_001, seed=5151)
        say(f"gather records, n={ids.size}")
        got = t.gather_records(torch.from_numpy(ids).cuda())
        torch.cuda.synchronize()
        R = t.record_bytes
        assert (got.cpu().numpy()[: ids.size * R].reshape(ids.size, R) == oracle.gather_records(recs, rows, ids)).all()
        assert t.check()
    finally:
        t.close()


@pytest.mark.parametrize("d,kv", [(512, 4), (512, 6), (128, 3), (64, 4)])
def test_staged_decode_matches_the_oracle(d, kv):
    nrec = 4_099
    recv = workload.random_records(nrec, d, kv, seed=5200 + d + kv)
    R = recv.shape[1]
    buf = torch.zeros(nrec * R + 64, dtype=torch.uint8, device="cuda")
    buf[: nrec * R].copy_(torch.from_numpy(recv.reshape(-1)))
    t = cp.Table(1, d, kv, LUT)  # the requester's own table: only its codebook and shape are used
    try:
        rng = np.random.default_rng(d * kv)
        pos = rng.integers(0, nrec, 20_000).astype(np.int64)
        pos[[3, 9, 11]] = [-1, nrec, 2**40]
        say(f"staged decode d{d} kv{kv}")
        got = t.lookup_decode_staged(buf, nrec, torch.from_numpy(pos).cuda())
        torch.cuda.synchronize()
        exp, bad = oracle.lookup_decode(LUT, recv, nrec, d, kv, pos)
        assert bad == 3
        assert_scaled_matches(got.view(torch.int16).cpu().numpy().view(np.uint16), exp, f"staged d{d} kv{kv}")
        assert not t.check()
        assert t.check()
    finally:
        t.close()


def sharded_lookup(tables, rps: int, ids: np.ndarray, d: int):
    """The per-GPU steps chained over shard tables held on one GPU: plan,
    each owner's gather into its slice of the received buffer, decode."""
    shards = len(tables)
    R = tables[0].record_bytes
    dev_ids = torch.from_numpy(ids).cuda()
    loc, pos, cnt = cp.shard_plan(dev_ids, rps, shards)
    counts = cnt.cpu().numpy()
    total = int(counts.sum())
    recv = torch.zeros(total * R + 64, dtype=torch.uint8, device="cuda")
    start = 0
    for s, t in enumerate(tables):
        c = int(counts[s])
        if c:
            t.gather_records(loc[start:start + c], dst=recv[start * R:])
        start += c
    return tables[0].lookup_decode_staged(recv, total, pos)


@pytest.mark.parametrize("shards", [2, 4, 7])
def test_sharded_lookup_equals_the_oracle_on_the_whole_table(shards):
    d, kv, rps = 512, 4, 12_007
    rows = shards * rps
    recs = workload.random_records(rows, d, kv, seed=5300 + shards)
    tables = [make_table(LUT, recs[s * rps:(s + 1) * rps], d, kv) for s in range(shards)]
    try:
        for n in (96, 5_000, 100_003):
            ids = workload.zipf_ids(rows, n, seed=5301 + n)
            ids[: min(2, n)] = [-1, rows][: min(2, n)]
            say(f"sharded lookup: {shards} shards, n={n}")
            got = sharded_lookup(tables, rps, ids, d)
            torch.cuda.synchronize()
            exp, bad = oracle.lookup_decode(LUT, recs, rows, d, kv, ids)
            assert bad == min(2, n)
            assert_scaled_matches(got.view(torch.int16).cpu().numpy().view(np.uint16), exp,
                                  f"sharded {shards} n{n}")
            assert not tables[0].check()  # ids owned by no shard decode to zero rows and raise the flag
    finally:
        for t in tables:
            t.close()
