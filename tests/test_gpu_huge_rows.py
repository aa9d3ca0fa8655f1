"""Row ids past 2^32: a d64, 3-bit table of 2^32 + 4,099 rows (14-byte
records, 60 GB of HBM) whose records are uploaded around rows 0, 2^31 and
2^32 only. The lookup (raw and scaled), the dedup lookup, the owner's record
gather and the shard plan must keep row ids and record offsets 64-bit all
the way; every output against the oracle on the uploaded records, bad ids
(rows, -1) included."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import trellis_coded_row_amd as cp
import workload
from parity import assert_bit_exact, assert_scaled_matches, device_lookup, say

pytestmark = pytest.mark.gpu

LUT = workload.lut_fp16(0)
D, KV = 64, 3
ROWS = (1 << 32) + 4099


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    torch.cuda.init()


def test_row_ids_past_2_32():
    R = cp.cp_record_bytes(D, KV)
    assert R == 14
    free, _ = torch.cuda.mem_get_info()
    if free < ROWS * R + (8 << 30):
        pytest.skip(f"needs {ROWS * R / 2**30:.0f} GiB of free device memory")
    # uploaded row ranges [start, start + count): the table's first rows, rows
    # around 2^31, and the last 6,147 rows, which hold 2^32 - 1 .. 2^32 + 1
    ranges = [(0, 4096), ((1 << 31) - 2048, 4096), ((1 << 32) - 2048, ROWS - ((1 << 32) - 2048))]
    say(f"a {ROWS:,}-row d{D} kv{KV} table ({ROWS * R / 2**30:.1f} GiB), records in {len(ranges)} ranges")
    t = cp.Table(ROWS, D, KV, LUT)
    try:
        parts = []
        for k, (start, count) in enumerate(ranges):
            recs = workload.random_records(count, D, KV, seed=7100 + k)
            t.upload(recs, first_row=start)
            parts.append(recs)
        small = np.concatenate(parts)  # the uploaded records, as one table for the oracle
        base = np.cumsum([0] + [c for _, c in ranges])[:-1]

        def to_small(ids: np.ndarray) -> np.ndarray:
            out = np.full(ids.shape, small.shape[0], dtype=np.int64)  # outside the small table: a bad id
            for (start, count), b in zip(ranges, base):
                inr = (ids >= start) & (ids < start + count)
                out[inr] = ids[inr] - start + b
            return out

        rng = np.random.default_rng(7200)
        edge = np.array([0, 1, 4095, (1 << 31) - 1, 1 << 31, (1 << 32) - 1, 1 << 32, (1 << 32) + 1, ROWS - 1],
                        dtype=np.int64)
        ids = np.concatenate([edge, edge[::-1],
                              rng.integers((1 << 32) - 2048, ROWS, 3000, dtype=np.int64),
                              rng.integers((1 << 31) - 2048, (1 << 31) + 2048, 1000, dtype=np.int64),
                              rng.integers(0, 4096, 1000, dtype=np.int64)])
        ids = ids[rng.permutation(ids.size)]
        ids[[3, 77]] = [ROWS, -1]  # two ids outside the table
        sids = to_small(ids)
        sids[[3, 77]] = [small.shape[0], -1]

        say(f"lookup of {ids.size} ids")
        exp_raw, bad = oracle.lookup_decode(LUT, small, small.shape[0], D, KV, sids, raw=True)
        exp, _ = oracle.lookup_decode(LUT, small, small.shape[0], D, KV, sids, raw=False)
        assert bad == 2
        assert_bit_exact(device_lookup(t, ids, raw=True), exp_raw, "f(c) past 2^32")
        assert not t.check()
        got = device_lookup(t, ids)
        assert not t.check()
        assert_scaled_matches(got, exp, "rows past 2^32")
        assert_bit_exact(device_lookup(t, ids, dedup=True), got, "dedup past 2^32")
        assert not t.check()

        say("owner's gather")
        for shift in (0, 6):
            buf = torch.full((ids.size * R + 64,), 0xEE, dtype=torch.uint8, device="cuda")
            t.gather_records(torch.from_numpy(ids).cuda(), dst=buf[shift:])
            torch.cuda.synchronize()
            g = buf.cpu().numpy()
            assert (g[shift:shift + ids.size * R].reshape(ids.size, R) ==
                    oracle.gather_records(small, small.shape[0], sids)).all(), shift
            assert (g[:shift] == 0xEE).all() and (g[shift + ids.size * R:] == 0xEE).all()
            assert not t.check()

        say("shard plan over 3 shards of 2^31 + 3 rows")
        rps = (1 << 31) + 3
        loc, pos, cnt = cp.shard_plan(torch.from_numpy(ids).cuda(), rps, 3)
        torch.cuda.synchronize()
        e_loc, e_pos, e_cnt = oracle.shard_plan(ids, rps, 3)
        assert (cnt.cpu().numpy() == e_cnt).all()
        assert (pos.cpu().numpy() == e_pos).all()
        assert (loc.cpu().numpy()[: e_loc.size] == e_loc).all()
        assert e_cnt[2] > 0  # ids past 2^32 are owned by the third shard
    finally:
        t.close()
        torch.cuda.empty_cache()
