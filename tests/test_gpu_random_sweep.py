"""Seeded random sweep of the HIP lookup against the CPU oracle: table shape
(d, kv), table size, batch size (every launch shape), id distribution with
out-of-range ids sprinkled in, residency, touch-ahead tables, and entry
point (raw, scaled, dedup), plus mixed-rate tables and the steps of a lookup into a
row-sharded table. Each case runs twice, so a result that changed from one launch to
the next would fail as well as a wrong one."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import trellis_coded_row_amd as cp
import workload
from parity import assert_scaled_matches, assert_bit_exact, device_lookup, make_table, say, shape_change_sizes

pytestmark = pytest.mark.gpu

LUT = workload.lut_fp16(0)
CASES = 24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    torch.cuda.init()


def draw_ids(rng, rows, n):
    kind = rng.integers(0, 3)
    if kind == 0:
        ids = rng.integers(0, rows, n, dtype=np.int64)
    elif kind == 1:
        ids = workload.zipf_ids(rows, n, seed=int(rng.integers(1 << 30)))
    else:  # runs of consecutive rows (neighbouring records share cache lines)
        start = rng.integers(0, rows, (n + 15) // 16)
        ids = ((start[:, None] + np.arange(16)[None, :]) % rows).reshape(-1)[:n].astype(np.int64)
    nbad = int(rng.integers(0, 4))
    pos = rng.choice(n, size=min(nbad, n), replace=False)
    ids[pos] = rng.choice(np.array([-1, rows, rows + 7, 2**62, -(2**40)], dtype=np.int64), size=pos.size)
    return ids


def sizes():
    s = shape_change_sizes()
    return [1, 5, 96, 777, 3001, s[0], s[2], s[3], s[5]]


@pytest.mark.parametrize("case", range(CASES))
def test_random_single_rate(case):
    rng = np.random.default_rng(9000 + case)
    d = int(rng.choice([64, 128, 256, 512]))
    kv = int(rng.choice([3, 4, 5, 6]))
    rows = int(rng.choice([1, 2, 33, 1000, 20_011]))
    n = int(rng.choice(sizes()))
    host = bool(rng.random() < 0.25)
    recs = workload.random_records(rows, d, kv, seed=int(rng.integers(1 << 30)))
    ids = draw_ids(rng, rows, n)
    # every third device table touches ahead (CP_FLAG_TOUCH_AHEAD); decided by
    # the case number, so the drawn parameters stay as they were
    ahead = not host and case % 3 == 1
    label = f"case {case}: d{d} kv{kv} rows {rows} n {n} {'host' if host else 'hbm'}{' touch-ahead' if ahead else ''}"
    say(label)
    t = make_table(LUT, recs, d, kv, residency=cp.CP_RESIDENCY_HOST_MAPPED if host else cp.CP_RESIDENCY_DEVICE,
                   flags=cp.CP_FLAG_TOUCH_AHEAD if ahead else 0)
    try:
        exp_raw, nbad = oracle.lookup_decode(LUT, recs, rows, d, kv, ids, raw=True)
        exp, _ = oracle.lookup_decode(LUT, recs, rows, d, kv, ids)
        for rep in range(2):
            got_raw = device_lookup(t, ids, raw=True)
            assert t.check() == (nbad == 0), label
            assert_bit_exact(got_raw, exp_raw, f"{label} f(c) run {rep}")
            got = device_lookup(t, ids)
            assert t.check() == (nbad == 0), label
            assert_scaled_matches(got, exp, f"{label} rows run {rep}")
            got_d = device_lookup(t, ids, dedup=True)
            assert t.check() == (nbad == 0), label
            assert_bit_exact(got_d, got, f"{label} dedup run {rep}")
    finally:
        t.close()


@pytest.mark.parametrize("case", range(8))
def test_random_mixed_rate(case):
    rng = np.random.default_rng(9500 + case)
    d = int(rng.choice([64, 128, 256, 512]))
    nclass = int(rng.integers(1, 5))
    kvs = tuple(int(k) for k in rng.choice([3, 4, 5, 6], size=nclass, replace=False))
    rows = int(rng.choice([1, 31, 32, 33, 5000]))
    n = int(rng.choice(sizes()))
    cls = rng.integers(0, nclass, size=rows).astype(np.uint8)
    packed = workload.random_mixed_records(d, kvs, cls, seed=int(rng.integers(1 << 30)))
    ids = draw_ids(rng, rows, n)
    label = f"mixed case {case}: d{d} rates {kvs} rows {rows} n {n}"
    say(label)
    t = cp.MixedTable(d, kvs, cls, LUT)
    try:
        t.upload_bytes(packed, 0, rows)
        exp_raw, nbad = oracle.lookup_decode_mixed(LUT, packed, d, kvs, cls, ids, raw=True)
        exp, _ = oracle.lookup_decode_mixed(LUT, packed, d, kvs, cls, ids)
        for rep in range(2):
            got_raw = device_lookup(t, ids, raw=True)
            assert t.check() == (nbad == 0), label
            assert_bit_exact(got_raw, exp_raw, f"{label} f(c) run {rep}")
            got = device_lookup(t, ids)
            assert t.check() == (nbad == 0), label
            assert_scaled_matches(got, exp, f"{label} rows run {rep}")
            got_d = device_lookup(t, ids, dedup=True)
            assert t.check() == (nbad == 0), label
            assert_bit_exact(got_d, got, f"{label} dedup run {rep}")
    finally:
        t.close()


@pytest.mark.parametrize("case", range(10))
def test_random_sharded(case):
    """This GPU's steps of a lookup into a row-sharded table, chained over
    shard tables on one GPU (each owner's gather into its own buffer, copied
    to the requester's received buffer at the plan's offsets, as the exchange
    would), against the oracle's lookup of the whole table; the plan and the
    gathered records against the oracle's too."""
    rng = np.random.default_rng(9800 + case)
    d = int(rng.choice([64, 128, 256, 512]))
    kv = int(rng.choice([3, 4, 5, 6]))
    shards = int(rng.choice([1, 2, 3, 5, 8]))
    rps = int(rng.choice([1, 7, 1000, 6_007]))
    rows = shards * rps
    n = int(rng.choice(sizes()))
    host = bool(rng.random() < 0.25)
    recs = workload.random_records(rows, d, kv, seed=int(rng.integers(1 << 30)))
    ids = draw_ids(rng, rows, n)
    label = f"sharded case {case}: d{d} kv{kv} {shards} x {rps} rows, n {n} {'host' if host else 'hbm'}"
    say(label)
    res = cp.CP_RESIDENCY_HOST_MAPPED if host else cp.CP_RESIDENCY_DEVICE
    tables = [make_table(LUT, recs[s * rps:(s + 1) * rps], d, kv, residency=res) for s in range(shards)]
    try:
        e_loc, e_pos, e_cnt = oracle.shard_plan(ids, rps, shards)
        exp, nbad = oracle.lookup_decode(LUT, recs, rows, d, kv, ids)
        R = tables[0].record_bytes
        for rep in range(2):
            loc, pos, cnt = cp.shard_plan(torch.from_numpy(ids).cuda(), rps, shards)
            torch.cuda.synchronize()
            assert (cnt.cpu().numpy() == e_cnt).all() and (pos.cpu().numpy() == e_pos).all(), label
            assert (loc.cpu().numpy()[: e_loc.size] == e_loc).all(), label
            total = int(e_cnt.sum())
            recv = torch.zeros(total * R + 64, dtype=torch.uint8, device="cuda")
            start = 0
            for s, t in enumerate(tables):
                c = int(e_cnt[s])
                if c:
                    sent = t.gather_records(loc[start:start + c])
                    recv[start * R:(start + c) * R].copy_(sent[: c * R])
                    part = oracle.gather_records(recs[s * rps:(s + 1) * rps], rps, e_loc[start:start + c])
                    assert (sent.cpu().numpy()[: c * R].reshape(c, R) == part).all(), f"{label} shard {s}"
                start += c
            out = tables[0].lookup_decode_staged(recv, total, pos)
            torch.cuda.synchronize()
            assert tables[0].check() == (nbad == 0), label
            assert_scaled_matches(out.view(torch.int16).cpu().numpy().view(np.uint16), exp, f"{label} run {rep}")
            for t in tables[1:]:
                assert t.check(), label  # owners only ever see their own rows
    finally:
        for t in tables:
            t.close()
