"""Lookups captured in a HIP graph and replayed: the way a serving loop runs
one decode step after another without a host launch per call. Every entry
point's launch sequence has no memset node (the dedup path clears its hash
table with a kernel), so each replay must give exactly the eager rows. Each
graph is replayed several times, with eager work on the output and a
synchronisation between replays, and every replay is compared with the CPU
oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import trellis_coded_row_amd as cp
import workload
from parity import assert_scaled_matches, assert_bit_exact, make_table, say, shape_change_sizes

pytestmark = pytest.mark.gpu

LUT = workload.lut_fp16(0)
REPLAYS = 4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    torch.cuda.init()


def replay_and_compare(step, out, expected, label, exact=False):
    """Captures step() in a graph, then replays it REPLAYS times, each time
    after overwriting the output eagerly, comparing every replay."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(REPLAYS):
        out.view(torch.int16).fill_(0x7F7F)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.view(torch.int16).cpu().numpy().view(np.uint16)
        if exact:
            assert_bit_exact(got, expected, f"{label} replay {r}")
        else:
            assert_scaled_matches(got, expected, f"{label} replay {r}")
    say(f"{label}: {REPLAYS} graph replays match the oracle")
    del g


@pytest.mark.parametrize("d,kv", [(512, 4), (256, 3), (64, 6)])
def test_lookup_replayed_from_a_graph(d, kv):
    rows = 4003
    recs = workload.random_records(rows, d, kv, seed=1200 + d + kv)
    t = make_table(LUT, recs, d, kv)
    rng = np.random.default_rng(d + kv)
    try:
        sizes = [96, shape_change_sizes()[2], shape_change_sizes()[5]]  # one per launch shape
        for n in sizes:
            ids_np = rng.integers(0, rows, n, dtype=np.int64)
            ids = torch.from_numpy(ids_np).cuda()
            exp, bad = oracle.lookup_decode(LUT, recs, rows, d, kv, ids_np)
            exp_raw, _ = oracle.lookup_decode(LUT, recs, rows, d, kv, ids_np, raw=True)
            assert bad == 0
            out = torch.empty((n, d), dtype=torch.bfloat16, device="cuda")
            replay_and_compare(lambda: t.lookup_decode(ids, out), out, exp, f"d{d} kv{kv} n{n}")
            raw = torch.empty((n, d), dtype=torch.float16, device="cuda")
            replay_and_compare(lambda: t.lookup_decode_raw(ids, raw), raw, exp_raw, f"d{d} kv{kv} n{n} raw",
                               exact=True)
            assert t.check()
    finally:
        t.close()


def test_touch_ahead_lookup_replayed_from_a_graph():
    # a batch large enough for several residency rounds, so that the first
    # round touches the later rounds' records on every replay
    d, kv, rows = 512, 4, 50_021
    recs = workload.random_records(rows, d, kv, seed=1250)
    t = make_table(LUT, recs, d, kv, flags=cp.CP_FLAG_TOUCH_AHEAD)
    try:
        n = shape_change_sizes()[5] * 3 + 11
        ids_np = workload.zipf_ids(rows, n, seed=1251)
        ids = torch.from_numpy(ids_np).cuda()
        exp, bad = oracle.lookup_decode(LUT, recs, rows, d, kv, ids_np)
        assert bad == 0
        out = torch.empty((n, d), dtype=torch.bfloat16, device="cuda")
        replay_and_compare(lambda: t.lookup_decode(ids, out), out, exp, f"touch-ahead n{n}")
        assert t.check()
    finally:
        t.close()


def test_bad_ids_in_a_graph_raise_the_flag_on_every_replay():
    d, kv, rows = 512, 4, 300
    recs = workload.random_records(rows, d, kv, seed=1300)
    t = make_table(LUT, recs, d, kv)
    try:
        ids_np = np.array([5, rows, 7, -3, 299], dtype=np.int64)
        exp, bad = oracle.lookup_decode(LUT, recs, rows, d, kv, ids_np)
        assert bad == 2
        ids = torch.from_numpy(ids_np).cuda()
        out = torch.empty((5, d), dtype=torch.bfloat16, device="cuda")
        replay_and_compare(lambda: t.lookup_decode(ids, out), out, exp, "bad ids")
        assert not t.check()  # raised by the replays, cleared by the check
        assert t.check()
    finally:
        t.close()


def test_dedup_lookup_replayed_from_a_graph():
    d, kv, rows = 512, 4, 5000
    recs = workload.random_records(rows, d, kv, seed=1400)
    t = make_table(LUT, recs, d, kv)
    try:
        ids_np = workload.zipf_ids(rows, 6000, seed=9)
        exp, _ = oracle.lookup_decode(LUT, recs, rows, d, kv, ids_np)
        ids = torch.from_numpy(ids_np).cuda()
        out = torch.empty((ids_np.size, d), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(t.dedup_workspace_bytes(ids_np.size), dtype=torch.uint8, device="cuda")
        replay_and_compare(lambda: t.lookup_decode_dedup(ids, out, workspace=ws), out, exp, "dedup zipf")
        assert t.check()
    finally:
        t.close()


def test_host_table_with_hot_rows_replayed_from_a_graph():
    d, kv, rows = 512, 4, 7000
    recs = workload.random_records(rows, d, kv, seed=1500)
    t = make_table(LUT, recs, d, kv, residency=cp.CP_RESIDENCY_HOST_MAPPED)
    try:
        rng = np.random.default_rng(15)
        t.set_hot_rows(rng.choice(rows, size=700, replace=False))
        ids_np = rng.integers(0, rows, 96, dtype=np.int64)
        exp, _ = oracle.lookup_decode(LUT, recs, rows, d, kv, ids_np)
        ids = torch.from_numpy(ids_np).cuda()
        out = torch.empty((96, d), dtype=torch.bfloat16, device="cuda")
        replay_and_compare(lambda: t.lookup_decode(ids, out), out, exp, "host table, hot rows, 96 ids")
        assert t.check()
    finally:
        t.close()


def test_mixed_rate_lookup_replayed_from_a_graph():
    d, kvs, rows = 256, (6, 4, 3), 3000
    cls = np.random.default_rng(21).integers(0, len(kvs), size=rows).astype(np.uint8)
    packed = workload.random_mixed_records(d, kvs, cls, seed=22)
    t = cp.MixedTable(d, kvs, cls, LUT)
    try:
        t.upload_bytes(packed, 0, rows)
        ids_np = np.random.default_rng(23).integers(0, rows, 2000).astype(np.int64)
        exp, _ = oracle.lookup_decode_mixed(LUT, packed, d, kvs, cls, ids_np)
        ids = torch.from_numpy(ids_np).cuda()
        out = torch.empty((ids_np.size, d), dtype=torch.bfloat16, device="cuda")
        replay_and_compare(lambda: t.lookup_decode(ids, out), out, exp, "mixed rates")
        assert t.check()
    finally:
        t.close()


def test_mixed_rate_dedup_replayed_from_a_graph():
    d, kvs, rows = 512, (6, 5, 4, 3), 9000
    cls = np.random.default_rng(31).integers(0, len(kvs), size=rows).astype(np.uint8)
    packed = workload.random_mixed_records(d, kvs, cls, seed=32)
    t = cp.MixedTable(d, kvs, cls, LUT)
    try:
        t.upload_bytes(packed, 0, rows)
        ids_np = workload.zipf_ids(rows, 7000, seed=33)
        exp, _ = oracle.lookup_decode_mixed(LUT, packed, d, kvs, cls, ids_np)
        ids = torch.from_numpy(ids_np).cuda()
        out = torch.empty((ids_np.size, d), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(t.dedup_workspace_bytes(ids_np.size), dtype=torch.uint8, device="cuda")
        replay_and_compare(lambda: t.lookup_decode_dedup(ids, out, workspace=ws), out, exp, "mixed-rate dedup")
        assert t.check()
    finally:
        t.close()


def test_sharded_steps_replayed_from_a_graph():
    """The three per-GPU steps of a lookup into a 3-shard table (plan, owner
    gather, decode of the received records), with every buffer allocated
    beforehand, captured as one graph."""
    d, kv, shards, rps = 512, 4, 3, 4001
    rows = shards * rps
    recs = workload.random_records(rows, d, kv, seed=1600)
    t = make_table(LUT, recs[:rps], d, kv)  # this GPU's shard 0
    try:
        ids_np = workload.zipf_ids(rows, 5000, seed=34)
        n = ids_np.size
        # the owner gather of every planned record from shard 0 stands in for
        # the requests of all owners, as in the benchmark: rows id % rps
        exp, _ = oracle.lookup_decode(LUT, recs[:rps], rps, d, kv, ids_np % rps)
        ids = torch.from_numpy(ids_np).cuda()
        loc = torch.empty(n, dtype=torch.int64, device="cuda")
        pos = torch.empty(n, dtype=torch.int64, device="cuda")
        cnt = torch.empty(shards, dtype=torch.int64, device="cuda")
        wsb = cp.cp_shard_plan_workspace_bytes(n, shards)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        recv = torch.zeros(n * t.record_bytes + 64, dtype=torch.uint8, device="cuda")
        out = torch.empty((n, d), dtype=torch.bfloat16, device="cuda")

        def step():
            s = torch.cuda.current_stream().cuda_stream
            assert cp.cp_shard_plan(ids.data_ptr(), n, rps, shards, loc.data_ptr(), pos.data_ptr(), cnt.data_ptr(),
                                    ws.data_ptr(), wsb, s) == cp.CP_OK
            assert cp.cp_table_gather_records(t.handle, loc.data_ptr(), n, recv.data_ptr(), s) == cp.CP_OK
            assert cp.cp_lookup_decode_staged(t.handle, recv.data_ptr(), n, pos.data_ptr(), n, out.data_ptr(),
                                              s) == cp.CP_OK

        replay_and_compare(step, out, exp, "sharded steps")
        assert t.check()
    finally:
        t.close()
