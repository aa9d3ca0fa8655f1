"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times: every output of each 393,216-lookup replay is compared with
the CPU oracle (raw f(c) and scaled rows bit-exact).

Encoded rows are encoded by the oracle here: rows 0..4095 of each rate-sweep
table, and the 16,384 most looked-up rows of the 1,048,576-row d256 table
(84% of its replay's lookups; all of its rows would take the oracle about a
quarter of an hour on 16 threads, so the benchmark encodes that table on the
GPU and checks a sample against the oracle)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import trellis_coded_row_amd as cp
import workload
from parity import assert_scaled_matches, check_lookup, device_lookup, make_table, say

pytestmark = pytest.mark.gpu

LUT = workload.lut_fp16(0)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    torch.cuda.init()


def encoder(cfg):
    return lambda e: oracle.encode_rows(e, cfg.d, cfg.kv, LUT, oracle.ENC_HEURISTIC)[0]


SMALL_ENCODED = 16384


def test_small_d256_replay():
    cfg = workload.CONFIGS["small_d256"]
    say(f"building the 1,048,576 x d256 table ({SMALL_ENCODED} hottest rows encoded by the oracle)")
    recs = workload.build_records(cfg, encode_fn=encoder(cfg), encode_limit=SMALL_ENCODED)
    t = make_table(LUT, recs, cfg.d, cfg.kv)
    try:
        ids = cfg.ids()
        assert np.isin(ids, cfg.encoded_row_ids(SMALL_ENCODED)).mean() > 0.8
        check_lookup(t, LUT, recs, cfg.d, cfg.kv, ids, "small_d256 zipf replay")
        check_lookup(t, LUT, recs, cfg.d, cfg.kv, cfg.encoded_row_ids(SMALL_ENCODED), "small_d256 encoded rows")
    finally:
        t.close()


@pytest.mark.parametrize("kv", [3, 4, 5, 6])
def test_rate_sweep_replay(kv):
    cfg = workload.CONFIGS[f"rate_d512_kv{kv}"]
    say(f"building the 4,194,304 x d512 table at kv={kv}")
    recs = workload.build_records(cfg, encode_fn=encoder(cfg))
    t = make_table(LUT, recs, cfg.d, cfg.kv)
    try:
        check_lookup(t, LUT, recs, cfg.d, cfg.kv, cfg.ids(), f"rate kv{kv} zipf replay")
        check_lookup(t, LUT, recs, cfg.d, cfg.kv, cfg.encoded_row_ids(), f"rate kv{kv} encoded rows (0..4095)")
    finally:
        t.close()


@pytest.fixture(scope="module")
def big_records():
    cfg = workload.CONFIGS["gpu_d512"]
    say("generating the 97,690,000 x d512 records (12.70 GB)")
    recs = workload.build_records(cfg)
    yield cfg, recs
    del recs


def test_gpu_d512_replays(big_records):
    cfg, recs = big_records
    t = make_table(LUT, recs, cfg.d, cfg.kv)
    try:
        check_lookup(t, LUT, recs, cfg.d, cfg.kv, cfg.ids(), "gpu_d512 zipf replay", dedup=True)
        check_lookup(t, LUT, recs, cfg.d, cfg.kv, cfg.uniform_variant_ids(), "gpu_d512 uniform replay")
    finally:
        t.close()
        torch.cuda.empty_cache()


def test_gpu_d512_sharded_replay(big_records):
    """The benchmark's sharded workload: the 12.70 GB table as shard 0 of 4 x
    97,690,000 rows, the replay's ids Zipf over all four shards. This GPU's
    steps in full: the plan of the whole replay (bit-exact), the owner's
    gather of every planned record from this table (bit-exact) and the
    decode of the gathered buffer (every row against the oracle)."""
    cfg, recs = big_records
    shards, rps = 4, cfg.rows
    ids = workload.zipf_ids(shards * rps, cfg.n_ids, cfg.ids_seed)
    t = make_table(LUT, recs, cfg.d, cfg.kv)
    try:
        say("sharded replay: plan")
        loc, pos, cnt = cp.shard_plan(torch.from_numpy(ids).cuda(), rps, shards)
        e_loc, e_pos, e_cnt = oracle.shard_plan(ids, rps, shards)
        torch.cuda.synchronize()
        assert (cnt.cpu().numpy() == e_cnt).all() and (pos.cpu().numpy() == e_pos).all()
        assert (loc.cpu().numpy() == e_loc).all()
        say("sharded replay: owner gather of all planned records")
        recv = t.gather_records(loc)
        torch.cuda.synchronize()
        R = t.record_bytes
        got = recv.cpu().numpy()[: ids.size * R].reshape(ids.size, R)
        assert (got == oracle.gather_records(recs, rps, e_loc)).all()
        say("sharded replay: staged decode")
        out = t.lookup_decode_staged(recv, ids.size, pos)
        torch.cuda.synchronize()
        exp, bad = oracle.lookup_decode(LUT, recs, rps, cfg.d, cfg.kv, ids % rps)
        assert bad == 0 and t.check()
        assert_scaled_matches(out.view(torch.int16).cpu().numpy().view(np.uint16), exp, "sharded gpu_d512 replay")
    finally:
        t.close()
        torch.cuda.empty_cache()


def test_host_d512_replay(big_records):
    cfg, recs = big_records
    hcfg = workload.CONFIGS["host_d512"]
    t = make_table(LUT, recs, cfg.d, cfg.kv, residency=cp.CP_RESIDENCY_HOST_MAPPED)
    try:
        ids = hcfg.ids()
        check_lookup(t, LUT, recs, cfg.d, cfg.kv, ids, "host_d512 zipf replay", dedup=True)
        check_lookup(t, LUT, recs, cfg.d, cfg.kv, ids[:96], "host_d512 one-token slice", dedup=True)
    finally:
        t.close()


def test_mixed_d512_replay():
    """The 97.69 M-row mixed-rate table (rates by Zipf access rank), the whole
    replay compared with the oracle's mixed-rate lookup."""
    from test_gpu_mixed import check_mixed, make_mixed

    cfg = workload.CONFIGS["mixed_d512"]
    kvs = cfg.extra["kv_of_class"]
    say("building the 97,690,000-row mixed-rate table")
    cls = workload.rank_classes(cfg.rows, cfg.ids_seed, cfg.extra["shares"])
    packed = workload.random_mixed_records(cfg.d, kvs, cls, cfg.table_seed)
    off = oracle.mixed_offsets(cfg.d, kvs, cls)
    t = make_mixed(cfg.d, kvs, cls, packed, chunk=1 << 24)
    try:
        for r in (0, 12_345_678, cfg.rows - 1):
            assert t.record_range(r) == (int(off[r]), int(off[r + 1] - off[r]))
        check_mixed(t, cfg.d, kvs, cls, packed, cfg.ids(), "mixed_d512 zipf replay", offsets=off)
        say("mixed_d512 zipf replay, each distinct record fetched once")
        exp, _ = oracle.lookup_decode_mixed(LUT, packed, cfg.d, kvs, cls, cfg.ids(), offsets=off)
        got = device_lookup(t, cfg.ids(), dedup=True)
        assert t.check()
        assert_scaled_matches(got, exp, "mixed_d512 zipf replay, dedup")
    finally:
        t.close()


def test_host_mixed_d512_replay_dedup():
    """The same mixed-rate table in pinned host memory, the replay with each
    distinct record fetched once over PCIe, against the oracle."""
    from test_gpu_mixed import make_mixed

    cfg = workload.CONFIGS["host_mixed_d512"]
    kvs = cfg.extra["kv_of_class"]
    say("building the 97,690,000-row mixed-rate table in pinned host memory")
    cls = workload.rank_classes(cfg.rows, cfg.ids_seed, cfg.extra["shares"])
    packed = workload.random_mixed_records(cfg.d, kvs, cls, cfg.table_seed)
    off = oracle.mixed_offsets(cfg.d, kvs, cls)
    t = make_mixed(cfg.d, kvs, cls, packed, residency=cp.CP_RESIDENCY_HOST_MAPPED, chunk=1 << 24)
    try:
        exp, _ = oracle.lookup_decode_mixed(LUT, packed, cfg.d, kvs, cls, cfg.ids(), offsets=off)
        got = device_lookup(t, cfg.ids(), dedup=True)
        assert t.check()
        assert_scaled_matches(got, exp, "host_mixed_d512 zipf replay, dedup")
    finally:
        t.close()


def test_host_d512_replay_with_hot_rows(big_records):
    """The pinned-host table with device copies of the 5% most looked-up rows
    (by Zipf rank): the whole replay against the oracle."""
    _, recs = big_records
    cfg = workload.CONFIGS["host_d512"]
    hot = workload.keyed_permutation(np.arange(cfg.rows // 20, dtype=np.int64), cfg.rows, cfg.ids_seed)
    say("building the pinned-host table with 4,884,500 hot rows")
    t = make_table(LUT, recs, cfg.d, cfg.kv, residency=cp.CP_RESIDENCY_HOST_MAPPED, chunk_rows=1 << 24)
    try:
        assert t.set_hot_rows(hot) == hot.size
        check_lookup(t, LUT, recs, cfg.d, cfg.kv, cfg.ids(), "host_d512 zipf replay, hot rows")
    finally:
        t.close()


@pytest.mark.parametrize("kv", [3, 4, 5, 6])
def test_encode_of_the_benchmark_batch(kv):
    """The encoder benchmark's batch (4,096 Gaussian rows of d = 512, the
    benchmark's seed), encoded in the benchmark's launch: every record against
    the oracle's encoding of the same rows."""
    from test_gpu_encode import check_records, gpu_encode, oracle_encode

    d, n = 512, 4096
    e = workload.gaussian_rows(n, d, seed=9100).astype(np.float32)
    say(f"encode of the benchmark batch, kv={kv}")
    t, got = gpu_encode(e, d, kv)
    t.close()
    check_records(got, oracle_encode(e, d, kv), f"benchmark batch kv{kv}")
