"""GPU parity of the HIP gather-decode against the CPU oracle: every compiled
(d, kv) instance, ragged batch sizes, alignment, order, duplicates, bad ids,
record independence, and the 4,096 x d64 table of oracle-encoded rows."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import trellis_coded_row_amd as cp
import workload
from parity import assert_scaled_matches, check_lookup, device_lookup, make_table, say, shape_change_sizes

pytestmark = pytest.mark.gpu

LUT = workload.lut_fp16(0)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    torch.cuda.init()


@pytest.fixture(scope="module")
def tiny_table():
    cfg = workload.CONFIGS["tiny_d64"]
    say("encoding the 4,096 x d64 table with the oracle")
    recs = workload.build_records(
        cfg, encode_fn=lambda e: oracle.encode_rows(e, cfg.d, cfg.kv, LUT, oracle.ENC_EXACT,
                                                    max_starts=8)[0])
    t = make_table(LUT, recs, cfg.d, cfg.kv)
    yield cfg, recs, t
    t.close()


def test_tiny_d64_encoded_table(tiny_table):
    cfg, recs, t = tiny_table
    check_lookup(t, LUT, recs, cfg.d, cfg.kv, cfg.ids(), "tiny_d64 uniform ids")
    check_lookup(t, LUT, recs, cfg.d, cfg.kv, np.arange(cfg.rows, dtype=np.int64), "tiny_d64 every row")


@pytest.mark.parametrize("d", [64, 128, 256, 512])
@pytest.mark.parametrize("kv", [3, 4, 5, 6])
def test_every_instance_ragged_batches(d, kv):
    rows = 3001
    recs = workload.random_records(rows, d, kv, seed=500 + d + kv)
    t = make_table(LUT, recs, d, kv)
    rng = np.random.default_rng(d * 10 + kv)
    try:
        for n in (1, 2, 7, 64, 1000, 4099):
            ids = rng.integers(0, rows, n, dtype=np.int64)
            check_lookup(t, LUT, recs, d, kv, ids, f"d{d} kv{kv} n{n}")
    finally:
        t.close()


@pytest.mark.parametrize("d,kv", [(64, 4), (128, 5), (256, 3), (512, 4), (512, 6)])
def test_batch_sizes_around_launch_shape_changes(d, kv):
    # the launch picks 1-, 4- or 16-lookup wave chunks by batch size: every
    # shape, at its edges and with ragged tails, against the oracle (with a
    # few ids outside the table in each batch); the dedup path at one size
    rows = 5003
    recs = workload.random_records(rows, d, kv, seed=800 + d + kv)
    t = make_table(LUT, recs, d, kv)
    rng = np.random.default_rng(d + kv)
    try:
        for n in shape_change_sizes():
            ids = rng.integers(0, rows, n, dtype=np.int64)
            ids[n // 3] = rows
            ids[-1] = -5
            check_lookup(t, LUT, recs, d, kv, ids, f"d{d} kv{kv} n{n}", expect_bad=2,
                         dedup=(n == shape_change_sizes()[2]))
    finally:
        t.close()


@pytest.mark.parametrize("d,kv", [(64, 4), (256, 4), (512, 4), (512, 3), (512, 6)])
def test_order_duplicates_alignment_and_table_ends(d, kv):
    rows = 1001  # odd: the last record starts at an offset = 2 (mod 4)
    recs = workload.random_records(rows, d, kv, seed=600 + d + kv)
    t = make_table(LUT, recs, d, kv)
    try:
        cases = {
            "reversed": np.arange(rows - 1, -1, -1, dtype=np.int64),
            "all same": np.full(777, 123, dtype=np.int64),
            "ends": np.array([0, rows - 1, 1, rows - 2, rows - 1, 0], dtype=np.int64),
            "odd ids": np.arange(1, rows, 2, dtype=np.int64),
            "even ids": np.arange(0, rows, 2, dtype=np.int64),
        }
        for name, ids in cases.items():
            check_lookup(t, LUT, recs, d, kv, ids, f"d{d} kv{kv} {name}")
    finally:
        t.close()


@pytest.mark.parametrize("d,kv", [(64, 4), (512, 4), (512, 5)])
def test_out_of_range_ids_give_zero_rows_and_raise_the_flag(d, kv):
    rows = 200
    recs = workload.random_records(rows, d, kv, seed=700 + d)
    t = make_table(LUT, recs, d, kv)
    try:
        ids = np.array([3, -1, 199, 200, 2**62, 5, -(2**63), 7], dtype=np.int64)
        check_lookup(t, LUT, recs, d, kv, ids, f"d{d} kv{kv} bad ids", expect_bad=4)
        # the flag was cleared by the check: a clean batch reports clean
        out = device_lookup(t, np.array([1, 2], dtype=np.int64))
        assert out.shape == (2, d)
        assert t.check()
    finally:
        t.close()


def test_empty_batch_launches_nothing():
    d, kv, rows = 512, 4, 10
    recs = workload.random_records(rows, d, kv, seed=800)
    t = make_table(LUT, recs, d, kv)
    try:
        ids = torch.empty(0, dtype=torch.int64, device="cuda")
        out = t.lookup_decode(ids)
        assert tuple(out.shape) == (0, d)
        assert t.check()
    finally:
        t.close()


def test_records_are_independent():
    # poisoning the neighbours of a record (and everything else) leaves its row unchanged
    d, kv, rows = 512, 4, 64
    recs = workload.random_records(rows, d, kv, seed=900)
    ids = np.array([31, 32, 33], dtype=np.int64)
    t = make_table(LUT, recs, d, kv)
    try:
        before = device_lookup(t, ids)
        poisoned = recs.copy()
        keep = set(ids.tolist())
        for r in range(rows):
            if r not in keep:
                poisoned[r] ^= 0xFF
        t.upload(poisoned)
        after = device_lookup(t, ids)
        assert (before == after).all()
        check_lookup(t, LUT, poisoned, d, kv, np.arange(rows, dtype=np.int64), "poisoned table")
    finally:
        t.close()


def test_caller_stream_is_used():
    d, kv, rows = 256, 4, 500
    recs = workload.random_records(rows, d, kv, seed=901)
    t = make_table(LUT, recs, d, kv)
    try:
        ids_np = np.random.default_rng(0).integers(0, rows, 5000, dtype=np.int64)
        exp, _ = oracle.lookup_decode(LUT, recs, rows, d, kv, ids_np)
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            ids = torch.from_numpy(ids_np).cuda()
            out = t.lookup_decode(ids, stream=s)
        s.synchronize()
        got = out.view(torch.int16).cpu().numpy().view(np.uint16)
        assert_scaled_matches(got, exp, "side stream")
        # a side stream that is not the current one: the binding allocates the
        # output and the dedup workspace on the current stream and records
        # their use on the side stream; allocations made meanwhile on the
        # current stream must not take their memory
        ids = torch.from_numpy(ids_np).cuda()
        torch.cuda.synchronize()
        outs = []
        for _ in range(3):
            outs.append(t.lookup_decode_dedup(ids, stream=s))
            junk = [torch.full((1 << 20,), 7, dtype=torch.int32, device="cuda") for _ in range(4)]
            del junk
        s.synchronize()
        for o in outs:
            got = o.view(torch.int16).cpu().numpy().view(np.uint16)
            assert_scaled_matches(got, exp, "dedup on a side stream")
    finally:
        t.close()


def test_record_offsets_beyond_2_and_4_gib():
    # records whose byte offset id * R passes 2^31 and 2^32: the kernel's
    # offsets and addresses must stay 64-bit unsigned all the way
    d, kv = 512, 4
    R = cp.cp_record_bytes(d, kv)
    rows = (1 << 32) // R + 4096
    say(f"generating a {rows:,}-row table ({rows * R / 2**30:.2f} GiB)")
    recs = workload.random_records(rows, d, kv, seed=4242)
    t = make_table(LUT, recs, d, kv)
    try:
        b31, b32 = (1 << 31) // R, (1 << 32) // R
        edge = [b31 - 1, b31, b31 + 1, b32 - 1, b32, b32 + 1, rows - 1, 0]
        rng = np.random.default_rng(11)
        ids = np.concatenate([np.array(edge * 3, dtype=np.int64),
                              rng.integers(b31 - 2000, b31 + 2000, 500, dtype=np.int64),
                              rng.integers(b32 - 2000, rows, 500, dtype=np.int64)])
        check_lookup(t, LUT, recs, d, kv, ids, "offsets across 2 and 4 GiB")
    finally:
        t.close()
        del recs
        torch.cuda.empty_cache()


@pytest.mark.parametrize("d,kv", [(64, 4), (256, 4), (512, 4), (512, 3), (512, 6)])
def test_dedup_path_matches(d, kv):
    rows = 2000
    recs = workload.random_records(rows, d, kv, seed=1000 + d + kv)
    t = make_table(LUT, recs, d, kv)
    rng = np.random.default_rng(5)
    try:
        cases = {
            "zipf": workload.zipf_ids(rows, 5000, seed=7),
            "all same": np.full(300, 17, dtype=np.int64),
            "all distinct": rng.permutation(rows).astype(np.int64),
            "one": np.array([rows - 1], dtype=np.int64),
        }
        for name, ids in cases.items():
            check_lookup(t, LUT, recs, d, kv, ids, f"d{d} kv{kv} dedup {name}", dedup=True)
        bad = np.array([3, -1, 3, rows, 3, 2**62, 5], dtype=np.int64)
        check_lookup(t, LUT, recs, d, kv, bad, f"d{d} kv{kv} dedup bad ids", expect_bad=3, dedup=True)
    finally:
        t.close()


def test_dedup_rejects_a_small_workspace():
    d, kv, rows = 512, 4, 100
    recs = workload.random_records(rows, d, kv, seed=1100)
    t = make_table(LUT, recs, d, kv)
    try:
        ids = torch.arange(50, dtype=torch.int64, device="cuda")
        need = t.dedup_workspace_bytes(50)
        small = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
        with pytest.raises(cp.CPError):
            t.lookup_decode_dedup(ids, workspace=small)
        ok = torch.empty(need, dtype=torch.uint8, device="cuda")
        out = t.lookup_decode_dedup(ids, workspace=ok)
        torch.cuda.synchronize()
        exp, _ = oracle.lookup_decode(LUT, recs, rows, d, kv, np.arange(50))
        assert (out.view(torch.int16).cpu().numpy().view(np.uint16) == exp).all()
    finally:
        t.close()


@pytest.mark.parametrize("d,kv", [(512, 4), (512, 3), (512, 6), (256, 4), (64, 5)])
def test_touch_ahead_tables(d, kv):
    # CP_FLAG_TOUCH_AHEAD: the first round of workgroups also reads the later
    # rounds' ids and touches their records; the rows must not change. Batch
    # sizes with two and more rounds at 4- and 16-lookup chunks, ragged,
    # with ids outside the table (whose touches read record 0)
    rows = 200_003
    recs = workload.random_records(rows, d, kv, seed=1700 + d + kv)
    t = cp.Table(rows, d, kv, LUT, flags=cp.CP_FLAG_TOUCH_AHEAD)
    try:
        t.upload(recs)
        rng = np.random.default_rng(d + 3 * kv)
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        for n in (20 * cus * 4 + 17, 3 * cus * 16 * 16 + 5, 393_216):
            ids = workload.zipf_ids(rows, n, seed=n + d)
            ids[rng.integers(0, n, 5)] = rows + 7
            ids[-1] = -1
            check_lookup(t, LUT, recs, d, kv, ids, f"touch-ahead d{d} kv{kv} n{n}", expect_bad=int((ids >= rows).sum() + 1))
    finally:
        t.close()
