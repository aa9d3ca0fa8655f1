"""GPU parity of the scale step (e_hat = alpha * f(c), rounded once to bf16)
at its edges, against the oracle element by element.

The pages fix the rule and that the scale is a bf16 ("2비트 코드와 공유
트렐리스로 n-gram 룩업 테이블을 4~8배 압축한다", onedev.kr, sections "How
it works" and "How it is used"); these inputs reach the corners of that
arithmetic that Gaussian tables never do:
  - a codebook holding +-0, fp16 subnormals (0x0001, 0x03FF, ...), the
    smallest normal and the largest finite values, besides ordinary ones;
  - scales 0x0000, 0x8000, bf16 subnormals (0x0001, 0x007F), the smallest
    normal, values just below and at 2^-102 (where the kernels switch to the
    exact tiny-scale arithmetic), negative scales, the largest bf16 (products
    overflow to inf), +-inf and NaN, and random scales over every exponent;
so products fall below 2^-126, overflow, or are 0 * inf.

Bars: f(c) bit-exact; scaled rows bit-exact wherever the oracle's value is a
number, and NaN wherever it is NaN (the bit pattern of a NaN is not fixed by
the arithmetic). Covered for the d = 512 kernel (scale in a scalar register),
the d < 512 kernels (scale per lane), every launch shape (1-, 4- and
16-lookup wave chunks), the mixed-rate kernel, the dedup path and a
pinned-host table with rows copied to HBM."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import trellis_coded_row_amd as cp
import workload
from parity import assert_bit_exact, assert_scaled_matches, device_lookup, make_table, say

pytestmark = pytest.mark.gpu

SPECIAL_FP16 = [0x0000, 0x8000, 0x0001, 0x8001, 0x0002, 0x03FF, 0x83FF, 0x0200, 0x8155, 0x0400, 0x8400,
                0x7BFF, 0xFBFF, 0x3C00, 0xBC00, 0x0001, 0x0401, 0x1000]
SPECIAL_BF16 = [0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x8080, 0x0081, 0x0BFF, 0x0C00, 0x0C7F,
                0x8C7F, 0x0C80, 0x8C80, 0x0D00, 0x3F80, 0xBF80, 0x3FC1, 0x7F7F, 0xFF7F, 0x7F00, 0x7F80,
                0xFF80, 0x7FC0, 0xFFC1, 0x4780, 0x2000, 0x1234]

# Pairs (scale, codebook value) whose exact product lies just below a
# rounding midpoint of the bf16 subnormal grid, within fp32's own spacing
# there: an fp32 product would round onto the midpoint and the bf16 rounding
# would then go the wrong way (by 1 ulp). Found by enumerating every scale
# below 2^-102 against every finite fp16 value (56 pairs in all, made of
# these values).
DOUBLE_ROUNDING_BF16 = [0x00B9, 0x00CF, 0x0139, 0x014F, 0x01B9, 0x01CF, 0x0239, 0x024F, 0x02B9, 0x02CF, 0x0339, 0x034F, 0x03CF, 0x044F,
                        0x80B9, 0x80CF, 0x8139, 0x814F, 0x81B9, 0x81CF, 0x8239, 0x824F, 0x82B9, 0x82CF, 0x8339, 0x834F, 0x83CF, 0x844F]
DOUBLE_ROUNDING_FP16 = [0x0589, 0x062F, 0x0989, 0x0A2F, 0x0D89, 0x0E2F, 0x1189, 0x122F, 0x1589, 0x162F, 0x1989, 0x1A2F, 0x1E2F, 0x222F,
                        0x8589, 0x862F, 0x8989, 0x8A2F, 0x8D89, 0x8E2F, 0x9189, 0x922F, 0x9589, 0x962F, 0x9989, 0x9A2F, 0x9E2F, 0xA22F]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    torch.cuda.init()


def edge_codebook(seed: int = 11) -> np.ndarray:
    """512 x 2 fp16 patterns: a third special values, a third fp16
    subnormals, a third ordinary N(0,1) values (all finite)."""
    rng = np.random.default_rng(seed)
    normal = rng.standard_normal(1024).astype(np.float16).view(np.uint16)
    sub = rng.integers(0, 0x0400, size=1024, dtype=np.uint16) | (rng.integers(0, 2, 1024, dtype=np.uint16) << 15)
    spec = np.array(SPECIAL_FP16, dtype=np.uint16)[rng.integers(0, len(SPECIAL_FP16), 1024)]
    pick = rng.integers(0, 3, size=1024)
    lut = np.where(pick == 0, spec, np.where(pick == 1, sub, normal)).astype(np.uint16)
    return lut.reshape(512, 2)


def edge_scales(n: int, seed: int) -> np.ndarray:
    """n bf16 scales: every special value several times, the rest with a
    random sign, mantissa and exponent field (0..254, so subnormals and
    values near the top included)."""
    rng = np.random.default_rng(seed)
    exp = rng.integers(0, 255, size=n, dtype=np.uint16)
    a = (rng.integers(0, 2, n, dtype=np.uint16) << 15) | (exp << 7) | rng.integers(0, 128, n, dtype=np.uint16)
    spec = np.array(SPECIAL_BF16, dtype=np.uint16)
    k = min(n, 4 * spec.size)
    a[:k] = np.tile(spec, 4)[:k]
    return rng.permutation(a)


def with_scales(records: np.ndarray, d: int, kv: int, scales: np.ndarray) -> np.ndarray:
    nb = kv * d // 16
    out = records.copy()
    out[:, nb] = (scales & 0xFF).astype(np.uint8)
    out[:, nb + 1] = (scales >> 8).astype(np.uint8)
    return out


def regimes(exp: np.ndarray) -> dict:
    """How many expected values fall in each regime (what the case reached)."""
    mag = exp & 0x7FFF
    return {"zero": int((mag == 0).sum()), "bf16_subnormal": int(((mag > 0) & (mag < 0x0080)).sum()),
            "inf": int((mag == 0x7F80).sum()), "nan": int((mag > 0x7F80).sum())}


def check(table, lut, records, d, kv, ids, label):
    rows = records.shape[0]
    exp_raw, _ = oracle.lookup_decode(lut, records, rows, d, kv, ids, raw=True)
    exp, _ = oracle.lookup_decode(lut, records, rows, d, kv, ids, raw=False)
    got_raw = device_lookup(table, ids, raw=True)
    assert_bit_exact(got_raw, exp_raw, label + " f(c)")
    got = device_lookup(table, ids)
    assert_scaled_matches(got, exp, label + " rows")
    assert table.check(), label
    return got, exp


@pytest.mark.parametrize("d,kv", [(512, 4), (512, 3), (512, 6), (256, 4), (128, 5), (64, 4), (64, 3)])
def test_scale_edges_every_launch_shape(d, kv):
    lut = edge_codebook()
    rows = 4096
    recs = with_scales(workload.random_records(rows, d, kv, seed=900 + d + kv), d, kv, edge_scales(rows, d + kv))
    t = make_table(lut, recs, d, kv)
    rng = np.random.default_rng(d * 7 + kv)
    seen = {"zero": 0, "bf16_subnormal": 0, "inf": 0, "nan": 0}
    try:
        # 1-, 4- and 16-lookup wave chunks (chosen by batch size), ragged tails
        for n in (rows, 9001, 40000 + 3):
            ids = np.arange(rows, dtype=np.int64) if n == rows else rng.integers(0, rows, n, dtype=np.int64)
            say(f"scale edges d={d} kv={kv} n={n}")
            _, exp = check(t, lut, recs, d, kv, ids, f"scale edges d{d} kv{kv} n{n}")
            for k, v in regimes(exp).items():
                seen[k] += v
    finally:
        t.close()
    # the inputs reached every regime
    assert all(v > 0 for v in seen.values()), seen
    say(f"scale edges d={d} kv={kv}: ok {seen}")


def test_scale_edges_with_bad_ids_and_tiny_record_zero():
    # an id outside the table decodes record 0 before its row is zeroed; with
    # record 0's scale tiny, the exact tiny-scale pass must not bring it back
    d, kv, rows = 512, 4, 300
    lut = edge_codebook(12)
    scales = edge_scales(rows, 5)
    scales[0] = 0x0001
    recs = with_scales(workload.random_records(rows, d, kv, seed=950), d, kv, scales)
    t = make_table(lut, recs, d, kv)
    try:
        ids = np.arange(rows, dtype=np.int64)
        ids[7], ids[100], ids[-1] = rows, -3, 2**40
        exp, bad = oracle.lookup_decode(lut, recs, rows, d, kv, ids)
        assert bad == 3
        got = device_lookup(t, ids)
        assert_scaled_matches(got, exp, "bad ids with a tiny record 0")
        assert (got[[7, 100, rows - 1]] == 0).all()
        assert not t.check()
    finally:
        t.close()


@pytest.mark.parametrize("d", [512, 128])
def test_scale_edges_mixed_rate(d):
    lut = edge_codebook(13)
    rows = 3001
    kvs = (6, 5, 4, 3)
    rng = np.random.default_rng(d)
    cls = rng.integers(0, 4, size=rows).astype(np.uint8)
    off = workload.mixed_layout(d, kvs, cls)
    packed = workload.random_mixed_records(d, kvs, cls, seed=d + 77, offsets=off)
    nb = np.array([k * d // 16 for k in kvs], dtype=np.int64)
    pos = off[:-1].astype(np.int64) + nb[cls]
    scales = edge_scales(rows, d + 1)
    packed[pos] = (scales & 0xFF).astype(np.uint8)
    packed[pos + 1] = (scales >> 8).astype(np.uint8)
    t = cp.MixedTable(d, kvs, cls, lut)
    t.upload_bytes(packed, 0, rows)
    try:
        for n in (rows, 50000):
            ids = np.arange(rows, dtype=np.int64) if n == rows else rng.integers(0, rows, n, dtype=np.int64)
            say(f"mixed scale edges d={d} n={n}")
            exp_raw, _ = oracle.lookup_decode_mixed(lut, packed, d, kvs, cls, ids, raw=True)
            exp, _ = oracle.lookup_decode_mixed(lut, packed, d, kvs, cls, ids)
            assert_bit_exact(device_lookup(t, ids, raw=True), exp_raw, f"mixed d{d} n{n} f(c)")
            assert_scaled_matches(device_lookup(t, ids), exp, f"mixed d{d} n{n} rows")
    finally:
        t.close()


def test_scale_edges_dedup_and_hot_rows():
    d, kv, rows = 512, 4, 5000
    lut = edge_codebook(14)
    recs = with_scales(workload.random_records(rows, d, kv, seed=960), d, kv, edge_scales(rows, 6))
    ids = workload.zipf_ids(rows, 30000, seed=61)
    exp, _ = oracle.lookup_decode(lut, recs, rows, d, kv, ids)
    t = make_table(lut, recs, d, kv)
    try:
        say("scale edges: dedup path")
        direct = device_lookup(t, ids)
        assert_scaled_matches(direct, exp, "direct")
        assert_bit_exact(device_lookup(t, ids, dedup=True), direct, "dedup path")
    finally:
        t.close()
    h = make_table(lut, recs, d, kv, residency=cp.CP_RESIDENCY_HOST_MAPPED)
    try:
        say("scale edges: pinned-host table with half the rows in HBM")
        h.set_hot_rows(np.arange(0, rows, 2, dtype=np.int64))
        assert_scaled_matches(device_lookup(h, ids), exp, "host table with hot rows")
    finally:
        h.close()


@pytest.mark.parametrize("d,kv", [(512, 4), (64, 4), (256, 5)])
def test_products_where_an_fp32_product_would_round_twice(d, kv):
    # a codebook made of the fp16 values and scales made of the bf16 values
    # of those pairs: every row meets them; the rows must still be the single
    # rounding of the exact product
    lut = np.array(DOUBLE_ROUNDING_FP16 * 37, dtype=np.uint16)[:1024].reshape(512, 2)
    rows = 28 * 8
    scales = np.array(DOUBLE_ROUNDING_BF16 * 8, dtype=np.uint16)
    recs = with_scales(workload.random_records(rows, d, kv, seed=970 + d), d, kv, scales)
    t = make_table(lut, recs, d, kv)
    try:
        ids = np.arange(rows, dtype=np.int64)
        say(f"double-rounding pairs d={d} kv={kv}")
        check(t, lut, recs, d, kv, ids, f"double-rounding pairs d{d} kv{kv}")
    finally:
        t.close()
