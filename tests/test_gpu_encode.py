"""GPU trellis-coded quantisation (cp_table_encode) against the oracle's
heuristic encoder: every record bit-exact (code bytes and the bf16 alpha).

Both sides run the same two-pass tail-biting search in fp64 with one rounding
per operation in the same order and the same tie rules, so the records must
agree bit for bit; alpha is rounded once from fp64 to bf16 on both sides."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import trellis_coded_row_amd as cp
import workload
from parity import assert_bit_exact, assert_scaled_matches, check_lookup, device_lookup, say

pytestmark = pytest.mark.gpu

LUT = workload.lut_fp16()


def gpu_encode(e32: np.ndarray, d: int, kv: int, table_rows: int | None = None, first_row: int = 0, lut=LUT):
    n = e32.shape[0]
    rows = table_rows if table_rows is not None else max(n, 1)
    t = cp.Table(rows, d, kv, lut)
    if first_row or rows != n:
        t.upload(np.zeros((rows, t.record_bytes), dtype=np.uint8))
    dev = torch.from_numpy(np.ascontiguousarray(e32, dtype=np.float32)).cuda()
    t.encode(dev, first_row=first_row)
    torch.cuda.synchronize()
    return t, t.download()


def oracle_encode(e32: np.ndarray, d: int, kv: int, lut=LUT) -> np.ndarray:
    recs, _ = oracle.encode_rows(e32.astype(np.float64), d, kv, lut, mode=oracle.ENC_HEURISTIC)
    return recs


def check_records(got: np.ndarray, exp: np.ndarray, label: str) -> None:
    assert got.shape == exp.shape, (label, got.shape, exp.shape)
    bad = np.nonzero((got != exp).any(axis=1))[0]
    if bad.size:
        r = int(bad[0])
        raise AssertionError(f"{label}: {bad.size} of {got.shape[0]} records differ, first row {r}: "
                             f"got {got[r].tobytes().hex()} want {exp[r].tobytes().hex()}")


@pytest.mark.parametrize("d,kv,n", [
    (64, 4, 600),   # more rows than resident workgroups: the grid-stride loop
    (64, 3, 300),
    (64, 5, 257),
    (64, 6, 129),
    (64, 5, 1100),  # kv 5 and 6 run two 512-thread workgroups per CU: past 512 rows
    (64, 6, 1100),
    (128, 3, 41),
    (128, 4, 97),
    (128, 5, 45),
    (128, 6, 39),
    (256, 3, 23),
    (256, 4, 29),
    (256, 5, 33),
    (256, 6, 31),
    (512, 3, 19),
    (512, 4, 24),
    (512, 5, 17),
    (512, 6, 13),
])
def test_encode_matches_oracle(d, kv, n):
    e = workload.gaussian_rows(n, d, seed=7000 + d + kv).astype(np.float32)
    say(f"encode d={d} kv={kv} n={n}")
    exp = oracle_encode(e, d, kv)
    t, got = gpu_encode(e, d, kv)
    check_records(got, exp, f"encode d{d} kv{kv}")
    # the encoded table decodes like the oracle's records (the oracle decodes
    # its own encoding, equal to the table's as just checked)
    ids = np.arange(n, dtype=np.int64)[::-1].copy()
    check_lookup(t, LUT, exp, d, kv, ids, f"decode of encoded d{d} kv{kv}")
    t.close()
    say(f"encode d={d} kv={kv} n={n}: ok")


@pytest.mark.parametrize("kind", ["paired", "constant", "two-valued"])
@pytest.mark.parametrize("kv", [3, 4, 5, 6])
def test_encode_tie_codebooks(kv, kind):
    """Codebooks under which many paths and many branch metrics are equal
    (the same ones whose tie rule the CPU tests pin by brute force): the
    GPU's add-compare-select must keep the same predecessor and end memory
    as the oracle on every tie."""
    from test_oracle import _tie_lut

    d = 64
    lut = _tie_lut(kind)
    rng = np.random.default_rng(900 + kv)
    rows = [np.full(d, 0.5), np.eye(d)[0] - np.eye(d)[d // 2], np.tile([2.0, 0, 0, 0.75, -1.0, 0, 0.25, 0.5], d // 8),
            np.round(rng.standard_normal(d) * 2) / 2, rng.standard_normal(d)]
    e = np.stack(rows).astype(np.float32)
    say(f"encode tie codebook {kind} kv={kv}")
    exp = oracle_encode(e, d, kv, lut)
    t, got = gpu_encode(e, d, kv, lut=lut)
    check_records(got, exp, f"tie codebook {kind} kv{kv}")
    t.close()


@pytest.mark.parametrize("d", [64, 512])
def test_encode_special_rows(d):
    kv = 4
    rng = np.random.default_rng(77)
    with_inf = rng.standard_normal(d)
    with_inf[3] = np.inf
    with_nan = rng.standard_normal(d)
    with_nan[d - 1] = np.nan
    rows = [
        np.zeros(d),                                   # zero row: zero code, alpha 0
        np.eye(d)[5] * 3.0,                            # one non-zero coordinate
        np.full(d, 0.25),                              # constant row
        rng.standard_normal(d) * 1e-40,                # float subnormals: alpha a bf16 subnormal
        rng.standard_normal(d) * 3e37,                 # large values, alpha near the bf16 top
        np.full(d, 3.3e38),                            # alpha rounds past the largest bf16
        -np.full(d, 1.0),
        with_inf,                                      # norm not finite: the zero record
        with_nan,
        -with_inf,
        rng.standard_normal(d),
    ]
    e = np.stack(rows).astype(np.float32)
    e = np.concatenate([e, e[::-1]])                   # duplicates in another order
    say(f"encode special rows d={d} kv={kv} n={e.shape[0]}")
    exp = oracle_encode(e, d, kv)
    assert (exp[0] == 0).all() and (exp[7:10] == 0).all()
    t, got = gpu_encode(e, d, kv)
    check_records(got, exp, "special rows")
    # and the rows decode like the oracle's, raw and scaled (alpha a bf16
    # subnormal, +inf, 0): bit-exact, NaN where the oracle has NaN
    ids = np.arange(e.shape[0], dtype=np.int64)
    n = e.shape[0]
    exp_raw, _ = oracle.lookup_decode(LUT, exp, n, d, kv, ids, raw=True)
    exp_rows, _ = oracle.lookup_decode(LUT, exp, n, d, kv, ids)
    assert_bit_exact(device_lookup(t, ids, raw=True), exp_raw, "special rows f(c)")
    assert_scaled_matches(device_lookup(t, ids), exp_rows, "special rows scaled")
    t.close()


def test_encode_into_a_range_of_a_larger_table():
    d, kv = 128, 5
    e = workload.gaussian_rows(40, d, seed=4242).astype(np.float32)
    exp = oracle_encode(e, d, kv)
    say("encode rows 100..139 of a 300-row table")
    t, got = gpu_encode(e, d, kv, table_rows=300, first_row=100)
    check_records(got[100:140], exp, "range")
    assert (got[:100] == 0).all() and (got[140:] == 0).all()
    t.close()


def test_encode_rejects_bad_arguments():
    d, kv = 64, 4
    t = cp.Table(16, d, kv, LUT)
    rows = torch.zeros((8, d), dtype=torch.float32, device="cuda")
    need = t.encode_workspace_bytes(8)
    assert need > 0
    small = torch.empty(need - 1, dtype=torch.uint8, device="cuda")
    st = cp.cp_table_encode(t.handle, 0, 8, rows.data_ptr(), small.data_ptr(), need - 1, None)
    assert st == cp.CP_ERR_INVALID_ARGUMENT
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    assert cp.cp_table_encode(t.handle, 10, 8, rows.data_ptr(), ws.data_ptr(), need, None) == \
        cp.CP_ERR_INVALID_ARGUMENT                   # rows 10..17 of 16
    assert cp.cp_table_encode(t.handle, 0, 0, 0, 0, 0, None) == cp.CP_OK
    assert cp.cp_table_encode(t.handle, 0, 8, rows.data_ptr(), ws.data_ptr() + 8, need, None) == \
        cp.CP_ERR_INVALID_ARGUMENT                   # workspace not 256-byte aligned
    assert cp.cp_table_encode(t.handle, 0, 8, rows.data_ptr(), ws.data_ptr(), need, None) == cp.CP_OK
    torch.cuda.synchronize()
    got = t.download(0, 8)
    assert (got == 0).all()                          # zero rows
    t.close()
