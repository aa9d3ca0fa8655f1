"""Helpers shared by the GPU parity tests: run the HIP path through the C-ABI
binding and compare with the CPU oracle element by element.

Bars: f(c) (fp16) bit-exact; scaled rows (bf16) bit-exact as well, NaN
wherever the oracle's value is NaN. The required tolerance is 1 bf16 ulp
(relative error <= 2^-8); the arithmetic is exact on both sides (the oracle
rounds the exact fp64 product once; the kernels form the exact product in
fp32, and for scales below 2^-102, where an fp32 product could itself round,
take an exact path scaled by 2^64), so the tests hold them to equality.
assert_bf16_within_ulp keeps the looser bar for reference."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import trellis_coded_row_amd as cp

BF16_REL = 2.0 ** -8


def shape_change_sizes() -> list[int]:
    """Batch sizes just below, at and above the two sizes where the lookup
    launch moves to longer wave chunks (1 -> 4 rows at 32 lookups per compute
    unit, 4 -> 16 at 128 per compute unit), with ragged tails."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    b4, b16 = 32 * cus, 128 * cus
    return [b4 - 1, b4, b4 + 37, b16 - 1, b16, b16 + 1001]


def say(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def ordered_bf16(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_bf16_within_ulp(got: np.ndarray, exp: np.ndarray, label: str) -> int:
    """Returns the number of elements that differ at all (expected 0)."""
    assert got.shape == exp.shape, (label, got.shape, exp.shape)
    ulp = np.abs(ordered_bf16(got) - ordered_bf16(exp))
    bad = ulp > 1
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{label}: {int(bad.sum())} values beyond 1 ulp, first at {tuple(i)}: "
                             f"got {got[tuple(i)]:#06x} want {exp[tuple(i)]:#06x}")
    gv, ev = bf16_values(got), bf16_values(exp)
    nz = ev != 0
    rel = np.abs(gv[nz] - ev[nz]) / np.abs(ev[nz])
    assert rel.size == 0 or rel.max() <= BF16_REL, (label, float(rel.max()))
    assert (gv[~nz] == 0).all(), label
    return int((got != exp).sum())


def assert_scaled_matches(got: np.ndarray, exp: np.ndarray, label: str) -> None:
    """Bit-exact, except that a NaN of the oracle must be some NaN here."""
    assert got.shape == exp.shape, (label, got.shape, exp.shape)
    is_nan = lambda b: ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)
    en, gn = is_nan(exp), is_nan(got)
    assert (gn == en).all(), f"{label}: NaN where the oracle has a number, or the reverse ({int((gn != en).sum())})"
    neq = (got != exp) & ~en
    if neq.any():
        i = tuple(np.argwhere(neq)[0])
        raise AssertionError(f"{label}: {int(neq.sum())} of {got.size} differ, first at {i}: "
                             f"got {got[i]:#06x} want {exp[i]:#06x}")


def assert_bit_exact(got: np.ndarray, exp: np.ndarray, label: str) -> None:
    assert got.shape == exp.shape, (label, got.shape, exp.shape)
    neq = got != exp
    if neq.any():
        i = np.argwhere(neq)[0]
        raise AssertionError(f"{label}: {int(neq.sum())} of {got.size} differ, first at {tuple(i)}: "
                             f"got {got[tuple(i)]:#06x} want {exp[tuple(i)]:#06x}")


def device_lookup(table: cp.Table, ids: np.ndarray, raw: bool = False, dedup: bool = False) -> np.ndarray:
    dev_ids = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int64)).cuda()
    if dedup:
        out = table.lookup_decode_dedup(dev_ids)
    else:
        out = table.lookup_decode_raw(dev_ids) if raw else table.lookup_decode(dev_ids)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16)


def make_table(lut: np.ndarray, records: np.ndarray, d: int, kv: int,
               residency: int = cp.CP_RESIDENCY_DEVICE, flags: int = 0,
               chunk_rows: int = 1 << 22) -> cp.Table:
    t = cp.Table(records.shape[0], d, kv, lut, residency=residency, flags=flags)
    for r0 in range(0, records.shape[0], chunk_rows):
        t.upload(records[r0:r0 + chunk_rows], first_row=r0)
    return t


def check_lookup(table: cp.Table, lut: np.ndarray, records: np.ndarray, d: int, kv: int,
                 ids: np.ndarray, label: str, expect_bad: int = 0, dedup: bool = False) -> None:
    """Raw and scaled outputs of the HIP path against the oracle, every element."""
    say(f"{label}: n={ids.shape[0]} d={d} kv={kv} rows={records.shape[0]}")
    rows = records.shape[0]
    exp_raw, bad = oracle.lookup_decode(lut, records, rows, d, kv, ids, raw=True)
    exp, bad2 = oracle.lookup_decode(lut, records, rows, d, kv, ids, raw=False)
    assert bad == bad2 == expect_bad, (label, bad)
    got_raw = device_lookup(table, ids, raw=True)
    assert table.check() == (expect_bad == 0), label
    assert_bit_exact(got_raw, exp_raw, label + " f(c)")
    got = device_lookup(table, ids, raw=False)
    assert table.check() == (expect_bad == 0), label
    assert_scaled_matches(got, exp, label + " rows")
    ndiff = int((got != exp).sum())
    if dedup:
        got_d = device_lookup(table, ids, dedup=True)
        assert table.check() == (expect_bad == 0), label
        assert_bit_exact(got_d, got, label + " dedup path")
    say(f"{label}: ok (f(c) bit-exact; scaled rows differing from the oracle: {ndiff}"
        f"{'; dedup path identical' if dedup else ''})")
