"""CPU oracle for Conditional Program (CP) row decoding: Python access.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. The arithmetic lives in plain C
(``cp_oracle.c``, which also states the page citations and the readings it
follows); this module only compiles it with gcc and marshals numpy arrays.
It imports nothing from the HIP library and the library imports nothing
from here.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "cp_oracle.c")
_HDR = os.path.join(_HERE, "cp_oracle.h")
_LIB = os.path.join(_HERE, "libcp_oracle.so")

ENC_EXACT = 0
ENC_HEURISTIC = 1


def build(force: bool = True) -> str:
    """Compiles the oracle with gcc (no fast-math, no FMA contraction)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= max(
        os.path.getmtime(_SRC), os.path.getmtime(_HDR)
    ):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = [
        "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
        "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
        "-o", tmp, _SRC, "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


class EncodeInfo(ctypes.Structure):
    _fields_ = [
        ("cost", ctypes.c_double),
        ("starts", ctypes.c_uint32),
        ("certified", ctypes.c_int32),
        ("gap", ctypes.c_double),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """The compiled oracle; CP_ORACLE_LIBRARY names another build of the same
    source (for instance one compiled with sanitizers)."""
    global _lib
    if _lib is None:
        path = os.environ.get("CP_ORACLE_LIBRARY")
        if not path:
            build(force=False)
            path = _LIB
        L = ctypes.CDLL(path)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        u32p = ctypes.POINTER(ctypes.c_uint32)
        f64p = ctypes.POINTER(ctypes.c_double)
        i64p = ctypes.POINTER(ctypes.c_int64)
        sig = {
            "cpo_code_bits": (ctypes.c_uint64, [ctypes.c_uint32, ctypes.c_uint32]),
            "cpo_record_bytes": (ctypes.c_uint64, [ctypes.c_uint32, ctypes.c_uint32]),
            "cpo_fp16_to_double": (ctypes.c_double, [ctypes.c_uint16]),
            "cpo_bf16_to_double": (ctypes.c_double, [ctypes.c_uint16]),
            "cpo_bf16_from_double": (ctypes.c_uint16, [ctypes.c_double]),
            "cpo_code_bit": (ctypes.c_int, [u8p, ctypes.c_uint64, ctypes.c_int64]),
            "cpo_window": (ctypes.c_uint32, [u8p, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32]),
            "cpo_hash": (None, [ctypes.c_uint32, u32p, u32p]),
            "cpo_decode_code": (ctypes.c_int, [u16p, u8p, ctypes.c_uint32, ctypes.c_uint32, u16p]),
            "cpo_decode_record": (ctypes.c_int, [u16p, u8p, ctypes.c_uint32, ctypes.c_uint32, u16p]),
            "cpo_lookup_decode": (
                ctypes.c_int64,
                [u16p, u8p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, i64p,
                 ctypes.c_uint64, u16p, ctypes.c_int, ctypes.c_int],
            ),
            "cpo_mixed_offsets": (
                ctypes.c_int,
                [ctypes.c_uint64, ctypes.c_uint32, u32p, ctypes.c_uint32, u8p, ctypes.POINTER(ctypes.c_uint64)],
            ),
            "cpo_lookup_decode_mixed": (
                ctypes.c_int64,
                [u16p, u8p, ctypes.c_uint64, ctypes.c_uint32, u32p, ctypes.c_uint32, u8p,
                 ctypes.POINTER(ctypes.c_uint64), i64p, ctypes.c_uint64, u16p, ctypes.c_int, ctypes.c_int],
            ),
            "cpo_tcq_encode": (
                ctypes.c_double,
                [f64p, ctypes.c_uint32, ctypes.c_uint32, u16p, ctypes.c_int, ctypes.c_uint32,
                 u8p, ctypes.POINTER(EncodeInfo)],
            ),
            "cpo_distortion": (ctypes.c_double, [f64p, u16p, u8p, ctypes.c_uint32, ctypes.c_uint32]),
            "cpo_encode_row": (
                ctypes.c_int,
                [f64p, ctypes.c_uint32, ctypes.c_uint32, u16p, ctypes.c_int, ctypes.c_uint32,
                 u8p, ctypes.POINTER(EncodeInfo), f64p],
            ),
            "cpo_encode_rows": (
                ctypes.c_int,
                [f64p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, u16p, ctypes.c_int,
                 ctypes.c_uint32, u8p, ctypes.POINTER(EncodeInfo), ctypes.c_int],
            ),
            "cpo_bruteforce_min": (
                ctypes.c_double,
                [f64p, ctypes.c_uint32, ctypes.c_uint32, u16p, u8p, ctypes.c_int],
            ),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a: np.ndarray, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct))


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# --------------------------------------------------------------------------
# scalar helpers
# --------------------------------------------------------------------------

def code_bits(d: int, kv: int) -> int:
    return int(lib().cpo_code_bits(d, kv))


def record_bytes(d: int, kv: int) -> int:
    return int(lib().cpo_record_bytes(d, kv))


def fp16_to_double(h: int) -> float:
    return lib().cpo_fp16_to_double(h)


def bf16_to_double(b: int) -> float:
    return lib().cpo_bf16_to_double(b)


def bf16_from_double(x: float) -> int:
    return int(lib().cpo_bf16_from_double(x))


def window(code: np.ndarray, d: int, kv: int, t: int) -> int:
    code = _c(code, np.uint8)
    return int(lib().cpo_window(_p(code, ctypes.c_uint8), d, kv, t))


def hash_window(s: int) -> tuple[int, int]:
    idx = ctypes.c_uint32()
    neg = ctypes.c_uint32()
    lib().cpo_hash(s, ctypes.byref(idx), ctypes.byref(neg))
    return int(idx.value), int(neg.value)


# --------------------------------------------------------------------------
# decode
# --------------------------------------------------------------------------

def decode_code(lut: np.ndarray, code: np.ndarray, d: int, kv: int) -> np.ndarray:
    """f(c) as fp16 bit patterns (uint16[d])."""
    lut = _c(lut, np.uint16).reshape(-1)
    code = _c(code, np.uint8)
    out = np.empty(d, dtype=np.uint16)
    st = lib().cpo_decode_code(_p(lut, ctypes.c_uint16), _p(code, ctypes.c_uint8), d, kv,
                               _p(out, ctypes.c_uint16))
    if st:
        raise ValueError("unsupported (d, kv)")
    return out


def decode_record(lut: np.ndarray, record: np.ndarray, d: int, kv: int) -> np.ndarray:
    """alpha * f(c) as bf16 bit patterns (uint16[d])."""
    lut = _c(lut, np.uint16).reshape(-1)
    record = _c(record, np.uint8)
    out = np.empty(d, dtype=np.uint16)
    st = lib().cpo_decode_record(_p(lut, ctypes.c_uint16), _p(record, ctypes.c_uint8), d, kv,
                                 _p(out, ctypes.c_uint16))
    if st:
        raise ValueError("unsupported (d, kv)")
    return out


def lookup_decode(lut, records, rows: int, d: int, kv: int, ids, raw: bool = False,
                  nthreads: int | None = None) -> tuple[np.ndarray, int]:
    """Rows ids[j] of a packed record table, in lookup order.

    Returns (out uint16[n, d], count of ids outside [0, rows)); out holds bf16
    bits, or fp16 bits of f(c) when raw.
    """
    lut = _c(lut, np.uint16).reshape(-1)
    records = np.ascontiguousarray(records, dtype=np.uint8)
    ids = _c(ids, np.int64).reshape(-1)
    n = ids.shape[0]
    out = np.empty((n, d), dtype=np.uint16)
    if nthreads is None:
        nthreads = default_threads()
    bad = lib().cpo_lookup_decode(
        _p(lut, ctypes.c_uint16), _p(records, ctypes.c_uint8), rows, d, kv,
        _p(ids, ctypes.c_int64), n, _p(out, ctypes.c_uint16), int(raw), nthreads)
    if bad < 0:
        raise ValueError("unsupported (d, kv)")
    return out, int(bad)


def mixed_offsets(d: int, kv_of_class, row_class) -> np.ndarray:
    """uint64[rows + 1]: where each row's record starts in a mixed-rate table
    (records packed in row order, each at its class's rate); the last entry
    is the total size."""
    kvs = _c(kv_of_class, np.uint32).reshape(-1)
    cls = _c(row_class, np.uint8).reshape(-1)
    rows = cls.shape[0]
    off = np.empty(rows + 1, dtype=np.uint64)
    st = lib().cpo_mixed_offsets(rows, d, _p(kvs, ctypes.c_uint32), kvs.shape[0], _p(cls, ctypes.c_uint8),
                                 _p(off, ctypes.c_uint64))
    if st:
        raise ValueError("bad class or rate")
    return off


def shard_plan(ids, rows_per_shard: int, shards: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """A lookup batch into a table split by rows over `shards` GPUs, 12.7 GB
    each in the pages' 4-GPU setup ("2비트 코드와 공유 트렐리스로 n-gram 룩업
    테이블을 4~8배 압축한다", onedev.kr, "Assumptions and limits"): the owner of
    global row i is i // rows_per_shard (for 0 <= i < shards * rows_per_shard;
    other ids belong to no shard). Returns (local_ids, positions, counts):
    the owned ids sorted by owner with a stable sort (batch order kept within
    a shard), each as its row within its shard; for each lookup its index in
    that order (-1 when no shard owns the id); ids per shard."""
    ids = np.asarray(ids, dtype=np.int64).reshape(-1)
    valid = (ids >= 0) & (ids < shards * rows_per_shard)
    owner = np.where(valid, ids // rows_per_shard, shards)
    order = np.argsort(owner, kind="stable")[: int(valid.sum())]
    local_ids = ids[order] - owner[order] * rows_per_shard
    positions = np.full(ids.shape[0], -1, dtype=np.int64)
    positions[order] = np.arange(order.shape[0], dtype=np.int64)
    counts = np.bincount(owner[valid], minlength=shards).astype(np.int64)
    return local_ids.astype(np.int64), positions, counts


def gather_records(records, rows: int, ids) -> np.ndarray:
    """The owner's part of a sharded lookup: the packed records of rows
    ids[k] (uint8[n, R]), a zero record for an id outside [0, rows)."""
    recs = np.asarray(records, dtype=np.uint8).reshape(rows, -1)
    ids = np.asarray(ids, dtype=np.int64).reshape(-1)
    ok = (ids >= 0) & (ids < rows)
    out = np.zeros((ids.shape[0], recs.shape[1]), dtype=np.uint8)
    out[ok] = recs[ids[ok]]
    return out


def lookup_decode_mixed(lut, records, d: int, kv_of_class, row_class, ids, raw: bool = False,
                        offsets=None, nthreads: int | None = None) -> tuple[np.ndarray, int]:
    """Rows ids[j] of a mixed-rate table, in lookup order; as lookup_decode.
    offsets: from mixed_offsets (computed here when None)."""
    lut = _c(lut, np.uint16).reshape(-1)
    records = np.ascontiguousarray(records, dtype=np.uint8).reshape(-1)
    kvs = _c(kv_of_class, np.uint32).reshape(-1)
    cls = _c(row_class, np.uint8).reshape(-1)
    if offsets is None:
        offsets = mixed_offsets(d, kvs, cls)
    offsets = _c(offsets, np.uint64)
    ids = _c(ids, np.int64).reshape(-1)
    n = ids.shape[0]
    out = np.empty((n, d), dtype=np.uint16)
    if nthreads is None:
        nthreads = default_threads()
    bad = lib().cpo_lookup_decode_mixed(
        _p(lut, ctypes.c_uint16), _p(records, ctypes.c_uint8), cls.shape[0], d, _p(kvs, ctypes.c_uint32),
        kvs.shape[0], _p(cls, ctypes.c_uint8), _p(offsets, ctypes.c_uint64), _p(ids, ctypes.c_int64), n,
        _p(out, ctypes.c_uint16), int(raw), nthreads)
    if bad < 0:
        raise ValueError("unsupported (d, kv)")
    return out, int(bad)


# --------------------------------------------------------------------------
# encode
# --------------------------------------------------------------------------

@dataclass
class Encoded:
    code: np.ndarray
    cost: float
    starts: int
    certified: bool
    gap: float


def tcq_encode(z, d: int, kv: int, lut, mode: int = ENC_EXACT, max_starts: int = 0) -> Encoded:
    z = _c(z, np.float64)
    lut = _c(lut, np.uint16).reshape(-1)
    code = np.zeros((code_bits(d, kv) + 7) // 8, dtype=np.uint8)
    info = EncodeInfo()
    cost = lib().cpo_tcq_encode(_p(z, ctypes.c_double), d, kv, _p(lut, ctypes.c_uint16), mode,
                                max_starts, _p(code, ctypes.c_uint8), ctypes.byref(info))
    return Encoded(code, cost, int(info.starts), bool(info.certified), float(info.gap))


def distortion(z, lut, code, d: int, kv: int) -> float:
    z = _c(z, np.float64)
    lut = _c(lut, np.uint16).reshape(-1)
    code = _c(code, np.uint8)
    return lib().cpo_distortion(_p(z, ctypes.c_double), _p(lut, ctypes.c_uint16),
                                _p(code, ctypes.c_uint8), d, kv)


def encode_row(e, d: int, kv: int, lut, mode: int = ENC_EXACT, max_starts: int = 0):
    """Returns (record uint8[R], EncodeInfo, unrounded fp64 alpha)."""
    e = _c(e, np.float64)
    lut = _c(lut, np.uint16).reshape(-1)
    rec = np.zeros(record_bytes(d, kv), dtype=np.uint8)
    info = EncodeInfo()
    alpha = ctypes.c_double()
    st = lib().cpo_encode_row(_p(e, ctypes.c_double), d, kv, _p(lut, ctypes.c_uint16), mode,
                              max_starts, _p(rec, ctypes.c_uint8), ctypes.byref(info),
                              ctypes.byref(alpha))
    if st:
        raise ValueError("encode failed")
    return rec, info, float(alpha.value)


def encode_rows(e, d: int, kv: int, lut, mode: int = ENC_EXACT, max_starts: int = 0,
                nthreads: int | None = None):
    """Encodes rows e[nrows, d]; returns (records uint8[nrows, R], info array)."""
    e = _c(e, np.float64)
    nrows = e.shape[0]
    lut = _c(lut, np.uint16).reshape(-1)
    recs = np.zeros((nrows, record_bytes(d, kv)), dtype=np.uint8)
    infos = (EncodeInfo * max(nrows, 1))()
    if nthreads is None:
        nthreads = default_threads()
    st = lib().cpo_encode_rows(_p(e, ctypes.c_double), nrows, d, kv, _p(lut, ctypes.c_uint16),
                               mode, max_starts, _p(recs, ctypes.c_uint8), infos, nthreads)
    if st:
        raise ValueError("encode failed")
    return recs, infos


def bruteforce_min(z, d: int, kv: int, lut, nthreads: int | None = None):
    """Exhaustive minimum of ||z - f(c)||^2 over all codes; returns (cost, code)."""
    z = _c(z, np.float64)
    lut = _c(lut, np.uint16).reshape(-1)
    code = np.zeros(max((code_bits(d, kv) + 7) // 8, 1), dtype=np.uint8)
    if nthreads is None:
        nthreads = default_threads()
    v = lib().cpo_bruteforce_min(_p(z, ctypes.c_double), d, kv, _p(lut, ctypes.c_uint16),
                                 _p(code, ctypes.c_uint8), nthreads)
    return float(v), code
