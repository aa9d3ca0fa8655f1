"""Python binding of libcp_probe.so (include/cp_probe.h): measurement probes
that give the floors the lookup is compared against (a streaming read, the
lookup's output stream alone, its record fetch alone). Argument marshalling
only; not used by the lookup path."""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (torch's HIP runtime first, as for libcp.so)

from . import build as _build

_lib: ctypes.CDLL | None = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_build.PROBE_LIB):
            _build.build()
        L = ctypes.CDLL(_build.PROBE_LIB)
        vp, u64, u32 = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32
        for name, args in {
            "cpp_read_stream": [vp, u64, vp, vp],
            "cpp_store_rows": [vp, u64, u32, u32, vp],
            "cpp_gather_records": [vp, u64, vp, u64, vp, vp],
        }.items():
            fn = getattr(L, name)
            fn.restype = ctypes.c_int
            fn.argtypes = args
        _lib = L
    return _lib


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{what} failed: hipError {rc}")


def cpp_read_stream(src_ptr: int, nbytes: int, sink_ptr: int, stream: int | None) -> None:
    _check(load().cpp_read_stream(src_ptr, nbytes, sink_ptr, stream), "cpp_read_stream")


def cpp_store_rows(out_ptr: int, n: int, d: int, chunk: int, stream: int | None) -> None:
    _check(load().cpp_store_rows(out_ptr, n, d, chunk, stream), "cpp_store_rows")


def cpp_gather_records(records_ptr: int, record_bytes: int, ids_ptr: int, n: int, sink_ptr: int,
                       stream: int | None) -> None:
    _check(load().cpp_gather_records(records_ptr, record_bytes, ids_ptr, n, sink_ptr, stream), "cpp_gather_records")
