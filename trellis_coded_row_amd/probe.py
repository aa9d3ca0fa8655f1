"""Python binding of libcp_probe.so (include/cp_probe.h): measurement probes
that give the floors the lookup is compared against (a streaming read, the
lookup's output stream alone, its record fetch alone) and a two-lane LDS
access for the LDS's lane grouping. Argument marshalling only; not used by
the lookup path.

    python -m trellis_coded_row_amd.probe lds-lanes

launches the two-lane LDS probe for every access kind and lane pair (a in
0, 5, 37; b in 0..63), one dispatch each, in the order it prints; run it
under rocprofv3 --pmc SQ_LDS_BANK_CONFLICT to see which pairs collide."""
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
            "cpp_lds_pair": [u32, u32, u32, u32, u32, vp, vp],
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


def cpp_lds_pair(width: int, write: bool, lane_a: int, lane_b: int, iters: int, sink_ptr: int,
                 stream: int | None) -> None:
    _check(load().cpp_lds_pair(width, int(write), lane_a, lane_b, iters, sink_ptr, stream), "cpp_lds_pair")


def lds_lane_cases() -> list[tuple[int, bool, int, int]]:
    """(width, write, lane a, lane b) of every dispatch of the lds-lanes run,
    in launch order."""
    return [(w, wr, a, b) for w in (4, 8, 16) for wr in (False, True) for a in (0, 5, 37) for b in range(64) if b != a]


def _lds_lanes() -> None:
    import json

    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    cases = lds_lane_cases()
    for w, wr, a, b in cases:
        cpp_lds_pair(w, wr, a, b, 64, sink.data_ptr(), None)
    torch.cuda.synchronize()
    print(json.dumps({"cases": cases}))


if __name__ == "__main__":
    import sys

    if sys.argv[1:] == ["lds-lanes"]:
        _lds_lanes()
    else:
        sys.exit("usage: python -m trellis_coded_row_amd.probe lds-lanes")
