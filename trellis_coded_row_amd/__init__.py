"""Conditional Program (CP) row decode for AMD Instinct MI355X (gfx950).

Python binding of ``libcp.so`` (C interface in ``include/cp.h``). This module
only marshals arguments: every step of a lookup (record gather, trellis walk,
codebook lookup, scaling, ordered write) runs in the library's HIP kernels.
PyTorch supplies device memory and streams. There is no fallback: if the
library cannot be loaded, importing this package raises.

The functions below carry the C names; ``Table`` wraps them for torch
tensors.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

# torch first: its HIP runtime must be the one libcp.so binds to. Loaded the
# other way round, the library pulls in the system's libamdhip64 and torch
# then brings its own, so the process holds two HIP runtimes and the streams
# and device pointers torch hands over belong to the other one.
import torch  # noqa: F401

from . import build as _build

__all__ = [
    "CPError", "Table", "load_library",
    "cp_record_bytes", "cp_supported", "cp_table_create", "cp_table_upload", "cp_lookup_decode",
    "cp_lookup_decode_raw", "cp_dedup_workspace_bytes", "cp_lookup_decode_dedup",
    "cp_lookup_decode_dedup_noalloc", "CP_DEDUP_NOALLOC_MAX_IDS",
    "cp_shard_plan_workspace_bytes", "cp_shard_plan", "cp_table_gather_records", "cp_lookup_decode_staged",
    "CP_MAX_SHARDS", "shard_plan",
    "cp_table_download", "cp_encode_workspace_bytes", "cp_table_encode",
    "cp_table_set_hot_rows", "cp_table_hot_rows",
    "cp_table_create_mixed", "cp_table_record_range", "cp_table_describe_mixed", "cp_mixed_desc", "MixedTable",
    "cp_table_check", "cp_table_describe", "cp_table_destroy",
    "cp_status_string", "cp_last_hip_error",
    "CP_OK", "CP_ERR_INVALID_ARGUMENT", "CP_ERR_UNSUPPORTED", "CP_ERR_OUT_OF_MEMORY", "CP_ERR_HIP",
    "CP_ERR_ID_OUT_OF_RANGE", "CP_RESIDENCY_DEVICE", "CP_RESIDENCY_HOST_MAPPED",
    "CP_FLAG_HOST_NONCOHERENT", "CP_FLAG_TOUCH_AHEAD",
]

CP_OK = 0
CP_ERR_INVALID_ARGUMENT = 1
CP_ERR_UNSUPPORTED = 2
CP_ERR_OUT_OF_MEMORY = 3
CP_ERR_HIP = 4
CP_ERR_ID_OUT_OF_RANGE = 5
CP_RESIDENCY_DEVICE = 0
CP_RESIDENCY_HOST_MAPPED = 1
CP_FLAG_HOST_NONCOHERENT = 1
CP_FLAG_TOUCH_AHEAD = 2
CP_DEDUP_NOALLOC_MAX_IDS = 65536
CP_MAX_SHARDS = 64


class cp_table_desc(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("d", ctypes.c_uint32),
        ("bits_per_step", ctypes.c_uint32),
        ("residency", ctypes.c_uint32),
        ("rows", ctypes.c_uint64),
        ("flags", ctypes.c_uint32),
        ("reserved", ctypes.c_uint32),
    ]


class cp_mixed_desc(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("d", ctypes.c_uint32),
        ("nclass", ctypes.c_uint32),
        ("bits_per_step", ctypes.c_uint32 * 4),
        ("residency", ctypes.c_uint32),
        ("rows", ctypes.c_uint64),
        ("flags", ctypes.c_uint32),
        ("reserved", ctypes.c_uint32),
    ]


_lib: ctypes.CDLL | None = None


def library_path() -> str:
    """The in-tree libcp.so this package loads (the only one it loads)."""
    return _build.LIB


def load_library() -> ctypes.CDLL:
    """Loads libcp.so, building it first only if it does not exist."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        _build.build()
    L = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    sig = {
        "cp_record_bytes": (ctypes.c_uint64, [ctypes.c_uint32, ctypes.c_uint32]),
        "cp_supported": (ctypes.c_int, [ctypes.c_uint32, ctypes.c_uint32]),
        "cp_table_create": (ctypes.c_int, [ctypes.POINTER(cp_table_desc), vp, ctypes.POINTER(vp)]),
        "cp_table_create_mixed": (ctypes.c_int, [ctypes.POINTER(cp_mixed_desc), vp, vp, ctypes.POINTER(vp)]),
        "cp_table_record_range": (ctypes.c_int, [vp, ctypes.c_uint64, ctypes.POINTER(ctypes.c_uint64),
                                                 ctypes.POINTER(ctypes.c_uint64)]),
        "cp_table_describe_mixed": (ctypes.c_int, [vp, ctypes.POINTER(cp_mixed_desc)]),
        "cp_table_upload": (ctypes.c_int, [vp, ctypes.c_uint64, ctypes.c_uint64, vp]),
        "cp_lookup_decode": (ctypes.c_int, [vp, vp, ctypes.c_uint64, vp, vp]),
        "cp_lookup_decode_raw": (ctypes.c_int, [vp, vp, ctypes.c_uint64, vp, vp]),
        "cp_dedup_workspace_bytes": (ctypes.c_uint64, [vp, ctypes.c_uint64]),
        "cp_lookup_decode_dedup": (ctypes.c_int, [vp, vp, ctypes.c_uint64, vp, vp, ctypes.c_uint64, vp]),
        "cp_lookup_decode_dedup_noalloc": (ctypes.c_int, [vp, vp, ctypes.c_uint64, vp, vp]),
        "cp_shard_plan_workspace_bytes": (ctypes.c_uint64, [ctypes.c_uint64, ctypes.c_uint32]),
        "cp_shard_plan": (ctypes.c_int, [vp, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint32, vp, vp, vp, vp,
                                         ctypes.c_uint64, vp]),
        "cp_table_gather_records": (ctypes.c_int, [vp, vp, ctypes.c_uint64, vp, vp]),
        "cp_lookup_decode_staged": (ctypes.c_int, [vp, vp, ctypes.c_uint64, vp, ctypes.c_uint64, vp, vp]),
        "cp_table_download": (ctypes.c_int, [vp, ctypes.c_uint64, ctypes.c_uint64, vp]),
        "cp_encode_workspace_bytes": (ctypes.c_uint64, [vp, ctypes.c_uint64]),
        "cp_table_encode": (ctypes.c_int, [vp, ctypes.c_uint64, ctypes.c_uint64, vp, vp, ctypes.c_uint64, vp]),
        "cp_table_set_hot_rows": (ctypes.c_int, [vp, vp, ctypes.c_uint64]),
        "cp_table_hot_rows": (ctypes.c_uint64, [vp]),
        "cp_table_check": (ctypes.c_int, [vp, vp]),
        "cp_table_describe": (ctypes.c_int, [vp, ctypes.POINTER(cp_table_desc)]),
        "cp_table_destroy": (ctypes.c_int, [vp]),
        "cp_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "cp_last_hip_error": (ctypes.c_int, []),
    }
    for name, (res, args) in sig.items():
        if not hasattr(L, name):
            raise ImportError(f"{path} does not export {name}: it is older than its sources; "
                              "rebuild it (python trellis_coded_row_amd/build.py)")
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


_L = load_library()


class CPError(RuntimeError):

    def __init__(self, status: int, what: str):
        self.status = status
        msg = f"{what}: {cp_status_string(status)}"
        if status == CP_ERR_HIP:
            msg += f" (hipError {cp_last_hip_error()})"
        super().__init__(msg)


# --------------------------------------------------------------------------
# the C functions, same names, raw pointers and integers
# --------------------------------------------------------------------------

def cp_record_bytes(d: int, bits_per_step: int) -> int:
    return int(_L.cp_record_bytes(d, bits_per_step))


def cp_supported(d: int, bits_per_step: int) -> bool:
    return bool(_L.cp_supported(d, bits_per_step))


def cp_table_create(desc: cp_table_desc, lut_ptr: int) -> tuple[int, int]:
    """Returns (status, table handle or 0)."""
    h = ctypes.c_void_p()
    st = _L.cp_table_create(ctypes.byref(desc), lut_ptr, ctypes.byref(h))
    return st, (h.value or 0)


def cp_table_create_mixed(desc: cp_mixed_desc, lut_ptr: int, row_class_ptr: int) -> tuple[int, int]:
    """Returns (status, table handle or 0)."""
    h = ctypes.c_void_p()
    st = _L.cp_table_create_mixed(ctypes.byref(desc), lut_ptr, row_class_ptr, ctypes.byref(h))
    return st, (h.value or 0)


def cp_table_record_range(table: int, row: int) -> tuple[int, int, int]:
    """Returns (status, byte offset, bytes) of a row's record."""
    off, nb = ctypes.c_uint64(), ctypes.c_uint64()
    st = _L.cp_table_record_range(table, row, ctypes.byref(off), ctypes.byref(nb))
    return st, int(off.value), int(nb.value)


def cp_table_describe_mixed(table: int) -> tuple[int, cp_mixed_desc]:
    desc = cp_mixed_desc()
    st = _L.cp_table_describe_mixed(table, ctypes.byref(desc))
    return st, desc


def cp_table_upload(table: int, first_row: int, nrows: int, src_ptr: int) -> int:
    return _L.cp_table_upload(table, first_row, nrows, src_ptr)


def cp_lookup_decode(table: int, ids_ptr: int, n: int, out_ptr: int, stream: int | None) -> int:
    return _L.cp_lookup_decode(table, ids_ptr, n, out_ptr, stream)


def cp_lookup_decode_raw(table: int, ids_ptr: int, n: int, out_ptr: int, stream: int | None) -> int:
    return _L.cp_lookup_decode_raw(table, ids_ptr, n, out_ptr, stream)


def cp_dedup_workspace_bytes(table: int, n: int) -> int:
    return int(_L.cp_dedup_workspace_bytes(table, n))


def cp_lookup_decode_dedup(table: int, ids_ptr: int, n: int, out_ptr: int, workspace_ptr: int,
                           workspace_bytes: int, stream: int | None) -> int:
    return _L.cp_lookup_decode_dedup(table, ids_ptr, n, out_ptr, workspace_ptr, workspace_bytes, stream)


def cp_lookup_decode_dedup_noalloc(table: int, ids_ptr: int, n: int, out_ptr: int, stream: int | None) -> int:
    return _L.cp_lookup_decode_dedup_noalloc(table, ids_ptr, n, out_ptr, stream)


def cp_shard_plan_workspace_bytes(n: int, shards: int) -> int:
    return int(_L.cp_shard_plan_workspace_bytes(n, shards))


def cp_shard_plan(ids_ptr: int, n: int, rows_per_shard: int, shards: int, local_ids_ptr: int, positions_ptr: int,
                  counts_ptr: int, workspace_ptr: int, workspace_bytes: int, stream: int | None) -> int:
    return _L.cp_shard_plan(ids_ptr, n, rows_per_shard, shards, local_ids_ptr, positions_ptr, counts_ptr,
                            workspace_ptr, workspace_bytes, stream)


def cp_table_gather_records(table: int, ids_ptr: int, n: int, dst_ptr: int, stream: int | None) -> int:
    return _L.cp_table_gather_records(table, ids_ptr, n, dst_ptr, stream)


def cp_lookup_decode_staged(table: int, records_ptr: int, nrecords: int, positions_ptr: int, n: int, out_ptr: int,
                            stream: int | None) -> int:
    return _L.cp_lookup_decode_staged(table, records_ptr, nrecords, positions_ptr, n, out_ptr, stream)


def shard_plan(ids, rows_per_shard: int, shards: int, stream=None):
    """(local_ids int64[n], positions int64[n], counts int64[shards]) of
    cp_shard_plan for a contiguous 1-D int64 device tensor of global ids:
    the ids grouped by owning shard (owner = id // rows_per_shard), each as
    its row within the shard, in batch order within a shard; for each
    lookup its index in that grouping (-1 when no shard owns the id); and
    the number of ids per shard."""
    if not (ids.is_cuda and ids.dtype == torch.int64 and ids.dim() == 1 and ids.is_contiguous()):
        raise ValueError("ids must be a contiguous 1-D int64 device tensor")
    n = ids.shape[0]
    local_ids = torch.empty(max(n, 1), dtype=torch.int64, device=ids.device)
    positions = torch.empty(max(n, 1), dtype=torch.int64, device=ids.device)
    counts = torch.empty(max(shards, 1), dtype=torch.int64, device=ids.device)
    need = cp_shard_plan_workspace_bytes(n, shards)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=ids.device)
    st = cp_shard_plan(ids.data_ptr(), n, rows_per_shard, shards, local_ids.data_ptr(), positions.data_ptr(),
                       counts.data_ptr(), ws.data_ptr(), ws.numel(), _stream_handle(stream))
    if st != CP_OK:
        raise CPError(st, "cp_shard_plan")
    for t in (local_ids, positions, counts, ws):
        _keep_for_stream(t, stream)
    return local_ids[:n], positions[:n], counts[:shards]


def cp_table_download(table: int, first_row: int, nrows: int, dst_ptr: int) -> int:
    return _L.cp_table_download(table, first_row, nrows, dst_ptr)


def cp_encode_workspace_bytes(table: int, nrows: int) -> int:
    return int(_L.cp_encode_workspace_bytes(table, nrows))


def cp_table_encode(table: int, first_row: int, nrows: int, rows_ptr: int, workspace_ptr: int,
                    workspace_bytes: int, stream: int | None) -> int:
    return _L.cp_table_encode(table, first_row, nrows, rows_ptr, workspace_ptr, workspace_bytes, stream)


def cp_table_set_hot_rows(table: int, rows_ptr: int, count: int) -> int:
    return _L.cp_table_set_hot_rows(table, rows_ptr, count)


def cp_table_hot_rows(table: int) -> int:
    return int(_L.cp_table_hot_rows(table))


def cp_table_check(table: int, stream: int | None) -> int:
    return _L.cp_table_check(table, stream)


def cp_table_describe(table: int) -> tuple[int, cp_table_desc]:
    desc = cp_table_desc()
    st = _L.cp_table_describe(table, ctypes.byref(desc))
    return st, desc


def cp_table_destroy(table: int) -> int:
    return _L.cp_table_destroy(table)


def cp_status_string(status: int) -> str:
    return _L.cp_status_string(status).decode()


def cp_last_hip_error() -> int:
    return int(_L.cp_last_hip_error())


# --------------------------------------------------------------------------
# torch convenience wrapper
# --------------------------------------------------------------------------

def _stream_handle(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _keep_for_stream(tensor, stream) -> None:
    """A tensor allocated here on torch's current stream and used by work on
    `stream`: tell torch's caching allocator, so the memory is not handed out
    again before that work is done."""
    if stream is None:
        return
    s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(int(stream))
    if s != torch.cuda.current_stream():
        tensor.record_stream(s)


class Table:
    """A CP table on the current device (or in pinned host memory).

    lut_fp16: uint16[512, 2] codebook bit patterns. Records are uploaded
    with ``upload`` (packed bytes, ``record_bytes`` each)."""

    def __init__(self, rows: int, d: int, bits_per_step: int, lut_fp16: np.ndarray,
                 residency: int = CP_RESIDENCY_DEVICE, flags: int = 0):
        lut = np.ascontiguousarray(lut_fp16, dtype=np.uint16).reshape(-1)
        if lut.size != 1024:
            raise ValueError("the codebook has 512 entries of 2 fp16 values")
        desc = cp_table_desc(ctypes.sizeof(cp_table_desc), d, bits_per_step, residency, rows, flags, 0)
        st, h = cp_table_create(desc, lut.ctypes.data)
        if st != CP_OK:
            raise CPError(st, "cp_table_create")
        self.handle = h
        self.rows, self.d, self.bits_per_step = rows, d, bits_per_step
        self.residency = residency
        self.record_bytes = cp_record_bytes(d, bits_per_step)

    def upload(self, records: np.ndarray, first_row: int = 0) -> None:
        rec = np.ascontiguousarray(records, dtype=np.uint8)
        if rec.ndim != 2 or rec.shape[1] != self.record_bytes:
            raise ValueError(f"records must be uint8[nrows, {self.record_bytes}]")
        st = cp_table_upload(self.handle, first_row, rec.shape[0], rec.ctypes.data)
        if st != CP_OK:
            raise CPError(st, "cp_table_upload")

    def record_range(self, row: int) -> tuple[int, int]:
        """(byte offset, bytes) of a row's record in the packed records."""
        st, off, nb = cp_table_record_range(self.handle, row)
        if st != CP_OK:
            raise CPError(st, "cp_table_record_range")
        return off, nb

    def _check_io(self, ids, out, dtype):
        if not (ids.is_cuda and ids.dtype == torch.int64 and ids.dim() == 1 and ids.is_contiguous()):
            raise ValueError("ids must be a contiguous 1-D int64 device tensor")
        n = ids.shape[0]
        if out is None:
            out = torch.empty((n, self.d), dtype=dtype, device=ids.device)
        if not (out.is_cuda and out.dtype == dtype and tuple(out.shape) == (n, self.d)
                and out.is_contiguous()):
            raise ValueError(f"out must be a contiguous {dtype} device tensor of shape ({n}, {self.d})")
        return n, out

    def lookup_decode(self, ids, out=None, stream=None):
        """bf16[n, d]: alpha * f(c) of rows ids[j], in lookup order."""
        own = out is None
        n, out = self._check_io(ids, out, torch.bfloat16)
        st = cp_lookup_decode(self.handle, ids.data_ptr(), n, out.data_ptr(), _stream_handle(stream))
        if st != CP_OK:
            raise CPError(st, "cp_lookup_decode")
        if own:
            _keep_for_stream(out, stream)
        return out

    def lookup_decode_raw(self, ids, out=None, stream=None):
        """fp16[n, d]: the unscaled f(c) of rows ids[j], in lookup order."""
        own = out is None
        n, out = self._check_io(ids, out, torch.float16)
        st = cp_lookup_decode_raw(self.handle, ids.data_ptr(), n, out.data_ptr(), _stream_handle(stream))
        if st != CP_OK:
            raise CPError(st, "cp_lookup_decode_raw")
        if own:
            _keep_for_stream(out, stream)
        return out

    def dedup_workspace_bytes(self, n: int) -> int:
        return cp_dedup_workspace_bytes(self.handle, n)

    def lookup_decode_dedup(self, ids, out=None, workspace=None, stream=None):
        """bf16[n, d] like lookup_decode, each distinct record fetched once.
        workspace: a uint8 device tensor of at least dedup_workspace_bytes(n)
        bytes (allocated here when None); scratch, reusable across calls that
        do not overlap."""
        own_out = out is None
        n, out = self._check_io(ids, out, torch.bfloat16)
        need = self.dedup_workspace_bytes(n)
        own = workspace is None
        if own:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=ids.device)
        st = cp_lookup_decode_dedup(self.handle, ids.data_ptr(), n, out.data_ptr(), workspace.data_ptr(),
                                    workspace.numel() * workspace.element_size(), _stream_handle(stream))
        if st != CP_OK:
            raise CPError(st, "cp_lookup_decode_dedup")
        if own:
            _keep_for_stream(workspace, stream)
        if own_out:
            _keep_for_stream(out, stream)
        return out

    def lookup_decode_dedup_noalloc(self, ids, out, stream=None):
        """bf16[n, d] like lookup_decode_dedup, with the library's fixed
        per-device scratch instead of a workspace (n <= CP_DEDUP_NOALLOC_MAX_IDS;
        `out` must be given: nothing is allocated; calls must not overlap on
        one device)."""
        if out is None:
            raise ValueError("out must be given (this call allocates nothing)")
        n, out = self._check_io(ids, out, torch.bfloat16)
        st = cp_lookup_decode_dedup_noalloc(self.handle, ids.data_ptr(), n, out.data_ptr(), _stream_handle(stream))
        if st != CP_OK:
            raise CPError(st, "cp_lookup_decode_dedup_noalloc")
        return out

    def gather_records(self, ids, dst=None, stream=None):
        """uint8[n, R] device tensor: the records of rows ids[k], packed (the
        owner's step of a sharded lookup); 64 bytes of padding follow the
        last record when allocated here, so the result can be decoded by
        lookup_decode_staged directly."""
        if not (ids.is_cuda and ids.dtype == torch.int64 and ids.dim() == 1 and ids.is_contiguous()):
            raise ValueError("ids must be a contiguous 1-D int64 device tensor")
        n, R = ids.shape[0], self.record_bytes
        own = dst is None
        if own:
            dst = torch.zeros(n * R + 64, dtype=torch.uint8, device=ids.device)
        elif not (dst.is_cuda and dst.dtype == torch.uint8 and dst.is_contiguous() and dst.numel() >= n * R):
            raise ValueError(f"dst must be a contiguous uint8 device tensor of at least {n * R} bytes")
        st = cp_table_gather_records(self.handle, ids.data_ptr(), n, dst.data_ptr(), _stream_handle(stream))
        if st != CP_OK:
            raise CPError(st, "cp_table_gather_records")
        if own:
            _keep_for_stream(dst, stream)
        return dst

    def lookup_decode_staged(self, records, nrecords: int, positions, out=None, stream=None):
        """bf16[n, d]: row j decodes record positions[j] of the packed
        buffer `records` (a uint8 device tensor of at least nrecords * R + 64
        bytes), with this table's codebook (the requester's step of a
        sharded lookup)."""
        R = self.record_bytes
        if not (records.is_cuda and records.dtype == torch.uint8 and records.is_contiguous()
                and records.numel() >= nrecords * R + 64 and records.data_ptr() % 16 == 0):
            raise ValueError("records must be a contiguous, 16-byte aligned uint8 device tensor of at least "
                             f"{nrecords * R + 64} bytes")
        own = out is None
        n, out = self._check_io(positions, out, torch.bfloat16)
        st = cp_lookup_decode_staged(self.handle, records.data_ptr(), nrecords, positions.data_ptr(), n,
                                     out.data_ptr(), _stream_handle(stream))
        if st != CP_OK:
            raise CPError(st, "cp_lookup_decode_staged")
        if own:
            _keep_for_stream(out, stream)
        return out

    def download(self, first_row: int = 0, nrows: int | None = None) -> np.ndarray:
        """uint8[nrows, record_bytes]: the stored records (waits for the device)."""
        if nrows is None:
            nrows = self.rows - first_row
        out = np.empty((nrows, self.record_bytes), dtype=np.uint8)
        st = cp_table_download(self.handle, first_row, nrows, out.ctypes.data)
        if st != CP_OK:
            raise CPError(st, "cp_table_download")
        return out

    def encode_workspace_bytes(self, nrows: int) -> int:
        return cp_encode_workspace_bytes(self.handle, nrows)

    def encode(self, rows, first_row: int = 0, workspace=None, stream=None) -> None:
        """Encodes fp32 device rows [nrows, d] into records first_row.. of the
        table (asynchronous on `stream`). workspace: a uint8 device tensor of
        at least encode_workspace_bytes(nrows) bytes (allocated when None)."""
        if not (rows.is_cuda and rows.dtype == torch.float32 and rows.dim() == 2 and rows.shape[1] == self.d
                and rows.is_contiguous()):
            raise ValueError(f"rows must be a contiguous float32 device tensor of shape (n, {self.d})")
        n = rows.shape[0]
        need = self.encode_workspace_bytes(n)
        own = workspace is None
        if own:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=rows.device)
        st = cp_table_encode(self.handle, first_row, n, rows.data_ptr(), workspace.data_ptr(),
                             workspace.numel() * workspace.element_size(), _stream_handle(stream))
        if st != CP_OK:
            raise CPError(st, "cp_table_encode")
        if own:
            _keep_for_stream(workspace, stream)

    def set_hot_rows(self, rows) -> int:
        """Keeps device copies of these rows' records (pinned-host tables);
        returns the number of distinct rows cached. Empty: drop the copies."""
        r = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1)
        st = cp_table_set_hot_rows(self.handle, r.ctypes.data if r.size else 0, r.size)
        if st != CP_OK:
            raise CPError(st, "cp_table_set_hot_rows")
        return cp_table_hot_rows(self.handle)

    def check(self, stream=None) -> bool:
        """Synchronises; False (and the flag cleared) if an id was out of range."""
        st = cp_table_check(self.handle, _stream_handle(stream))
        if st == CP_ERR_ID_OUT_OF_RANGE:
            return False
        if st != CP_OK:
            raise CPError(st, "cp_table_check")
        return True

    def close(self) -> None:
        if getattr(self, "handle", 0):
            st = cp_table_destroy(self.handle)
            self.handle = 0
            if st != CP_OK:
                raise CPError(st, "cp_table_destroy")

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class MixedTable(Table):
    """A mixed-rate CP table: row i is coded at bits_per_step[row_class[i]].
    Records are uploaded as the rows' packed bytes (``upload_bytes``); lookups
    are those of ``Table``."""

    def __init__(self, d: int, bits_per_step, row_class: np.ndarray, lut_fp16: np.ndarray,
                 residency: int = CP_RESIDENCY_DEVICE, flags: int = 0):
        lut = np.ascontiguousarray(lut_fp16, dtype=np.uint16).reshape(-1)
        if lut.size != 1024:
            raise ValueError("the codebook has 512 entries of 2 fp16 values")
        cls = np.ascontiguousarray(row_class, dtype=np.uint8).reshape(-1)
        kvs = list(bits_per_step)
        if not 1 <= len(kvs) <= 4:
            raise ValueError("1 to 4 rate classes")
        arr = (ctypes.c_uint32 * 4)(*(kvs + [0] * (4 - len(kvs))))
        desc = cp_mixed_desc(ctypes.sizeof(cp_mixed_desc), d, len(kvs), arr, residency, cls.size, flags, 0)
        st, h = cp_table_create_mixed(desc, lut.ctypes.data, cls.ctypes.data)
        if st != CP_OK:
            raise CPError(st, "cp_table_create_mixed")
        self.handle = h
        self.rows, self.d, self.bits_per_step = cls.size, d, 0
        self.rates = tuple(kvs)
        self.residency = residency
        self.record_bytes = 0

    def upload(self, records: np.ndarray, first_row: int = 0) -> None:
        raise TypeError("use upload_bytes(packed, first_row, nrows) on a mixed-rate table")

    def upload_bytes(self, packed: np.ndarray, first_row: int, nrows: int) -> None:
        """packed: the uint8 records of rows [first_row, first_row + nrows), back to back."""
        buf = np.ascontiguousarray(packed, dtype=np.uint8).reshape(-1)
        off0, _ = self.record_range(first_row)
        off1, nb1 = self.record_range(first_row + nrows - 1)
        if buf.size != off1 + nb1 - off0:
            raise ValueError(f"expected {off1 + nb1 - off0} bytes, got {buf.size}")
        st = cp_table_upload(self.handle, first_row, nrows, buf.ctypes.data)
        if st != CP_OK:
            raise CPError(st, "cp_table_upload")

    def download(self, first_row: int = 0, nrows: int | None = None) -> np.ndarray:
        """uint8[bytes]: the packed records of rows [first_row, first_row + nrows)."""
        if nrows is None:
            nrows = self.rows - first_row
        off0, _ = self.record_range(first_row)
        off1, nb1 = self.record_range(first_row + nrows - 1)
        out = np.empty(off1 + nb1 - off0, dtype=np.uint8)
        st = cp_table_download(self.handle, first_row, nrows, out.ctypes.data)
        if st != CP_OK:
            raise CPError(st, "cp_table_download")
        return out
