"""The measurement probes (include/cp_probe.h) measure what the bench says
they measure: the store-only probe writes every output row of the lookup,
exactly once and in the lookup's places, so its time is the floor of the
lookup's output stream; the read and gather probes and the LDS lane probe
run to completion on valid arguments."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workload
from parity import say
from trellis_coded_row_amd import probe

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    torch.cuda.init()


def expected_store(n: int, d: int) -> np.ndarray:
    """What cpp_store_rows writes: lane l of row r stores the 4 dwords v, v^1,
    v^2, v^3 with v = r * 0x9E3779B9 + l (mod 2^32), at dwords [4l, 4l + 4)
    of the row."""
    lanes = d // 8
    r = np.arange(n, dtype=np.uint64)[:, None]
    l = np.arange(lanes, dtype=np.uint64)[None, :]
    v = ((r * np.uint64(0x9E3779B9) + l) & np.uint64(0xFFFFFFFF)).astype(np.uint32)
    return np.stack([v, v ^ 1, v ^ 2, v ^ 3], axis=-1).reshape(n, d // 2)


@pytest.mark.parametrize("d", [64, 256, 512])
@pytest.mark.parametrize("chunk", [1, 4, 16])
def test_store_probe_writes_every_row_once(d, chunk):
    for n in (1, 1000, 16_385):
        say(f"store probe d{d} chunk{chunk} n{n}")
        out = torch.full((n, d), -1, dtype=torch.int16, device="cuda")
        probe.cpp_store_rows(out.data_ptr(), n, d, chunk, None)
        torch.cuda.synchronize()
        got = out.cpu().numpy().view(np.uint32).reshape(n, d // 2)
        assert (got == expected_store(n, d)).all()


def test_read_and_gather_probes_run():
    rows, d, kv = 5000, 512, 4
    recs = torch.from_numpy(workload.random_records(rows, d, kv, seed=77).reshape(-1).copy())
    dev = torch.empty(recs.numel() + 64, dtype=torch.uint8, device="cuda")
    dev[: recs.numel()].copy_(recs)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    ids = torch.from_numpy(workload.zipf_ids(rows, 3001, seed=78)).cuda()
    probe.cpp_gather_records(dev.data_ptr(), recs.numel() // rows, ids.data_ptr(), ids.numel(), sink.data_ptr(), None)
    buf = torch.arange(1 << 18, dtype=torch.int32, device="cuda")
    probe.cpp_read_stream(buf.data_ptr(), buf.numel() * 4, sink.data_ptr(), None)
    for width in (4, 8, 16):
        for write in (False, True):
            probe.cpp_lds_pair(width, write, 0, 12, 8, sink.data_ptr(), None)
    torch.cuda.synchronize()
