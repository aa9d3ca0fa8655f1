#!/usr/bin/env python3
"""Benchmark of the CP fused gather-and-decode on one GPU.

Workload (default): the 393,216-lookup replay (4,096 tokens x 48 rows x 2
memory layers, ids Zipf(1.1) over a permuted table) into the 97,690,000 x d512
table of 130-byte records (12.70 GB, kv = 4, i.e. 2 bits per element plus one
bf16 scale per row) resident in HBM. One step = one cp_lookup_decode call over
the whole replay: gather every requested record, walk the trellis, scale, and
write the 393,216 x 512 bf16 rows in lookup order.

Prints one JSON line. value = decoded rows/s over the K timed steps (inputs
resident in HBM before timing starts); roofline = effective bytes per launch
(records read + bf16 rows written, n * (R + 2d)) over the average launch time
measured with events on the launch stream, against the 8 TB/s HBM peak;
cpu_baseline = the CPU oracle decoding a sample of the same replay;
flushed_* = the same launch timed one at a time after L2 and MALL are evicted
(cold records), alongside the warm back-to-back figure that is the value.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decoded rows/s + effective GB/s (% of HBM peak), 393,216-lookup replay"
HBM_PEAK_GBPS = 8000.0
CSRC = os.path.join(ROOT, "trellis_coded_row_amd", "csrc")
# the sources of each lookup kernel (a counter summary is valid for these bytes)
KERNEL_SOURCES = {
    "single": ("cp_decode.hip", "cp_lane.h"),
    "mixed": ("cp_mixed.hip", "cp_lane.h"),
    "encode": ("cp_encode.hip", "cp_encode_copies.h"),
    "shard": ("cp_shard.hip", "cp_decode.hip", "cp_lane.h"),
}
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_hash(kind: str = "single") -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind]:
        with open(os.path.join(CSRC, name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_counter_summary(config: str, ids_kind: str, kind: str = "single") -> dict | None:
    """Memory traffic per launch from a committed rocprofv3 --pmc summary, if
    it was taken on the current kernel sources: HBM bytes (FETCH_SIZE and
    WRITE_SIZE, scaled by what they read for a copy of known size) and, for a
    table in host memory, the bytes read over PCIe."""
    path = os.path.join(PROFILES, f"counters_gather_decode_{config}_{ids_kind}.txt")
    if not os.path.exists(path):
        return None
    vals: dict[str, str] = {}
    with open(path) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#") and ":" in line:
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != kernel_source_hash(kind):
        return None
    try:
        fetch = float(vals["FETCH_SIZE_KiB_per_dispatch"]) * 1024 * float(vals["fetch_scale"])
        write = float(vals["WRITE_SIZE_KiB_per_dispatch"]) * 1024 * float(vals["write_scale"])
    except (KeyError, ValueError):
        return None
    res = {"fetch_bytes": fetch, "write_bytes": write, "bytes": fetch + write, "file": os.path.basename(path)}
    if "PCIE_READ_BYTES_per_dispatch" in vals:
        res["pcie_bytes"] = float(vals["PCIE_READ_BYTES_per_dispatch"])
    return res


def read_shard_counters(G: int) -> dict | None:
    """HBM bytes per dispatch of each kernel of the sharded workload's steps,
    from a committed rocprofv3 --pmc summary taken on the current sources."""
    path = os.path.join(PROFILES, f"counters_shard_steps_sharded_d512_g{G}.txt")
    if not os.path.exists(path):
        return None
    vals: dict[str, str] = {}
    with open(path) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#") and ":" in line:
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != kernel_source_hash("shard"):
        return None
    try:
        fs, ws = float(vals["fetch_scale"]), float(vals["write_scale"])
        res = {}
        for k in ("shard_count", "shard_scan", "shard_scatter", "gather_records", "gather_decode"):
            f = float(vals[f"{k}_FETCH_SIZE_KiB_per_dispatch"]) * 1024 * fs
            w = float(vals[f"{k}_WRITE_SIZE_KiB_per_dispatch"]) * 1024 * ws
            res[k] = {"fetch_bytes": f, "write_bytes": w, "bytes": f + w}
    except (KeyError, ValueError):
        return None
    res["file"] = os.path.basename(path)
    return res


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def time_region(fn, steps: int, torch) -> float:
    """ms of `steps` back-to-back calls of fn() on the current stream, between
    one pair of events (synchronised before and after)."""
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(steps):
        fn()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1)


def time_each(fn, steps: int, torch, before=None) -> list[float]:
    """ms of each call of fn(), each between its own pair of events; before()
    runs outside the timed pairs."""
    stream = torch.cuda.current_stream()
    out = []
    for _ in range(steps):
        if before is not None:
            before()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b))
    return out


def graph_timing(step, out, steps: int, torch, per_graph: int = 16) -> dict:
    """Per-lookup ms when `per_graph` lookups are captured in one HIP graph
    and the graph is replayed (no host launch cost per lookup). Every check
    replay is compared bit for bit with the eager result, with eager work and
    a synchronisation between replays."""
    torch.cuda.synchronize()
    ref = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            step()
    same = 0
    checks = 4
    for _ in range(checks):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same += int(torch.equal(out.view(torch.int16), ref.view(torch.int16)))
    reps = max(2, steps // per_graph)
    for _ in range(2):
        g.replay()
    ms = time_region(g.replay, reps, torch)
    del g
    return {"lookups_per_graph": per_graph, "replays": reps, "launch_ms_mean": ms / (reps * per_graph),
            "replays_matching_eager": f"{same}/{checks}"}


def graph_call_ms(fn, steps: int, torch, per_graph: int = 16) -> float:
    """ms per call of fn() when `per_graph` calls are captured in one HIP
    graph and the graph is replayed."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            fn()
    reps = max(2, steps // per_graph)
    for _ in range(2):
        g.replay()
    ms = time_region(g.replay, reps, torch)
    del g
    return ms / (reps * per_graph)


def batch_scan(table, ids_np, d: int, bytes_per_lookup: float, torch, np) -> dict:
    """ms per launch for batches of growing size (the replay's ids tiled),
    launched one by one and replayed from a captured graph (device time
    without the host's launch cost), and the marginal rate between the two
    largest: what one more lookup costs once the launch's fixed start-up and
    drain are paid."""
    sizes = [96, 1536, 12288, 49152, 98304, 196608, 393216, 786432, 1572864]
    rows = []
    for n in sizes:
        reps = -(-n // len(ids_np))
        ids = torch.from_numpy(np.tile(ids_np, reps)[:n]).cuda()
        out = torch.empty((n, d), dtype=torch.bfloat16, device="cuda")
        step = lambda: table.lookup_decode(ids, out)
        for _ in range(20):
            step()
        steps = max(20, min(400, int(4e7 // n)))
        ms = time_region(step, steps, torch) / steps
        g = graph_timing(step, out, steps, torch, per_graph=8)
        if not g["replays_matching_eager"].startswith("4/"):
            raise RuntimeError(f"a graph replay differs from the eager lookup at n = {n}")
        gms = g["launch_ms_mean"]
        rows.append({"n": n, "launch_ms": ms, "graph_launch_ms": gms,
                     "effective_GBps": n * bytes_per_lookup / (ms / 1e3) / 1e9,
                     "graph_effective_GBps": n * bytes_per_lookup / (gms / 1e3) / 1e9})
        del ids, out
    a, b = rows[-2], rows[-1]
    marg_s = (b["launch_ms"] - a["launch_ms"]) / 1e3 / (b["n"] - a["n"])
    fixed_ms = a["launch_ms"] - a["n"] * marg_s * 1e3
    torch.cuda.empty_cache()
    return {"points": rows, "marginal_rows_per_s": 1.0 / marg_s,
            "marginal_effective_GBps": bytes_per_lookup / marg_s / 1e9,
            "marginal_pct_hbm_peak": 100.0 * bytes_per_lookup / marg_s / 1e9 / HBM_PEAK_GBPS,
            "fixed_ms_per_launch": fixed_ms}


def probes(torch, mib: int = 1024) -> dict:
    """Achievable HBM bandwidth of a plain copy and a plain fill (torch's own
    kernels) of `mib` MiB, for context next to the 8 TB/s peak."""
    n = mib * (1 << 20) // 4
    a = torch.empty(n, dtype=torch.int32, device="cuda")
    b = torch.empty(n, dtype=torch.int32, device="cuda")
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    copy_ms = time_region(lambda: b.copy_(a), 10, torch) / 10
    fill_ms = time_region(lambda: b.fill_(7), 10, torch) / 10
    nbytes = n * 4
    out = {"copy_GBps": 2 * nbytes / copy_ms / 1e6, "fill_GBps": nbytes / fill_ms / 1e6, "MiB": mib}
    del a, b
    torch.cuda.empty_cache()
    return out


def pcie_probe(torch, mib: int = 1024) -> dict:
    """Host-to-device bandwidth from pinned host memory, two ways: a DMA copy
    (torch copy of `mib` MiB, the denominator for a table read over PCIe) and
    a kernel reading the same pinned buffer in place (zero-copy, as the
    lookup reads a host-resident table: cpp_read_stream)."""
    from trellis_coded_row_amd import probe as cpp

    n = mib * (1 << 20) // 4
    h = torch.empty(n, dtype=torch.int32, pin_memory=True)
    d = torch.empty(n, dtype=torch.int32, device="cuda")
    h.fill_(3)
    for _ in range(2):
        d.copy_(h, non_blocking=True)
    ms = time_region(lambda: d.copy_(h, non_blocking=True), 5, torch) / 5
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    zc = lambda: cpp.cpp_read_stream(h.data_ptr(), n * 4, sink.data_ptr(), stream)
    for _ in range(2):
        zc()
    zc_ms = time_region(zc, 5, torch) / 5
    del h, d
    torch.cuda.empty_cache()
    return {"h2d_GBps": n * 4 / ms / 1e6, "zero_copy_read_GBps": n * 4 / zc_ms / 1e6, "MiB": mib}


def lookup_chunk(n: int, cus: int) -> int:
    """Rows per wave chunk the lookup launch picks for n lookups (at least 8
    waves per CU: 16 rows from 16 * 8 * cus lookups, 4 from 4 * 8 * cus)."""
    waves = cus * 8
    return 16 if n >= 16 * waves else (4 if n >= 4 * waves else 1)


def floor_probes(torch, np, records, R: int, d: int, ids_np, host: bool, flush) -> dict:
    """The lookup's two halves timed alone on the same workload: its output
    stream (cpp_store_rows: the same rows, same placement, no loads) and its
    record fetch (cpp_gather_records: the same ids and record reads from a
    copy of the records in the same kind of memory, no decode, no stores),
    each back to back (warm) and after an L2/MALL eviction (cold)."""
    from trellis_coded_row_amd import probe as cpp

    n = ids_np.shape[0]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream().cuda_stream
    out = torch.empty((n, d), dtype=torch.bfloat16, device="cuda")
    ids = torch.from_numpy(ids_np).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    flat = np.ascontiguousarray(records).reshape(-1)
    if host:
        rec = torch.empty(flat.size + 64, dtype=torch.uint8, pin_memory=True)
        rec[: flat.size].numpy()[:] = flat
    else:
        rec = torch.empty(flat.size + 64, dtype=torch.uint8, device="cuda")
        step = 1 << 30
        for a in range(0, flat.size, step):
            b = min(a + step, flat.size)
            rec[a:b].copy_(torch.from_numpy(flat[a:b]))
    rec[flat.size:].zero_()  # loads of the last record may touch a few bytes past it
    store = lambda: cpp.cpp_store_rows(out.data_ptr(), n, d, lookup_chunk(n, cus), stream)
    gather = lambda: cpp.cpp_gather_records(rec.data_ptr(), R, ids.data_ptr(), n, sink.data_ptr(), stream)
    res = {}
    for name, fn in (("store_only", store), ("gather_only", gather)):
        for _ in range(10):
            fn()
        warm = time_region(fn, 50, torch) / 50
        cold = time_each(fn, 20, torch, before=flush)
        res[f"{name}_ms"] = warm
        res[f"{name}_flushed_ms"] = sum(cold) / len(cold)
    res["store_only_GBps"] = n * 2 * d / (res["store_only_ms"] / 1e3) / 1e9
    del out, ids, rec, sink
    torch.cuda.empty_cache()
    return res


VALU_PEAK_TOPS = 39.3  # 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz: one 64-bit VALU op per lane-slot


def bench_encode(args, np, torch, cp, workload) -> int:
    """Trellis-coded quantisation of a batch of rows (cp_table_encode): one
    step = encode the whole batch. The add-compare-select of the Viterbi
    recursion dominates: 2 passes x T steps x 2^16 branches per row, each an
    fp64 add and an fp64 compare, i.e. 2 * 2 * (d/2) * 2^16 algorithmic fp64
    operations per row, bounded by the VALU issue rate."""
    d, kv, n = args.encode_d, args.encode_kv, args.encode_rows
    lut = workload.lut_fp16(0)
    e = workload.gaussian_rows(n, d, seed=9100).astype(np.float32)
    table = cp.Table(n, d, kv, lut)
    rows = torch.from_numpy(e).cuda()
    ws = torch.empty(table.encode_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    step = lambda: table.encode(rows, workspace=ws)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    total_ms = time_region(step, args.steps, torch)
    wall_s = time.perf_counter() - wall0
    ms = total_ms / args.steps
    branches = 2 * (d // 2) * (1 << 16) * n
    ops = 2 * branches
    achieved = ops / (ms / 1e3) / 1e12
    res = {
        "metric": "encoded rows/s (trellis-coded quantisation, two-pass tail-biting Viterbi)",
        "value": n / (ms / 1e3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "config": {
            "workload": f"encode_d{d}_kv{kv}: {n:,} Gaussian rows (d={d}) quantised to {kv / 2:g} bits/element "
                        f"+ bf16 scale ({table.record_bytes}-byte records)",
            "rows": n, "d": d, "bits_per_step": kv, "entry_point": "cp_table_encode",
            "workspace_bytes": table.encode_workspace_bytes(n),
        },
        "wall_s_timed_region": wall_s,
        "roofline": {
            "bound": "alu",
            "achieved": achieved,
            "peak": VALU_PEAK_TOPS,
            "unit": "TOP/s",
            "frac": achieved / VALU_PEAK_TOPS,
            "traffic": None,
            "algorithmic_ops_per_launch": ops,
            "kernel": f"tcq_encode_rows<{kv}>",
        },
    }
    if not args.no_cpu_baseline:
        import oracle  # CPU baseline leg only

        threads = max(1, min(16, os.cpu_count() or 1))
        cal = min(n, threads)
        t = time.perf_counter()
        oracle.encode_rows(e[:cal].astype(np.float64), d, kv, lut, mode=oracle.ENC_HEURISTIC, nthreads=threads)
        per_row = (time.perf_counter() - t) / cal
        sample = int(min(n, max(cal, args.cpu_seconds / max(per_row, 1e-9))))
        t = time.perf_counter()
        exp, _ = oracle.encode_rows(e[:sample].astype(np.float64), d, kv, lut, mode=oracle.ENC_HEURISTIC,
                                    nthreads=threads)
        cpu_s = time.perf_counter() - t
        got = table.download(0, sample)
        res["cpu_baseline"] = {
            "value": sample / cpu_s,
            "unit": "rows/s",
            "cores": threads,
            "kind": "oracle",
            "sample": f"first {sample:,} of the {n:,} rows ({cpu_s:.1f} s, {threads} threads, plain C oracle, "
                      "same two-pass search)",
            "gpu_records_matching_oracle": int((got == exp).all(axis=1).sum()),
        }
    table.close()
    print(json.dumps(res), flush=True)
    return 0


def bench_sharded(args, np, torch, cp, workload) -> int:
    """One GPU's share of a lookup into a table split by rows over G GPUs
    (--sharded G): this GPU holds the 12.7 GB d512 table as shard 0 of G x
    97,690,000 rows and runs, for the 393,216-lookup replay drawn over the
    whole sharded table, the three steps that are its own: the plan
    (cp_shard_plan), the owner's record gather (cp_table_gather_records) and
    the decode of the received records (cp_lookup_decode_staged). With the
    ids spread evenly over the shards, an owner serves as many lookups as a
    requester makes, so the gather here copies the records of all the
    replay's local ids from this GPU's table, standing in for the requests
    of all G requesters. The two exchanges between them are not timed (one
    GPU); their bytes are reported."""
    G = args.sharded
    cfg = workload.CONFIGS["gpu_d512"]
    lut = workload.lut_fp16(0)
    rps, d, kv, R = cfg.rows, cfg.d, cfg.kv, cfg.R
    t_gen = time.time()
    records = workload.random_records(rps, d, kv, cfg.table_seed)
    ids_np = workload.zipf_ids(G * rps, cfg.n_ids, cfg.ids_seed)
    gen_s = time.time() - t_gen
    table = cp.Table(rps, d, kv, lut)
    for r0 in range(0, rps, 1 << 22):
        table.upload(records[r0:r0 + (1 << 22)], first_row=r0)
    n = ids_np.size
    ids = torch.from_numpy(ids_np).cuda()
    local_ids = torch.empty(n, dtype=torch.int64, device="cuda")
    positions = torch.empty(n, dtype=torch.int64, device="cuda")
    counts = torch.empty(G, dtype=torch.int64, device="cuda")
    ws_bytes = cp.cp_shard_plan_workspace_bytes(n, G)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    recv = torch.zeros(n * R + 64, dtype=torch.uint8, device="cuda")
    out = torch.empty((n, d), dtype=torch.bfloat16, device="cuda")

    def plan():
        st = cp.cp_shard_plan(ids.data_ptr(), n, rps, G, local_ids.data_ptr(), positions.data_ptr(),
                              counts.data_ptr(), ws.data_ptr(), ws_bytes, torch.cuda.current_stream().cuda_stream)
        if st != cp.CP_OK:
            raise cp.CPError(st, "cp_shard_plan")

    def gather():
        st = cp.cp_table_gather_records(table.handle, local_ids.data_ptr(), n, recv.data_ptr(),
                                        torch.cuda.current_stream().cuda_stream)
        if st != cp.CP_OK:
            raise cp.CPError(st, "cp_table_gather_records")

    def decode():
        st = cp.cp_lookup_decode_staged(table.handle, recv.data_ptr(), n, positions.data_ptr(), n, out.data_ptr(),
                                        torch.cuda.current_stream().cuda_stream)
        if st != cp.CP_OK:
            raise cp.CPError(st, "cp_lookup_decode_staged")

    def step():
        plan()
        gather()
        decode()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    per_shard = counts.cpu().numpy()
    if int(per_shard.sum()) != n or not table.check():
        print("an id was owned by no shard", file=sys.stderr)
        return 1
    # the staged rows against the direct lookup of the same records on this
    # GPU's table (id - owner * rows_per_shard)
    direct = table.lookup_decode(torch.from_numpy(ids_np % rps).cuda())
    torch.cuda.synchronize()
    same_as_direct = torch.equal(direct.view(torch.int16), out.view(torch.int16))
    wall0 = time.perf_counter()
    total_ms = time_region(step, args.steps, torch)
    wall_s = time.perf_counter() - wall0
    ms = total_ms / args.steps
    stages = (("plan", plan), ("gather", gather), ("decode", decode))
    stage_eager_ms = {name: time_region(fn, args.steps, torch) / args.steps for name, fn in stages}
    # device time per call without the host's launch cost: 16 calls captured
    # in one graph, the graph replayed
    stage_ms = {name: graph_call_ms(fn, args.steps, torch) for name, fn in stages}
    step_graph_ms = graph_call_ms(step, args.steps, torch)
    torch.cuda.synchronize()
    same_as_direct = same_as_direct and torch.equal(direct.view(torch.int16), out.view(torch.int16))
    del direct
    # algorithmic bytes of each step: plan reads the ids twice (count, then
    # place) and writes local ids and positions; the gather reads local ids
    # and records and writes records; the decode reads positions and records
    # and writes the rows
    algo = {"plan": 8 * n * 2 + 16 * n, "gather": 8 * n + 2 * R * n, "decode": 8 * n + R * n + 2 * d * n}
    gbps = {k: algo[k] / (stage_ms[k] / 1e3) / 1e9 for k in algo}
    remote = n * (G - 1) / G
    res = {
        "metric": "decoded rows/s per GPU, row-sharded table (this GPU's plan, owner gather and staged decode)",
        "value": n / (ms / 1e3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": (f"sharded_d512_g{G}: {n:,} lookups (zipf ids) into a {G} x {rps:,}-row d512 table split "
                         f"by rows; this GPU holds one {cfg.table_bytes / 1e9:.2f} GB shard ({R}-byte records) "
                         "and runs the plan, the owner's record gather and the staged decode"),
            "shards": G, "rows_per_shard": rps, "d": d, "bits_per_step": kv, "record_bytes": R, "lookups": n,
            "ids_sha256_16": workload.ids_digest(ids_np),
            "entry_points": ["cp_shard_plan", "cp_table_gather_records", "cp_lookup_decode_staged"],
        },
        "stage_ms": stage_ms,
        "stage_ms_note": "device time per call: 16 calls captured in a HIP graph, the graph replayed",
        "stage_ms_eager": stage_eager_ms,
        "step_ms_graph": step_graph_ms,
        "stage_effective_GBps": gbps,
        "lookups_per_shard": [int(c) for c in per_shard],
        "rows_identical_to_direct_lookup": bool(same_as_direct),
        "rows_identical_note": "after the eager steps and again after the graph replays, every row equal to "
                               "cp_lookup_decode of id - owner * rows_per_shard on this GPU's table",
        "exchange_bytes_per_gpu_not_timed": {
            "ids_sent": int(8 * remote), "records_received": int(R * remote),
            "decoded_rows_instead": int(2 * d * remote),
            "note": "per step with the ids spread evenly over the shards: ids to their owners and records back "
                    "(an all-to-all each way); shipping decoded rows would move 2d bytes per lookup instead of R",
        },
        "wall_s_timed_region": wall_s,
        "setup_s": {"generate": round(gen_s, 2)},
        "roofline": {
            "bound": "hbm",
            "achieved": gbps["decode"],
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": gbps["decode"] / HBM_PEAK_GBPS,
            "traffic": None,
            "algorithmic_bytes_per_launch": algo["decode"],
            "kernel": f"gather_decode<{d},{kv}> (staged)",
            "step_effective_GBps": sum(algo.values()) / (ms / 1e3) / 1e9,
        },
    }
    counters = read_shard_counters(G)
    if counters:
        res["roofline"]["traffic"] = counters["gather_decode"]["bytes"]
        res["stage_hbm_traffic_bytes"] = {
            "plan": sum(counters[k]["bytes"] for k in ("shard_count", "shard_scan", "shard_scatter")),
            "gather": counters["gather_records"]["bytes"], "decode": counters["gather_decode"]["bytes"],
            "file": counters["file"]}
    if not args.no_probes:
        # the 1 GiB copy also calibrates the byte counters of a profiled run
        res["probes"] = probes(torch)
    if not same_as_direct:
        print("the staged rows differ from the direct lookup's", file=sys.stderr)
        return 1
    if not args.no_cpu_baseline:
        import oracle  # CPU check of a sample only

        k = min(n, 4096)
        exp, _ = oracle.lookup_decode(lut, records, rps, d, kv, ids_np[:k] % rps)
        got = out[:k].view(torch.int16).cpu().numpy().view(np.uint16)
        res["oracle_check"] = f"{int((got == exp).all(axis=1).sum())} of the first {k} lookups' rows equal the oracle's"
    table.close()
    print(json.dumps(res), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", default="gpu_d512",
                    help="workload: gpu_d512 (default), host_d512, mixed_d512, host_mixed_d512, small_d256, "
                         "rate_d512_kv{3,4,5,6}, tiny_d64")
    ap.add_argument("--ids", default=None, choices=["zipf", "uniform", "slice96"],
                    help="id stream (default: the config's own)")
    ap.add_argument("--noncoherent", action="store_true", help="host_d512: non-coherent pinned memory")
    ap.add_argument("--dedup", action="store_true",
                    help="use cp_lookup_decode_dedup (each distinct record fetched once)")
    ap.add_argument("--hot-share", type=float, default=0.0,
                    help="host_d512: keep device copies of this share of the rows, the most looked-up first")
    ap.add_argument("--flushed", action="store_true",
                    help="time launches with L2/MALL flushed before each (512 MiB read; and 512 MiB written); "
                         "on by default")
    ap.add_argument("--no-flushed", action="store_true", help="skip the flushed launches")
    ap.add_argument("--probes", action="store_true", help="run the 1 GiB copy and fill probes (on by default)")
    ap.add_argument("--no-probes", action="store_true", help="skip the copy and fill probes")
    ap.add_argument("--extra", action="store_true", help="kept for older command lines; probes and flushed "
                                                          "launches are on by default")
    ap.add_argument("--encode", action="store_true",
                    help="time cp_table_encode instead (trellis-coded quantisation of --encode-rows rows)")
    ap.add_argument("--encode-rows", type=int, default=4096)
    ap.add_argument("--encode-d", type=int, default=512)
    ap.add_argument("--encode-kv", type=int, default=4)
    ap.add_argument("--graph", action="store_true",
                    help="also time lookups replayed from a captured HIP graph (no host launch cost per lookup)")
    ap.add_argument("--batch-scan", action="store_true",
                    help="also time batches of 96 .. 1,572,864 ids (the replay tiled) and report the marginal rate")
    ap.add_argument("--sharded", type=int, default=0, metavar="G",
                    help="time this GPU's steps of a lookup into the d512 table split by rows over G GPUs "
                         "(plan, owner record gather, staged decode)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle sample")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the lookup is measured on one GPU's share of the table", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import trellis_coded_row_amd as cp
    import workload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    if args.encode:
        return bench_encode(args, np, torch, cp, workload)
    if args.sharded:
        if not 2 <= args.sharded <= cp.CP_MAX_SHARDS:
            print(f"--sharded takes 2 .. {cp.CP_MAX_SHARDS} shards", file=sys.stderr)
            return 2
        return bench_sharded(args, np, torch, cp, workload)
    cfg = workload.CONFIGS[args.config]
    ids_kind = args.ids or cfg.ids_kind
    lut = workload.lut_fp16(0)

    mixed = cfg.kv == 0
    t_gen = time.time()
    # every row a random code: the decode cost does not depend on how codes
    # were chosen (any bit string is a valid tail-biting code)
    if mixed:
        kvs = cfg.extra["kv_of_class"]
        classes = workload.rank_classes(cfg.rows, cfg.ids_seed, cfg.extra["shares"])
        offsets = workload.mixed_layout(cfg.d, kvs, classes)
        records = workload.random_mixed_records(cfg.d, kvs, classes, cfg.table_seed, offsets)
        class_bytes = np.array([workload.record_bytes(cfg.d, k) for k in kvs], dtype=np.int64)
    else:
        records = workload.random_records(cfg.rows, cfg.d, cfg.kv, cfg.table_seed)
    if ids_kind == cfg.ids_kind:
        ids_seed = cfg.ids_seed  # the workload's own id stream
        ids_np = cfg.ids()
    elif ids_kind == "uniform":
        ids_seed = cfg.uniform_seed or cfg.ids_seed + 100
        ids_np = workload.uniform_ids(cfg.rows, cfg.n_ids, ids_seed)
    elif ids_kind == "zipf":
        ids_seed = cfg.ids_seed
        ids_np = workload.zipf_ids(cfg.rows, cfg.n_ids, ids_seed)
    else:  # one token's decode step: the first 96 ids of the workload's stream
        ids_seed = cfg.ids_seed
        ids_np = cfg.ids()[:96]
    gen_s = time.time() - t_gen

    residency = cp.CP_RESIDENCY_HOST_MAPPED if cfg.host_resident else cp.CP_RESIDENCY_DEVICE
    flags = cp.CP_FLAG_HOST_NONCOHERENT if args.noncoherent else 0
    encoded = (not mixed) and cfg.encoded_rows > 0

    def fill(t) -> float | None:
        """Uploads the records; for tables whose rows hold TCQ-encoded Gaussian
        rows (the d64 and d256 tables all of them, the rate sweep rows
        0..4095), the library's own encoder (cp_table_encode, bit-exact with
        the oracle's: checked on a sample in the CPU-baseline leg) then writes
        those rows over the random codes. Returns the encoding seconds."""
        chunk = 1 << 22
        if mixed:
            for r0 in range(0, cfg.rows, chunk):
                r1 = min(cfg.rows, r0 + chunk)
                t.upload_bytes(records[int(offsets[r0]):int(offsets[r1])], r0, r1 - r0)
        else:
            for r0 in range(0, cfg.rows, chunk):
                t.upload(records[r0:r0 + chunk], first_row=r0)
        if not encoded:
            return None
        t_enc = time.time()
        enc_ids = cfg.encoded_row_ids()
        step = 1 << 16
        ws = torch.empty(t.encode_workspace_bytes(step), dtype=torch.uint8, device="cuda")
        for a in range(0, enc_ids.size, step):
            b = min(a + step, enc_ids.size)
            e = workload.table_rows(cfg.rows, cfg.d, cfg.rows_seed, enc_ids[a:b]).astype(np.float32)
            t.encode(torch.from_numpy(e).cuda(), first_row=int(enc_ids[a]), workspace=ws)
        torch.cuda.synchronize()
        return time.time() - t_enc

    t_up = time.time()
    if mixed:
        table = cp.MixedTable(cfg.d, kvs, classes, lut, residency=residency, flags=flags)
    else:
        table = cp.Table(cfg.rows, cfg.d, cfg.kv, lut, residency=residency, flags=flags)
    enc_s = fill(table)
    upload_s = time.time() - t_up - (enc_s or 0.0)
    hot_rows = 0
    hot_lookups = 0
    hot_set_np = None
    if args.hot_share > 0:
        # the rows of the smallest Zipf ranks of the id stream (its most frequent rows)
        k = int(args.hot_share * cfg.rows)
        hot_set_np = workload.keyed_permutation(np.arange(k, dtype=np.int64), cfg.rows, cfg.ids_seed)
        hot_rows = table.set_hot_rows(hot_set_np)
        hot_lookups = int(np.isin(ids_np, hot_set_np).sum())

    n = ids_np.shape[0]
    ids = torch.from_numpy(ids_np).cuda()
    out = torch.empty((n, cfg.d), dtype=torch.bfloat16, device="cuda")
    if args.dedup:
        workspace = torch.empty(table.dedup_workspace_bytes(n), dtype=torch.uint8, device="cuda")
        step = lambda: table.lookup_decode_dedup(ids, out, workspace=workspace)
    else:
        step = lambda: table.lookup_decode(ids, out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if not table.check():
        print("an id was out of range", file=sys.stderr)
        return 1

    # timed region: K steps back to back, bracketed by synchronisation; the
    # events sit on the stream the kernels are launched on
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    total_ms = time_region(step, args.steps, torch)
    wall_s = time.perf_counter() - wall0
    ms_per_step = total_ms / args.steps
    launch_ms = ms_per_step  # one kernel launch per step

    if mixed:
        # each lookup reads its row's own record and the 16-byte index entry
        # of its block of 32 rows
        rec_bytes = int(class_bytes[classes[ids_np]].sum())
        algo_bytes = rec_bytes + n * (16 + 2 * cfg.d)
        R = rec_bytes / n
        table_bytes = int(offsets[-1])
    else:
        R = cfg.R
        algo_bytes = n * (R + 2 * cfg.d)
        table_bytes = cfg.table_bytes
    rows_per_s = n * args.steps / (total_ms / 1e3)
    achieved = algo_bytes / (launch_ms / 1e3) / 1e9
    res = {
        "metric": METRIC,
        "value": rows_per_s,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": (f"{cfg.name}: {n:,} lookups ({ids_kind} ids) into a {cfg.rows:,} x d{cfg.d} CP table, "
                         + (f"rates {'/'.join(f'{k / 2:g}' for k in kvs)} bits/element by access rank "
                            f"({R:.1f} record bytes per lookup on average" if mixed else
                            f"{cfg.kv / 2:g} bits/element + bf16 scale ({R}-byte records")
                         + f", {table_bytes / 1e9:.2f} GB, {'pinned host memory' if cfg.host_resident else 'HBM'})"),
            "rows": cfg.rows, "d": cfg.d, "bits_per_step": list(kvs) if mixed else cfg.kv, "record_bytes": R,
            "lookups": n,
            "ids": ids_kind, "ids_sha256_16": workload.ids_digest(ids_np),
            "residency": "host" + ("-noncoherent" if args.noncoherent else "") if cfg.host_resident else "hbm",
            "hot_rows_in_hbm": hot_rows,
            "entry_point": "cp_lookup_decode_dedup" if args.dedup else "cp_lookup_decode",
            "seeds": {"codebook": 0, "table": cfg.table_seed, "ids": ids_seed},
        },
        "versions": {"hip": torch.version.hip, "torch": torch.__version__, "numpy": np.__version__,
                     "library": os.path.basename(cp.library_path())},
        "effective_GBps": algo_bytes * args.steps / (total_ms / 1e3) / 1e9,
        "pct_hbm_peak": 100.0 * algo_bytes * args.steps / (total_ms / 1e3) / 1e9 / HBM_PEAK_GBPS,
        "launch_ms_mean": launch_ms,
        "wall_s_timed_region": wall_s,
        "setup_s": {"generate": round(gen_s, 2), "upload": round(upload_s, 2),
                    "encode": round(enc_s, 2) if enc_s is not None else None},
    }
    if encoded:
        # reconstruction error of the encoded rows, from the lookup's own
        # output: rows 0..4095 against the Gaussian rows they encode
        mse_ids = np.arange(min(4096, cfg.encoded_rows), dtype=np.int64)
        y = table.lookup_decode(torch.from_numpy(mse_ids).cuda()).float().cpu().numpy().astype(np.float64)
        e = workload.table_rows(cfg.rows, cfg.d, cfg.rows_seed, mse_ids)
        err2 = ((y - e) ** 2).sum(axis=1)
        res["reconstruction"] = {
            "rows": f"ids 0..{mse_ids.size - 1} (TCQ-encoded Gaussian rows)",
            "mse_per_element": float(err2.sum() / e.size),
            "relative_mse": float(err2.sum() / (e ** 2).sum()),
            "mean_row_relative_error": float(np.mean(err2 / (e ** 2).sum(axis=1))),
            "context": f"per-element MSE of the normalised row at {cfg.kv / 2:g} bits per element: Gaussian "
                       f"rate-distortion bound {2.0 ** (-cfg.kv):.4f}",
            "encoded_rows": int(cfg.encoded_rows), "encoded_by": "cp_table_encode (GPU)",
        }
    counters = read_counter_summary(cfg.name, ids_kind, "mixed" if mixed else "single")
    kernel_name = f"gather_decode_mixed<{cfg.d}>" if mixed else f"gather_decode<{cfg.d},{cfg.kv}>"
    if cfg.host_resident:
        # The records cross PCIe, so PCIe bounds the launch, not HBM. The
        # bytes that must cross are each distinct record once (a repeat can
        # be served from the GPU's caches; rows with HBM copies never cross);
        # the denominator is a measured pinned host-to-device copy.
        probe = pcie_probe(torch)
        res["pcie_probe"] = probe
        uniq = np.unique(ids_np)
        if hot_rows:
            uniq = uniq[~np.isin(uniq, hot_set_np)]
            res["lookups_served_from_hbm_copies"] = hot_lookups
        if mixed:
            starts, sizes = offsets[uniq].astype(np.int64), class_bytes[classes[uniq]]
        else:
            starts, sizes = uniq * R, np.full(uniq.size, R, dtype=np.int64)
        pcie_bytes = int(sizes.sum())
        # granules of 64 bytes the distinct records touch: what the reads move
        # if every distinct record is fetched once
        first, last = starts // 64, (starts + sizes - 1) // 64
        res["pcie_distinct_records"] = int(uniq.size)
        res["pcie_distinct_64B_granule_bytes"] = int((last - first + 1).sum()) * 64
        res["pcie_per_lookup_record_GBps"] = (n - hot_lookups) * R / (launch_ms / 1e3) / 1e9
        pcie_achieved = pcie_bytes / (launch_ms / 1e3) / 1e9
        res["roofline"] = {
            "bound": "pcie",
            "achieved": pcie_achieved,
            "peak": probe["h2d_GBps"],
            "unit": "GB/s",
            "frac": pcie_achieved / probe["h2d_GBps"],
            "traffic": counters.get("pcie_bytes") if counters else None,
            "algorithmic_bytes_per_launch": pcie_bytes,
            "kernel": kernel_name,
            "hbm_effective_frac": achieved / HBM_PEAK_GBPS,
        }
    else:
        res["roofline"] = {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": counters["bytes"] if counters else None,
            "algorithmic_bytes_per_launch": algo_bytes,
            "kernel": kernel_name,
        }

    # per-launch distribution (each launch between its own pair of events)
    per = sorted(time_each(step, min(100, max(10, args.steps)), torch))
    q = lambda a, f: a[min(len(a) - 1, int(f * len(a)))]
    res["launch_ms_p10_p50_p90"] = [q(per, 0.1), q(per, 0.5), q(per, 0.9)]
    # 512 MiB > L2 + MALL. A read of it leaves the caches holding clean lines
    # of the flush buffer (cold records, nothing to write back); a write of it
    # leaves dirty lines, whose write-back then competes with the lookup's own
    # traffic (as after a layer that wrote its output).
    flush = torch.empty(512 << 18, dtype=torch.int32, device="cuda")
    flush.fill_(1)
    sink = torch.empty((), dtype=torch.int64, device="cuda")
    clean_flush = lambda: torch.sum(flush, 0, dtype=torch.int64, out=sink)
    if not args.no_flushed:
        reps = max(5, args.steps // 2)
        per = time_each(step, reps, torch, before=clean_flush)
        flushed_ms = sum(per) / len(per)
        per.sort()
        res["flushed_launch_ms_p10_p50_p90"] = [q(per, 0.1), q(per, 0.5), q(per, 0.9)]
        res["flushed_launch_ms_mean"] = flushed_ms
        res["flushed_rows_per_s"] = n / (flushed_ms / 1e3)
        res["flushed_pct_hbm_peak"] = 100.0 * algo_bytes / (flushed_ms / 1e3) / 1e9 / HBM_PEAK_GBPS
        per = time_each(step, reps, torch, before=lambda: flush.fill_(0))
        dirty_ms = sum(per) / len(per)
        res["flushed_dirty_launch_ms_mean"] = dirty_ms
        res["flushed_dirty_pct_hbm_peak"] = 100.0 * algo_bytes / (dirty_ms / 1e3) / 1e9 / HBM_PEAK_GBPS
        res["flush"] = "512 MiB read before each launch (clean eviction); dirty: 512 MiB written before each launch"
    if not args.no_flushed and not (mixed or cfg.host_resident or args.dedup or args.hot_share):
        # The same lookups on a second table created with CP_FLAG_TOUCH_AHEAD
        # (the first round of workgroups touches the later rounds' records):
        # the choice for lookups that start with none of the table cached.
        ta = cp.Table(cfg.rows, cfg.d, cfg.kv, lut, flags=cp.CP_FLAG_TOUCH_AHEAD)
        fill(ta)
        out_ta = torch.empty_like(out)
        step_ta = lambda: ta.lookup_decode(ids, out_ta)
        for _ in range(args.warmup):
            step_ta()
        ta_ms = time_region(step_ta, args.steps, torch) / args.steps
        reps = max(5, args.steps // 2)
        cold = time_each(step_ta, reps, torch, before=clean_flush)
        dirty = time_each(step_ta, reps, torch, before=lambda: flush.fill_(0))
        same = torch.equal(out_ta.view(torch.int16), out.view(torch.int16))
        res["touch_ahead"] = {
            "flag": "CP_FLAG_TOUCH_AHEAD",
            "launch_ms_mean": ta_ms,
            "pct_hbm_peak": 100.0 * algo_bytes / (ta_ms / 1e3) / 1e9 / HBM_PEAK_GBPS,
            "flushed_launch_ms_mean": sum(cold) / len(cold),
            "flushed_pct_hbm_peak": 100.0 * algo_bytes / (sum(cold) / len(cold) / 1e3) / 1e9 / HBM_PEAK_GBPS,
            "flushed_dirty_launch_ms_mean": sum(dirty) / len(dirty),
            "flushed_dirty_pct_hbm_peak": 100.0 * algo_bytes / (sum(dirty) / len(dirty) / 1e3) / 1e9
            / HBM_PEAK_GBPS,
            "rows_identical_to_default_table": bool(same),
        }
        ta.close()
        del out_ta
        torch.cuda.empty_cache()
        if not same:
            print("the touch-ahead table's rows differ from the default table's", file=sys.stderr)
            return 1
    if not args.no_probes:
        # what plain HBM streams reach on this GPU: the lookup is mostly a
        # write stream, so the fill is its closest measured ceiling; and the
        # lookup's own output stream and record fetch timed alone
        res["probes"] = probes(torch)
        res["probes"]["effective_over_fill"] = res["effective_GBps"] / res["probes"]["fill_GBps"]
        if not mixed:
            fl = floor_probes(torch, np, records, R, cfg.d, ids_np, cfg.host_resident, clean_flush)
            fl["lookup_over_store_only"] = launch_ms / fl["store_only_ms"]
            res["probes"].update(fl)
    del flush, sink
    torch.cuda.empty_cache()

    if args.graph:
        res["graph"] = graph_timing(step, out, args.steps, torch)
        if not res["graph"]["replays_matching_eager"].startswith("4/"):
            print("a graph replay differs from the eager lookup", file=sys.stderr)
            return 1
    if args.batch_scan:
        if mixed or args.dedup:
            print("--batch-scan times the single-rate cp_lookup_decode only", file=sys.stderr)
            return 2
        res["batch_scan"] = batch_scan(table, ids_np, cfg.d, algo_bytes / n, torch, np)
    if not args.no_cpu_baseline:
        import oracle  # CPU baseline leg only

        threads = max(1, min(16, os.cpu_count() or 1))
        if mixed:
            o_off = oracle.mixed_offsets(cfg.d, kvs, classes)
            decode = lambda sel, th=threads: oracle.lookup_decode_mixed(lut, records, cfg.d, kvs, classes, sel,
                                                                        offsets=o_off, nthreads=th)
        else:
            decode = lambda sel, th=threads: oracle.lookup_decode(lut, records, cfg.rows, cfg.d, cfg.kv, sel,
                                                                  nthreads=th)
        cal = min(n, 2048)
        t = time.perf_counter()
        decode(ids_np[:cal])
        per_row = (time.perf_counter() - t) / cal
        sample = int(min(n, max(cal, args.cpu_seconds / max(per_row, 1e-9))))
        # when the whole replay takes less than the target time, it is decoded
        # again (the same work each pass) until the target is reached, so the
        # rate rests on seconds of CPU work rather than a fraction of one
        t = time.perf_counter()
        exp, _ = decode(ids_np[:sample])
        passes = 1
        while sample == n and time.perf_counter() - t < args.cpu_seconds and passes < 1000:
            decode(ids_np)
            passes += 1
        cpu_s = time.perf_counter() - t
        got = out[:sample].view(torch.int16).cpu().numpy().view(np.uint16)
        # lookups of rows the GPU encoded are checked in encoder_check below
        plain = np.ones(sample, dtype=bool)
        if encoded:
            plain = ids_np[:sample] >= cfg.encoded_rows if cfg.encoded == "first" else np.zeros(sample, dtype=bool)
        res["cpu_baseline"] = {
            "value": sample * passes / cpu_s,
            "unit": "rows/s",
            "cores": threads,
            "kind": "oracle",
            "sample": (f"first {sample:,} of the {n:,} replay ids" + (f", decoded {passes} times" if passes > 1 else "")
                       + f" ({cpu_s:.1f} s, {threads} threads, plain C oracle, bit-by-bit trellis walk, fp64 scaling)"),
            "gpu_rows_matching_oracle": f"{int((got[plain] == exp[plain]).all(axis=1).sum())} of {int(plain.sum())}"
                                        + (" (rows with random codes; encoded rows: encoder_check)" if encoded else ""),
        }
        # the same oracle on one thread, over a bounded slice of the replay
        one = min(n, 32768)
        t = time.perf_counter()
        decode(ids_np[:one], 1)
        one_s = time.perf_counter() - t
        res["cpu_baseline"]["single_thread"] = {"value": one / one_s, "unit": "rows/s",
                                                "sample": f"first {one:,} replay ids ({one_s:.2f} s)"}
        res["cpu_baseline"]["host"] = {"cpus": os.cpu_count(), "model": host_cpu_model()}
        if encoded:
            # The GPU-encoded rows against the oracle's own encoding of the same
            # Gaussian rows, and their lookup against the oracle decoding its
            # own records (nothing the GPU produced goes into the oracle). The
            # check ids: when every row is encoded, the first 4,096 replay ids
            # (the hot rows) and 4,096 rows drawn uniformly over the table with
            # a fixed seed; else ids 0..4095. The replay sample above decodes
            # the random-code records, which time the same as encoded ones.
            if cfg.encoded == "all":
                spread = np.random.default_rng(cfg.rows_seed + 1).choice(cfg.rows, size=min(4096, cfg.rows),
                                                                          replace=False).astype(np.int64)
                chk_ids = np.concatenate([ids_np[:4096], spread])
            else:
                chk_ids = np.arange(min(4096, cfg.encoded_rows), dtype=np.int64)
            chk_rows = np.unique(chk_ids)
            t = time.perf_counter()
            own, _ = oracle.encode_rows(workload.table_rows(cfg.rows, cfg.d, cfg.rows_seed, chk_rows), cfg.d,
                                        cfg.kv, lut, mode=oracle.ENC_HEURISTIC, nthreads=threads)
            enc_cpu_s = time.perf_counter() - t
            lo, hi = int(chk_rows.min()), int(chk_rows.max()) + 1
            gpu_recs = table.download(lo, hi - lo)[chk_rows - lo]
            table_own = records.copy()
            table_own[chk_rows] = own
            exp_chk, _ = oracle.lookup_decode(lut, table_own, cfg.rows, cfg.d, cfg.kv, chk_ids, nthreads=threads)
            got_chk = table.lookup_decode(torch.from_numpy(chk_ids).cuda()).view(torch.int16).cpu().numpy()
            res["cpu_baseline"]["encoder_check"] = {
                "rows": int(chk_rows.size),
                "sample": ("the first 4,096 replay ids' rows and 4,096 rows drawn uniformly (seeded)"
                           if cfg.encoded == "all" else f"rows 0..{chk_ids.size - 1}"),
                "gpu_records_matching_oracle_encoding": int((gpu_recs == own).all(axis=1).sum()),
                "gpu_rows_matching_oracle_decode": int((got_chk.view(np.uint16) == exp_chk).all(axis=1).sum()),
                "lookups_checked": int(chk_ids.size),
                "oracle_encode_rows_per_s": chk_rows.size / enc_cpu_s,
            }
            del table_own
    table.close()
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
