"""Seeded synthetic inputs for Conditional Program (CP) lookup tables.

This module only draws random numbers and lays bytes out in the record
format; it holds none of the method's arithmetic (no trellis, no hash, no
decoding, no scaling). The CPU oracle and the HIP library both take what it
produces as plain inputs.

Record format (the pages describe each row as an independently addressable
record holding a code and one 16-bit scale; the byte layout is this
library's choice): N/8 code bytes, then the scale as bf16 little endian,
packed with no padding, N = kv * d / 2 code bits.

Workloads stand in for the pages' lookup replay (a 4,096-token sequence, 48
rows per token, 2 memory layers) whose text, tokenizer and trained tables are
not available: ids are drawn Zipf(1.1) over a seeded permutation of the rows,
table rows are N(0,1) directions times a lognormal(0, 0.5) norm, and the
shared codebook is 512 x 2 N(0,1) values stored as fp16.
"""
from __future__ import annotations

import hashlib
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

LUT_SEED = 0
TOKENS, ROWS_PER_TOKEN, LAYERS = 4096, 48, 2
REPLAY_IDS = TOKENS * ROWS_PER_TOKEN * LAYERS  # 393,216
ZIPF_S = 1.1
CHUNK_ROWS = 1 << 20


def record_bytes(d: int, kv: int) -> int:
    """Bytes of one packed record: kv*d/2 code bits, then a 2-byte scale."""
    return kv * d // 16 + 2


def lut_fp16(seed: int = LUT_SEED) -> np.ndarray:
    """512 x 2 codebook entries drawn N(0,1), stored as fp16 bit patterns."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((512, 2)).astype(np.float16).view(np.uint16).copy()


def gaussian_rows(n: int, d: int, seed: int) -> np.ndarray:
    """n rows e = rho * g / ||g||, g ~ N(0, I_d), rho ~ LogNormal(0, 0.5)."""
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((n, d))
    rho = rng.lognormal(0.0, 0.5, size=n)
    return g / np.linalg.norm(g, axis=1, keepdims=True) * rho[:, None]


ROW_CHUNK = 1 << 16


def table_rows(rows: int, d: int, seed: int, row_ids: np.ndarray, threads: int | None = None) -> np.ndarray:
    """The Gaussian rows (as gaussian_rows) of a table's rows `row_ids`, each
    row fixed by (seed, row id) alone: chunk c of ROW_CHUNK rows is drawn from
    default_rng([seed, c]), so any subset of the rows can be produced without
    the others. float64[len(row_ids), d], in the order given."""
    row_ids = np.asarray(row_ids, dtype=np.int64)
    out = np.empty((row_ids.size, d), dtype=np.float64)
    chunk_of = row_ids // ROW_CHUNK

    def fill(c: int) -> None:
        sel = np.nonzero(chunk_of == c)[0]
        n = min(ROW_CHUNK, rows - c * ROW_CHUNK)
        rng = np.random.default_rng([seed, int(c)])
        g = rng.standard_normal((n, d))
        rho = rng.lognormal(0.0, 0.5, size=n)
        local = row_ids[sel] - c * ROW_CHUNK
        gs = g[local]
        out[sel] = gs / np.linalg.norm(gs, axis=1, keepdims=True) * rho[local][:, None]

    chunks = np.unique(chunk_of)
    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(fill, [int(c) for c in chunks]))
    return out


def hottest_rows(rows: int, k: int, ids_seed: int) -> np.ndarray:
    """The rows of the k smallest Zipf ranks of the id stream of `ids_seed`
    (zipf_ids sends rank r to row keyed_permutation(r)): its most looked-up
    rows, hottest first."""
    return keyed_permutation(np.arange(min(k, rows), dtype=np.int64), rows, ids_seed)


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """Nearest bf16 (ties to even) of each value's float32, as uint16."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def random_record_chunk(d: int, kv: int, seed: int, chunk: int, nrows: int) -> np.ndarray:
    """Rows of chunk `chunk` (CHUNK_ROWS rows each) of a random-code table:
    uniform code bytes (every bit string is a valid tail-biting code) and a
    scale drawn LogNormal(0, 0.5) stored as bf16. Each chunk has its own
    stream, so any chunk can be regenerated alone."""
    nb = kv * d // 16
    rng = np.random.default_rng([seed, chunk])
    out = np.empty((nrows, nb + 2), dtype=np.uint8)
    words = rng.integers(0, 2**64 - 1, size=(nrows * nb + 7) // 8, dtype=np.uint64,
                         endpoint=True)
    out[:, :nb] = words.view(np.uint8)[: nrows * nb].reshape(nrows, nb)
    a = _bf16_bits(rng.lognormal(0.0, 0.5, size=nrows))
    out[:, nb] = (a & 0xFF).astype(np.uint8)
    out[:, nb + 1] = (a >> 8).astype(np.uint8)
    return out


def random_records(rows: int, d: int, kv: int, seed: int, first: int = 0,
                   count: int | None = None, out: np.ndarray | None = None,
                   threads: int | None = None) -> np.ndarray:
    """Rows [first, first+count) of a random-code table, chunk-deterministic
    (the bytes do not depend on first/count or on the thread count)."""
    if count is None:
        count = rows - first
    R = record_bytes(d, kv)
    if out is None:
        out = np.empty((count, R), dtype=np.uint8)
    assert out.shape == (count, R) and out.dtype == np.uint8
    if count == 0:
        return out
    c_lo, c_hi = first // CHUNK_ROWS, (first + count - 1) // CHUNK_ROWS

    def fill(c: int) -> None:
        c0 = c * CHUNK_ROWS
        blk = random_record_chunk(d, kv, seed, c, min(CHUNK_ROWS, rows - c0))
        lo, hi = max(first, c0), min(first + count, c0 + blk.shape[0])
        out[lo - first:hi - first] = blk[lo - c0:hi - c0]

    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    if c_hi == c_lo or threads <= 1:
        for c in range(c_lo, c_hi + 1):
            fill(c)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(c_lo, c_hi + 1)))
    return out


_M64 = np.uint64(0xFFFFFFFFFFFFFFFF)


def _mix64(x: np.ndarray) -> np.ndarray:
    """A 64-bit finaliser (multiply / xor-shift) used as a Feistel round
    function; any fixed keyed mixing would do."""
    x = x ^ (x >> np.uint64(30))
    x = x * np.uint64(0xBF58476D1CE4E5B9)
    x = x ^ (x >> np.uint64(27))
    x = x * np.uint64(0x94D049BB133111EB)
    return x ^ (x >> np.uint64(31))


def keyed_permutation(x: np.ndarray, rows: int, seed: int) -> np.ndarray:
    """A seeded pseudo-random bijection of [0, rows), evaluated at x only: a
    4-round balanced Feistel network on 2h bits (2^2h >= rows), cycle-walked
    until the value falls inside [0, rows)."""
    h = max(1, (int(rows - 1).bit_length() + 1) // 2)
    mask = np.uint64((1 << h) - 1)
    keys = np.random.default_rng([seed, 0x5EED]).integers(0, 2**63, size=4, dtype=np.uint64)
    v = np.asarray(x, dtype=np.uint64).copy()
    todo = np.ones(v.shape, dtype=bool)
    with np.errstate(over="ignore"):
        while todo.any():
            w = v[todo]
            left, right = w >> np.uint64(h), w & mask
            for k in keys:
                left, right = right, left ^ (_mix64(right ^ k) & mask)
            w = (left << np.uint64(h)) | right
            v[todo] = w
            todo[todo] = w >= np.uint64(rows)
    return v.astype(np.int64)


def zipf_ids(rows: int, n: int, seed: int, s: float = ZIPF_S) -> np.ndarray:
    """n ids: rank r ~ Zipf(s) truncated to [1, rows] by rejection, id =
    perm(r - 1) for a seeded pseudo-random permutation perm of the rows."""
    rng = np.random.default_rng(seed)
    ranks = np.empty(0, dtype=np.int64)
    while ranks.size < n:
        draw = rng.zipf(s, size=n)
        ranks = np.concatenate([ranks, draw[draw <= rows]])
    return keyed_permutation(ranks[:n] - 1, rows, seed)


def uniform_ids(rows: int, n: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.integers(0, rows, size=n, dtype=np.int64)


# Mixed-rate tables: rate classes by access rank (class 0 = most looked-up
# rows). With these shares the mean rate is 3.75 bits per step (1.875 bits
# per element), inside the 2-bit budget of the single-rate table.
MIXED_KV = (6, 5, 4, 3)
MIXED_SHARES = (0.05, 0.15, 0.30, 0.50)


def rank_classes(rows: int, seed: int, shares=MIXED_SHARES, threads: int | None = None) -> np.ndarray:
    """uint8[rows]: each row's rate class from its access rank under the Zipf
    id stream of `seed` (zipf_ids sends rank r to row keyed_permutation(r)):
    the first shares[0] of the ranks get class 0, the next shares[1] class 1,
    and so on. A stand-in for access counts taken from a text corpus."""
    bounds = np.floor(np.cumsum(np.asarray(shares, dtype=np.float64)) * rows).astype(np.int64)
    bounds[-1] = rows
    cls = np.empty(rows, dtype=np.uint8)
    step = 1 << 22

    def fill(a: int) -> None:
        r = np.arange(a, min(a + step, rows), dtype=np.int64)
        cls[keyed_permutation(r, rows, seed)] = np.searchsorted(bounds, r, side="right").astype(np.uint8)

    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(fill, range(0, rows, step)))
    return cls


def mixed_layout(d: int, kv_of_class, row_class: np.ndarray) -> np.ndarray:
    """uint64[rows + 1]: byte offset of each row's record when the records
    are packed in row order at their classes' sizes (last entry: total)."""
    sizes = np.array([record_bytes(d, k) for k in kv_of_class], dtype=np.uint64)
    off = np.zeros(row_class.shape[0] + 1, dtype=np.uint64)
    np.cumsum(sizes[row_class], out=off[1:])
    return off


def random_mixed_records(d: int, kv_of_class, row_class: np.ndarray, seed: int,
                         offsets: np.ndarray | None = None, threads: int | None = None) -> np.ndarray:
    """uint8[total]: the packed records of a random-code mixed-rate table.
    Every row gets uniform code bytes and a LogNormal(0, 0.5) bf16 scale;
    chunk c (CHUNK_ROWS rows) draws from its own stream."""
    if offsets is None:
        offsets = mixed_layout(d, kv_of_class, row_class)
    rows = row_class.shape[0]
    nb = np.array([k * d // 16 for k in kv_of_class], dtype=np.int64)
    out = np.empty(int(offsets[-1]), dtype=np.uint8)

    def fill(c: int) -> None:
        r0, r1 = c * CHUNK_ROWS, min(rows, (c + 1) * CHUNK_ROWS)
        a, b = int(offsets[r0]), int(offsets[r1])
        rng = np.random.default_rng([seed, 0x3A7E, c])
        words = rng.integers(0, 2**64 - 1, size=(b - a + 7) // 8, dtype=np.uint64, endpoint=True)
        out[a:b] = words.view(np.uint8)[: b - a]
        alpha = _bf16_bits(rng.lognormal(0.0, 0.5, size=r1 - r0))
        pos = offsets[r0:r1].astype(np.int64) + nb[row_class[r0:r1]]
        out[pos] = (alpha & 0xFF).astype(np.uint8)
        out[pos + 1] = (alpha >> 8).astype(np.uint8)

    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(fill, range((rows + CHUNK_ROWS - 1) // CHUNK_ROWS)))
    return out


def ids_digest(ids: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(ids, dtype=np.int64).tobytes()).hexdigest()[:16]


@dataclass(frozen=True)
class TableConfig:
    """One workload: a table shape, how its records are made, and its ids."""
    name: str
    rows: int
    d: int
    kv: int
    table_seed: int
    ids_kind: str              # "uniform" or "zipf"
    n_ids: int
    ids_seed: int
    encoded_rows: int          # how many rows hold TCQ-encoded Gaussian rows (see encoded_row_ids)
    encoded: str = "first"     # which: "first" (rows 0..encoded_rows-1) or "all"
    host_resident: bool = False
    uniform_seed: int | None = None
    description: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def R(self) -> int:
        return record_bytes(self.d, self.kv)

    @property
    def table_bytes(self) -> int:
        return self.rows * self.R

    def ids(self) -> np.ndarray:
        if self.ids_kind == "uniform":
            return uniform_ids(self.rows, self.n_ids, self.ids_seed)
        return zipf_ids(self.rows, self.n_ids, self.ids_seed)

    def uniform_variant_ids(self) -> np.ndarray:
        assert self.uniform_seed is not None
        return uniform_ids(self.rows, self.n_ids, self.uniform_seed)

    @property
    def rows_seed(self) -> int:
        """Seed of the table's Gaussian rows (table_rows)."""
        return self.table_seed + 1000

    def encoded_row_ids(self, limit: int | None = None) -> np.ndarray:
        """The rows that hold encoded Gaussian rows (the others hold random
        codes). With `limit` below that count (a test that encodes on the
        CPU), the `limit` most looked-up rows of the config's id stream
        among them instead: where most lookups go."""
        if self.encoded == "all":
            if limit is None or limit >= self.rows:
                return np.arange(self.rows, dtype=np.int64)
            return hottest_rows(self.rows, limit, self.ids_seed)
        k = self.encoded_rows if limit is None else min(limit, self.encoded_rows)
        return np.arange(k, dtype=np.int64)


CONFIGS = {
    "tiny_d64": TableConfig(
        "tiny_d64", 4096, 64, 4, 100, "uniform", 1024, 300, encoded_rows=4096,
        description="4,096 x d64 table, every row TCQ-encoded; 1,024 uniform ids"),
    "small_d256": TableConfig(
        "small_d256", 1 << 20, 256, 4, 101, "zipf", REPLAY_IDS, 201, encoded_rows=1 << 20, encoded="all",
        description="1,048,576 x d256 table (66-byte records), every row TCQ-encoded; 393,216-id Zipf(1.1) "
                    "replay"),
    "gpu_d512": TableConfig(
        "gpu_d512", 97_690_000, 512, 4, 102, "zipf", REPLAY_IDS, 202, encoded_rows=0,
        uniform_seed=302,
        description="97,690,000 x d512 table (130-byte records, 12.70 GB in HBM); "
                    "393,216-id Zipf(1.1) replay"),
    "host_d512": TableConfig(
        "host_d512", 97_690_000, 512, 4, 102, "zipf", REPLAY_IDS, 202, encoded_rows=0,
        host_resident=True,
        description="the 12.70 GB d512 table in pinned host memory, read over PCIe"),
}
CONFIGS["mixed_d512"] = TableConfig(
    "mixed_d512", 97_690_000, 512, 0, 104, "zipf", REPLAY_IDS, 202, encoded_rows=0,
    description="97,690,000 x d512 mixed-rate table: rows coded at 3 / 2.5 / 2 / 1.5 bits per element "
                "by Zipf access rank (5% / 15% / 30% / 50% of rows), ~11.5 GB in HBM; the Zipf(1.1) replay",
    extra={"kv_of_class": MIXED_KV, "shares": MIXED_SHARES})
CONFIGS["host_mixed_d512"] = TableConfig(
    "host_mixed_d512", 97_690_000, 512, 0, 104, "zipf", REPLAY_IDS, 202, encoded_rows=0, host_resident=True,
    description="the mixed-rate d512 table (mixed_d512) in pinned host memory, read over PCIe",
    extra={"kv_of_class": MIXED_KV, "shares": MIXED_SHARES})
for _kv in (3, 4, 5, 6):
    CONFIGS[f"rate_d512_kv{_kv}"] = TableConfig(
        f"rate_d512_kv{_kv}", 1 << 22, 512, _kv, 103, "zipf", REPLAY_IDS, 203,
        encoded_rows=4096,
        description=f"4,194,304 x d512 table at {_kv} bits per step "
                    f"({_kv / 2:g} bits per element), rows 0..4095 TCQ-encoded")


def build_records(cfg: TableConfig, encode_fn=None, encode_limit: int | None = None) -> np.ndarray:
    """All records of a config's table: random codes, with the rows
    cfg.encoded_row_ids(encode_limit) replaced by encode_fn(e[n, d]) ->
    uint8[n, R] of their Gaussian rows (the caller passes the encoder, e.g.
    the oracle's). With encode_fn None, every row is a random code."""
    out = random_records(cfg.rows, cfg.d, cfg.kv, cfg.table_seed)
    if encode_fn is not None and cfg.encoded_rows:
        sel = cfg.encoded_row_ids(encode_limit)
        out[sel] = encode_fn(table_rows(cfg.rows, cfg.d, cfg.rows_seed, sel))
    return out
