// Internal interface between the C-ABI layer (cp_api.hip) and the kernels
// (cp_decode.hip). Not installed; not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpk {

// Hot-row cache of a host-resident table: one entry per 32 rows.
struct alignas(8) HotEntry {
    uint32_t base;  // cache slot of the block's first hot row
    uint32_t bits;  // bit j: row 32b + j has a copy in the cache
};

// Rows per wave chunk for a batch of n lookups on a device with num_cus
// compute units: the largest of 16, 4 and 1 rows that still gives the batch
// at least 8 waves per CU. A wave decodes its chunk's rows one after another
// behind one round of record loads, so long chunks suit batches that fill the
// chip (fewer id loads and codebook stagings per row), and short ones let a
// small batch (one decode step: tens to thousands of ids) spread over more
// waves and finish sooner.
inline int lookup_chunk_rows(uint64_t n, int num_cus)
{
    const uint64_t waves = (uint64_t)(num_cus > 0 ? num_cus : 256) * 8u;
    if (n >= 16u * waves) return 16;
    if (n >= 4u * waves) return 4;
    return 1;
}

// Launch parameters of one gather-decode call.
struct LaunchArgs {
    const uint8_t *records;   // device-accessible base of the packed records
    uint64_t rows;
    const uint32_t *lut;      // device copy of the 512-entry codebook (fp16 pairs)
    const int64_t *ids;       // row ids, or (by_offset) record byte offsets, -1 = invalid
    uint64_t n;
    bool by_offset;           // ids hold byte offsets of records (a staging area)
    bool touch_ahead = false; // the first round touches the later rounds' records
    uint32_t *out;            // n * d / 2 dwords (pairs of bf16 or fp16)
    int *err;                 // sticky out-of-range flag
    int num_cus;              // compute units of the device
    hipStream_t stream;
    // hot-row cache (hot_index null: none): records = the lower of the host
    // records' and the cache's addresses, each region at its offset from it
    const HotEntry *hot_index = nullptr;
    uint64_t host_off0 = 0, hot_off0 = 0;
};

// Byte offsets of the regions of a dedup workspace (see cp_dedup.hip).
struct DedupLayout {
    uint64_t slots;       // hash slots (power of two)
    uint64_t slot_bytes;  // bytes per staging slot (16-byte aligned record window)
    uint64_t keys, sidx, slot_of, uniq, staged_ids, count, staging, total;
};

struct DedupArgs {
    const uint8_t *records;  // device-accessible table records
    uint64_t rows, record_bytes;
    const int64_t *ids;
    uint64_t n;
    uint8_t *workspace;
    DedupLayout layout;
    int num_cus;
    hipStream_t stream;
};

// Workspace layout for n lookups: slots = next power of two >= 2n (load factor
// <= 1/2), then keys[slots] (8 B), sidx[slots], slot_of[n] (4 B), uniq[n],
// staged_off[n] (8 B), count (8 B), staging (n slots of slot_bytes + tail
// pad), each region 256-byte aligned. A staging slot holds a record's 16-byte
// aligned window: 16 * ceil((R + 15) / 16) bytes.
constexpr uint64_t dedup_align256(uint64_t x) { return (x + 255) & ~(uint64_t)255; }

constexpr uint32_t dedup_window_units(uint64_t record_bytes) { return (uint32_t)((record_bytes + 15 + 15) / 16); }

constexpr DedupLayout dedup_layout(uint64_t n, uint64_t record_bytes, uint64_t tail_pad)
{
    DedupLayout L{};
    uint64_t slots = 1;
    while (slots < 2 * n) slots <<= 1;
    L.slots = slots;
    L.slot_bytes = 16ull * dedup_window_units(record_bytes);
    uint64_t off = 0;
    L.keys = off;
    off = dedup_align256(off + 8 * slots);
    L.sidx = off;
    off = dedup_align256(off + 4 * slots);
    L.slot_of = off;
    off = dedup_align256(off + 4 * n);
    L.uniq = off;
    off = dedup_align256(off + 8 * n);
    L.staged_ids = off;
    off = dedup_align256(off + 8 * n);
    L.count = off;
    off = dedup_align256(off + 8);
    L.staging = off;
    off = dedup_align256(off + n * L.slot_bytes + tail_pad);
    L.total = off;
    return L;
}

// Dedups ids into the workspace and stages each distinct record once; after
// it, staged_ids[j] is the byte offset of lookup j's record in the staging
// area (or -1 for a bad id).
hipError_t dedup_prepare(const DedupArgs &a);
// The hash step alone (clear, insert): afterwards uniq[0 .. *count) are the
// distinct valid ids in a fixed order, sidx[slot] the index in uniq of the
// id in hash slot `slot`, and slot_of[j] lookup j's slot (0xFFFFFFFF for an
// id outside [0, rows)); pad[0 .. pad_bytes) is zeroed.
hipError_t dedup_hash(const DedupArgs &a, uint8_t *pad, uint64_t pad_bytes);

// Launch parameters of one encode call (see cp_encode.hip).
struct EncodeArgs {
    const float *rows;         // nrows * d fp32 values, row-major, device
    uint64_t nrows;
    uint32_t d, kv;
    const uint32_t *lut;       // device codebook (fp16 pairs)
    uint8_t *out;              // nrows packed records (device-accessible)
    uint64_t record_bytes;
    uint8_t *workspace;        // blocks * encode_workspace_per_block(d, kv) bytes
    uint32_t blocks;           // from encode_grid
    hipStream_t stream;
};

bool encode_supported(uint32_t d, uint32_t kv);
// Workgroups one encode launch uses for nrows rows (all resident at once).
hipError_t encode_grid(uint32_t kv, int num_cus, uint64_t nrows, uint32_t *blocks);
// Back-pointer bytes per workgroup: (d / 2) steps * 2^(16 - kv) memories.
uint64_t encode_workspace_per_block(uint32_t d, uint32_t kv);
hipError_t encode(const EncodeArgs &a);
// Mixed-rate tables: encodes input rows src_row[0..nrows) (of a.rows) at a.kv
// and writes record r at byte dst_off[r] of a.out, through staging buffers of
// nrows * d floats and nrows * record_bytes bytes (device, caller workspace).
hipError_t encode_listed(const EncodeArgs &a, const uint32_t *src_row, const uint64_t *dst_off, float *staged_rows,
                         uint8_t *staged_recs);

// Mixed-rate tables (see cp_mixed.hip): one index entry per 32 rows.
struct alignas(16) MixedEntry {
    uint64_t base;  // byte offset of the block's first record
    uint32_t p0;    // bit j: bit 0 of row (32b + j)'s rate class
    uint32_t p1;    // bit j: bit 1 of that class
};

struct MixedRates {
    uint32_t kv_packed;  // kv of class c in bits [8c, 8c + 8)
    uint32_t R[4];       // record bytes of class c (0 for unused classes)
};

struct MixedLaunchArgs {
    const uint8_t *records;  // device-accessible packed records
    uint64_t rows;
    const uint32_t *lut;
    const int64_t *ids;
    uint64_t n;
    uint32_t *out;
    int *err;
    const MixedEntry *index;  // device
    MixedRates rates;
    int num_cus;             // compute units of the device
    hipStream_t stream;
};

bool mixed_supported(uint32_t d);
hipError_t launch_mixed(uint32_t d, bool raw, const MixedLaunchArgs &a);
uint64_t mixed_index_entries(uint64_t rows);
// Builds the index on the host; -1 when a class is >= nclass.
int mixed_index_build(const uint8_t *row_class, uint64_t rows, uint32_t nclass, const uint32_t R[4],
                      MixedEntry *index, uint64_t *total_bytes);
// Byte offset (and class) of a row's record, from a host copy of the index.
uint64_t mixed_record_offset(const MixedEntry *index, const uint32_t R[4], uint64_t row, uint32_t *cls);

// Dedup lookups on a mixed-rate table (see cp_dedup_mixed.hip). Workspace:
// the hash regions of a single-rate dedup (keys, sidx, slot_of, uniq, count;
// staged_ids holds each lookup's staged row), then a mixed-rate index over
// the staged rows (16 bytes per 32), the record bytes per 32 staged rows and
// per tile of kMixedDedupTile such blocks, and the staging area: the distinct
// records packed in staged order (at most n of the largest record, plus the
// tail pad), each region 256-byte aligned.
constexpr uint32_t kMixedDedupTile = 8;  // blocks of 32 staged rows per tile (one 256-thread workgroup)

struct MixedDedupLayout {
    DedupLayout hash;  // staging and slot_bytes unused
    uint64_t blocks, tiles;
    uint64_t index, bsum, tsum, staging, total;
};

constexpr MixedDedupLayout mixed_dedup_layout(uint64_t n, uint64_t max_record_bytes, uint64_t tail_pad)
{
    MixedDedupLayout M{};
    M.hash = dedup_layout(n, 0, 0);
    M.blocks = (n + 31) / 32;
    M.tiles = (M.blocks + kMixedDedupTile - 1) / kMixedDedupTile;
    uint64_t off = M.hash.staging;  // the single-rate staging area is not used
    M.index = off;
    off = dedup_align256(off + 16 * M.blocks);
    M.bsum = off;
    off = dedup_align256(off + 8 * M.blocks);
    M.tsum = off;
    off = dedup_align256(off + 8 * M.tiles);
    M.staging = off;
    off = dedup_align256(off + n * max_record_bytes + tail_pad);
    M.total = off;
    return M;
}

struct MixedDedupArgs {
    DedupArgs hash;  // records (the table's), rows, ids, n, workspace, num_cus, stream; layout = M.hash
    MixedDedupLayout layout;
    const MixedEntry *index;  // the table's index (device)
    MixedRates rates;
    uint64_t tail_pad;
};

// Stages each distinct record of the batch once; afterwards the staging area
// holds a mixed-rate table of the staged rows, indexed by the workspace's
// own index, and staged_ids[j] is lookup j's staged row (-1 for a bad id),
// ready for the mixed-rate decode kernel.
hipError_t mixed_dedup_prepare(const MixedDedupArgs &a);

// Row-sharded tables (see cp_shard.hip): the requester's plan, a stable
// counting sort of its ids by owning shard (owner of row i =
// i / rows_per_shard, for i < shards * rows_per_shard).
constexpr uint32_t kMaxShards = 64;

struct ShardPlanArgs {
    const int64_t *ids;
    uint64_t n;
    uint64_t rows_per_shard;
    uint32_t shards;          // 1..kMaxShards
    int64_t *local_ids;       // n entries: ids within their shard, grouped by shard in batch order
    int64_t *positions;       // n entries: lookup j's place in local_ids, -1 when no shard owns it
    uint64_t *counts;         // shards entries
    uint8_t *workspace;       // shard_plan_workspace_bytes(n, shards), 256-byte aligned
    hipStream_t stream;
};

uint64_t shard_plan_workspace_bytes(uint64_t n, uint32_t shards);
hipError_t shard_plan(const ShardPlanArgs &a);
// counts[0..shards) = 0 (the plan of an empty batch)
hipError_t shard_plan_zero_counts(const ShardPlanArgs &a);
// Copies the records of rows ids[0..n) into dst, packed (record k at byte
// k * R); zeros and the error flag for an id outside [0, rows).
hipError_t gather_records_launch(const uint8_t *records, uint64_t rows, uint64_t R, const int64_t *ids, uint64_t n,
                                 uint8_t *dst, int *err, int num_cus, hipStream_t stream);

// True when a kernel for (d, kv) is compiled in.
bool supported(uint32_t d, uint32_t kv);

// Launches the gather-decode kernel; raw selects fp16 f(c) output instead of
// bf16 alpha * f(c). Returns the launch's hipError_t.
hipError_t launch(uint32_t d, uint32_t kv, bool raw, const LaunchArgs &a);

}  // namespace cpk
