// cp_shard.hip - the per-GPU steps of a lookup into a table sharded by rows.
//
// The pages run CP on 4 (and 8) GPUs of one node with 12.7 GB of the table on
// each ("2비트 코드와 공유 트렐리스로 n-gram 룩업 테이블을 4~8배 압축한다",
// onedev.kr, section "Assumptions and limits"). Records are independently
// addressable and only requested rows are decoded (same page, "How it
// differs"), so a lookup into a row-sharded table moves records, not rows:
//   1. the requester buckets its ids by owning shard (shard_plan: a stable
//      counting sort; owner of row i = i / rows_per_shard);
//   2. [ids go to their owners: an all-to-all]
//   3. each owner copies the requested records into one packed buffer
//      (gather_records);
//   4. [the records come back: a second all-to-all, 2 + kv d / 16 bytes per
//      lookup instead of 2 d for a decoded bf16 row]
//   5. the requester decodes the received records into its rows, in its
//      original lookup order (the gather-decode kernel run on the received
//      buffer, each lookup naming its record's position there).
// Steps 1, 3 and 5 run here; the exchanges need more than one GPU.
#include "cp_internal.h"
#include "cp_lane.h"

namespace cpk {

namespace {

constexpr int kPlanTile = 512;  // ids per workgroup in the plan kernels
constexpr int kPlanBlock = 256;  // threads per plan workgroup (4 waves)
constexpr uint32_t kInvalid = 0xFFFFFFFFu;

__device__ __forceinline__ uint32_t owner_of(int64_t id, uint64_t rows_per_shard, uint32_t shards)
{
    const uint64_t u = (uint64_t)id;
    if (id < 0 || u / rows_per_shard >= shards) return kInvalid;
    return (uint32_t)(u / rows_per_shard);
}

// Per tile: how many of its ids each shard owns, into tile_counts[tile][s].
__global__ __launch_bounds__(kPlanBlock) void shard_count(const int64_t *__restrict__ ids, uint64_t n,
                                                          uint64_t rows_per_shard, uint32_t shards,
                                                          uint32_t *__restrict__ tile_counts)
{
    __shared__ uint32_t cnt[kMaxShards];
    const uint64_t ntiles = (n + kPlanTile - 1) / kPlanTile;
    for (uint64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        for (uint32_t s = threadIdx.x; s < shards; s += kPlanBlock) cnt[s] = 0;
        constexpr int ROUNDS = kPlanTile / kPlanBlock;
        int64_t id[ROUNDS];
#pragma unroll
        for (int r = 0; r < ROUNDS; ++r) {
            const uint64_t j = tile * kPlanTile + r * kPlanBlock + threadIdx.x;
            id[r] = j < n ? ids[j] : -1;
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < ROUNDS; ++r) {
            const uint32_t s = owner_of(id[r], rows_per_shard, shards);
            if (s != kInvalid) atomicAdd(&cnt[s], 1u);
        }
        __syncthreads();
        for (uint32_t s = threadIdx.x; s < shards; s += kPlanBlock) tile_counts[tile * shards + s] = cnt[s];
        __syncthreads();
    }
}

// Inclusive prefix sum of v over the workgroup (kPlanBlock threads, in
// thread order); *total = the sum over all threads.
__device__ __forceinline__ uint64_t block_inclusive_sum(uint64_t v, uint64_t *wave_sum, uint64_t *total)
{
    constexpr int WAVES = kPlanBlock / 64;
    const uint32_t lane = threadIdx.x & 63u, w = threadIdx.x >> 6;
    uint64_t incl = v;
    for (int k = 1; k < 64; k <<= 1) {
        const uint64_t up = __shfl_up(incl, (unsigned)k, 64);
        if (lane >= (uint32_t)k) incl += up;
    }
    if (lane == 63) wave_sum[w] = incl;
    __syncthreads();
    uint64_t before = 0, all = 0;
    for (int q = 0; q < WAVES; ++q) {
        if (q < (int)w) before += wave_sum[q];
        all += wave_sum[q];
    }
    __syncthreads();
    *total = all;
    return before + incl;
}

// Within shard s, tile t's entries start after those of tiles 0..t-1:
// tile_start[tile][s] (relative to the shard's first entry); counts[s] the
// shard totals. One workgroup per shard scans its column of tile counts:
// each thread a run of up to kScanPer consecutive tiles (all its loads in
// flight together), or, for more tiles than that covers, 256 tiles at a time.
constexpr uint32_t kScanPer = 8;

__global__ __launch_bounds__(kPlanBlock) void shard_scan(const uint32_t *__restrict__ tile_counts, uint64_t ntiles,
                                                         uint32_t shards, uint64_t *__restrict__ tile_start,
                                                         uint64_t *__restrict__ counts)
{
    __shared__ uint64_t wave_sum[kPlanBlock / 64];
    const uint32_t s = blockIdx.x;
    uint64_t total = 0;
    if (ntiles <= (uint64_t)kPlanBlock * kScanPer) {
        const uint32_t per = (uint32_t)((ntiles + kPlanBlock - 1) / kPlanBlock);
        const uint64_t t0 = (uint64_t)threadIdx.x * per;
        uint32_t v[kScanPer];
        uint64_t mine = 0;
#pragma unroll
        for (uint32_t k = 0; k < kScanPer; ++k) {
            v[k] = (k < per && t0 + k < ntiles) ? tile_counts[(t0 + k) * shards + s] : 0u;
            mine += v[k];
        }
        uint64_t run = block_inclusive_sum(mine, wave_sum, &total) - mine;
#pragma unroll
        for (uint32_t k = 0; k < kScanPer; ++k) {
            if (k < per && t0 + k < ntiles) {
                tile_start[(t0 + k) * shards + s] = run;
                run += v[k];
            }
        }
    } else {
        for (uint64_t t0 = 0; t0 < ntiles; t0 += kPlanBlock) {
            const uint64_t t = t0 + threadIdx.x;
            const uint64_t v = t < ntiles ? tile_counts[t * shards + s] : 0;
            uint64_t all;
            const uint64_t incl = block_inclusive_sum(v, wave_sum, &all);
            if (t < ntiles) tile_start[t * shards + s] = total + incl - v;
            total += all;
        }
    }
    if (threadIdx.x == 0) counts[s] = total;
}

// Every id's place in its shard's list, in batch order (a stable sort): the
// shard's first entry (the counts of the shards before it), plus the tile's
// start within the shard, plus the id's rank within the tile. Wave w of the
// workgroup ranks quarter w of the tile, 64 ids per round: each lane among
// the wave's earlier lanes of the same shard (one ballot per distinct shard
// present), on top of the wave's running count for that shard; the quarters
// then follow one another. positions[j] = place of id j, -1 for an id owned
// by no shard; local_ids[place] = the id within its shard.
__global__ __launch_bounds__(kPlanBlock) void shard_scatter(const int64_t *__restrict__ ids, uint64_t n,
                                                            uint64_t rows_per_shard, uint32_t shards,
                                                            const uint64_t *__restrict__ tile_start,
                                                            const uint64_t *__restrict__ counts,
                                                            int64_t *__restrict__ local_ids,
                                                            int64_t *__restrict__ positions)
{
    constexpr int WAVES = kPlanBlock / 64;
    constexpr int ROUNDS = kPlanTile / kPlanBlock;     // 64-id rounds per wave
    __shared__ uint64_t base[kMaxShards];              // shard s's first entry: counts of shards 0..s-1
    __shared__ uint32_t wave_cnt[WAVES][kMaxShards];  // ids of shard s ranked by wave w so far
    const uint32_t lane = threadIdx.x & 63u, w = threadIdx.x >> 6;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const uint64_t ntiles = (n + kPlanTile - 1) / kPlanTile;
    if (threadIdx.x < shards) base[threadIdx.x] = counts[threadIdx.x];
    __syncthreads();
    uint64_t my_base = 0;
    for (uint32_t q = 0; q < threadIdx.x && q < shards; ++q) my_base += base[q];
    __syncthreads();
    if (threadIdx.x < shards) base[threadIdx.x] = my_base;
    for (uint64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        for (uint32_t i = threadIdx.x; i < WAVES * kMaxShards; i += kPlanBlock) (&wave_cnt[0][0])[i] = 0;
        // the wave's ids, all loaded before any is ranked
        const uint64_t j0 = tile * kPlanTile + (uint64_t)w * (64 * ROUNDS) + lane;
        int64_t id[ROUNDS];
        uint32_t sh[ROUNDS], rank[ROUNDS];
#pragma unroll
        for (int r = 0; r < ROUNDS; ++r) id[r] = j0 + 64u * r < n ? ids[j0 + 64u * r] : -1;
        __syncthreads();
#pragma unroll
        for (int r = 0; r < ROUNDS; ++r) {
            const uint32_t s = j0 + 64u * r < n ? owner_of(id[r], rows_per_shard, shards) : kInvalid;
            sh[r] = s;
            rank[r] = 0;
            uint64_t todo = __ballot(s != kInvalid);
            while (todo) {
                const uint32_t leader = (uint32_t)__builtin_ctzll(todo);
                const uint32_t sl = (uint32_t)__shfl((int)s, (int)leader, 64);
                const uint64_t m = __ballot(s == sl);
                const uint32_t prev = wave_cnt[w][sl];
                if (s == sl) rank[r] = prev + (uint32_t)__builtin_popcountll(m & below);
                if (lane == leader) wave_cnt[w][sl] = prev + (uint32_t)__builtin_popcountll(m);
                todo &= ~m;
            }
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < ROUNDS; ++r) {
            const uint64_t j = j0 + 64u * r;
            if (j < n) {
                const uint32_t s = sh[r];
                if (s == kInvalid) {
                    positions[j] = -1;
                } else {
                    uint64_t p = base[s] + tile_start[tile * shards + s] + rank[r];
                    for (uint32_t q = 0; q < w; ++q) p += wave_cnt[q][s];
                    positions[j] = (int64_t)p;
                    if (p < n) local_ids[p] = id[r] - (int64_t)((uint64_t)s * rows_per_shard);
                }
            }
        }
        __syncthreads();
    }
}

// dst record k = the table's record of row ids[k] (R bytes, 2-byte aligned
// both sides), or zeros for an id outside [0, rows) (which raises the flag).
// A wave copies groups of 16 records, the bytes [16 g R, 16 g R + 16 R) of
// dst, in two phases with the wave's LDS between them:
//   - loads: each 16-lane row loads one record per pass, four passes in
//     flight together; lane l loads the 16 bytes at 16 l from the record's
//     first aligned dword (lanes past the record's end load its last piece
//     again) and writes them unchanged to the record's 256-byte LDS slot, so
//     byte b of record j sits at slot j + b, plus 2 when the record starts
//     mid-dword (bit j of a per-group mask);
//   - stores: the range is written as aligned 16-byte chunks; chunk byte 2h
//     is byte t0 + 2h of the group's records, a half-word read from the slot
//     of the record it falls in (a chunk touches two records at most, three
//     when R < 16). Chunks that the range only partly covers (a destination
//     not 16-byte aligned, the batch's last group) write their half-words
//     inside it.
// The loads' pieces go to LDS as they came, so the per-byte work is one
// half-word read and a select per output half-word: the copy is bound by
// memory, not by instruction issue.
constexpr int kGatherPasses = 4;                      // records per row in flight together
constexpr uint32_t kGatherRecords = 4 * kGatherPasses;  // records per wave group
constexpr uint32_t kGatherMinR = 14;                  // the smallest record (d 64, 3 bits per step)
constexpr uint32_t kGatherMaxR = 194;                 // the largest record (d 512, 6 bits per step)
constexpr uint32_t kGatherSlot = 256;                 // LDS bytes per record (16 lanes x 16 bytes)
constexpr uint32_t kGatherPad = 16;                   // before slot 0: a range's first chunk may start 14 bytes early
// two spare slots: the last chunk's half-words past the group's records read there
constexpr uint32_t kGatherWaveLds = kGatherPad + (kGatherRecords + 2) * kGatherSlot;
static_assert(kGatherMaxR + 15 <= kGatherSlot, "a record's pieces fit its slot");
// four dwords at a 4-byte aligned address (one 16-byte access on the GPU),
// and at a 16-byte aligned one
typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// SPAN: records a 16-byte chunk can touch (2 for R >= 16, 3 below);
// BIGROWS: ids of 2^32 rows and more. Rmagic = ceil(2^32 / R): t / R is the
// high half of t Rmagic for every t below 2^32 / R.
template <int SPAN, bool BIGROWS>
__global__ __launch_bounds__(256) void gather_records(const uint8_t *__restrict__ tab, uint64_t rows, uint32_t R,
                                                      uint32_t Rmagic, const int64_t *__restrict__ ids, uint64_t n,
                                                      uint8_t *__restrict__ dst, int *__restrict__ err)
{
    __shared__ __attribute__((aligned(16))) uint8_t s_lds[4 * kGatherWaveLds];
    const uint32_t lane = threadIdx.x & 63u, row = lane >> 4, l = lane & 15u;
    const uint32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint64_t wave = (uint64_t)blockIdx.x * 4 + w;
    const uint64_t waves = (uint64_t)gridDim.x * 4;
    const uint64_t ngroups = (n + kGatherRecords - 1) / kGatherRecords;
    const uint32_t wbase = w * kGatherWaveLds + kGatherPad;  // slot 0's byte offset in s_lds
    // this lane's piece of record j (row j % 4, pass j / 4): + (j / 4) 4 slots
    uint8_t *const mypiece = s_lds + wbase + 16u * lane;
    bool bad = false;
    for (uint64_t g = wave; g < ngroups; g += waves) {
        const uint64_t k0 = g * kGatherRecords;
        const uint32_t cnt = (uint32_t)((n - k0) < kGatherRecords ? (n - k0) : kGatherRecords);
        const int64_t *gids = ids + k0;
        int64_t id[kGatherPasses];
#pragma unroll
        for (int p = 0; p < kGatherPasses; ++p) {
            const uint32_t j = 4u * p + row;
            id[p] = gids[j < cnt ? j : cnt - 1];
        }
        // lane j < 16 takes record j's id once more for the group's masks:
        // which records start mid-dword, which ids are outside the table
        const int64_t idj = gids[l < cnt ? l : cnt - 1];
        const bool okj = (uint64_t)idj < rows;
        const uint64_t offj = (okj ? (uint64_t)idj : 0) * R;
        const uint32_t shb = (uint32_t)__ballot(((uint32_t)offj & 2u) != 0) & 0xFFFFu;
        const uint32_t badg = (uint32_t)__ballot(!okj && l < cnt) & 0xFFFFu;
        bad |= badg != 0;
#pragma unroll
        for (int p = 0; p < kGatherPasses; ++p) {
            // an id outside the table reads record 0 (zeroed below)
            const bool ok = (uint64_t)id[p] < rows;
            uint64_t off;
            if constexpr (BIGROWS) off = (ok ? (uint64_t)id[p] : 0) * R;
            else off = (uint64_t)(ok ? (uint32_t)id[p] : 0u) * R;
            const uint32_t sh = (uint32_t)off & 2u;  // records are 2-byte aligned
            const uint32_t lastoff = (sh + R - 1) & ~15u;
            const uint32_t loff = 16u * l < lastoff ? 16u * l : lastoff;
            const u32x4a4 S = *reinterpret_cast<const u32x4a4 *>(tab + (off - sh) + loff);
            *reinterpret_cast<u32x4 *>(mypiece + 4u * p * kGatherSlot) = (u32x4)S;
        }
        // the wave's LDS writes before its reads (one wave: in order once issued)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // the range [start, end) of dst, from the 16-byte boundary below start
        const uint64_t start = (uint64_t)(uintptr_t)dst + k0 * R;
        const uint32_t o0 = (uint32_t)(start & 15u);  // even
        const uint32_t last = o0 + cnt * R;
        const uint32_t chunks = (last + 15) >> 4;
        uint8_t *const base = dst + k0 * R - o0;
        // LDS offsets of chunk byte 0 as read from records j0, j0 + 1 and
        // j0 + 2 (b0: the chunk's first byte in record j0; may be negative for
        // a range's first chunk), and the half-word read for chunk byte 2h
        auto chunk_bytes = [&](uint32_t j0, int32_t b0) -> u32x4 {
            uint32_t a0 = wbase + j0 * kGatherSlot + 2u * ((shb >> j0) & 1u) + (uint32_t)b0;
            uint32_t a1 = wbase + (j0 + 1) * kGatherSlot + 2u * ((shb >> (j0 + 1)) & 1u) + (uint32_t)b0 - R;
            uint32_t a2 = 0;
            if constexpr (SPAN == 3)
                a2 = wbase + (j0 + 2) * kGatherSlot + 2u * ((shb >> (j0 + 2)) & 1u) + (uint32_t)b0 - 2 * R;
            // kept apart, so that each half-word's address is one select
            asm volatile("" : "+v"(a0), "+v"(a1), "+v"(a2));
            const int32_t e1 = (int32_t)R - b0;  // chunk bytes below e1 are record j0's
            uint32_t hw[8];
#pragma unroll
            for (int h = 0; h < 8; ++h) {
                uint32_t a = 2 * h < e1 ? a0 : a1;
                if constexpr (SPAN == 3) a = 2 * h < e1 + (int32_t)R ? a : a2;
                hw[h] = *reinterpret_cast<const uint16_t *>(s_lds + a + 2 * h);
            }
            return u32x4{hw[0] | (hw[1] << 16), hw[2] | (hw[3] << 16), hw[4] | (hw[5] << 16), hw[6] | (hw[7] << 16)};
        };
        if (o0 == 0 && cnt == kGatherRecords) {
            // a whole group from a 16-byte boundary: R whole chunks
            for (uint32_t c = lane; c < chunks; c += 64) {
                const uint32_t t0 = 16u * c;
                const uint32_t j0 = (uint32_t)(((uint64_t)t0 * Rmagic) >> 32);
                *reinterpret_cast<u32x4 *>(base + t0) = chunk_bytes(j0, (int32_t)(t0 - j0 * R));
            }
        } else {
            for (uint32_t c = lane; c < chunks; c += 64) {
                const int32_t t0 = (int32_t)(16u * c) - (int32_t)o0;
                const uint32_t j0 = (uint32_t)(((uint64_t)(uint32_t)(t0 > 0 ? t0 : 0) * Rmagic) >> 32);
                const u32x4 v = chunk_bytes(j0, t0 - (int32_t)(j0 * R));
                const uint32_t c0 = 16u * c;
                if (c0 >= o0 && c0 + 16 <= last) {
                    *reinterpret_cast<u32x4 *>(base + c0) = v;
                } else {
                    // a chunk at an end of the range: its half-words inside it
#pragma unroll
                    for (int h = 0; h < 8; ++h) {
                        const uint32_t b = c0 + 2u * h;
                        const uint32_t word = h < 2 ? v.x : h < 4 ? v.y : h < 6 ? v.z : v.w;
                        if (b >= o0 && b < last)
                            *reinterpret_cast<uint16_t *>(base + b) = (uint16_t)(word >> (16 * (h & 1)));
                    }
                }
            }
        }
        if (__builtin_expect(badg != 0, 0)) {
            // records of ids outside the table are zeros: written once this
            // group's stores have completed (same addresses)
            __builtin_amdgcn_s_waitcnt(0);
            for (uint32_t j = 0; j < kGatherRecords; ++j)
                if ((badg >> j) & 1u)
                    for (uint32_t b = 2u * lane; b < R; b += 128)
                        *reinterpret_cast<uint16_t *>(dst + (k0 + j) * R + b) = 0;
        }
        // this group's LDS reads before the next group's writes
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    if (bad && lane == 0) atomicOr(err, 1);
}

}  // namespace

uint64_t shard_plan_workspace_bytes(uint64_t n, uint32_t shards)
{
    const uint64_t ntiles = (n + kPlanTile - 1) / kPlanTile;
    return dedup_align256(ntiles * shards * 4) + dedup_align256(ntiles * shards * 8);
}

hipError_t shard_plan(const ShardPlanArgs &a)
{
    if (a.n == 0) return hipSuccess;
    const uint64_t ntiles = (a.n + kPlanTile - 1) / kPlanTile;
    uint32_t *tile_counts = reinterpret_cast<uint32_t *>(a.workspace);
    uint64_t *tile_start = reinterpret_cast<uint64_t *>(a.workspace + dedup_align256(ntiles * a.shards * 4));
    const unsigned grid = (unsigned)(ntiles < 65536 ? ntiles : 65536);
    hipLaunchKernelGGL(shard_count, dim3(grid), dim3(kPlanBlock), 0, a.stream, a.ids, a.n, a.rows_per_shard, a.shards,
                       tile_counts);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(shard_scan, dim3(a.shards), dim3(kPlanBlock), 0, a.stream, tile_counts, ntiles, a.shards,
                       tile_start, a.counts);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(shard_scatter, dim3(grid), dim3(kPlanBlock), 0, a.stream, a.ids, a.n, a.rows_per_shard,
                       a.shards, tile_start, a.counts, a.local_ids, a.positions);
    return hipGetLastError();
}

__global__ void zero_counts(uint64_t *__restrict__ counts, uint32_t shards)
{
    if (threadIdx.x < shards) counts[threadIdx.x] = 0;
}

hipError_t shard_plan_zero_counts(const ShardPlanArgs &a)
{
    hipLaunchKernelGGL(zero_counts, dim3(1), dim3(kMaxShards), 0, a.stream, a.counts, a.shards);
    return hipGetLastError();
}

hipError_t gather_records_launch(const uint8_t *records, uint64_t rows, uint64_t R, const int64_t *ids, uint64_t n,
                                 uint8_t *dst, int *err, int num_cus, hipStream_t stream)
{
    if (n == 0) return hipSuccess;
    if (R < kGatherMinR || R > kGatherMaxR || (R & 1u)) return hipErrorInvalidValue;
    const uint32_t r = (uint32_t)R;
    const uint32_t magic = (uint32_t)(((1ull << 32) + r - 1) / r);
    // one wave per 16 records, at most 32 workgroups of 4 waves per CU (the
    // group loop strides over the rest)
    const uint64_t cap = (uint64_t)(num_cus > 0 ? num_cus : 256) * 32;
    const uint64_t blocks = ((n + kGatherRecords - 1) / kGatherRecords + 3) / 4;
    const dim3 grid((unsigned)(blocks < cap ? blocks : cap));
    typedef void (*gather_fn)(const uint8_t *, uint64_t, uint32_t, uint32_t, const int64_t *, uint64_t, uint8_t *,
                              int *);
    const bool big = rows > 0xFFFFFFFFull;
    const gather_fn fn = r >= 16 ? (big ? gather_records<2, true> : gather_records<2, false>)
                                 : (big ? gather_records<3, true> : gather_records<3, false>);
    hipLaunchKernelGGL(fn, grid, dim3(256), 0, stream, records, rows, r, magic, ids, n, dst, err);
    return hipGetLastError();
}

}  // namespace cpk
