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
// A wave copies 16 records, the bytes [16 g R, 16 g R + 16 R) of dst:
//   - each 16-lane row loads one record per pass, four passes with all
//     loads in flight together: lane l loads the record's aligned source
//     dwords 4l..4l+3 (one 16-byte load);
//   - the row writes the record into the wave's LDS area where it sits in
//     dst relative to a 16-byte boundary, dword by dword: when source and
//     destination start at different offsets within a dword, a dword takes
//     one half from the next or previous source dword, which may be the
//     neighbouring lane's (a row shift), and a dword shared with the next
//     record gets its own half only (16-bit LDS writes);
//   - the wave then stores its range from LDS as aligned 16-byte chunks,
//     half-words only at the range's two ends (shared with the
//     neighbouring waves' ranges).
constexpr int kGatherPasses = 4;  // records per row in flight together
constexpr uint32_t kGatherRecords = 4 * kGatherPasses;  // records per wave
constexpr uint32_t kGatherMaxR = 194;                 // the largest record (d 512, 6 bits per step)
constexpr uint32_t kGatherStage = (kGatherRecords * kGatherMaxR + 16 + 15) & ~15u;  // staged bytes per wave
constexpr uint32_t kGatherLds = kGatherStage + 256;  // and a spare dword per lane
// four dwords at a 4-byte aligned address (one 16-byte access on the GPU),
// and at a 16-byte aligned one
typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void gather_records(const uint8_t *__restrict__ tab, uint64_t rows, uint32_t R,
                                                      const int64_t *__restrict__ ids, uint64_t n,
                                                      uint8_t *__restrict__ dst, int *__restrict__ err)
{
    __shared__ __attribute__((aligned(16))) uint8_t s_stage[4][kGatherLds];
    const uint32_t lane = threadIdx.x & 63u, row = lane >> 4, l = lane & 15u;
    const uint32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint64_t wave = (uint64_t)blockIdx.x * 4 + w;
    const uint64_t waves = (uint64_t)gridDim.x * 4;
    const uint64_t ngroups = (n + kGatherRecords - 1) / kGatherRecords;
    uint8_t *stage = s_stage[w];
    bool bad = false;
    for (uint64_t g = wave; g < ngroups; g += waves) {
        const uint64_t k0 = g * kGatherRecords;
        const uint32_t cnt = (uint32_t)((n - k0) < kGatherRecords ? (n - k0) : kGatherRecords);
        int64_t id[kGatherPasses];
#pragma unroll
        for (int p = 0; p < kGatherPasses; ++p) {
            const uint32_t j = 4u * p + row;
            id[p] = j < cnt ? ids[k0 + j] : 0;
        }
        u32x4a4 S[kGatherPasses];
        uint32_t sh[kGatherPasses];
#pragma unroll
        for (int p = 0; p < kGatherPasses; ++p) {
            const uint32_t j = 4u * p + row;
            const bool ok = (uint64_t)id[p] < rows;
            bad |= j < cnt && !ok;
            const uint8_t *rec = tab + (ok ? (uint64_t)id[p] : 0) * R;
            sh[p] = (uint32_t)((uintptr_t)rec & 3u);
            const uint32_t nsrc = (sh[p] + R + 3) >> 2;  // aligned source dwords holding the record
            // lanes past the record load the record's first 16 bytes again
            const u32x4a4 *src = reinterpret_cast<const u32x4a4 *>(rec - sh[p]) + (4 * l < nsrc ? l : 0);
            S[p] = *src;
            if (!ok || j >= cnt) S[p] = u32x4a4{0, 0, 0, 0};
        }
        // the range [start, end) of dst, staged from the 16-byte boundary below start
        const uint64_t start = (uint64_t)(uintptr_t)dst + k0 * R;
        const uint32_t o0 = (uint32_t)(start & 15u);  // even
#pragma unroll
        for (int p = 0; p < kGatherPasses; ++p) {
            const uint32_t j = 4u * p + row;
            const uint32_t at = o0 + j * R;  // the record's first byte in the stage
            const uint32_t dsh = at & 3u;
            // the source dwords before and after this lane's four
            const uint32_t before =
                (uint32_t)__builtin_amdgcn_update_dpp((int)S[p].w, (int)S[p].w, 0x111 /* row_shr:1 */, 0xF, 0xF, false);
            const uint32_t after =
                (uint32_t)__builtin_amdgcn_update_dpp((int)S[p].x, (int)S[p].x, 0x101 /* row_shl:1 */, 0xF, 0xF, false);
            const uint32_t src6[6] = {before, S[p].x, S[p].y, S[p].z, S[p].w, after};
            // the lane's eight stage half-words, written without branches: a
            // half-word outside the record (or of a record past the batch)
            // goes to the lane's spare dword after the stage instead
            const int r0 = 16 * (int)l - (int)dsh;  // record byte at this lane's first stage byte
            const uint32_t q = (at - dsh) + 16u * l;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                // stage dword 4l+m starts at source byte 4(4l+m) + sh - dsh
                const uint32_t D = sh[p] == dsh ? src6[m + 1]
                                   : sh[p] > dsh ? (src6[m + 1] >> 16) | (src6[m + 2] << 16)
                                                 : (src6[m] >> 16) | (src6[m + 1] << 16);
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int r = r0 + 4 * m + 2 * e;
                    const bool in = j < cnt && r >= 0 && r < (int)R;
                    *reinterpret_cast<uint16_t *>(stage + (in ? q + 4u * m + 2u * e : kGatherStage + 4u * lane)) =
                        (uint16_t)(D >> (16 * e));
                }
            }
        }
        // the wave's LDS writes before its reads (one wave: in order once issued)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const uint32_t last = o0 + cnt * R;  // stage offset of end
        const uint32_t chunks = (last + 15) >> 4;
        uint8_t *base = dst + k0 * R - o0;
        for (uint32_t c = lane; c < chunks; c += 64) {
            const u32x4 v = *reinterpret_cast<const u32x4 *>(stage + 16u * c);
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
        // this group's LDS reads before the next group's writes
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    if (bad) atomicOr(err, 1);
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
    if (R > kGatherMaxR || (R & 1u)) return hipErrorInvalidValue;
    // one wave per 16 records, at most 32 workgroups of 4 waves per CU (the
    // group loop strides over the rest)
    const uint64_t cap = (uint64_t)(num_cus > 0 ? num_cus : 256) * 32;
    const uint64_t blocks = ((n + kGatherRecords - 1) / kGatherRecords + 3) / 4;
    hipLaunchKernelGGL(gather_records, dim3((unsigned)(blocks < cap ? blocks : cap)), dim3(256), 0, stream, records,
                       rows, (uint32_t)R, ids, n, dst, err);
    return hipGetLastError();
}

}  // namespace cpk
