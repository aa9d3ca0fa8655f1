// cp_dedup_mixed.hip - fetch each distinct record of a lookup batch once, for
// a mixed-rate table (every row has a rate class; records packed in row
// order at their own sizes, located through a 16-byte index entry per 32
// rows).
//
// The pages measure lookups from pinned host memory, where the fetch over
// PCIe dominates ("2비트 코드와 공유 트렐리스로 n-gram 룩업 테이블을 4~8배
// 압축한다", onedev.kr, section "Assumptions and limits"), and pair
// allocating bits by access frequency with caching (same section; "Two-bit
// lookup tables shrink DeepSeek's 203 GB memory to 51 GB ...", ai4snews,
// "Perspective"). Records are independently addressable, so the distinct
// records of a batch, copied byte for byte into a packed staging area, form a
// mixed-rate table of their own ("staged rows", numbered in the order the
// hash step found them), which the ordinary mixed-rate decode kernel reads
// by staged row:
//   1. the hash step of the single-rate path: the distinct valid ids, each
//      lookup's hash slot (dedup_hash);
//   2. per block of 32 staged rows, the rate classes (two bit planes, as in
//      a table's index) and the block's record bytes; per tile of 8 blocks
//      their sum (mixed_dedup_blocks);
//   3. an exclusive scan of the tile sums (mixed_dedup_scan_tiles), then of
//      the blocks within each tile: the staging index's byte offsets
//      (mixed_dedup_base);
//   4. every distinct record copied from the table to its staged place
//      (mixed_dedup_stage);
//   5. each lookup's staged row (mixed_dedup_resolve);
// after which gather_decode_mixed decodes the staged rows in lookup order.
#include "cp_internal.h"
#include "cp_lane.h"

namespace cpk {

namespace {

constexpr uint32_t kBad = 0xFFFFFFFFu;  // hash slot of an out-of-range id

// Byte offset and class of row `row` of a mixed-rate table (index entry per
// 32 rows: base offset, class bit planes).
__device__ __forceinline__ uint64_t locate(const MixedEntry *__restrict__ index, const MixedRates &r, uint64_t row,
                                           uint32_t *cls)
{
    const MixedEntry e = index[row >> 5];
    const uint32_t j = (uint32_t)row & 31u, below = (1u << j) - 1u;
    const uint32_t n1 = __builtin_popcount(e.p0 & ~e.p1 & below);
    const uint32_t n2 = __builtin_popcount(~e.p0 & e.p1 & below);
    const uint32_t n3 = __builtin_popcount(e.p0 & e.p1 & below);
    const uint32_t n0 = j - n1 - n2 - n3;
    *cls = ((e.p0 >> j) & 1u) | (((e.p1 >> j) & 1u) << 1);
    return e.base + (uint64_t)n0 * r.R[0] + (uint64_t)n1 * r.R[1] + (uint64_t)n2 * r.R[2] + (uint64_t)n3 * r.R[3];
}

// Lane i of each 32-lane half of a wave takes staged row 32b + i of block b
// (a workgroup takes the kMixedDedupTile = 8 blocks of one tile): the
// classes of the block's rows (rows past the distinct count get class 0 and
// size 0) into its index entry, its record bytes into bsum[b], and the
// tile's total into tsum[tile].
__global__ __launch_bounds__(256) void mixed_dedup_blocks(const MixedEntry *__restrict__ index,
                                                          const MixedRates rates, const int64_t *__restrict__ uniq,
                                                          const unsigned long long *__restrict__ count,
                                                          uint64_t blocks, MixedEntry *__restrict__ stage_index,
                                                          uint64_t *__restrict__ bsum, uint64_t *__restrict__ tsum)
{
    static_assert(kMixedDedupTile * 32 == 256, "a workgroup covers one tile");
    __shared__ uint64_t part[kMixedDedupTile];
    const uint64_t nuniq = *count;
    const uint32_t i = threadIdx.x & 31u, half = (threadIdx.x >> 5) & 1u;
    const uint64_t b = (uint64_t)blockIdx.x * kMixedDedupTile + (threadIdx.x >> 5);
    const uint64_t k = 32 * b + i;
    uint32_t cls = 0, size = 0;
    if (b < blocks && k < nuniq) {
        (void)locate(index, rates, (uint64_t)uniq[k], &cls);
        size = rates.R[cls];
    }
    const uint64_t m0 = __ballot(cls & 1u), m1 = __ballot(cls >> 1);
    uint64_t sum = size;
    for (int x = 16; x >= 1; x >>= 1) sum += __shfl_xor(sum, x, 32);
    if (i == 0) {
        if (b < blocks) {
            MixedEntry e;
            e.base = 0;  // set by mixed_dedup_base
            e.p0 = (uint32_t)(m0 >> (32 * half));
            e.p1 = (uint32_t)(m1 >> (32 * half));
            stage_index[b] = e;
            bsum[b] = sum;
        }
        part[threadIdx.x >> 5] = sum;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t t = 0;
        for (uint32_t q = 0; q < kMixedDedupTile; ++q) t += part[q];
        tsum[blockIdx.x] = t;
    }
}

// Inclusive prefix sum over a 1024-thread workgroup, in thread order; *total
// = the sum over all threads.
__device__ __forceinline__ uint64_t inclusive_1024(uint64_t v, uint64_t *wave_sum, uint64_t *total)
{
    const uint32_t lane = threadIdx.x & 63u, w = threadIdx.x >> 6;
    uint64_t incl = v;
    for (int k = 1; k < 64; k <<= 1) {
        const uint64_t up = __shfl_up(incl, (unsigned)k, 64);
        if (lane >= (uint32_t)k) incl += up;
    }
    if (lane == 63) wave_sum[w] = incl;
    __syncthreads();
    uint64_t before = 0, all = 0;
    for (uint32_t q = 0; q < 16; ++q) {
        if (q < w) before += wave_sum[q];
        all += wave_sum[q];
    }
    __syncthreads();
    *total = all;
    return before + incl;
}

// tsum[0 .. tiles) := its exclusive prefix sums (one workgroup, 1024 tiles
// at a time).
__global__ __launch_bounds__(1024) void mixed_dedup_scan_tiles(uint64_t *__restrict__ tsum, uint64_t tiles)
{
    __shared__ uint64_t wave_sum[16];
    uint64_t carry = 0;
    for (uint64_t t0 = 0; t0 < tiles; t0 += 1024) {
        const uint64_t t = t0 + threadIdx.x;
        const uint64_t v = t < tiles ? tsum[t] : 0;
        uint64_t all;
        const uint64_t incl = inclusive_1024(v, wave_sum, &all);
        if (t < tiles) tsum[t] = carry + incl - v;
        carry += all;
    }
}

// Each block's byte offset in the staging area: its tile's offset plus the
// bytes of the tile's blocks before it (thread per block; the tile's 8
// blocks are 8 neighbouring lanes).
__global__ __launch_bounds__(256) void mixed_dedup_base(const uint64_t *__restrict__ bsum,
                                                        const uint64_t *__restrict__ tsum, uint64_t blocks,
                                                        MixedEntry *__restrict__ stage_index)
{
    const uint64_t b = (uint64_t)blockIdx.x * 256 + threadIdx.x;
    const uint64_t v = b < blocks ? bsum[b] : 0;
    uint64_t incl = v;
    for (uint32_t x = 1; x < kMixedDedupTile; x <<= 1) {
        const uint64_t up = __shfl_up(incl, x, kMixedDedupTile);
        if ((threadIdx.x & (kMixedDedupTile - 1)) >= x) incl += up;
    }
    if (b < blocks) stage_index[b].base = tsum[b / kMixedDedupTile] + incl - v;
}

// Copies distinct record k (row uniq[k] of the table) to its staged place:
// each 16-lane row of a wave copies one record per pass, four passes with
// all loads in flight together. Lane l loads the record's aligned source
// dwords 4l..4l+3 (one 16-byte load; lanes past the record load its first
// 16 bytes again) and writes destination dwords 4l..4l+3; when source and
// destination start at different offsets within a dword, a destination
// dword takes one half from the next or previous source dword, which may be
// the neighbouring lane's (a row shift). A destination dword the record
// shares with a neighbouring record gets a 16-bit store of its own half.
constexpr int kStagePasses = 4;
typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));

__global__ __launch_bounds__(256) void mixed_dedup_stage(const uint8_t *__restrict__ tab,
                                                         const MixedEntry *__restrict__ index,
                                                         const MixedRates rates, const int64_t *__restrict__ uniq,
                                                         const unsigned long long *__restrict__ count,
                                                         const MixedEntry *__restrict__ stage_index,
                                                         uint8_t *__restrict__ staging)
{
    const uint32_t lane = threadIdx.x & 63u, row = lane >> 4, l = lane & 15u;
    const uint64_t wave = (uint64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint64_t waves = (uint64_t)gridDim.x * 4;
    const uint64_t nuniq = *count;
    constexpr uint32_t G = 4 * kStagePasses;  // records per wave
    for (uint64_t k0 = wave * G; k0 < nuniq; k0 += waves * G) {
        u32x4a4 S[kStagePasses];
        uint32_t sh[kStagePasses], R[kStagePasses];
        uint64_t dst[kStagePasses];
#pragma unroll
        for (int p = 0; p < kStagePasses; ++p) {
            const uint64_t k = k0 + 4u * p + row;
            const bool in = k < nuniq;
            uint32_t cls = 0, scls = 0;
            const uint64_t src_off = locate(index, rates, in ? (uint64_t)uniq[k] : 0, &cls);
            dst[p] = locate(stage_index, rates, in ? k : 0, &scls);
            R[p] = in ? rates.R[cls] : 0u;
            const uint8_t *rec = tab + src_off;
            sh[p] = (uint32_t)((uintptr_t)rec & 3u);
            const uint32_t nsrc = (sh[p] + R[p] + 3) >> 2;  // aligned source dwords holding the record
            const u32x4a4 *src = reinterpret_cast<const u32x4a4 *>(rec - sh[p]) + (4 * l < nsrc ? l : 0);
            S[p] = *src;
        }
#pragma unroll
        for (int p = 0; p < kStagePasses; ++p) {
            uint8_t *rec = staging + dst[p];
            const uint32_t dsh = (uint32_t)((uintptr_t)rec & 3u);
            const uint32_t before =
                (uint32_t)__builtin_amdgcn_update_dpp((int)S[p].w, (int)S[p].w, 0x111 /* row_shr:1 */, 0xF, 0xF, false);
            const uint32_t after =
                (uint32_t)__builtin_amdgcn_update_dpp((int)S[p].x, (int)S[p].x, 0x101 /* row_shl:1 */, 0xF, 0xF, false);
            const uint32_t src6[6] = {before, S[p].x, S[p].y, S[p].z, S[p].w, after};
            const int r0 = 16 * (int)l - (int)dsh;  // record byte at this lane's first destination byte
            uint8_t *q = rec - dsh + 16u * l;
            const int Rp = (int)R[p];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                // destination dword 4l+m starts at source byte 4(4l+m) + sh - dsh
                const uint32_t D = sh[p] == dsh ? src6[m + 1]
                                   : sh[p] > dsh ? (src6[m + 1] >> 16) | (src6[m + 2] << 16)
                                                 : (src6[m] >> 16) | (src6[m + 1] << 16);
                const int r = r0 + 4 * m;
                if (r >= 0 && r + 4 <= Rp) {
                    *reinterpret_cast<uint32_t *>(q + 4 * m) = D;
                } else if (r == -2 && Rp > 0) {
                    *reinterpret_cast<uint16_t *>(q + 4 * m + 2) = (uint16_t)(D >> 16);
                } else if (r >= 0 && r + 2 == Rp) {
                    *reinterpret_cast<uint16_t *>(q + 4 * m) = (uint16_t)D;
                }
            }
        }
    }
}

// staged[j] = lookup j's staged row, -1 for an id outside the table.
__global__ __launch_bounds__(256) void mixed_dedup_resolve(const uint32_t *__restrict__ slot_of, uint64_t n,
                                                           const uint32_t *__restrict__ sidx,
                                                           int64_t *__restrict__ staged)
{
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride) {
        const uint32_t s = slot_of[j];
        staged[j] = s == kBad ? -1 : (int64_t)sidx[s];
    }
}

}  // namespace

hipError_t mixed_dedup_prepare(const MixedDedupArgs &a)
{
    const MixedDedupLayout &M = a.layout;
    uint8_t *ws = a.hash.workspace;
    const int64_t *uniq = reinterpret_cast<const int64_t *>(ws + M.hash.uniq);
    const uint32_t *sidx = reinterpret_cast<const uint32_t *>(ws + M.hash.sidx);
    const uint32_t *slot_of = reinterpret_cast<const uint32_t *>(ws + M.hash.slot_of);
    int64_t *staged = reinterpret_cast<int64_t *>(ws + M.hash.staged_ids);
    const unsigned long long *count = reinterpret_cast<const unsigned long long *>(ws + M.hash.count);
    MixedEntry *stage_index = reinterpret_cast<MixedEntry *>(ws + M.index);
    uint64_t *bsum = reinterpret_cast<uint64_t *>(ws + M.bsum);
    uint64_t *tsum = reinterpret_cast<uint64_t *>(ws + M.tsum);
    uint8_t *staging = ws + M.staging;
    // the staging area's last tail_pad bytes (reads past the last staged
    // record stay inside the area) are zeroed with the hash table
    const uint64_t area = M.total - M.staging;
    hipError_t e = dedup_hash(a.hash, staging + area - a.tail_pad, a.tail_pad);
    if (e != hipSuccess) return e;
    const int cus = a.hash.num_cus > 0 ? a.hash.num_cus : 256;
    const hipStream_t st = a.hash.stream;
    hipLaunchKernelGGL(mixed_dedup_blocks, dim3((unsigned)M.tiles), dim3(256), 0, st, a.index, a.rates, uniq,
                       count, M.blocks, stage_index, bsum, tsum);
    hipLaunchKernelGGL(mixed_dedup_scan_tiles, dim3(1), dim3(1024), 0, st, tsum, M.tiles);
    hipLaunchKernelGGL(mixed_dedup_base, dim3((unsigned)((M.blocks + 255) / 256)), dim3(256), 0, st, bsum, tsum,
                       M.blocks, stage_index);
    const uint64_t n = a.hash.n;
    uint64_t sblocks = (n + 4 * kStagePasses * 4 - 1) / (4 * kStagePasses * 4);
    const uint64_t scap = (uint64_t)cus * 32;
    hipLaunchKernelGGL(mixed_dedup_stage, dim3((unsigned)(sblocks < scap ? sblocks : scap)), dim3(256), 0, st,
                       a.hash.records, a.index, a.rates, uniq, count, stage_index, staging);
    uint64_t rblocks = (n + 255) / 256;
    const uint64_t rcap = (uint64_t)cus * 8;
    hipLaunchKernelGGL(mixed_dedup_resolve, dim3((unsigned)(rblocks < rcap ? rblocks : rcap)), dim3(256), 0, st,
                       slot_of, n, sidx, staged);
    return hipGetLastError();
}

}  // namespace cpk
