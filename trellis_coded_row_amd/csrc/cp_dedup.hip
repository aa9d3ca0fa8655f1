// cp_dedup.hip - fetch each distinct record of a lookup batch once.
//
// The pages measure lookups from a table in pinned host memory, where the
// fetch over PCIe dominates, and note that the row-wise layout's advantage
// grows there ("2비트 코드와 공유 트렐리스로 n-gram 룩업 테이블을 4~8배 압축한다",
// onedev.kr, section "Assumptions and limits"). A lookup batch repeats hot
// rows (the replay's ids are ~27% distinct), so this path
//   1. hashes the batch's valid ids into an open-addressing table in device
//      memory, numbering each distinct id once (dedup_insert),
//   2. copies each distinct record once from the table into a packed staging
//      area in device memory (dedup_gather),
//   3. gives every lookup the staging index of its id (dedup_resolve),
// after which the ordinary gather-decode kernel decodes the staging area in
// the original lookup order. Records are independently addressable, so a
// record copied byte for byte decodes exactly as it would in place.
#include "cp_internal.h"

namespace cpk {

static constexpr int64_t kEmpty = -1;            // free hash slot (valid ids are >= 0)
static constexpr uint32_t kBadSlot = 0xFFFFFFFFu;  // lookup with an out-of-range id

// 64-bit finaliser (xor-shift / multiply) spreading ids over the slots.
__device__ __forceinline__ uint64_t mix64(uint64_t x)
{
    x ^= x >> 30;
    x *= 0xBF58476D1CE4E5B9ull;
    x ^= x >> 27;
    x *= 0x94D049BB133111EBull;
    return x ^ (x >> 31);
}

// Empties the hash table, zeroes the counter and the staging area's tail pad
// (a kernel rather than a memset, so the sequence can be captured in a graph).
__global__ __launch_bounds__(256) void dedup_clear(int64_t *__restrict__ keys, uint64_t slots,
                                                   unsigned long long *__restrict__ count,
                                                   uint8_t *__restrict__ pad, uint64_t pad_bytes)
{
    const uint64_t tid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = tid; i < slots; i += stride) keys[i] = kEmpty;
    for (uint64_t i = tid; i < pad_bytes; i += stride) pad[i] = 0;
    if (tid == 0) *count = 0;
}

static constexpr int kTile = 1024;       // ids per workgroup tile
static constexpr int kTileSlots = 2048;  // LDS hash slots per tile

// Two-level insertion. Repeats of a hot id (a Zipf batch has thousands) would
// all contend on one global slot, so each 256-thread workgroup first dedups a
// tile of 1,024 ids in an LDS hash table and then inserts only the tile's
// distinct ids into the global table; new global ids are numbered with one
// counter update per wave. slot_of[j] is the id's global slot, or kBadSlot
// for an id outside [0, rows).
__global__ __launch_bounds__(256) void dedup_insert(const int64_t *__restrict__ ids, uint64_t n, uint64_t rows,
                                                    int64_t *__restrict__ keys, uint32_t *__restrict__ sidx,
                                                    uint64_t slot_mask, uint32_t *__restrict__ slot_of,
                                                    int64_t *__restrict__ uniq,
                                                    unsigned long long *__restrict__ count)
{
    __shared__ int64_t lkeys[kTileSlots];
    __shared__ uint32_t lslot[kTileSlots];
    const uint32_t tid = threadIdx.x, lane = tid & 63u;
    const uint64_t ntiles = (n + kTile - 1) / kTile;
    for (uint64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        for (int t = tid; t < kTileSlots; t += 256) lkeys[t] = kEmpty;
        __syncthreads();
        // 1. the tile's valid ids into the LDS table
        uint32_t lsl[kTile / 256];
#pragma unroll
        for (int r = 0; r < kTile / 256; ++r) {
            const uint64_t j = tile * kTile + r * 256 + tid;
            const int64_t id = j < n ? ids[j] : -1;
            lsl[r] = kBadSlot;
            if (j < n && (uint64_t)id < rows) {
                uint32_t h = (uint32_t)mix64((uint64_t)id) & (kTileSlots - 1);
                for (int probe = 0; probe < kTileSlots; ++probe) {
                    const int64_t k = (int64_t)atomicCAS(reinterpret_cast<unsigned long long *>(&lkeys[h]),
                                                         (unsigned long long)kEmpty, (unsigned long long)id);
                    if (k == kEmpty || k == id) {
                        lsl[r] = h;
                        break;
                    }
                    h = (h + 1) & (kTileSlots - 1);
                }
            }
        }
        __syncthreads();
        // 2. each distinct id of the tile into the global table; a thread's
        // 8 slots are resolved side by side (their loads and swaps in flight
        // together) and new ids are numbered with one counter update per wave
        constexpr int PER = kTileSlots / 256;
        int64_t key[PER];
        uint64_t h[PER];
        uint32_t gslot[PER];
        bool won[PER], done[PER];
#pragma unroll
        for (int r = 0; r < PER; ++r) {
            key[r] = lkeys[r * 256 + tid];
            done[r] = key[r] == kEmpty;
            won[r] = false;
            gslot[r] = kBadSlot;
            h[r] = mix64((uint64_t)key[r]) & slot_mask;
        }
        // the table has at least twice as many slots as the batch has ids, so
        // every id ends within slot_mask + 1 rounds
        for (uint64_t round = 0; round <= slot_mask; ++round) {
            bool all = true;
#pragma unroll
            for (int r = 0; r < PER; ++r) all &= done[r];
            if (all) break;
            int64_t cur[PER];
#pragma unroll
            for (int r = 0; r < PER; ++r)
                cur[r] = done[r] ? 0 : __hip_atomic_load(&keys[h[r]], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
            for (int r = 0; r < PER; ++r) {
                if (!done[r] && cur[r] == kEmpty) {
                    // a stale empty read is harmless: the swap returns the real key
                    cur[r] = (int64_t)atomicCAS(reinterpret_cast<unsigned long long *>(&keys[h[r]]),
                                                (unsigned long long)kEmpty, (unsigned long long)key[r]);
                    won[r] = cur[r] == kEmpty;
                }
            }
#pragma unroll
            for (int r = 0; r < PER; ++r) {
                if (done[r]) continue;
                if (won[r] || cur[r] == key[r]) {
                    gslot[r] = (uint32_t)h[r];
                    done[r] = true;
                } else {
                    h[r] = (h[r] + 1) & slot_mask;
                }
            }
        }
        uint64_t masks[PER];
        uint32_t total = 0;
#pragma unroll
        for (int r = 0; r < PER; ++r) {
            masks[r] = __ballot(won[r]);
            total += (uint32_t)__builtin_popcountll(masks[r]);
            lslot[r * 256 + tid] = gslot[r];
        }
        if (total) {
            unsigned long long first = 0;
            if (lane == 0) first = atomicAdd(count, (unsigned long long)total);
            first = __shfl(first, 0, 64);
            const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
            for (int r = 0; r < PER; ++r) {
                if (won[r]) {
                    const uint32_t k = (uint32_t)(first + __builtin_popcountll(masks[r] & below));
                    sidx[gslot[r]] = k;
                    uniq[k] = key[r];
                }
                first += (unsigned long long)__builtin_popcountll(masks[r]);
            }
        }
        __syncthreads();
        // 3. every id's global slot
#pragma unroll
        for (int r = 0; r < kTile / 256; ++r) {
            const uint64_t j = tile * kTile + r * 256 + tid;
            if (j < n) slot_of[j] = lsl[r] == kBadSlot ? kBadSlot : lslot[lsl[r]];
        }
        __syncthreads();
    }
}

// Copies the 16-byte-aligned window holding record uniq[k] (at most
// `units` 16-byte units, which covers the record wherever it starts) to
// staging slot k (slot_bytes apart, 16-byte aligned): large aligned reads, a
// few per record, which matters most when the table is across PCIe. The
// record then sits at byte offset (uniq[k] * record_bytes) % 16 of its slot.
__global__ __launch_bounds__(256) void dedup_gather(const uint8_t *__restrict__ table, uint64_t record_bytes,
                                                    const int64_t *__restrict__ uniq,
                                                    const unsigned long long *__restrict__ count,
                                                    uint8_t *__restrict__ staging, uint64_t max_records,
                                                    uint32_t units, uint64_t slot_bytes)
{
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const uint64_t nuniq = *count < max_records ? *count : max_records;
    const uint64_t tid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = tid; i < nuniq * units; i += stride) {
        const uint64_t k = i / units, u = i % units;
        const uint64_t start = ((uint64_t)uniq[k] * record_bytes) & ~(uint64_t)15;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(table + start + 16 * u);
        *reinterpret_cast<u32x4 *>(staging + k * slot_bytes + 16 * u) = v;
    }
}

// Byte offset of every lookup's record in the staging area; out-of-range
// ids map to -1, which the decode kernel turns into a zero row and the
// sticky flag.
__global__ __launch_bounds__(256) void dedup_resolve(const uint32_t *__restrict__ slot_of, uint64_t n,
                                                     const uint32_t *__restrict__ sidx,
                                                     const int64_t *__restrict__ uniq, uint64_t record_bytes,
                                                     uint64_t slot_bytes, int64_t *__restrict__ staged_off)
{
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride) {
        const uint32_t s = slot_of[j];
        if (s == kBadSlot) {
            staged_off[j] = -1;
        } else {
            const uint64_t k = sidx[s];
            staged_off[j] = (int64_t)(k * slot_bytes + (((uint64_t)uniq[k] * record_bytes) & 15));
        }
    }
}

static unsigned dedup_grid(uint64_t items, uint64_t per_block, int num_cus)
{
    const uint64_t b = (items + per_block - 1) / per_block;
    const uint64_t cap = (uint64_t)(num_cus > 0 ? num_cus : 256) * 8;
    return (unsigned)(b < 1 ? 1 : (b > cap ? cap : b));
}

hipError_t dedup_hash(const DedupArgs &a, uint8_t *pad, uint64_t pad_bytes)
{
    const DedupLayout &L = a.layout;
    uint8_t *ws = a.workspace;
    int64_t *keys = reinterpret_cast<int64_t *>(ws + L.keys);
    uint32_t *sidx = reinterpret_cast<uint32_t *>(ws + L.sidx);
    uint32_t *slot_of = reinterpret_cast<uint32_t *>(ws + L.slot_of);
    int64_t *uniq = reinterpret_cast<int64_t *>(ws + L.uniq);
    unsigned long long *count = reinterpret_cast<unsigned long long *>(ws + L.count);
    hipLaunchKernelGGL(dedup_clear, dim3(dedup_grid(L.slots, 256, a.num_cus)), dim3(256), 0, a.stream, keys, L.slots,
                       count, pad, pad_bytes);
    hipLaunchKernelGGL(dedup_insert, dim3(dedup_grid(a.n, kTile, a.num_cus)), dim3(256), 0, a.stream, a.ids, a.n,
                       a.rows, keys, sidx, L.slots - 1, slot_of, uniq, count);
    return hipGetLastError();
}

hipError_t dedup_prepare(const DedupArgs &a)
{
    const DedupLayout &L = a.layout;
    uint8_t *ws = a.workspace;
    uint32_t *sidx = reinterpret_cast<uint32_t *>(ws + L.sidx);
    uint32_t *slot_of = reinterpret_cast<uint32_t *>(ws + L.slot_of);
    int64_t *uniq = reinterpret_cast<int64_t *>(ws + L.uniq);
    int64_t *staged = reinterpret_cast<int64_t *>(ws + L.staged_ids);
    unsigned long long *count = reinterpret_cast<unsigned long long *>(ws + L.count);
    uint8_t *staging = ws + L.staging;
    hipError_t e = dedup_hash(a, staging + a.n * L.slot_bytes, L.total - L.staging - a.n * L.slot_bytes);
    if (e != hipSuccess) return e;
    const uint32_t units = dedup_window_units(a.record_bytes);
    hipLaunchKernelGGL(dedup_gather, dim3(dedup_grid(a.n * units, 256, a.num_cus)), dim3(256), 0, a.stream,
                       a.records, a.record_bytes, uniq, count, staging, a.n, units, L.slot_bytes);
    hipLaunchKernelGGL(dedup_resolve, dim3(dedup_grid(a.n, 256, a.num_cus)), dim3(256), 0, a.stream, slot_of, a.n,
                       sidx, uniq, a.record_bytes, L.slot_bytes, staged);
    return hipGetLastError();
}

}  // namespace cpk
