// cp_probe.hip - measurement probes (include/cp_probe.h): a streaming read,
// the lookup's output stream alone, the lookup's record fetch alone, and a
// two-lane LDS access that shows which lanes the LDS serves together. They
// give the floors and the hardware facts the kernels are designed against;
// none is on the lookup path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/cp_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// A word the data's XOR is compared with, so the loads cannot be dropped
// (the store behind it practically never happens).
constexpr uint32_t kSinkMagic = 0x9E3779B9u;

__global__ __launch_bounds__(256) void read_stream(const u32x4 *__restrict__ src, uint64_t n16,
                                                   uint32_t *__restrict__ sink)
{
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        acc ^= __builtin_nontemporal_load(&src[i]);
    const uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (v == kSinkMagic) sink[0] = v;
}

// d/8 lanes per row (one 16-byte store each); a wave takes CHUNK consecutive
// rows per chunk, as the gather-decode kernel does.
template <int D, int CHUNK>
__global__ __launch_bounds__(1024) void store_rows(uint32_t *__restrict__ out, uint64_t n)
{
    constexpr int LANES = D / 8, GROUPS = 64 / LANES, CI = CHUNK / GROUPS;
    const uint32_t lane = threadIdx.x & 63u, l = lane % LANES, g = lane / LANES;
    const uint64_t wave = (uint64_t)blockIdx.x * 16 + (threadIdx.x >> 6);
    const uint64_t waves = (uint64_t)gridDim.x * 16;
    const uint64_t nchunks = (n + CHUNK - 1) / CHUNK;
    for (uint64_t c = wave; c < nchunks; c += waves) {
#pragma unroll
        for (int i = 0; i < CI; ++i) {
            const uint64_t row = c * CHUNK + (uint64_t)i * GROUPS + g;
            const uint32_t v = (uint32_t)row * 0x9E3779B9u + l;
            if (row < n) __builtin_nontemporal_store((u32x4){v, v ^ 1u, v ^ 2u, v ^ 3u},
                                                     reinterpret_cast<u32x4 *>(out + row * (D / 2) + 4u * l));
        }
    }
}

// One wave per chunk of 16 ids: lane k loads id k, then each row's record is
// read by 2-byte loads (lane l takes half-words l, l + 64), all 16 records
// requested before any is used.
__global__ __launch_bounds__(1024) void gather_records(const uint8_t *__restrict__ tab, uint64_t R,
                                                       const int64_t *__restrict__ ids, uint64_t n,
                                                       uint32_t *__restrict__ sink)
{
    constexpr int CHUNK = 16;
    const uint32_t lane = threadIdx.x & 63u;
    const uint64_t wave = (uint64_t)blockIdx.x * 16 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint64_t waves = (uint64_t)gridDim.x * 16;
    const uint64_t nchunks = (n + CHUNK - 1) / CHUNK;
    const uint32_t halves = (uint32_t)(R / 2);
    uint32_t acc = 0;
    for (uint64_t c = wave; c < nchunks; c += waves) {
        const uint64_t j = c * CHUNK + lane;
        const uint64_t off = (lane < CHUNK && j < n) ? (uint64_t)ids[j] * R : 0;
        uint32_t v[CHUNK];
#pragma unroll
        for (int i = 0; i < CHUNK; ++i) {
            const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)off, i);
            const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(off >> 32), i);
            const uint8_t *rec = tab + (((uint64_t)hi << 32) | lo);
            uint32_t w = lane < halves ? *reinterpret_cast<const uint16_t *>(rec + 2u * lane) : 0u;
            if (lane + 64 < halves) w ^= *reinterpret_cast<const uint16_t *>(rec + 2u * (lane + 64));
            v[i] = w;
        }
#pragma unroll
        for (int i = 0; i < CHUNK; ++i) acc ^= v[i] * (uint32_t)(i + 1);
    }
    if (acc == kSinkMagic) sink[0] = acc;
}

int blocks_for(uint64_t items, uint64_t per_block, uint64_t cap)
{
    uint64_t b = (items + per_block - 1) / per_block;
    if (b < 1) b = 1;
    if (b > cap) b = cap;
    return (int)b;
}

template <int D>
hipError_t launch_store(uint16_t *out, uint64_t n, uint32_t chunk, hipStream_t s)
{
    constexpr int GROUPS = 64 / (D / 8);
    auto go = [&](auto kernel, uint64_t ch) {
        const uint64_t nchunks = (n + ch - 1) / ch;
        hipLaunchKernelGGL(kernel, dim3(blocks_for(nchunks, 16, 0x7FFFFFFFull)), dim3(1024), 0, s,
                           reinterpret_cast<uint32_t *>(out), n);
    };
    if (chunk <= (uint32_t)GROUPS) go(store_rows<D, (GROUPS > 1 ? GROUPS : 1)>, GROUPS > 1 ? GROUPS : 1);
    else if (chunk <= 4) go(store_rows<D, (GROUPS > 4 ? GROUPS : 4)>, GROUPS > 4 ? GROUPS : 4);
    else go(store_rows<D, (GROUPS > 16 ? GROUPS : 16)>, GROUPS > 16 ? GROUPS : 16);
    return hipGetLastError();
}

// Two lanes of one wave touch LDS addresses 256 bytes apart (the same banks
// on a 64-bank LDS) `iters` times, every other lane idle: the accesses
// collide, and so count bank-conflict cycles, only if the LDS serves the
// two lanes in the same cycle. W: bytes per access (4, 8, 16).
template <int W, bool WRITE>
__global__ __launch_bounds__(64) void lds_pair(uint32_t a, uint32_t b, uint32_t iters, uint32_t *__restrict__ sink)
{
    __shared__ __attribute__((aligned(16))) uint32_t lds[256];
    for (uint32_t i = threadIdx.x; i < 256; i += 64) lds[i] = i;
    __syncthreads();
    const uint32_t l = threadIdx.x;
    uint32_t acc = 0;
    if (l == a || l == b) {
        uint32_t off = l == a ? 0u : 64u;  // dwords
        for (uint32_t it = 0; it < iters; ++it) {
            uint32_t *p = lds + (off & 127u);
            if constexpr (WRITE) {
                if constexpr (W == 4) *p = it;
                else if constexpr (W == 8) *reinterpret_cast<uint64_t *>(p) = it;
                else *reinterpret_cast<u32x4 *>(p) = (u32x4){it, l, it, l};
            } else {
                if constexpr (W == 4) acc ^= *p;
                else if constexpr (W == 8) acc ^= (uint32_t)*reinterpret_cast<const uint64_t *>(p);
                else { const u32x4 v = *reinterpret_cast<const u32x4 *>(p); acc ^= v.x ^ v.w; }
            }
            asm volatile("" : "+v"(off));
        }
    }
    // what the stores left is read back, so they are not dropped
    __syncthreads();
    acc ^= lds[l];  // one bank per lane: no conflict of its own
    if (acc == kSinkMagic) *sink = acc;
}

}  // namespace

extern "C" {

int cpp_lds_pair(uint32_t width, uint32_t write, uint32_t lane_a, uint32_t lane_b, uint32_t iters, uint32_t *sink,
                 void *stream)
{
    if (!sink || lane_a >= 64 || lane_b >= 64 || lane_a == lane_b) return (int)hipErrorInvalidValue;
    (void)hipGetLastError();
    const hipStream_t s = (hipStream_t)stream;
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3(1), dim3(64), 0, s, lane_a, lane_b, iters, sink);
        return (int)hipGetLastError();
    };
    switch (width * 2 + (write ? 1 : 0)) {
    case 8: return go(lds_pair<4, false>);
    case 9: return go(lds_pair<4, true>);
    case 16: return go(lds_pair<8, false>);
    case 17: return go(lds_pair<8, true>);
    case 32: return go(lds_pair<16, false>);
    case 33: return go(lds_pair<16, true>);
    default: return (int)hipErrorInvalidValue;
    }
}

int cpp_read_stream(const void *src, uint64_t bytes, uint32_t *sink, void *stream)
{
    if (!src || !sink || (bytes & 15u) || ((uintptr_t)src & 15u)) return (int)hipErrorInvalidValue;
    if (bytes == 0) return 0;
    (void)hipGetLastError();
    int dev = 0, cus = 256;
    (void)hipGetDevice(&dev);
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const uint64_t n16 = bytes / 16;
    hipLaunchKernelGGL(read_stream, dim3(blocks_for(n16, 256, (uint64_t)cus * 16)), dim3(256), 0,
                       (hipStream_t)stream, reinterpret_cast<const u32x4 *>(src), n16, sink);
    return (int)hipGetLastError();
}

int cpp_store_rows(uint16_t *out, uint64_t n, uint32_t d, uint32_t chunk, void *stream)
{
    if (!out || ((uintptr_t)out & 15u)) return (int)hipErrorInvalidValue;
    if (n == 0) return 0;
    (void)hipGetLastError();
    const hipStream_t s = (hipStream_t)stream;
    switch (d) {
    case 64: return (int)launch_store<64>(out, n, chunk, s);
    case 128: return (int)launch_store<128>(out, n, chunk, s);
    case 256: return (int)launch_store<256>(out, n, chunk, s);
    case 512: return (int)launch_store<512>(out, n, chunk, s);
    default: return (int)hipErrorInvalidValue;
    }
}

int cpp_gather_records(const void *records, uint64_t record_bytes, const int64_t *ids, uint64_t n, uint32_t *sink,
                       void *stream)
{
    if (!records || !ids || !sink || (record_bytes & 1u) || record_bytes < 18 || record_bytes > 194)
        return (int)hipErrorInvalidValue;
    if (n == 0) return 0;
    (void)hipGetLastError();
    const uint64_t nchunks = (n + 15) / 16;
    hipLaunchKernelGGL(gather_records, dim3(blocks_for(nchunks, 16, 0x7FFFFFFFull)), dim3(1024), 0,
                       (hipStream_t)stream, static_cast<const uint8_t *>(records), record_bytes, ids, n, sink);
    return (int)hipGetLastError();
}

}  // extern "C"
