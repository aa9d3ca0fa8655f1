// cp_mixed.hip - gather-and-decode for mixed-rate CP tables: every row has a
// rate class, class c coded at kv_c bits per step.
//
// The pages study allocating bits by how often a row is looked up, over the
// code rates they evaluate (1.5 / 2 / 2.5 / 3 bits per element), and find
// that the access counts behind it may not carry over between text domains
// ("2비트 코드와 공유 트렐리스로 n-gram 룩업 테이블을 4~8배 압축한다",
// onedev.kr, sections "How it is used" and "Assumptions and limits"). They
// give no format; this library stores the records of all rows packed in row
// order, each at its own class's rate, so a row's record starts at the sum of
// the record sizes before it. To find it in O(1) the library keeps an index
// of one 16-byte entry per 32 rows:
//   base - byte offset of the block's first record;
//   p0   - bit j = bit 0 of the class of row 32b + j;
//   p1   - bit j = bit 1 of that class;
// so row 32b + j starts at base + sum over c of n_c * R_c, n_c being the
// number of rows of class c among the block's first j rows (popcounts of the
// two bit planes under a mask), and has class bit j of (p0, p1).
//
// The kernel is the single-rate gather-decode with the record located through
// the index and one trellis walk that takes the rate as an operand: shift
// amounts come from kv, the history bits from the two previous lanes of the
// row. Rows of different rates can therefore share a wave (d < 512) with
// uniform control flow, and at d = 512 the code stays one walk per row rather
// than four (a version with a compile-time walk per rate and a branch per row
// was 3x the code and 8% slower on the d512 replay).
#include "cp_lane.h"

namespace cpk {

namespace {

// One row's 8 outputs of this lane for a rate known only at run time (kv per
// lane): the history bits come from the two previous lanes of the row (kv = 3
// needs both; for kv >= 4 the second contributes nothing), the window field
// is 64 bits wide and the shifts take the rate as an operand.
template <int D, Emit MODE, bool SALPHA>
__device__ __forceinline__ u32x4 decode_any_rate(uint32_t newbits, uint32_t kv, uint32_t alpha_bits, uint32_t l,
                                                 uint32_t g, const uint32_t *s_lut, uint32_t lds_off)
{
    constexpr int LANES = D / 8;
    const uint32_t newb = 4u * kv, m = 16u - kv;
    uint32_t prev, prev2;
    if constexpr (LANES == 64) {
        prev = __builtin_amdgcn_update_dpp(newbits, newbits, 0x13C /* wave_ror:1 */, 0xF, 0xF, false);
        prev2 = __builtin_amdgcn_update_dpp(prev, prev, 0x13C, 0xF, 0xF, false);
    } else {
        prev = __shfl(newbits, (int)(g * LANES + (l + LANES - 1) % LANES), 64);
        prev2 = __shfl(newbits, (int)(g * LANES + (l + LANES - 2) % LANES), 64);
    }
    // the m bits of the code just below this lane's new bits
    const uint32_t hist = (uint32_t)((((uint64_t)prev << newb) | prev2) >> (2u * newb - m));
    const uint64_t field = ((uint64_t)newbits << m) | hist;
    const float alpha = __builtin_bit_cast(float, alpha_bits);
    u32x4 v;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t x = (uint32_t)(field >> (kv * (uint32_t)k));
        const uint32_t h = hash_mad(x);
        const uint32_t e = *reinterpret_cast<const uint32_t *>(
            reinterpret_cast<const char *>(s_lut) + and_or(h, 0xFF80u, and_or(x >> 9, 0x40u, lds_off)));
        v[k] = emit_pair<MODE, SALPHA>(e, alpha, alpha_bits);
    }
    return v;
}

template <int D, bool RAW, int BLOCK, int CHUNK>
__global__ __launch_bounds__(BLOCK) void gather_decode_mixed(const uint8_t *__restrict__ tab, const uint64_t rows,
                                                             const uint32_t *__restrict__ lut,
                                                             const int64_t *__restrict__ ids, const uint64_t n,
                                                             uint32_t *__restrict__ out, int *__restrict__ err,
                                                             const MixedEntry *__restrict__ index,
                                                             const MixedRates rates)
{
    constexpr int LANES = D / 8;
    constexpr int GROUPS = 64 / LANES;
    constexpr int WAVES = BLOCK / 64;
    constexpr int CI = CHUNK / GROUPS;
    static_assert(CHUNK <= 64 && CI >= 1 && CI * GROUPS == CHUNK, "one id per lane per chunk");

    __shared__ __attribute__((aligned(16))) uint32_t s_lut[kLdsLutWords];

    const uint32_t lane = threadIdx.x & 63;
    const uint32_t l = lane % LANES;
    const uint32_t g = lane / LANES;
    const uint32_t lds_off = (lane & 15u) * 4u;
    const uint64_t wave =
        (uint64_t)blockIdx.x * WAVES + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint64_t waves = (uint64_t)gridDim.x * WAVES;
    const uint64_t nchunks = (n + CHUNK - 1) / CHUNK;
    bool bad = false;

    auto row_of = [&](uint64_t c, uint32_t i) -> uint64_t { return c * CHUNK + i; };
    auto load_id = [&](uint64_t c) -> int64_t {
        const uint64_t j = row_of(c, lane);
        return (c < nchunks && lane < CHUNK && j < n) ? ids[j] : 0;
    };
    // index entry of the row a lane looks up (row 0 for an id outside the
    // table or a lane past the chunk, whose rate and extent agree)
    auto entry_of = [&](int64_t id) -> MixedEntry {
        return index[((uint64_t)id < rows ? (uint64_t)id : 0) >> 5];
    };
    // the first chunk's ids and index entries are requested before the
    // codebook is staged, so their latencies overlap
    int64_t my_id = load_id(wave);
    MixedEntry e = entry_of(my_id);
    stage_lut<BLOCK>(s_lut, lut);
    for (uint64_t c = wave; c < nchunks; c += waves) {
        uint32_t cn = __builtin_amdgcn_readfirstlane((uint32_t)((n - c * CHUNK) < CHUNK ? (n - c * CHUNK) : CHUNK));
        asm volatile("" : "+s"(cn));
        const bool in = lane < cn;
        const bool ok = in && (uint64_t)my_id < rows;
        bad |= in && !ok;
        // lane k locates chunk row k's record (a lane past the chunk gets
        // id 0 from load_id, so its entry is row 0's as well)
        const uint64_t rid = ok ? (uint64_t)my_id : 0;
        const uint32_t j = (uint32_t)rid & 31u, below = (1u << j) - 1u;
        const uint32_t n1 = __builtin_popcount(e.p0 & ~e.p1 & below);
        const uint32_t n2 = __builtin_popcount(~e.p0 & e.p1 & below);
        const uint32_t n3 = __builtin_popcount(e.p0 & e.p1 & below);
        const uint32_t n0 = j - n1 - n2 - n3;
        const uint64_t my_off = e.base + (uint64_t)n0 * rates.R[0] + (uint64_t)n1 * rates.R[1] +
                                (uint64_t)n2 * rates.R[2] + (uint64_t)n3 * rates.R[3];
        const uint32_t cls = ((e.p0 >> j) & 1u) | (((e.p1 >> j) & 1u) << 1);
        const uint32_t my_kv = (rates.kv_packed >> (8u * cls)) & 0xFFu;
        const uint64_t okmask = __ballot(ok);
        my_id = load_id(c + waves);

        // record offset and rate of the row that lane group g decodes i-th
        auto row_offset = [&](uint32_t i) -> uint64_t {
            if constexpr (GROUPS == 1) return readlane_u64(my_off, i);
            else return __shfl(my_off, (int)(i * GROUPS + g), 64);
        };
        // d = 512: the rows' rates as three bit planes (bit i of plane b is bit b
        // of row i's kv), from which a row's rate is taken again where it is
        // used rather than held in a register for the whole chunk
        uint64_t kvb0 = 0, kvb1 = 0, kvb2 = 0;
        if constexpr (GROUPS == 1) {
            kvb0 = __ballot(my_kv & 1u);
            kvb1 = __ballot((my_kv >> 1) & 1u);
            kvb2 = __ballot((my_kv >> 2) & 1u);
        }
        auto row_kv = [&](uint32_t i) -> uint32_t {
            if constexpr (GROUPS == 1)
                return (uint32_t)((kvb0 >> i) & 1u) | ((uint32_t)((kvb1 >> i) & 1u) << 1) |
                       ((uint32_t)((kvb2 >> i) & 1u) << 2);
            else return (uint32_t)__shfl((int)my_kv, (int)(i * GROUPS + g), 64);
        };
        // smallest exponent field (in place) among the chunk's scales
        uint32_t amin = 0x7F800000u;
        {
            uint32_t nb[CI], ab[CI], kv[CI];
#pragma unroll
            for (int i = 0; i < CI; ++i) {
                const uint64_t o = row_offset((uint32_t)i);
                kv[i] = row_kv((uint32_t)i);
                nb[i] = lane_bits(tab, o, 4u * kv[i], l);
                ab[i] = scale_bits(tab, o, kv[i] * (uint32_t)(D / 16));
            }
            if constexpr (GROUPS == 1) asm volatile("" : "+s"(kvb0), "+s"(kvb1), "+s"(kvb2));
#pragma unroll
            for (int i = 0; i < CI; ++i) {
                const uint32_t r = i * GROUPS + g;
                const uint32_t kvi = GROUPS == 1 ? row_kv((uint32_t)i) : kv[i];
                const u32x4 v = decode_any_rate<D, RAW ? kRaw : kScaled, (GROUPS == 1)>(nb[i], kvi, ab[i], l, g,
                                                                                          s_lut, lds_off);
                if (r < cn) store16(out + row_of(c, r) * (D / 2) + 4u * l, v);
                if constexpr (!RAW) {
                    amin = __builtin_elementwise_min(amin, ab[i] & 0x7F800000u);
                    // taken here, so the row's scale register is free afterwards
                    if constexpr (GROUPS == 1) asm volatile("" : "+s"(amin));
                    else asm volatile("" : "+v"(amin));
                }
            }
        }
        // rows with a tiny scale again, exactly (see the single-rate kernel)
        if constexpr (!RAW) {
            if (__builtin_expect(__ballot(scale_is_tiny(amin)) != 0, 0)) {
                __builtin_amdgcn_s_waitcnt(0);
#pragma unroll 1
                for (uint32_t i = 0; i < (uint32_t)CI; ++i) {
                    const uint32_t r = i * GROUPS + g;
                    const uint64_t o = row_offset(i);
                    const uint32_t kv = row_kv(i);
                    const uint32_t ab = scale_bits(tab, o, kv * (uint32_t)(D / 16));
                    const u32x4 v = decode_any_rate<D, kTiny, (GROUPS == 1)>(lane_bits(tab, o, 4u * kv, l), kv, ab,
                                                                              l, g, s_lut, lds_off);
                    if (r < cn && scale_is_tiny(ab)) store16(out + row_of(c, r) * (D / 2) + 4u * l, v);
                }
            }
        }
        // the next chunk's index entries load while this chunk's stores drain
        e = entry_of(my_id);
        const uint64_t badmask = __ballot(in) & ~okmask;
        if (badmask) {
            __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
            for (int i = 0; i < CI; ++i) {
                const uint32_t r = i * GROUPS + g;
                if ((badmask >> r) & 1u)
                    store16(out + row_of(c, r) * (D / 2) + 4u * l, (u32x4){0u, 0u, 0u, 0u});
            }
        }
    }
    if (bad) atomicOr(err, 1);
}

template <int D, bool RAW, int CHUNK_ROWS>
hipError_t launch_mixed_shape(const MixedLaunchArgs &a)
{
    constexpr int BLOCK = kBlock;
    constexpr int GROUPS = 64 / (D / 8);
    constexpr int CHUNK = (CHUNK_ROWS / GROUPS > 0 ? CHUNK_ROWS / GROUPS : 1) * GROUPS;
    const uint64_t nchunks = (a.n + CHUNK - 1) / CHUNK;
    uint64_t blocks = (nchunks + BLOCK / 64 - 1) / (BLOCK / 64);
    if (blocks > 0x7FFFFFFFull) blocks = 0x7FFFFFFFull;  // the chunk loop strides over any excess
    hipLaunchKernelGGL((gather_decode_mixed<D, RAW, BLOCK, CHUNK>), dim3((unsigned)blocks), dim3(BLOCK), 0,
                       a.stream, a.records, a.rows, a.lut, a.ids, a.n, a.out, a.err, a.index, a.rates);
    return hipGetLastError();
}

// chunk length by batch size, as for single-rate tables (lookup_chunk_rows)
template <int D, bool RAW>
hipError_t launch_mixed_one(const MixedLaunchArgs &a)
{
    switch (lookup_chunk_rows(a.n, a.num_cus)) {
    case 1: return launch_mixed_shape<D, RAW, 1>(a);
    case 4: return launch_mixed_shape<D, RAW, 4>(a);
    default: return launch_mixed_shape<D, RAW, kChunk>(a);
    }
}

}  // namespace

bool mixed_supported(uint32_t d) { return d == 64 || d == 128 || d == 256 || d == 512; }

hipError_t launch_mixed(uint32_t d, bool raw, const MixedLaunchArgs &a)
{
    if (a.n == 0) return hipSuccess;
    switch (d) {
    case 64: return raw ? launch_mixed_one<64, true>(a) : launch_mixed_one<64, false>(a);
    case 128: return raw ? launch_mixed_one<128, true>(a) : launch_mixed_one<128, false>(a);
    case 256: return raw ? launch_mixed_one<256, true>(a) : launch_mixed_one<256, false>(a);
    case 512: return raw ? launch_mixed_one<512, true>(a) : launch_mixed_one<512, false>(a);
    default: return hipErrorInvalidValue;
    }
}

uint64_t mixed_index_entries(uint64_t rows) { return (rows + 31) / 32; }

int mixed_index_build(const uint8_t *row_class, uint64_t rows, uint32_t nclass, const uint32_t R[4],
                      MixedEntry *index, uint64_t *total_bytes)
{
    uint64_t acc = 0;
    const uint64_t nblk = mixed_index_entries(rows);
    for (uint64_t b = 0; b < nblk; ++b) {
        MixedEntry e;
        e.base = acc;
        e.p0 = 0;
        e.p1 = 0;
        const uint64_t r0 = b * 32;
        const uint32_t cnt = (uint32_t)(rows - r0 < 32 ? rows - r0 : 32);
        for (uint32_t j = 0; j < cnt; ++j) {
            const uint32_t c = row_class[r0 + j];
            if (c >= nclass) return -1;
            e.p0 |= (c & 1u) << j;
            e.p1 |= ((c >> 1) & 1u) << j;
            acc += R[c];
        }
        index[b] = e;
    }
    *total_bytes = acc;
    return 0;
}

uint64_t mixed_record_offset(const MixedEntry *index, const uint32_t R[4], uint64_t row, uint32_t *cls)
{
    const MixedEntry &e = index[row >> 5];
    const uint32_t j = (uint32_t)row & 31u, below = (1u << j) - 1u;
    const uint32_t n1 = __builtin_popcount(e.p0 & ~e.p1 & below);
    const uint32_t n2 = __builtin_popcount(~e.p0 & e.p1 & below);
    const uint32_t n3 = __builtin_popcount(e.p0 & e.p1 & below);
    const uint32_t n0 = j - n1 - n2 - n3;
    if (cls) *cls = ((e.p0 >> j) & 1u) | (((e.p1 >> j) & 1u) << 1);
    return e.base + (uint64_t)n0 * R[0] + (uint64_t)n1 * R[1] + (uint64_t)n2 * R[2] + (uint64_t)n3 * R[3];
}

}  // namespace cpk
