// cp_decode.hip - fused gather-and-decode of Conditional Program (CP) rows
// for CDNA4 (gfx950).
//
// For every id of a lookup batch the kernel fetches that row's record (a
// tail-biting trellis code and one bf16 scale), walks the shared trellis to
// rebuild f(c), multiplies by the scale and writes the row at the id's
// position in the batch. The pages describe exactly this fused step: only
// requested records are fetched, restored by one kernel and handed on in the
// original lookup order ("2비트 코드와 공유 트렐리스로 n-gram 룩업 테이블을
// 4~8배 압축한다", onedev.kr, sections "How it works" and "How it differs").
//
// Trellis reading (the pages name a tail-biting Gaussian HYB bitshift trellis
// without parameters): code = little-endian N-bit integer, N = kv * d / 2;
// step t reads the 16-bit window of the circular code ending at bit kv(t+1);
// h = s*s + s (mod 2^32), idx = (h >> 7) & 511, outputs 2t, 2t+1 =
// LUT[idx] (fp16 pair), sign bits flipped when bit 15 of s is set; the row
// is alpha * f rounded once to bf16 (nearest, ties to even).
//
// Work mapping (memory-bound gather + streaming write; no MFMA):
//   - a row is handled by d/8 lanes (a full wave64 at d = 512); lane l makes
//     outputs [8l, 8l+8): steps 4l .. 4l+3, one 16-byte store;
//   - lane l loads the 4kv code bits its steps introduce (one aligned dword
//     at kv = 4, two otherwise); the 16-kv older bits each window also needs
//     come from the neighbouring lane(s) through a lane shuffle, circular
//     within the row, which is exactly the tail-biting wrap;
//   - records are 2-byte aligned (R = kv*d/16 + 2 is even), so every load is
//     an aligned dword and bits are taken out with shifts;
//   - the 2 KB codebook is staged in LDS once per workgroup, replicated
//     COPIES times so that lane k reads copy k % COPIES, which spreads the
//     random codebook reads over more banks;
//   - a wave takes a chunk of consecutive lookups: one load brings all their
//     ids (one per lane), then every record of the chunk is requested before
//     any is decoded and the next chunk's ids are requested before decoding,
//     so a whole chunk of record loads is in flight per wave;
//   - the scale, the window hash and the fp16 -> fp32 widening run on the
//     scalar unit, v_mad_u32_u24 and v_fma_mix_f32 respectively;
//   - outputs are written with nontemporal stores: they are not re-read, and
//     keeping them out of the caches leaves room for hot (Zipf) records.
#include <type_traits>

#include "cp_internal.h"

// Launch-shape knobs (overridable at build time for tuning).
#ifndef CPK_COPIES
#define CPK_COPIES 16
#endif
#ifndef CPK_BLOCK
#define CPK_BLOCK 1024
#endif
#ifndef CPK_NT_STORE
#define CPK_NT_STORE 1
#endif
#ifndef CPK_FMA_MIX
#define CPK_FMA_MIX 1
#endif
#ifndef CPK_BLOCKS_PER_CU
#define CPK_BLOCKS_PER_CU 0
#endif
#ifndef CPK_CHUNK
#define CPK_CHUNK 16
#endif


namespace cpk {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// 64-bit value of lane `lane` (wave-uniform result). The builtin works on
// int; both halves go through uint32_t so the low half is not sign-extended.
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, uint32_t lane)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, (int)lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), (int)lane);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint32_t ld32(const uint8_t *p)
{
    return *reinterpret_cast<const uint32_t *>(p);
}

// alpha * (fp16 half of e) in one v_fma_mix_f32: the half is widened exactly,
// the product of a bf16 and an fp16 is exact in fp32, and adding -0 leaves
// every product (signed zeros included) unchanged.
__device__ __forceinline__ float mix_lo(uint32_t e, float a, float negz)
{
    float r;
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(e), "v"(a), "v"(negz));
    return r;
}

__device__ __forceinline__ float mix_hi(uint32_t e, float a, float negz)
{
    float r;
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(e), "v"(a), "v"(negz));
    return r;
}

// The same with the scale in an SGPR (uniform per row when a row fills the
// wave), which saves moving it into a VGPR for every row.
__device__ __forceinline__ float mix_lo_s(uint32_t e, float a, float negz)
{
    float r;
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(e), "s"(a), "v"(negz));
    return r;
}

__device__ __forceinline__ float mix_hi_s(uint32_t e, float a, float negz)
{
    float r;
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(e), "s"(a), "v"(negz));
    return r;
}

// One output pair: e = LUT entry (fp16 lo = element 2t, hi = element 2t+1),
// negmask = 0x80008000 when the window's bit 15 is set. Scaled: bf16 pair of
// alpha * value, rounded to nearest even; that rounding is symmetric in sign,
// so the sign flip can be applied to the packed result.
template <bool RAW, bool SALPHA = false>
__device__ __forceinline__ uint32_t emit_pair(uint32_t e, uint32_t negmask, float alpha)
{
    if constexpr (RAW) {
        return e ^ negmask;
    } else {
        f32x2 v;
#if CPK_FMA_MIX
        const float negz = __builtin_bit_cast(float, 0x80000000u);
        if constexpr (SALPHA) {
            v.x = mix_lo_s(e, alpha, negz);
            v.y = mix_hi_s(e, alpha, negz);
        } else {
            v.x = mix_lo(e, alpha, negz);
            v.y = mix_hi(e, alpha, negz);
        }
#else
        v.x = alpha * (float)__builtin_bit_cast(_Float16, (uint16_t)(e & 0xFFFFu));
        v.y = alpha * (float)__builtin_bit_cast(_Float16, (uint16_t)(e >> 16));
#endif
        bf16x2 b = __builtin_convertvector(v, bf16x2);
        return __builtin_bit_cast(uint32_t, b) ^ negmask;
    }
}

// h = x*x + x (mod 2^32) on the low 24 bits of x. Bits 7..15 of h, the only
// bits the output rule reads, depend on bits 0..15 of x alone (the higher
// bits only add multiples of 2^16), so x may carry the following code bits.
__device__ __forceinline__ uint32_t hash_mad(uint32_t x)
{
    uint32_t h;
    asm("v_mad_u32_u24 %0, %1, %1, %1" : "=v"(h) : "v"(x));
    return h;
}

// (a & mask) | b in one v_and_or_b32 (kept as written: the compiler otherwise
// reassociates the LDS address into more instructions).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t b)
{
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(b));
    return r;
}

// Code bits a lane needs for its 4 windows: 16 + 3kv; they fit in 32 bits up
// to kv = 5.
template <int KV>
using field_t = typename std::conditional<(16 + 3 * KV <= 32), uint32_t, uint64_t>::type;

// Decodes one row's 8 outputs of this lane from `newbits` (the lane's 4kv
// new code bits) and the row's scale, and returns them packed (4 dwords).
template <int D, int KV, bool RAW, int COPIES, bool SALPHA>
__device__ __forceinline__ u32x4 decode_lane(uint32_t newbits, uint32_t alpha_bits, uint32_t l, uint32_t g,
                                             const uint32_t *s_lut, uint32_t lds_off)
{
    constexpr int LANES = D / 8;
    constexpr int M = 16 - KV;
    constexpr int NEWB = 4 * KV;
    using F = field_t<KV>;
    // older bits from the previous lane(s) of the same row; lane 0 takes them
    // from the last lane: the circular (tail-biting) wrap
    uint32_t prev;
    if constexpr (LANES == 64)
        prev = __builtin_amdgcn_update_dpp(newbits, newbits, 0x13C /* wave_ror:1 */, 0xF, 0xF, false);
    else
        prev = __shfl(newbits, (int)(g * LANES + (l + LANES - 1) % LANES), 64);
    F hist;
    if constexpr (NEWB < M) {
        // kv = 3: 13 history bits span the two previous lanes
        const uint32_t prev2 = __shfl(newbits, (int)(g * LANES + (l + LANES - 2) % LANES), 64);
        hist = (F)((((uint64_t)prev << NEWB) | prev2) >> (2 * NEWB - M));
    } else {
        hist = (F)(prev >> (NEWB - M));
    }
    const F field = ((F)newbits << M) | hist;  // bit 0 = code bit NEWB*l - M
    const float alpha = __builtin_bit_cast(float, alpha_bits);
    u32x4 v;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t x = (uint32_t)(field >> (KV * k));  // low 16 bits: window s_t
        const uint32_t h = hash_mad(x);
        // LDS block of entry idx = (h >> 7) & 511 starts at byte idx * 128,
        // i.e. h & 0xFF80; bit 15 of the window (the sign) picks the negated
        // half (+64 bytes); the lane picks one of the 16 copies
        const uint32_t e = *reinterpret_cast<const uint32_t *>(
            reinterpret_cast<const char *>(s_lut) + and_or(h, 0xFF80u, and_or(x >> 9, 0x40u, lds_off)));
        v[k] = emit_pair<RAW, SALPHA>(e, 0u, alpha);
    }
    return v;
}

__device__ __forceinline__ void store16(uint32_t *dst, u32x4 v)
{
#if CPK_NT_STORE
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(dst));
#else
    *reinterpret_cast<u32x4 *>(dst) = v;
#endif
}

template <int D, int KV, bool RAW, int COPIES, int BLOCK, int CHUNK>
__global__ __launch_bounds__(BLOCK) void gather_decode(const uint8_t *__restrict__ tab, const uint64_t rows,
                                                       const uint32_t *__restrict__ lut,
                                                       const int64_t *__restrict__ ids, const uint64_t n,
                                                       uint32_t *__restrict__ out, int *__restrict__ err,
                                                       const bool by_offset)
{
    constexpr int LANES = D / 8;        // lanes per row
    constexpr int GROUPS = 64 / LANES;  // rows decoded side by side in a wave
    constexpr int NB = KV * D / 16;     // code bytes per record
    constexpr int R = NB + 2;           // record bytes
    constexpr int NEWB = 4 * KV;        // code bits introduced by one lane's 4 steps
    constexpr int WAVES = BLOCK / 64;
    constexpr int CI = CHUNK / GROUPS;  // rows per lane group per chunk
    static_assert(LANES >= 2 && LANES <= 64 && (LANES & (LANES - 1)) == 0, "d/8 lanes");
    static_assert((KV * D) % 64 == 0, "code must be whole dwords");
    static_assert(NEWB <= 32 && 2 * NEWB >= 16 - KV, "history within two lanes");
    static_assert(COPIES == 16, "the LDS layout holds 16 copies per sign");
    static_assert(CHUNK <= 64 && CI >= 1 && CI * GROUPS == CHUNK, "one id per lane per chunk");

    // codebook in LDS: per entry a 128-byte block of 16 copies of the fp16
    // pair followed by 16 copies of its negation (both sign bits flipped)
    __shared__ __attribute__((aligned(16))) uint32_t s_lut[512 * 32];
    for (int u = threadIdx.x; u < 4096; u += BLOCK) {
        // 16-byte unit u holds 4 copies of entry u >> 3, negated when bit 2 of
        // u is set; consecutive lanes write consecutive units (no bank conflicts)
        const uint32_t v = lut[u >> 3] ^ ((u & 4) ? 0x80008000u : 0u);
        reinterpret_cast<u32x4 *>(s_lut)[u] = (u32x4){v, v, v, v};
    }
    __syncthreads();

    const uint32_t lane = threadIdx.x & 63;
    const uint32_t l = lane % LANES;
    const uint32_t g = lane / LANES;
    const uint32_t lds_off = (lane & 15u) * 4u;
    // wave index made provably uniform so that per-row values of a one-row
    // wave (d = 512) stay scalar
    const uint64_t wave =
        (uint64_t)blockIdx.x * WAVES + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint64_t waves = (uint64_t)gridDim.x * WAVES;
    const uint64_t nchunks = (n + CHUNK - 1) / CHUNK;
    bool bad = false;

    // A wave takes chunks of CHUNK consecutive lookups. Lane k loads the id of
    // the chunk's row k and works out, once for the whole chunk, whether it is
    // valid and where its record starts; rows then read those from lane k.
    // Every record of a chunk is requested before any is decoded, and the next
    // chunk's ids before the decoding starts.
    // row index of row i of chunk c (a wave writes its chunk's rows as one
    // contiguous run of output)
    auto row_of = [&](uint64_t c, uint32_t i) -> uint64_t { return c * CHUNK + i; };
    auto load_id = [&](uint64_t c) -> int64_t {
        const uint64_t j = row_of(c, lane);
        return (c < nchunks && lane < CHUNK && j < n) ? ids[j] : 0;
    };
    int64_t my_id = load_id(wave);
    for (uint64_t c = wave; c < nchunks; c += waves) {
        // rows in this chunk
        uint32_t cn = __builtin_amdgcn_readfirstlane((uint32_t)((n - c * CHUNK) < CHUNK ? (n - c * CHUNK) : CHUNK));
        // opaque to the optimiser so that the per-row checks stay 32-bit scalar
        asm volatile("" : "+s"(cn));
        const bool in = lane < cn;
        // a row id in [0, rows) (negative ids wrap above rows), or with
        // by_offset a record's byte offset in a staging area (-1: invalid)
        const bool ok = in && (by_offset ? my_id >= 0 : (uint64_t)my_id < rows);
        bad |= in && !ok;
        const uint64_t my_off = !ok ? 0 : by_offset ? (uint64_t)my_id : (uint64_t)my_id * R;  // even
        const uint64_t okmask = __ballot(ok);
        my_id = load_id(c + waves);

        if constexpr (GROUPS == 1) {
            // d = 512: one row at a time across the whole wave; the row's
            // record offset is uniform (scalar), the scale comes by a scalar load
            uint32_t nb[CI], ab[CI];
#pragma unroll
            for (int i = 0; i < CI; ++i) {
                const uint64_t o = readlane_u64(my_off, (uint32_t)i);
                const uint8_t *rec = tab + o;
                if constexpr (KV == 4) {
                    // lane l's 16 new bits are code half-word l (records are 2-byte aligned)
                    nb[i] = *reinterpret_cast<const uint16_t *>(rec + 2u * l);
                } else {
                    const uint64_t bit = o * 8 + (uint64_t)NEWB * l;
                    const uint8_t *p = tab + ((bit >> 5) << 2);
                    const uint64_t both = ((uint64_t)ld32(p + 4) << 32) | ld32(p);
                    nb[i] = (uint32_t)(both >> (bit & 31)) & ((1u << NEWB) - 1u);
                }
                const uint64_t ao = o + NB;  // scale: bf16 at bytes [NB, NB + 2)
                const uint32_t adw = ld32(tab + (ao & ~(uint64_t)3));
                ab[i] = ((adw >> ((ao & 2) << 3)) & 0xFFFFu) << 16;
            }
#pragma unroll
            for (int i = 0; i < CI; ++i) {
                // every row is decoded (an invalid id reads record 0), so the
                // loads above stay ahead of their uses
                const u32x4 v = decode_lane<D, KV, RAW, COPIES, true>(nb[i], ab[i], l, g, s_lut, lds_off);
                if ((uint32_t)i < cn) store16(out + row_of(c, i) * (D / 2) + 4u * l, v);
            }
        } else {
            // several rows side by side: group g decodes rows g*CI .. g*CI+CI-1
            uint32_t nb[CI], ab[CI];
#pragma unroll
            for (int i = 0; i < CI; ++i) {
                const int r = (int)(g * CI + i);
                const uint64_t o = __shfl(my_off, r, 64);
                if constexpr (KV == 4) {
                    nb[i] = *reinterpret_cast<const uint16_t *>(tab + o + 2u * l);
                } else {
                    const uint64_t bit = o * 8 + (uint64_t)NEWB * l;
                    const uint8_t *p = tab + ((bit >> 5) << 2);
                    const uint64_t both = ((uint64_t)ld32(p + 4) << 32) | ld32(p);
                    nb[i] = (uint32_t)(both >> (bit & 31)) & ((1u << NEWB) - 1u);
                }
                const uint64_t ao = o + NB;
                const uint32_t adw = ld32(tab + (ao & ~(uint64_t)3));
                ab[i] = ((adw >> ((ao & 2) << 3)) & 0xFFFFu) << 16;
            }
#pragma unroll
            for (int i = 0; i < CI; ++i) {
                const uint32_t r = g * CI + i;
                const u32x4 v = decode_lane<D, KV, RAW, COPIES, false>(nb[i], ab[i], l, g, s_lut, lds_off);
                if (r < cn) store16(out + row_of(c, r) * (D / 2) + 4u * l, v);
            }
        }
        // Rows with an id outside the table were decoded from record 0 above;
        // overwrite them with zeros. Rare, so kept off the main path; the wait
        // orders the two stores to the same address.
        const uint64_t badmask = __ballot(in) & ~okmask;
        if (badmask) {
            __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
            for (int i = 0; i < CI; ++i) {
                const uint32_t r = g * CI + i;
                if ((badmask >> r) & 1u)
                    store16(out + row_of(c, r) * (D / 2) + 4u * l, (u32x4){0u, 0u, 0u, 0u});
            }
        }
    }
    if (bad) atomicOr(err, 1);
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------

// Launch shape (measured on MI355X, d = 512 replay): the codebook in LDS as
// 16 copies x 2 signs (64 KB) in 1024-thread workgroups (2 per CU = 32
// waves); one wave
// holds a chunk of 16 lookups; the grid covers all chunks (no persistent cap),
// which balances the tail better than a fixed number of workgroups per CU.
template <int D, int KV>
struct Tune {
    static constexpr int COPIES = CPK_COPIES;
    static constexpr int BLOCK = CPK_BLOCK;
    static constexpr int BLOCKS_PER_CU = CPK_BLOCKS_PER_CU;
    static constexpr int CHUNK = CPK_CHUNK;
};

template <int D, int KV, bool RAW>
static hipError_t launch_one(const LaunchArgs &a)
{
    using T = Tune<D, KV>;
    constexpr int GROUPS = 64 / (D / 8);
    // lookups per wave chunk: a multiple of the rows decoded side by side, <= 64
    constexpr int CHUNK = (T::CHUNK / GROUPS > 0 ? T::CHUNK / GROUPS : 1) * GROUPS;
    const uint64_t nchunks = (a.n + CHUNK - 1) / CHUNK;
    uint64_t blocks = (nchunks + T::BLOCK / 64 - 1) / (T::BLOCK / 64);
    if (T::BLOCKS_PER_CU > 0) {  // persistent grid: at most this many workgroups per CU
        const uint64_t cap = (uint64_t)T::BLOCKS_PER_CU * (a.num_cus > 0 ? a.num_cus : 256);
        if (blocks > cap) blocks = cap;
    }
    hipLaunchKernelGGL((gather_decode<D, KV, RAW, T::COPIES, T::BLOCK, CHUNK>), dim3((unsigned)blocks),
                       dim3(T::BLOCK), 0, a.stream, a.records, a.rows, a.lut, a.ids, a.n, a.out, a.err,
                       a.by_offset);
    return hipGetLastError();
}

typedef hipError_t (*launch_fn)(const LaunchArgs &);

struct Entry {
    uint32_t d, kv;
    launch_fn scaled, raw;
};

#define CPK_ENTRY(D, KV) {D, KV, &launch_one<D, KV, false>, &launch_one<D, KV, true>}

static const Entry kTable[] = {
    CPK_ENTRY(64, 3),  CPK_ENTRY(64, 4),  CPK_ENTRY(64, 5),  CPK_ENTRY(64, 6),
    CPK_ENTRY(128, 3), CPK_ENTRY(128, 4), CPK_ENTRY(128, 5), CPK_ENTRY(128, 6),
    CPK_ENTRY(256, 3), CPK_ENTRY(256, 4), CPK_ENTRY(256, 5), CPK_ENTRY(256, 6),
    CPK_ENTRY(512, 3), CPK_ENTRY(512, 4), CPK_ENTRY(512, 5), CPK_ENTRY(512, 6),
};

static const Entry *find(uint32_t d, uint32_t kv)
{
    for (const Entry &e : kTable)
        if (e.d == d && e.kv == kv) return &e;
    return nullptr;
}

bool supported(uint32_t d, uint32_t kv) { return find(d, kv) != nullptr; }

hipError_t launch(uint32_t d, uint32_t kv, bool raw, const LaunchArgs &a)
{
    const Entry *e = find(d, kv);
    if (!e) return hipErrorInvalidValue;
    return raw ? e->raw(a) : e->scaled(a);
}

}  // namespace cpk
