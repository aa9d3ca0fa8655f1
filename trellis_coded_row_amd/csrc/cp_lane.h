// cp_lane.h - per-lane decode helpers shared by the gather-decode kernels
// (cp_decode.hip: one rate per table; cp_mixed.hip: a rate per row).
// Device code for gfx950 only; included by .hip sources.
#pragma once

#include <type_traits>

#include "cp_internal.h"

namespace cpk {

// Launch shape of the gather-decode kernels (measured on MI355X, d = 512
// replay): the codebook in LDS as 16 copies per sign (64 KB), wave chunks of
// up to 16 lookups, workgroups of 1024 threads or, for the instances where
// that measured faster, two workgroups of 512 per CU (the LDS holds two
// codebooks; 16 waves per CU either way).
constexpr int kBlock = 1024;
constexpr int kBlockPair = 512;
constexpr int kCopies = 16;
constexpr int kChunk = 16;
// Residency rounds ahead whose chunks the first round touches (the replay of
// 393,216 lookups at d = 512 has 6 rounds on 256 CUs).
constexpr int kPrefetchRounds = 8;

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

// alpha * (fp16 half of e) in one v_fma_mix_f32: the half is widened exactly
// and the product is rounded once to fp32; adding -0 leaves every product
// (signed zeros included) unchanged. The product of a bf16 and an fp16 has at
// most 8 + 11 significant bits, so it is exact in fp32 whenever it is zero or
// at least 2^-126 in magnitude (see scale_is_tiny for the other case).
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

// What a decode writes: the raw f(c) (fp16), the scaled row (bf16, the fast
// path), or the scaled row computed for a tiny scale (scale_pair_tiny).
enum Emit { kRaw, kScaled, kTiny };

// One scaled output pair: e = signed codebook pair (fp16 lo = element 2t, hi =
// element 2t+1) -> the bf16 pair of alpha * value, each product formed in
// fp32 (exact unless the scale is tiny) and rounded once to nearest even by
// v_cvt_pk_bf16_f32.
template <bool SALPHA>
__device__ __forceinline__ uint32_t emit_scaled(uint32_t e, float alpha)
{
    const float negz = __builtin_bit_cast(float, 0x80000000u);
    f32x2 v;
    if constexpr (SALPHA) {
        v.x = mix_lo_s(e, alpha, negz);
        v.y = mix_hi_s(e, alpha, negz);
    } else {
        v.x = mix_lo(e, alpha, negz);
        v.y = mix_hi(e, alpha, negz);
    }
    const bf16x2 b = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, b);
}

// A scale below 2^-102 (fp32 bits of the bf16; zeros and bf16 subnormals
// included): with it a product with a nonzero fp16 (>= 2^-24 in magnitude)
// // can fall below 2^-126, where fp32 keeps fewer than the product's 19
// significant bits and the fp32 product followed by the bf16 rounding would
// round twice. The kernels decode such rows again with scale_pair_tiny in a
// rarely taken pass after the chunk's main stores.
__device__ __forceinline__ bool scale_is_tiny(uint32_t alpha_bits)
{
    return (alpha_bits & 0x7F800000u) < (25u << 23);
}

// bf16 bits of alpha * h, rounded once to nearest even, for a tiny scale
// (|alpha| < 2^-102) and a finite fp16 h. Done on a copy scaled by 2^64, where
// every operation is exact on normal floats, so the result does not depend on
// the float denormal modes except for widening h:
//   a2 = |alpha| * 2^64, built from the bits (exact; a bf16 subnormal alpha is
//        its integer significand times 2^-85);
//   p  = h * a2, exact (normal or zero: 2^-93 <= |p| < 2^-22);
//   |alpha * h| = |p| * 2^-64 is a bf16 normal when |p| >= 2^-62: round |p| to
//        bf16 and lower its exponent by 64; otherwise it lies below 2^-126,
//        where bf16 steps are 2^-133: round |p| * 2^69 (< 2^7) to an integer
//        with ties to even by adding and removing 2^23, and that integer is
//        the bf16 pattern (128 is the smallest normal, 0x0080).
__device__ __forceinline__ uint32_t scale_half_tiny(uint32_t h16, uint32_t alpha_bits)
{
    const uint32_t mag = alpha_bits & 0x7FFFFFFFu;
    const float a2 = (mag >> 23) ? __builtin_bit_cast(float, mag + (64u << 23))
                                 : (float)(mag & 0x7FFFFFu) * 0x1p-85f;
    const float p = (float)__builtin_bit_cast(_Float16, (uint16_t)h16) * a2;
    const uint32_t sign = ((__builtin_bit_cast(uint32_t, p) ^ alpha_bits) & 0x80000000u) >> 16;
    const float ap = __builtin_fabsf(p);
    uint32_t r;
    if (ap >= 0x1p-62f) {
        r = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)ap) - (64u << 7);
    } else {
        r = __builtin_bit_cast(uint32_t, ap * 0x1p69f + 0x1p23f) - 0x4B000000u;
    }
    return sign | r;
}

__device__ __forceinline__ uint32_t scale_pair_tiny(uint32_t e, uint32_t alpha_bits)
{
    return scale_half_tiny(e & 0xFFFFu, alpha_bits) | (scale_half_tiny(e >> 16, alpha_bits) << 16);
}

template <Emit MODE, bool SALPHA>
__device__ __forceinline__ uint32_t emit_pair(uint32_t e, float alpha, uint32_t alpha_bits)
{
    if constexpr (MODE == kRaw) return e;
    else if constexpr (MODE == kScaled) return emit_scaled<SALPHA>(e, alpha);
    else return scale_pair_tiny(e, alpha_bits);
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
template <int D, int KV, Emit MODE, int COPIES, bool SALPHA>
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
        v[k] = emit_pair<MODE, SALPHA>(e, alpha, alpha_bits);
    }
    return v;
}

// Codebook in LDS: per entry a 128-byte block of 16 copies of the fp16 pair
// followed by 16 copies of its negation (both sign bits flipped), 64 KB.
constexpr int kLdsLutWords = 512 * 32;

template <int BLOCK>
__device__ __forceinline__ void stage_lut(uint32_t *s_lut, const uint32_t *__restrict__ lut)
{
    for (int u = threadIdx.x; u < 4096; u += BLOCK) {
        // 16-byte unit u holds 4 copies of entry u >> 3, negated when bit 2 of
        // u is set; consecutive lanes write consecutive units (no bank conflicts)
        const uint32_t v = lut[u >> 3] ^ ((u & 4) ? 0x80008000u : 0u);
        reinterpret_cast<u32x4 *>(s_lut)[u] = (u32x4){v, v, v, v};
    }
    __syncthreads();
}

// The 4kv new code bits of lane l of the record at byte offset o, for any kv
// (two aligned dword loads; records are 2-byte aligned).
__device__ __forceinline__ uint32_t lane_bits(const uint8_t *__restrict__ tab, uint64_t o, uint32_t newb,
                                              uint32_t l)
{
    // a base that is uniform when o is (d = 512) plus a small lane offset
    const uint8_t *base = tab + (o & ~(uint64_t)3);
    const uint32_t bit = (uint32_t)(o & 3u) * 8u + newb * l;
    const uint8_t *p = base + ((bit >> 5) << 2);
    const uint64_t both = ((uint64_t)ld32(p + 4) << 32) | ld32(p);
    return (uint32_t)(both >> (bit & 31)) & ((1u << newb) - 1u);
}

// The scale of the record at byte offset o with nb code bytes, as fp32 bits.
__device__ __forceinline__ uint32_t scale_bits(const uint8_t *__restrict__ tab, uint64_t o, uint32_t nb)
{
    const uint64_t ao = o + nb;  // bf16 at bytes [nb, nb + 2)
    const uint32_t adw = ld32(tab + (ao & ~(uint64_t)3));
    return ((adw >> ((ao & 2) << 3)) & 0xFFFFu) << 16;
}

// Output rows are written once and not read back by the kernel: nontemporal
// stores keep them from evicting hot records from the caches.
__device__ __forceinline__ void store16(uint32_t *dst, u32x4 v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(dst));
}

}  // namespace cpk
