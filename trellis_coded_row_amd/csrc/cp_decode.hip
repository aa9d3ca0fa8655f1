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
//   - lane l loads the 4kv code bits its steps introduce (at kv = 4 one
//     16-bit load of code half-word l, otherwise the two aligned dwords that
//     cover them); the 16-kv older bits each window also needs come from the
//     neighbouring lane(s) through a lane shuffle (DPP rotation at d = 512),
//     circular within the row, which is exactly the tail-biting wrap;
//   - records are only 2-byte aligned (R = kv*d/16 + 2 is even), so loads
//     are half-words or aligned dwords and bits are taken out with shifts;
//   - the 2 KB codebook is staged in LDS once per workgroup, replicated
//     COPIES times so that lane k reads copy k % COPIES, which spreads the
//     random codebook reads over more banks;
//   - a wave takes a chunk of consecutive lookups: one load brings all their
//     ids (one per lane), then every record of the chunk is requested before
//     any is decoded and the next chunk's ids are requested before decoding,
//     so a whole chunk of record loads is in flight per wave; chunks hold 16
//     lookups for batches that fill the chip, and 4 or 1 for smaller ones;
//   - the scale of a one-row wave (d = 512) comes by a scalar load and stays
//     in an SGPR; the window hash is one v_mad_u32_u24, and the fp16 -> fp32
//     widening and the scaling are one v_fma_mix_f32 per output;
//   - outputs are written with nontemporal stores: they are not re-read, and
//     keeping them out of the caches leaves room for hot (Zipf) records.
#include "cp_lane.h"

namespace cpk {

// With HOT, some rows' records also sit in a device-memory copy (a cache of
// looked-up-often rows of a table in pinned host memory): hot_index holds per
// block of 32 rows the cache slot of its first hot row and a bitmap of its hot
// rows, so hot row 32b + j is slot base + popcount(bits below j). Offsets are
// then taken from `tab` = the lower of the two regions' addresses, the host
// records starting at host_off0 and the cache at hot_off0.
template <int D, int KV, bool RAW, int COPIES, int BLOCK, int CHUNK, bool HOT, bool AHEAD>
__global__ __launch_bounds__(BLOCK) void gather_decode(const uint8_t *__restrict__ tab, const uint64_t rows,
                                                       const uint32_t *__restrict__ lut,
                                                       const int64_t *__restrict__ ids, const uint64_t n,
                                                       uint32_t *__restrict__ out, int *__restrict__ err,
                                                       const bool by_offset, const HotEntry *__restrict__ hot_index,
                                                       const uint64_t host_off0, const uint64_t hot_off0,
                                                       const uint32_t gen)
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

    __shared__ __attribute__((aligned(16))) uint32_t s_lut[kLdsLutWords];

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
    // the first chunk's ids are requested before the codebook is staged, so
    // the two loads' latencies overlap (what a small batch waits for)
    int64_t my_id = load_id(wave);
    // Workgroups of the first residency round (blockIdx < gen: the
    // workgroups one CU holds, times the CUs) also read the ids, and touch
    // the record lines, of the chunks
    // that workgroups gen, 2 gen, ... later take with the same wave index (up
    // to kPrefetchRounds rounds). Those run on the same XCD (workgroups are
    // dealt to the XCDs in turn, and gen is a multiple of their count), so
    // their id and record reads find the lines in the caches: uncached records
    // come from HBM in one burst at the start, before the output stream is
    // under way, instead of one round of misses after another while it is.
    // The loaded words are only kept alive.
    uint32_t touched = 0;
    const bool pf_wave = AHEAD && blockIdx.x < gen && gridDim.x > gen;
    const uint64_t pf_step = (uint64_t)gen * WAVES;
    int64_t pid[kPrefetchRounds];
    if constexpr (AHEAD) {
        if (pf_wave) {
#pragma unroll
            for (int k = 0; k < kPrefetchRounds; ++k) pid[k] = load_id(wave + (uint64_t)(k + 1) * pf_step);
        }
    }
    // The touches, issued right after this wave's own record loads: loads
    // complete in order, so the wave's own decode never waits for them
    // (issued before, they held up the first round's own work).
    auto touch_later = [&]() {
        if constexpr (AHEAD) {
            if (pf_wave) {
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int k = 0; k < kPrefetchRounds; ++k) {
                    const uint64_t pc = wave + (uint64_t)(k + 1) * pf_step;
                    if (pc >= nchunks) break;
                    const uint64_t rid = (uint64_t)pid[k];
                    const uint64_t off = by_offset ? ((int64_t)rid >= 0 ? rid : 0) : (rid < rows ? rid * R : 0);
                    // lane l touches 64-byte segment l % 4 of the record of chunk row l / 4
                    const uint64_t o = __shfl(off, (int)(lane >> 2), 64);
                    const uint64_t seg = (o & ~(uint64_t)63) + 64u * (lane & 3u);
                    if ((lane >> 2) < (uint32_t)CHUNK && seg < o + R) touched ^= ld32(tab + seg);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    bool first_chunk = true;
    stage_lut<BLOCK>(s_lut, lut);
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
        uint64_t my_off;
        if constexpr (HOT) {
            // an invalid id reads the first host record (its row is zeroed below)
            const uint64_t rid = ok ? (uint64_t)my_id : 0;
            const HotEntry h = hot_index[rid >> 5];
            const uint32_t j = (uint32_t)rid & 31u;
            my_off = ((h.bits >> j) & 1u)
                         ? hot_off0 + (uint64_t)(h.base + __builtin_popcount(h.bits & ((1u << j) - 1u))) * R
                         : host_off0 + rid * R;
        } else {
            my_off = !ok ? 0 : by_offset ? (uint64_t)my_id : (uint64_t)my_id * R;  // even
        }
        const uint64_t okmask = __ballot(ok);
        my_id = load_id(c + waves);

        // Code bits of lane l, and the scale (fp32 bits), of the record at
        // byte offset o.
        auto row_bits = [&](uint64_t o) -> uint32_t {
            if constexpr (KV == 4) {
                // lane l's 16 new bits are code half-word l (records are 2-byte aligned)
                return *reinterpret_cast<const uint16_t *>(tab + o + 2u * l);
            } else {
                // the two aligned dwords that hold lane l's bits: a base that
                // is uniform when o is (d = 512) plus a small per-lane offset,
                // so the loads take a scalar base and a 32-bit lane offset
                const uint8_t *base = tab + (o & ~(uint64_t)3);
                const uint32_t bit = (uint32_t)(o & 3u) * 8u + NEWB * l;
                const uint8_t *p = base + ((bit >> 5) << 2);
                const uint64_t both = ((uint64_t)ld32(p + 4) << 32) | ld32(p);
                return (uint32_t)(both >> (bit & 31)) & ((1u << NEWB) - 1u);
            }
        };
        auto row_scale = [&](uint64_t o) -> uint32_t {
            const uint64_t ao = o + NB;  // bf16 at bytes [NB, NB + 2)
            const uint32_t adw = ld32(tab + (ao & ~(uint64_t)3));
            return ((adw >> ((ao & 2) << 3)) & 0xFFFFu) << 16;
        };
        // record offset of the row that lane group g decodes i-th in the chunk
        auto row_offset = [&](uint32_t i) -> uint64_t {
            if constexpr (GROUPS == 1) return readlane_u64(my_off, i);
            else return __shfl(my_off, (int)(i * GROUPS + g), 64);
        };
        // smallest exponent field (in place) among the chunk's scales; the
        // rows past the chunk's end, which decode record 0, may count too
        uint32_t amin = 0x7F800000u;

        if constexpr (GROUPS == 1) {
            // d = 512: one row at a time across the whole wave; the row's
            // record offset is uniform (scalar), the scale comes by a scalar load
            uint32_t nb[CI], ab[CI];
#pragma unroll
            for (int i = 0; i < CI; ++i) {
                const uint64_t o = row_offset((uint32_t)i);
                nb[i] = row_bits(o);
                ab[i] = row_scale(o);
            }
            if (first_chunk) touch_later();
#pragma unroll
            for (int i = 0; i < CI; ++i) {
                // every row is decoded (an invalid id reads record 0), so the
                // loads above stay ahead of their uses
                const u32x4 v = decode_lane<D, KV, RAW ? kRaw : kScaled, COPIES, true>(nb[i], ab[i], l, g, s_lut,
                                                                                        lds_off);
                if ((uint32_t)i < cn) store16(out + row_of(c, i) * (D / 2) + 4u * l, v);
                if constexpr (!RAW) {
                    amin = __builtin_elementwise_min(amin, ab[i] & 0x7F800000u);
                    // taken here, so the row's scale register is free afterwards
                    asm volatile("" : "+s"(amin));
                }
            }
        } else {
            // several rows side by side: group g decodes rows g, g + GROUPS, ...
            // of the chunk, so each store instruction writes GROUPS adjacent
            // rows (1 KB contiguous) rather than GROUPS separate pieces
            uint32_t nb[CI], ab[CI];
#pragma unroll
            for (int i = 0; i < CI; ++i) {
                const uint64_t o = row_offset((uint32_t)i);
                nb[i] = row_bits(o);
                ab[i] = row_scale(o);
            }
            if (first_chunk) touch_later();
#pragma unroll
            for (int i = 0; i < CI; ++i) {
                const uint32_t r = i * GROUPS + g;
                const u32x4 v = decode_lane<D, KV, RAW ? kRaw : kScaled, COPIES, false>(nb[i], ab[i], l, g, s_lut,
                                                                                         lds_off);
                if (r < cn) store16(out + row_of(c, r) * (D / 2) + 4u * l, v);
                if constexpr (!RAW) {
                    amin = __builtin_elementwise_min(amin, ab[i] & 0x7F800000u);
                    asm volatile("" : "+v"(amin));
                }
            }
        }
        // Rows whose scale is below 2^-102 went through the fast scaling
        // above, which can round twice when a product falls below 2^-126:
        // decode them again with the exact tiny-scale arithmetic. Rare (a row
        // norm that small), so kept off the main path like the bad-row pass
        // below; the wait orders the two stores to the same address, and the
        // bad-row pass comes after it (an invalid id decodes record 0, whose
        // scale may be tiny).
        if constexpr (!RAW) {
            if (__builtin_expect(__ballot(scale_is_tiny(amin)) != 0, 0)) {
                __builtin_amdgcn_s_waitcnt(0);
#pragma unroll 1
                for (uint32_t i = 0; i < (uint32_t)CI; ++i) {
                    const uint32_t r = i * GROUPS + g;
                    const uint64_t o = row_offset(i);
                    const uint32_t ab = row_scale(o);
                    const u32x4 v = decode_lane<D, KV, kTiny, COPIES, (GROUPS == 1)>(row_bits(o), ab, l, g, s_lut,
                                                                                      lds_off);
                    if (r < cn && scale_is_tiny(ab)) store16(out + row_of(c, r) * (D / 2) + 4u * l, v);
                }
            }
        }
        first_chunk = false;
        // Rows with an id outside the table were decoded from record 0 above;
        // overwrite them with zeros. Rare, so kept off the main path; the wait
        // orders the two stores to the same address.
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
    // the touched words count as used (no memory effect)
    if constexpr (AHEAD) asm volatile("" ::"v"(touched));
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------

// Launch shape (measured on MI355X, d = 512 replay): the codebook in LDS as
// 16 copies x 2 signs (64 KB); one wave holds a chunk of up to 16 lookups
// (fewer for small batches, lookup_chunk_rows); the grid covers all chunks
// (no persistent cap), which balances the tail better than a fixed number of
// workgroups per CU. A CU runs 16 waves: one 1024-thread workgroup, or two of
// 512 (the LDS holds two codebooks), which run out of step: one decodes and
// writes while the other waits for its records. Two of 512 are faster for the
// touch-ahead kernels (warm and cold: 72.6 / 79.0 against 73.1 / 80.2 us at
// kv 4, 69.3 / 76.7 against 75.7 / 86.8 at kv 3) and for the default kernels
// at kv 4 (69.2 against 69.9 us warm, cold the same; 35.2 against 38.0 at
// d = 256); one of 1024 for the default kernels at kv 3, 5 and 6 (cold 99-101
// against 107-109 us), the host-table kernels and the mixed-rate kernel.
template <int D, int KV, bool RAW, bool HOT, bool AHEAD, int CHUNK_ROWS>
static hipError_t launch_shape(const LaunchArgs &a)
{
    constexpr int GROUPS = 64 / (D / 8);
    // lookups per wave chunk: a multiple of the rows decoded side by side, <= 64
    constexpr int CHUNK = (CHUNK_ROWS / GROUPS > 0 ? CHUNK_ROWS / GROUPS : 1) * GROUPS;
    constexpr int BLOCK = (AHEAD || (KV == 4 && !HOT)) ? kBlockPair : kBlock;
    const uint64_t nchunks = (a.n + CHUNK - 1) / CHUNK;
    uint64_t blocks = (nchunks + BLOCK / 64 - 1) / (BLOCK / 64);
    if (blocks > 0x7FFFFFFFull) blocks = 0x7FFFFFFFull;  // the chunk loop strides over any excess
    // workgroups of one residency round
    const uint32_t gen = (uint32_t)(a.num_cus > 0 ? a.num_cus : 256) * (uint32_t)(kBlock / BLOCK);
    hipLaunchKernelGGL((gather_decode<D, KV, RAW, kCopies, BLOCK, CHUNK, HOT, AHEAD>), dim3((unsigned)blocks),
                       dim3(BLOCK), 0, a.stream, a.records, a.rows, a.lut, a.ids, a.n, a.out, a.err, a.by_offset,
                       a.hot_index, a.host_off0, a.hot_off0, gen);
    return hipGetLastError();
}

template <int D, int KV, bool RAW, bool HOT, bool AHEAD>
static hipError_t launch_chunked(const LaunchArgs &a)
{
    switch (lookup_chunk_rows(a.n, a.num_cus)) {
    case 1: return launch_shape<D, KV, RAW, HOT, AHEAD, 1>(a);
    case 4: return launch_shape<D, KV, RAW, HOT, AHEAD, 4>(a);
    default: return launch_shape<D, KV, RAW, HOT, AHEAD, kChunk>(a);
    }
}

// the table's residency and flags pick the variant: records partly in an HBM
// copy (HOT, pinned-host tables), touch-ahead (device tables), or plain
template <int D, int KV, bool RAW>
static hipError_t launch_one(const LaunchArgs &a)
{
    if (a.hot_index) return launch_chunked<D, KV, RAW, true, false>(a);
    if (a.touch_ahead) return launch_chunked<D, KV, RAW, false, true>(a);
    return launch_chunked<D, KV, RAW, false, false>(a);
}

typedef hipError_t (*launch_fn)(const LaunchArgs &);

struct Entry {
    uint32_t d, kv;
    launch_fn scaled, raw;
};

#define CP_ENTRY(D, KV) {D, KV, &launch_one<D, KV, false>, &launch_one<D, KV, true>}

static const Entry kTable[] = {
    CP_ENTRY(64, 3),  CP_ENTRY(64, 4),  CP_ENTRY(64, 5),  CP_ENTRY(64, 6),
    CP_ENTRY(128, 3), CP_ENTRY(128, 4), CP_ENTRY(128, 5), CP_ENTRY(128, 6),
    CP_ENTRY(256, 3), CP_ENTRY(256, 4), CP_ENTRY(256, 5), CP_ENTRY(256, 6),
    CP_ENTRY(512, 3), CP_ENTRY(512, 4), CP_ENTRY(512, 5), CP_ENTRY(512, 6),
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
