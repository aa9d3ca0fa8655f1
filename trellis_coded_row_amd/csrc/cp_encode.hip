// cp_encode.hip - trellis-coded quantisation (TCQ) of table rows on the GPU.
//
// Produces the records the lookup path decodes: row e_i -> {c_i, alpha_i}
// (Conditional Program digest on onedev.kr, sections "How it works" and "How
// it differs"):
//   - z = sqrt(d) e / ||e||, the magnitude split off the content;
//   - c = the tail-biting path through the Gaussian HYB bitshift trellis that
//     the search below picks for all d coordinates jointly, no rotation;
//   - alpha = ||e|| / ||f(c)||, the norm-restoring scale, stored as bf16.
// Trellis reading as in the decoder: the window of step t is bits
// [kv(t+1)-16, kv(t+1)) of the circular code; its output pair is
// +-LUT[((s*s + s) >> 7) & 511], negated when bit 15 of the window is set.
//
// Search (two-pass tail-biting heuristic). A memory is the M = 16 - kv oldest
// bits of the next window. From memory m the kv new bits u form the window
// s = m | u << M and lead to memory s >> kv; a next memory m2 therefore has
// the 2^kv predecessors (m2 << kv | r) mod 2^M. Pass A runs the Viterbi
// recursion from every memory at cost 0 over the steps rotated by T/2 and
// reads, on the best path, the memory W held at the original start; pass B
// runs it from W alone, and the path of pass B that ends in W is the code.
//
// Arithmetic: fp64, one rounding per operation, in a fixed order (no fused
// multiply-add; sums in index order; an add-compare-select keeps the smallest
// r among equal metrics; the end memory is the smallest among equal metrics).
// The result is therefore one specific code, reproducible bit for bit.
//
// Layout on the GPU: one workgroup per row (1,024 threads at kv 3 and 4, 512
// at kv 5 and 6); path metrics of both time steps, the per-step branch costs, z and the codebook in LDS; the
// back-pointers (one byte per memory per step) in a caller workspace.
#pragma clang fp contract(off)

#include "cp_encode_copies.h"
#include "cp_internal.h"

#include <type_traits>

namespace cpk {

namespace {

constexpr uint32_t kMaxThreads = 1024;

__device__ __forceinline__ double half_to_double(uint32_t h16)
{
    return (double)(float)__builtin_bit_cast(_Float16, (uint16_t)h16);
}

// Nearest bf16 (ties to even) of a double with a single rounding: truncate to
// float and set the lowest bit when inexact (round to odd keeps what the
// second rounding needs, float having 16 more significant bits than bf16),
// then round to nearest even at 8 significant bits.
__device__ __forceinline__ uint16_t bf16_rne(double x)
{
    if (x != x) return 0x7FC0;
    const float f = __double2float_rz(x);
    uint32_t b = __builtin_bit_cast(uint32_t, f);
    if ((double)f != x) b |= 1u;
    if ((b & 0x7F800000u) == 0x7F800000u) return (uint16_t)(b >> 16);
    return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

template <int KV>
struct Tcq {
    static constexpr uint32_t M = 16 - KV;             // memory bits
    static constexpr uint32_t S = 1u << M;             // memories
    static constexpr uint32_t BR = 1u << KV;           // predecessors (and successors) per group
    static constexpr uint32_t G = S / BR;              // groups sharing one predecessor set
    // threads per workgroup. At kv 5 and 6 a workgroup of 512 holds two next
    // memories per thread or more (so kv 6 can pair them, below) and two
    // workgroups share a CU; at kv 4 the LDS admits one workgroup either way
    // and 1,024 threads hide more latency; kv 3 with 512 threads would need
    // 16 next memories per thread, more than a group's 8. Measured on 4,096 rows at
    // d = 512 (ms with 1,024 / 512 threads): kv 4: 31.4 / 35.1; kv 5: 30.7 /
    // 26.0; kv 6: 37.1 (unpaired) / 26.8.
    static constexpr uint32_t NT = KV >= 5 ? 512 : kMaxThreads;
    static constexpr uint32_t IPT = S / NT;            // next memories per thread
    static constexpr uint32_t TPG = BR / IPT;          // threads per group
    // Path-metric storage. A thread reads the BR metrics (L << kv) | r of
    // its group L, consecutive lanes taking consecutive groups. At kv >= 4
    // each run of BR metrics is followed by two doubles of padding: a lane's
    // run then starts BR/2 + 1 (odd) 16-byte units after its neighbour's, so
    // 16 lanes' 16-byte loads of metric pairs fall on 16 different bank
    // groups. At kv 3 the LDS has room for one double per 16 metrics only.
    static constexpr uint32_t PAD_SHIFT = KV == 3 ? 4 : KV;
    static constexpr uint32_t PAD_UNITS = KV == 3 ? 1 : 2;
    static constexpr uint32_t SP = S + (S >> PAD_SHIFT) * PAD_UNITS;  // padded metric array length
    static __device__ __forceinline__ uint32_t pad(uint32_t m) { return m + (m >> PAD_SHIFT) * PAD_UNITS; }
    // When the padding period divides 2^(M - kv), the padded position of
    // next memory L | u << (M - kv) is pad(L) + u * USTRIDE: one register
    // per thread and a constant per successor.
    static constexpr bool LINEAR_NEXT = PAD_SHIFT <= M - KV;
    // Steps unrolled by two: at kv 6 the 64 gather addresses that this
    // hoists out of the step loop do not fit in the registers.
    static constexpr bool PARITY_UNROLL = KV <= 5;
    // The running best as a min (one instruction instead of two selects);
    // at kv 6 the compiler then runs out of registers.
    static constexpr bool MIN_SELECT = KV <= 5;
    // VALU instructions the scheduler places after each predecessor's cost
    // loads (a branch is four); measured on 4,096 rows of d = 512, ms with
    // 4 / 5 / 6 / 8 / 12 x IPT: kv 3: 30.9 / 31.1 / 31.1 / 31.3 / 31.2;
    // kv 4: 24.2 / 23.2 / 22.4 / 23.2 / 23.1; kv 5: 21.5 / 21.3 / 21.3 /
    // 21.5 / 21.5; kv 6: 26.5 / 26.6 / 26.8 / 26.6 / 26.1.
    static constexpr uint32_t SCHED_VALU = (KV == 4 || KV == 5 ? 6 : KV == 6 ? 12 : 4) * IPT;
    static constexpr uint32_t USTRIDE = LINEAR_NEXT ? (1u << (M - KV)) + (1u << (M - KV - PAD_SHIFT)) * PAD_UNITS : 0;
    // Copies of each branch cost. Copy c of the pair with key k sits at the
    // 16-byte unit unit(k, c), in bank group unit mod 16 (64 banks of 4
    // bytes). The LDS serves a wave's 16-byte loads in four cycles of 16
    // lanes (lanes sharing l >> 5 and the parity of bits 2..4 of l), one
    // more cycle for every further unit in a bank group. Each thread reads,
    // for each of its gathers, the copy that a fixed table (kEncodeCopies4
    // and 5, generated offline by a bipartite matching per 16 such lanes:
    // the keys a thread gathers depend only on the thread) assigns it: 1.19
    // cycles per 16 lanes at kv 4 where one fixed copy per lane (copy = lane
    // mod CC, copies side by side) takes 1.88; 1.75 where 1.88 at kv 5. kv 3
    // has no LDS left for a second copy, kv 6 no registers.
    static constexpr uint32_t CC = KV == 4 ? 4 : KV == 5 ? 2 : 1;
    static constexpr uint32_t CBITS = CC == 4 ? 2 : CC == 2 ? 1 : 0;  // bits per table entry
    static __device__ __forceinline__ uint32_t unit(uint32_t k, uint32_t c)
    {
        // four copies in the bank groups k .. k + 3; else side by side
        if constexpr (CC == 4) return 16u * (CC * (k >> 4) + c) + ((k + c) & 15u);
        else return CC * k + c;
    }
    // this thread's copy choices, CBITS bits per gather q = r * H + j
    static __device__ __forceinline__ uint64_t copies(uint32_t tid)
    {
        if constexpr (KV == 4) return kEncodeCopies4[tid];
        else if constexpr (KV == 5) return kEncodeCopies5[tid];
        else return 0;
    }
    // The windows s and s ^ 0x8000 hash to idx and idx ^ 256 (adding 2^15 to
    // s flips bit 15 of s*s + s and changes only higher bits otherwise) and
    // carry opposite signs, so both branch costs share the key
    // idx ^ (sign << 8). With the costs stored by key (the sign in the low
    // position) one 16-byte load fetches the pair. A thread holds its
    // successors in such pairs, u and u + BR/2, which needs IPT >= 2.
    static constexpr uint32_t H = IPT / 2;             // cost loads per predecessor
    static_assert(IPT >= 2 && TPG * G == NT && NT >= 512 && NT <= kMaxThreads, "thread mapping");

    // successor u of slot i of thread slot tq (tq = tid / G)
    static __device__ __forceinline__ uint32_t succ(uint32_t tq, uint32_t i)
    {
        return i < H ? tq * H + i : tq * H + (i - H) + BR / 2;
    }
};

template <int KV>
struct Shared {
    // branch costs of one step: copy c of the pair with key
    // k = idx ^ negated << 8 at doubles 2 unit(k, c) + negated. First in LDS: the gathers address both buffers from one
    // per-thread register, with the buffer's offset (below 64 KB) in the
    // instruction.
    alignas(16) double cost[2][1024 * Tcq<KV>::CC];
    alignas(16) double D[2][Tcq<KV>::SP];
    double z[512];
    uint32_t lut[512];
    uint8_t code[6 * 512 / 16 + 2];
    double red_v[kMaxThreads / 64];
    uint32_t red_i[kMaxThreads / 64];
    uint32_t W;
    double norm;
};

// cost of the pair g = +-LUT[idx]: (z0 - g0)^2 + (z1 - g1)^2, for every copy
// c, at 2 unit(idx ^ neg << 8, c) + neg; i = 2 idx + neg.
template <int KV>
__device__ __forceinline__ void fill_cost(double *cost, const uint32_t *lut, double z0, double z1, uint32_t i)
{
    const uint32_t e = lut[i >> 1];
    double g0 = half_to_double(e & 0xFFFFu), g1 = half_to_double(e >> 16);
    if (i & 1u) {
        g0 = -g0;
        g1 = -g1;
    }
    const double e0 = z0 - g0, e1 = z1 - g1;
    const double c = e0 * e0 + e1 * e1;
    const uint32_t key = (i >> 1) ^ ((i & 1u) << 8);
#pragma unroll
    for (uint32_t k = 0; k < Tcq<KV>::CC; ++k) cost[Tcq<KV>::unit(key, k) * 2 + (i & 1u)] = c;
}

template <int KV>
__device__ __forceinline__ void fill_costs(double *cost, const uint32_t *lut, double z0, double z1)
{
    // at kv 5 the entry addresses are recomputed every step (a few integer
    // operations): kept in registers across the step loop they spill
    uint32_t i0 = threadIdx.x;
    if constexpr (KV == 5) asm volatile("" : "+v"(i0));
#pragma unroll
    for (uint32_t i = i0; i < 1024; i += Tcq<KV>::NT)
        fill_cost<KV>(cost, lut, z0, z1, i);
}

// One store of a thread's IPT back-pointers (consecutive bytes).
template <uint32_t IPT>
__device__ __forceinline__ void store_bp(uint8_t *p, const uint32_t *br)
{
    if constexpr (IPT == 8) {
        uint64_t v = 0;
#pragma unroll
        for (uint32_t i = 0; i < 8; ++i) v |= (uint64_t)br[i] << (8 * i);
        *reinterpret_cast<uint64_t *>(p) = v;
    } else if constexpr (IPT == 4) {
        *reinterpret_cast<uint32_t *>(p) = br[0] | br[1] << 8 | br[2] << 16 | br[3] << 24;
    } else if constexpr (IPT == 2) {
        *reinterpret_cast<uint16_t *>(p) = (uint16_t)(br[0] | br[1] << 8);
    } else {
        *p = (uint8_t)br[0];
    }
}

// Thread mapping: thread tid serves group L = tid mod G (the next memories
// m2 = L | u << (M - kv) share the predecessors L << kv | r) and its IPT
// successors u = succ(tid / G, i), the pairs u, u + BR/2 for
// u = (tid / G) * IPT/2 + j. Consecutive lanes thus take consecutive groups,
// whose windows differ in their low bits, which spreads the branch cost
// gathers over the LDS banks (lanes sharing a group would read costs at
// indices that agree in their low bits). A thread stores the back-pointers
// of its IPT next memories as IPT consecutive bytes at tid * IPT; this is
// the position of next memory m2 within one step's S bytes.
template <int KV>
__device__ __forceinline__ uint32_t bp_pos(uint32_t m2)
{
    using P = Tcq<KV>;
    const uint32_t L = m2 & (P::G - 1), u = m2 >> (P::M - KV);
    const uint32_t lo = u & (P::BR / 2 - 1);
    return ((lo / P::H) * P::G + L) * P::IPT + lo % P::H + (u >= P::BR / 2 ? P::H : 0u);
}

typedef double dbl2 __attribute__((ext_vector_type(2)));

// Branch costs of predecessor r for the IPT successors of thread slot tq in
// group L, into cv[i] for successor succ(tq, i).
template <int KV>
__device__ __forceinline__ void load_costs(double *cv, const double *cst, uint32_t L, uint32_t tq, uint32_t r,
                                           uint64_t copies)
{
    using P = Tcq<KV>;
    const dbl2 *c2 = reinterpret_cast<const dbl2 *>(cst);
#pragma unroll
    for (uint32_t j = 0; j < P::H; ++j) {
        const uint32_t u = P::succ(tq, j);  // below BR/2: sign bit clear
        const uint32_t s = (L << KV) | (u << P::M) | r;
        const uint32_t h = s * s + s;
        const uint32_t q = r * P::H + j;
        const uint32_t cp = (uint32_t)(copies >> (P::CBITS * q)) & (P::CC - 1);
        const dbl2 c = c2[P::unit((h >> 7) & 511u, cp)];
        cv[j] = c.x;
        cv[j + P::H] = c.y;
    }
}

// One Viterbi pass over the T steps t = (k + rot) mod T; start < 0: every
// memory starts at cost 0, else only `start`. bp receives T * S bytes.
// Returns which metric buffer holds the end metrics.
template <int KV>
__device__ __forceinline__ int viterbi_pass(Shared<KV> &sh, uint32_t T, int32_t start, uint32_t rot, uint8_t *__restrict__ bp)
{
    using P = Tcq<KV>;
    const uint32_t tid = threadIdx.x;
    const uint32_t L = tid % P::G, tq = tid / P::G;
    const uint64_t cpy = P::copies(tid);
    for (uint32_t m = tid; m < P::S; m += P::NT)
        sh.D[0][P::pad(m)] = (start < 0 || (int32_t)m == start) ? 0.0 : __builtin_inf();
    fill_costs<KV>(sh.cost[0], sh.lut, sh.z[2 * (rot % T)], sh.z[2 * (rot % T) + 1]);
    __syncthreads();
    // this thread's first metric read and first metric write (next memory
    // L | succ(tq, 0) << (M - kv), the others at constant distances)
    const double *rp = &sh.D[0][P::pad(L << KV)];
    double *wp = &sh.D[0][P::LINEAR_NEXT ? P::pad(L) + tq * P::H * P::USTRIDE : 0u];
    // One step. Step k reads metric and cost buffer k & 1 and writes buffer
    // (k & 1) ^ 1. Unrolled by two (the parity a constant), every LDS address
    // is a per-thread register plus an immediate offset.
    auto step = [&](uint32_t k, auto parity) {
        const int B = (int)parity;
        double *Dn = sh.D[B ^ 1];  // the next metrics when their positions are not linear (kv 6)
        const double *cst = sh.cost[B];
        double best[P::IPT];
        uint32_t br[P::IPT];
#pragma unroll
        for (uint32_t i = 0; i < P::IPT; ++i) {
            best[i] = __builtin_inf();
            br[i] = 0;
        }
        // software-pipelined: the branch costs of predecessor r + 1 are
        // requested before the add-compare-selects of predecessor r. The
        // back-pointer moves to r only on a strictly smaller candidate, so
        // ties keep the smallest r; the metric is the same either way.
        double cv[2][P::IPT];
        const double *dr = rp + B * P::SP;
        dbl2 dv2 = {0.0, 0.0};
        load_costs<KV>(cv[0], cst, L, tq, 0, cpy);
#pragma unroll
        for (uint32_t r = 0; r < P::BR; ++r) {
            if (r + 1 < P::BR) load_costs<KV>(cv[(r + 1) & 1], cst, L, tq, r + 1, cpy);
            double dv;
            if constexpr (KV >= 4) {
                // the run of BR metrics is contiguous and 16-byte aligned
                if (r % 2 == 0) dv2 = reinterpret_cast<const dbl2 *>(dr)[r / 2];
                dv = (r & 1u) ? dv2.y : dv2.x;
            } else {
                dv = dr[r];
            }
#pragma unroll
            for (uint32_t i = 0; i < P::IPT; ++i) {
                const double v = dv + cv[r & 1][i];
                if constexpr (P::MIN_SELECT) {
                    br[i] = v < best[i] ? r : br[i];
                    best[i] = __builtin_fmin(best[i], v);
                } else if (v < best[i]) {
                    best[i] = v;
                    br[i] = r;
                }
            }
            if (KV < 4 || r % 2 == 0)
                __builtin_amdgcn_sched_group_barrier(0x100, P::H + 1, 0);
            else
                __builtin_amdgcn_sched_group_barrier(0x100, P::H, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, P::SCHED_VALU, 0);
        }
#pragma unroll
        for (uint32_t i = 0; i < P::IPT; ++i) {
            if constexpr (P::LINEAR_NEXT) {
                wp[(B ^ 1) * P::SP + P::succ(0, i) * P::USTRIDE] = best[i];
            } else {
                const uint32_t u = P::succ(tq, i);
                Dn[P::pad(L | (u << (P::M - KV)))] = best[i];
            }
        }
        store_bp<P::IPT>(bp + (uint64_t)k * P::S + tid * P::IPT, br);
        if (k + 1 < T) {
            const uint32_t t1 = (k + 1 + rot) % T;
            fill_costs<KV>(sh.cost[B ^ 1], sh.lut, sh.z[2 * t1], sh.z[2 * t1 + 1]);
        }
        __syncthreads();
    };
    if constexpr (P::PARITY_UNROLL) {
        for (uint32_t k = 0; k < T; k += 2) {
            step(k, std::integral_constant<int, 0>{});
            if (k + 1 < T) step(k + 1, std::integral_constant<int, 1>{});
        }
    } else {
        for (uint32_t k = 0; k < T; ++k) step(k, (int)(k & 1u));
    }
    return (int)(T & 1u);
}

// Smallest metric over all memories, the smallest memory on ties.
template <int KV>
__device__ __forceinline__ uint32_t argmin_memory(Shared<KV> &sh, const double *D)
{
    using P = Tcq<KV>;
    const uint32_t tid = threadIdx.x, lane = tid & 63u, w = tid >> 6;
    double bv = __builtin_inf();
    uint32_t bi = 0xFFFFFFFFu;
    for (uint32_t m = tid; m < P::S; m += P::NT) {
        const double v = D[P::pad(m)];
        if (v < bv || (v == bv && m < bi)) {
            bv = v;
            bi = m;
        }
    }
    for (int off = 32; off > 0; off >>= 1) {
        const double ov = __shfl_down(bv, off, 64);
        const uint32_t oi = __shfl_down(bi, off, 64);
        if (lane + off < 64 && (ov < bv || (ov == bv && oi < bi))) {
            bv = ov;
            bi = oi;
        }
    }
    if (lane == 0) {
        sh.red_v[w] = bv;
        sh.red_i[w] = bi;
    }
    __syncthreads();
    if (tid == 0) {
        double v = sh.red_v[0];
        uint32_t i = sh.red_i[0];
        for (uint32_t q = 1; q < P::NT / 64; ++q)
            if (sh.red_v[q] < v || (sh.red_v[q] == v && sh.red_i[q] < i)) {
                v = sh.red_v[q];
                i = sh.red_i[q];
            }
        // every metric infinite (not reachable from a finite row): memory 0
        sh.W = i == 0xFFFFFFFFu ? 0u : i;
    }
    __syncthreads();
    const uint32_t r = sh.W;
    __syncthreads();
    return r;
}

// Walk of the back-pointers from the next memory `end` after the last step
// down to step 0, run by one whole wave (every lane follows the same path).
// Several steps per load latency: while the back-pointer r of step k loads,
// lane j < BR loads the back-pointer at step k - 1 of the memory that r = j
// leads to, and (when BR^2 <= 64) lane j * BR + i the back-pointer at step
// k - 2 of the memory that the choices j at step k and i at step k - 1 lead
// to; r then picks the lane, and the two choices the lane of the next. Returns the memory held after step kw; with `emit`
// sets each step's kv new bits in the code, without it the walk ends once
// step kw is reached.
template <int KV>
__device__ __forceinline__ uint32_t walk_back(const uint8_t *bp, uint32_t T, uint32_t end, uint32_t kw, bool emit,
                                              uint8_t *code)
{
    using P = Tcq<KV>;
    constexpr uint32_t BR = P::BR;
    // three steps per load latency when the BR^2 step k - 2 loads take one per
    // lane (kv 3); four a lane (kv 4) measured slower than two steps
    constexpr bool DEEP = BR * BR <= 64;
    constexpr uint32_t PER = 1;  // step k - 2 loads per lane
    const uint32_t lane = threadIdx.x & 63u;
    uint32_t m2 = end, w = 0;
    auto step = [&](uint32_t k, uint32_t r) {
        if (k == kw) w = m2;
        const uint32_t s = ((m2 << KV) | r) & 0xFFFFu;
        if (emit && lane == 0) {
            const uint32_t u = s >> P::M;
            for (uint32_t i = 0; i < (uint32_t)KV; ++i)
                if ((u >> i) & 1u) {
                    const uint32_t j = KV * k + i;
                    code[j >> 3] |= (uint8_t)(1u << (j & 7));
                }
        }
        m2 = s & (P::S - 1);
    };
    auto next = [&](uint32_t m, uint32_t r) { return ((m << KV) | r) & (P::S - 1); };
    constexpr int32_t STRIDE = DEEP ? 3 : 2;
    for (int32_t k = (int32_t)T - 1; k >= 0; k -= STRIDE) {
        if (!emit && (uint32_t)k < kw) break;  // step kw is done: w is set
        const uint32_t rk = bp[(uint64_t)k * P::S + bp_pos<KV>(m2)];
        uint32_t cand = 0;
        if (k >= 1 && lane < BR) cand = bp[(uint64_t)(k - 1) * P::S + bp_pos<KV>(next(m2, lane))];
        // pair p = q * 64 + lane: the choices j = p / BR at step k and
        // i = p % BR at step k - 1
        uint32_t cand2[PER];
#pragma unroll
        for (uint32_t q = 0; q < PER; ++q) {
            const uint32_t pidx = q * 64 + lane;
            cand2[q] = 0;
            if (DEEP && k >= 2 && pidx < BR * BR)
                cand2[q] = bp[(uint64_t)(k - 2) * P::S + bp_pos<KV>(next(next(m2, pidx / BR), pidx % BR))];
        }
        step((uint32_t)k, rk);
        if (k >= 1) {
            const uint32_t rk1 = (uint32_t)__shfl((int)cand, (int)rk, 64);
            step((uint32_t)k - 1, rk1);
            if (DEEP && k >= 2) {
                const uint32_t pidx = rk * BR + rk1;  // wave-uniform
                uint32_t v = cand2[0];
#pragma unroll
                for (uint32_t q = 1; q < PER; ++q)
                    if (pidx / 64 == q) v = cand2[q];
                step((uint32_t)k - 2, (uint32_t)__shfl((int)v, (int)(pidx % 64), 64));
            }
        }
    }
    return w;
}

template <int KV>
__global__ __launch_bounds__(Tcq<KV>::NT) __attribute__((amdgpu_waves_per_eu(4))) void tcq_encode_rows(const float *__restrict__ e, uint64_t nrows,
                                                            uint32_t d, const uint32_t *__restrict__ lut,
                                                            uint8_t *__restrict__ out, uint64_t record_bytes,
                                                            uint8_t *__restrict__ workspace)
{
    using P = Tcq<KV>;
    __shared__ Shared<KV> sh;
    const uint32_t tid = threadIdx.x;
    const uint32_t T = d / 2, N = KV * T, NB = N / 8;
    uint8_t *bp = workspace + (uint64_t)blockIdx.x * T * P::S;
    if (tid < 512) sh.lut[tid] = lut[tid];

    for (uint64_t row = blockIdx.x; row < nrows; row += gridDim.x) {
        const float *er = e + row * d;
        uint8_t *rec = out + row * record_bytes;
        for (uint32_t b = tid; b < NB + 2; b += P::NT) sh.code[b] = 0;
        if (tid == 0) {
            double n2 = 0.0;
            for (uint32_t i = 0; i < d; ++i) {
                const double v = (double)er[i];
                n2 = n2 + v * v;
            }
            sh.norm = __builtin_sqrt(n2);
        }
        __syncthreads();
        const double norm = sh.norm;
        // alpha = ||e|| / ||f(c)|| needs a finite nonzero norm: a row of zeros,
        // or one holding an inf or a NaN, keeps the all-zero code and alpha 0
        if (norm > 0.0 && norm < __builtin_inf()) {
            const double sd = __builtin_sqrt((double)d);
            for (uint32_t i = tid; i < d; i += P::NT) sh.z[i] = sd * (double)er[i] / norm;
            __syncthreads();

            // pass A (p = 0): every start, steps rotated by T/2; W = the best
            // path's memory before step 0, i.e. after step T-1, which pass A
            // visits as k = T-rot-1. Pass B (p = 1): from W alone; the path
            // ending in W is the code.
            const uint32_t rot = T / 2;
            uint32_t W = 0;
            for (int p = 0; p < 2; ++p) {
                const int cend = viterbi_pass<KV>(sh, T, p == 0 ? -1 : (int32_t)W, p == 0 ? rot : 0, bp);
                const uint32_t end = p == 0 ? argmin_memory<KV>(sh, sh.D[cend]) : W;
                if (tid < 64) {
                    const uint32_t w = walk_back<KV>(bp, T, end, T - rot - 1, p == 1, sh.code);
                    if (tid == 0) sh.W = w;
                }
                __syncthreads();
                if (p == 0) W = sh.W;
                __syncthreads();
            }

            // f(c) of the emitted code (in the cost buffer, free now), then alpha
            uint32_t *f = reinterpret_cast<uint32_t *>(sh.cost[0]);
            for (uint32_t t = tid; t < T; t += P::NT) {
                uint32_t s = 0;
                for (uint32_t q = 0; q < 16; ++q) {
                    const uint32_t j = (KV * (t + 1) + N - 16 + q) % N;
                    s |= (uint32_t)((sh.code[j >> 3] >> (j & 7)) & 1u) << q;
                }
                const uint32_t h = s * s + s;
                uint32_t pr = sh.lut[(h >> 7) & 511u];
                if (s & 0x8000u) pr ^= 0x80008000u;
                f[t] = pr;
            }
            __syncthreads();
            if (tid == 0) {
                double fn2 = 0.0;
                for (uint32_t t = 0; t < T; ++t) {
                    const double a = half_to_double(f[t] & 0xFFFFu), b = half_to_double(f[t] >> 16);
                    fn2 = fn2 + a * a;
                    fn2 = fn2 + b * b;
                }
                const double alpha = fn2 > 0.0 ? norm / __builtin_sqrt(fn2) : 0.0;
                const uint16_t ab = bf16_rne(alpha);
                sh.code[NB] = (uint8_t)(ab & 0xFFu);
                sh.code[NB + 1] = (uint8_t)(ab >> 8);
            }
        }
        __syncthreads();
        for (uint32_t b = tid; b < NB + 2; b += P::NT) rec[b] = sh.code[b];
        __syncthreads();
    }
}

uint32_t encode_threads(uint32_t kv)
{
    switch (kv) {
    case 3: return Tcq<3>::NT;
    case 4: return Tcq<4>::NT;
    case 5: return Tcq<5>::NT;
    case 6: return Tcq<6>::NT;
    default: return 0;
    }
}

const void *encode_kernel(uint32_t kv)
{
    switch (kv) {
    case 3: return reinterpret_cast<const void *>(&tcq_encode_rows<3>);
    case 4: return reinterpret_cast<const void *>(&tcq_encode_rows<4>);
    case 5: return reinterpret_cast<const void *>(&tcq_encode_rows<5>);
    case 6: return reinterpret_cast<const void *>(&tcq_encode_rows<6>);
    default: return nullptr;
    }
}

}  // namespace

bool encode_supported(uint32_t d, uint32_t kv)
{
    return (d == 64 || d == 128 || d == 256 || d == 512) && kv >= 3 && kv <= 6;
}

hipError_t encode_grid(uint32_t kv, int num_cus, uint64_t nrows, uint32_t *blocks)
{
    *blocks = 0;
    const void *k = encode_kernel(kv);
    if (!k) return hipErrorInvalidValue;
    int per_cu = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, (int)encode_threads(kv), 0);
    if (e != hipSuccess) return e;
    if (per_cu < 1) return hipErrorInvalidConfiguration;
    const uint64_t most = (uint64_t)per_cu * (uint64_t)(num_cus > 0 ? num_cus : 1);
    *blocks = (uint32_t)(nrows < most ? nrows : most);
    return hipSuccess;
}

uint64_t encode_workspace_per_block(uint32_t d, uint32_t kv) { return (uint64_t)(d / 2) << (16 - kv); }

hipError_t encode(const EncodeArgs &a)
{
    if (a.nrows == 0 || a.blocks == 0) return hipSuccess;
    switch (a.kv) {
    case 3:
        hipLaunchKernelGGL(tcq_encode_rows<3>, dim3(a.blocks), dim3(Tcq<3>::NT), 0, a.stream, a.rows, a.nrows, a.d,
                           a.lut, a.out, a.record_bytes, a.workspace);
        break;
    case 4:
        hipLaunchKernelGGL(tcq_encode_rows<4>, dim3(a.blocks), dim3(Tcq<4>::NT), 0, a.stream, a.rows, a.nrows, a.d,
                           a.lut, a.out, a.record_bytes, a.workspace);
        break;
    case 5:
        hipLaunchKernelGGL(tcq_encode_rows<5>, dim3(a.blocks), dim3(Tcq<5>::NT), 0, a.stream, a.rows, a.nrows, a.d,
                           a.lut, a.out, a.record_bytes, a.workspace);
        break;
    case 6:
        hipLaunchKernelGGL(tcq_encode_rows<6>, dim3(a.blocks), dim3(Tcq<6>::NT), 0, a.stream, a.rows, a.nrows, a.d,
                           a.lut, a.out, a.record_bytes, a.workspace);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Copy kernels for encoding into a mixed-rate table: the rows of one rate
// class are gathered into a contiguous batch, encoded by the kernel above into
// contiguous records, and the records scattered to their offsets (the encode
// kernel itself stays as it is measured fastest).
__global__ void gather_rows(const float *__restrict__ e, const uint32_t *__restrict__ src_row, uint64_t n,
                            uint32_t d, float *__restrict__ staged)
{
    const uint64_t total = n * d;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (uint64_t)gridDim.x * blockDim.x)
        staged[i] = e[(uint64_t)src_row[i / d] * d + i % d];
}

__global__ void scatter_records(const uint8_t *__restrict__ staged, uint64_t record_bytes,
                                const uint64_t *__restrict__ dst_off, uint64_t n, uint8_t *__restrict__ out)
{
    const uint64_t total = n * record_bytes;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (uint64_t)gridDim.x * blockDim.x)
        out[dst_off[i / record_bytes] + i % record_bytes] = staged[i];
}

static unsigned copy_grid(uint64_t items)
{
    const uint64_t b = (items + 255) / 256;
    return (unsigned)(b < 1 ? 1 : (b > 65536 ? 65536 : b));
}

hipError_t encode_listed(const EncodeArgs &a, const uint32_t *src_row, const uint64_t *dst_off, float *staged_rows,
                         uint8_t *staged_recs)
{
    if (a.nrows == 0 || a.blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(gather_rows, dim3(copy_grid(a.nrows * a.d)), dim3(256), 0, a.stream, a.rows, src_row,
                       a.nrows, a.d, staged_rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    EncodeArgs b = a;
    b.rows = staged_rows;
    b.out = staged_recs;
    e = encode(b);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(scatter_records, dim3(copy_grid(a.nrows * a.record_bytes)), dim3(256), 0, a.stream,
                       staged_recs, a.record_bytes, dst_off, a.nrows, a.out);
    return hipGetLastError();
}

}  // namespace cpk
