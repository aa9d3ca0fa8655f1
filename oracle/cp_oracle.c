/*
 * cp_oracle.c - plain CPU oracle for Conditional Program (CP) row decoding.
 *
 * TEST INFRASTRUCTURE. This is the slow, obviously-correct reference that the
 * HIP library is checked against. Only the test suite, the smoke check and
 * the CPU-baseline leg of the benchmark load it; the product never links,
 * imports or calls anything here, and nothing here is shared with it.
 * Scalar C, fp64 wherever floating point is involved, no intrinsics.
 *
 * Pages this follows (cited by key below):
 *   [KO] "2비트 코드와 공유 트렐리스로 n-gram 룩업 테이블을 4~8배 압축한다"
 *        (onedev.kr paper digest), sections "How it works" (어떻게 동작하나),
 *        "How it differs" (무엇과 다른가), "How it is used" (어떻게 쓰나),
 *        "Assumptions and limits" (전제와 한계).
 *   [EN] "Two-bit lookup tables shrink DeepSeek's 203 GB memory to 51 GB and
 *        cut prefill from 64.66 s to 13.27 s" (ai4snews digest), sections
 *        Synopsis and Interpretation.
 *   [RU] "Conditional Program сжимает n-gram память DeepSeek с 203 до 51 ГБ
 *        при 2 битах" (news.hamidun.com), section "Как устроен CP".
 *
 * Facts the pages fix:
 *   - a row is rebuilt as e_hat = alpha * f(c): a short per-row code c, a
 *     per-row scale alpha, and one rule f shared by the whole table, run only
 *     for rows that are looked up [KO "How it works"; RU "Как устроен CP"];
 *   - a row costs b + 16/d bits per parameter at code rate b, the 16 being
 *     the one scale per row [KO "How it works"];
 *   - the encoder normalises z = sqrt(d) e / ||e||, codes z with trellis-coded
 *     quantisation on a tail-biting Gaussian HYB bitshift trellis (joint choice
 *     along a state path, no per-row rotation), and sets
 *     alpha = ||e|| / ||f(c)|| so the row norm is restored [KO "How it differs"];
 *   - each row is an independently addressable record holding its code and
 *     scale; only requested records are fetched, decoded and handed on in the
 *     original lookup order [KO "How it differs"; EN Interpretation];
 *   - the per-row scale is a bf16 [KO "How it is used"].
 *
 * Readings where the pages are silent (the pages name the trellis family but
 * give none of its parameters):
 *   R1 trellis: 16-bit window, V = 2 outputs per step, kv code bits per step,
 *      T = d/2 steps, N = kv*T code bits per row.
 *   R2 bit order: the code is one little-endian N-bit integer; bit j is bit
 *      (j & 7) of byte j >> 3.
 *   R3 window of step t: bits [kv(t+1) - 16, kv(t+1)) of the circular code
 *      (indices mod N), oldest bit in bit 0 of s, so step t's own kv bits are
 *      the top kv bits of s. Indices wrap mod N: this is the tail-biting.
 *   R4 output rule: h = (s*s + s) mod 2^32, idx = (h >> 7) & 511, pair =
 *      LUT[idx] (two fp16), both sign bits flipped when bit 15 of s is set;
 *      LUT[idx][0] is element 2t, LUT[idx][1] element 2t+1.
 *   R5 record: N/8 code bytes, then alpha as bf16 little endian; packed.
 *   R6 scaled output: the exact product alpha * f, rounded once to bf16,
 *      round-to-nearest-even.
 *   R7 encoder objective: minimise ||z - f(c)||^2 over tail-biting codes with
 *      unit scale; alpha is set afterwards from the norms. Ties keep the
 *      smallest predecessor and then the smallest start memory.
 *   R11 mixed-rate table (the pages study allocating bits by access frequency
 *      over their code rates but give no format): each row has a rate class,
 *      class c codes at kv_c bits per step, and the records of all rows are
 *      packed in row order, so row i's record starts at the sum of the record
 *      sizes of rows 0..i-1.
 */
#include "cp_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#define WINDOW_BITS 16u
#define NWINDOWS (1u << WINDOW_BITS)

/* ------------------------------------------------------------------------ */
/* parameters                                                               */
/* ------------------------------------------------------------------------ */

/* Code bits per row, or 0 when (d, kv) cannot form a tail-biting code with
 * a 16-bit window (reading R1). Codes are held in ceil(N/8) bytes. */
uint64_t cpo_code_bits(uint32_t d, uint32_t kv)
{
    if (d == 0 || (d & 1u) || kv < 1 || kv > 15) return 0;
    uint64_t n = (uint64_t)kv * (d / 2);
    if (n < WINDOW_BITS) return 0;
    return n;
}

static uint64_t code_bytes(uint64_t nbits) { return (nbits + 7) / 8; }

/* Record size: code bytes plus one 16-bit scale, or 0 when the code does not
 * fill whole bytes (reading R5). [KO "How it works"]: b + 16/d bits per
 * parameter, so R = (b*d + 16) / 8 bytes with b = kv / 2. */
uint64_t cpo_record_bytes(uint32_t d, uint32_t kv)
{
    uint64_t n = cpo_code_bits(d, kv);
    return (n && n % 8 == 0) ? n / 8 + 2 : 0;
}

/* ------------------------------------------------------------------------ */
/* number formats                                                           */
/* ------------------------------------------------------------------------ */

/* IEEE binary16 bit pattern -> value, from the format's definition. */
double cpo_fp16_to_double(uint16_t h)
{
    int neg = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);
    return neg ? -v : v;
}

/* bfloat16 bit pattern -> value (8 exponent bits, 7 fraction bits). */
double cpo_bf16_to_double(uint16_t b)
{
    int neg = b >> 15, e = (b >> 7) & 255, m = b & 127;
    double v;
    if (e == 0)
        v = ldexp((double)m, -133);
    else if (e == 255)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + m), e - 134);
    return neg ? -v : v;
}

/* Value -> bfloat16, round to nearest, ties to even, in one step from the
 * double: find the binade, scale to the bf16 spacing there, round to an
 * integer with ties to even, re-encode. The subnormal range uses the spacing
 * of the smallest normal binade; a carry into the next binade and the
 * overflow to infinity fall out of the same encoding. */
uint16_t cpo_bf16_from_double(double x)
{
    uint16_t sgn = signbit(x) ? 0x8000u : 0u;
    if (isnan(x)) return (uint16_t)(sgn | 0x7FC0u);
    double a = fabs(x);
    if (a == 0.0) return sgn;
    if (isinf(a)) return (uint16_t)(sgn | 0x7F80u);
    int ex;
    (void)frexp(a, &ex);          /* a in [2^(ex-1), 2^ex) */
    int E = ex - 1;
    if (E > 127) return (uint16_t)(sgn | 0x7F80u);
    if (E < -126) E = -126;
    double k = nearbyint(a / ldexp(1.0, E - 7)); /* default mode: ties to even */
    long bits = ((long)(E + 127) << 7) + ((long)k - 128);
    if (bits >= 0x7F80) bits = 0x7F80;
    return (uint16_t)(sgn | (uint16_t)bits);
}

/* ------------------------------------------------------------------------ */
/* the shared reconstruction rule f (readings R1-R4)                        */
/* ------------------------------------------------------------------------ */

/* Bit j of the circular code (R2, R3). */
int cpo_code_bit(const uint8_t *code, uint64_t nbits, int64_t j)
{
    int64_t jj = j % (int64_t)nbits;
    if (jj < 0) jj += (int64_t)nbits;
    return (code[jj >> 3] >> (jj & 7)) & 1;
}

/* State window of step t: 16 consecutive bits of the circular code ending
 * (exclusive) at kv*(t+1), gathered one bit at a time (R3). */
uint32_t cpo_window(const uint8_t *code, uint32_t d, uint32_t kv, uint32_t t)
{
    uint64_t nbits = cpo_code_bits(d, kv);
    int64_t end = (int64_t)kv * (int64_t)(t + 1);
    uint32_t s = 0;
    for (uint32_t m = 0; m < WINDOW_BITS; ++m)
        s |= (uint32_t)cpo_code_bit(code, nbits, end - (int64_t)WINDOW_BITS + m) << m;
    return s;
}

/* Output selector of a window (R4). */
void cpo_hash(uint32_t s, uint32_t *idx, uint32_t *negate)
{
    uint64_t h = ((uint64_t)s * (uint64_t)s + (uint64_t)s) % 4294967296ull;
    *idx = (uint32_t)((h >> 7) & 511u);
    *negate = (s >> 15) & 1u;
}

/* One output pair as fp16 bit patterns (R4). Negation flips the sign bit,
 * so +0 and -0 swap exactly. */
static void pair_of_window(const uint16_t *lut, uint32_t s, uint16_t *p0, uint16_t *p1)
{
    uint32_t idx, neg;
    cpo_hash(s, &idx, &neg);
    *p0 = lut[2 * idx];
    *p1 = lut[2 * idx + 1];
    if (neg) {
        *p0 ^= 0x8000u;
        *p1 ^= 0x8000u;
    }
}

/* f(c): the unscaled row, d fp16 bit patterns, walking all T = d/2 steps of
 * the tail-biting trellis [KO "How it differs"; R1-R4]. */
int cpo_decode_code(const uint16_t *lut, const uint8_t *code, uint32_t d, uint32_t kv,
                    uint16_t *f_out)
{
    if (!cpo_code_bits(d, kv)) return -1;
    for (uint32_t t = 0; t < d / 2; ++t) {
        uint32_t s = cpo_window(code, d, kv, t);
        pair_of_window(lut, s, &f_out[2 * t], &f_out[2 * t + 1]);
    }
    return 0;
}

/* e_hat = alpha * f(c) [KO "How it works"], product exact in fp64 (8 + 11
 * significant bits), rounded once to bf16 (R6). */
int cpo_decode_record(const uint16_t *lut, const uint8_t *record, uint32_t d, uint32_t kv,
                      uint16_t *out_bf16)
{
    uint64_t nbits = cpo_code_bits(d, kv);
    if (!cpo_record_bytes(d, kv)) return -1;
    uint16_t *f = (uint16_t *)malloc(sizeof(uint16_t) * d);
    if (!f) return -2;
    cpo_decode_code(lut, record, d, kv, f);
    uint16_t abits = (uint16_t)(record[nbits / 8] | (record[nbits / 8 + 1] << 8));
    double alpha = cpo_bf16_to_double(abits);
    for (uint32_t i = 0; i < d; ++i)
        out_bf16[i] = cpo_bf16_from_double(alpha * cpo_fp16_to_double(f[i]));
    free(f);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* the lookup: gather requested records, decode, write in lookup order      */
/* ------------------------------------------------------------------------ */

typedef struct {
    const uint16_t *lut;
    const uint8_t *records;
    uint64_t rows;
    uint32_t d, kv;
    /* mixed-rate tables (R11): NULL for a single-rate table */
    const uint32_t *kv_of_class;
    const uint8_t *row_class;
    const uint64_t *offsets;
    const int64_t *ids;
    uint64_t begin, end;
    uint16_t *out;
    int raw;
    uint64_t bad;
} lookup_job;

static void *lookup_worker(void *arg)
{
    lookup_job *job = (lookup_job *)arg;
    uint64_t rbytes = cpo_record_bytes(job->d, job->kv);
    for (uint64_t j = job->begin; j < job->end; ++j) {
        int64_t id = job->ids[j];
        uint16_t *dst = job->out + j * (uint64_t)job->d;
        if (id < 0 || (uint64_t)id >= job->rows) {
            /* an id outside the table yields a zero row (the pages' table-removal
             * baseline returns 0 for a lookup [KO "How it is used"]) */
            memset(dst, 0, sizeof(uint16_t) * job->d);
            job->bad++;
            continue;
        }
        uint32_t kv = job->kv;
        const uint8_t *rec = job->records + (uint64_t)id * rbytes;
        if (job->row_class) {
            kv = job->kv_of_class[job->row_class[id]];
            rec = job->records + job->offsets[id];
        }
        if (job->raw)
            cpo_decode_code(job->lut, rec, job->d, kv, dst);
        else
            cpo_decode_record(job->lut, rec, job->d, kv, dst);
    }
    return NULL;
}

/* Runs the lookup jobs on nthreads threads; returns the bad-id count. */
static int64_t run_lookup(lookup_job proto, uint64_t n, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    lookup_job jobs[256];
    pthread_t th[256];
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = proto;
        jobs[i].begin = n * (uint64_t)i / (uint64_t)nthreads;
        jobs[i].end = n * (uint64_t)(i + 1) / (uint64_t)nthreads;
        jobs[i].bad = 0;
    }
    for (int i = 1; i < nthreads; ++i) pthread_create(&th[i], NULL, lookup_worker, &jobs[i]);
    lookup_worker(&jobs[0]);
    for (int i = 1; i < nthreads; ++i) pthread_join(th[i], NULL);
    int64_t bad = 0;
    for (int i = 0; i < nthreads; ++i) bad += (int64_t)jobs[i].bad;
    return bad;
}

/* Decodes rows ids[0..n) of a packed record table into out[n][d] (bf16 bits,
 * or with raw != 0 the unscaled f(c) as fp16 bits), in lookup order
 * [KO "How it differs"]. The lookups are split into nthreads contiguous
 * slices. Returns the number of ids outside [0, rows), or -1 on bad
 * parameters. */
int64_t cpo_lookup_decode(const uint16_t *lut, const uint8_t *records, uint64_t rows,
                          uint32_t d, uint32_t kv, const int64_t *ids, uint64_t n,
                          uint16_t *out, int raw, int nthreads)
{
    if (!cpo_record_bytes(d, kv)) return -1;
    lookup_job proto = {lut, records, rows, d, kv, NULL, NULL, NULL, ids, 0, 0, out, raw, 0};
    return run_lookup(proto, n, nthreads);
}

/* ------------------------------------------------------------------------ */
/* mixed-rate tables (R11)                                                   */
/* ------------------------------------------------------------------------ */

/* Record offsets of a mixed-rate table: row i is coded at
 * kv_of_class[row_class[i]] bits per step, and the records are packed in row
 * order with nothing between them, so row i starts at the sum of the record
 * sizes of rows 0..i-1. offsets[0..rows] (offsets[rows] = total bytes).
 * Returns 0, or -1 for a class >= nclass or a rate without whole-byte
 * records. The pages study bit allocation by access frequency over their code
 * rates [KO "How it is used" (1.5 / 2 / 2.5 / 3 bits), "Assumptions and
 * limits"; EN Perspective]; how rates are chosen is the caller's. */
int cpo_mixed_offsets(uint64_t rows, uint32_t d, const uint32_t *kv_of_class, uint32_t nclass,
                      const uint8_t *row_class, uint64_t *offsets)
{
    uint64_t acc = 0;
    for (uint64_t i = 0; i < rows; ++i) {
        if (row_class[i] >= nclass) return -1;
        uint64_t r = cpo_record_bytes(d, kv_of_class[row_class[i]]);
        if (!r) return -1;
        offsets[i] = acc;
        acc += r;
    }
    offsets[rows] = acc;
    return 0;
}

/* Lookup into a mixed-rate table: as cpo_lookup_decode, row id's record
 * being the one at offsets[id], decoded at its class's rate. */
int64_t cpo_lookup_decode_mixed(const uint16_t *lut, const uint8_t *records, uint64_t rows, uint32_t d,
                                const uint32_t *kv_of_class, uint32_t nclass, const uint8_t *row_class,
                                const uint64_t *offsets, const int64_t *ids, uint64_t n, uint16_t *out,
                                int raw, int nthreads)
{
    for (uint32_t c = 0; c < nclass; ++c)
        if (!cpo_record_bytes(d, kv_of_class[c])) return -1;
    lookup_job proto = {lut, records, rows, d, kv_of_class[0], kv_of_class, row_class, offsets, ids, 0, 0,
                        out, raw, 0};
    return run_lookup(proto, n, nthreads);
}

/* ------------------------------------------------------------------------ */
/* encoder: TCQ on the tail-biting trellis [KO "How it differs"]            */
/* ------------------------------------------------------------------------ */

/* Decoded output values of every one of the 2^16 windows, as doubles. */
static double *window_values(const uint16_t *lut)
{
    double *g = (double *)malloc(sizeof(double) * 2 * NWINDOWS);
    if (!g) return NULL;
    for (uint32_t s = 0; s < NWINDOWS; ++s) {
        uint16_t p0, p1;
        pair_of_window(lut, s, &p0, &p1);
        g[2 * s] = cpo_fp16_to_double(p0);
        g[2 * s + 1] = cpo_fp16_to_double(p1);
    }
    return g;
}

/*
 * One Viterbi pass over the memory-state trellis (reading R7).
 * A memory is the M = 16 - kv oldest bits of the next window. From memory m,
 * kv new bits u form the window s = m | u << M, and the next memory is
 * s >> kv. Equivalently, a next memory m2 fixes u = m2 >> (M - kv) and has
 * 2^kv predecessors m = (m2 << kv | r) mod 2^M, r in [0, 2^kv), with window
 * s = (m2 << kv | r) mod 2^16.
 *
 * start >= 0: only memory `start` may begin (cost 0); start < 0: every memory
 * begins at cost 0 (free start). Steps are visited in the order
 * t_k = (k + rot) mod T. D_final receives the path metric of every end
 * memory; bp[k * 2^M + m2] the chosen r of step k (smallest r on ties).
 */
static void viterbi_pass(const double *z, uint32_t T, uint32_t kv, const double *g,
                         int64_t start, uint32_t rot, double *D_final, uint8_t *bp)
{
    uint32_t M = WINDOW_BITS - kv, S = 1u << M, R = 1u << kv;
    double *D = (double *)malloc(sizeof(double) * S);
    double *Dn = (double *)malloc(sizeof(double) * S);
    for (uint32_t m = 0; m < S; ++m) D[m] = (start < 0 || (int64_t)m == start) ? 0.0 : INFINITY;
    for (uint32_t k = 0; k < T; ++k) {
        uint32_t t = (k + rot) % T;
        double z0 = z[2 * t], z1 = z[2 * t + 1];
        for (uint32_t m2 = 0; m2 < S; ++m2) {
            double best = INFINITY;
            uint32_t br = 0;
            for (uint32_t r = 0; r < R; ++r) {
                uint32_t s = ((m2 << kv) | r) & (NWINDOWS - 1);
                uint32_t m = s & (S - 1);
                double e0 = z0 - g[2 * s], e1 = z1 - g[2 * s + 1];
                double v = D[m] + (e0 * e0 + e1 * e1);
                if (v < best) {
                    best = v;
                    br = r;
                }
            }
            Dn[m2] = best;
            bp[(uint64_t)k * S + m2] = (uint8_t)br;
        }
        double *tmp = D;
        D = Dn;
        Dn = tmp;
    }
    memcpy(D_final, D, sizeof(double) * S);
    free(D);
    free(Dn);
}

/* Walks the back-pointers from end memory `end`. Writes the kv bits chosen
 * at each visited step into the code (bit kv*t + i of the code is bit i of
 * step t's u) and mem[k + 1] = memory after step k, mem[0] = start memory. */
static void backtrack(uint32_t T, uint32_t kv, uint32_t rot, const uint8_t *bp, uint32_t end,
                      uint8_t *code, uint32_t *mem)
{
    uint32_t M = WINDOW_BITS - kv, S = 1u << M;
    uint32_t m2 = end;
    if (code) memset(code, 0, code_bytes((uint64_t)kv * T));
    for (int64_t k = (int64_t)T - 1; k >= 0; --k) {
        if (mem) mem[k + 1] = m2;
        uint32_t r = bp[(uint64_t)k * S + m2];
        uint32_t s = ((m2 << kv) | r) & (NWINDOWS - 1);
        uint32_t u = s >> M;
        uint32_t t = ((uint32_t)k + rot) % T;
        if (code)
            for (uint32_t i = 0; i < kv; ++i)
                if ((u >> i) & 1u) {
                    uint64_t j = (uint64_t)kv * t + i;
                    code[j >> 3] |= (uint8_t)(1u << (j & 7));
                }
        m2 = s & (S - 1);
    }
    if (mem) mem[0] = m2;
}

typedef struct {
    uint32_t idx;
    double f;
} start_rank;

static int cmp_rank(const void *a, const void *b)
{
    const start_rank *x = (const start_rank *)a, *y = (const start_rank *)b;
    if (x->f < y->f) return -1;
    if (x->f > y->f) return 1;
    return (x->idx > y->idx) - (x->idx < y->idx);
}

/*
 * Tail-biting TCQ of a unit-scale source z (length d).
 * A code is tail-biting when its path starts and ends in the same memory W
 * (the last M code bits). The fixed-start Viterbi from W, read at end memory
 * W, gives the best code with that W.
 *   Both modes first run a heuristic: one free-start pass on the step
 *     sequence rotated by T/2 reads the memory W_h the best path holds at the
 *     original start, and one fixed-start pass from W_h gives a closed code.
 *   mode CPO_ENC_HEURISTIC stops there.
 *   mode CPO_ENC_EXACT then runs branch and bound over W with that code as
 *     incumbent. A free-start pass gives F(W) <= cost(W) for every W (each
 *     W-closed path is also a free-start path ending in W). Starts are tried
 *     in increasing F; the search stops once F reaches the best closed cost
 *     found, which certifies optimality. max_starts > 0 caps the number of
 *     fixed-start passes (the result is then uncertified unless the bound
 *     closed first; see info->certified and info->gap).
 * Returns the closed path metric (sum of squared errors) or NAN on bad input.
 */
double cpo_tcq_encode(const double *z, uint32_t d, uint32_t kv, const uint16_t *lut, int mode,
                      uint32_t max_starts, uint8_t *code_out, cpo_encode_info *info)
{
    uint64_t nbits = cpo_code_bits(d, kv);
    if (!nbits) return NAN;
    uint32_t T = d / 2, M = WINDOW_BITS - kv, S = 1u << M;
    double *g = window_values(lut);
    double *Dend = (double *)malloc(sizeof(double) * S);
    uint8_t *bp = (uint8_t *)malloc((size_t)T * S);
    uint8_t *code = (uint8_t *)malloc(code_bytes(nbits));
    double best = INFINITY;
    uint32_t starts = 0;
    int certified = 0;
    double lower = 0.0;

    /* heuristic start: one free-start pass on the step sequence rotated by
     * T/2; the best path's memory at the original start position (before step
     * 0 = after step T-1) names the start W_h. */
    uint32_t W_h;
    {
        uint32_t rot = T / 2;
        uint32_t *mem = (uint32_t *)malloc(sizeof(uint32_t) * (T + 1));
        viterbi_pass(z, T, kv, g, -1, rot, Dend, bp);
        uint32_t end = 0;
        for (uint32_t m = 1; m < S; ++m)
            if (Dend[m] < Dend[end]) end = m;
        backtrack(T, kv, rot, bp, end, NULL, mem);
        /* step 0 is visited at k0 = T - rot; mem[k0] is the memory before it */
        W_h = mem[T - rot];
        free(mem);
        viterbi_pass(z, T, kv, g, (int64_t)W_h, 0, Dend, bp);
        best = Dend[W_h];
        backtrack(T, kv, 0, bp, W_h, code_out, NULL);
        starts = 1;
    }
    if (mode != CPO_ENC_HEURISTIC) {
        /* branch and bound over every other start, the heuristic result being
         * the incumbent */
        viterbi_pass(z, T, kv, g, -1, 0, Dend, bp);
        start_rank *order = (start_rank *)malloc(sizeof(start_rank) * S);
        for (uint32_t m = 0; m < S; ++m) {
            order[m].idx = m;
            order[m].f = Dend[m];
        }
        qsort(order, S, sizeof(start_rank), cmp_rank);
        lower = order[0].f;
        certified = 1;
        for (uint32_t i = 0; i < S; ++i) {
            if (order[i].f >= best) break; /* no remaining start can do better */
            uint32_t W = order[i].idx;
            if (W == W_h) continue;
            if (max_starts && starts >= max_starts) {
                certified = 0;
                lower = order[i].f;
                break;
            }
            viterbi_pass(z, T, kv, g, (int64_t)W, 0, Dend, bp);
            ++starts;
            if (Dend[W] < best) {
                best = Dend[W];
                backtrack(T, kv, 0, bp, W, code, NULL);
                memcpy(code_out, code, code_bytes(nbits));
            }
        }
        free(order);
    }
    if (info) {
        info->cost = best;
        info->starts = starts;
        info->certified = certified;
        info->gap = certified ? 0.0 : (best - lower);
    }
    free(g);
    free(Dend);
    free(bp);
    free(code);
    return best;
}

/* Sum of squared errors ||z - f(c)||^2 with f decoded by the bit-by-bit
 * decoder above. */
double cpo_distortion(const double *z, const uint16_t *lut, const uint8_t *code, uint32_t d,
                      uint32_t kv)
{
    uint16_t *f = (uint16_t *)malloc(sizeof(uint16_t) * d);
    if (!f || cpo_decode_code(lut, code, d, kv, f)) {
        free(f);
        return NAN;
    }
    double acc = 0.0;
    for (uint32_t i = 0; i < d; ++i) {
        double e = z[i] - cpo_fp16_to_double(f[i]);
        acc += e * e;
    }
    free(f);
    return acc;
}

/*
 * Encodes one row e (length d) into a packed record [KO "How it differs"]:
 * z = sqrt(d) e / ||e||; tail-biting TCQ of z; f(c) recomputed by decoding the
 * emitted code; alpha = ||e|| / ||f(c)|| in fp64, rounded once to bf16;
 * record = code bytes then alpha (R5). A row whose norm is zero or not finite
 * gets an all-zero code and alpha = 0. alpha_exact (optional) receives the
 * unrounded fp64 alpha.
 */
int cpo_encode_row(const double *e, uint32_t d, uint32_t kv, const uint16_t *lut, int mode,
                   uint32_t max_starts, uint8_t *record, cpo_encode_info *info,
                   double *alpha_exact)
{
    uint64_t nbits = cpo_code_bits(d, kv);
    if (!cpo_record_bytes(d, kv)) return -1;
    double norm2 = 0.0;
    for (uint32_t i = 0; i < d; ++i) norm2 += e[i] * e[i];
    double norm = sqrt(norm2);
    double *z = (double *)malloc(sizeof(double) * d);
    if (!z) return -2;
    memset(record, 0, nbits / 8 + 2);
    double alpha = 0.0;
    /* z = sqrt(d) e / ||e|| and alpha = ||e|| / ||f(c)|| [KO "How it
     * differs"] are defined for a finite nonzero norm only. A row of zeros, or
     * one holding an inf or a NaN (norm inf or NaN), is stored as the all-zero
     * code with alpha = 0 (a reading: the pages do not treat such rows). */
    if (norm > 0.0 && norm < INFINITY) {
        double sd = sqrt((double)d);
        for (uint32_t i = 0; i < d; ++i) z[i] = sd * e[i] / norm;
        cpo_tcq_encode(z, d, kv, lut, mode, max_starts, record, info);
        uint16_t *f = (uint16_t *)malloc(sizeof(uint16_t) * d);
        cpo_decode_code(lut, record, d, kv, f);
        double fn2 = 0.0;
        for (uint32_t i = 0; i < d; ++i) {
            double v = cpo_fp16_to_double(f[i]);
            fn2 += v * v;
        }
        free(f);
        alpha = fn2 > 0.0 ? norm / sqrt(fn2) : 0.0;
    } else if (info) {
        memset(info, 0, sizeof(*info));
        info->certified = 1;
    }
    uint16_t ab = cpo_bf16_from_double(alpha);
    record[nbits / 8] = (uint8_t)(ab & 0xFF);
    record[nbits / 8 + 1] = (uint8_t)(ab >> 8);
    if (alpha_exact) *alpha_exact = alpha;
    free(z);
    return 0;
}

typedef struct {
    const double *e;
    uint32_t d, kv;
    const uint16_t *lut;
    int mode;
    uint32_t max_starts;
    uint8_t *records;
    cpo_encode_info *infos;
    uint64_t begin, end;
    int status;
} encode_job;

static void *encode_worker(void *arg)
{
    encode_job *j = (encode_job *)arg;
    uint64_t rb = cpo_record_bytes(j->d, j->kv);
    for (uint64_t r = j->begin; r < j->end; ++r) {
        int st = cpo_encode_row(j->e + r * j->d, j->d, j->kv, j->lut, j->mode, j->max_starts,
                                j->records + r * rb, j->infos ? &j->infos[r] : NULL, NULL);
        if (st) j->status = st;
    }
    return NULL;
}

/* Encodes nrows rows (row-major [nrows][d]) into packed records, rows split
 * into nthreads contiguous slices. */
int cpo_encode_rows(const double *e, uint64_t nrows, uint32_t d, uint32_t kv,
                    const uint16_t *lut, int mode, uint32_t max_starts, uint8_t *records,
                    cpo_encode_info *infos, int nthreads)
{
    if (!cpo_record_bytes(d, kv)) return -1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    encode_job jobs[256];
    pthread_t th[256];
    for (int i = 0; i < nthreads; ++i) {
        encode_job j = {e, d, kv, lut, mode, max_starts, records, infos,
                        nrows * (uint64_t)i / (uint64_t)nthreads,
                        nrows * (uint64_t)(i + 1) / (uint64_t)nthreads, 0};
        jobs[i] = j;
    }
    for (int i = 1; i < nthreads; ++i) pthread_create(&th[i], NULL, encode_worker, &jobs[i]);
    encode_worker(&jobs[0]);
    for (int i = 1; i < nthreads; ++i) pthread_join(th[i], NULL);
    for (int i = 0; i < nthreads; ++i)
        if (jobs[i].status) return jobs[i].status;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* exhaustive search over every code, for tiny rows                         */
/* ------------------------------------------------------------------------ */

typedef struct {
    const double *z;
    uint32_t d, kv;
    const uint16_t *lut;
    uint64_t begin, end;
    double best;
    uint64_t best_code;
} brute_job;

static void *brute_worker(void *arg)
{
    brute_job *j = (brute_job *)arg;
    uint64_t nbits = cpo_code_bits(j->d, j->kv);
    uint8_t code[8];
    j->best = INFINITY;
    j->best_code = 0;
    for (uint64_t c = j->begin; c < j->end; ++c) {
        for (uint64_t b = 0; b < code_bytes(nbits); ++b) code[b] = (uint8_t)(c >> (8 * b));
        double v = cpo_distortion(j->z, j->lut, code, j->d, j->kv);
        if (v < j->best) {
            j->best = v;
            j->best_code = c;
        }
    }
    return NULL;
}

/* Minimum of ||z - f(c)||^2 over all 2^N codes (N <= 32), by decoding each
 * one with the bit-by-bit decoder; best_code (N/8 bytes) gets the first
 * minimiser in increasing code order. */
double cpo_bruteforce_min(const double *z, uint32_t d, uint32_t kv, const uint16_t *lut,
                          uint8_t *best_code, int nthreads)
{
    uint64_t nbits = cpo_code_bits(d, kv);
    if (!nbits || nbits > 32) return NAN;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    uint64_t total = 1ull << nbits;
    brute_job jobs[256];
    pthread_t th[256];
    for (int i = 0; i < nthreads; ++i) {
        brute_job j = {z, d, kv, lut, total * (uint64_t)i / (uint64_t)nthreads,
                       total * (uint64_t)(i + 1) / (uint64_t)nthreads, INFINITY, 0};
        jobs[i] = j;
    }
    for (int i = 1; i < nthreads; ++i) pthread_create(&th[i], NULL, brute_worker, &jobs[i]);
    brute_worker(&jobs[0]);
    for (int i = 1; i < nthreads; ++i) pthread_join(th[i], NULL);
    double best = INFINITY;
    uint64_t bc = 0;
    for (int i = 0; i < nthreads; ++i)
        if (jobs[i].best < best) {
            best = jobs[i].best;
            bc = jobs[i].best_code;
        }
    if (best_code)
        for (uint64_t b = 0; b < code_bytes(nbits); ++b) best_code[b] = (uint8_t)(bc >> (8 * b));
    return best;
}
