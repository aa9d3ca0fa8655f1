/*
 * cp_oracle.h - C interface of the CPU oracle for Conditional Program row
 * decoding. TEST INFRASTRUCTURE: loaded only by the test suite, the smoke
 * check and the benchmark's CPU-baseline leg. The definitions, the readings
 * they follow and the page citations are in cp_oracle.c.
 */
#ifndef CP_ORACLE_H
#define CP_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { CPO_ENC_EXACT = 0, CPO_ENC_HEURISTIC = 1 };

typedef struct {
    double cost;      /* closed-path metric ||z - f(c)||^2 */
    uint32_t starts;  /* fixed-start Viterbi passes run */
    int32_t certified;/* 1 when the exact search proved optimality */
    double gap;       /* upper bound on (cost - optimum) when not certified */
} cpo_encode_info;

uint64_t cpo_code_bits(uint32_t d, uint32_t kv);
uint64_t cpo_record_bytes(uint32_t d, uint32_t kv);

double cpo_fp16_to_double(uint16_t h);
double cpo_bf16_to_double(uint16_t b);
uint16_t cpo_bf16_from_double(double x);

int cpo_code_bit(const uint8_t *code, uint64_t nbits, int64_t j);
uint32_t cpo_window(const uint8_t *code, uint32_t d, uint32_t kv, uint32_t t);
void cpo_hash(uint32_t s, uint32_t *idx, uint32_t *negate);

int cpo_decode_code(const uint16_t *lut, const uint8_t *code, uint32_t d, uint32_t kv,
                    uint16_t *f_out);
int cpo_decode_record(const uint16_t *lut, const uint8_t *record, uint32_t d, uint32_t kv,
                      uint16_t *out_bf16);
int64_t cpo_lookup_decode(const uint16_t *lut, const uint8_t *records, uint64_t rows,
                          uint32_t d, uint32_t kv, const int64_t *ids, uint64_t n,
                          uint16_t *out, int raw, int nthreads);

int cpo_mixed_offsets(uint64_t rows, uint32_t d, const uint32_t *kv_of_class, uint32_t nclass,
                      const uint8_t *row_class, uint64_t *offsets);
int64_t cpo_lookup_decode_mixed(const uint16_t *lut, const uint8_t *records, uint64_t rows, uint32_t d,
                                const uint32_t *kv_of_class, uint32_t nclass, const uint8_t *row_class,
                                const uint64_t *offsets, const int64_t *ids, uint64_t n, uint16_t *out,
                                int raw, int nthreads);

double cpo_tcq_encode(const double *z, uint32_t d, uint32_t kv, const uint16_t *lut, int mode,
                      uint32_t max_starts, uint8_t *code_out, cpo_encode_info *info);
double cpo_distortion(const double *z, const uint16_t *lut, const uint8_t *code, uint32_t d,
                      uint32_t kv);
int cpo_encode_row(const double *e, uint32_t d, uint32_t kv, const uint16_t *lut, int mode,
                   uint32_t max_starts, uint8_t *record, cpo_encode_info *info,
                   double *alpha_exact);
int cpo_encode_rows(const double *e, uint64_t nrows, uint32_t d, uint32_t kv,
                    const uint16_t *lut, int mode, uint32_t max_starts, uint8_t *records,
                    cpo_encode_info *infos, int nthreads);
double cpo_bruteforce_min(const double *z, uint32_t d, uint32_t kv, const uint16_t *lut,
                          uint8_t *best_code, int nthreads);

#ifdef __cplusplus
}
#endif

#endif
