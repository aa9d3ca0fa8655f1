/*
 * cp_probe.h - measurement probes for the CP row-decode library (gfx950).
 *
 * Not part of the lookup path: small kernels that measure the ceilings the
 * lookup is compared against, so that the floors quoted next to the lookup's
 * timings can be reproduced. The pages time the lookup with the table in HBM
 * and in pinned host memory over PCIe, and note that the row-wise layout's
 * advantage grows in the latter ("2비트 코드와 공유 트렐리스로 n-gram 룩업
 * 테이블을 4~8배 압축한다", onedev.kr, section "Assumptions and limits").
 *
 * All calls are asynchronous on `stream` (NULL: the null stream), launch
 * kernels only and allocate nothing; they return 0 or the launch's
 * hipError_t. Pointers are device-accessible (device memory, or pinned host
 * memory mapped into the device's address space).
 */
#ifndef CP_PROBE_H
#define CP_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` (a multiple of 16, 16-byte aligned) from `src` once, in
 * 16-byte loads spread over the whole device, and writes nothing but a
 * data-dependent word into `sink` (4 bytes, device memory) in the unlikely
 * case that the data's XOR takes one fixed value. With `src` in pinned host
 * memory this is the zero-copy (kernel-read) bandwidth over PCIe; in device
 * memory, the HBM read bandwidth. */
int cpp_read_stream(const void *src, uint64_t bytes, uint32_t *sink, void *stream);

/* The lookup's output stream alone: writes n rows of d bf16 (d = 64..512,
 * a power of two) into `out` exactly as the gather-decode kernel places them
 * (1024-thread workgroups; a wave writes chunks of `chunk` consecutive rows,
 * 16 bytes per lane per row, nontemporal stores), with values that cost no
 * loads. Its time is the store-only floor of a lookup of n rows. */
int cpp_store_rows(uint16_t *out, uint64_t n, uint32_t d, uint32_t chunk, void *stream);

/* The lookup's record fetch alone: for each of the n ids (int64, device
 * memory; each in [0, rows)) reads the R-byte record at byte id * R of
 * `records` in the gather-decode kernel's pattern (2-byte loads by lane,
 * a chunk of 16 rows per wave, records of a chunk requested together) and
 * keeps only a data-dependent word as in cpp_read_stream. Its time is the
 * gather-only floor of a lookup: with the records in pinned host memory, the
 * cost of fetching them over PCIe. R: even, 18..194. */
int cpp_gather_records(const void *records, uint64_t record_bytes, const int64_t *ids, uint64_t n,
                       uint32_t *sink, void *stream);

/* Which lanes of a wave the LDS serves in the same cycle: one workgroup of
 * one wave in which only lanes `lane_a` and `lane_b` (0..63, distinct) access
 * LDS, `iters` times each, at addresses 256 bytes apart (the same banks of a
 * 64-bank LDS); `width` bytes per access (4, 8 or 16), loads when `write` is
 * 0, stores otherwise. Under rocprofv3 the dispatch counts bank-conflict
 * cycles (SQ_LDS_BANK_CONFLICT) exactly when the two lanes share a cycle.
 * The encoder's choice of branch-cost copies rests on this grouping for
 * 16-byte loads. `sink`: 4 bytes of device memory, written only in the
 * unlikely case that the data's XOR takes one fixed value. */
int cpp_lds_pair(uint32_t width, uint32_t write, uint32_t lane_a, uint32_t lane_b, uint32_t iters, uint32_t *sink,
                 void *stream);

#ifdef __cplusplus
}
#endif

#endif /* CP_PROBE_H */
