/*
 * cp.h - C interface of the Conditional Program (CP) row-decode library for
 * AMD Instinct MI355X (gfx950).
 *
 * CP stores each row e_i of a hashed n-gram lookup table as an independently
 * addressable record {c_i, alpha_i}: a short trellis code and one bf16 scale.
 * One reconstruction rule f, shared by the whole table, rebuilds a requested
 * row as e_hat_i = alpha_i * f(c_i); only the rows a batch asks for are
 * fetched and decoded, and they come back in the order they were asked for.
 *   - reconstruction and storage cost (b + 16/d bits per parameter):
 *     "2비트 코드와 공유 트렐리스로 n-gram 룩업 테이블을 4~8배 압축한다"
 *     (onedev.kr paper digest), section "How it works" (어떻게 동작하나);
 *   - tail-biting Gaussian HYB bitshift trellis, no rotation, norm-restoring
 *     scale, records fetched and decoded by a fused kernel and returned in
 *     lookup order: same page, section "How it differs" (무엇과 다른가);
 *   - the scale is a bf16: same page, section "How it is used" (어떻게 쓰나).
 *
 * The pages name the trellis but do not give its parameters. This library
 * reads it as follows (the same reading is stated wherever it is used):
 *   - d outputs per row, V = 2 outputs per step, T = d/2 steps, kv code bits
 *     per step ("bits_per_step"; kv/2 bits per element), N = kv*T code bits;
 *   - the code is one little-endian N-bit integer (bit j = bit j&7 of byte
 *     j>>3); step t reads the 16-bit window s_t = bits [kv(t+1)-16, kv(t+1))
 *     of the circular code, oldest bit lowest (tail-biting: indices mod N);
 *   - h = (s*s + s) mod 2^32, idx = (h >> 7) & 511; outputs 2t and 2t+1 are
 *     LUT[idx][0] and LUT[idx][1] (fp16), both negated when bit 15 of s is 1;
 *   - e_hat = bf16_rne(alpha * f): the exact product rounded once to nearest
 *     even. A bf16 times an fp16 has at most 19 significant bits, so the
 *     kernels form it in fp32, where it is exact unless it lies below 2^-126;
 *     rows whose scale is below 2^-102 (the only ones where that can happen)
 *     are rounded from a copy scaled by 2^64 instead, so every row is the
 *     single rounding of the exact product.
 *
 * Record layout (this library's choice): N/8 code bytes, then alpha as a
 * little-endian bf16; records packed back to back with no padding, record i
 * at byte offset i * cp_record_bytes(d, kv) (a mixed-rate table packs records
 * of different sizes; see cp_mixed_desc).
 *
 * Error convention: every call returns a cp_status; nothing aborts. A status
 * of CP_ERR_HIP keeps the HIP error code for cp_last_hip_error() (per
 * thread). Ids outside [0, rows) do not fault: their output row is written
 * as zeros (like a lookup into a removed table, which the pages use as a
 * baseline, "How it is used") and a sticky per-table flag is raised, which
 * cp_table_check() reports and clears.
 *
 * Threading: lookups only read the table and may run concurrently on any
 * streams. cp_table_upload, cp_table_encode and cp_table_destroy write or free
 * the table and must not overlap lookups of the rows they touch; the caller
 * synchronises (cp_table_set_hot_rows and cp_table_download synchronise the
 * device themselves).
 *
 * Devices: a table lives on the device that was current at creation. Every
 * call that touches it makes that device current for the duration of the
 * call and restores the caller's device afterwards; a stream passed in must
 * belong to the table's device.
 */
#ifndef CP_H
#define CP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct cp_table cp_table; /* opaque; owned by the library */

typedef enum {
    CP_OK = 0,
    CP_ERR_INVALID_ARGUMENT = 1, /* NULL pointer, size mismatch, bad descriptor */
    CP_ERR_UNSUPPORTED = 2,      /* no kernel for the shape, or the call does not apply to this table */
    CP_ERR_OUT_OF_MEMORY = 3,    /* device or pinned host allocation failed */
    CP_ERR_HIP = 4,              /* a HIP runtime call failed; see cp_last_hip_error */
    CP_ERR_ID_OUT_OF_RANGE = 5,  /* reported by cp_table_check: some id was outside [0, rows) */
    /* not a status: makes every nonnegative 32-bit value a valid cp_status, so
     * cp_status_string may be handed any such code (it names unknown ones) */
    CP_STATUS_MAX_ENUM = 0x7FFFFFFF
} cp_status;

typedef enum {
    CP_RESIDENCY_DEVICE = 0,     /* records in device memory (HBM) */
    CP_RESIDENCY_HOST_MAPPED = 1 /* records in pinned host memory, read by the kernel over PCIe */
} cp_residency;

enum {
    /* with CP_RESIDENCY_HOST_MAPPED: allocate the pinned memory non-coherent,
     * so the GPU may cache records it has read */
    CP_FLAG_HOST_NONCOHERENT = 1u << 0,
    /* with CP_RESIDENCY_DEVICE (single-rate tables): in lookups that take
     * more than one round of workgroups, the first round also reads the ids
     * and touches the record lines of the later rounds' lookups, so that
     * records not in the caches come from HBM in one burst before the output
     * stream is under way. Pays when a lookup starts with none of the table in
     * the caches (after other kernels; the replay's launch drops from ~90 to
     * ~80 us on MI355X), costs a few percent when lookups of the same rows run
     * back to back. Results are the same either way. */
    CP_FLAG_TOUCH_AHEAD = 1u << 1
};

typedef struct {
    uint32_t struct_size;   /* sizeof(cp_table_desc) */
    uint32_t d;             /* outputs per row: 64, 128, 256 or 512 */
    uint32_t bits_per_step; /* kv: 3, 4, 5 or 6 (1.5, 2, 2.5, 3 bits per element) */
    uint32_t residency;     /* cp_residency */
    uint64_t rows;          /* records in the table, >= 1 */
    uint32_t flags;         /* CP_FLAG_* */
    uint32_t reserved;      /* 0 */
} cp_table_desc;

/* Shape of a mixed-rate table: every row has a rate class, and class c is
 * coded at bits_per_step[c]. The pages study giving rows bits by how often
 * they are looked up, over their code rates of 1.5 / 2 / 2.5 / 3 bits per
 * element ("How it is used"; "Assumptions and limits", which also warns that
 * the access counts behind such an allocation may not carry over between text
 * domains); they give no format. Here the records of all rows are packed in
 * row order, each at its own class's rate (cp_record_bytes(d, kv_c)), so a
 * row's record starts at the sum of the sizes of the records before it. */
typedef struct {
    uint32_t struct_size;      /* sizeof(cp_mixed_desc) */
    uint32_t d;                /* 64, 128, 256 or 512 */
    uint32_t nclass;           /* 1..4 rate classes */
    uint32_t bits_per_step[4]; /* kv of class c, 3..6; 0 for c >= nclass */
    uint32_t residency;        /* cp_residency */
    uint64_t rows;             /* >= 1 */
    uint32_t flags;            /* CP_FLAG_* */
    uint32_t reserved;         /* 0 */
} cp_mixed_desc;

/* Bytes of one record: kv*d/16 code bytes + 2 scale bytes, i.e. b + 16/d bits
 * per parameter at b = kv/2 ("How it works"). Returns 0 when (d, kv) cannot
 * form a whole-byte code of at least 16 bits. */
uint64_t cp_record_bytes(uint32_t d, uint32_t bits_per_step);

/* 1 when a kernel for (d, bits_per_step) is compiled in, else 0. */
int cp_supported(uint32_t d, uint32_t bits_per_step);

/* Creates a table on the current HIP device.
 *   desc     - shape and residency; copied.
 *   lut_fp16 - host pointer to the shared codebook, 512 x 2 fp16 bit patterns
 *              (entry idx: lut_fp16[2*idx], lut_fp16[2*idx+1]); copied. Every
 *              entry must be finite (the codebook of a Gaussian trellis).
 *   out      - receives the table handle (NULL on failure).
 * The records are not passed here: the table is created empty and
 * cp_table_upload (or cp_table_encode) fills it, in as many row ranges as the
 * caller likes, so a table of many GB never needs a second full copy in host
 * memory. They are uninitialised until then; device memory is rows * R bytes
 * (+ a small zeroed tail), pinned host memory the same for
 * CP_RESIDENCY_HOST_MAPPED.
 * Errors: INVALID_ARGUMENT (NULL pointers, struct_size, rows == 0, unknown
 * residency or flags (CP_FLAG_TOUCH_AHEAD with host residency), a codebook
 * entry that is +-inf or NaN), UNSUPPORTED,
 * OUT_OF_MEMORY (the records do not fit in device or pinned host memory; the
 * library stays usable), HIP. */
cp_status cp_table_create(const cp_table_desc *desc, const uint16_t *lut_fp16, cp_table **out);

/* Creates a mixed-rate table on the current HIP device.
 *   desc      - shape, rate classes and residency; copied.
 *   lut_fp16  - as in cp_table_create.
 *   row_class - host uint8[rows], the class (< nclass) of each row; read
 *               during the call only.
 * Besides the records (their total size follows from the classes) the table
 * keeps an index of 16 bytes per 32 rows in device memory (a byte offset and
 * two class bit planes per block of rows), from which a lookup finds any
 * record with a few popcounts. cp_table_upload / cp_table_download /
 * cp_lookup_decode / cp_lookup_decode_raw / cp_table_check /
 * cp_table_destroy work as for single-rate tables (record ranges given by the
 * rows' own sizes); cp_table_encode codes each row at its own class's rate;
 * cp_table_describe reports bits_per_step = 0; cp_lookup_decode_dedup and
 * cp_lookup_decode_dedup_noalloc stage the batch's distinct records, each at
 * its own size, as a mixed-rate table of their own and decode that.
 * Errors: INVALID_ARGUMENT (NULL pointers, struct_size, rows == 0, nclass, a
 * codebook entry that is +-inf or NaN,
 * a class's rate without whole-byte records, a nonzero unused rate, a row
 * class >= nclass, residency or flags), UNSUPPORTED (no kernel for d or a
 * rate), OUT_OF_MEMORY, HIP. */
cp_status cp_table_create_mixed(const cp_mixed_desc *desc, const uint16_t *lut_fp16, const uint8_t *row_class,
                                cp_table **out);

/* Byte offset and size of row `row`'s record within the table's packed
 * records (row * R and R for a single-rate table).
 * Errors: INVALID_ARGUMENT (NULL pointers, row >= rows). */
cp_status cp_table_record_range(const cp_table *table, uint64_t row, uint64_t *offset, uint64_t *bytes);

/* Copies records [first_row, first_row + nrows) from host memory `src`
 * (the rows' packed records: nrows * R bytes, or the sum of the rows' own
 * sizes for a mixed-rate table) into the table. Synchronous: the data
 * has landed when it returns. nrows == 0 is a no-op.
 * Errors: INVALID_ARGUMENT (NULL table/src, range beyond rows), HIP. */
cp_status cp_table_upload(cp_table *table, uint64_t first_row, uint64_t nrows, const void *src);

/* The hot path: for j in [0, n), out[j][0..d) = bf16 bits of
 * alpha_{ids[j]} * f(c_{ids[j]}) ("How it works", "How it differs").
 *   ids    - device-accessible int64[n], row ids in lookup order; read only.
 *   out    - device-accessible uint16[n][d] (bf16 bit patterns), row-major,
 *            16-byte aligned; fully overwritten.
 *   stream - hipStream_t to launch on (NULL: the null stream). Asynchronous:
 *            returns after the launch; synchronise the stream before reading.
 * Duplicate ids decode once per occurrence. n == 0 launches nothing; any
 * larger n is accepted (beyond 2^31 - 1 workgroups the kernel's chunk loop
 * strides over the rest). The call allocates nothing and does not
 * synchronise, so it may be captured in a HIP graph.
 * Errors: INVALID_ARGUMENT (NULL table, NULL ids/out with n > 0, misaligned
 * out), HIP (launch failure). Bad ids: see the error convention above. */
cp_status cp_lookup_decode(const cp_table *table, const int64_t *ids, uint64_t n, uint16_t *out,
                           void *stream);

/* As cp_lookup_decode, but writes the unscaled f(c) as fp16 bit patterns
 * (exactly the shared-codebook values, sign applied); used to check the
 * trellis walk bit for bit. */
cp_status cp_lookup_decode_raw(const cp_table *table, const int64_t *ids, uint64_t n,
                               uint16_t *out_fp16, void *stream);

/* Device workspace bytes that cp_lookup_decode_dedup needs for a batch of n
 * lookups on this table (0 for a NULL table). About 36 bytes per lookup plus
 * n records: 71 MB for n = 393,216 at d = 512, kv = 4 (a mixed-rate table:
 * about 37 bytes per lookup plus n of its largest records). */
uint64_t cp_dedup_workspace_bytes(const cp_table *table, uint64_t n);

/* Same result as cp_lookup_decode, fetching each distinct record of the batch
 * only once: the valid ids are deduplicated in a hash table in `workspace`,
 * each distinct record is copied once from the table into a staging area in
 * `workspace`, and the rows are decoded from there in the original lookup
 * order. Meant for a table in pinned host memory, where every record read
 * crosses PCIe (the pages find that regime dominated by the fetch and the
 * row-wise layout's advantage growing there: "Assumptions and limits").
 * Mixed-rate tables too: the distinct records are staged packed, each at its
 * own class's size, with an index of their own, and decoded by the
 * mixed-rate kernel.
 *   workspace       - device memory, 256-byte aligned, at least
 *                     cp_dedup_workspace_bytes(table, n) bytes, caller-owned;
 *                     its contents are scratch (undefined after the call).
 *                     Calls that share a workspace must not overlap.
 *   ids, out, stream - as in cp_lookup_decode; n < 2^31.
 * Asynchronous on `stream` (several kernels, no allocation, no host sync).
 * Out-of-range ids give zero rows and raise the table's sticky flag.
 * Errors: INVALID_ARGUMENT (as cp_lookup_decode, or workspace NULL, unaligned
 * or too small), HIP. */
cp_status cp_lookup_decode_dedup(const cp_table *table, const int64_t *ids, uint64_t n, uint16_t *out,
                                 void *workspace, uint64_t workspace_bytes, void *stream);

/* Largest batch cp_lookup_decode_dedup_noalloc accepts. */
#define CP_DEDUP_NOALLOC_MAX_IDS 65536u

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * result as cp_lookup_decode_dedup, with its scratch (hash table, staging
 * area) in a fixed device array that the library holds on each device it
 * runs on until the process ends (about 16.8 MB per device, enough for
 * CP_DEDUP_NOALLOC_MAX_IDS lookups of any supported record size, single- or
 * mixed-rate). The call
 * allocates nothing: no hipMalloc, no hipFree, no memset; it launches kernels
 * on `stream` only (the first call on a device also looks up the array's
 * address once).
 *   ids, out, stream - as in cp_lookup_decode; 1 <= n <= CP_DEDUP_NOALLOC_MAX_IDS.
 * All calls on one device share that array, which keeps the last call's
 * contents: calls that overlap on one device (concurrent streams or host
 * threads) race and give undefined rows; serialise them.
 * Errors: INVALID_ARGUMENT (as cp_lookup_decode_dedup, or n above
 * CP_DEDUP_NOALLOC_MAX_IDS), HIP. */
cp_status cp_lookup_decode_dedup_noalloc(const cp_table *table, const int64_t *ids, uint64_t n, uint16_t *out,
                                         void *stream);

/* Copies records [first_row, first_row + nrows) of the table to host memory
 * `dst` (nrows * R bytes, packed records). Waits for all work on the table's
 * device first, so records written by cp_table_encode on any stream are
 * included. nrows == 0 is a no-op.
 * Errors: INVALID_ARGUMENT (NULL table/dst, range beyond rows), HIP. */
cp_status cp_table_download(const cp_table *table, uint64_t first_row, uint64_t nrows, void *dst);

/* Device workspace bytes that cp_table_encode needs for nrows rows on this
 * table (0 for a NULL table or nrows == 0): one byte per trellis memory and
 * step, (d / 2) * 2^(16 - kv) bytes, for each row encoded concurrently (at
 * most one per resident workgroup: one per compute unit at kv 3 and 4, two
 * at kv 5 and 6), 1 MB per concurrent row at d = 512, kv = 4; for a
 * mixed-rate table the largest such need of its
 * rates plus, per row, 12 bytes of row lists, a staged copy of the input row
 * (4d bytes) and a staged record. */
uint64_t cp_encode_workspace_bytes(const cp_table *table, uint64_t nrows);

/* Encodes rows e_j (fp32, device, row-major nrows x d) into records
 * [first_row, first_row + nrows) of the table: z = sqrt(d) e / ||e||, a
 * tail-biting trellis-coded quantisation of z on the table's trellis, and
 * alpha = ||e|| / ||f(c)|| rounded once to bf16 ("How it works", "How it
 * differs": magnitude split from content, TCQ on a tail-biting trellis, the
 * norm-restoring scale). The search is the two-pass tail-biting Viterbi
 * heuristic: a pass from every start over the steps rotated by half a row
 * picks the start memory, a pass from that memory alone picks the code. All
 * arithmetic is fp64 in a fixed order with fixed tie rules, so the records
 * are fully determined by the input. A row whose norm is zero or not finite
 * (a row of zeros, or one holding an inf or a NaN) is stored as the all-zero
 * code with alpha = 0. A scale too large for bf16 is stored as +inf.
 *   rows      - device fp32[nrows][d], 4-byte aligned; read only.
 *   workspace - device memory, 256-byte aligned, at least
 *               cp_encode_workspace_bytes(table, nrows) bytes, caller-owned
 *               scratch; calls sharing a workspace must not overlap.
 *   stream    - as in cp_lookup_decode. Asynchronous, except that for a
 *               mixed-rate table the call first copies its per-rate row lists
 *               into the workspace on `stream` and waits for that copy; no
 *               device allocation.
 * Lookups of the rows being encoded must not overlap the call.
 * Errors: INVALID_ARGUMENT (NULL table/rows/workspace, range beyond rows,
 * misaligned pointers, workspace too small, more than 2^32 - 1 rows at once
 * for a mixed-rate table), UNSUPPORTED (no encoder for the shape, or a table
 * with hot-row copies: set those after encoding), OUT_OF_MEMORY (host lists
 * of a mixed-rate table), HIP. */
cp_status cp_table_encode(cp_table *table, uint64_t first_row, uint64_t nrows, const float *rows, void *workspace,
                          uint64_t workspace_bytes, void *stream);

/* Keeps device-memory copies of the records of `rows` (host int64[count], any
 * order, repeats allowed) for a table in pinned host memory, so that lookups
 * of those rows read HBM instead of crossing PCIe. Meant for the rows looked
 * up most often: the pages name caching of hot rows, and note that the access
 * counts it rests on may change with the text a model serves ("Assumptions
 * and limits"; ai4snews digest, Perspective).
 *   - Replaces any previous set; count == 0 drops the copies.
 *   - Waits for the device first (no lookup may still read the old copies).
 *   - cp_lookup_decode / cp_lookup_decode_raw use the copies; results are the
 *     same as without them. cp_table_upload keeps the copies current.
 *   - Device memory: count * R bytes plus an index of 8 bytes per 32 rows.
 * Errors: INVALID_ARGUMENT (NULL table, NULL rows with count > 0, a row
 * outside [0, rows)), UNSUPPORTED (a table in device memory or a mixed-rate
 * table), OUT_OF_MEMORY, HIP. */
cp_status cp_table_set_hot_rows(cp_table *table, const int64_t *rows, uint64_t count);

/* Number of distinct rows with a device copy (0 for NULL or none). */
uint64_t cp_table_hot_rows(const cp_table *table);

/* ---------------------------------------------------------------------
 * A table sharded by rows over several GPUs: the steps each GPU runs.
 *
 * The pages run CP with the table split over 4 (or 8) GPUs of one node,
 * 12.7 GB on each ("2비트 코드와 공유 트렐리스로 n-gram 룩업 테이블을 4~8배
 * 압축한다", onedev.kr, section "Assumptions and limits"). Records are
 * independently addressable and only requested rows are decoded (same page,
 * "How it differs"), so a lookup moves records rather than decoded rows:
 *   1. the requester plans: cp_shard_plan groups its ids by owning shard;
 *   2. (the caller sends shard s the ids local_ids[start_s, start_s +
 *      counts[s]), start_s = counts[0] + ... + counts[s - 1]: an all-to-all)
 *   3. each owner copies the requested records: cp_table_gather_records;
 *   4. (the records come back in the same order: a second all-to-all, R
 *      bytes per lookup where a decoded row is 2 d)
 *   5. the requester decodes: cp_lookup_decode_staged on the received
 *      buffer, with the plan's positions, writes its rows in its original
 *      lookup order.
 * Steps 2 and 4 are the caller's (RCCL, or a copy when owners share a GPU).
 * The shards are tables of rows_per_shard rows (the last may be shorter)
 * with the same codebook and shape; shard s holds global rows
 * [s * rows_per_shard, (s + 1) * rows_per_shard).
 * --------------------------------------------------------------------- */

/* Largest number of shards cp_shard_plan takes. */
#define CP_MAX_SHARDS 64u

/* Device workspace bytes cp_shard_plan needs for n ids over `shards` shards
 * (0 when n == 0 or shards is 0 or above CP_MAX_SHARDS). */
uint64_t cp_shard_plan_workspace_bytes(uint64_t n, uint32_t shards);

/* Groups a batch of global row ids by owning shard, keeping batch order
 * within each shard (a stable counting sort), on the current device.
 *   ids       - device int64[n], 8-byte aligned; global row ids.
 *   n         - 0 <= n <= 2^31 - 1.
 *   rows_per_shard, shards - the owner of id i is i / rows_per_shard when
 *               0 <= i < shards * rows_per_shard; other ids belong to no
 *               shard. 1 <= shards <= CP_MAX_SHARDS.
 *   local_ids - device int64[n] (written: the first counts[0] + ... +
 *               counts[shards - 1] entries): the valid ids grouped by
 *               shard, shard 0 first, each as its row within its shard.
 *   positions - device int64[n]: positions[j] = the index in local_ids of
 *               lookup j's entry (= where its record will sit in the
 *               received buffer), or -1 for an id no shard owns.
 *   counts    - device uint64[shards]: valid ids per shard.
 *   workspace - device, 256-byte aligned, >= cp_shard_plan_workspace_bytes.
 * Asynchronous on `stream`; allocates nothing. The result does not depend on
 * how the GPU schedules the work (stable order).
 * Errors: INVALID_ARGUMENT (NULL or misaligned pointers, n too large,
 * shards out of range, rows_per_shard == 0 or shards * rows_per_shard
 * above 2^64 - 1, workspace too small), HIP. */
cp_status cp_shard_plan(const int64_t *ids, uint64_t n, uint64_t rows_per_shard, uint32_t shards, int64_t *local_ids,
                        int64_t *positions, uint64_t *counts, void *workspace, uint64_t workspace_bytes,
                        void *stream);

/* The owner's step: copies the records of rows ids[0..n) of the table into
 * `dst` (device, 2-byte aligned), packed: record k at bytes [k R, k R + R).
 * An id outside [0, rows) writes a zero record and raises the table's flag
 * (cp_table_check). Rows of a pinned-host table are read over PCIe (its
 * device copies of hot rows hold the same bytes). A 16-byte aligned `dst` is
 * written in whole 16-byte stores only (else each group of 16 records also
 * has two partial ones). Asynchronous on `stream`.
 * Errors: INVALID_ARGUMENT (NULL table, NULL or misaligned ids / dst),
 * UNSUPPORTED (a mixed-rate table), HIP. */
cp_status cp_table_gather_records(cp_table *table, const int64_t *ids, uint64_t n, void *dst, void *stream);

/* The requester's step: decodes received records. `records` (device,
 * 16-byte aligned) holds nrecords packed records of this table's shape (R
 * bytes each) followed by at least 64 readable bytes (loads of the last
 * record may touch up to 7 bytes past it; their values do not matter).
 * Row j of `out` (bf16 [n][d], 16-byte aligned) becomes alpha * f(c) of
 * record positions[j] (device int64[n], 8-byte aligned), decoded with this
 * table's codebook exactly as cp_lookup_decode decodes a row; a position
 * outside [0, nrecords) gives a zero row and raises the table's flag.
 * Asynchronous on `stream`; allocates nothing.
 * Errors: INVALID_ARGUMENT (NULL table, NULL or misaligned pointers),
 * UNSUPPORTED (a mixed-rate table), HIP. */
cp_status cp_lookup_decode_staged(const cp_table *table, const void *records, uint64_t nrecords,
                                  const int64_t *positions, uint64_t n, uint16_t *out, void *stream);

/* Synchronises `stream`, then returns CP_ERR_ID_OUT_OF_RANGE and clears the
 * table's flag if any lookup since the last check saw an id outside
 * [0, rows); otherwise CP_OK. Errors: INVALID_ARGUMENT, HIP. */
cp_status cp_table_check(cp_table *table, void *stream);

/* Reads back the table's shape. Errors: INVALID_ARGUMENT. */
cp_status cp_table_describe(const cp_table *table, cp_table_desc *desc_out);

/* Reads back the shape with its rate classes (a single-rate table reports one
 * class). Errors: INVALID_ARGUMENT. */
cp_status cp_table_describe_mixed(const cp_table *table, cp_mixed_desc *desc_out);

/* Frees the table (no pending lookups may use it). NULL is a no-op (CP_OK). */
cp_status cp_table_destroy(cp_table *table);

/* Static text for a status code. */
const char *cp_status_string(cp_status status);

/* hipError_t of the last CP_ERR_HIP on the calling thread (0 if none). */
int cp_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CP_H */
