// cp_api.hip - the C ABI of the CP row-decode library (declared in
// include/cp.h): argument checks, table memory, upload, launch, error flag.
// All arithmetic of the lookup runs in the kernels of cp_decode.hip.
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "../../include/cp.h"
#include "cp_internal.h"

struct cp_table {
    cp_table_desc desc;     // bits_per_step = 0 for a mixed-rate table
    uint64_t record_bytes;  // single-rate tables; 0 for a mixed-rate table
    uint64_t alloc_bytes;
    uint64_t records_bytes;  // bytes of all records (without the tail pad)
    // mixed-rate tables
    uint32_t mixed, nclass;
    uint32_t kv_of_class[4];
    cpk::MixedRates rates;
    cpk::MixedEntry *index_dev;
    cpk::MixedEntry *index_host;
    // hot-row cache of a host-resident table (none when hot_count == 0)
    uint64_t hot_count;
    cpk::HotEntry *hot_index_dev;
    cpk::HotEntry *hot_index_host;
    uint8_t *hot_recs;  // device copies of the hot rows' records, in row order
    uint8_t *records;      // hipMalloc'd (device) or hipHostMalloc'd (host)
    uint8_t *records_dev;  // device-accessible address of the same memory
    uint32_t *lut_dev;
    int *err_dev;
    int device;
    int num_cus;
};

static thread_local int g_last_hip_error = 0;

// Records a failed HIP call's error for cp_last_hip_error and takes it off
// the runtime's per-thread "last error", so that neither the caller's next
// hipGetLastError nor a later launch check of this library reports it again.
static cp_status hip_fail(hipError_t e)
{
    g_last_hip_error = (int)e;
    (void)hipGetLastError();
    return (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation) ? CP_ERR_OUT_OF_MEMORY
                                                                         : CP_ERR_HIP;
}

// Makes the table's device current for the duration of a call and restores
// the caller's device afterwards (launches on the null stream, copies and
// synchronisation then all address the device that holds the table). It
// also clears the runtime's per-thread "last error" first: the launches read
// their status with hipGetLastError, which would otherwise return an earlier
// failure of an unrelated call as their own.
struct DeviceGuard {
    int prev = -1;
    hipError_t err = hipSuccess;
    explicit DeviceGuard(int dev)
    {
        (void)hipGetLastError();
        int cur = -1;
        err = hipGetDevice(&cur);
        if (err == hipSuccess && cur != dev) {
            err = hipSetDevice(dev);
            if (err == hipSuccess) prev = cur;
        }
    }
    ~DeviceGuard()
    {
        if (prev >= 0) (void)hipSetDevice(prev);
    }
};

// Bytes after the last record that loads of the last record may touch
// (aligned dwords straddling the record end); zeroed at creation.
static constexpr uint64_t kTailPad = 64;

extern "C" {

uint64_t cp_record_bytes(uint32_t d, uint32_t bits_per_step)
{
    if (d == 0 || (d & 1u) || bits_per_step < 1 || bits_per_step > 15) return 0;
    const uint64_t nbits = (uint64_t)bits_per_step * (d / 2);
    if (nbits < 16 || nbits % 8) return 0;
    return nbits / 8 + 2;
}

int cp_supported(uint32_t d, uint32_t bits_per_step)
{
    return cp_record_bytes(d, bits_per_step) != 0 && cpk::supported(d, bits_per_step);
}

const char *cp_status_string(cp_status s)
{
    switch (s) {
    case CP_OK: return "ok";
    case CP_ERR_INVALID_ARGUMENT: return "invalid argument";
    case CP_ERR_UNSUPPORTED: return "unsupported (d, bits_per_step)";
    case CP_ERR_OUT_OF_MEMORY: return "out of memory";
    case CP_ERR_HIP: return "HIP runtime error";
    case CP_ERR_ID_OUT_OF_RANGE: return "a lookup id was outside [0, rows)";
    case CP_STATUS_MAX_ENUM: break;
    }
    return "unknown status";
}

int cp_last_hip_error(void) { return g_last_hip_error; }

static void drop_hot(cp_table *t)
{
    if (t->hot_index_dev) (void)hipFree(t->hot_index_dev);
    if (t->hot_recs) (void)hipFree(t->hot_recs);
    free(t->hot_index_host);
    t->hot_index_dev = nullptr;
    t->hot_recs = nullptr;
    t->hot_index_host = nullptr;
    t->hot_count = 0;
}

static void release(cp_table *t)
{
    if (!t) return;
    drop_hot(t);
    if (t->records) {
        if (t->desc.residency == CP_RESIDENCY_HOST_MAPPED)
            (void)hipHostFree(t->records);
        else
            (void)hipFree(t->records);
    }
    if (t->lut_dev) (void)hipFree(t->lut_dev);
    if (t->index_dev) (void)hipFree(t->index_dev);
    free(t->index_host);
    if (t->err_dev) (void)hipFree(t->err_dev);
    free(t);
}

// Allocates the record storage (rows' records + the zeroed tail pad), the
// codebook and the error flag of a table whose descriptor fields are set.
static cp_status allocate(cp_table *t, const uint16_t *lut_fp16)
{
    t->alloc_bytes = t->records_bytes + kTailPad;
    hipError_t e = hipGetDevice(&t->device);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&t->num_cus, hipDeviceAttributeMultiprocessorCount, t->device);
    if (e != hipSuccess) return hip_fail(e);
    if (t->desc.residency == CP_RESIDENCY_HOST_MAPPED) {
        unsigned flags = hipHostMallocMapped;
        if (t->desc.flags & CP_FLAG_HOST_NONCOHERENT) flags |= hipHostMallocNonCoherent;
        e = hipHostMalloc((void **)&t->records, t->alloc_bytes, flags);
        if (e == hipSuccess) e = hipHostGetDevicePointer((void **)&t->records_dev, t->records, 0);
        if (e == hipSuccess) memset(t->records + t->records_bytes, 0, kTailPad);
    } else {
        e = hipMalloc((void **)&t->records, t->alloc_bytes);
        t->records_dev = t->records;
        if (e == hipSuccess) e = hipMemset(t->records + t->records_bytes, 0, kTailPad);
    }
    if (e == hipSuccess) e = hipMalloc((void **)&t->lut_dev, 512 * sizeof(uint32_t));
    if (e == hipSuccess) e = hipMemcpy(t->lut_dev, lut_fp16, 512 * sizeof(uint32_t), hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMalloc((void **)&t->err_dev, sizeof(int));
    if (e == hipSuccess) e = hipMemset(t->err_dev, 0, sizeof(int));
    return e == hipSuccess ? CP_OK : hip_fail(e);
}

// The shared codebook holds the values of a Gaussian trellis (onedev.kr
// digest, "How it differs"): every entry must be a finite fp16 (exponent
// field below 31), which the tiny-scale arithmetic of the kernels relies on.
static bool finite_codebook(const uint16_t *lut_fp16)
{
    for (int i = 0; i < 1024; ++i)
        if ((lut_fp16[i] & 0x7C00u) == 0x7C00u) return false;
    return true;
}

static bool valid_residency(uint32_t residency, uint32_t flags)
{
    if (residency != CP_RESIDENCY_DEVICE && residency != CP_RESIDENCY_HOST_MAPPED) return false;
    if (residency == CP_RESIDENCY_HOST_MAPPED && (flags & CP_FLAG_TOUCH_AHEAD)) return false;
    return (flags & ~(uint32_t)(CP_FLAG_HOST_NONCOHERENT | CP_FLAG_TOUCH_AHEAD)) == 0;
}

cp_status cp_table_create(const cp_table_desc *desc, const uint16_t *lut_fp16, cp_table **out)
{
    if (out) *out = nullptr;
    if (!desc || !lut_fp16 || !out) return CP_ERR_INVALID_ARGUMENT;
    if (desc->struct_size != sizeof(cp_table_desc) || desc->rows == 0 || desc->reserved != 0)
        return CP_ERR_INVALID_ARGUMENT;
    if (!valid_residency(desc->residency, desc->flags) || !finite_codebook(lut_fp16)) return CP_ERR_INVALID_ARGUMENT;
    const uint64_t R = cp_record_bytes(desc->d, desc->bits_per_step);
    if (R == 0) return CP_ERR_INVALID_ARGUMENT;
    if (!cpk::supported(desc->d, desc->bits_per_step)) return CP_ERR_UNSUPPORTED;
    if (desc->rows > (UINT64_MAX - kTailPad) / R) return CP_ERR_INVALID_ARGUMENT;

    cp_table *t = (cp_table *)calloc(1, sizeof(cp_table));
    if (!t) return CP_ERR_OUT_OF_MEMORY;
    t->desc = *desc;
    t->record_bytes = R;
    t->records_bytes = desc->rows * R;
    const cp_status st = allocate(t, lut_fp16);
    if (st != CP_OK) {
        release(t);
        return st;
    }
    *out = t;
    return CP_OK;
}

cp_status cp_table_create_mixed(const cp_mixed_desc *desc, const uint16_t *lut_fp16, const uint8_t *row_class,
                                cp_table **out)
{
    if (out) *out = nullptr;
    if (!desc || !lut_fp16 || !row_class || !out) return CP_ERR_INVALID_ARGUMENT;
    if (desc->struct_size != sizeof(cp_mixed_desc) || desc->rows == 0 || desc->reserved != 0)
        return CP_ERR_INVALID_ARGUMENT;
    if (desc->nclass < 1 || desc->nclass > 4) return CP_ERR_INVALID_ARGUMENT;
    if (!valid_residency(desc->residency, desc->flags) || !finite_codebook(lut_fp16)) return CP_ERR_INVALID_ARGUMENT;
    if (desc->flags & CP_FLAG_TOUCH_AHEAD) return CP_ERR_INVALID_ARGUMENT;  // single-rate tables only
    uint32_t R[4] = {0, 0, 0, 0};
    for (uint32_t c = 0; c < desc->nclass; ++c) {
        R[c] = (uint32_t)cp_record_bytes(desc->d, desc->bits_per_step[c]);
        if (R[c] == 0) return CP_ERR_INVALID_ARGUMENT;
        if (!cpk::supported(desc->d, desc->bits_per_step[c])) return CP_ERR_UNSUPPORTED;
    }
    for (uint32_t c = desc->nclass; c < 4; ++c)
        if (desc->bits_per_step[c] != 0) return CP_ERR_INVALID_ARGUMENT;
    if (!cpk::mixed_supported(desc->d)) return CP_ERR_UNSUPPORTED;
    if (desc->rows > (UINT64_MAX - kTailPad) / 256) return CP_ERR_INVALID_ARGUMENT;

    cp_table *t = (cp_table *)calloc(1, sizeof(cp_table));
    if (!t) return CP_ERR_OUT_OF_MEMORY;
    t->desc.struct_size = sizeof(cp_table_desc);
    t->desc.d = desc->d;
    t->desc.bits_per_step = 0;
    t->desc.residency = desc->residency;
    t->desc.rows = desc->rows;
    t->desc.flags = desc->flags;
    t->mixed = 1;
    t->nclass = desc->nclass;
    t->rates.kv_packed = 0;
    for (uint32_t c = 0; c < 4; ++c) {
        t->kv_of_class[c] = desc->bits_per_step[c];
        t->rates.R[c] = R[c];
        t->rates.kv_packed |= (desc->bits_per_step[c] & 0xFFu) << (8 * c);
    }
    const uint64_t nidx = cpk::mixed_index_entries(desc->rows);
    t->index_host = (cpk::MixedEntry *)aligned_alloc(16, nidx * sizeof(cpk::MixedEntry));
    if (!t->index_host) {
        release(t);
        return CP_ERR_OUT_OF_MEMORY;
    }
    if (cpk::mixed_index_build(row_class, desc->rows, desc->nclass, R, t->index_host, &t->records_bytes) != 0) {
        release(t);
        return CP_ERR_INVALID_ARGUMENT;  // a class >= nclass
    }
    cp_status st = allocate(t, lut_fp16);
    if (st == CP_OK) {
        hipError_t e = hipMalloc((void **)&t->index_dev, nidx * sizeof(cpk::MixedEntry));
        if (e == hipSuccess)
            e = hipMemcpy(t->index_dev, t->index_host, nidx * sizeof(cpk::MixedEntry), hipMemcpyHostToDevice);
        if (e != hipSuccess) st = hip_fail(e);
    }
    if (st != CP_OK) {
        release(t);
        return st;
    }
    *out = t;
    return CP_OK;
}

// Byte range of records [first_row, first_row + nrows) (nrows >= 1, in range).
static void record_span(const cp_table *t, uint64_t first_row, uint64_t nrows, uint64_t *off, uint64_t *bytes)
{
    if (!t->mixed) {
        *off = first_row * t->record_bytes;
        *bytes = nrows * t->record_bytes;
        return;
    }
    const uint64_t last = first_row + nrows - 1;
    uint32_t cls = 0;
    const uint64_t a = cpk::mixed_record_offset(t->index_host, t->rates.R, first_row, nullptr);
    const uint64_t b = cpk::mixed_record_offset(t->index_host, t->rates.R, last, &cls);
    *off = a;
    *bytes = b + t->rates.R[cls] - a;
}

cp_status cp_table_record_range(const cp_table *t, uint64_t row, uint64_t *offset, uint64_t *bytes)
{
    if (!t || !offset || !bytes || row >= t->desc.rows) return CP_ERR_INVALID_ARGUMENT;
    record_span(t, row, 1, offset, bytes);
    return CP_OK;
}

// Slot of row r in the hot-row cache (r must be hot).
static uint64_t hot_slot(const cp_table *t, uint64_t r)
{
    const cpk::HotEntry &h = t->hot_index_host[r >> 5];
    const uint32_t j = (uint32_t)r & 31u;
    return h.base + (uint64_t)__builtin_popcount(h.bits & ((1u << j) - 1u));
}

static bool is_hot(const cp_table *t, uint64_t r) { return (t->hot_index_host[r >> 5].bits >> (r & 31u)) & 1u; }

// Copies the host records of the hot rows among [first_row, first_row + nrows)
// into their cache slots (consecutive rows' hot copies are consecutive slots).
static cp_status refresh_hot(cp_table *t, uint64_t first_row, uint64_t nrows)
{
    uint64_t lo = UINT64_MAX, hi = 0;
    for (uint64_t r = first_row; r < first_row + nrows; ++r) {
        if ((r & 31u) == 0 && t->hot_index_host[r >> 5].bits == 0 && r + 32 <= first_row + nrows) {
            r += 31;  // no hot row in this block
            continue;
        }
        if (!is_hot(t, r)) continue;
        if (lo == UINT64_MAX) lo = r;
        hi = r;
    }
    if (lo == UINT64_MAX) return CP_OK;
    const uint64_t R = t->record_bytes, s0 = hot_slot(t, lo), s1 = hot_slot(t, hi);
    uint8_t *stage = (uint8_t *)malloc((s1 - s0 + 1) * R);
    if (!stage) return CP_ERR_OUT_OF_MEMORY;
    for (uint64_t r = lo; r <= hi; ++r)
        if (is_hot(t, r)) memcpy(stage + (hot_slot(t, r) - s0) * R, t->records + r * R, R);
    hipError_t e = hipMemcpy(t->hot_recs + s0 * R, stage, (s1 - s0 + 1) * R, hipMemcpyHostToDevice);
    free(stage);
    return e == hipSuccess ? CP_OK : hip_fail(e);
}

cp_status cp_table_set_hot_rows(cp_table *t, const int64_t *rows, uint64_t count)
{
    if (!t || (count && !rows)) return CP_ERR_INVALID_ARGUMENT;
    if (t->mixed || t->desc.residency != CP_RESIDENCY_HOST_MAPPED) return CP_ERR_UNSUPPORTED;
    for (uint64_t i = 0; i < count; ++i)
        if (rows[i] < 0 || (uint64_t)rows[i] >= t->desc.rows) return CP_ERR_INVALID_ARGUMENT;
    DeviceGuard guard(t->device);
    hipError_t e = guard.err;
    if (e == hipSuccess) e = hipDeviceSynchronize();  // no lookup may still read the old cache
    if (e != hipSuccess) return hip_fail(e);
    drop_hot(t);
    if (count == 0) return CP_OK;
    const uint64_t nblk = (t->desc.rows + 31) / 32;
    t->hot_index_host = (cpk::HotEntry *)calloc(nblk, sizeof(cpk::HotEntry));
    if (!t->hot_index_host) return CP_ERR_OUT_OF_MEMORY;
    for (uint64_t i = 0; i < count; ++i) t->hot_index_host[rows[i] >> 5].bits |= 1u << (rows[i] & 31);
    uint64_t slots = 0;
    for (uint64_t b = 0; b < nblk; ++b) {
        if (slots > UINT32_MAX) {
            drop_hot(t);
            return CP_ERR_INVALID_ARGUMENT;  // more than 2^32 hot rows
        }
        t->hot_index_host[b].base = (uint32_t)slots;
        slots += (uint64_t)__builtin_popcount(t->hot_index_host[b].bits);
    }
    t->hot_count = slots;
    e = hipMalloc((void **)&t->hot_index_dev, nblk * sizeof(cpk::HotEntry));
    if (e == hipSuccess)
        e = hipMemcpy(t->hot_index_dev, t->hot_index_host, nblk * sizeof(cpk::HotEntry), hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMalloc((void **)&t->hot_recs, slots * t->record_bytes + kTailPad);
    if (e == hipSuccess) e = hipMemset(t->hot_recs + slots * t->record_bytes, 0, kTailPad);
    if (e != hipSuccess) {
        drop_hot(t);
        return hip_fail(e);
    }
    const cp_status st = refresh_hot(t, 0, t->desc.rows);
    if (st != CP_OK) drop_hot(t);
    return st;
}

uint64_t cp_table_hot_rows(const cp_table *t) { return t ? t->hot_count : 0; }

cp_status cp_table_upload(cp_table *t, uint64_t first_row, uint64_t nrows, const void *src)
{
    if (!t) return CP_ERR_INVALID_ARGUMENT;
    if (nrows == 0) return CP_OK;
    if (!src || first_row > t->desc.rows || nrows > t->desc.rows - first_row)
        return CP_ERR_INVALID_ARGUMENT;
    DeviceGuard guard(t->device);
    if (guard.err != hipSuccess) return hip_fail(guard.err);
    uint64_t off, bytes;
    record_span(t, first_row, nrows, &off, &bytes);
    if (t->desc.residency == CP_RESIDENCY_HOST_MAPPED) {
        memcpy(t->records + off, src, bytes);
        return t->hot_count ? refresh_hot(t, first_row, nrows) : CP_OK;
    }
    hipError_t e = hipMemcpy(t->records + off, src, bytes, hipMemcpyHostToDevice);
    return e == hipSuccess ? CP_OK : hip_fail(e);
}

static cp_status lookup(const cp_table *t, const int64_t *ids, uint64_t n, uint16_t *out, void *stream,
                        bool raw)
{
    if (!t) return CP_ERR_INVALID_ARGUMENT;
    if (n == 0) return CP_OK;
    if (!ids || !out || ((uintptr_t)out & 15u) || ((uintptr_t)ids & 7u)) return CP_ERR_INVALID_ARGUMENT;
    DeviceGuard guard(t->device);
    if (guard.err != hipSuccess) return hip_fail(guard.err);
    if (t->mixed) {
        cpk::MixedLaunchArgs m;
        m.records = t->records_dev;
        m.rows = t->desc.rows;
        m.lut = t->lut_dev;
        m.ids = ids;
        m.n = n;
        m.out = reinterpret_cast<uint32_t *>(out);
        m.err = t->err_dev;
        m.index = t->index_dev;
        m.rates = t->rates;
        m.num_cus = t->num_cus;
        m.stream = (hipStream_t)stream;
        hipError_t e = cpk::launch_mixed(t->desc.d, raw, m);
        return e == hipSuccess ? CP_OK : hip_fail(e);
    }
    cpk::LaunchArgs a;
    a.records = t->records_dev;
    if (t->hot_count) {
        const uintptr_t host = (uintptr_t)t->records_dev, hot = (uintptr_t)t->hot_recs;
        const uintptr_t base = host < hot ? host : hot;
        a.records = (const uint8_t *)base;
        a.hot_index = t->hot_index_dev;
        a.host_off0 = host - base;
        a.hot_off0 = hot - base;
    }
    a.rows = t->desc.rows;
    a.lut = t->lut_dev;
    a.ids = ids;
    a.n = n;
    a.by_offset = false;
    a.touch_ahead = (t->desc.flags & CP_FLAG_TOUCH_AHEAD) != 0;
    a.out = reinterpret_cast<uint32_t *>(out);
    a.err = t->err_dev;
    a.num_cus = t->num_cus;
    a.stream = (hipStream_t)stream;
    hipError_t e = cpk::launch(t->desc.d, t->desc.bits_per_step, raw, a);
    return e == hipSuccess ? CP_OK : hip_fail(e);
}

cp_status cp_lookup_decode(const cp_table *t, const int64_t *ids, uint64_t n, uint16_t *out, void *stream)
{
    return lookup(t, ids, n, out, stream, false);
}

cp_status cp_lookup_decode_raw(const cp_table *t, const int64_t *ids, uint64_t n, uint16_t *out_fp16,
                               void *stream)
{
    return lookup(t, ids, n, out_fp16, stream, true);
}

// largest record of a mixed-rate table's classes
static uint64_t mixed_max_record(const cp_table *t)
{
    uint64_t r = 0;
    for (uint32_t c = 0; c < 4; ++c) r = t->rates.R[c] > r ? t->rates.R[c] : r;
    return r;
}

static uint64_t dedup_total_bytes(const cp_table *t, uint64_t n)
{
    return t->mixed ? cpk::mixed_dedup_layout(n, mixed_max_record(t), kTailPad).total
                    : cpk::dedup_layout(n, t->record_bytes, kTailPad).total;
}

uint64_t cp_dedup_workspace_bytes(const cp_table *t, uint64_t n)
{
    if (!t) return 0;
    return dedup_total_bytes(t, n);
}

// Shared body of the two dedup entry points: `ws` is device memory of at
// least dedup_layout(n, R, kTailPad).total bytes, 256-byte aligned; the
// caller has checked the arguments and made the table's device current.
static cp_status dedup_lookup(const cp_table *t, const int64_t *ids, uint64_t n, uint16_t *out, uint8_t *ws,
                              void *stream)
{
    if (t->mixed) {
        // the distinct records staged as a mixed-rate table of their own,
        // decoded by staged row with the table's codebook and rates
        const cpk::MixedDedupLayout M = cpk::mixed_dedup_layout(n, mixed_max_record(t), kTailPad);
        cpk::MixedDedupArgs d;
        d.hash.records = t->records_dev;
        d.hash.rows = t->desc.rows;
        d.hash.record_bytes = 0;
        d.hash.ids = ids;
        d.hash.n = n;
        d.hash.workspace = ws;
        d.hash.layout = M.hash;
        d.hash.num_cus = t->num_cus;
        d.hash.stream = (hipStream_t)stream;
        d.layout = M;
        d.index = t->index_dev;
        d.rates = t->rates;
        d.tail_pad = kTailPad;
        hipError_t e = cpk::mixed_dedup_prepare(d);
        if (e != hipSuccess) return hip_fail(e);
        cpk::MixedLaunchArgs m;
        m.records = ws + M.staging;
        m.rows = n;  // staged rows are numbered below the batch size
        m.lut = t->lut_dev;
        m.ids = reinterpret_cast<const int64_t *>(ws + M.hash.staged_ids);
        m.n = n;
        m.out = reinterpret_cast<uint32_t *>(out);
        m.err = t->err_dev;
        m.index = reinterpret_cast<const cpk::MixedEntry *>(ws + M.index);
        m.rates = t->rates;
        m.num_cus = t->num_cus;
        m.stream = (hipStream_t)stream;
        e = cpk::launch_mixed(t->desc.d, false, m);
        return e == hipSuccess ? CP_OK : hip_fail(e);
    }
    const cpk::DedupLayout L = cpk::dedup_layout(n, t->record_bytes, kTailPad);
    cpk::DedupArgs d;
    d.records = t->records_dev;
    d.rows = t->desc.rows;
    d.record_bytes = t->record_bytes;
    d.ids = ids;
    d.n = n;
    d.workspace = ws;
    d.layout = L;
    d.num_cus = t->num_cus;
    d.stream = (hipStream_t)stream;
    hipError_t e = cpk::dedup_prepare(d);
    if (e != hipSuccess) return hip_fail(e);
    cpk::LaunchArgs a;
    a.records = ws + L.staging;
    a.rows = n;  // unused with by_offset
    a.lut = t->lut_dev;
    a.ids = reinterpret_cast<const int64_t *>(ws + L.staged_ids);  // record byte offsets in the staging area
    a.n = n;
    a.by_offset = true;
    a.out = reinterpret_cast<uint32_t *>(out);
    a.err = t->err_dev;
    a.num_cus = t->num_cus;
    a.stream = (hipStream_t)stream;
    e = cpk::launch(t->desc.d, t->desc.bits_per_step, false, a);
    return e == hipSuccess ? CP_OK : hip_fail(e);
}

static cp_status dedup_check(const cp_table *t, const int64_t *ids, uint64_t n, const uint16_t *out)
{
    if (!ids || !out || ((uintptr_t)out & 15u) || ((uintptr_t)ids & 7u)) return CP_ERR_INVALID_ARGUMENT;
    if (n > 0x7FFFFFFFull) return CP_ERR_INVALID_ARGUMENT;  // staging indices are 32-bit
    return CP_OK;
}

cp_status cp_lookup_decode_dedup(const cp_table *t, const int64_t *ids, uint64_t n, uint16_t *out,
                                 void *workspace, uint64_t workspace_bytes, void *stream)
{
    if (!t) return CP_ERR_INVALID_ARGUMENT;
    if (n == 0) return CP_OK;
    const cp_status st = dedup_check(t, ids, n, out);
    if (st != CP_OK) return st;
    if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < dedup_total_bytes(t, n))
        return CP_ERR_INVALID_ARGUMENT;
    DeviceGuard guard(t->device);
    if (guard.err != hipSuccess) return hip_fail(guard.err);
    return dedup_lookup(t, ids, n, out, static_cast<uint8_t *>(workspace), stream);
}

}  // extern "C"

// Scratch of cp_lookup_decode_dedup_noalloc: a file-scope device array sized
// for the largest batch it accepts with the largest record any supported
// shape has (d = 512 at 3 bits per element: 194 bytes), about 16.8 MB. The
// runtime places one copy on every device the library's code runs on, at an
// address of its own, and keeps it until the process ends. Host code never
// uses the array's name as an address (on the host it names a stand-in, not
// device memory): scratch_address() asks the runtime for this device's copy.
static constexpr uint64_t kNoallocMaxRecordBytes = 194;
static constexpr uint64_t kNoallocScratchBytes =
    cpk::dedup_layout(CP_DEDUP_NOALLOC_MAX_IDS, kNoallocMaxRecordBytes, kTailPad).total;
static_assert(cpk::mixed_dedup_layout(CP_DEDUP_NOALLOC_MAX_IDS, kNoallocMaxRecordBytes, kTailPad).total <=
                  kNoallocScratchBytes,
              "a mixed-rate table's dedup workspace fits the no-allocation scratch");
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

// Device address of `scratch` on the current device, looked up once per
// device (hipGetSymbolAddress with that device current) and kept.
static constexpr int kMaxDevices = 256;
static std::mutex g_scratch_mutex;
static uint8_t *g_scratch_ptr[kMaxDevices];

static hipError_t scratch_address(int device, uint8_t **ptr)
{
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[device]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[device] = static_cast<uint8_t *>(p);
    }
    *ptr = g_scratch_ptr[device];
    return hipSuccess;
}

extern "C" {

cp_status cp_lookup_decode_dedup_noalloc(const cp_table *t, const int64_t *ids, uint64_t n, uint16_t *out,
                                         void *stream)
{
    if (!t) return CP_ERR_INVALID_ARGUMENT;
    if (n == 0) return CP_OK;
    const cp_status st = dedup_check(t, ids, n, out);
    if (st != CP_OK) return st;
    if (n > CP_DEDUP_NOALLOC_MAX_IDS) return CP_ERR_INVALID_ARGUMENT;
    if (dedup_total_bytes(t, n) > kNoallocScratchBytes)
        return CP_ERR_INVALID_ARGUMENT;  // not reached: every supported record fits
    DeviceGuard guard(t->device);
    if (guard.err != hipSuccess) return hip_fail(guard.err);
    uint8_t *ws = nullptr;
    const hipError_t e = scratch_address(t->device, &ws);
    if (e != hipSuccess) return hip_fail(e);
    return dedup_lookup(t, ids, n, out, ws, stream);
}

cp_status cp_table_download(const cp_table *t, uint64_t first_row, uint64_t nrows, void *dst)
{
    if (!t) return CP_ERR_INVALID_ARGUMENT;
    if (nrows == 0) return CP_OK;
    if (!dst || first_row > t->desc.rows || nrows > t->desc.rows - first_row) return CP_ERR_INVALID_ARGUMENT;
    uint64_t off, bytes;
    record_span(t, first_row, nrows, &off, &bytes);
    DeviceGuard guard(t->device);
    hipError_t e = guard.err;
    if (e == hipSuccess) e = hipDeviceSynchronize();  // encodes in flight on any stream land first
    if (e != hipSuccess) return hip_fail(e);
    if (t->desc.residency == CP_RESIDENCY_HOST_MAPPED) {
        memcpy(dst, t->records + off, bytes);
        return CP_OK;
    }
    e = hipMemcpy(dst, t->records + off, bytes, hipMemcpyDeviceToHost);
    return e == hipSuccess ? CP_OK : hip_fail(e);
}

// Workspace of an encode call: for a mixed-rate table the per-class row lists
// (input row index, record offset) come first, then the back-pointers (sized
// for the largest need of any rate, each class being encoded in turn).
struct EncodeLayout {
    uint64_t src_row, dst_off, staged_rows, staged_recs, bp, total;
};

static hipError_t encode_layout(const cp_table *t, uint64_t nrows, EncodeLayout *L)
{
    uint64_t bp = 0;
    const uint32_t nclass = t->mixed ? t->nclass : 1;
    for (uint32_t c = 0; c < nclass; ++c) {
        const uint32_t kv = t->mixed ? t->kv_of_class[c] : t->desc.bits_per_step;
        uint32_t blocks = 0;
        const hipError_t e = cpk::encode_grid(kv, t->num_cus, nrows, &blocks);
        if (e != hipSuccess) return e;
        const uint64_t need = (uint64_t)blocks * cpk::encode_workspace_per_block(t->desc.d, kv);
        if (need > bp) bp = need;
    }
    auto up = [](uint64_t x) { return (x + 255) & ~(uint64_t)255; };
    uint64_t rmax = 0;
    for (uint32_t c = 0; c < nclass && t->mixed; ++c) rmax = t->rates.R[c] > rmax ? t->rates.R[c] : rmax;
    L->src_row = 0;
    L->dst_off = t->mixed ? up(nrows * sizeof(uint32_t)) : 0;
    L->staged_rows = t->mixed ? L->dst_off + up(nrows * sizeof(uint64_t)) : 0;
    L->staged_recs = t->mixed ? L->staged_rows + up(nrows * t->desc.d * sizeof(float)) : 0;
    L->bp = t->mixed ? L->staged_recs + up(nrows * rmax) : 0;
    L->total = L->bp + bp;
    return hipSuccess;
}

uint64_t cp_encode_workspace_bytes(const cp_table *t, uint64_t nrows)
{
    if (!t || nrows == 0) return 0;
    DeviceGuard guard(t->device);
    if (guard.err != hipSuccess) return 0;
    EncodeLayout L;
    if (encode_layout(t, nrows, &L) != hipSuccess) return 0;
    return L.total;
}

cp_status cp_table_encode(cp_table *t, uint64_t first_row, uint64_t nrows, const float *rows, void *workspace,
                          uint64_t workspace_bytes, void *stream)
{
    if (!t) return CP_ERR_INVALID_ARGUMENT;
    if (nrows == 0) return CP_OK;
    if (!rows || ((uintptr_t)rows & 3u) || first_row > t->desc.rows || nrows > t->desc.rows - first_row)
        return CP_ERR_INVALID_ARGUMENT;
    if (t->mixed && nrows > UINT32_MAX) return CP_ERR_INVALID_ARGUMENT;  // 32-bit row lists
    // a table with hot-row copies would need them refreshed after the kernel
    if (t->hot_count) return CP_ERR_UNSUPPORTED;
    for (uint32_t c = 0; c < (t->mixed ? t->nclass : 1); ++c)
        if (!cpk::encode_supported(t->desc.d, t->mixed ? t->kv_of_class[c] : t->desc.bits_per_step))
            return CP_ERR_UNSUPPORTED;
    DeviceGuard guard(t->device);
    if (guard.err != hipSuccess) return hip_fail(guard.err);
    EncodeLayout L;
    hipError_t e = encode_layout(t, nrows, &L);
    if (e != hipSuccess) return hip_fail(e);
    if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < L.total) return CP_ERR_INVALID_ARGUMENT;
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    const hipStream_t st = (hipStream_t)stream;
    if (!t->mixed) {
        uint32_t blocks = 0;
        e = cpk::encode_grid(t->desc.bits_per_step, t->num_cus, nrows, &blocks);
        if (e != hipSuccess) return hip_fail(e);
        cpk::EncodeArgs a;
        a.rows = rows;
        a.nrows = nrows;
        a.d = t->desc.d;
        a.kv = t->desc.bits_per_step;
        a.lut = t->lut_dev;
        a.out = t->records_dev + first_row * t->record_bytes;
        a.record_bytes = t->record_bytes;
        a.workspace = ws + L.bp;
        a.blocks = blocks;
        a.stream = st;
        e = cpk::encode(a);
        return e == hipSuccess ? CP_OK : hip_fail(e);
    }
    // mixed rates: the rows of each class, as (input row, record offset) lists
    uint32_t *src = (uint32_t *)malloc(nrows * sizeof(uint32_t));
    uint64_t *dst = (uint64_t *)malloc(nrows * sizeof(uint64_t));
    uint8_t *cls = (uint8_t *)malloc(nrows);
    if (!src || !dst || !cls) {
        free(src);
        free(dst);
        free(cls);
        return CP_ERR_OUT_OF_MEMORY;
    }
    uint64_t start[5] = {0, 0, 0, 0, 0};
    for (uint64_t r = 0; r < nrows; ++r) {
        uint32_t c = 0;
        (void)cpk::mixed_record_offset(t->index_host, t->rates.R, first_row + r, &c);
        cls[r] = (uint8_t)c;
        ++start[c + 1];
    }
    for (uint32_t c = 1; c < 5; ++c) start[c] += start[c - 1];
    uint64_t fill[4] = {start[0], start[1], start[2], start[3]};
    for (uint64_t r = 0; r < nrows; ++r) {
        const uint64_t k = fill[cls[r]]++;
        src[k] = (uint32_t)r;
        dst[k] = cpk::mixed_record_offset(t->index_host, t->rates.R, first_row + r, nullptr);
    }
    free(cls);
    // the lists land on the stream before the kernels; the host copies are freed
    // once they have
    e = hipMemcpyAsync(ws + L.src_row, src, nrows * sizeof(uint32_t), hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipMemcpyAsync(ws + L.dst_off, dst, nrows * sizeof(uint64_t), hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    free(src);
    free(dst);
    if (e != hipSuccess) return hip_fail(e);
    for (uint32_t c = 0; c < t->nclass; ++c) {
        const uint64_t cnt = start[c + 1] - start[c];
        if (cnt == 0) continue;
        uint32_t blocks = 0;
        e = cpk::encode_grid(t->kv_of_class[c], t->num_cus, cnt, &blocks);
        if (e != hipSuccess) return hip_fail(e);
        cpk::EncodeArgs a;
        a.rows = rows;
        a.nrows = cnt;
        a.d = t->desc.d;
        a.kv = t->kv_of_class[c];
        a.lut = t->lut_dev;
        a.out = t->records_dev;
        a.record_bytes = t->rates.R[c];
        a.workspace = ws + L.bp;
        a.blocks = blocks;
        a.stream = st;
        e = cpk::encode_listed(a, reinterpret_cast<const uint32_t *>(ws + L.src_row) + start[c],
                               reinterpret_cast<const uint64_t *>(ws + L.dst_off) + start[c],
                               reinterpret_cast<float *>(ws + L.staged_rows), ws + L.staged_recs);
        if (e != hipSuccess) return hip_fail(e);
    }
    return CP_OK;
}

uint64_t cp_shard_plan_workspace_bytes(uint64_t n, uint32_t shards)
{
    if (n == 0 || shards == 0 || shards > cpk::kMaxShards) return 0;
    return cpk::shard_plan_workspace_bytes(n, shards);
}

cp_status cp_shard_plan(const int64_t *ids, uint64_t n, uint64_t rows_per_shard, uint32_t shards, int64_t *local_ids,
                        int64_t *positions, uint64_t *counts, void *workspace, uint64_t workspace_bytes,
                        void *stream)
{
    if (shards == 0 || shards > cpk::kMaxShards || rows_per_shard == 0) return CP_ERR_INVALID_ARGUMENT;
    if (!counts || ((uintptr_t)counts & 7u)) return CP_ERR_INVALID_ARGUMENT;
    if (n > 0x7FFFFFFFull) return CP_ERR_INVALID_ARGUMENT;
    if (shards > UINT64_MAX / rows_per_shard) return CP_ERR_INVALID_ARGUMENT;  // shards * rows_per_shard overflows
    if (n > 0) {
        if (!ids || !local_ids || !positions || ((uintptr_t)ids & 7u) || ((uintptr_t)local_ids & 7u) ||
            ((uintptr_t)positions & 7u))
            return CP_ERR_INVALID_ARGUMENT;
        if (!workspace || ((uintptr_t)workspace & 255u) ||
            workspace_bytes < cpk::shard_plan_workspace_bytes(n, shards))
            return CP_ERR_INVALID_ARGUMENT;
    }
    (void)hipGetLastError();
    if (n == 0) {
        // nothing to sort: the counts are zero (a kernel, so the call stays
        // capturable and asynchronous like the others)
        cpk::ShardPlanArgs a{};
        a.counts = counts;
        a.shards = shards;
        a.stream = (hipStream_t)stream;
        const hipError_t e = cpk::shard_plan_zero_counts(a);
        return e == hipSuccess ? CP_OK : hip_fail(e);
    }
    cpk::ShardPlanArgs a;
    a.ids = ids;
    a.n = n;
    a.rows_per_shard = rows_per_shard;
    a.shards = shards;
    a.local_ids = local_ids;
    a.positions = positions;
    a.counts = counts;
    a.workspace = static_cast<uint8_t *>(workspace);
    a.stream = (hipStream_t)stream;
    const hipError_t e = cpk::shard_plan(a);
    return e == hipSuccess ? CP_OK : hip_fail(e);
}

cp_status cp_table_gather_records(cp_table *t, const int64_t *ids, uint64_t n, void *dst, void *stream)
{
    if (!t) return CP_ERR_INVALID_ARGUMENT;
    if (t->mixed) return CP_ERR_UNSUPPORTED;
    if (n == 0) return CP_OK;
    if (!ids || !dst || ((uintptr_t)ids & 7u) || ((uintptr_t)dst & 1u)) return CP_ERR_INVALID_ARGUMENT;
    DeviceGuard guard(t->device);
    if (guard.err != hipSuccess) return hip_fail(guard.err);
    // rows with device copies read the same bytes from the host records
    const hipError_t e = cpk::gather_records_launch(t->records_dev, t->desc.rows, t->record_bytes, ids, n,
                                                    static_cast<uint8_t *>(dst), t->err_dev, t->num_cus,
                                                    (hipStream_t)stream);
    return e == hipSuccess ? CP_OK : hip_fail(e);
}

cp_status cp_lookup_decode_staged(const cp_table *t, const void *records, uint64_t nrecords, const int64_t *positions,
                                  uint64_t n, uint16_t *out, void *stream)
{
    if (!t) return CP_ERR_INVALID_ARGUMENT;
    if (t->mixed) return CP_ERR_UNSUPPORTED;
    if (n == 0) return CP_OK;
    // the kernel's dword loads are aligned relative to the buffer's start
    if (!records || ((uintptr_t)records & 15u)) return CP_ERR_INVALID_ARGUMENT;
    if (!positions || !out || ((uintptr_t)out & 15u) || ((uintptr_t)positions & 7u)) return CP_ERR_INVALID_ARGUMENT;
    DeviceGuard guard(t->device);
    if (guard.err != hipSuccess) return hip_fail(guard.err);
    // the gather-decode kernel with the received buffer as the table: row j
    // of the output decodes record positions[j] (a position outside
    // [0, nrecords) gives a zero row and raises the flag)
    cpk::LaunchArgs a;
    a.records = static_cast<const uint8_t *>(records);
    a.rows = nrecords;
    a.lut = t->lut_dev;
    a.ids = positions;
    a.n = n;
    a.by_offset = false;
    a.out = reinterpret_cast<uint32_t *>(out);
    a.err = t->err_dev;
    a.num_cus = t->num_cus;
    a.stream = (hipStream_t)stream;
    const hipError_t e = cpk::launch(t->desc.d, t->desc.bits_per_step, false, a);
    return e == hipSuccess ? CP_OK : hip_fail(e);
}

cp_status cp_table_check(cp_table *t, void *stream)
{
    if (!t) return CP_ERR_INVALID_ARGUMENT;
    DeviceGuard guard(t->device);
    if (guard.err != hipSuccess) return hip_fail(guard.err);
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    int flag = 0;
    if (e == hipSuccess) e = hipMemcpy(&flag, t->err_dev, sizeof(int), hipMemcpyDeviceToHost);
    if (e == hipSuccess && flag) e = hipMemset(t->err_dev, 0, sizeof(int));
    if (e != hipSuccess) return hip_fail(e);
    return flag ? CP_ERR_ID_OUT_OF_RANGE : CP_OK;
}

cp_status cp_table_describe(const cp_table *t, cp_table_desc *desc_out)
{
    if (!t || !desc_out) return CP_ERR_INVALID_ARGUMENT;
    *desc_out = t->desc;
    return CP_OK;
}

cp_status cp_table_describe_mixed(const cp_table *t, cp_mixed_desc *desc_out)
{
    if (!t || !desc_out) return CP_ERR_INVALID_ARGUMENT;
    memset(desc_out, 0, sizeof(*desc_out));
    desc_out->struct_size = sizeof(cp_mixed_desc);
    desc_out->d = t->desc.d;
    desc_out->residency = t->desc.residency;
    desc_out->rows = t->desc.rows;
    desc_out->flags = t->desc.flags;
    if (t->mixed) {
        desc_out->nclass = t->nclass;
        for (uint32_t c = 0; c < 4; ++c) desc_out->bits_per_step[c] = t->kv_of_class[c];
    } else {
        desc_out->nclass = 1;
        desc_out->bits_per_step[0] = t->desc.bits_per_step;
    }
    return CP_OK;
}

cp_status cp_table_destroy(cp_table *t)
{
    if (!t) return CP_OK;
    hipError_t e;
    {
        DeviceGuard guard(t->device);
        e = guard.err;
        if (e == hipSuccess) e = hipDeviceSynchronize();
        release(t);
    }
    return e == hipSuccess ? CP_OK : hip_fail(e);
}

}  // extern "C"
