// Internal interface between the C-ABI layer (cp_api.hip) and the kernels
// (cp_decode.hip). Not installed; not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpk {

// Launch parameters of one gather-decode call.
struct LaunchArgs {
    const uint8_t *records;   // device-accessible base of the packed records
    uint64_t rows;
    const uint32_t *lut;      // device copy of the 512-entry codebook (fp16 pairs)
    const int64_t *ids;
    uint64_t n;
    uint32_t *out;            // n * d / 2 dwords (pairs of bf16 or fp16)
    int *err;                 // sticky out-of-range flag
    int num_cus;              // compute units of the device
    hipStream_t stream;
};

// True when a kernel for (d, kv) is compiled in.
bool supported(uint32_t d, uint32_t kv);

// Launches the gather-decode kernel; raw selects fp16 f(c) output instead of
// bf16 alpha * f(c). Returns the launch's hipError_t.
hipError_t launch(uint32_t d, uint32_t kv, bool raw, const LaunchArgs &a);

}  // namespace cpk
