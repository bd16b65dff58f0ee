// Launch-side pieces shared between the library's translation units (not
// part of the C ABI): the current device's compute-unit count and the
// short-row selection kernel's launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <cstring>

#include "exact_topk.h"

namespace topk {

// Compute units of the current device when it is a gfx950 (cached per
// device); 0 when no device is current or it is another target: the library
// holds gfx950 code only. Entry points return TOPK_ERR_DEVICE then.
inline int device_cus() {
    static std::atomic<int> cached[64];  // 0 not yet asked, -1 unusable, else CUs
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (dev >= 0 && dev < 64) {
        const int v = cached[dev].load(std::memory_order_relaxed);
        if (v != 0) return v > 0 ? v : 0;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
    const bool gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 &&
                        (prop.gcnArchName[6] == '\0' || prop.gcnArchName[6] == ':');
    const int n = gfx950 && prop.multiProcessorCount > 0 ? prop.multiProcessorCount : -1;
    if (dev >= 0 && dev < 64) cached[dev].store(n, std::memory_order_relaxed);
    return n > 0 ? n : 0;
}

// Widest rows the short-row kernel takes: the automatic path of topk_select
// routes batches whose n_cols is at most this to it.
#ifndef TOPK_SHORT_MAX_COLS
#define TOPK_SHORT_MAX_COLS 32768
#endif
constexpr int64_t kShortMaxCols = TOPK_SHORT_MAX_COLS;

// Most rows one short-row launch takes (one 256-thread workgroup per row, a
// grid of at most 2^32 - 1 work-items); larger batches go to the persistent
// kernel.
constexpr int64_t kShortMaxBatch = 0xFFFFFFFFll / 256;

// Survivor entries the short-row kernel holds in LDS per row.
constexpr int32_t kShortCapacity = 3840;

// One workgroup per row: sample, one streaming pass into an LDS survivor
// buffer, exact selection there (full-row selection on overflow or
// underflow). Arguments as for topk_select_ex; the caller has checked all but
// the capacity (0 = kShortCapacity; above it TOPK_ERR_ARG). Returns a TOPK_*
// status.
int launch_short_rows(const float* scores, int64_t batch, int64_t row_stride, int64_t n_cols,
                      const int32_t* lengths, int32_t k, int32_t* out_idx, const int32_t* page_table,
                      int64_t page_table_stride, int32_t page_size, const topk_options& opt, hipStream_t stream);

// The same kernel over bf16 rows (bit patterns, 16-byte aligned rows with
// row_stride % 8 == 0): each score widened exactly to fp32, so the selection
// is the fp32 one on the widened row.
int launch_short_rows_bf16(const uint16_t* scores, int64_t batch, int64_t row_stride, int64_t n_cols,
                           const int32_t* lengths, int32_t k, int32_t* out_idx, const int32_t* page_table,
                           int64_t page_table_stride, int32_t page_size, const topk_options& opt,
                           hipStream_t stream);

}  // namespace topk
