// Launch-side pieces shared between the library's translation units (not
// part of the C ABI): the current device's compute-unit count and the
// short-row selection kernel's launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace topk {

// Compute units of the current device (cached per device), 0 on error.
inline int device_cus() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (dev >= 0 && dev < 64) {
        const int v = cached[dev].load(std::memory_order_relaxed);
        if (v > 0) return v;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (dev >= 0 && dev < 64) cached[dev].store(n, std::memory_order_relaxed);
    return n;
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

// One workgroup per row: sample, one streaming pass into an LDS survivor
// buffer, exact selection there (full-row selection on overflow or
// underflow). Arguments as for topk_select; the caller has checked them.
// Returns a TOPK_* status.
int launch_short_rows(const float* scores, int64_t batch, int64_t row_stride, int64_t n_cols,
                      const int32_t* lengths, int32_t k, int32_t* out_idx, const int32_t* page_table,
                      int64_t page_table_stride, int32_t page_size, int32_t* row_stats, hipStream_t stream);

// The same kernel over bf16 rows (bit patterns, 16-byte aligned rows with
// row_stride % 8 == 0): each score widened exactly to fp32, so the selection
// is the fp32 one on the widened row.
int launch_short_rows_bf16(const uint16_t* scores, int64_t batch, int64_t row_stride, int64_t n_cols,
                           const int32_t* lengths, int32_t k, int32_t* out_idx, const int32_t* page_table,
                           int64_t page_table_stride, int32_t page_size, hipStream_t stream);

}  // namespace topk
