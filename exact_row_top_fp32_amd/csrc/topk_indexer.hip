// The kernels beside the fp32 selection in a two-level sparse-attention
// indexer, for gfx950 ("dsv4.1: Top-k kernels and candidate selection",
// implementation section 2 and code excerpts):
//
//  * bf16 top-k (topk_select_bf16): rows of at most 16384 scores, each
//    widened exactly to fp32 as it is loaded, selected by the short-row
//    kernel (one workgroup per row, sampled cutoff, survivors in LDS);
//  * amax8_kernel: the level-one keys, the largest of every 8 scores (NaN
//    ignored, +0 above -0) with the newest block +inf; a streaming kernel in
//    which two lanes read the two halves of a block, so that every wave load
//    covers 1 KB of consecutive scores, and one DPP step joins the halves;
//  * block_table_kernel: the selected block ids of a row in ascending order
//    by a bitmap counting sort in LDS, with their pool slots.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "exact_topk.h"
#include "topk_device.h"
#include "topk_short.h"

namespace topk {
namespace {

constexpr int kBfMaxCols = 16384;  // bf16 rows: at most this many scores

// ----------------------------------------------------------------------------
// block max of every 8 scores
// ----------------------------------------------------------------------------

constexpr int kAmaxThreads = 256;
constexpr int kAmaxPer = 4;                                 // blocks per lane: 8 per lane pair
constexpr int64_t kAmaxTile = kAmaxThreads * kAmaxPer;      // blocks per workgroup

struct Amax8Params {
    const float* scores;
    int64_t row_stride;
    int64_t n_cols;
    const int32_t* lengths;
    int32_t topk;
    float* out;
    int64_t out_stride;
    int64_t tiles;  // workgroups per row
};

// the largest key of a block, NaN as key 0 (below every number's key)
__device__ __forceinline__ uint32_t live_key(float x) { return x != x ? 0u : order_key(x); }

__global__ __launch_bounds__(kAmaxThreads) void amax8_kernel(Amax8Params p) {
    const int64_t b = blockIdx.x / (uint64_t)p.tiles;
    const int64_t tile = blockIdx.x % (uint64_t)p.tiles;
    int64_t L = p.lengths ? (int64_t)p.lengths[b] : p.n_cols;
    L = L < 0 ? 0 : (L > p.n_cols ? p.n_cols : L);
    const int64_t nb = (L + 7) >> 3;
    if (nb == 0 || (p.topk > 0 && nb <= p.topk)) return;
    const f4* row = reinterpret_cast<const f4*>(p.scores + b * p.row_stride);
    float* out = p.out + b * p.out_stride;
    // lane pairs share a block: lane t holds half (t & 1) of block
    // tile * kAmaxTile + j * 128 + t / 2, so each load of a wave reads 1 KB
    // of consecutive scores
    const int64_t blk0 = tile * kAmaxTile + (threadIdx.x >> 1);
    const uint32_t half = threadIdx.x & 1u;
    f4 x[2 * kAmaxPer];
#pragma unroll
    for (int j = 0; j < 2 * kAmaxPer; ++j) {
        const int64_t i = blk0 + j * (kAmaxThreads / 2);
        if (i < nb - 1) x[j] = load_nt(row + 2 * i + half);
    }
#pragma unroll
    for (int j = 0; j < 2 * kAmaxPer; ++j) {
        const int64_t i = blk0 + j * (kAmaxThreads / 2);
        uint32_t k = 0u;
        if (i < nb - 1) k = max(max(live_key(x[j].x), live_key(x[j].y)), max(live_key(x[j].z), live_key(x[j].w)));
        k = max(k, dpp<0xB1>(0u, k));  // quad_perm [1,0,3,2]: the pair's other half
        if (half == 0u) {
            if (i < nb - 1) {
                // key -> pattern: the inverse of order_key; an all-NaN block gives +qNaN
                const uint32_t bits = k == 0u ? 0x7FC00000u : ((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
                out[i] = __uint_as_float(bits);
            } else if (i == nb - 1) {
                out[i] = __builtin_inff();
            }
        }
    }
}

// ----------------------------------------------------------------------------
// candidate block table
// ----------------------------------------------------------------------------

constexpr int kTabThreads = 256;
constexpr int kTabMaxBlocks = 262144;              // blocks per row (2^21 positions)
constexpr int kTabWords = kTabMaxBlocks / 32;      // bitmap words
constexpr int32_t kPad = 0x7FFFFFFF;

struct TableParams {
    int32_t* blocks;  // [batch, k], rewritten in place
    int32_t k;
    const int32_t* lengths;
    int64_t n_cols;
    const int32_t* page_table;
    int64_t pt_stride;
    int32_t bpp;      // blocks per page
    int32_t* pages;   // [batch, k]
};

__global__ __launch_bounds__(kTabThreads) void block_table_kernel(TableParams p) {
    __shared__ uint32_t bitmap[kTabWords];
    __shared__ uint32_t wave_total[kTabThreads / 64];
    const int64_t b = blockIdx.x;
    int64_t L = p.lengths ? (int64_t)p.lengths[b] : p.n_cols;
    L = L < 0 ? 0 : (L > p.n_cols ? p.n_cols : L);
    const uint32_t nb = (uint32_t)((L + 7) >> 3);
    int32_t* table = p.blocks + b * (int64_t)p.k;
    int32_t* pages = p.pages + b * (int64_t)p.k;
    const int32_t* pt = p.page_table + b * p.pt_stride;
    const uint32_t bpp = (uint32_t)p.bpp;
    auto slot_of = [&](uint32_t id) {
        return (int32_t)((int64_t)pt[id / bpp] * (int64_t)bpp + (int64_t)(id % bpp));
    };
    if (nb <= (uint32_t)p.k) {  // every block: the identity table, input unread
        for (int j = (int)threadIdx.x; j < p.k; j += kTabThreads) {
            const bool live = (uint32_t)j < nb;
            table[j] = live ? j : kPad;
            pages[j] = live ? slot_of((uint32_t)j) : kPad;
        }
        return;
    }
    // bitmap of the ids in [0, nb) the row holds; lane t owns words
    // [t * per, t * per + per) of the nw in use
    const uint32_t nw = (nb + 31u) / 32u;
    const uint32_t per = (nw + kTabThreads - 1) / kTabThreads;
    for (uint32_t w = threadIdx.x; w < nw; w += kTabThreads) bitmap[w] = 0u;
    __syncthreads();
    for (int j = (int)threadIdx.x; j < p.k; j += kTabThreads) {
        const int32_t id = table[j];
        if (id >= 0 && (uint32_t)id < nb) atomicOr(&bitmap[(uint32_t)id >> 5], 1u << ((uint32_t)id & 31u));
    }
    __syncthreads();  // every read of the input row is done before it is rewritten
    const uint32_t w0 = threadIdx.x * per;
    uint32_t mine = 0u;
    for (uint32_t q = 0; q < per; ++q)
        if (w0 + q < nw) mine += (uint32_t)__popc(bitmap[w0 + q]);
    const uint32_t incl = wave_inclusive_sum(mine);
    if (lane_id() == 63) wave_total[wave_id()] = incl;
    __syncthreads();
    uint32_t before = incl - mine;
    for (uint32_t w = 0; w < wave_id(); ++w) before += wave_total[w];
    uint32_t total = 0u;
    for (int w = 0; w < kTabThreads / 64; ++w) total += wave_total[w];
    uint32_t rank = before;
    for (uint32_t q = 0; q < per; ++q) {
        if (w0 + q >= nw) break;
        uint32_t bits = bitmap[w0 + q];
        while (bits != 0u) {
            const uint32_t id = (w0 + q) * 32u + (uint32_t)__ffs(bits) - 1u;
            bits &= bits - 1u;
            if (rank < (uint32_t)p.k) {
                table[rank] = (int32_t)id;
                pages[rank] = slot_of(id);
            }
            ++rank;
        }
    }
    for (uint32_t j = total + threadIdx.x; j < (uint32_t)p.k; j += kTabThreads) {
        table[j] = kPad;
        pages[j] = kPad;
    }
}

}  // namespace
}  // namespace topk

using namespace topk;

extern "C" {

int topk_select_bf16_ex(const uint16_t* scores, int64_t batch, int64_t row_stride, int64_t n_cols,
                        const int32_t* lengths, int32_t k, int32_t* out_idx,
                        const int32_t* page_table, int64_t page_table_stride, int32_t page_size,
                        void* hip_stream, const topk_options* options) {
    if (batch < 0 || batch > (int64_t)(UINT32_MAX / 256)) return TOPK_ERR_ARG;
    if (k < 1 || k > TOPK_MAX_K) return TOPK_ERR_K;
    if (n_cols < 0 || n_cols > kBfMaxCols || row_stride < n_cols) return TOPK_ERR_ARG;
    topk_options opt{TOPK_PATH_AUTO, 0, nullptr, TOPK_KERNEL_AUTO};
    if (options != nullptr) opt = *options;
    if (opt.force_path < TOPK_PATH_AUTO || opt.force_path > TOPK_PATH_FULLROW) return TOPK_ERR_ARG;
    if (opt.capacity < 0 || opt.capacity > kShortCapacity) return TOPK_ERR_ARG;
    if (opt.kernel != TOPK_KERNEL_AUTO && opt.kernel != TOPK_KERNEL_SHORT) return TOPK_ERR_ARG;
    if (page_table != nullptr) {
        if (page_size < 1) return TOPK_ERR_ARG;
        if (page_table_stride < (n_cols + page_size - 1) / page_size) return TOPK_ERR_ARG;
    }
    if (batch == 0) return TOPK_OK;
    if (scores == nullptr || out_idx == nullptr) return TOPK_ERR_ARG;
    if ((reinterpret_cast<uintptr_t>(scores) & 15u) != 0) return TOPK_ERR_ALIGN;
    if (batch > 1 && (row_stride & 7) != 0) return TOPK_ERR_ALIGN;
    if (device_cus() <= 0) return TOPK_ERR_DEVICE;
    return launch_short_rows_bf16(scores, batch, row_stride, n_cols, lengths, k, out_idx, page_table,
                                  page_table_stride, page_size, opt, static_cast<hipStream_t>(hip_stream));
}

int topk_select_bf16(const uint16_t* scores, int64_t batch, int64_t row_stride, int64_t n_cols,
                     const int32_t* lengths, int32_t k, int32_t* out_idx,
                     const int32_t* page_table, int64_t page_table_stride, int32_t page_size,
                     void* hip_stream) {
    return topk_select_bf16_ex(scores, batch, row_stride, n_cols, lengths, k, out_idx, page_table,
                               page_table_stride, page_size, hip_stream, nullptr);
}

int amax8_varlen(const float* scores, int64_t batch, int64_t row_stride, int64_t n_cols, const int32_t* lengths,
                 int32_t topk, float* out, int64_t out_stride, void* hip_stream) {
    if (batch < 0 || batch > INT32_MAX || topk < 0) return TOPK_ERR_ARG;
    if (n_cols < 0 || n_cols > INT32_MAX || row_stride < n_cols) return TOPK_ERR_ARG;
    const int64_t blocks = (n_cols + 7) / 8;
    if (out_stride < blocks) return TOPK_ERR_ARG;
    if (batch == 0 || blocks == 0) return TOPK_OK;
    if (scores == nullptr || out == nullptr) return TOPK_ERR_ARG;
    if ((reinterpret_cast<uintptr_t>(scores) & 31u) != 0) return TOPK_ERR_ALIGN;
    if (batch > 1 && (row_stride & 7) != 0) return TOPK_ERR_ALIGN;
    const int64_t tiles = (blocks + kAmaxTile - 1) / kAmaxTile;
    if (batch * tiles * kAmaxThreads > (int64_t)UINT32_MAX) return TOPK_ERR_ARG;
    if (device_cus() <= 0) return TOPK_ERR_DEVICE;
    Amax8Params p{scores, row_stride, n_cols, lengths, topk, out, out_stride, tiles};
    void* args[] = {&p};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&amax8_kernel), dim3((uint32_t)(batch * tiles)),
                                         dim3(kAmaxThreads), args, 0, static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? TOPK_OK : TOPK_ERR_LAUNCH;
}

int sort_candidate_blocks(int32_t* blocks, int64_t batch, int32_t k, const int32_t* lengths, int64_t n_cols,
                          const int32_t* page_table, int64_t page_table_stride, int32_t page_size,
                          int32_t* out_pages, void* hip_stream) {
    if (batch < 0 || batch > (int64_t)(UINT32_MAX / kTabThreads) || k < 1) return TOPK_ERR_ARG;
    if (n_cols < 0 || n_cols > 8 * (int64_t)kTabMaxBlocks) return TOPK_ERR_ARG;
    if (page_size < 8 || (page_size & (page_size - 1)) != 0) return TOPK_ERR_ARG;
    const int64_t bpp = page_size / 8;
    const int64_t max_blocks = (n_cols + 7) / 8;
    if (page_table_stride < (max_blocks + bpp - 1) / bpp) return TOPK_ERR_ARG;
    if (batch == 0) return TOPK_OK;
    if (blocks == nullptr || page_table == nullptr || out_pages == nullptr) return TOPK_ERR_ARG;
    if (device_cus() <= 0) return TOPK_ERR_DEVICE;
    TableParams p{blocks, k, lengths, n_cols, page_table, page_table_stride, (int32_t)bpp, out_pages};
    void* args[] = {&p};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&block_table_kernel), dim3((uint32_t)batch),
                                         dim3(kTabThreads), args, 0, static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? TOPK_OK : TOPK_ERR_LAUNCH;
}

}  // extern "C"
