// The kernels beside the fp32 selection in a two-level sparse-attention
// indexer, for gfx950 ("dsv4.1: Top-k kernels and candidate selection",
// implementation section 2 and code excerpts):
//
//  * topk_bf16_kernel: exact top-k of bf16 rows of at most 16384 scores, one
//    workgroup per row, the row held in registers as 16-bit order keys; the
//    same radix selection (11-bit digits, then the tie cutoff on inverted
//    positions) and emission as the fp32 LDS paths;
//  * amax8_kernel: the level-one keys, the largest of every 8 scores (NaN
//    ignored, +0 above -0) with the newest block +inf; a streaming kernel;
//  * block_table_kernel: the selected block ids of a row in ascending order
//    by a bitmap counting sort in LDS, with their pool slots.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "exact_topk.h"
#include "topk_device.h"

namespace topk {
namespace {

// ----------------------------------------------------------------------------
// bf16 rows
// ----------------------------------------------------------------------------

constexpr int kBfThreads = 256;
constexpr int kBfMaxCols = 16384;
constexpr int kBfChunks = kBfMaxCols / 8 / kBfThreads;  // 16-byte chunks per lane

typedef uint32_t u4 __attribute__((ext_vector_type(4)));

struct Bf16Params {
    const uint16_t* scores;
    int64_t row_stride;
    int64_t n_cols;
    const int32_t* lengths;
    int32_t* out;
    const int32_t* page_table;
    int64_t pt_stride;
    int32_t page_size;
    int32_t k;
};

// bf16 pattern -> 16-bit key in value order (negative patterns inverted,
// non-negative ones get the top bit): -0 just below +0, -inf lowest.
__device__ __forceinline__ uint32_t bf16_key(uint32_t h) {
    return (h ^ ((0u - (h >> 15)) | 0x8000u)) & 0xFFFFu;
}

// A row of 16-bit keys in LDS, two per word (position 2w in the low half).
struct Bf16LdsRow {
    const uint32_t* word;
    uint32_t L;
    template <class F>
    __device__ __forceinline__ void for_each(F&& f) const {
        const uint32_t nw = (L + 1u) / 2u;
        for (uint32_t w = threadIdx.x; w < nw; w += kBfThreads) {
            const uint32_t x = word[w];
            f(x & 0xFFFFu, 2u * w);
            if (2u * w + 1u < L) f(x >> 16, 2u * w + 1u);
        }
    }
};

__global__ __launch_bounds__(kBfThreads) void topk_bf16_kernel(Bf16Params p) {
    using B = BlockScope<kBfThreads>;
    __shared__ uint32_t keys[kBfMaxCols / 2];
    __shared__ uint32_t hist[kBins];
    __shared__ uint32_t found[3];
    __shared__ uint32_t emitted;
    const int64_t b = blockIdx.x;
    int64_t Lr = p.lengths ? (int64_t)p.lengths[b] : p.n_cols;
    Lr = Lr < 0 ? 0 : (Lr > p.n_cols ? p.n_cols : Lr);
    const uint32_t L = (uint32_t)Lr;
    const uint32_t m = L < (uint32_t)p.k ? L : (uint32_t)p.k;
    OutRow out{p.out + b * (int64_t)p.k, p.page_table ? p.page_table + b * p.pt_stride : nullptr, p.page_size, m,
               &emitted};
    if (L <= (uint32_t)p.k) {  // every position, then -1
        for (int i = (int)threadIdx.x; i < p.k; i += kBfThreads) out.row[i] = (uint32_t)i < L ? out.map((uint32_t)i) : -1;
        return;
    }
    // lane t loads 16-byte chunks c = 0..7 at positions (c * 256 + t) * 8,
    // all in flight before any is used, and stores them as keys
    const uint16_t* row = p.scores + b * p.row_stride;
    u4 v[kBfChunks];
#pragma unroll
    for (int c = 0; c < kBfChunks; ++c) {
        const uint32_t base = (uint32_t)(c * kBfThreads + threadIdx.x) * 8u;
        if (base + 8u <= L) {
            v[c] = __builtin_nontemporal_load(reinterpret_cast<const u4*>(row + base));
        } else {
            uint32_t w[4] = {0u, 0u, 0u, 0u};
            for (uint32_t e = 0; e < 8u && base + e < L; ++e) w[e >> 1] |= (uint32_t)row[base + e] << (16 * (e & 1));
            v[c] = u4{w[0], w[1], w[2], w[3]};
        }
    }
#pragma unroll
    for (int c = 0; c < kBfChunks; ++c) {
        const uint32_t base = (uint32_t)(c * kBfThreads + threadIdx.x) * 8u;
        if (base < L) {
            u4 k;
#pragma unroll
            for (int q = 0; q < 4; ++q) k[q] = bf16_key(v[c][q] & 0xFFFFu) | (bf16_key(v[c][q] >> 16) << 16);
            *reinterpret_cast<u4*>(keys + base / 2u) = k;
        }
    }
    for (int i = (int)threadIdx.x; i < kBins; i += kBfThreads) hist[i] = 0u;
    if (threadIdx.x == 0) emitted = 0u;
    B::sync();
    const Bf16LdsRow src{keys, L};
    const Selection s = select_top<B>(SelectLds{hist, found}, src, m, L, 0u, 0xFFFFu, bits_for(L));
    emit(src, s, out);
}

// ----------------------------------------------------------------------------
// block max of every 8 scores
// ----------------------------------------------------------------------------

constexpr int kAmaxThreads = 256;
constexpr int kAmaxPer = 4;                                 // blocks per lane
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
    const int64_t i0 = tile * kAmaxTile + threadIdx.x;
    f4 lo[kAmaxPer], hi[kAmaxPer];
#pragma unroll
    for (int j = 0; j < kAmaxPer; ++j) {  // every full block below the newest
        const int64_t i = i0 + j * kAmaxThreads;
        if (i < nb - 1) {
            lo[j] = load_nt(row + 2 * i);
            hi[j] = load_nt(row + 2 * i + 1);
        }
    }
#pragma unroll
    for (int j = 0; j < kAmaxPer; ++j) {
        const int64_t i = i0 + j * kAmaxThreads;
        if (i < nb - 1) {
            uint32_t k = max(max(max(live_key(lo[j].x), live_key(lo[j].y)), max(live_key(lo[j].z), live_key(lo[j].w))),
                             max(max(live_key(hi[j].x), live_key(hi[j].y)), max(live_key(hi[j].z), live_key(hi[j].w))));
            // key -> pattern: the inverse of order_key; an all-NaN block gives +qNaN
            const uint32_t bits = k == 0u ? 0x7FC00000u : ((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
            out[i] = __uint_as_float(bits);
        } else if (i == nb - 1) {
            out[i] = __builtin_inff();
        }
    }
}

// ----------------------------------------------------------------------------
// candidate block table
// ----------------------------------------------------------------------------

constexpr int kTabThreads = 256;
constexpr int kTabMaxBlocks = 262144;              // blocks per row (2^21 positions)
constexpr int kTabWords = kTabMaxBlocks / 32;      // bitmap words
constexpr int kTabWordsPerLane = kTabWords / kTabThreads;
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

int topk_select_bf16(const uint16_t* scores, int64_t batch, int64_t row_stride, int64_t n_cols,
                     const int32_t* lengths, int32_t k, int32_t* out_idx,
                     const int32_t* page_table, int64_t page_table_stride, int32_t page_size,
                     void* hip_stream) {
    if (batch < 0 || batch > (int64_t)(UINT32_MAX / kBfThreads)) return TOPK_ERR_ARG;
    if (k < 1 || k > TOPK_MAX_K) return TOPK_ERR_K;
    if (n_cols < 0 || n_cols > kBfMaxCols || row_stride < n_cols) return TOPK_ERR_ARG;
    if (page_table != nullptr) {
        if (page_size < 1) return TOPK_ERR_ARG;
        if (page_table_stride < (n_cols + page_size - 1) / page_size) return TOPK_ERR_ARG;
    }
    if (batch == 0) return TOPK_OK;
    if (scores == nullptr || out_idx == nullptr) return TOPK_ERR_ARG;
    if ((reinterpret_cast<uintptr_t>(scores) & 15u) != 0) return TOPK_ERR_ALIGN;
    if (batch > 1 && (row_stride & 7) != 0) return TOPK_ERR_ALIGN;
    Bf16Params p{scores, row_stride, n_cols, lengths, out_idx, page_table, page_table_stride, page_size, k};
    void* args[] = {&p};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&topk_bf16_kernel), dim3((uint32_t)batch),
                                         dim3(kBfThreads), args, 0, static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? TOPK_OK : TOPK_ERR_LAUNCH;
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
    TableParams p{blocks, k, lengths, n_cols, page_table, page_table_stride, (int32_t)bpp, out_pages};
    void* args[] = {&p};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&block_table_kernel), dim3((uint32_t)batch),
                                         dim3(kTabThreads), args, 0, static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? TOPK_OK : TOPK_ERR_LAUNCH;
}

}  // extern "C"
