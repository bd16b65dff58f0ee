// Exact per-row top-k over long, ragged fp32 rows, for gfx950 (CDNA4).
//
// One workgroup of 512 lanes (8 wave64s) owns one row. Every comparison is on
// a uint32 key that orders the float bit patterns by value, so no float
// compare, rounding or denormal flush is involved anywhere.
//
// Paths inside the one launch (vLLM PR #56346 report, implementation item 1:
// long and short rows share a launch):
//  * L <= k: every position is selected.
//  * L <= capacity: the row is copied into LDS once and selected there.
//  * longer rows: a uniform sample of contiguous runs gives a cutoff key T
//    (vLLM PR #56346 report, summary and item 1: sampled cutoff, then exact
//    selection among survivors); one coalesced pass over the row appends every
//    key >= T to an LDS survivor buffer with one LDS atomic per wave, counting
//    on past the capacity without writing; the exact cutoff is then found
//    among the survivors by radix histogram passes.
//  * survivors > capacity or < m: the full-row path, which finds the exact
//    cutoff with histogram-only passes over the row and writes the result in
//    one final pass ("Fix incorrect sparse-attention top-k selection when
//    candidate bins overflow", comment thread, cutoff-first fallback: refine
//    with histograms, then one scan writes values above the cutoff and the
//    cutoff ties into disjoint ranges).
//
// Every path returns the same set: all positions with key above the cutoff
// key K*, plus the lowest-index positions equal to K* until m are taken.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "exact_topk.h"

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kCapacity = 8192;   // survivor entries held in LDS
constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;
constexpr int kUnroll = 4;        // float4 loads per lane per streaming step
constexpr int kRunLen = 64;       // floats per contiguous sample run
constexpr int kMaxRuns = 64;      // runs per sample (4096 keys at most)

typedef float f4 __attribute__((ext_vector_type(4)));

struct Params {
    const float* scores;
    int64_t row_stride;
    int64_t n_cols;
    const int32_t* lengths;
    int32_t* out;
    const int32_t* page_table;
    int64_t pt_stride;
    int32_t page_size;
    int32_t k;
    int32_t force_path;
    int32_t capacity;
    int32_t* row_stats;
};

struct Shared {
    uint32_t key[kCapacity];
    uint32_t idx[kCapacity];
    uint32_t hist[kBins];
    uint32_t wave_sum[kWaves];
    uint32_t count;
    uint32_t found_digit;
    uint32_t found_above;
    uint32_t found_count;
    uint32_t vmin;
    uint32_t vmax;
};

// fp32 bits -> uint32 whose unsigned order is the value order: negative
// patterns are inverted, non-negative ones get the sign bit set. -0 lands just
// below +0, -inf at the bottom of the finite range, +inf at the top (vLLM PR
// #56346 report, implementation item 1: a uint32 total-order key).
__device__ __forceinline__ uint32_t order_key(float x) {
    const uint32_t u = __float_as_uint(x);
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x & 63u; }

// number of set bits of `mask` below this lane
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t x) {
    const uint32_t lane = lane_id();
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = __shfl_up(x, d, 64);
        if (lane >= (uint32_t)d) x += y;
    }
    return x;
}

// Exclusive prefix sum of one value per lane over the whole workgroup.
__device__ uint32_t block_exclusive_sum(Shared& sm, uint32_t v) {
    const uint32_t incl = wave_inclusive_sum(v);
    const uint32_t wave = threadIdx.x >> 6;
    if (lane_id() == 63) sm.wave_sum[wave] = incl;
    __syncthreads();
    uint32_t before = 0;
    for (uint32_t w = 0; w < wave; ++w) before += sm.wave_sum[w];
    __syncthreads();
    return before + incl - v;
}

// Over sm.hist read from the top bin down, find the bin d holding the
// `rank`-th element (1-based): above(d) < rank <= above(d) + hist[d].
// Writes found_digit / found_above / found_count; ends with a barrier.
__device__ void find_rank_bin(Shared& sm, uint32_t rank) {
    constexpr int kPer = kBins / kThreads;
    uint32_t c[kPer];
    uint32_t s = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        c[j] = sm.hist[kBins - 1 - (kPer * threadIdx.x + j)];
        s += c[j];
    }
    uint32_t above = block_exclusive_sum(sm, s);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        if (above < rank && rank <= above + c[j]) {
            sm.found_digit = kBins - 1 - (kPer * threadIdx.x + j);
            sm.found_above = above;
            sm.found_count = c[j];
        }
        above += c[j];
    }
    __syncthreads();
}

// ----------------------------------------------------------------------------
// element sources: the LDS buffer, or the row itself in global memory
// ----------------------------------------------------------------------------

struct LdsSource {
    const Shared* sm;
    uint32_t n;
    template <class F>
    __device__ void for_each(F&& f) const {
        for (uint32_t e = threadIdx.x; e < n; e += kThreads) f(sm->key[e], sm->idx[e]);
    }
};

struct RowSource {
    const float* row;
    int64_t len;
    template <class F>
    __device__ void for_each(F&& f) const {
        const f4* r4 = reinterpret_cast<const f4*>(row);
        const int64_t nvec = len >> 2;
        for (int64_t v = threadIdx.x; v < nvec; v += kThreads) {
            const f4 x = r4[v];
            const uint32_t i = (uint32_t)(4 * v);
            f(order_key(x.x), i);
            f(order_key(x.y), i + 1);
            f(order_key(x.z), i + 2);
            f(order_key(x.w), i + 3);
        }
        for (int64_t i = 4 * nvec + threadIdx.x; i < len; i += kThreads) f(order_key(row[i]), (uint32_t)i);
    }
};

// value views for selection: the key itself, or (among keys equal to `tie`)
// the inverted index, so that "largest first" means "lowest index first"
struct KeyView {
    __device__ bool operator()(uint32_t key, uint32_t, uint32_t& v) const {
        v = key;
        return true;
    }
};
struct TieIndexView {
    uint32_t tie;
    __device__ bool operator()(uint32_t key, uint32_t idx, uint32_t& v) const {
        v = ~idx;
        return key == tie;
    }
};

template <class Src, class View>
__device__ void value_range(Shared& sm, const Src& src, View view, uint32_t& vmin, uint32_t& vmax) {
    if (threadIdx.x == 0) {
        sm.vmin = 0xFFFFFFFFu;
        sm.vmax = 0u;
    }
    __syncthreads();
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    src.for_each([&](uint32_t key, uint32_t idx) {
        uint32_t v;
        if (view(key, idx, v)) {
            lo = min(lo, v);
            hi = max(hi, v);
        }
    });
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        lo = min(lo, (uint32_t)__shfl_xor(lo, d, 64));
        hi = max(hi, (uint32_t)__shfl_xor(hi, d, 64));
    }
    if (lane_id() == 0) {
        atomicMin(&sm.vmin, lo);
        atomicMax(&sm.vmax, hi);
    }
    __syncthreads();
    vmin = sm.vmin;
    vmax = sm.vmax;
    __syncthreads();
}

struct Cut {
    uint32_t value;  // the rank-th largest value V*
    uint32_t need;   // how many elements equal to V* belong to the top `rank`
    uint32_t equal;  // how many elements equal V*
};

// Radix selection (vLLM PR #56346 report, implementation item 1: coarse
// histogram bin, then refinement down to the exact cutoff): the rank-th
// largest viewed value among the participating elements, whose values all
// share the bits of `prefix` above bit `nbits`. Histograms of 11-bit digits in
// LDS, highest digit first; each pass keeps only elements matching the digits
// chosen so far. 1 <= rank <= number of participating elements.
template <class Src, class View>
__device__ Cut radix_select(Shared& sm, const Src& src, View view, uint32_t rank,
                            uint32_t prefix, int nbits, uint32_t equal_if_none) {
    Cut cut{prefix, rank, equal_if_none};
    while (nbits > 0) {
        const int w = nbits < kDigitBits ? nbits : kDigitBits;
        const int shift = nbits - w;
        const uint32_t done_mask = nbits >= 32 ? 0u : (0xFFFFFFFFu << nbits);
        const uint32_t want = prefix & done_mask;
        const uint32_t dmask = (1u << w) - 1u;
        for (int i = threadIdx.x; i < kBins; i += kThreads) sm.hist[i] = 0u;
        __syncthreads();
        src.for_each([&](uint32_t key, uint32_t idx) {
            uint32_t v;
            if (view(key, idx, v) && (v & done_mask) == want) atomicAdd(&sm.hist[(v >> shift) & dmask], 1u);
        });
        __syncthreads();
        find_rank_bin(sm, rank);
        const uint32_t d = sm.found_digit;
        const uint32_t above = sm.found_above;
        const uint32_t cnt = sm.found_count;
        __syncthreads();  // found_* and hist are rewritten by the next pass
        rank -= above;
        prefix = want | (d << shift);
        nbits = shift;
        cut.equal = cnt;
    }
    cut.value = prefix;
    cut.need = rank;
    return cut;
}

// Exact cutoff of the top m among `src`: take key > kth, and key == kth with
// idx <= icut (icut = INT32_MAX when every tie is taken).
struct Selection {
    uint32_t kth;
    int32_t icut;
};

template <class Src>
__device__ Selection select_top(Shared& sm, const Src& src, uint32_t m, uint32_t n, bool know_range,
                                int idx_bits) {
    uint32_t prefix = 0u;
    int nbits = 32;
    if (know_range) {
        uint32_t lo, hi;
        value_range(sm, src, KeyView{}, lo, hi);
        prefix = lo;
        nbits = lo == hi ? 0 : 32 - __clz(lo ^ hi);
    }
    const Cut c = radix_select(sm, src, KeyView{}, m, prefix, nbits, n);
    Selection s{c.value, INT32_MAX};
    if (c.need < c.equal) {
        // lowest-index ties: the need-th largest inverted index among them;
        // inverted indices below 2^idx_bits share their top 32 - idx_bits bits
        const uint32_t iprefix = idx_bits >= 32 ? 0u : (0xFFFFFFFFu << idx_bits);
        const Cut t = radix_select(sm, src, TieIndexView{c.value}, c.need, iprefix, idx_bits, c.equal);
        s.icut = (int32_t)(~t.value);
    }
    return s;
}

__device__ __forceinline__ int32_t map_slot(const Params& p, int64_t b, uint32_t i) {
    if (p.page_table == nullptr) return (int32_t)i;
    const int64_t page = p.page_table[b * p.pt_stride + (int64_t)(i / (uint32_t)p.page_size)];
    return (int32_t)(page * p.page_size + (int64_t)(i % (uint32_t)p.page_size));
}

// Writes every selected element of `src` to out row slots [0, m); slots are
// handed out by one LDS atomic per wave (ballot + mbcnt). The selection holds
// exactly m elements; the slot bound only keeps a defect from writing outside
// the row.
template <class Src>
__device__ void emit(Shared& sm, const Src& src, Selection s, uint32_t m, const Params& p, int64_t b,
                     int32_t* orow) {
    if (threadIdx.x == 0) sm.count = 0u;
    __syncthreads();
    src.for_each([&](uint32_t key, uint32_t idx) {
        const bool take = key > s.kth || (key == s.kth && (int32_t)idx <= s.icut);
        const uint64_t mask = __ballot(take);
        if (take) {
            const uint32_t leader = (uint32_t)__ffsll((unsigned long long)mask) - 1u;
            uint32_t base = 0u;
            if (lane_id() == leader) base = atomicAdd(&sm.count, (uint32_t)__popcll(mask));
            base = __shfl(base, (int)leader, 64);
            const uint32_t slot = base + lanes_below(mask);
            if (slot < m) orow[slot] = map_slot(p, b, idx);
        }
    });
    __syncthreads();
}

// Cutoff key from a sample of `runs` runs of kRunLen contiguous scores spread
// evenly over [0, L): the rank-th largest sample key, rank chosen so that the
// expected survivor count sits several standard deviations above m (the
// sample fraction above the true m-th key is binomial).
__device__ uint32_t sample_cutoff(Shared& sm, const float* row, int64_t L, uint32_t m) {
    const int64_t fit = L / (2 * kRunLen);
    const int runs = fit < kMaxRuns ? (int)fit : kMaxRuns;
    if (runs < 2) return 0u;  // too short to sample: keep everything
    const uint32_t S = (uint32_t)runs * kRunLen;
    constexpr int kVecPerRun = kRunLen / 4;
    for (int t = threadIdx.x; t < runs * kVecPerRun; t += kThreads) {
        const int r = t / kVecPerRun;
        const int j = t % kVecPerRun;
        const int64_t start = ((int64_t)r * (L - kRunLen) / (runs - 1)) & ~(int64_t)3;
        const f4 x = reinterpret_cast<const f4*>(row + start)[j];
        sm.key[4 * t + 0] = order_key(x.x);
        sm.key[4 * t + 1] = order_key(x.y);
        sm.key[4 * t + 2] = order_key(x.z);
        sm.key[4 * t + 3] = order_key(x.w);
        sm.idx[4 * t + 0] = 4 * t + 0;
        sm.idx[4 * t + 1] = 4 * t + 1;
        sm.idx[4 * t + 2] = 4 * t + 2;
        sm.idx[4 * t + 3] = 4 * t + 3;
    }
    __syncthreads();
    const float mu = (float)m * (float)S / (float)L;
    const float want = ceilf(mu + 6.0f * sqrtf(mu) + 4.0f);
    if (want >= (float)S) return 0u;
    const uint32_t rank = (uint32_t)want;
    const LdsSource src{&sm, S};
    uint32_t lo, hi;
    value_range(sm, src, KeyView{}, lo, hi);
    const Cut c = radix_select(sm, src, KeyView{}, rank, lo, lo == hi ? 0 : 32 - __clz(lo ^ hi), S);
    return c.value;
}

// One coalesced pass over [0, L): every key >= T goes to the LDS buffer.
// Each wave reserves its slots with a single LDS atomic per step and stops
// early once the running count passes the capacity (the overflow fallback
// then re-reads the row anyway). Returns the survivor count (> cap means
// overflow; the buffer then holds an arbitrary subset).
__device__ uint32_t stream_survivors(Shared& sm, const float* row, int64_t L, uint32_t T, uint32_t cap) {
    if (threadIdx.x == 0) sm.count = 0u;
    __syncthreads();
    const f4* r4 = reinterpret_cast<const f4*>(row);
    const int64_t nvec = L >> 2;
    const uint32_t lane = lane_id();
    constexpr int64_t kStep = (int64_t)kThreads * kUnroll;
    for (int64_t v0 = 0; v0 < nvec; v0 += kStep) {
        f4 x[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t v = v0 + u * kThreads + threadIdx.x;
            x[u] = v < nvec ? __builtin_nontemporal_load(r4 + v) : f4{0.f, 0.f, 0.f, 0.f};
        }
        uint64_t masks[4 * kUnroll];
        uint32_t total = 0;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const bool ok = v0 + u * kThreads + threadIdx.x < nvec;
            masks[4 * u + 0] = __ballot(ok && order_key(x[u].x) >= T);
            masks[4 * u + 1] = __ballot(ok && order_key(x[u].y) >= T);
            masks[4 * u + 2] = __ballot(ok && order_key(x[u].z) >= T);
            masks[4 * u + 3] = __ballot(ok && order_key(x[u].w) >= T);
#pragma unroll
            for (int c = 0; c < 4; ++c) total += (uint32_t)__popcll(masks[4 * u + c]);
        }
        if (total == 0) continue;
        uint32_t base = 0u;
        if (lane == 0) base = atomicAdd(&sm.count, total);
        base = __builtin_amdgcn_readfirstlane(base);
        if (base < cap) {
            uint32_t off = base;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const uint32_t i0 = (uint32_t)(4 * (v0 + u * kThreads + threadIdx.x));
                const float xs[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint64_t mk = masks[4 * u + c];
                    if ((mk >> lane) & 1u) {
                        const uint32_t pos = off + lanes_below(mk);
                        if (pos < cap) {
                            sm.key[pos] = order_key(xs[c]);
                            sm.idx[pos] = i0 + (uint32_t)c;
                        }
                    }
                    off += (uint32_t)__popcll(mk);
                }
            }
        }
        if (base + total > cap) break;
    }
    // the last L % 4 positions, by the first wave
    const int64_t tail = 4 * nvec;
    if (threadIdx.x < 64) {
        const int64_t i = tail + lane;
        const bool hit = i < L && order_key(row[i]) >= T;
        const uint64_t mk = __ballot(hit);
        if (mk != 0) {
            uint32_t base = 0u;
            if (lane == 0) base = atomicAdd(&sm.count, (uint32_t)__popcll(mk));
            base = __builtin_amdgcn_readfirstlane(base);
            if (hit) {
                const uint32_t pos = base + lanes_below(mk);
                if (pos < cap) {
                    sm.key[pos] = order_key(row[i]);
                    sm.idx[pos] = (uint32_t)i;
                }
            }
        }
    }
    __syncthreads();
    const uint32_t n = sm.count;
    __syncthreads();
    return n;
}

__device__ void load_row_to_lds(Shared& sm, const float* row, int64_t L) {
    const f4* r4 = reinterpret_cast<const f4*>(row);
    const int64_t nvec = L >> 2;
    for (int64_t v = threadIdx.x; v < nvec; v += kThreads) {
        const f4 x = r4[v];
        const uint32_t i = (uint32_t)(4 * v);
        sm.key[i + 0] = order_key(x.x);
        sm.key[i + 1] = order_key(x.y);
        sm.key[i + 2] = order_key(x.z);
        sm.key[i + 3] = order_key(x.w);
        sm.idx[i + 0] = i + 0;
        sm.idx[i + 1] = i + 1;
        sm.idx[i + 2] = i + 2;
        sm.idx[i + 3] = i + 3;
    }
    for (int64_t i = 4 * nvec + threadIdx.x; i < L; i += kThreads) {
        sm.key[i] = order_key(row[i]);
        sm.idx[i] = (uint32_t)i;
    }
    __syncthreads();
}

__device__ __forceinline__ int bits_for(int64_t L) {  // bits to hold indices 0..L-1, L >= 2
    return 64 - __clzll((unsigned long long)(L - 1));
}

__global__ __launch_bounds__(kThreads) void topk_rows_kernel(Params p) {
    __shared__ Shared sm;
    const int64_t b = blockIdx.x;
    int64_t L = p.lengths ? (int64_t)p.lengths[b] : p.n_cols;
    L = L < 0 ? 0 : (L > p.n_cols ? p.n_cols : L);
    const int32_t k = p.k;
    const uint32_t m = (uint32_t)(L < k ? L : k);
    int32_t* orow = p.out + b * (int64_t)k;
    const float* row = p.scores + b * p.row_stride;

    for (int j = (int)m + threadIdx.x; j < k; j += kThreads) orow[j] = -1;
    int code = TOPK_ROW_EMPTY;
    uint32_t seen = (uint32_t)L;
    if (m == 0) {
        // idle row: only -1 slots
    } else if (L <= k) {
        for (int64_t i = threadIdx.x; i < L; i += kThreads) orow[i] = map_slot(p, b, (uint32_t)i);
        code = TOPK_ROW_ALL;
    } else {
        const uint32_t cap = (uint32_t)p.capacity;
        int path = p.force_path;
        if (path == TOPK_PATH_AUTO) path = L <= (int64_t)cap ? TOPK_PATH_LDS : TOPK_PATH_SAMPLED;
        code = TOPK_ROW_FULL_FORCED;
        if (path == TOPK_PATH_LDS && L <= (int64_t)cap) {
            load_row_to_lds(sm, row, L);
            const LdsSource src{&sm, (uint32_t)L};
            const Selection s = select_top(sm, src, m, (uint32_t)L, true, bits_for(L));
            emit(sm, src, s, m, p, b, orow);
            code = TOPK_ROW_LDS;
        } else if (path == TOPK_PATH_SAMPLED) {
            const uint32_t T = sample_cutoff(sm, row, L, m);
            const uint32_t n = stream_survivors(sm, row, L, T, cap);
            seen = n;
            if (n >= m && n <= cap) {
                const LdsSource src{&sm, n};
                const Selection s = select_top(sm, src, m, n, true, bits_for(L));
                emit(sm, src, s, m, p, b, orow);
                code = TOPK_ROW_SAMPLED;
            } else {
                code = n > cap ? TOPK_ROW_FULL_OVERFLOW : TOPK_ROW_FULL_UNDERFLOW;
            }
        }
        if (code >= TOPK_ROW_FULL_OVERFLOW) {
            const RowSource src{row, L};
            const Selection s = select_top(sm, src, m, (uint32_t)L, false, bits_for(L));
            emit(sm, src, s, m, p, b, orow);
        }
    }
    if (p.row_stats != nullptr && threadIdx.x == 0) {
        p.row_stats[2 * b + 0] = code;
        p.row_stats[2 * b + 1] = (int32_t)seen;
    }
}

}  // namespace

extern "C" {

const char* topk_status_string(int status) {
    switch (status) {
        case TOPK_OK: return "ok";
        case TOPK_ERR_ARG: return "invalid argument";
        case TOPK_ERR_K: return "k outside [1, 2048]";
        case TOPK_ERR_ALIGN: return "scores must be 16-byte aligned with row_stride % 4 == 0";
        case TOPK_ERR_LAUNCH: return "kernel launch failed";
        default: return "unknown status";
    }
}

int32_t topk_max_capacity(void) { return kCapacity; }

int topk_select_ex(const float* scores, int64_t batch, int64_t row_stride, int64_t n_cols,
                   const int32_t* lengths, int32_t k, int32_t* out_idx,
                   const int32_t* page_table, int64_t page_table_stride, int32_t page_size,
                   void* hip_stream, const topk_options* options) {
    if (batch < 0 || batch > INT32_MAX) return TOPK_ERR_ARG;
    if (k < 1 || k > TOPK_MAX_K) return TOPK_ERR_K;
    if (n_cols < 0 || n_cols > INT32_MAX || row_stride < n_cols) return TOPK_ERR_ARG;
    topk_options opt{TOPK_PATH_AUTO, 0, nullptr};
    if (options != nullptr) opt = *options;
    if (opt.force_path < TOPK_PATH_AUTO || opt.force_path > TOPK_PATH_FULLROW) return TOPK_ERR_ARG;
    if (opt.capacity < 0 || opt.capacity > kCapacity) return TOPK_ERR_ARG;
    if (opt.capacity == 0) opt.capacity = kCapacity;
    if (page_table != nullptr) {
        if (page_size < 1) return TOPK_ERR_ARG;
        if (page_table_stride < (n_cols + page_size - 1) / page_size) return TOPK_ERR_ARG;
    }
    if (batch == 0) return TOPK_OK;
    if (scores == nullptr || out_idx == nullptr) return TOPK_ERR_ARG;
    if ((reinterpret_cast<uintptr_t>(scores) & 15u) != 0) return TOPK_ERR_ALIGN;
    if (batch > 1 && (row_stride & 3) != 0) return TOPK_ERR_ALIGN;

    Params p{scores, row_stride, n_cols, lengths, out_idx, page_table, page_table_stride,
             page_size, k, opt.force_path, opt.capacity, opt.row_stats};
    void* args[] = {&p};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&topk_rows_kernel),
                                         dim3((uint32_t)batch), dim3(kThreads), args, 0,
                                         static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? TOPK_OK : TOPK_ERR_LAUNCH;
}

int topk_select(const float* scores, int64_t batch, int64_t row_stride, int64_t n_cols,
                const int32_t* lengths, int32_t k, int32_t* out_idx,
                const int32_t* page_table, int64_t page_table_stride, int32_t page_size,
                void* hip_stream) {
    return topk_select_ex(scores, batch, row_stride, n_cols, lengths, k, out_idx, page_table,
                          page_table_stride, page_size, hip_stream, nullptr);
}

}  // extern "C"
