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
//    key >= T to an LDS survivor buffer with one LDS atomic per wave and step,
//    counting on past the capacity without writing; the exact cutoff is then
//    found among the survivors by radix histogram passes.
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
constexpr int kCapacity = 8192;   // survivor entries held in LDS
constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;
constexpr int kBinsPerLane = kBins / 64;
constexpr int kUnroll = 4;        // 16-byte loads per lane per streaming step
constexpr int kRunLen = 64;       // floats per contiguous sample run
constexpr int kMaxRuns = 64;      // runs per sample (4096 keys at most)
constexpr int kSampleShift = 10;  // the sample cutoff keeps the top 22 key bits
constexpr int kMaxCand = 64;      // cutoff-bin entries one wave resolves directly

static_assert(kMaxRuns * kRunLen / 4 <= 2 * kThreads, "two sample loads per lane");

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
    uint32_t hist[kBins];  // all zero between histogram passes
    uint32_t count;        // survivor slots handed out
    uint32_t emitted;      // output slots handed out
    uint32_t found_digit;
    uint32_t found_above;
    uint32_t found_count;
    uint32_t vmin;
    uint32_t vmax;
    uint32_t smax;    // largest sample key
    uint32_t ncand;   // cutoff-bin entries gathered
    uint32_t cand_key[kMaxCand];
    uint32_t cand_idx[kMaxCand];
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

__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) x = max(x, (uint32_t)__shfl_xor(x, d, 64));
    return x;
}

__device__ __forceinline__ uint32_t wave_min(uint32_t x) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) x = min(x, (uint32_t)__shfl_xor(x, d, 64));
    return x;
}

struct Found {
    uint32_t digit;  // bin holding the rank-th element from the top
    uint32_t above;  // elements in higher bins
    uint32_t count;  // elements in that bin
};

// Called by every lane after the histogram atomics and a barrier. The first
// wave finds the bin of the rank-th element from the top: a wave prefix sum
// over 32-bin groups (lane 0 holding the top group) picks the group, a second
// one over that group's bins picks the bin. It then zeroes the histogram for
// the next pass and publishes the bin. 1 <= rank <= histogram total.
__device__ Found find_rank_bin(Shared& sm, uint32_t rank) {
    if (threadIdx.x < 64) {
        const uint32_t lane = threadIdx.x;
        const uint32_t base = kBins - kBinsPerLane * (lane + 1);
        uint4* h4 = reinterpret_cast<uint4*>(&sm.hist[base]);
        uint32_t s = 0;
#pragma unroll
        for (int q = 0; q < kBinsPerLane / 4; ++q) {
            const uint4 v = h4[q];
            s += v.x + v.y + v.z + v.w;
        }
        const uint32_t incl = wave_inclusive_sum(s);
        const uint64_t own = __ballot(incl - s < rank && rank <= incl);
        if (own != 0) {
            const int owner = __ffsll((unsigned long long)own) - 1;
            const uint32_t obase = kBins - kBinsPerLane * (uint32_t)(owner + 1);
            const uint32_t oabove = (uint32_t)__builtin_amdgcn_readlane((int)(incl - s), owner);
            const bool mine = lane < (uint32_t)kBinsPerLane;
            const uint32_t bin = obase + kBinsPerLane - 1 - (lane & (kBinsPerLane - 1));
            const uint32_t c = mine ? sm.hist[bin] : 0u;
            const uint32_t ci = oabove + wave_inclusive_sum(c);
            if (mine && ci - c < rank && rank <= ci) {
                sm.found_digit = bin;
                sm.found_above = ci - c;
                sm.found_count = c;
            }
        }
#pragma unroll
        for (int q = 0; q < kBinsPerLane / 4; ++q) h4[q] = make_uint4(0u, 0u, 0u, 0u);
    }
    __syncthreads();
    return Found{sm.found_digit, sm.found_above, sm.found_count};
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

// value views for selection: the key; the key's top 22 bits; or (among keys
// equal to `tie`) the inverted index, so that "largest first" means "lowest
// index first"
struct KeyView {
    __device__ bool operator()(uint32_t key, uint32_t, uint32_t& v) const {
        v = key;
        return true;
    }
};
struct CoarseKeyView {
    __device__ bool operator()(uint32_t key, uint32_t, uint32_t& v) const {
        v = key >> kSampleShift;
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

template <class Src>
__device__ void key_range(Shared& sm, const Src& src, uint32_t& vmin, uint32_t& vmax) {
    if (threadIdx.x == 0) {
        sm.vmin = 0xFFFFFFFFu;
        sm.vmax = 0u;
    }
    __syncthreads();
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    src.for_each([&](uint32_t key, uint32_t) {
        lo = min(lo, key);
        hi = max(hi, key);
    });
    lo = wave_min(lo);
    hi = wave_max(hi);
    if (lane_id() == 0) {
        atomicMin(&sm.vmin, lo);
        atomicMax(&sm.vmax, hi);
    }
    __syncthreads();
    vmin = sm.vmin;
    vmax = sm.vmax;
}

struct Cut {
    uint32_t value;  // exact: the rank-th largest value V*; range: lower edge
    uint32_t need;   // exact: how many elements equal to V* are in the top rank
    uint32_t equal;  // exact: how many elements equal V*
    bool range;      // the top rank are exactly the elements >= value
};

// Radix selection (vLLM PR #56346 report, implementation item 1: coarse
// histogram bin, then refinement down to the exact cutoff): the rank-th
// largest viewed value among the participating elements, whose values all
// share the bits of `prefix` above bit `nbits`. Histograms of 11-bit digits
// in LDS, highest digit first; each pass counts only the elements matching
// the digits chosen so far. When the chosen bin is taken whole, the top rank
// are exactly the elements at or above its lower edge and the search stops
// early. 1 <= rank <= number of participating elements.
template <class Src, class View>
__device__ Cut radix_select(Shared& sm, const Src& src, View view, uint32_t rank, uint32_t prefix,
                            int nbits, uint32_t equal_if_none) {
    Cut cut{prefix, rank, equal_if_none, false};
    while (nbits > 0) {
        const int w = nbits < kDigitBits ? nbits : kDigitBits;
        const int shift = nbits - w;
        const uint32_t done_mask = nbits >= 32 ? 0u : (0xFFFFFFFFu << nbits);
        const uint32_t want = prefix & done_mask;
        const uint32_t dmask = (1u << w) - 1u;
        src.for_each([&](uint32_t key, uint32_t idx) {
            uint32_t v;
            if (view(key, idx, v) && (v & done_mask) == want) atomicAdd(&sm.hist[(v >> shift) & dmask], 1u);
        });
        __syncthreads();
        const Found f = find_rank_bin(sm, rank);
        rank -= f.above;
        prefix = want | (f.digit << shift);
        nbits = shift;
        cut.equal = f.count;
        if (nbits > 0 && f.count == rank) {
            cut.value = prefix;
            cut.range = true;
            return cut;
        }
    }
    cut.value = prefix;
    cut.need = rank;
    return cut;
}

// The top m of a source: take key > kth, and key == kth with idx <= icut.
struct Selection {
    uint32_t kth;
    int32_t icut;
};

__device__ __forceinline__ Selection at_least(uint32_t lo) {
    return lo == 0u ? Selection{0u, INT32_MAX} : Selection{lo - 1u, -1};
}

// Exact top m among `src`, whose keys all lie in [lo, hi]; idx < 2^idx_bits.
template <class Src>
__device__ Selection select_top(Shared& sm, const Src& src, uint32_t m, uint32_t n, uint32_t lo,
                                uint32_t hi, int idx_bits) {
    const int nbits = lo == hi ? 0 : 32 - __clz(lo ^ hi);
    const Cut c = radix_select(sm, src, KeyView{}, m, lo, nbits, n);
    if (c.range) return at_least(c.value);
    Selection s{c.value, INT32_MAX};
    if (c.need < c.equal) {
        // the lowest-index ties: the need-th largest inverted index among them;
        // inverted indices below 2^idx_bits share their top 32 - idx_bits bits
        const uint32_t iprefix = idx_bits >= 32 ? 0u : (0xFFFFFFFFu << idx_bits);
        const Cut t = radix_select(sm, src, TieIndexView{c.value}, c.need, iprefix, idx_bits, c.equal);
        s.icut = (int32_t)(~t.value);  // exact or range: inverted index >= value
    }
    return s;
}

__device__ __forceinline__ int32_t map_slot(const Params& p, int64_t b, uint32_t i) {
    if (p.page_table == nullptr) return (int32_t)i;
    const int64_t page = p.page_table[b * p.pt_stride + (int64_t)(i / (uint32_t)p.page_size)];
    return (int32_t)(page * p.page_size + (int64_t)(i % (uint32_t)p.page_size));
}

// Slot for every active lane with `pred` from a shared counter: one LDS
// atomic per wave, lanes ranked by mbcnt over the ballot.
__device__ __forceinline__ uint32_t wave_reserve(uint32_t* counter, bool pred) {
    const uint64_t mask = __ballot(pred);
    uint32_t base = 0u;
    if (mask != 0) {
        const int leader = __ffsll((unsigned long long)mask) - 1;
        if ((int)lane_id() == leader) base = atomicAdd(counter, (uint32_t)__popcll(mask));
        base = __shfl(base, leader, 64);
    }
    return base + lanes_below(mask);
}

// Appends `idx` (mapped) to the out row for every lane with `take`; slots are
// handed out by one LDS atomic per wave (ballot + mbcnt). A row's selection
// holds exactly m elements; the slot bound only keeps a defect from writing
// outside the row.
__device__ __forceinline__ void out_append(Shared& sm, bool take, uint32_t idx, uint32_t m, const Params& p,
                                           int64_t b, int32_t* orow) {
    const uint32_t slot = wave_reserve(&sm.emitted, take);
    if (take && slot < m) orow[slot] = map_slot(p, b, idx);
}

// Writes every selected element of `src` to the out row.
template <class Src>
__device__ void emit(Shared& sm, const Src& src, Selection s, uint32_t m, const Params& p, int64_t b,
                     int32_t* orow) {
    src.for_each([&](uint32_t key, uint32_t idx) {
        out_append(sm, key > s.kth || (key == s.kth && (int32_t)idx <= s.icut), idx, m, p, b, orow);
    });
}

// Bin of a survivor in the histogram built while streaming: bins of width
// 2^sh upward from the cutoff T, the last bin open-ended.
struct StreamBins {
    uint32_t T;
    uint32_t sh;
    __device__ __forceinline__ uint32_t operator()(uint32_t key) const {
        const uint32_t d = (key - T) >> sh;
        return d < (uint32_t)kBins ? d : (uint32_t)kBins - 1u;
    }
};

__device__ __forceinline__ f4 load_nt(const f4* p) { return __builtin_nontemporal_load(p); }

// Streaming survivor compaction over the row's float4 groups [0, nvec) with
// one step of loads always in flight ahead of the step being filtered.
// `a` holds step 0, already issued by the caller. Hits (key >= T) are
// appended to the LDS buffer and counted in the survivor histogram; each wave
// reserves its slots for a step with a single LDS atomic and stops once the
// running count passes the capacity.
// kNonNegT: T is the key of a non-negative float, so the test needs only a
// signed compare of the raw bits.
template <bool kNonNegT>
__device__ void stream_steps(Shared& sm, const f4* r4, int64_t nvec, StreamBins bins, uint32_t cap,
                             f4 (&a)[kUnroll], uint32_t& hmax) {
    const uint32_t T = bins.T;
    constexpr int64_t kStep = (int64_t)kThreads * kUnroll;
    const int32_t Ts = (int32_t)(T ^ 0x80000000u);
    const uint32_t lane = lane_id();
    auto hit = [&](float x) -> bool {
        if constexpr (kNonNegT) return (int32_t)__float_as_uint(x) >= Ts;
        else return order_key(x) >= T;
    };
    auto load = [&](f4 (&x)[kUnroll], int64_t v0) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t v = v0 + u * kThreads + threadIdx.x;
            x[u] = v < nvec ? load_nt(r4 + v) : f4{0.f, 0.f, 0.f, 0.f};
        }
    };
    // false once the running count has passed the capacity
    auto filter = [&](const f4 (&x)[kUnroll], int64_t v0) -> bool {
        uint64_t masks[4 * kUnroll];
        uint32_t total = 0;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const bool ok = v0 + u * kThreads + threadIdx.x < nvec;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                masks[4 * u + c] = __ballot(ok && hit(x[u][c]));
                total += (uint32_t)__popcll(masks[4 * u + c]);
            }
        }
        if (total == 0) return true;
        uint32_t base = 0u;
        if (lane == 0) base = atomicAdd(&sm.count, total);
        base = __builtin_amdgcn_readfirstlane(base);
        if (base >= cap) return false;
        uint32_t off = base;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t i0 = (uint32_t)(4 * (v0 + u * kThreads + threadIdx.x));
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint64_t mk = masks[4 * u + c];
                if ((mk >> lane) & 1u) {
                    const uint32_t pos = off + lanes_below(mk);
                    const uint32_t key = order_key(x[u][c]);
                    hmax = max(hmax, key);
                    if (pos < cap) {
                        sm.key[pos] = key;
                        sm.idx[pos] = i0 + (uint32_t)c;
                        atomicAdd(&sm.hist[bins(key)], 1u);
                    }
                }
                off += (uint32_t)__popcll(mk);
            }
        }
        return base + total <= cap;
    };
    f4 b[kUnroll];
    int64_t v0 = 0;
    while (v0 < nvec) {
        load(b, v0 + kStep);
        if (!filter(a, v0)) break;
        v0 += kStep;
        if (v0 >= nvec) break;
        load(a, v0 + kStep);
        if (!filter(b, v0)) break;
        v0 += kStep;
    }
}

// Sampled path for a row with L > k: returns the survivor count n (n > cap
// means the buffer overflowed and holds an arbitrary subset). On return the
// buffer holds the survivors, [bins.T, vmax] bounds their keys, and the
// histogram counts them by bins(key) (unless the buffer overflowed).
//
// The cutoff T comes from a sample of `runs` runs of 64 contiguous scores
// spread evenly over [0, L): the lower edge of the 22-bit key bucket holding
// the rank-th largest sample key, the rank chosen so that the expected
// survivor count sits several standard deviations above m (the number of
// sample keys above the true m-th key is binomial).
__device__ uint32_t sampled_survivors(Shared& sm, const float* row, int64_t L, uint32_t m, uint32_t cap,
                                      StreamBins& bins, uint32_t& vmax) {
    const f4* r4 = reinterpret_cast<const f4*>(row);
    const int64_t nvec = L >> 2;
    const int64_t fit = L / (2 * kRunLen);
    const int runs = fit < kMaxRuns ? (int)fit : kMaxRuns;
    constexpr int kVecPerRun = kRunLen / 4;
    const int nsv = runs >= 2 ? runs * kVecPerRun : 0;

    // sample loads first, then step 0 of the stream, all in flight together
    f4 sv[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int t = threadIdx.x + h * kThreads;
        if (t < nsv) {
            const int r = t / kVecPerRun;
            const int64_t start = ((int64_t)r * (L - kRunLen) / (runs - 1)) & ~(int64_t)3;
            sv[h] = r4[start / 4 + t % kVecPerRun];
        }
    }
    f4 a[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t v = u * kThreads + threadIdx.x;
        a[u] = v < nvec ? load_nt(r4 + v) : f4{0.f, 0.f, 0.f, 0.f};
    }
    uint32_t smax = 0u;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int t = threadIdx.x + h * kThreads;
        if (t < nsv) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t key = order_key(sv[h][c]);
                sm.key[4 * t + c] = key;
                smax = max(smax, key);
            }
        }
    }
    smax = wave_max(smax);
    if (lane_id() == 0) atomicMax(&sm.smax, smax);
    __syncthreads();

    uint32_t T = 0u;  // too short to sample: keep everything
    if (nsv > 0) {
        const uint32_t S = (uint32_t)nsv * 4;
        const float mu = (float)m * (float)S / (float)L;
        const float want = ceilf(mu + 6.0f * sqrtf(mu) + 4.0f);
        if (want < (float)S) {
            const Cut c = radix_select(sm, LdsSource{&sm, S}, CoarseKeyView{}, (uint32_t)want, 0u,
                                       32 - kSampleShift, S);
            T = c.value << kSampleShift;
        }
    }

    // survivor histogram: the span [T, sample max] covers about half the bins
    const uint32_t span = sm.smax - T;
    const int wbits = span == 0u ? 0 : 32 - __clz(span);
    bins = StreamBins{T, (uint32_t)(wbits > kDigitBits - 1 ? wbits - (kDigitBits - 1) : 0)};

    uint32_t hmax = 0u;
    if (T >= 0x80000000u) stream_steps<true>(sm, r4, nvec, bins, cap, a, hmax);
    else stream_steps<false>(sm, r4, nvec, bins, cap, a, hmax);

    // the last L % 4 positions, by the first wave
    if (threadIdx.x < 64) {
        const int64_t i = 4 * nvec + lane_id();
        const uint32_t key = i < L ? order_key(row[i]) : 0u;
        const bool hit = i < L && key >= T;
        const uint64_t mk = __ballot(hit);
        if (mk != 0) {
            uint32_t base = 0u;
            if (lane_id() == 0) base = atomicAdd(&sm.count, (uint32_t)__popcll(mk));
            base = __builtin_amdgcn_readfirstlane(base);
            if (hit) {
                const uint32_t pos = base + lanes_below(mk);
                hmax = max(hmax, key);
                if (pos < cap) {
                    sm.key[pos] = key;
                    sm.idx[pos] = (uint32_t)i;
                    atomicAdd(&sm.hist[bins(key)], 1u);
                }
            }
        }
    }
    hmax = wave_max(hmax);
    if (lane_id() == 0) atomicMax(&sm.vmax, hmax);
    __syncthreads();
    vmax = sm.vmax;
    return sm.count;
}

// Exact top m of the n >= m survivors, from the histogram built while
// streaming: every survivor in a bin above the cutoff bin is written out in
// one pass over the buffer, which also gathers the cutoff bin's entries; one
// wave ranks those by (key descending, index ascending) and writes the first
// `need`. A crowded or open-ended cutoff bin takes the radix select instead.
__device__ void finish_survivors(Shared& sm, uint32_t n, uint32_t m, StreamBins bins, uint32_t hi,
                                 int idx_bits, const Params& p, int64_t b, int32_t* orow) {
    const Found f = find_rank_bin(sm, m);
    const LdsSource src{&sm, n};
    if (f.count > (uint32_t)kMaxCand || f.digit == (uint32_t)kBins - 1u) {
        const Selection s = select_top(sm, src, m, n, bins.T, hi, idx_bits);
        emit(sm, src, s, m, p, b, orow);
        return;
    }
    const uint32_t d = f.digit;
    const uint32_t need = m - f.above;
    const bool whole = f.count == need;  // the cutoff bin is taken whole
    src.for_each([&](uint32_t key, uint32_t idx) {
        const uint32_t bk = bins(key);
        out_append(sm, bk > d || (whole && bk == d), idx, m, p, b, orow);
        const bool cand = !whole && bk == d;
        const uint32_t slot = wave_reserve(&sm.ncand, cand);
        if (cand && slot < (uint32_t)kMaxCand) {
            sm.cand_key[slot] = key;
            sm.cand_idx[slot] = idx;
        }
    });
    if (whole) return;
    __syncthreads();
    if (threadIdx.x < 64) {
        const uint32_t lane = lane_id();
        const uint32_t nc = f.count;
        const bool have = lane < nc;
        const uint32_t kj = have ? sm.cand_key[lane] : 0u;
        const uint32_t ij = have ? sm.cand_idx[lane] : 0u;
        uint32_t r = 0;  // candidates ranked before this one
        for (uint32_t i = 0; i < nc; ++i) {
            const uint32_t ki = sm.cand_key[i];
            const uint32_t ii = sm.cand_idx[i];
            r += (ki > kj || (ki == kj && ii < ij)) ? 1u : 0u;
        }
        out_append(sm, have && r < need, ij, m, p, b, orow);
    }
}

__device__ void load_row_to_lds(Shared& sm, const float* row, int64_t L) {
    const f4* r4 = reinterpret_cast<const f4*>(row);
    const int64_t nvec = L >> 2;
    for (int64_t v = threadIdx.x; v < nvec; v += kThreads) {
        const f4 x = r4[v];
        const uint32_t i = (uint32_t)(4 * v);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            sm.key[i + c] = order_key(x[c]);
            sm.idx[i + c] = i + (uint32_t)c;
        }
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

    for (int i = threadIdx.x; i < kBins; i += kThreads) sm.hist[i] = 0u;
    if (threadIdx.x == 0) {
        sm.count = 0u;
        sm.emitted = 0u;
        sm.vmax = 0u;
        sm.smax = 0u;
        sm.ncand = 0u;
    }
    for (int j = (int)m + threadIdx.x; j < k; j += kThreads) orow[j] = -1;
    __syncthreads();

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
            uint32_t lo, hi;
            key_range(sm, src, lo, hi);
            const Selection s = select_top(sm, src, m, (uint32_t)L, lo, hi, bits_for(L));
            emit(sm, src, s, m, p, b, orow);
            code = TOPK_ROW_LDS;
        } else if (path == TOPK_PATH_SAMPLED) {
            StreamBins bins;
            uint32_t hi;
            const uint32_t n = sampled_survivors(sm, row, L, m, cap, bins, hi);
            seen = n;
            if (n >= m && n <= cap) {
                finish_survivors(sm, n, m, bins, hi, bits_for(L), p, b, orow);
                code = TOPK_ROW_SAMPLED;
            } else {
                // the survivor histogram is of no use to the full-row passes
                for (int i = threadIdx.x; i < kBins; i += kThreads) sm.hist[i] = 0u;
                __syncthreads();
                code = n > cap ? TOPK_ROW_FULL_OVERFLOW : TOPK_ROW_FULL_UNDERFLOW;
            }
        }
        if (code >= TOPK_ROW_FULL_OVERFLOW) {
            const RowSource src{row, L};
            const Selection s = select_top(sm, src, m, (uint32_t)L, 0u, 0xFFFFFFFFu, bits_for(L));
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
