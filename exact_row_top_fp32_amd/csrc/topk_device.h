// Device building blocks of the exact per-row top-k kernels (gfx950, wave64).
//
// Everything selects on a uint32 key that orders the fp32 bit patterns by
// value, so no float compare, rounding or denormal flush is involved.
// The cooperative helpers are written once for two scopes: a whole workgroup
// (barriers) or a single wave (no barriers), so the same radix selection runs
// either on all lanes of a workgroup or on one wave while the others stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace topk {

constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;
constexpr int kBinsPerLane = kBins / 64;
constexpr int kMaxCand = 64;  // cutoff-bin entries one wave ranks directly

typedef float f4 __attribute__((ext_vector_type(4)));

// fp32 bits -> uint32 whose unsigned order is the value order: negative
// patterns are inverted, non-negative ones get the sign bit set. -0 lands just
// below +0, -inf at the bottom of the finite range, +inf at the top (vLLM PR
// #56346 report, implementation item 1: a uint32 total-order key).
__device__ __forceinline__ uint32_t order_key(float x) {
    const uint32_t u = __float_as_uint(x);
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x & 63u; }
// wave index in the workgroup, known to the compiler to be wave-uniform
__device__ __forceinline__ uint32_t wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// number of set bits of `mask` below this lane
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Cross-lane steps use DPP row operations (VALU only; no LDS round trip).
// dpp controls: row_shr:n = 0x110 + n, row_bcast:15 = 0x142 (lane 15 of a
// row to the next row), row_bcast:31 = 0x143 (lane 31 to rows 2 and 3). A
// lane whose source lies outside its row, or whose row is masked off, takes
// `fill`. Every lane of the wave must be active.
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ uint32_t dpp(uint32_t fill, uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)fill, (int)x, kCtrl, kRowMask, 0xF, false);
}

__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t x) {
    x += dpp<0x111>(0u, x);  // within rows of 16: Hillis-Steele over 1, 2, 4, 8
    x += dpp<0x112>(0u, x);
    x += dpp<0x114>(0u, x);
    x += dpp<0x118>(0u, x);
    x += dpp<0x142, 0xA>(0u, x);  // rows 1 and 3 add the row before
    x += dpp<0x143, 0xC>(0u, x);  // rows 2 and 3 add rows 0 and 1
    return x;
}

// Reductions: each row's lane 15 ends up holding its row's result; the four
// are combined in scalar registers, so the result is wave-uniform.
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
    x = max(x, dpp<0x111>(0u, x));
    x = max(x, dpp<0x112>(0u, x));
    x = max(x, dpp<0x114>(0u, x));
    x = max(x, dpp<0x118>(0u, x));
    const uint32_t a = __builtin_amdgcn_readlane(x, 15), b = __builtin_amdgcn_readlane(x, 31);
    const uint32_t c = __builtin_amdgcn_readlane(x, 47), d = __builtin_amdgcn_readlane(x, 63);
    return max(max(a, b), max(c, d));
}

__device__ __forceinline__ uint32_t wave_min(uint32_t x) {
    x = min(x, dpp<0x111>(0xFFFFFFFFu, x));
    x = min(x, dpp<0x112>(0xFFFFFFFFu, x));
    x = min(x, dpp<0x114>(0xFFFFFFFFu, x));
    x = min(x, dpp<0x118>(0xFFFFFFFFu, x));
    const uint32_t a = __builtin_amdgcn_readlane(x, 15), b = __builtin_amdgcn_readlane(x, 31);
    const uint32_t c = __builtin_amdgcn_readlane(x, 47), d = __builtin_amdgcn_readlane(x, 63);
    return min(min(a, b), min(c, d));
}

// Slot for every active lane with `pred` from a shared LDS counter: one
// atomic per wave, lanes ranked by mbcnt over the ballot.
__device__ __forceinline__ uint32_t wave_reserve(uint32_t* counter, bool pred) {
    const uint64_t mask = __ballot(pred);
    uint32_t base = 0u;
    if (mask != 0) {
        const int leader = __ffsll((unsigned long long)mask) - 1;
        if ((int)lane_id() == leader) base = atomicAdd(counter, (uint32_t)__popcll(mask));
        base = __builtin_amdgcn_readlane(base, leader);
    }
    return base + lanes_below(mask);
}

// Slots for every lane's `cnt` entries from a counter (LDS or device
// memory): one atomic per wave, lanes placed by a wave prefix sum. Every lane
// of the wave must be active.
__device__ __forceinline__ uint32_t wave_reserve_count(uint32_t* counter, uint32_t cnt) {
    const uint32_t incl = wave_inclusive_sum(cnt);
    const uint32_t total = __builtin_amdgcn_readlane(incl, 63);
    uint32_t base = 0u;
    if (total != 0u) {
        if (lane_id() == 0) base = atomicAdd(counter, total);
        base = __builtin_amdgcn_readfirstlane(base);
    }
    return base + incl - cnt;
}

__device__ __forceinline__ f4 load_nt(const f4* p) { return __builtin_nontemporal_load(p); }
// A selection's output, written once and never read back by the kernel:
// streamed past the L2 so that it takes no lines the rows' loads still use.
__device__ __forceinline__ void store_nt(int32_t* p, int32_t v) { __builtin_nontemporal_store(v, p); }

// ----------------------------------------------------------------------------
// cooperative scopes
// ----------------------------------------------------------------------------

template <int NT>
struct BlockScope {
    static constexpr int kSize = NT;
    __device__ static uint32_t rank() { return threadIdx.x; }
    __device__ static bool first_wave() { return threadIdx.x < 64; }
    // A workgroup barrier that orders LDS only. Waves share data through LDS
    // alone, so no wave has to wait for its outstanding global loads (a
    // full __syncthreads would drain every wave's loads in flight).
    __device__ static void sync() {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    }
};

struct WaveScope {
    static constexpr int kSize = 64;
    __device__ static uint32_t rank() { return lane_id(); }
    __device__ static bool first_wave() { return true; }
    __device__ static void sync() {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
};

// LDS state a selection works in: a histogram that is all zero between
// passes, and three words for the bin a search found.
struct SelectLds {
    uint32_t* hist;
    uint32_t* found;
};

struct Found {
    uint32_t digit;  // bin holding the rank-th element from the top
    uint32_t above;  // elements in higher bins
    uint32_t count;  // elements in that bin
};

// A lane's q-th 16-byte read of its own run of 32 words, the runs of all
// lanes 128 bytes apart: the lanes take the run's 8 pieces in rotated orders
// (q + lane + lane / 8, mod 8), so that the lanes of one read touch distinct
// LDS banks, 8 lanes at a time over 32 banks or 16 at a time over 64 (in
// plain order every lane would touch the same four banks).
__device__ __forceinline__ int run_piece(int q, uint32_t lane) {
    return (int)(((uint32_t)q + lane + (lane >> 3)) & 7u);
}

// One wave: the bin of the rank-th element from the top of a 2048-bin
// histogram (a wave prefix sum over 32-bin groups, lane 0 holding the top
// group, then one over the chosen group's bins). Every lane gets the result;
// the histogram is left as it is. 1 <= rank <= histogram total. kSpread:
// the group reads in rotated order (run_piece), free of bank conflicts at
// the cost of a few registers.
template <bool kSpread = false>
__device__ __forceinline__ Found wave_locate(const uint32_t* hist, uint32_t rank) {
    static_assert(kBinsPerLane == 32, "a run of 8 16-byte pieces per lane");
    const uint32_t lane = lane_id();
    const uint32_t base = kBins - kBinsPerLane * (lane + 1);
    const uint4* h4 = reinterpret_cast<const uint4*>(hist + base);
    uint32_t s = 0;
#pragma unroll
    for (int q = 0; q < kBinsPerLane / 4; ++q) {
        const uint4 v = h4[kSpread ? run_piece(q, lane) : q];
        s += v.x + v.y + v.z + v.w;
    }
    const uint32_t incl = wave_inclusive_sum(s);
    const uint64_t own = __ballot(incl - s < rank && rank <= incl);
    Found f{0u, 0u, 0u};
    if (own != 0) {
        const int owner = __ffsll((unsigned long long)own) - 1;
        const uint32_t obase = kBins - kBinsPerLane * (uint32_t)(owner + 1);
        const uint32_t oabove = (uint32_t)__builtin_amdgcn_readlane((int)(incl - s), owner);
        const bool mine = lane < (uint32_t)kBinsPerLane;
        const uint32_t bin = obase + kBinsPerLane - 1 - (lane & (kBinsPerLane - 1));
        const uint32_t c = mine ? hist[bin] : 0u;
        const uint32_t ci = oabove + wave_inclusive_sum(c);
        const uint64_t at = __ballot(mine && ci - c < rank && rank <= ci);
        const int who = __ffsll((unsigned long long)at) - 1;
        f.digit = (uint32_t)__builtin_amdgcn_readlane((int)bin, who);
        f.above = (uint32_t)__builtin_amdgcn_readlane((int)(ci - c), who);
        f.count = (uint32_t)__builtin_amdgcn_readlane((int)c, who);
    }
    return f;
}

// After the histogram atomics of a pass and a sync: the scope's first wave
// locates the bin of the rank-th element from the top, zeroes the histogram
// for the next pass and publishes the bin to the scope. kSpread as for
// wave_locate.
template <class S, bool kSpread = false>
__device__ __forceinline__ Found find_rank_bin(SelectLds lds, uint32_t rank) {
    if (S::first_wave()) {
        const Found f = wave_locate<kSpread>(lds.hist, rank);
        const uint32_t lane = lane_id();
        uint4* h4 = reinterpret_cast<uint4*>(lds.hist + kBins - kBinsPerLane * (lane + 1));
#pragma unroll
        for (int q = 0; q < kBinsPerLane / 4; ++q)
            h4[kSpread ? run_piece(q, lane) : q] = make_uint4(0u, 0u, 0u, 0u);
        if (lane == 0) {
            lds.found[0] = f.digit;
            lds.found[1] = f.above;
            lds.found[2] = f.count;
        }
    }
    S::sync();
    return Found{lds.found[0], lds.found[1], lds.found[2]};
}

// ----------------------------------------------------------------------------
// element sources: keys held in LDS, or a row of fp32 scores in global memory
// ----------------------------------------------------------------------------

// Survivors held in LDS as (raw score bits, position) pairs; yields keys.
template <class S>
struct PairSource {
    const uint2* entry;
    uint32_t n;
    template <class F>
    __device__ void for_each(F&& f) const {
        for (uint32_t e = S::rank(); e < n; e += S::kSize) {
            const uint2 v = entry[e];
            f(order_key(__uint_as_float(v.x)), v.y);
        }
    }
};

template <class S>
struct RowSource {
    const float* row;
    int64_t len;
    template <class F>
    __device__ void for_each(F&& f) const {
        const f4* r4 = reinterpret_cast<const f4*>(row);
        const int64_t nvec = len >> 2;
        for (int64_t v = S::rank(); v < nvec; v += S::kSize) {
            const f4 x = r4[v];
            const uint32_t i = (uint32_t)(4 * v);
            f(order_key(x.x), i);
            f(order_key(x.y), i + 1);
            f(order_key(x.z), i + 2);
            f(order_key(x.w), i + 3);
        }
        for (int64_t i = 4 * nvec + S::rank(); i < len; i += S::kSize) f(order_key(row[i]), (uint32_t)i);
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
template <int kShift>
struct CoarseKeyView {
    __device__ bool operator()(uint32_t key, uint32_t, uint32_t& v) const {
        v = key >> kShift;
        return true;
    }
};
struct AtLeastView {
    uint32_t lo;
    __device__ bool operator()(uint32_t key, uint32_t, uint32_t& v) const {
        v = key;
        return key >= lo;
    }
};
struct TieIndexView {
    uint32_t tie;
    __device__ bool operator()(uint32_t key, uint32_t idx, uint32_t& v) const {
        v = ~idx;
        return key == tie;
    }
};

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
template <class S, class Src, class View>
__device__ __forceinline__ Cut radix_select(SelectLds lds, const Src& src, View view, uint32_t rank, uint32_t prefix,
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
            if (view(key, idx, v) && (v & done_mask) == want) atomicAdd(&lds.hist[(v >> shift) & dmask], 1u);
        });
        S::sync();
        const Found f = find_rank_bin<S>(lds, rank);
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

// Exact top m among `src`, whose keys all lie in [lo, hi]; indices < 2^idx_bits.
// Ties at the cutoff go to the lowest indices, so the selected set is unique.
template <class S, class Src>
__device__ __forceinline__ Selection select_top(SelectLds lds, const Src& src, uint32_t m, uint32_t n, uint32_t lo,
                                uint32_t hi, int idx_bits) {
    const int nbits = lo == hi ? 0 : 32 - __clz(lo ^ hi);
    const Cut c = radix_select<S>(lds, src, KeyView{}, m, lo, nbits, n);
    if (c.range) return at_least(c.value);
    Selection s{c.value, INT32_MAX};
    if (c.need < c.equal) {
        // the need-th largest inverted index among the ties; inverted indices
        // below 2^idx_bits share their top 32 - idx_bits bits
        const uint32_t iprefix = idx_bits >= 32 ? 0u : (0xFFFFFFFFu << idx_bits);
        const Cut t = radix_select<S>(lds, src, TieIndexView{c.value}, c.need, iprefix, idx_bits, c.equal);
        s.icut = (int32_t)(~t.value);  // exact or range: inverted index >= value
    }
    return s;
}

__device__ __forceinline__ int bits_for(int64_t L) {  // bits to hold indices 0..L-1, L >= 2
    return 64 - __clzll((unsigned long long)(L - 1));
}

// One output row: slots [0, m) receive selected positions (mapped through the
// page table in paged mode), handed out by an LDS counter.
struct OutRow {
    int32_t* row;
    const int32_t* pages;  // this row's page-table entries, or null
    int32_t page_size;
    uint32_t m;
    uint32_t* emitted;  // LDS counter, zero before the row's first append
    __device__ __forceinline__ int32_t map(uint32_t i) const {
        if (pages == nullptr) return (int32_t)i;
        const int64_t page = pages[i / (uint32_t)page_size];
        return (int32_t)(page * page_size + (int64_t)(i % (uint32_t)page_size));
    }
    // A row's selection holds exactly m elements; the bound only keeps a
    // defect from writing outside the row.
    __device__ __forceinline__ void append(bool take, uint32_t idx) const {
        const uint32_t slot = wave_reserve(emitted, take);
        if (take && slot < m) row[slot] = map(idx);
    }
};

// Output slots handed out by one wave alone: a counter that every lane keeps,
// so appends need no atomics. Every lane must run every append (uniform
// loops only): a lane idle during an append misses the count.
struct WaveOutRow {
    OutRow out;
    uint32_t next;
    __device__ __forceinline__ void append(bool take, uint32_t idx) {
        const uint64_t mask = __ballot(take);
        if (take) {
            const uint32_t slot = next + lanes_below(mask);
            if (slot < out.m) out.row[slot] = out.map(idx);
        }
        next += (uint32_t)__popcll(mask);
    }
};

// Writes every element of `src` the selection takes; `out` is an OutRow
// (workgroup) or a WaveOutRow (one wave).
template <class Src, class Out>
__device__ __forceinline__ void emit(const Src& src, Selection s, Out& out) {
    src.for_each([&](uint32_t key, uint32_t idx) {
        out.append(key > s.kth || (key == s.kth && (int32_t)idx <= s.icut), idx);
    });
}

}  // namespace topk
