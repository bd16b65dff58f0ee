// Exact per-row top-k with each row split over several workgroups, for
// batches too small to fill the chip one row per compute unit (gfx950).
//
// With one workgroup per row, a batch of 40 rows keeps 40 of 256 compute
// units busy. Here every row is cut into pieces of equal size, one workgroup
// each, so the grid fills the chip at any batch (the counterpart of the
// cluster-split rows of "dsv4.1: Top-k kernels and candidate selection",
// implementation section 4, where several blocks share one long row). Three
// launches on the caller's stream, and a workspace the caller owns:
//
//  1. split_sample_kernel, one workgroup per row: a row with L <= k is written
//     out directly; any other row gets its cutoff key T from a sample of the
//     row (vLLM PR #56346 report, summary and implementation item 1: a
//     sampled cutoff, then exact selection among the survivors) and a fresh
//     header in the workspace.
//  2. split_stream_kernel, one workgroup per piece: reads its piece once and
//     appends every (raw score bits, position) with key >= T to the row's
//     survivor area in the workspace, one device-scope reservation per wave
//     and load round, counting on past the capacity without writing (same
//     page, implementation item 1).
//  3. split_finish_kernel, one workgroup per row: loads the row's survivors
//     into LDS (all loads in flight at once) and selects the exact top m
//     there, or, when they overflowed the area or fell short of m, runs the
//     full-row exact selection: histogram passes down to the cutoff, then one
//     emission scan ("Fix incorrect sparse-attention top-k selection when
//     candidate bins overflow", comment thread: cutoff first).
//
// Kernel boundaries order the three steps, so no workgroup waits for another
// and no device-scope fence is needed.
//
// The same pieces serve short rows in a single launch (short_rows_kernel):
// one workgroup per row takes the sample, streams the row once into an LDS
// survivor buffer and selects there, falling back to the full-row selection
// when the buffer overflows or the survivors fall short of m. topk_select
// sends rows of at most 32768 scores here; topk_select_bf16 sends every bf16
// row, widening each score exactly to fp32 as it is loaded.
//
// The selected set is the one every other path returns: all positions whose
// key is above the cutoff key, then the lowest positions equal to it.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "exact_topk.h"
#include "topk_device.h"
#include "topk_short.h"

namespace topk {
namespace {

constexpr int kThreads = 256;                   // 4 waves per workgroup
constexpr int kUnroll = 8;                      // 16-byte loads per lane per round
constexpr int64_t kRound = kThreads * kUnroll;  // 4-score groups per workgroup round (32 KB)
constexpr int kRunLen = 64;                     // scores per contiguous sample run
constexpr int kMaxRuns = 64;                    // sample runs of a split row
constexpr int kShortRuns = 32;                  // sample runs of a short row up to kShortLong scores
constexpr int64_t kShortLong = 16384;           // longer short rows take kMaxRuns runs
constexpr int kMaxPieces = 256;                 // workgroups per row at most
constexpr int kFinThreads = 1024;               // finisher workgroup: 16 waves

constexpr uint32_t kKindSampled = 0, kKindAll = 1, kKindFull = 2, kKindDirect = 3;

// Per-row header in the workspace; the sample kernel writes all of it.
struct SplitHead {
    uint32_t count;  // survivors reserved (may exceed the capacity)
    uint32_t spare;  // unused (keeps the header 16 bytes)
    uint32_t T;      // cutoff key: survivors have key >= T
    uint32_t kind;   // kKind*
};

struct SplitParams {
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
    int32_t capacity;  // survivor entries per row, <= kSplitCapacity
    int32_t* row_stats;
    int64_t batch;
    SplitHead* head;     // [batch]
    uint2* surv;         // [batch][kSplitCapacity]: (raw score bits, position)
    int64_t piece_vec;   // 4-score groups per piece, a multiple of kRound
    int32_t pieces;      // workgroups per row
    uint32_t page_magic;  // position / page_size = (position * page_magic) >> page_shift
    int32_t page_shift;
};

// Division by the page size as a multiply, exact for positions below 2^31
// (Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994: with l = ceil(log2 d), the 32-bit multiplier
// ceil(2^(31 + l) / d) and a shift by 31 + l).
inline void page_divider(int32_t page_size, uint32_t& magic, int32_t& shift) {
    magic = 0u;
    shift = 0;
    if (page_size < 1) return;
    const uint64_t d = (uint64_t)page_size;
    int l = 0;
    while ((1ull << l) < d) ++l;
    magic = (uint32_t)(((1ull << (31 + l)) + d - 1) / d);
    shift = 31 + l;
}

constexpr int64_t kSplitCapacity = 8192;  // survivor entries per row in the workspace

constexpr int64_t head_bytes(int64_t batch) { return (batch * (int64_t)sizeof(SplitHead) + 255) & ~(int64_t)255; }
constexpr int64_t split_workspace_bytes(int64_t batch) {
    return head_bytes(batch) + batch * kSplitCapacity * (int64_t)sizeof(uint2);
}

__device__ __forceinline__ int64_t split_row_len(const SplitParams& p, int64_t b) {
    int64_t L = p.lengths ? (int64_t)p.lengths[b] : p.n_cols;
    return L < 0 ? 0 : (L > p.n_cols ? p.n_cols : L);
}

__device__ __forceinline__ OutRow split_out_row(const SplitParams& p, int64_t b, uint32_t m, uint32_t* emitted) {
    return OutRow{p.out + b * (int64_t)p.k, p.page_table ? p.page_table + b * p.pt_stride : nullptr,
                  p.page_size, m, emitted};
}

__device__ __forceinline__ void split_stats(const SplitParams& p, int64_t b, int code, uint32_t seen) {
    if (p.row_stats != nullptr) {
        p.row_stats[2 * b + 0] = code;
        p.row_stats[2 * b + 1] = (int32_t)seen;
    }
}

// A lane's sample keys held in registers: kLoads loads of kPer keys each,
// load h present when h * kThreads + threadIdx.x < nload (the workgroup's
// loads). The views of the sample ignore positions.
template <int kLoads, int kPer>
struct RegKeys {
    const uint32_t (&key)[kLoads * kPer];
    int nload;
    template <class F>
    __device__ void for_each_slot(F&& f) const {
#pragma unroll
        for (int h = 0; h < kLoads; ++h) {
            const bool valid = h * kThreads + (int)threadIdx.x < nload;
#pragma unroll
            for (int j = 0; j < kPer; ++j) f(key[h * kPer + j], 0u, valid);
        }
    }
};

// Survivors held in registers, N slots per lane: slot i of a lane holds the
// order key and the position of one survivor, or key 0 and the position
// 0xFFFFFFFF (no survivor; positions are below 2^31, and key 0 lies below
// every cutoff, which is at least kMinT). Slots at or
// past `nslot` are empty on every lane. Slots are visited in groups of
// kGroup, a group wholly past nslot skipped by one uniform test (a test per
// slot would hold a mask register per slot).
constexpr int kGroup = 4;
template <int N>
struct RegPairs {
    uint32_t key[N];
    uint32_t idx[N];
    int nslot;
    template <class F>
    __device__ __forceinline__ void for_each_group(F&& f) const {
#pragma unroll
        for (int g = 0; g < N; g += kGroup) {
            if (g < nslot) {
#pragma unroll
                for (int i = g; i < (g + kGroup < N ? g + kGroup : N); ++i) f(i);
            }
        }
    }
    template <class F>
    __device__ __forceinline__ void for_each_slot(F&& f) const {
        for_each_group([&](int i) { f(key[i], idx[i], idx[i] != 0xFFFFFFFFu); });
    }
};

// ----------------------------------------------------------------------------
// score rows and their sampled cutoff (both the split-row and short-row kernels)
// ----------------------------------------------------------------------------

// The least sh with (d >> sh) <= kBins - 3, so that a span of d + 1 keys
// fits kBins - 2 bins of width 2^sh: the top bit of d placed at bit 10, one
// more when that still leaves d >> sh at kBins - 2 or above.
__device__ __forceinline__ int bin_shift(uint32_t d) {
    const int top = 31 - (int)__clz(d | 1u);
    const int sh0 = top > kDigitBits - 1 ? top - (kDigitBits - 1) : 0;
    return sh0 + ((d >> sh0) >= (uint32_t)(kBins - 2) ? 1 : 0);
}

// Radix selection as radix_select does it, over a source that yields every
// register slot, valid or not (Src::for_each_slot): the histogram updates
// take no branches, a slot outside the pass adding to its lane's sink bin
// hist[kBins + lane], which nothing reads. hist holds kBins + 64 words.
template <class S, class Src, class View>
__device__ __forceinline__ Cut radix_select_slots(SelectLds lds, const Src& src, View view, uint32_t rank,
                                                  uint32_t prefix, int nbits, uint32_t equal_if_none) {
    Cut cut{prefix, rank, equal_if_none, false};
    const uint32_t sink = (uint32_t)kBins + lane_id();
    while (nbits > 0) {
        const int w = nbits < kDigitBits ? nbits : kDigitBits;
        const int shift = nbits - w;
        const uint32_t done_mask = nbits >= 32 ? 0u : (0xFFFFFFFFu << nbits);
        const uint32_t want = prefix & done_mask;
        const uint32_t dmask = (1u << w) - 1u;
        src.for_each_slot([&](uint32_t key, uint32_t idx, bool valid) {
            uint32_t v;
            const bool in = view(key, idx, v) && valid && (v & done_mask) == want;
            atomicAdd(&lds.hist[in ? (v >> shift) & dmask : sink], 1u);
        });
        S::sync();
        const Found f = find_rank_bin<S, true>(lds, rank);
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

typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// Element types of a score row, read 16 bytes at a time: fp32, or bf16 (its
// bit pattern, the top half of the fp32 it denotes exactly). bits() gives the
// fp32 pattern of element j of a load, so keys, survivors and selection are
// the fp32 ones for both.
//
// pass<kPos>() is the survivor test key >= T on a load's raw bits, one integer
// compare per score, exact for every non-NaN score (SurvivorBound holds the
// bounds): with T at or above the key of +0 (kPos), a score passes when its
// bits as a signed integer reach T ^ 0x80000000, and below it when its bits as
// an unsigned integer are at most ~T. A load of all-ones words (a NaN
// pattern) fails both tests once T is at least kMinT: lanes past a row's end
// load it instead (g_pad).
struct SurvivorBound {
    uint32_t t;   // kPos: T ^ 0x80000000 (signed compare); else ~T (unsigned)
    uint32_t th;  // bf16: the same bound for a score's 16 bits, compared in place in its half word
};
constexpr uint32_t kMinT = 0x10000u;  // below -inf's key 0x007FFFFF: every non-NaN score passes
__device__ __align__(16) const uint32_t g_pad[4] = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};

struct F32Elem {
    typedef f4 Vec;
    typedef float Scalar;
    static constexpr int kPerVec = 4;
    static constexpr int kUnroll = 8;  // loads per lane per round: 32 scores
    static constexpr bool kSecondAtCutoff = false;  // see short_rows_kernel
    __device__ static uint32_t bits(const Vec& v, int j) { return __float_as_uint(v[j]); }
    __device__ static uint32_t scalar_bits(Scalar x) { return __float_as_uint(x); }
    static constexpr int kKeyShift = 0;  // every key bit carries information
    __device__ static uint32_t full_key(uint32_t v) { return v; }
    __device__ __forceinline__ static SurvivorBound bound(uint32_t T, bool pos) {
        const uint32_t t = pos ? (T ^ 0x80000000u) : ~T;
        return SurvivorBound{t, t};
    }
    template <bool kPos>
    __device__ static bool pass(const Vec& v, int j, SurvivorBound b) {
        const uint32_t x = __float_as_uint(v[j]);
        return kPos ? (int32_t)x >= (int32_t)b.t : x <= b.t;
    }
    // the 32-bit word of a load holding element j, the fp32 bits of the
    // score at position i held in such a word, and a word holding bits there
    __device__ static uint32_t word(const Vec& v, int j) { return __float_as_uint(v[j]); }
    __device__ static uint32_t word_bits(uint32_t w, uint32_t) { return w; }
    __device__ static uint32_t bits_word(uint32_t bits, uint32_t) { return bits; }
};
struct Bf16Elem {
    typedef u4 Vec;
    typedef uint16_t Scalar;
    static constexpr int kPerVec = 8;
    static constexpr int kUnroll = 4;  // loads per lane per round: 32 scores
    static constexpr bool kSecondAtCutoff = true;  // see short_rows_kernel
    __device__ static uint32_t bits(const Vec& v, int j) {
        return (j & 1) ? (v[j >> 1] & 0xFFFF0000u) : (v[j >> 1] << 16);
    }
    __device__ static uint32_t scalar_bits(Scalar x) { return (uint32_t)x << 16; }
    // The order key of a widened bf16 score is fixed by its top 16 bits: the
    // low 16 are 0 for a non-negative score (key bit 31 set) and all ones for
    // a negative one, so selecting on key >> 16 is exact.
    static constexpr int kKeyShift = 16;
    __device__ static uint32_t full_key(uint32_t v) { return (v << 16) | ((v >> 15) & 1u ? 0u : 0xFFFFu); }
    // A score is tested on its 16 bits in place: its widened bits h << 16,
    // as a signed integer, reach t >= 0 exactly when h as a signed 16-bit
    // integer reaches ceil(t / 2^16); as an unsigned integer they stay at or
    // below t exactly when h stays at or below floor(t / 2^16).
    __device__ __forceinline__ static SurvivorBound bound(uint32_t T, bool pos) {
        if (pos) {
            const uint32_t t = T ^ 0x80000000u;  // at most 0x7FFFFFFF
            return SurvivorBound{t, (uint32_t)(((uint64_t)t + 0xFFFFu) >> 16)};  // at most 2^15
        }
        const uint32_t t = ~T;
        return SurvivorBound{t, t >> 16};
    }
    template <bool kPos>
    __device__ static bool pass(const Vec& v, int j, SurvivorBound b) {
        const uint32_t w = v[j >> 1];
        const uint32_t h = (j & 1) ? (w >> 16) : (w & 0xFFFFu);
        return kPos ? (int32_t)(int16_t)h >= (int32_t)b.th : h <= b.th;
    }
    // Element j of a load is half j & 1 of word j >> 1, and positions keep
    // that parity (a load starts at a multiple of 8): a survivor is kept as
    // its whole word and its position.
    __device__ static uint32_t word(const Vec& v, int j) { return v[j >> 1]; }
    __device__ static uint32_t word_bits(uint32_t w, uint32_t i) { return (i & 1u) ? (w & 0xFFFF0000u) : (w << 16); }
    __device__ static uint32_t bits_word(uint32_t bits, uint32_t i) { return (i & 1u) ? bits : bits >> 16; }
};

template <class E>
__device__ __forceinline__ uint32_t elem_key(uint32_t bits) { return order_key(__uint_as_float(bits)); }

// Every score of a row in global memory (the full-row selection's source),
// E::kUnroll loads per lane in flight as in the streaming rounds (one at a
// time, a workgroup reads a long row at a small fraction of its share of the
// memory bandwidth).
template <class S, class E>
struct ElemRowSource {
    const typename E::Scalar* row;
    int64_t len;
    template <class F>
    __device__ void for_each(F&& f) const {
        constexpr int kU = E::kUnroll;
        const typename E::Vec* rv = reinterpret_cast<const typename E::Vec*>(row);
        const int64_t nvec = len / E::kPerVec;
        for (int64_t v0 = S::rank(); v0 < nvec; v0 += (int64_t)kU * S::kSize) {
            typename E::Vec x[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int64_t v = v0 + (int64_t)u * S::kSize;
                if (v < nvec) x[u] = rv[v];
            }
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int64_t v = v0 + (int64_t)u * S::kSize;
                if (v < nvec) {
#pragma unroll
                    for (int j = 0; j < E::kPerVec; ++j)
                        f(elem_key<E>(E::bits(x[u], j)), (uint32_t)(E::kPerVec * v + j));
                }
            }
        }
        for (int64_t i = E::kPerVec * nvec + S::rank(); i < len; i += S::kSize)
            f(elem_key<E>(E::scalar_bits(row[i])), (uint32_t)i);
    }
};

constexpr uint32_t kInfKey = 0xFF800000u;  // order key of +inf

// A sample key at or above lo: keys up to hi binned (key - base) >> sh,
// keys above hi (+inf) in the top bin.
struct SampleBinView {
    uint32_t lo, hi, base;
    int sh;
    __device__ bool operator()(uint32_t key, uint32_t, uint32_t& v) const {
        v = key > hi ? (uint32_t)(kBins - 1) : (key - base) >> sh;
        return key >= lo;
    }
};

// A sample key the first histogram put in the bin [edge, top] (keys from lo
// on), in sub-bins of width 2^sh from edge.
struct SubBinView {
    uint32_t edge, lo, top;
    int sh;
    __device__ bool operator()(uint32_t key, uint32_t, uint32_t& v) const {
        v = (key - edge) >> sh;
        return key >= lo && key <= top;
    }
};

// The cutoff key of a row from its sample: `runs` runs of 64 contiguous
// scores at evenly spaced offsets over [0, L). When the sample has fewer than
// `want` keys above the row's m-th largest, fewer than m scores can be at or
// above T; the rank is set so that this is a six-sigma event: the number of
// sample keys at or above the m-th largest score is binomial with mean
// mu = m n / L, and want = ceil(mu + 6 sqrt(mu) + 4). T is at or below the
// want-th largest sample key: the lower edge of its bin in one histogram of
// the keys in [lo, hi] (lo a bound from each lane's largest keys, hi the
// largest below +inf's, bins a power of two wide; a bin crowded below the
// wanted key is split once more), or, when the lanes hold
// too few keys for that bound, the lowest key of its top 22 bits (two 11-bit
// digits, at most 2^10 keys below it).
//
// The sample has at most kRuns runs: 64 for the split rows and for short rows
// longer than kShortLong, 32 for the others, where the sample's own work is a
// larger part of the row's. Over N(0,1) rows, 2048 keys of a 16384-score row
// leave about 1.4 m survivors for m = 2048 and 1.8 m for m = 512; at 32768
// scores and m = 2048 they would leave 1.6 m (p99 3680 of the short-row
// kernel's 3840 entries, before the cutoff moves down to its bin's edge),
// 4096 keys about 1.4 m.
//
// `issue(true)` runs right after the sample's loads are issued (`issue(false)`
// on the early return of a row too short to sample), so that a caller's own
// loads are in flight while the cutoff is found.
struct NoIssue {
    __device__ void operator()(bool) const {}
};

struct Cutoff {
    uint32_t T;   // the cutoff key
    uint32_t hi;  // the sample's largest key below +inf's (0xFFFFFFFF: no sample)
};

template <class E, int kRuns = kMaxRuns, class Issue = NoIssue>
__device__ __forceinline__ Cutoff short_cutoff(const typename E::Scalar* row, int64_t L, uint32_t m, SelectLds lds,
                                               Issue&& issue = Issue{}) {
    using B = BlockScope<kThreads>;
    const int64_t fit = L / (2 * kRunLen);
    const int runs = fit < kRuns ? (int)fit : kRuns;
    if (runs < 2) {
        issue(false);
        return Cutoff{0u, 0xFFFFFFFFu};
    }
    constexpr int kVecPerRun = kRunLen / E::kPerVec;
    constexpr int kPer = kRuns * kRunLen / E::kPerVec / kThreads;  // loads per lane, all in flight
    static_assert(kPer >= 1 && kPer * E::kPerVec * kThreads == kRuns * kRunLen, "whole loads per lane");
    constexpr int kLineVecs = 128 / 16;                       // loads per 128-byte line
    const int nsv = runs * kVecPerRun;
    const int64_t span = L - kRunLen;
    const typename E::Vec* rv = reinterpret_cast<const typename E::Vec*>(row);
    // the row's first load lies `lead` loads into its 128-byte line
    const int64_t lead = (int64_t)((reinterpret_cast<uintptr_t>(row) & 127u) >> 4);
    // floor(r * span / (runs - 1)) = r quo + floor(r rem / (runs - 1)), the
    // last term taken in fp32 as floor((r rem + 1/2) / (runs - 1)): r rem is
    // below 2^12 and (r rem + 1/2) / (runs - 1) lies at least 1/126 from
    // every integer, far more than the rounding error of the product
    const int64_t quo = runs == kRuns ? span / (kRuns - 1) : span / (runs - 1);  // uniform; a constant divisor mostly
    const uint32_t rem = (uint32_t)(span - quo * (runs - 1));
    const float inv = 1.0f / (float)(runs - 1);
    typename E::Vec x[kPer];
#pragma unroll
    for (int h = 0; h < kPer; ++h) {
        const int t = h * kThreads + (int)threadIdx.x;
        const int r = t / kVecPerRun;
        // run r starts near floor(r * span / (runs - 1)), moved down to the
        // start of a 128-byte line (a run of 64 scores then covers whole
        // lines only; the first run stays at 0 when that would go below it)
        const uint32_t frac = (uint32_t)(((float)((uint32_t)r * rem) + 0.5f) * inv);
        int64_t start = ((int64_t)r * quo + frac) / E::kPerVec;
        start = (start + lead) / kLineVecs * kLineVecs - lead;
        start = start < 0 ? 0 : start;
        if (t < nsv) x[h] = rv[start + t % kVecPerRun];
    }
    issue(true);
    const uint32_t n = (uint32_t)(E::kPerVec * nsv);
    const float mu = (float)m * (float)n / (float)L;
    const float wantf = ceilf(mu + 6.0f * sqrtf(mu) + 4.0f);
    const uint32_t want = wantf < (float)n ? (uint32_t)wantf : 0u;  // 0: keep every score
    // Each lane also keeps its q largest keys (and so its largest), q =
    // ceil(want / kThreads) when that is at most kQ. The smallest of the
    // lanes' q-th largest keys, lo, has at least want keys at or above it (a
    // lane with fewer than q keys gives lo = 0).
    constexpr int kQ = 4;
    const uint32_t q = (want + kThreads - 1) / kThreads;
    const bool one_pass = want > 0u && q <= (uint32_t)kQ;  // uniform
    uint32_t lane_lo = 0u;  // the lane's q-th largest key
    uint32_t fin = 0u;      // the lane's largest key below +inf's
    uint32_t skey[kPer * E::kPerVec];
    const RegKeys<kPer, E::kPerVec> keys{skey, nsv};
#pragma unroll
    for (int h = 0; h < kPer; ++h) {
#pragma unroll
        for (int j = 0; j < E::kPerVec; ++j) skey[h * E::kPerVec + j] = elem_key<E>(E::bits(x[h], j));
    }
    // the lane's K largest keys by insertion, K = q rounded up to 1, 2 or kQ
    auto lane_tops = [&](auto k_tag) {
        constexpr int K = decltype(k_tag)::value;
        uint32_t top[K];
#pragma unroll
        for (int i = 0; i < K; ++i) top[i] = 0u;
#pragma unroll
        for (int h = 0; h < kPer; ++h) {
            if (h * kThreads + (int)threadIdx.x < nsv) {
#pragma unroll
                for (int j = 0; j < E::kPerVec; ++j) {
                    uint32_t key = skey[h * E::kPerVec + j];
                    fin = max(fin, key < kInfKey ? key : 0u);
#pragma unroll
                    for (int i = 0; i < K; ++i) {
                        const uint32_t hi = max(top[i], key);
                        key = min(top[i], key);
                        top[i] = hi;
                    }
                }
            }
        }
        lane_lo = top[0];
#pragma unroll
        for (int i = 1; i < K; ++i) lane_lo = (uint32_t)(i + 1) == q ? top[i] : lane_lo;
    };
    if (q <= 1u)
        lane_tops(std::integral_constant<int, 1>{});
    else if (q == 2u)
        lane_tops(std::integral_constant<int, 2>{});
    else
        lane_tops(std::integral_constant<int, kQ>{});
    // the workgroup's lo and hi from one word per wave
    __shared__ uint32_t s_lo[kThreads / 64], s_hi[kThreads / 64];
    const uint32_t wlo = wave_min(lane_lo), whi = wave_max(fin);
    if (lane_id() == 0) {
        s_lo[wave_id()] = wlo;
        s_hi[wave_id()] = whi;
    }
    B::sync();
    uint32_t blo = s_lo[0], shi = s_hi[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) {
        blo = min(blo, s_lo[i]);
        shi = max(shi, s_hi[i]);
    }
    if (want == 0u) return Cutoff{0u, shi};
    if (one_pass) {
        // one histogram of the keys in [lo, hi] (hi the largest below +inf),
        // in at most kBins - 1 bins of width 2^sh from a base aligned to it,
        // keys above hi in the top bin: T is the lower edge of the bin holding
        // the want-th largest key, or hi + 1 when that key is above hi (bf16
        // keys differ by at least 2^16, so their bins hold one value each)
        const uint32_t lo = blo, hi = max(shi, lo);
        const int sh = bin_shift(hi - lo);
        const uint32_t base = lo & ~((1u << sh) - 1u);  // (hi - base) >> sh <= kBins - 2
        const Cut c = radix_select_slots<B>(lds, keys, SampleBinView{lo, hi, base, sh}, want, 0u, kDigitBits, n);
        if (c.value == (uint32_t)(kBins - 1)) return Cutoff{hi + 1u, shi};
        const uint32_t edge = base + (c.value << sh);
        // A few far keys (peaks well above a dense bulk) stretch [lo, hi] so
        // that one bin can hold much of the bulk: a cutoff at its lower edge
        // would let most of the row through and overflow the buffer. When
        // the sample keys in the cutoff bin below the wanted one would add
        // more than a quarter to the survivors, a second histogram of that
        // bin alone, 2^10 times finer, places T.
        if (sh > 0 && 4u * (c.equal - c.need) > want) {
            const int sh2 = sh > kDigitBits - 1 ? sh - (kDigitBits - 1) : 0;
            const uint32_t bin_top = min(edge + ((1u << sh) - 1u), hi);  // no overflow: hi < +inf's key
            const Cut c2 = radix_select_slots<B>(lds, keys, SubBinView{edge, max(edge, lo), bin_top, sh2},
                                           c.need, 0u, kDigitBits, c.equal);
            return Cutoff{edge + (c2.value << sh2), shi};
        }
        return Cutoff{edge, shi};
    }
    constexpr int kDropBits = 32 - 2 * kDigitBits;
    const uint32_t T =
        radix_select_slots<B>(lds, keys, CoarseKeyView<kDropBits>{}, want, 0u, 2 * kDigitBits, n).value
        << kDropBits;
    return Cutoff{T, shi};
}

// ----------------------------------------------------------------------------
// split rows, launch 1: direct rows, cutoffs and headers
// ----------------------------------------------------------------------------

__global__ __launch_bounds__(kThreads) void split_sample_kernel(SplitParams p) {
    using B = BlockScope<kThreads>;
    __shared__ uint32_t hist[kBins + 64];
    __shared__ uint32_t found[3];
    for (int i = (int)threadIdx.x; i < kBins; i += kThreads) hist[i] = 0u;
    B::sync();
    const int64_t b = blockIdx.x;
    const int64_t L = split_row_len(p, b);
    const uint32_t m = (uint32_t)(L < p.k ? L : p.k);
    uint32_t kind, T = 0u;
    if (L <= p.k) {
        kind = kKindDirect;
        const OutRow out = split_out_row(p, b, m, nullptr);
        for (int64_t i = threadIdx.x; i < p.k; i += kThreads) out.row[i] = i < L ? out.map((uint32_t)i) : -1;
        if (threadIdx.x == 0) split_stats(p, b, L == 0 ? TOPK_ROW_EMPTY : TOPK_ROW_ALL, (uint32_t)L);
    } else if (p.force_path == TOPK_PATH_FULLROW) {
        kind = kKindFull;
    } else if (p.force_path == TOPK_PATH_LDS) {
        kind = L <= p.capacity ? kKindAll : kKindFull;
    } else if (p.force_path == TOPK_PATH_AUTO && L <= p.capacity) {
        kind = kKindAll;
    } else {
        kind = kKindSampled;
        T = short_cutoff<F32Elem>(p.scores + b * p.row_stride, L, m, SelectLds{hist, found}).T;
    }
    if (threadIdx.x == 0) p.head[b] = SplitHead{0u, 0u, T, kind};
}

// ----------------------------------------------------------------------------
// launch 2: pieces append their survivors
// ----------------------------------------------------------------------------

__device__ __forceinline__ void load_round(const f4* r4, int64_t base, int64_t g1, f4 (&x)[kUnroll]) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t g = base + u * kThreads + threadIdx.x;
        x[u] = g < g1 ? load_nt(r4 + g) : f4{0.0f, 0.0f, 0.0f, 0.0f};
    }
}

__device__ __forceinline__ void filter_round(const f4 (&x)[kUnroll], int64_t base, int64_t g1, uint32_t T, SplitHead* h,
                                             uint2* surv, uint32_t cap) {
    uint32_t cnt = 0u;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const bool in = base + u * kThreads + threadIdx.x < g1;
#pragma unroll
        for (int j = 0; j < 4; ++j) cnt += (in && order_key(x[u][j]) >= T) ? 1u : 0u;
    }
    uint32_t slot = wave_reserve_count(&h->count, cnt);
    if (cnt != 0u) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t g = base + u * kThreads + threadIdx.x;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (g < g1 && order_key(x[u][j]) >= T) {
                    if (slot < cap) surv[slot] = make_uint2(__float_as_uint(x[u][j]), (uint32_t)(4 * g + j));
                    ++slot;
                }
            }
        }
    }
}

__device__ __forceinline__ void stream_piece(const SplitParams& p, int64_t b, int64_t L, uint32_t T, int piece,
                                             SplitHead* h, uint2* surv, uint32_t cap) {
    const int64_t nvec = L >> 2;
    const int64_t g0 = (int64_t)piece * p.piece_vec;
    const int64_t g1 = g0 + p.piece_vec < nvec ? g0 + p.piece_vec : nvec;
    const float* row = p.scores + b * p.row_stride;
    const f4* r4 = reinterpret_cast<const f4*>(row);
    // two rounds in flight: the next round's loads are issued before this
    // round is filtered (loops uniform over the workgroup)
    f4 a[kUnroll], c[kUnroll];
    int64_t base = g0;
    if (base < g1) load_round(r4, base, g1, a);
    while (base < g1) {
        if (base + kRound < g1) load_round(r4, base + kRound, g1, c);
        filter_round(a, base, g1, T, h, surv, cap);
        base += kRound;
        if (base >= g1) break;
        if (base + kRound < g1) load_round(r4, base + kRound, g1, a);
        filter_round(c, base, g1, T, h, surv, cap);
        base += kRound;
    }
    // the L % 4 scores past the last full group belong to the piece holding
    // that group's successor; its first wave appends them
    if (nvec * 4 < L && nvec / p.piece_vec == piece && threadIdx.x < 64) {
        const int64_t i = nvec * 4 + threadIdx.x;
        const float v = i < L ? row[i] : 0.0f;
        const bool hit = i < L && order_key(v) >= T;
        const uint32_t slot = wave_reserve_count(&h->count, hit ? 1u : 0u);
        if (hit && slot < cap) surv[slot] = make_uint2(__float_as_uint(v), (uint32_t)i);
    }
}

__global__ __launch_bounds__(kThreads) void split_stream_kernel(SplitParams p) {
    const int64_t b = blockIdx.x / (uint32_t)p.pieces;
    const int piece = (int)(blockIdx.x % (uint32_t)p.pieces);
    SplitHead* h = p.head + b;
    const uint32_t kind = h->kind;
    if (kind == kKindDirect || kind == kKindFull) return;
    stream_piece(p, b, split_row_len(p, b), h->T, piece, h, p.surv + b * kSplitCapacity, (uint32_t)p.capacity);
}

// key >> shift, for the keys in [lo, hi]
template <int kShift>
struct ShiftedRangeView {
    uint32_t lo, hi;
    __device__ bool operator()(uint32_t key, uint32_t, uint32_t& v) const {
        v = key >> kShift;
        return v >= lo && v <= hi;
    }
};

// The members of a cutoff bin, at most 64 survivors whose shifted keys lie in
// [lo_x, hi_x], ranked directly. They are gathered into LDS (`mem`: 64
// entries, then a spare entry per lane; `*mcount` zero on entry) as the
// filter appends survivors: per-lane counts, one reservation per wave,
// writes without branches. Then one wave holds a member per lane and ranks
// each by key, largest first, and position, lowest first, against every
// other (read across lanes); the member of rank need - 1 gives the cutoff
// key and the last position taken at it. When the members share one key,
// that position is found bit by bit from counts over the wave instead. This
// replaces a radix pass over the positions and any ranking of ties in the
// emission.
template <class B, int N, int kShift>
__device__ __forceinline__ Selection rank_members(const RegPairs<N>& sv, uint32_t lo_x, uint32_t hi_x,
                                                  uint32_t need, int idx_bits, uint2* mem, uint32_t* mcount,
                                                  uint2* pick) {
    // lo_x is at least the cutoff's shifted key, above the 0 of an empty slot
    const uint32_t width = hi_x - lo_x;
    auto member = [&](int i, uint32_t& key) {
        key = sv.key[i];
        return (key >> kShift) - lo_x <= width;
    };
    uint32_t cnt = 0u;
    sv.for_each_group([&](int i) {
        uint32_t key;
        cnt += member(i, key) ? 1u : 0u;
    });
    const uint32_t incl = wave_inclusive_sum(cnt);
    const uint32_t total = __builtin_amdgcn_readlane(incl, 63);
    if (total != 0u) {
        uint32_t wbase = 0u;
        if (lane_id() == 0) wbase = atomicAdd(mcount, total);
        uint32_t at = __builtin_amdgcn_readfirstlane(wbase) + incl - cnt;
        const uint32_t spare = (uint32_t)kMaxCand + lane_id();
        sv.for_each_group([&](int i) {
            uint32_t key;
            const bool in = member(i, key);
            mem[(in & (at < (uint32_t)kMaxCand)) ? at : spare] = make_uint2(key, sv.idx[i]);
            at += in ? 1u : 0u;
        });
    }
    B::sync();
    if (B::first_wave()) {
        const uint32_t ne = __builtin_amdgcn_readfirstlane(min(*mcount, (uint32_t)kMaxCand)), lane = lane_id();
        const uint2 me = lane < ne ? mem[lane] : make_uint2(0u, 0xFFFFFFFFu);
        if (lo_x == hi_x) {
            // One key (a shifted key fixes the full one): the need-th lowest
            // position P, built from the top bit down: a bit stays 0 when at
            // least need members lie below the value with it set (the
            // positions below 2^idx_bits; padding lanes hold 0xFFFFFFFF).
            uint32_t at = 0u;
            for (int bit = idx_bits - 1; bit >= 0; --bit) {
                const uint32_t t = at | (1u << bit);
                if ((uint32_t)__builtin_popcountll(__ballot(me.y < t)) < need) at = t;
            }
            if (lane == 0u) *pick = make_uint2(me.x, at);
        } else {
            uint32_t rank = 0u;
            for (uint32_t j = 0; j < ne; ++j) {
                const uint32_t ok = (uint32_t)__builtin_amdgcn_readlane((int)me.x, (int)j);
                const uint32_t op = (uint32_t)__builtin_amdgcn_readlane((int)me.y, (int)j);
                rank += ((ok > me.x) | ((ok == me.x) & (op < me.y))) ? 1u : 0u;
            }
            if ((lane < ne) & (rank == need - 1u)) *pick = me;
        }
    }
    B::sync();
    const uint2 w = *pick;
    return Selection{w.x, (int32_t)w.y};
}

// Exact top m of a row's survivors held in registers by workgroup scope B
// (keys at least T; the short-row and split-finish kernels), ties at the
// cutoff to the lowest positions, as select_top does, with three savings.
// Keys are selected on key >> E::kKeyShift, which drops only bits that carry
// no information (bf16: 16-bit keys). The first pass bins [T, hi] into at
// most 2047 bins of equal width (a power of two), keys above hi in a top bin
// of their own, so the survivors spread over many bins instead of the few
// that their top 11 bits share (bins of width 1 settle the cutoff in that
// pass); hi need not bound every survivor (the sample's largest finite key
// serves), and +inf does not stretch the bins. And a cutoff bin of at most
// 64 survivors is ranked directly (rank_members) instead of by further radix
// passes. `mem` (64 + 64 entries), `mcount` and `pick` are rank_members' LDS.
template <class E, class B, int N>
__device__ __forceinline__ Selection short_select(SelectLds lds, const RegPairs<N>& src, uint32_t m, uint32_t T,
                                                  uint32_t hi_key, int idx_bits, uint2* mem, uint32_t* mcount,
                                                  uint2* pick) {
    constexpr int kShift = E::kKeyShift;
    constexpr uint32_t kTop = 0xFFFFFFFFu >> kShift;
    const uint32_t lo = T >> kShift, hi = max(hi_key >> kShift, lo);
    const int sh = bin_shift(hi - lo);
    const uint32_t base = lo & ~((1u << sh) - 1u);  // (hi - base) >> sh <= kBins - 2
    // The first pass: keys x = key >> kShift up to hi in bins (x - base) >> sh
    // (base aligned to 2^sh, so bin d holds exactly the keys up to hi whose
    // top bits are (base >> sh) + d), keys above hi in the top bin, an empty
    // slot (key 0) in its lane's sink bin.
    const uint32_t sink = (uint32_t)kBins + lane_id();
    src.for_each_group([&](int i) {
        const uint32_t key = src.key[i], x = key >> kShift;
        const uint32_t d = x > hi ? (uint32_t)(kBins - 1) : (x - base) >> sh;
        atomicAdd(&lds.hist[key != 0u ? d : sink], 1u);
    });
    B::sync();
    const Found f1 = find_rank_bin<B, true>(lds, m);
    const Cut c1{f1.digit, m - f1.above, f1.count, false};
    Cut c;
    if (c1.value == (uint32_t)(kBins - 1)) {  // the cutoff is above hi (so hi < kTop)
        if (c1.need == c1.equal) return at_least((hi + 1u) << kShift);
        if (c1.equal <= (uint32_t)kMaxCand)
            return rank_members<B, N, kShift>(src, hi + 1u, kTop, c1.need, idx_bits, mem, mcount, pick);
        c = radix_select_slots<B>(lds, src, ShiftedRangeView<kShift>{hi + 1u, kTop}, c1.need, 0u, 32 - kShift,
                                  c1.equal);
        if (c.range) return at_least(c.value << kShift);
    } else {
        const uint32_t edge = base + (c1.value << sh);  // lowest value in the cutoff bin
        if (c1.need == c1.equal) return at_least(edge << kShift);  // the bin is taken whole
        // the bin's keys share the bits above sh; keys above hi with those
        // bits were counted in the top bin, so they stay out
        const uint32_t bin_hi = min(edge + ((1u << sh) - 1u), hi);
        if (c1.equal <= (uint32_t)kMaxCand)
            return rank_members<B, N, kShift>(src, edge, bin_hi, c1.need, idx_bits, mem, mcount, pick);
        c = Cut{edge, c1.need, c1.equal, false};
        if (sh > 0) {
            c = radix_select_slots<B>(lds, src, ShiftedRangeView<kShift>{edge, hi}, c1.need, edge, sh, c1.equal);
            if (c.range) return at_least(c.value << kShift);  // the least full key whose top bits reach c.value
        }
    }
    const uint32_t kth = E::full_key(c.value);
    if (c.need >= c.equal) return Selection{kth, INT32_MAX};
    if (c.equal <= (uint32_t)kMaxCand)
        return rank_members<B, N, kShift>(src, c.value, c.value, c.need, idx_bits, mem, mcount, pick);
    // the need-th largest inverted index among the ties (select_top's way)
    const uint32_t iprefix = idx_bits >= 32 ? 0u : (0xFFFFFFFFu << idx_bits);
    const Cut t = radix_select_slots<B>(lds, src, TieIndexView{kth}, c.need, iprefix, idx_bits, c.equal);
    return Selection{kth, (int32_t)(~t.value)};
}

// Positions to output values: the identity, or the page-table transform
// page_table[b, i / page_size] * page_size + i % page_size (truncated to
// int32 as the 64-bit value would be), with the row's entries staged in LDS
// for a power-of-two page size, else read from global memory with the
// division done by a multiply. Each takes any position a caller passes
// (the emission clamps unused lanes to 0 first).
struct NoMap {
    __device__ __forceinline__ int32_t operator()(uint32_t i) const { return (int32_t)i; }
};
typedef __attribute__((address_space(1))) const int32_t* GlobalI32;
typedef __attribute__((address_space(3))) const int32_t* LdsI32;
struct LdsShiftMap {
    LdsI32 pages;  // the row's entries, staged in LDS
    uint32_t l;    // page_size = 2^l
    __device__ __forceinline__ int32_t operator()(uint32_t i) const {
        return (int32_t)(((uint32_t)pages[i >> l] << l) | (i & ((1u << l) - 1u)));
    }
};
struct GlobalMagicMap {
    GlobalI32 pages;  // the row's entries in global memory
    uint32_t d, magic;
    int shift;
    __device__ __forceinline__ int32_t operator()(uint32_t i) const {
        const uint32_t q = (uint32_t)(((uint64_t)i * magic) >> shift);
        return (int32_t)((uint32_t)pages[q] * d + (i - q * d));
    }
};

__device__ __forceinline__ GlobalMagicMap global_map(const SplitParams& p, int64_t b) {
    return GlobalMagicMap{(GlobalI32)(p.page_table + b * p.pt_stride), (uint32_t)p.page_size, p.page_magic,
                          p.page_shift};
}

// LDS words the emission works in: the output list (m <= TOPK_MAX_K entries),
// then one spare word per lane.
constexpr int kListWords = TOPK_MAX_K + 64;

// Writes the survivors a Selection takes, from the registers that hold them.
// Each lane counts the entries it takes; a wave prefix sum and the waves'
// totals give every lane its run of places in an LDS list, where the lanes
// write their entries already mapped (an entry not taken goes to the lane's
// spare word, so no write branches); after a barrier the list is copied to
// the output row, coalesced. The work is vector instructions with few scalar
// round trips, so that a lone wave per SIMD is not held up between them.
// wtot holds a word per wave; lst kListWords words. A selection holds
// exactly m entries; the bounds only keep a defect from writing outside the
// row or the list.
template <class B, int N, class Map>
__device__ __forceinline__ void emit_slots(const RegPairs<N>& sv, Selection sel, uint32_t m, int32_t* row,
                                           const Map& map, uint32_t* wtot, uint32_t* lst) {
    constexpr int kWaves = B::kSize / 64;
    const uint32_t w = wave_id(), lane = lane_id();
    // an empty slot holds key 0, below every cutoff key, so it is never taken
    auto take = [&](int i) {
        const uint32_t key = sv.key[i];
        return (key > sel.kth) | ((key == sel.kth) & ((int32_t)sv.idx[i] <= sel.icut));
    };
    uint32_t cnt = 0u;
    sv.for_each_group([&](int i) { cnt += take(i) ? 1u : 0u; });
    const uint32_t incl = wave_inclusive_sum(cnt);
    if (lane == 63u) wtot[w] = incl;
    B::sync();
    uint32_t base = incl - cnt;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) base += (uint32_t)i < w ? wtot[i] : 0u;
    const uint32_t spare = (uint32_t)TOPK_MAX_K + lane;
    sv.for_each_group([&](int i) {
        const bool t = take(i);
        const int32_t o = map(t ? sv.idx[i] : 0u);
        lst[(t & (base < m)) ? base : spare] = (uint32_t)o;
        base += t ? 1u : 0u;
    });
    B::sync();
    constexpr int kPer = (TOPK_MAX_K + B::kSize - 1) / B::kSize;  // list words per thread, all read at once
    uint32_t o[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) o[i] = lst[(uint32_t)(i * B::kSize) + threadIdx.x];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const uint32_t j = (uint32_t)(i * B::kSize) + threadIdx.x;
        if (j < m) store_nt(row + j, (int32_t)o[i]);
    }
}

// launch 3: the exact top m of each row
__global__ __launch_bounds__(kFinThreads) void split_finish_kernel(SplitParams p) {
    using B = BlockScope<kFinThreads>;
    __shared__ __align__(16) uint32_t ews[kListWords];  // the emission's list; first the members a selection ranks
    __shared__ uint32_t mcount;
    __shared__ uint2 pick;
    __shared__ uint32_t hist[kBins + 64];
    __shared__ uint32_t found[3];
    __shared__ uint32_t emitted;
    __shared__ uint32_t wtot[kFinThreads / 64];
    __shared__ uint32_t smax;  // the largest survivor key
    const int64_t b = blockIdx.x;
    const SplitHead head = p.head[b];
    if (head.kind == kKindDirect) return;
    for (int i = (int)threadIdx.x; i < kBins; i += kFinThreads) hist[i] = 0u;
    if (threadIdx.x == 0) {
        emitted = 0u;
        smax = 0u;
        mcount = 0u;
    }
    const int64_t L = split_row_len(p, b);
    const uint32_t m = (uint32_t)(L < p.k ? L : p.k);
    const uint32_t n = head.count;
    const uint32_t cap = (uint32_t)p.capacity;
    const SelectLds lds{hist, found};
    OutRow out = split_out_row(p, b, m, &emitted);
    int code;
    if (head.kind == kKindFull || n > cap || n < m) {
        code = head.kind == kKindFull ? TOPK_ROW_FULL_FORCED : (n > cap ? TOPK_ROW_FULL_OVERFLOW : TOPK_ROW_FULL_UNDERFLOW);
        B::sync();
        const RowSource<B> src{p.scores + b * p.row_stride, L};
        const Selection s = select_top<B>(lds, src, m, (uint32_t)L, 0u, 0xFFFFFFFFu, bits_for(L));
        emit(src, s, out);
    } else {
        code = head.kind == kKindAll ? TOPK_ROW_LDS : TOPK_ROW_SAMPLED;
        // survivors straight into registers, all loads in flight at once
        constexpr int kSlots = (int)(kSplitCapacity / kFinThreads);
        const uint2* g = p.surv + b * kSplitCapacity;
        RegPairs<kSlots> sv;
        sv.nslot = (int)((n + kFinThreads - 1) / kFinThreads);
        sv.for_each_group([&](int i) {  // slots of the groups past nslot are never read
            const uint32_t e = (uint32_t)(i * kFinThreads) + threadIdx.x;
            uint2 v = make_uint2(0xFFFFFFFFu, 0xFFFFFFFFu);  // key 0: the NaN pattern all ones
            if (e < n) v = g[e];
            sv.key[i] = order_key(__uint_as_float(v.x));
            sv.idx[i] = v.y;
        });
        uint32_t hmax = 0u;
        sv.for_each_slot([&](uint32_t key, uint32_t, bool valid) { hmax = max(hmax, valid ? key : 0u); });
        hmax = wave_max(hmax);
        if (lane_id() == 0) atomicMax(&smax, hmax);
        B::sync();
        const Selection s = short_select<F32Elem, B>(lds, sv, m, head.T, smax, bits_for(L),
                                                     reinterpret_cast<uint2*>(ews), &mcount, &pick);
        int32_t* row = p.out + b * (int64_t)p.k;
        if (p.page_table == nullptr)
            emit_slots<B>(sv, s, m, row, NoMap{}, wtot, ews);
        else
            emit_slots<B>(sv, s, m, row, global_map(p, b), wtot, ews);
    }
    if (threadIdx.x == 0) split_stats(p, b, code, head.kind == kKindFull ? (uint32_t)L : n);
}

// ----------------------------------------------------------------------------
// short rows: one workgroup per row, survivors in LDS, one launch
// ----------------------------------------------------------------------------

// Survivor entries a short-row workgroup holds in LDS. Rows of at most
// kShortMaxCols scores with k <= 2048 keep about 2900 survivors at most on
// average (the sample's rank rule), so overflow needs a row far from its
// sample's picture; it then takes the full-row selection.
constexpr int kShortCap = kShortCapacity;

template <class E>
__global__ __launch_bounds__(kThreads, 4) void short_rows_kernel(SplitParams p) {
    constexpr int kU = E::kUnroll;
    constexpr int64_t kR = (int64_t)kThreads * kU;  // loads per workgroup round
    using B = BlockScope<kThreads>;
    typedef typename E::Vec Vec;
    // the survivors, seen as words (sw below): sw[e] is the 32-bit load word
    // that held survivor e, sw[kShortCap + e] its position; later the
    // selection's member list and the emission's output list
    __shared__ uint2 buf[kShortCap + 64];
    __shared__ uint32_t hist[kBins + 64];
    __shared__ uint32_t found[3];
    __shared__ uint32_t count;
    __shared__ uint32_t emitted;
    __shared__ uint32_t wtot[kThreads / 64];
    __shared__ uint32_t mcount;
    __shared__ uint2 pick;
    const int64_t b = blockIdx.x;
    const int64_t L = split_row_len(p, b);
    const uint32_t m = (uint32_t)(L < p.k ? L : p.k);
    if (L <= p.k) {
        const OutRow out = split_out_row(p, b, m, nullptr);
        for (int64_t i = threadIdx.x; i < p.k; i += kThreads) out.row[i] = i < L ? out.map((uint32_t)i) : -1;
        if (threadIdx.x == 0) split_stats(p, b, L == 0 ? TOPK_ROW_EMPTY : TOPK_ROW_ALL, (uint32_t)L);
        return;
    }
    for (int i = (int)threadIdx.x; i < kBins; i += kThreads) hist[i] = 0u;
    if (threadIdx.x == 0) {
        count = 0u;
        emitted = 0u;
        mcount = 0u;
    }
    B::sync();
    const SelectLds lds{hist, found};
    const typename E::Scalar* row = reinterpret_cast<const typename E::Scalar*>(p.scores) + b * p.row_stride;
    // the row's path: the caller may force one (topk_options); otherwise
    // rows up to the capacity keep every score and longer rows are sampled
    const uint32_t cap = (uint32_t)p.capacity;  // 1 .. kShortCap
    if (p.force_path == TOPK_PATH_FULLROW || (p.force_path == TOPK_PATH_LDS && L > (int64_t)cap)) {
        const ElemRowSource<B, E> src{row, L};
        const Selection s = select_top<B>(lds, src, m, (uint32_t)L, 0u, 0xFFFFFFFFu, bits_for(L));
        OutRow out = split_out_row(p, b, m, &emitted);
        emit(src, s, out);
        if (threadIdx.x == 0) split_stats(p, b, TOPK_ROW_FULL_FORCED, (uint32_t)L);
        return;
    }
    const bool keep_all = p.force_path != TOPK_PATH_SAMPLED && L <= (int64_t)cap;

    // One streaming pass, rounds of 16-byte loads, hits to LDS. A sampled
    // row's first round is issued right behind the sample's loads, so that
    // it lands while the cutoff is found.
    const int64_t nvec = L / E::kPerVec;
    // global-address-space pointers, so that the loads stay global loads
    typedef __attribute__((address_space(1))) const Vec* GVec;
    const GVec rv = (GVec)(reinterpret_cast<const Vec*>(row));
    const GVec pad = (GVec)(reinterpret_cast<const Vec*>(g_pad));
    // Every lane loads: a lane past the row's full loads reads the padding,
    // which no score test passes, so the filter needs no bounds. With a fixed
    // number of loads issued after the sample's, the sample can be used once
    // its own loads are in, those still in flight.
    // A round wholly inside the row (uniform) takes one scalar base and
    // the lane's offset for all its loads.
    auto load = [&](int64_t base, Vec (&x)[kU]) {
        if (base + kR <= nvec) {
            typedef __attribute__((address_space(1))) const char* GBytes;
            const GBytes r0 = (GBytes)(rv + base);
#pragma unroll
            for (int u = 0; u < kU; ++u)
                x[u] = __builtin_nontemporal_load((GVec)(r0 + (uint32_t)((u * kThreads + threadIdx.x) * sizeof(Vec))));
        } else {
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int64_t g = base + u * kThreads + threadIdx.x;
                x[u] = __builtin_nontemporal_load(g < nvec ? rv + g : pad);
            }
        }
    };
    Vec xa[kU], xc[kU];
    // the scores past the last full load, [tail0, L): one per lane of the
    // first wave, loaded with the first round (all ones, a NaN pattern that
    // fails the survivor test, on the other lanes)
    const int64_t tail0 = nvec * E::kPerVec;
    typedef __attribute__((address_space(1))) const typename E::Scalar* GScalar;
    uint32_t tbits = 0xFFFFFFFFu;  // the fp32 bits of the lane's tail score
    auto first_loads = [&](bool) {
        load(0, xa);
        if ((int64_t)threadIdx.x < L - tail0) tbits = E::scalar_bits(((GScalar)row)[tail0 + threadIdx.x]);
    };
    static_assert(kShortCap <= kR * E::kPerVec, "one round covers a row that keeps every score");
    Cutoff cut{0u, 0xFFFFFFFFu};  // a row that keeps every score has no sample
    if (keep_all) first_loads(false);
    else if (L <= kShortLong) cut = short_cutoff<E, kShortRuns>(row, L, m, lds, first_loads);
    else cut = short_cutoff<E, kMaxRuns>(row, L, m, lds, first_loads);
    // Raising a cutoff below kMinT changes nothing for non-NaN scores (all
    // pass either way) and lets the padded loads fail the survivor test.
    const uint32_t T = max(cut.T, kMinT);
    const bool pos = T >= 0x80000000u;  // at or above the key of +0
    const SurvivorBound sb = E::bound(T, pos);
    // The second round goes out once the cutoff is known (bf16: 16 KB rounds)
    // or once the first round has been filtered (fp32: 32 KB rounds), not
    // with the first: in a full batch every workgroup's first round then
    // reaches the memory queues ahead of every second round, so that the
    // workgroups launched last (whose loads queue behind the others') start
    // filtering sooner. Measured on 1024 rows of 16384: bf16 21.7 -> 21.0 us,
    // fp32 block keys 18.7 -> 17.5 us; on 256 rows within 0.3 us.
    if (E::kSecondAtCutoff && kR < nvec) load(kR, xc);

    // One round: each lane counts its survivors, one LDS reservation per wave
    // places them (a wave that would pass the capacity writes nothing; the
    // count still grows, so the row then takes the full-row selection), and
    // each lane writes its survivors to consecutive slots, only the lanes
    // whose score passes taking part in a write.
    uint32_t* const sw = reinterpret_cast<uint32_t*>(buf);
    auto filter = [&](auto pos_tag, const Vec (&x)[kU], int64_t base) {
        constexpr bool kPos = decltype(pos_tag)::value;
        uint32_t cnt = 0u;
#pragma unroll
        for (int u = 0; u < kU; ++u) {
#pragma unroll
            for (int j = 0; j < E::kPerVec; ++j) cnt += E::template pass<kPos>(x[u], j, sb) ? 1u : 0u;
        }
        const uint32_t incl = wave_inclusive_sum(cnt);
        const uint32_t total = __builtin_amdgcn_readlane(incl, 63);
        if (total == 0u) return;
        uint32_t wbase = 0u;
        if (lane_id() == 0) wbase = atomicAdd(&count, total);
        wbase = __builtin_amdgcn_readfirstlane(wbase);
        if (wbase + total > cap) return;
        // byte offset of the lane's next slot in the word array (positions
        // lie kShortCap words further on)
        uint32_t slot = (wbase + incl - cnt) * (uint32_t)sizeof(uint32_t);
        char* const bytes = reinterpret_cast<char*>(sw);
        const uint32_t p0 = (uint32_t)(E::kPerVec * (base + threadIdx.x));
        // The tests run again here rather than keep 32 results per lane live
        // across the reservation: the bounds are taken through wbase >> 31,
        // always 0 (counts stay below 2^31) but not known to the compiler.
        const uint32_t z = wbase >> 31;
        const SurvivorBound sb2{sb.t ^ z, sb.th ^ z};
#pragma unroll
        for (int u = 0; u < kU; ++u) {
#pragma unroll
            for (int j = 0; j < E::kPerVec; ++j) {
                // some lane of the wave nearly always passes: the hint keeps
                // the compiler from branching around each write
                if (__builtin_expect(E::template pass<kPos>(x[u], j, sb2), 1)) {
                    *reinterpret_cast<uint32_t*>(bytes + slot) = E::word(x[u], j);
                    *reinterpret_cast<uint32_t*>(bytes + slot + kShortCap * sizeof(uint32_t)) =
                        p0 + (uint32_t)(E::kPerVec * kThreads * u + j);
                    slot += (uint32_t)sizeof(uint32_t);
                }
            }
        }
    };
    // The first round is in flight since the sample, the second since the
    // cutoff (bf16) or from just after the first is filtered (fp32); a third
    // is loaded into the first buffer as soon as that has been filtered. Rows
    // past three rounds go on one round at a time.
    auto stream = [&](auto pos_tag) {
        filter(pos_tag, xa, 0);
        if (kR >= nvec) return;
        if (!E::kSecondAtCutoff) load(kR, xc);
        if (2 * kR < nvec) load(2 * kR, xa);
        filter(pos_tag, xc, kR);
        for (int64_t base = 2 * kR; base < nvec; base += kR) {  // uniform over the workgroup
            if (base > 2 * kR) load(base, xa);
            filter(pos_tag, xa, base);
        }
    };
    if (pos) stream(std::true_type{});
    else stream(std::false_type{});
    if (tail0 < L && wave_id() == 0) {
        const bool hit = pos ? (int32_t)tbits >= (int32_t)sb.t : tbits <= sb.t;  // exact widened bits
        const uint32_t slot = wave_reserve_count(&count, hit ? 1u : 0u);
        if (hit && slot < cap) {
            const uint32_t i = (uint32_t)(tail0 + threadIdx.x);
            sw[slot] = E::bits_word(tbits, i);
            sw[kShortCap + slot] = i;
        }
    }
    B::sync();
    const uint32_t n = count;
    OutRow out = split_out_row(p, b, m, &emitted);
    int code;
    if (n > cap || n < m) {
        code = n > cap ? TOPK_ROW_FULL_OVERFLOW : TOPK_ROW_FULL_UNDERFLOW;
        const ElemRowSource<B, E> src{row, L};
        const Selection s = select_top<B>(lds, src, m, (uint32_t)L, 0u, 0xFFFFFFFFu, bits_for(L));
        emit(src, s, out);
    } else {
        code = keep_all ? TOPK_ROW_LDS : TOPK_ROW_SAMPLED;
        // A paged row's page-table entries, when they fit the histogram, are
        // loaded now (their latency hidden by the selection) and staged there
        // once the selection is done with it.
        constexpr int kPg = kBins / kThreads;
        const int32_t* pages = p.page_table ? p.page_table + b * p.pt_stride : nullptr;
        const bool pow2 = (p.page_size & (p.page_size - 1)) == 0;
        const uint32_t npg = pages ? (uint32_t)((((uint64_t)(L - 1) * p.page_magic) >> p.page_shift) + 1u) : 0u;
        const bool stage = pow2 && npg != 0u && npg <= (uint32_t)kBins;
        int32_t pg[kPg];
        if (stage) {
#pragma unroll
            for (int i = 0; i < kPg; ++i) {
                if ((uint32_t)(i * kThreads) < npg) {  // uniform
                    const uint32_t t = (uint32_t)(i * kThreads) + threadIdx.x;
                    if (t < npg) pg[i] = pages[t];
                }
            }
        }
        // the survivors into registers, every read in flight at once (the LDS
        // buffer then holds the tie regions; the selection's first barrier
        // orders the two uses)
        constexpr int kSlots = (kShortCap + kThreads - 1) / kThreads;
        static_assert(kSlots * kThreads <= kShortCap, "every slot reads inside the word array");
        RegPairs<kSlots> sv;
        sv.nslot = (int)((n + kThreads - 1) / kThreads);
        sv.for_each_group([&](int i) {  // slots of the groups past nslot are never read
            const uint32_t e = (uint32_t)(i * kThreads) + threadIdx.x;
            const uint32_t w = sw[e], at = sw[kShortCap + e];
            sv.key[i] = e < n ? order_key(__uint_as_float(E::word_bits(w, at))) : 0u;
            sv.idx[i] = e < n ? at : 0xFFFFFFFFu;
        });
        const Selection s = short_select<E, B>(lds, sv, m, T, cut.hi, bits_for(L), buf, &mcount, &pick);
        if (stage) {  // the selection has left the histogram (the emission syncs before reading)
#pragma unroll
            for (int i = 0; i < kPg; ++i) {
                if ((uint32_t)(i * kThreads) < npg) {  // uniform
                    const uint32_t t = (uint32_t)(i * kThreads) + threadIdx.x;
                    if (t < npg) reinterpret_cast<int32_t*>(hist)[t] = pg[i];
                }
            }
        }
        int32_t* row = p.out + b * (int64_t)p.k;
        uint32_t* lst = reinterpret_cast<uint32_t*>(buf);
        static_assert(kListWords <= 2 * (kShortCap + 64), "the emission's list fits the buffer");
        if (pages == nullptr)
            emit_slots<B>(sv, s, m, row, NoMap{}, wtot, lst);
        else if (stage)
            emit_slots<B>(sv, s, m, row,
                          LdsShiftMap{(LdsI32)reinterpret_cast<const int32_t*>(hist),
                                      (uint32_t)(31 - __clz(p.page_size))},
                          wtot, lst);
        else
            emit_slots<B>(sv, s, m, row, global_map(p, b), wtot, lst);
    }
    if (threadIdx.x == 0) split_stats(p, b, code, n);
}

}  // namespace

template <class E>
int launch_short(const void* scores, int64_t batch, int64_t row_stride, int64_t n_cols, const int32_t* lengths,
                 int32_t k, int32_t* out_idx, const int32_t* page_table, int64_t page_table_stride,
                 int32_t page_size, const topk_options& opt, hipStream_t stream) {
    if (batch * kThreads > (int64_t)UINT32_MAX) return TOPK_ERR_ARG;
    const int32_t cap = opt.capacity == 0 ? kShortCap : opt.capacity;
    if (cap < 1 || cap > kShortCap) return TOPK_ERR_ARG;
    SplitParams p{static_cast<const float*>(scores), row_stride, n_cols, lengths, out_idx, page_table,
                  page_table_stride, page_size, k, opt.force_path, cap, opt.row_stats, batch, nullptr, nullptr, 0, 1,
                  0u, 0};
    page_divider(page_table != nullptr ? page_size : 1, p.page_magic, p.page_shift);
    void* args[] = {&p};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&short_rows_kernel<E>), dim3((uint32_t)batch),
                                         dim3(kThreads), args, 0, stream);
    return e == hipSuccess ? TOPK_OK : TOPK_ERR_LAUNCH;
}

int launch_short_rows(const float* scores, int64_t batch, int64_t row_stride, int64_t n_cols,
                      const int32_t* lengths, int32_t k, int32_t* out_idx, const int32_t* page_table,
                      int64_t page_table_stride, int32_t page_size, const topk_options& opt, hipStream_t stream) {
    return launch_short<F32Elem>(scores, batch, row_stride, n_cols, lengths, k, out_idx, page_table,
                                 page_table_stride, page_size, opt, stream);
}

int launch_short_rows_bf16(const uint16_t* scores, int64_t batch, int64_t row_stride, int64_t n_cols,
                           const int32_t* lengths, int32_t k, int32_t* out_idx, const int32_t* page_table,
                           int64_t page_table_stride, int32_t page_size, const topk_options& opt,
                           hipStream_t stream) {
    return launch_short<Bf16Elem>(scores, batch, row_stride, n_cols, lengths, k, out_idx, page_table,
                                  page_table_stride, page_size, opt, stream);
}

// The workspace of topk_select_split_noalloc: a fixed device array, one copy
// per GPU, held until the process ends. Host code never names it except to
// ask for its device address (the name is only a host-side stand-in).
constexpr int64_t kNoAllocBytes = split_workspace_bytes(TOPK_SPLIT_NOALLOC_MAX_BATCH);
static_assert(kNoAllocBytes % 256 == 0, "whole 256-byte lines");
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

// Device address of `scratch` on the current device, looked up once per
// device with that device current; TOPK_ERR_DEVICE if no gfx950 device is
// current or the lookup fails.
int scratch_address(void** ptr) {
    constexpr int kMaxDevices = 64;
    static std::once_flag once[kMaxDevices];
    static void* addr[kMaxDevices];
    static hipError_t rc[kMaxDevices];
    int dev = -1;
    if (device_cus() <= 0 || hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return TOPK_ERR_DEVICE;
    std::call_once(once[dev], [dev] {
        void* p = nullptr;
        rc[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        addr[dev] = p;
    });
    if (rc[dev] != hipSuccess || addr[dev] == nullptr) return TOPK_ERR_DEVICE;
    *ptr = addr[dev];
    return TOPK_OK;
}

// topk_select_split's checks and launches; with use_scratch, the workspace
// is the library's scratch array, looked up once every argument has passed.
inline bool options_default_capacity(const topk_options* o) { return o == nullptr || o->capacity == 0; }

int split_select(const float* scores, int64_t batch, int64_t row_stride, int64_t n_cols, const int32_t* lengths,
                 int32_t k, int32_t* out_idx, const int32_t* page_table, int64_t page_table_stride,
                 int32_t page_size, void* workspace, int64_t workspace_bytes, int32_t pieces, void* hip_stream,
                 const topk_options* options, bool use_scratch) {
    if (batch < 0 || batch > (use_scratch ? TOPK_SPLIT_NOALLOC_MAX_BATCH : INT32_MAX)) return TOPK_ERR_ARG;
    if (k < 1 || k > TOPK_MAX_K) return TOPK_ERR_K;
    if (n_cols < 0 || n_cols > INT32_MAX || row_stride < n_cols) return TOPK_ERR_ARG;
    if (pieces < 0 || pieces > kMaxPieces) return TOPK_ERR_ARG;
    topk_options opt{TOPK_PATH_AUTO, 0, nullptr, TOPK_KERNEL_AUTO};
    if (options != nullptr) opt = *options;
    if (opt.force_path < TOPK_PATH_AUTO || opt.force_path > TOPK_PATH_FULLROW) return TOPK_ERR_ARG;
    if (opt.capacity < 0 || opt.capacity > kSplitCapacity) return TOPK_ERR_ARG;
    if (opt.kernel != TOPK_KERNEL_AUTO) return TOPK_ERR_ARG;  // the split kernels only
    if (opt.capacity == 0) opt.capacity = (int32_t)kSplitCapacity;
    if (page_table != nullptr) {
        if (page_size < 1) return TOPK_ERR_ARG;
        if (page_table_stride < (n_cols + page_size - 1) / page_size) return TOPK_ERR_ARG;
    }
    if (batch == 0) return TOPK_OK;
    if (scores == nullptr || out_idx == nullptr || (!use_scratch && workspace == nullptr)) return TOPK_ERR_ARG;
    if (!use_scratch && workspace_bytes < split_workspace_bytes(batch)) return TOPK_ERR_ARG;
    if ((reinterpret_cast<uintptr_t>(scores) & 15u) != 0) return TOPK_ERR_ALIGN;
    if (!use_scratch && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return TOPK_ERR_ALIGN;
    if (batch > 1 && (row_stride & 3) != 0) return TOPK_ERR_ALIGN;
    // pieces per row: enough workgroups for about four per compute unit, each
    // piece a whole number of load rounds. A batch that already brings four
    // rows per compute unit gets one piece per row, and then one workgroup
    // per row in a single launch (topk_select's kernels) does the same work
    // without the survivors' round trip through the workspace, which is left
    // untouched (only with the default capacity, whose bound both paths
    // accept).
    int64_t want = pieces;
    if (want == 0) {
        const int cus = device_cus();
        if (cus <= 0) return TOPK_ERR_DEVICE;
        if (!use_scratch && options_default_capacity(options) && batch >= 4 * (int64_t)cus)
            return topk_select_ex(scores, batch, row_stride, n_cols, lengths, k, out_idx, page_table,
                                  page_table_stride, page_size, hip_stream, options);
        want = (4 * (int64_t)cus + batch - 1) / batch;
    }
    const int64_t nvec_max = (n_cols + 3) / 4;
    if (want > kMaxPieces) want = kMaxPieces;
    if (want < 1) want = 1;
    int64_t per = (nvec_max + want - 1) / want;
    per = (per + kRound - 1) / kRound * kRound;
    if (per < kRound) per = kRound;
    const int64_t P = nvec_max > 0 ? (nvec_max + per - 1) / per : 1;
    if (batch * P * kThreads > (int64_t)UINT32_MAX) return TOPK_ERR_ARG;
    if (device_cus() <= 0) return TOPK_ERR_DEVICE;
    if (use_scratch) {
        const int st = scratch_address(&workspace);
        if (st != TOPK_OK) return st;
    }

    char* ws = static_cast<char*>(workspace);
    SplitParams p{scores, row_stride, n_cols, lengths, out_idx, page_table, page_table_stride, page_size, k,
                  opt.force_path, opt.capacity, opt.row_stats, batch,
                  reinterpret_cast<SplitHead*>(ws), reinterpret_cast<uint2*>(ws + head_bytes(batch)),
                  per, (int32_t)P, 0u, 0};
    page_divider(page_table != nullptr ? page_size : 1, p.page_magic, p.page_shift);
    void* args[] = {&p};
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    if (hipLaunchKernel(reinterpret_cast<const void*>(&split_sample_kernel), dim3((uint32_t)batch), dim3(kThreads),
                        args, 0, st) != hipSuccess)
        return TOPK_ERR_LAUNCH;
    if (hipLaunchKernel(reinterpret_cast<const void*>(&split_stream_kernel), dim3((uint32_t)(batch * P)),
                        dim3(kThreads), args, 0, st) != hipSuccess)
        return TOPK_ERR_LAUNCH;
    if (hipLaunchKernel(reinterpret_cast<const void*>(&split_finish_kernel), dim3((uint32_t)batch),
                        dim3(kFinThreads), args, 0, st) != hipSuccess)
        return TOPK_ERR_LAUNCH;
    return TOPK_OK;
}

}  // namespace topk

using namespace topk;

extern "C" {

int64_t topk_split_workspace_bytes(int64_t batch) {
    if (batch < 0 || batch > INT32_MAX) return -1;
    return split_workspace_bytes(batch);
}

int32_t topk_split_capacity(void) { return (int32_t)kSplitCapacity; }

int topk_select_split(const float* scores, int64_t batch, int64_t row_stride, int64_t n_cols,
                      const int32_t* lengths, int32_t k, int32_t* out_idx,
                      const int32_t* page_table, int64_t page_table_stride, int32_t page_size,
                      void* workspace, int64_t workspace_bytes, int32_t pieces, void* hip_stream,
                      const topk_options* options) {
    return split_select(scores, batch, row_stride, n_cols, lengths, k, out_idx, page_table, page_table_stride,
                        page_size, workspace, workspace_bytes, pieces, hip_stream, options, false);
}

int topk_select_split_noalloc(const float* scores, int64_t batch, int64_t row_stride, int64_t n_cols,
                              const int32_t* lengths, int32_t k, int32_t* out_idx, const int32_t* page_table,
                              int64_t page_table_stride, int32_t page_size, int32_t pieces, void* hip_stream,
                              const topk_options* options) {
    return split_select(scores, batch, row_stride, n_cols, lengths, k, out_idx, page_table, page_table_stride,
                        page_size, nullptr, 0, pieces, hip_stream, options, true);
}

}  // extern "C"
