// Exact per-row top-k over long, ragged fp32 rows, for gfx950 (CDNA4).
//
// One persistent launch: one 12-wave workgroup per compute unit, each with
// two LDS survivor buffers. A workgroup's rows are dealt to it in a fixed
// order (longest first over the whole batch, dealt out in a snake, so every
// workgroup gets about the same number of scores) and flow through three
// roles that hand rows on through LDS progress counters, with no workgroup
// barrier between rows:
//
//  * wave 1 claims rows and estimates each one's cutoff key T from a sample
//    of the row (vLLM PR #56346 report, summary and implementation item 1: a
//    sampled cutoff, then exact selection among the survivors);
//  * waves 2-11 read each row once, in chunks handed out one at a time, with
//    16-byte buffer loads kept in flight across row boundaries, and append
//    every score with key >= T to the row's buffer with one LDS atomic per
//    wave and 4 loads, counting on past the capacity without writing (vLLM
//    PR #56346 report, implementation item 1: ballot hit masks, in-wave
//    prefix sums, one reservation per wave);
//  * wave 0 finishes each row once every streaming wave has left it: it
//    bins the survivors upward from T, writes out every survivor above the
//    bin holding the k-th largest and ranks the few in that bin exactly.
//
// Rows whose survivors overflow the buffer or fall short of k (and rows
// forced to it) take the full-row path when the queue is done:
// histogram-only radix passes over the row down to the exact cutoff, then
// one scan that writes the values above it and the cutoff ties ("Fix
// incorrect sparse-attention top-k selection when candidate bins overflow",
// comment thread: cutoff-first fallback; vLLM PR #56346 report,
// implementation items 1-2: the dual fallback). Rows with L <= k are written
// out directly.
//
// Every path selects the same set: all positions with key above the cutoff
// key K*, plus the lowest-index positions equal to K* until m are taken.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "exact_topk.h"
#include "topk_device.h"
#include "topk_short.h"

namespace topk {
namespace {

#ifndef TOPK_WAVES
#define TOPK_WAVES 12
#endif
constexpr int kThreads = 64 * TOPK_WAVES;                  // finisher, sampler, streamers
constexpr int kFirstStreamer = 2;                          // waves 2..11 stream
constexpr int kCapacity = 7168;                            // survivor entries per buffer
#ifndef TOPK_UNROLL
#define TOPK_UNROLL 8
#endif
constexpr int kUnroll = TOPK_UNROLL;                       // 16-byte loads per lane per chunk
constexpr int kPart = 4;                                   // loads filtered per LDS reservation
constexpr int kChunkVec = 64 * kUnroll;                    // float4 groups per chunk
constexpr int kRunLen = 64;                                // floats per contiguous sample run
constexpr int kMaxRuns = 64;                               // runs per sample
constexpr int kMaxSample = kMaxRuns * kRunLen;             // 4096 keys at most
constexpr int kFineShift = 14;                             // T to within 2^14 keys (1/512 octave)
constexpr int kPairFineShift = 16;                         // row 0's T: to within 2^16 keys (1/128 octave)
constexpr int kSlots = 4;                                  // rows i-1 .. i+2
constexpr int kTable = 64;                                 // queued rows fetched at a time
constexpr int kMaxDeferred = 64;                           // full-row rows per workgroup
constexpr int kOrderMaxRows = 2048;                        // longest-first order up to this batch

constexpr uint32_t kKindSampled = 0, kKindAll = 1, kKindFull = 2;
constexpr uint64_t kWatchdogTicks = 10ull * 100000000ull;  // 10 s

__device__ unsigned int g_watchdog_trips;  // workgroups that gave up a wait, since load

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
    int64_t batch;
};

struct RowSlot {
    int64_t b;
    int64_t L;
    int64_t nvec;
    uint32_t m;
    uint32_t T;
    uint32_t sh;
    uint32_t kind;
    uint32_t valid;
    uint32_t nsv;  // 4-score groups in the row's sample, when sampled
};

struct Shared {
    uint2 surv[2][kCapacity];   // survivors: (raw score bits, position)
    uint32_t hist[2][kBins];    // survivor histograms, all zero outside a row's use
    uint32_t skey[kMaxSample];  // the sampler's keys
    uint32_t shist[kBins];      // the sampler's histogram
    RowSlot slot[kSlots];
    uint32_t chunk_next[kSlots];  // next chunk of each slot's row to hand out
    uint32_t left[kSlots];        // streaming waves done with each slot's row
    uint32_t n_claimed;           // rows claimed into their slots
    uint32_t n_ready;             // rows whose cutoff is set
    uint32_t n_finished;          // rows finished
    int32_t last_row;             // the row finished by the whole workgroup, or -1
    uint32_t abort;               // a wait timed out: every role stops
    uint32_t count[2];            // survivors appended per buffer
    uint32_t vmax[2];             // largest survivor key per buffer
    uint32_t found[3];            // finisher's and whole-workgroup selections
    uint32_t sfound[3];           // sampler's selections
    uint32_t emitted;             // output slots, finisher and whole workgroup
    uint32_t semitted;            // output slots, sampler
    uint32_t ncand;
    alignas(16) uint32_t cand_key[kMaxCand];
    alignas(16) uint32_t cand_idx[kMaxCand];
    uint32_t pair;       // row 0's cutoff by waves 0 and 1: bounds posted, then halves counted
    uint32_t take_cand;  // the last row's slots: taken (low 16 bits) and candidates (high 16)
    uint32_t ndeferred;
    int32_t deferred[kMaxDeferred];
    int32_t deferred_code[kMaxDeferred];
    int32_t tab_b[kTable];
    int32_t tab_len[kTable];
    uint32_t nrank;  // workgroups whose first row is lighter than this one's
    uint32_t ndirect;
    uint32_t tab_n;
    uint32_t tab_pos;
    uint32_t tab_round;
    uint32_t nqueue;   // rows in the order
    uint32_t ordered;  // the order is longest first, fully tabled at start
};

__device__ __forceinline__ int64_t row_len(const Params& p, int64_t b) {
    int64_t L = p.lengths ? (int64_t)p.lengths[b] : p.n_cols;
    return L < 0 ? 0 : (L > p.n_cols ? p.n_cols : L);
}

__device__ __forceinline__ OutRow out_row(const Params& p, int64_t b, uint32_t m, uint32_t* emitted) {
    return OutRow{p.out + b * (int64_t)p.k, p.page_table ? p.page_table + b * p.pt_stride : nullptr,
                  p.page_size, m, emitted};
}

__device__ __forceinline__ void put_stats(const Params& p, int64_t b, int code, uint32_t seen) {
    if (p.row_stats != nullptr) {
        p.row_stats[2 * b + 0] = code;
        p.row_stats[2 * b + 1] = (int32_t)seen;
    }
}

// Position of this workgroup's j-th row in the queue: the order dealt out in
// a snake (workgroup w takes w, 2G-1-w, 2G+w, ...), pairing long rows with
// short ones.
__device__ __forceinline__ uint32_t snake(uint32_t j) {
    const uint32_t G = gridDim.x;
    return j * G + ((j & 1u) ? G - 1u - blockIdx.x : blockIdx.x);
}

__device__ __forceinline__ uint32_t length_bucket(int64_t L, int64_t n_cols) {
    return (uint32_t)(L * (kBins - 1) / (n_cols > 0 ? n_cols : 1));
}

// ----------------------------------------------------------------------------
// rows selected without a survivor buffer
// ----------------------------------------------------------------------------

// L <= k: every position, then -1 (an idle row gets only -1). Scope S.
template <class S>
__device__ __forceinline__ void direct_row(const Params& p, int64_t b, int64_t L) {
    const OutRow out = out_row(p, b, (uint32_t)L, nullptr);
    for (int64_t i = S::rank(); i < p.k; i += S::kSize) out.row[i] = i < L ? out.map((uint32_t)i) : -1;
    if (S::rank() == 0) put_stats(p, b, L == 0 ? TOPK_ROW_EMPTY : TOPK_ROW_ALL, (uint32_t)L);
}

// Full-row exact selection of row b by scope S with `hist` all zero.
template <class S>
__device__ __forceinline__ void full_row(const Params& p, SelectLds lds, uint32_t* emitted, int64_t b, int code) {
    const int64_t L = row_len(p, b);
    const uint32_t m = (uint32_t)(L < p.k ? L : p.k);
    if (S::rank() == 0) *emitted = 0u;
    S::sync();
    const RowSource<S> src{p.scores + b * p.row_stride, L};
    const Selection s = select_top<S>(lds, src, m, (uint32_t)L, 0u, 0xFFFFFFFFu, bits_for(L));
    // slots from the LDS counter: the row's loops leave lanes idle at their
    // ends, so a per-lane counter would fall out of step
    OutRow out = out_row(p, b, m, emitted);
    emit(src, s, out);
    S::sync();
    if (S::rank() == 0) {
        put_stats(p, b, code, (uint32_t)L);
        *emitted = 0u;
    }
    S::sync();
}

// One wave: remember row b for the workgroup's full-row pass; with the list
// full, select it here with this wave alone, in its own LDS state.
__device__ __forceinline__ void defer_row(const Params& p, Shared& sm, SelectLds own, uint32_t* own_emitted, int64_t b,
                          int code) {
    uint32_t n = 0u;
    if (lane_id() == 0) n = atomicAdd(&sm.ndeferred, 1u);
    n = __builtin_amdgcn_readfirstlane(n);
    if (n < (uint32_t)kMaxDeferred) {
        if (lane_id() == 0) {
            sm.deferred[n] = (int32_t)b;
            sm.deferred_code[n] = code;
        }
        WaveScope::sync();
    } else {
        full_row<WaveScope>(p, own, own_emitted, b, code);
    }
}

// ----------------------------------------------------------------------------
// the queue
// ----------------------------------------------------------------------------

// The queue is ordered longest first when the batch has at most this many
// rows and every workgroup's share fits one table; thread t then holds the
// lengths of rows t, t + kThreads, ... (kLenPer of them), loaded at start.
__device__ __forceinline__ bool queue_ordered(int64_t batch) {
    return batch <= kOrderMaxRows && batch <= (int64_t)kTable * gridDim.x;
}
constexpr int kLenPer = (kOrderMaxRows + kThreads - 1) / kThreads;

// Where in LDS the ordered queue is made: survivor buffer 1 and its
// histogram, both free until row 1 is claimed, so that the sampler wave can
// make the table while row 0 streams into buffer 0.
struct QueueLds {
    uint32_t* bucket;  // per row: its length bucket; kBins for L <= k or a first row
    int32_t* len;      // per row: its clamped length
    uint32_t* direct;  // this workgroup's rows with L <= k (at most kTable)
    uint32_t* cnt;     // per length bucket: queued rows in it (zero on entry and on exit)
};
static_assert(2 * kCapacity >= 2 * kOrderMaxRows + kTable, "the queue fits one survivor buffer");

__device__ __forceinline__ QueueLds queue_lds(Shared& sm) {
    uint32_t* b1 = reinterpret_cast<uint32_t*>(sm.surv[1]);
    return QueueLds{b1, reinterpret_cast<int32_t*>(b1 + kOrderMaxRows), b1 + 2 * kOrderMaxRows, sm.hist[1]};
}

// The ordered queue: the rows past the first G, longest first (by 2048
// length buckets, ties by row index, the same order in every workgroup);
// workgroup w takes positions q, G + q, 2G + q, ... of it, q being the rank
// of its first row among the first rows, shortest first: the lightest first
// row goes with the longest row of every round, so the totals even out.
// Rows with L <= k (dealt round-robin, row w among them) are written out
// directly.
//
// Two parts. The count, by the whole workgroup from the lengths its threads
// loaded at start: each row's length and bucket, the bucket counts, the
// direct rows and q.
__device__ __forceinline__ void queue_count(const Params& p, Shared& sm, const QueueLds& q, int64_t L0,
                                            const int64_t (&lens)[kLenPer]) {
    const uint32_t n = (uint32_t)p.batch;
    const uint32_t G = gridDim.x;
    static_assert(kThreads >= 256, "the first rows (one per compute unit) sit in every thread's first length");
    {
        // this workgroup's rank among the first rows: those with a lighter
        // load (L if L > k, else 0), ties by workgroup index
        const int64_t mine = L0 > p.k ? L0 : 0;
        const int64_t theirs = lens[0] > p.k ? lens[0] : 0;
        const bool lighter = threadIdx.x < G && (theirs < mine || (theirs == mine && threadIdx.x < blockIdx.x));
        const uint64_t lm = __ballot(lighter);
        if (lane_id() == 0 && lm != 0) atomicAdd(&sm.nrank, (uint32_t)__popcll(lm));
    }
#pragma unroll
    for (int j = 0; j < kLenPer; ++j) {
        const uint32_t b = threadIdx.x + (uint32_t)j * kThreads;
        if (b >= n) break;
        const int64_t L = lens[j];
        q.len[b] = (int32_t)L;
        uint32_t d = (uint32_t)kBins;
        if (L > p.k) {
            if (b >= G) {  // the first rows are not queued
                d = length_bucket(L, p.n_cols);
                atomicAdd(&q.cnt[d], 1u);
            }
        } else if (b % G == blockIdx.x) {
            q.direct[atomicAdd(&sm.ndirect, 1u)] = b;
        }
        q.bucket[b] = d;
    }
}

// The table, by one wave from the count in LDS (no memory loads: while rows
// stream, a load waits behind the streaming waves' loads). No sort: each
// position t is found by rank, its bucket from running sums of the bucket
// counts (higher buckets first), then its row as the one of rank
// t - (rows in higher buckets) among the bucket's rows, by index, from a
// running count over the rows. `first(b, L)` is called on the first
// position's row as soon as it is known. Then the direct rows. Leaves the
// counts zero.
template <class First>
__device__ __forceinline__ void queue_table(const Params& p, Shared& sm, const QueueLds& q, First&& first) {
    static_assert(kBins == 64 * 32, "32 buckets per lane");
    const uint32_t lane = lane_id();
    const uint32_t n = (uint32_t)p.batch;
    const uint32_t G = gridDim.x;
    const uint32_t ns = (n + 63u) / 64u;  // rows in strides of 64
    // lane l sums buckets 32l .. 32l + 31; higher buckets come first
    uint32_t own = 0;
    {
        const uint4* c4 = reinterpret_cast<const uint4*>(q.cnt + 32 * lane);
        uint4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = c4[j];
#pragma unroll
        for (int j = 0; j < 8; ++j) own += v[j].x + v[j].y + v[j].z + v[j].w;
    }
    const uint32_t incl = wave_inclusive_sum(own);
    const uint32_t total = __builtin_amdgcn_readlane(incl, 63);
    const uint32_t above = total - incl;  // queued rows in higher lanes' buckets
    const uint32_t q0 = sm.nrank;
    uint32_t nt = 0;
    for (uint32_t e = 0; e < (uint32_t)kTable; ++e) {
        const uint32_t t = e * G + q0;
        if (t >= total) break;
        // the lane whose buckets hold position t, then the bucket: lanes
        // j < 32 take that lane's buckets, the highest first
        const int ol = __ffsll((unsigned long long)__ballot(above <= t && t < above + own)) - 1;
        const uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)above, ol);
        const uint32_t cj = lane < 32u ? q.cnt[32u * (uint32_t)ol + 31u - lane] : 0u;
        const uint32_t ci = wave_inclusive_sum(cj);
        const int jl = __ffsll((unsigned long long)__ballot(lane < 32u && base + ci - cj <= t && t < base + ci)) - 1;
        const uint32_t d = 32u * (uint32_t)ol + 31u - (uint32_t)jl;
        uint32_t r = t - base - (uint32_t)__builtin_amdgcn_readlane((int)(ci - cj), jl);
        // the row of rank r among the bucket's rows, by index: 64 rows at a
        // time, four strides' reads issued together
        uint32_t row = 0;
        bool found = false;
        for (uint32_t j0 = 0; j0 < ns && !found; j0 += 4u) {
            uint32_t bv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t b = (j0 + (uint32_t)u) * 64u + lane;
                bv[u] = b < n ? q.bucket[b] : (uint32_t)kBins;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint64_t m = __ballot(bv[u] == d);
                const uint32_t pc = (uint32_t)__popcll(m);
                if (!found && r < pc) {
                    const int rl = __ffsll((unsigned long long)__ballot(bv[u] == d && lanes_below(m) == r)) - 1;
                    row = (j0 + (uint32_t)u) * 64u + (uint32_t)rl;
                    found = true;
                } else if (!found) {
                    r -= pc;
                }
            }
        }
        const int32_t len = __builtin_amdgcn_readfirstlane(q.len[row]);
        if (lane == 0) {
            sm.tab_b[e] = (int32_t)row;
            sm.tab_len[e] = len;
        }
        if (e == 0) first((int64_t)row, (int64_t)len);
        nt = e + 1u;
    }
    uint4* z4 = reinterpret_cast<uint4*>(q.cnt + 32 * lane);
#pragma unroll
    for (int j = 0; j < 8; ++j) z4[j] = make_uint4(0u, 0u, 0u, 0u);
    if (lane == 0) {
        sm.ordered = 1u;
        sm.nqueue = total;
        sm.tab_n = nt;
        sm.tab_pos = 0u;
        sm.tab_round = 0u;
    }
    WaveScope::sync();
    const uint32_t nd = sm.ndirect;
    for (uint32_t j = 0; j < nd; ++j) {
        const uint32_t b = q.direct[j];
        direct_row<WaveScope>(p, b, q.len[b]);
    }
    WaveScope::sync();
}

// Whole workgroup, at start, for a queue that is not ordered: with no more
// rows than workgroups there is nothing to queue (workgroup w takes row w);
// larger batches than one table per workgroup holds are dealt in index
// order, a table at a time.
__device__ __forceinline__ void build_queue(const Params& p, Shared& sm, int64_t L0) {
    using B = BlockScope<kThreads>;
    const int64_t batch = p.batch;
    const uint32_t G = gridDim.x;
    if (batch <= (int64_t)G) {
        // no more rows than workgroups (the grid is min(batch, CUs)):
        // workgroup w takes row w alone, so there is no order to compute
        if (L0 <= p.k) direct_row<B>(p, blockIdx.x, L0);
        if (threadIdx.x == 0) {
            sm.ordered = 1u;
            sm.nqueue = 0u;
            sm.tab_n = 0u;
            sm.tab_pos = 0u;
            sm.tab_round = 0u;
        }
        B::sync();
        return;
    }
    for (int64_t b = blockIdx.x; b < batch; b += G) {
        const int64_t L = row_len(p, b);
        if (L <= p.k) direct_row<B>(p, b, L);
    }
    if (threadIdx.x == 0) {
        sm.ordered = 0u;
        sm.nqueue = (uint32_t)batch;
        sm.tab_n = (uint32_t)kTable;  // an empty table that asks to be filled
        sm.tab_pos = (uint32_t)kTable;
        sm.tab_round = 1u;            // from the second row on: row w = snake(0) came first
    }
    B::sync();
}

// One wave: the next kTable rows of this workgroup in index order.
__device__ __forceinline__ void fill_table(const Params& p, Shared& sm) {
    const uint32_t lane = lane_id();
    const uint32_t t = snake(sm.tab_round + lane);
    const bool ok = t < sm.nqueue;
    const uint32_t n = (uint32_t)__popcll(__ballot(ok));  // snake() grows, so the valid ones lead
    if (ok) {
        sm.tab_b[lane] = (int32_t)t;
        sm.tab_len[lane] = (int32_t)row_len(p, t);
    }
    WaveScope::sync();
    if (lane == 0) {
        sm.tab_n = n;
        sm.tab_pos = 0u;
        sm.tab_round += kTable;
    }
    WaveScope::sync();
}

// Where a row's sample lies: `runs` runs of kRunLen scores; run r starts at
// floor(r (L - 64) / (runs - 1)) rounded down to a multiple of 4.
struct SamplePlan {
    int runs;
    int nsv;  // 4-score groups in the sample
    int64_t step_q;
    uint32_t step_r;
    __device__ __forceinline__ explicit SamplePlan(int64_t L) {
        const int64_t fit = L / (2 * kRunLen);
        runs = fit < kMaxRuns ? (int)fit : kMaxRuns;
        nsv = runs >= 2 ? runs * (kRunLen / 4) : 0;
        const int64_t span = runs >= 2 ? (L - kRunLen) : 0;
        step_q = runs >= 2 ? span / (runs - 1) : 0;
        step_r = runs >= 2 ? (uint32_t)(span - step_q * (runs - 1)) : 0u;
    }
    __device__ __forceinline__ int64_t run_start(int r) const {
        return ((int64_t)r * step_q + (int64_t)(((uint32_t)r * step_r) / (uint32_t)(runs - 1))) & ~(int64_t)3;
    }
    // first score of 4-score group t of the sample
    __device__ __forceinline__ int64_t group_start(int t) const {
        return run_start(t / (kRunLen / 4)) + 4 * (t % (kRunLen / 4));
    }
    // runs that lie wholly in [0, L): a leading run of them, as the starts grow
    __device__ __forceinline__ int runs_within(int64_t L) const {
        if (runs < 2) return 0;
        int lo = 0, hi = runs;  // run_start(r) + kRunLen <= L for r < lo, not for r >= hi
        while (lo < hi) {
            const int mid = (lo + hi) / 2;
            if (run_start(mid) + kRunLen <= L) lo = mid + 1;
            else hi = mid;
        }
        return lo;
    }
};

// How a row with L > k is selected: every key kept (L within the capacity),
// sampled, or the full-row path, as the caller's forced path allows.
__device__ __forceinline__ uint32_t row_kind(const Params& p, int64_t L) {
    const int64_t cap = p.capacity;
    if (p.force_path == TOPK_PATH_FULLROW || (p.force_path == TOPK_PATH_LDS && L > cap)) return kKindFull;
    if (p.force_path == TOPK_PATH_LDS || (p.force_path == TOPK_PATH_AUTO && L <= cap)) return kKindAll;
    return kKindSampled;
}

__device__ __forceinline__ void fill_slot(RowSlot& slot, const Params& p, int64_t b, int64_t L, uint32_t kind) {
    slot.b = b;
    slot.L = L;
    slot.nvec = L >> 2;
    slot.m = (uint32_t)p.k;
    slot.T = 0u;                // kKindAll: every key survives
    slot.sh = 32 - kDigitBits;  // and bins take the top 11 bits
    slot.kind = kind;
    slot.valid = 1u;
    slot.nsv = (uint32_t)SamplePlan(L).nsv;
}

// One wave: this workgroup's next row into `slot` (invalid once its share is
// done). Rows with L <= k were written at start; rows forced to the full-row
// path are deferred on the way. The cutoff of a sampled row is set later.
__device__ __forceinline__ void claim_row(const Params& p, Shared& sm, RowSlot& slot, SelectLds own, uint32_t* own_emitted) {
    for (;;) {
        if (sm.tab_pos == sm.tab_n) {
            if (sm.ordered || sm.tab_n < (uint32_t)kTable) {
                if (lane_id() == 0) slot.valid = 0u;
                break;
            }
            fill_table(p, sm);
            continue;
        }
        const int64_t b = sm.tab_b[sm.tab_pos];
        const int64_t L = sm.tab_len[sm.tab_pos];
        WaveScope::sync();
        if (lane_id() == 0) sm.tab_pos += 1u;
        WaveScope::sync();
        if (L <= p.k) continue;
        const uint32_t kind = row_kind(p, L);
        if (kind == kKindFull) {
            defer_row(p, sm, own, own_emitted, b, TOPK_ROW_FULL_FORCED);
            continue;
        }
        if (lane_id() == 0) fill_slot(slot, p, b, L, kind);
        break;
    }
    WaveScope::sync();
}

// The cutoff of a sampled row. A sample of `runs` runs of 64 contiguous
// scores spread evenly over [0, L) gives T at or just below the want-th
// largest sample key, want set so that the expected survivor count sits
// several standard deviations above m (the number of sample keys above the
// true m-th key is binomial).
//
// The sample goes straight from HBM to LDS (every load in flight at once, no
// registers held), except row 0's, which goes through registers. With one
// wave, each lane then keeps its q = ceil(want / lanes) largest keys; the
// smallest of the lanes' q-th largest, lo, has at least want keys at or
// above it (lo = 0 when q is too large to keep). The whole workgroup takes
// a bound per wave instead (see sample_select). A histogram of the keys in
// [lo, sample max], in 2048 bins, locates the want-th largest; its bin is
// narrowed by further histograms until bins are at most 2^kFineShift keys
// wide, and T is the lower edge of the last bin. The bin width of the
// survivor histogram makes [T, sample max] cover about half its bins.

// Scope S: issues the loads of row R's sample from HBM straight into LDS,
// group t at skey[4t, 4t + 4) whichever scope loads it (lane l of a wave
// writes 16 bytes at the wave's LDS base + 16 l).
template <class S>
__device__ __forceinline__ void sample_issue(const Params& p, Shared& sm, const RowSlot& R) {
    constexpr int kPer = (kMaxSample / 4 + S::kSize - 1) / S::kSize;  // 16-byte loads per lane
    const SamplePlan plan(R.L);
    const float* row = p.scores + R.b * p.row_stride;
    const uint32_t wave_base = S::rank() & ~63u;
#pragma unroll
    for (int h = 0; h < kPer; ++h) {
        const int t = h * S::kSize + (int)S::rank();
        if (t < plan.nsv)
            __builtin_amdgcn_global_load_lds(
                row + plan.group_start(t),
                (__attribute__((address_space(3))) void*)(sm.skey + 4 * (h * S::kSize + wave_base)), 16, 0, 0);
    }
}

// An s_waitcnt immediate (vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt at
// their maxima) given to the compiler as a builtin rather than inline asm, so
// that its own wait tracking knows the sample's LDS writes have landed and
// adds no wait of its own for them at later LDS accesses and barriers, where
// streaming loads may be in flight.
constexpr unsigned kWaitVm0 = 0x0F70u;  // vmcnt(0)

// The same, and waits for this wave's loads.
template <class S>
__device__ __forceinline__ void sample_load(const Params& p, Shared& sm, const RowSlot& R) {
    sample_issue<S>(p, sm, R);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
}

// How many of the sample's keys the cutoff keeps at or above it (0: every
// key, the sample being too small for the rule): with n keys from a row of
// L, the count above the row's m-th largest key has mean mu = m n / L, and
// want sits 6 standard deviations (sqrt(mu)) and 4 keys above it.
__device__ __forceinline__ uint32_t sample_want(const RowSlot& R) {
    const uint32_t n = R.nsv * 4u;
    const float mu = (float)R.m * (float)n / (float)R.L;
    const float wantf = ceilf(mu + 6.0f * sqrtf(mu) + 4.0f);
    return wantf < (float)n ? (uint32_t)wantf : 0u;
}

// Waves 0 and 1 together, wave w (row 0 at start, when neither has chunk
// loads of its own in flight): the loads of a sample laid out by `plan`
// from row b straight into LDS, groups h 128 + 64 w + lane.
__device__ __forceinline__ void sample_issue_pair(const Params& p, Shared& sm, int64_t b, const SamplePlan& plan,
                                                  uint32_t w) {
    constexpr int kPer = kMaxSample / 4 / 128;  // 16-byte loads per lane
    const float* row = p.scores + b * p.row_stride;
#pragma unroll
    for (int h = 0; h < kPer; ++h) {
        const int t = h * 128 + (int)(64u * w);
        if (t + (int)lane_id() < plan.nsv)
            __builtin_amdgcn_global_load_lds(row + plan.group_start(t + (int)lane_id()),
                                             (__attribute__((address_space(3))) void*)(sm.skey + 4 * t), 16, 0, 0);
    }
}

// Scope S: the cutoff of row R from the sample in LDS. The bound lo: with
// one wave, each lane keeps the q = ceil(want / 64) largest of its 4-key
// groups' maxima, and lo is the smallest of the lanes' q-th largest (each
// lane has q distinct keys at or above it; lo = 0 when q is too large to
// keep); with the whole workgroup, whose lanes hold a few keys each, each
// wave takes qw = ceil(want / waves) and finds the qw-th largest of its
// lanes' maxima, bit by bit from the top with one ballot per bit, and lo is
// the smallest over the waves. Either way at least want keys lie in
// [lo, sample max]. The workgroup's lanes hold their keys in registers for
// every pass; one wave reads its 64 keys per lane from LDS in each pass.
template <class S>
__device__ __forceinline__ void sample_select(Shared& sm, RowSlot& R, SelectLds lds) {
    constexpr int kPer = (kMaxSample / 4 + S::kSize - 1) / S::kSize;  // 4-key groups per lane
    constexpr uint32_t kWaves = S::kSize / 64;
    constexpr bool kHeld = kWaves > 1;  // keys held in registers
    constexpr int kQ = 4;               // largest group maxima kept per lane (one wave)
    const int nsv = (int)R.nsv;
    const uint32_t want = sample_want(R);
    auto group = [&](int h) -> uint4 {  // group h of this lane's keys (zero keys outside the sample)
        const int t = h * S::kSize + (int)S::rank();
        uint4 k = make_uint4(0u, 0u, 0u, 0u);
        if (t < nsv) {
            const uint4 g = *reinterpret_cast<const uint4*>(sm.skey + 4 * t);
            k = make_uint4(order_key(__uint_as_float(g.x)), order_key(__uint_as_float(g.y)),
                           order_key(__uint_as_float(g.z)), order_key(__uint_as_float(g.w)));
        }
        return k;
    };
    uint4 held[kHeld ? kPer : 1];
    if constexpr (kHeld) {
#pragma unroll
        for (int h = 0; h < kPer; ++h) held[h] = group(h);
    }
    // f(key) for every key of this lane in the sample
    auto each_key = [&](auto&& f) {
#pragma unroll
        for (int h = 0; h < kPer; ++h) {
            if (h * S::kSize + (int)S::rank() >= nsv) continue;
            uint4 k;
            if constexpr (kHeld) k = held[h];
            else k = group(h);
            f(k.x);
            f(k.y);
            f(k.z);
            f(k.w);
        }
    };
    uint32_t lo = 0u, hi = 0u;
    if constexpr (!kHeld) {
        const uint32_t q = (want + 63u) / 64u;
        uint32_t top[kQ] = {0u, 0u, 0u, 0u};  // the lane's largest group maxima, descending
#pragma unroll
        for (int h = 0; h < kPer; ++h) {
            const uint4 k = group(h);
            uint32_t v = max(max(k.x, k.y), max(k.z, k.w));  // 0 outside the sample
#pragma unroll
            for (int j = 0; j < kQ; ++j) {
                const uint32_t up = max(top[j], v);
                v = min(top[j], v);
                top[j] = up;
            }
        }
        uint32_t mine = 0u;
#pragma unroll
        for (int j = 0; j < kQ; ++j) mine = (uint32_t)(j + 1) == q ? top[j] : mine;
        lo = q >= 1u && q <= (uint32_t)kQ ? wave_min(mine) : 0u;
        hi = wave_max(top[0]);
    } else {
        uint32_t lmax = 0u;
        each_key([&](uint32_t k) { lmax = max(lmax, k); });
        const uint32_t hi_w = wave_max(lmax);
        uint32_t lo_w = 0u;
        const uint32_t qw = (want + kWaves - 1u) / kWaves;
        if (want > 0u && qw <= 64u) {
            // the largest v with at least qw lane maxima at or above it
            for (int bit = 31; bit >= 0; --bit) {
                const uint32_t c = lo_w | (1u << bit);
                if ((uint32_t)__popcll(__ballot(lmax >= c)) >= qw) lo_w = c;
            }
        }
        if (lane_id() == 0) {
            sm.cand_key[wave_id()] = lo_w;
            sm.cand_idx[wave_id()] = hi_w;
        }
        S::sync();
        // one lane reads the waves' bounds (the other lanes' reads would
        // cost LDS bandwidth), and shares them
        lo = 0xFFFFFFFFu;
        if (lane_id() == 0) {
#pragma unroll
            for (uint32_t w = 0; w < kWaves; ++w) {
                lo = min(lo, sm.cand_key[w]);
                hi = max(hi, sm.cand_idx[w]);
            }
        }
        lo = __builtin_amdgcn_readfirstlane(lo);
        hi = __builtin_amdgcn_readfirstlane(hi);
    }
    uint32_t T = 0u;  // too short to sample, or want out of reach: keep everything
    if (want > 0u) {
        // the rank-th largest key in [base, top] lies in one of 2048 bins of
        // width 2^sh; narrow to that bin until bins are fine enough
        uint32_t base = lo, top = hi, rank = want;
        for (;;) {
            const uint32_t span = top - base;
            const int wb = span == 0u ? 0 : 32 - __clz(span);
            const int sh = wb > kDigitBits ? wb - kDigitBits : 0;  // span >> sh < 2048
            each_key([&](uint32_t k) {
                if (k >= base && k <= top) atomicAdd(&lds.hist[(k - base) >> sh], 1u);
            });
            S::sync();
            const Found f = find_rank_bin<S>(lds, rank);
            const uint32_t edge = base + (f.digit << sh);
            if (sh <= kFineShift) {
                T = edge;
                break;
            }
            rank -= f.above;
            const uint32_t room = top - edge;
            top = edge + (room < (1u << sh) - 1u ? room : (1u << sh) - 1u);
            base = edge;
        }
    }
    const uint32_t span = hi - T;
    const int wbits = span == 0u ? 0 : 32 - __clz(span);
    if (S::rank() == 0) {
        R.T = T;
        R.sh = (uint32_t)(wbits > kDigitBits - 1 ? wbits - (kDigitBits - 1) : 0);
    }
    S::sync();
}



// ----------------------------------------------------------------------------
// progress counters between the roles
// ----------------------------------------------------------------------------
//
// Rows go through the workgroup in sequence i = 0, 1, ...: row i sits in slot
// i % kSlots and its survivors in buffer i % 2. The sampler wave claims rows
// (n_claimed) and sets their cutoffs (n_ready); the finisher wave finishes
// them (n_finished) once every streaming wave has left them (left[slot]). A
// streaming wave reads chunks of a claimed row, filters them once the row's
// cutoff is set and its buffer free (row i - 2 finished), and leaves the row
// after its last chunk of it. Every wait is on an earlier row, or on a row
// the waiting wave holds nothing of, so none can close a cycle.

// Counters are written by one lane after the wave's earlier LDS writes are
// done, and read by every lane of the waiting wave.
__device__ __forceinline__ void publish(uint32_t* ctr, uint32_t v) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (lane_id() == 0) __hip_atomic_store(ctr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void publish_add(uint32_t* ctr, uint32_t v) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (lane_id() == 0) __hip_atomic_fetch_add(ctr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ uint32_t peek(const uint32_t* ctr) {
    return __builtin_amdgcn_readfirstlane(__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
}

// Waits until *ctr >= v; false if the workgroup gave up instead. A wait that
// outlasts kWatchdogTicks of the 100 MHz wall clock (far beyond any row the
// API admits) gives the workgroup up, so that a defect ends the launch rather
// than hanging it, and counts a trip in g_watchdog_trips.
__device__ __forceinline__ bool wait_for(Shared& sm, const uint32_t* ctr, uint32_t v) {
    uint64_t t0 = 0;
    for (uint32_t n = 0;; ++n) {
        if (peek(ctr) >= v) {
            asm volatile("" ::: "memory");
            return true;
        }
        if (peek(&sm.abort) != 0u) return false;
        if ((n & 1023u) == 0u) {
            const uint64_t t = wall_clock64();
            if (n == 0u) {
                t0 = t;
            } else if (t - t0 > kWatchdogTicks) {
                if (lane_id() == 0) sm.abort = 1u;
                return false;
            }
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

// Waves 0 and 1 together, wave w: the cutoff of row R from its sample in LDS
// (groups [0, R.nsv), wave w reading groups h 128 + 64 w + lane, its keys
// held in registers). Each wave bounds its half as one wave does
// (q = ceil(want / 128)), the two bounds are exchanged through LDS and a
// counter, each wave adds its half's keys in [lo, sample max] to a 1024-bin
// histogram, and the wave that finishes second finds the want-th largest
// key's bin with one prefix sum (each lane summing 16 bins) and publishes
// the bin's lower edge as the cutoff (n_ready = 1); when that bin is wider
// than 2^kPairFineShift keys, the whole search by one wave instead. Returns
// whether this wave published.
__device__ __forceinline__ bool sample_select_pair(Shared& sm, RowSlot& R, SelectLds lds, uint32_t w) {
    constexpr int kPer = kMaxSample / 4 / 128;  // 4-key groups per lane
    constexpr int kQ = 4;
    constexpr int kPairBits = 10;  // 1024 bins, 16 per lane
    static_assert((1 << kPairBits) + 64 <= kBins, "room for a sink bin per lane past the bins");
    const int nsv = (int)R.nsv;
    const uint32_t want = sample_want(R);
    const uint32_t lane = lane_id();
    uint4 key[kPer];
    uint32_t gvalid = 0u;
#pragma unroll
    for (int h = 0; h < kPer; ++h) {
        const int t = h * 128 + (int)(64u * w + lane);
        uint4 k = make_uint4(0u, 0u, 0u, 0u);
        if (t < nsv) {
            const uint4 g = *reinterpret_cast<const uint4*>(sm.skey + 4 * t);
            k = make_uint4(order_key(__uint_as_float(g.x)), order_key(__uint_as_float(g.y)),
                           order_key(__uint_as_float(g.z)), order_key(__uint_as_float(g.w)));
            gvalid |= 1u << h;
        }
        key[h] = k;
    }
    const uint32_t q = (want + 127u) / 128u;
    uint32_t top[kQ] = {0u, 0u, 0u, 0u};  // the lane's largest group maxima, descending
    if (q <= 1u) {  // the lane's maximum is all the bound needs
#pragma unroll
        for (int h = 0; h < kPer; ++h) top[0] = max(top[0], max(max(key[h].x, key[h].y), max(key[h].z, key[h].w)));
    } else {
#pragma unroll
        for (int h = 0; h < kPer; ++h) {
            uint32_t v = max(max(key[h].x, key[h].y), max(key[h].z, key[h].w));  // 0 outside the sample
#pragma unroll
            for (int j = 0; j < kQ; ++j) {
                const uint32_t up = max(top[j], v);
                v = min(top[j], v);
                top[j] = up;
            }
        }
    }
    uint32_t mine = 0u;
#pragma unroll
    for (int j = 0; j < kQ; ++j) mine = (uint32_t)(j + 1) == q ? top[j] : mine;
    const uint32_t lo_w = q >= 1u && q <= (uint32_t)kQ ? wave_min(mine) : 0u;
    const uint32_t hi_w = wave_max(top[0]);
    if (lane == 0) {
        sm.cand_key[w] = lo_w;
        sm.cand_idx[w] = hi_w;
    }
    publish_add(&sm.pair, 1u);
    if (!wait_for(sm, &sm.pair, 2u)) return false;
    const uint32_t lo = min(sm.cand_key[0], sm.cand_key[1]);
    const uint32_t hi = max(sm.cand_idx[0], sm.cand_idx[1]);
    const uint32_t span = hi - lo;
    const int wb = span == 0u ? 0 : 32 - __clz(span);
    const int sh = wb > kPairBits ? wb - kPairBits : 0;  // span >> sh < 1024
    if (want > 0u) {
        // every key counted without a branch: keys below lo, and groups
        // outside the sample, into a bin of the lane's own past the 1024
        // (cleared by the wave that finishes)
        const uint32_t sink = 1024u + lane;
#pragma unroll
        for (int h = 0; h < kPer; ++h) {
            const bool in = (gvalid >> h) & 1u;
            const uint4 k = key[h];
            atomicAdd(&lds.hist[in && k.x >= lo ? (k.x - lo) >> sh : sink], 1u);
            atomicAdd(&lds.hist[in && k.y >= lo ? (k.y - lo) >> sh : sink], 1u);
            atomicAdd(&lds.hist[in && k.z >= lo ? (k.z - lo) >> sh : sink], 1u);
            atomicAdd(&lds.hist[in && k.w >= lo ? (k.w - lo) >> sh : sink], 1u);
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    uint32_t order = 0u;
    if (lane == 0) order = __hip_atomic_fetch_add(&sm.pair, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    order = __builtin_amdgcn_readfirstlane(order);
    if (order == 2u) return false;  // the other wave finishes
    asm volatile("" ::: "memory");
    uint32_t T = 0u;  // too short to sample, or want out of reach: keep everything
    bool narrow = false;
    if (want > 0u) {
        // lane l holds bins base .. base + 15, base = 1008 - 16 l (the top
        // bins in lane 0); the want-th key from the top lies in the first
        // lane whose running sum reaches want, in its bin where the lane's
        // own running sum, from its top bin down, does
        const uint32_t base = 1008u - 16u * lane;
        const uint4* h4 = reinterpret_cast<const uint4*>(lds.hist + base);
        const uint4 c0 = h4[0], c1 = h4[1], c2 = h4[2], c3 = h4[3];
        const uint32_t c[16] = {c3.w, c3.z, c3.y, c3.x, c2.w, c2.z, c2.y, c2.x,
                                c1.w, c1.z, c1.y, c1.x, c0.w, c0.z, c0.y, c0.x};
        uint32_t own = 0u;
#pragma unroll
        for (int j = 0; j < 16; ++j) own += c[j];
        const uint32_t incl = wave_inclusive_sum(own);
        const int ol = __ffsll((unsigned long long)__ballot(incl - own < want && want <= incl)) - 1;
        uint32_t acc = incl - own, digit = 0u;
        bool hit = false;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const bool here = !hit && acc + c[j] >= want;
            digit = here ? base + 15u - (uint32_t)j : digit;
            hit = hit || here;
            acc += c[j];
        }
        digit = (uint32_t)__builtin_amdgcn_readlane((int)digit, ol);
        T = lo + (digit << sh);
        narrow = sh > kPairFineShift;
        // the histogram back to zero for the sampler's next use
        uint4* z4 = reinterpret_cast<uint4*>(lds.hist + base);
#pragma unroll
        for (int j = 0; j < 4; ++j) z4[j] = make_uint4(0u, 0u, 0u, 0u);
        lds.hist[1024u + lane] = 0u;
        WaveScope::sync();
    }
    if (narrow) {
        // the bin is too wide: the whole search again by this wave
        sample_select<WaveScope>(sm, R, lds);
    } else {
        const uint32_t rest = hi - T;
        const int wbits = rest == 0u ? 0 : 32 - __clz(rest);
        if (lane == 0) {
            R.T = T;
            R.sh = (uint32_t)(wbits > kDigitBits - 1 ? wbits - (kDigitBits - 1) : 0);
        }
    }
    publish(&sm.n_ready, 1u);
    return true;
}

// ----------------------------------------------------------------------------
// streaming
// ----------------------------------------------------------------------------

constexpr int kStreamers = kThreads / 64 - kFirstStreamer;
constexpr uint32_t kNone = 0xFFFFFFFEu;  // no chunk within reach
constexpr uint32_t kEnd = 0xFFFFFFFFu;   // this workgroup's rows are done

// Streaming waves read a row's full groups of 4 scores in chunks of
// kChunkVec groups; the finisher takes the last L % 4 scores.
__device__ __forceinline__ uint32_t nchunks_of(int64_t L) {
    const int64_t groups = L >> 2;
    return (uint32_t)((groups + kChunkVec - 1) / kChunkVec);
}
__device__ __forceinline__ uint32_t nchunks(const RowSlot& R) { return nchunks_of(R.L); }

// A chunk in registers: kUnroll groups of 4 scores per lane.
struct Chunk {
    f4 v[kUnroll];
};

constexpr uint32_t kBufferConfig = 0x00020000u;  // raw buffer descriptor word 3 on CDNA
constexpr int kNonTemporal = 2;                  // buffer load cache policy: streaming

__device__ __forceinline__ uint64_t uniform(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Issues the loads of chunk c (full groups only) of a row of L scores;
// c >= kNone issues loads that touch no memory. Every call issues the same
// kUnroll buffer loads, so the count of loads in flight never depends on the
// path taken; loads past the descriptor's range return zero without a
// memory access.
__device__ __forceinline__ void load_chunk(Chunk& x, const float* row, int64_t L, uint32_t c) {
    const uint32_t lane = lane_id();
    L = (int64_t)uniform((uint64_t)L);
    const uint64_t rowp = uniform((uint64_t)reinterpret_cast<uintptr_t>(row));
    const int64_t g0 = c < kNone ? (int64_t)c * kChunkVec : 0;  // first group of the chunk
    int64_t nf = c < kNone ? (L >> 2) - g0 : 0;                  // full groups in it
    nf = nf < 0 ? 0 : (nf > kChunkVec ? kChunkVec : nf);
    const __amdgpu_buffer_rsrc_t body = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void*>(rowp + 16u * (uint64_t)g0), 0, (int)(16 * nf), (int)kBufferConfig);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const auto w = __builtin_amdgcn_raw_buffer_load_b128(body, (int)(16 * (lane + 64 * u)), 0, kNonTemporal);
        x.v[u] = f4{__uint_as_float(w[0]), __uint_as_float(w[1]), __uint_as_float(w[2]), __uint_as_float(w[3])};
    }
}

// The last L % 4 scores of a row, one per lane of the finisher wave, which
// appends their hits to the row's buffer as a streaming wave would. The
// buffer is free by then, and appends from several waves may interleave.
__device__ __forceinline__ float load_tail(const Params& p, const RowSlot& R) {
    const uint32_t lane = lane_id();
    return lane < (uint32_t)(R.L & 3) ? p.scores[R.b * p.row_stride + (R.L & ~(int64_t)3) + lane] : 0.f;
}

__device__ __forceinline__ void append_tail(Shared& sm, const RowSlot& R, int x, uint32_t cap, float t) {
    const uint32_t lane = lane_id();
    const uint32_t kk = order_key(t);
    const bool h = lane < (uint32_t)(R.L & 3) && kk >= R.T;
    const uint64_t mk = __ballot(h);
    if (mk != 0) {
        uint32_t base = 0u;
        if (lane == 0) base = atomicAdd(&sm.count[x], (uint32_t)__popcll(mk));
        base = __builtin_amdgcn_readfirstlane(base);
        const uint32_t pos = base + lanes_below(mk);
        if (h && pos < cap) {
            sm.surv[x][pos] = make_uint2(__float_as_uint(t), (uint32_t)(R.L & ~(int64_t)3) + lane);
        }
    }
    WaveScope::sync();
}

// One streaming wave.
struct Streamer {
    const Params& p;
    Shared& sm;
    uint32_t cap;
    int i;       // row of the chunk held
    uint32_t c;  // the chunk held
    int open;    // the row whose filter state below is loaded, or -1
    int ok;      // rows up to this one have their cutoff set and their buffer free
    uint32_t T, buf;
    int64_t L;
    uint32_t pre = kNone;  // a second chunk of row i issued at the start, into the other registers

    __device__ __forceinline__ void leave(int r) { publish_add(&sm.left[r % kSlots], 1u); }

    // The next chunk at or after row r (the row of the chunk held, if
    // `holding`), waiting for rows to be claimed only up to row lim. Rows
    // passed on the way are left, except r while a chunk of it is held.
    // Returns the chunk with r set to its row; kNone with r the first row not
    // looked at; kEnd past this workgroup's last row.
    __device__ __forceinline__ uint32_t grab(int& r, int lim, bool holding) {
        for (;;) {
            if (r > lim) return kNone;
            if (!wait_for(sm, &sm.n_claimed, (uint32_t)r + 1u)) return kEnd;
            const RowSlot& R = sm.slot[r % kSlots];
            if (!R.valid) return kEnd;
            uint32_t ch = 0u;
            if (lane_id() == 0) ch = atomicAdd(&sm.chunk_next[r % kSlots], 1u);
            ch = __builtin_amdgcn_readfirstlane(ch);
            if (ch < nchunks(R)) return ch;
            if (!holding) leave(r);
            holding = false;
            ++r;
        }
    }

    __device__ __forceinline__ void load(Chunk& v, int r, uint32_t ch) {
        const RowSlot& R = sm.slot[r % kSlots];
        load_chunk(v, p.scores + R.b * p.row_stride, R.L, ch);
    }

    // Appends the hits (key >= T) of loads [kPart H, kPart H + kPart) of
    // chunk ch to the row's buffer with one LDS atomic; false once the row's
    // count has passed the capacity. Survivors are stored as raw score bits
    // with their positions; the finisher turns the bits into keys.
    // kNonNegT: T is the key of a non-negative float, so a signed compare of
    // the raw bits decides.
    template <bool kNonNegT, int H>
    __device__ __forceinline__ bool filter_part(const Chunk& x, uint32_t ch) {
        const int64_t v0 = (int64_t)ch * kChunkVec + lane_id();
        const int32_t Ts = (int32_t)(T ^ 0x80000000u);
        const int64_t nfull = L >> 2;
        auto hit = [&](float f) -> bool {
            if constexpr (kNonNegT) return (int32_t)__float_as_uint(f) >= Ts;
            else return order_key(f) >= T;
        };
        // lanes whose group of load u lies inside the row (all but the
        // row's last chunk: every lane)
        uint64_t okm[kPart];
        uint64_t mk[4 * kPart];
        uint32_t total = 0;
#pragma unroll
        for (int u = 0; u < kPart; ++u) {
            okm[u] = __ballot(v0 + (kPart * H + u) * 64 < nfull);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                mk[4 * u + e] = __ballot(hit(x.v[kPart * H + u][e])) & okm[u];
                total += (uint32_t)__popcll(mk[4 * u + e]);
            }
        }
        if (total == 0) return true;
        uint32_t base = 0u;
        if (lane_id() == 0) base = atomicAdd(&sm.count[buf], total);
        base = __builtin_amdgcn_readfirstlane(base);
        if (base >= cap) return false;
        uint2* sv = sm.surv[buf];
        auto append = [&](auto check) {
            uint32_t off = base;
#pragma unroll
            for (int u = 0; u < kPart; ++u) {
                const uint32_t i0 = (uint32_t)(4 * (v0 + (kPart * H + u) * 64));
                const bool ok = v0 + (kPart * H + u) * 64 < nfull;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float f = x.v[kPart * H + u][e];
                    // the compare again, rather than a kept flag, so that
                    // its lane mask drives the append directly
                    if (ok && hit(f)) {
                        const uint64_t m = mk[4 * u + e];
                        const uint32_t pos =
                            __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, off));
                        if (check(pos)) sv[pos] = make_uint2(__float_as_uint(f), i0 + (uint32_t)e);
                    }
                    off += (uint32_t)__popcll(mk[4 * u + e]);
                }
            }
        };
        const bool fits = base + total <= cap;
        if (fits) append([](uint32_t) { return true; });
        else append([&](uint32_t pos) { return pos < cap; });
        return fits;
    }

    template <bool kNonNegT, int H = 0>
    __device__ __forceinline__ bool filter(const Chunk& x, uint32_t ch) {
        static_assert(kUnroll % kPart == 0, "whole parts per chunk");
        if (!filter_part<kNonNegT, H>(x, ch)) return false;
        if constexpr (H + 1 < kUnroll / kPart) return filter<kNonNegT, H + 1>(x, ch);
        return true;
    }

    __device__ __forceinline__ bool filter_held(const Chunk& v) {
        if (i != open) {
            if (i > ok) {
                if (!wait_for(sm, &sm.n_ready, (uint32_t)i + 1u)) return false;
                if (i >= 2 && !wait_for(sm, &sm.n_finished, (uint32_t)i - 1u)) return false;
                ok = i;
            }
            const RowSlot& R = sm.slot[i % kSlots];
            T = R.T;
            L = R.L;
            buf = (uint32_t)(i & 1);
            open = i;
        }
        return T >= 0x80000000u ? filter<true>(v, c) : filter<false>(v, c);
    }

    // Done with row r: its largest survivor key, then the count of waves out.
    __device__ __forceinline__ void close(int r) {
        leave(r);
    }

    // Holding chunk c of row i in `held`: issue the next chunk into `next`,
    // then filter `held`. False when this workgroup's rows are done.
    __device__ __forceinline__ bool step(Chunk& held, Chunk& next) {
        int r = i;
        uint32_t cn = pre;
        if (cn < kNone) {
            pre = kNone;
        } else {
            cn = grab(r, i + 2, true);
            load(next, r, cn);
        }
        if (!filter_held(held)) {
            // over capacity: no wave takes more of this row
            if (lane_id() == 0) atomicMax(&sm.chunk_next[i % kSlots], nchunks(sm.slot[i % kSlots]));
            if (r == i) {  // drop the chunk just issued
                r = i + 1;
                cn = kNone;
            }
        }
        if (r != i) close(i);
        if (cn == kNone) {  // nothing held now, so waiting for any row is safe
            cn = grab(r, INT32_MAX, false);
            if (cn < kNone) load(next, r, cn);
        }
        if (cn == kEnd) return false;
        i = r;
        c = cn;
        return true;
    }
};

// ----------------------------------------------------------------------------
// finishing a row from its survivors
// ----------------------------------------------------------------------------

// One wave: lane l < nc holds candidate (key kj, index ij), and all nc
// candidates are also in LDS (keys, idxs: 16-byte aligned, room for
// kMaxCand); returns how many of them rank before it (key descending, index
// ascending). Every lane reads the candidates with broadcast LDS loads, four
// at a time, all independent of each other (entries past nc are read but not
// counted): a cross-lane read per candidate would cost a dependent
// register-to-scalar round trip each.
__device__ __forceinline__ uint32_t rank_in_wave(const uint32_t* keys, const uint32_t* idxs, uint32_t kj,
                                                 uint32_t ij, uint32_t nc) {
    uint32_t r = 0;
    for (uint32_t i = 0; i < nc; i += 4) {
        const uint4 k4 = *reinterpret_cast<const uint4*>(keys + i);
        const uint4 i4 = *reinterpret_cast<const uint4*>(idxs + i);
        r += (k4.x > kj || (k4.x == kj && i4.x < ij)) ? 1u : 0u;
        r += (i + 1 < nc && (k4.y > kj || (k4.y == kj && i4.y < ij))) ? 1u : 0u;
        r += (i + 2 < nc && (k4.z > kj || (k4.z == kj && i4.z < ij))) ? 1u : 0u;
        r += (i + 3 < nc && (k4.w > kj || (k4.w == kj && i4.w < ij))) ? 1u : 0u;
    }
    return r;
}

// Scope S (wave 0 alone, or the whole workgroup for the last row): the exact
// top m of row R from its n survivors in buffer x, k <= m <= n <= capacity.
// One pass bins the survivors upward from T and finds the largest; the bin
// holding the m-th largest follows from the counts. Every survivor in a bin
// above it is written out in a second pass over the buffer, which also
// gathers the cutoff bin's entries; one wave ranks those by (key descending,
// index ascending) and writes the first `need`. A crowded or open-ended
// cutoff bin takes the radix select over the buffer instead.
// kNonNegT: T is the key of a non-negative float, so every survivor is one
// too and its raw bits order like its key (key = bits + 2^31); the passes
// then compare raw bits with thresholds moved into that space.
template <class S, bool kNonNegT>
__device__ __forceinline__ void finish_sampled(const Params& p, Shared& sm, const RowSlot& R, int x, uint32_t n,
                                               SelectLds lds) {
    constexpr bool kWave = S::kSize == 64;
    const uint32_t m = R.m;
    uint32_t* hist = lds.hist;
    const uint2* E = sm.surv[x];
    // the value survivors are compared in: raw bits, or the key
    auto val = [](uint32_t bits) -> uint32_t {
        if constexpr (kNonNegT) return bits;
        else return order_key(__uint_as_float(bits));
    };
    constexpr uint32_t kShift = kNonNegT ? 0x80000000u : 0u;  // key = val + kShift
    const uint32_t Tv = R.T - kShift;
    const uint32_t sh = R.sh;
    // one wave reads kU entries per lane per step, all loads issued before
    // any is used; reads past n stay inside the buffer (its capacity is a
    // multiple of kU * 64) and are ignored
    constexpr int kU = kWave ? 8 : 1;
    static_assert(!kWave || kCapacity % (kU * 64) == 0, "unmasked reads stay in the buffer");
    {
        // bin the survivors and find the largest
        uint32_t vm = 0u;
        for (uint32_t e0 = kWave ? 0u : S::rank(); e0 < n; e0 += kU * S::kSize) {
            uint2 v[kU];
#pragma unroll
            for (int j = 0; j < kU; ++j) v[j] = E[e0 + j * S::kSize + (kWave ? lane_id() : 0u)];
#pragma unroll
            for (int j = 0; j < kU; ++j) {
                // no branch per entry: an entry past n adds zero
                const bool ok = e0 + j * S::kSize + (kWave ? lane_id() : 0u) < n;
                const uint32_t kv = val(v[j].x);
                vm = max(vm, ok ? kv : 0u);
                const uint32_t d = (kv - Tv) >> sh;
                atomicAdd(&hist[d < (uint32_t)kBins ? d : (uint32_t)kBins - 1u], ok ? 1u : 0u);
            }
        }
        vm = wave_max(vm);
        if (lane_id() == 0) atomicMax(&sm.vmax[x], vm + kShift);
        S::sync();
    }
    const Found f = find_rank_bin<S>(lds, m);
    if (f.count > (uint32_t)kMaxCand || f.digit == (uint32_t)kBins - 1u) {
        const PairSource<S> src{E, n};
        const Selection s = select_top<S>(lds, src, m, n, R.T, sm.vmax[x], bits_for(R.L));
        OutRow out = out_row(p, R.b, m, &sm.emitted);
        emit(src, s, out);
        return;
    }
    const uint32_t need = m - f.above;
    const bool whole = f.count == need;  // the cutoff bin is taken whole
    // bin f.digit is [lo, hi) in key space, hi <= 2^32; in val space:
    // above <=> val > t_above, in the bin <=> !above && val >= t_lo
    const uint64_t hi = (uint64_t)R.T + ((uint64_t)(f.digit + 1u) << sh);
    const uint32_t t_above = (hi > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)(hi - 1u)) - kShift;
    const uint32_t t_lo = R.T + (f.digit << sh) - kShift;  // the bin holds a survivor, so no overflow
    // per entry: taken <=> val >= t_take (and not take_none); a candidate
    // <=> val - t_lo <= c_span (unsigned) and candidates are wanted. Plain
    // compares and bitwise ands, so that the entry loops have no branches.
    const uint32_t t_take = whole ? t_lo : t_above + 1u;
    const bool take_none = !whole && t_above == 0xFFFFFFFFu;
    const bool want_cand = !whole;
    const uint32_t c_span = t_above - t_lo;
    if constexpr (kWave) {
        // Selected positions are compacted in place into the buffer's first
        // words (after a step's entries are read, the selected count cannot
        // pass the words already read), then copied to the output row with
        // coalesced stores. Within a step each lane marks its taken entries
        // and cutoff-bin candidates in bit masks; one wave prefix sum of the
        // packed counts places them.
        const uint32_t lane = lane_id();
        uint32_t* stage = reinterpret_cast<uint32_t*>(sm.surv[x]);
        uint32_t next = 0u, ncand = 0u;
        for (uint32_t e0 = 0; e0 < n; e0 += kU * 64) {
            uint2 v[kU];
#pragma unroll
            for (int j = 0; j < kU; ++j) v[j] = E[e0 + 64 * j + lane];
            uint32_t tmask = 0u, cmask = 0u;
#pragma unroll
            for (int j = 0; j < kU; ++j) {
                const bool ok = e0 + 64 * j + lane < n;
                const uint32_t kv = val(v[j].x);
                const bool take = ok & !take_none & (kv >= t_take);
                const bool cand = ok & want_cand & (kv - t_lo <= c_span);
                tmask |= (uint32_t)take << j;
                cmask |= (uint32_t)cand << j;
            }
            const uint32_t packed = (uint32_t)__popc(tmask) | ((uint32_t)__popc(cmask) << 16);
            const uint32_t incl = wave_inclusive_sum(packed);
            const uint32_t excl = incl - packed;
            uint32_t ts = next + (excl & 0xFFFFu);
            uint32_t cs = ncand + (excl >> 16);
            const uint32_t total = __builtin_amdgcn_readlane(incl, 63);
            next += total & 0xFFFFu;
            ncand += total >> 16;
            // stores under the lane mask only: the streaming waves share the
            // LDS, so unneeded lane writes cost them bandwidth
#pragma unroll
            for (int j = 0; j < kU; ++j) {
                const uint32_t tb = (tmask >> j) & 1u;
                if (tb) stage[ts] = v[j].y;
                ts += tb;
            }
            if ((total >> 16) != 0u) {  // a cutoff-bin candidate in this step (rare)
#pragma unroll
                for (int j = 0; j < kU; ++j) {
                    const uint32_t cb = (cmask >> j) & 1u;
                    if (cb && cs < (uint32_t)kMaxCand) {
                        sm.cand_key[cs] = val(v[j].x);
                        sm.cand_idx[cs] = v[j].y;
                    }
                    cs += cb;
                }
            }
        }
        if (!whole) {
            S::sync();
            const uint32_t nc = f.count;
            const bool have = lane < nc;
            const uint32_t kj = have ? sm.cand_key[lane] : 0u;
            const uint32_t ij = have ? sm.cand_idx[lane] : 0u;
            const uint32_t r = rank_in_wave(sm.cand_key, sm.cand_idx, kj, ij, nc);
            if (have && r < need) stage[next + r] = ij;
        }
        S::sync();
        const OutRow out = out_row(p, R.b, m, nullptr);
        for (uint32_t i = lane; i < m; i += 64) out.row[i] = out.map(stage[i]);
    } else {
        OutRow out = out_row(p, R.b, m, &sm.emitted);
        for (uint32_t e = S::rank(); e < n; e += S::kSize) {
            const uint2 v = E[e];
            const uint32_t kv = val(v.x);
            out.append(!take_none & (kv >= t_take), v.y);
            const bool cand = want_cand & (kv - t_lo <= c_span);
            const uint32_t slot = wave_reserve(&sm.ncand, cand);
            if (cand && slot < (uint32_t)kMaxCand) {
                sm.cand_key[slot] = kv;
                sm.cand_idx[slot] = v.y;
            }
        }
        S::sync();
        if (!whole && S::first_wave()) {
            const uint32_t lane = lane_id();
            const uint32_t nc = f.count;
            const bool have = lane < nc;
            const uint32_t kj = have ? sm.cand_key[lane] : 0u;
            const uint32_t ij = have ? sm.cand_idx[lane] : 0u;
            const uint32_t r = rank_in_wave(sm.cand_key, sm.cand_idx, kj, ij, nc);
            out.append(have && r < need, ij);
        }
    }
}

// The whole workgroup's finish of a row (its last row): the selection of
// finish_sampled with each lane's survivors read from LDS once, into
// registers, for both passes, and one slot reservation per wave: the entries
// above the cutoff bin take slots [0, above), the cutoff bin's best `need`
// the slots [m - need, m). Row stats and counters as finish_sampled.
template <class S, bool kNonNegT>
__device__ __forceinline__ void finish_sampled_wg(const Params& p, Shared& sm, const RowSlot& R, int x, uint32_t n,
                                                  SelectLds lds) {
    constexpr int kPer = (kCapacity + S::kSize - 1) / S::kSize;  // entries per lane at most
    const uint32_t m = R.m;
    const uint2* E = sm.surv[x];
    auto val = [](uint32_t bits) -> uint32_t {
        if constexpr (kNonNegT) return bits;
        else return order_key(__uint_as_float(bits));
    };
    constexpr uint32_t kShift = kNonNegT ? 0x80000000u : 0u;  // key = val + kShift
    const uint32_t Tv = R.T - kShift;
    const uint32_t sh = R.sh;
    uint2 v[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {  // every load issued before any is used
        const uint32_t e = S::rank() + (uint32_t)j * S::kSize;
        v[j] = e < n ? E[e] : make_uint2(0u, 0u);
    }
    uint32_t vm = 0u;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        if (S::rank() + (uint32_t)j * S::kSize < n) {
            const uint32_t kv = val(v[j].x);
            vm = max(vm, kv);
            const uint32_t d = (kv - Tv) >> sh;
            atomicAdd(&lds.hist[d < (uint32_t)kBins ? d : (uint32_t)kBins - 1u], 1u);
        }
    }
    vm = wave_max(vm);
    if (lane_id() == 0) atomicMax(&sm.vmax[x], vm + kShift);
    S::sync();
    const Found f = find_rank_bin<S>(lds, m);
    if (f.count > (uint32_t)kMaxCand || f.digit == (uint32_t)kBins - 1u) {
        const PairSource<S> src{E, n};
        const Selection s = select_top<S>(lds, src, m, n, R.T, sm.vmax[x], bits_for(R.L));
        OutRow out = out_row(p, R.b, m, &sm.emitted);
        emit(src, s, out);
        return;
    }
    const uint32_t need = m - f.above;
    const bool whole = f.count == need;
    const uint64_t hi = (uint64_t)R.T + ((uint64_t)(f.digit + 1u) << sh);
    const uint32_t t_above = (hi > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)(hi - 1u)) - kShift;
    const uint32_t t_lo = R.T + (f.digit << sh) - kShift;
    const uint32_t t_take = whole ? t_lo : t_above + 1u;
    const bool take_none = !whole && t_above == 0xFFFFFFFFu;
    const uint32_t c_span = t_above - t_lo;
    uint32_t tmask = 0u, cmask = 0u;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const bool ok = S::rank() + (uint32_t)j * S::kSize < n;
        const uint32_t kv = val(v[j].x);
        tmask |= (uint32_t)(ok & !take_none & (kv >= t_take)) << j;
        cmask |= (uint32_t)(ok & !whole & (kv - t_lo <= c_span)) << j;
    }
    // both reservations in one: taken entries in the low 16 bits, candidates
    // in the high 16 (at most m <= 2048 and the buffer's capacity, so the
    // low half never carries)
    const uint32_t slots =
        wave_reserve_count(&sm.take_cand, (uint32_t)__popc(tmask) | ((uint32_t)__popc(cmask) << 16));
    uint32_t ts = slots & 0xFFFFu;
    uint32_t cs = slots >> 16;
    const OutRow out = out_row(p, R.b, m, nullptr);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        if ((tmask >> j) & 1u) {
            if (ts < m) out.row[ts] = out.map(v[j].y);
            ++ts;
        }
        if ((cmask >> j) & 1u) {
            if (cs < (uint32_t)kMaxCand) {
                sm.cand_key[cs] = val(v[j].x);
                sm.cand_idx[cs] = v[j].y;
            }
            ++cs;
        }
    }
    if (whole) return;
    S::sync();
    if (S::first_wave()) {
        const uint32_t lane = lane_id();
        const uint32_t nc = f.count;
        const bool have = lane < nc;
        const uint32_t kj = have ? sm.cand_key[lane] : 0u;
        const uint32_t ij = have ? sm.cand_idx[lane] : 0u;
        const uint32_t r = rank_in_wave(sm.cand_key, sm.cand_idx, kj, ij, nc);
        if (have && r < need) out.row[m - need + r] = out.map(ij);
    }
}

// Scope S: finishes row R from buffer x, or defers it to the full-row path
// when its survivors overflowed the buffer or fell short of m (returns
// whether it did, the same in every lane). One wave (rows before the last)
// leaves buffer x's counters and histogram zero.
template <class S>
__device__ __forceinline__ bool finish_row(const Params& p, Shared& sm, const RowSlot& R, int x, uint32_t cap) {
    const uint32_t n = sm.count[x];
    const SelectLds lds{sm.hist[x], sm.found};
    const bool deferred = n > cap || n < R.m;
    if (deferred) {
        const int code = n > cap ? TOPK_ROW_FULL_OVERFLOW : TOPK_ROW_FULL_UNDERFLOW;
        if (S::first_wave()) defer_row(p, sm, lds, &sm.emitted, R.b, code);
    } else {
        if constexpr (S::kSize == 64) {
            if (R.T >= 0x80000000u) finish_sampled<S, true>(p, sm, R, x, n, lds);
            else finish_sampled<S, false>(p, sm, R, x, n, lds);
        } else {
            if (R.T >= 0x80000000u) finish_sampled_wg<S, true>(p, sm, R, x, n, lds);
            else finish_sampled_wg<S, false>(p, sm, R, x, n, lds);
        }
        if (S::rank() == 0) put_stats(p, R.b, R.kind == kKindAll ? TOPK_ROW_LDS : TOPK_ROW_SAMPLED, n);
    }
    if constexpr (S::kSize == 64) {
        S::sync();
        if (S::rank() == 0) {
            sm.count[x] = 0u;
            sm.vmax[x] = 0u;
            sm.emitted = 0u;
            sm.ncand = 0u;
        }
        S::sync();
    }
    // the whole workgroup finishes only a workgroup's last row: no row
    // uses the buffer after it, and the full-row passes that may follow
    // reset their own counter, so nothing is cleared (a barrier precedes
    // them)
    return deferred;
}

// ----------------------------------------------------------------------------
// the kernel
// ----------------------------------------------------------------------------

__global__ __launch_bounds__(kThreads) void topk_rows_kernel(Params p) {
    using B = BlockScope<kThreads>;
    __shared__ Shared sm;
    for (int i = threadIdx.x; i < 2 * kBins; i += kThreads) (&sm.hist[0][0])[i] = 0u;
    for (int i = threadIdx.x; i < kBins; i += kThreads) sm.shist[i] = 0u;
    if (threadIdx.x == 0) {
        sm.count[0] = sm.count[1] = 0u;
        sm.vmax[0] = sm.vmax[1] = 0u;
        sm.emitted = sm.semitted = 0u;
        sm.ncand = 0u;
        sm.ndeferred = 0u;
        sm.ndirect = 0u;
        sm.nrank = 0u;
        sm.take_cand = 0u;
        sm.pair = 0u;
        sm.n_claimed = sm.n_ready = sm.n_finished = 0u;
        sm.last_row = -1;
        sm.abort = 0u;
        for (int s = 0; s < kSlots; ++s) {
            sm.slot[s].valid = 0u;
            sm.chunk_next[s] = 0u;
            sm.left[s] = 0u;
        }
    }
    B::sync();
    const uint32_t cap = (uint32_t)p.capacity;
    const SelectLds sampler_lds{sm.shist, sm.sfound};

    // start. Workgroup w's first row is row w in every queue layout, so it
    // is known before the queue is built: its sample's loads go out first,
    // then each streaming wave's first two chunks of it (160 KB per compute
    // unit), and the whole workgroup finds row 0's cutoff from the sample
    // while the chunks are in flight. An ordered queue is only counted
    // here; the sampler wave makes its table once the roles start (while
    // row 0 streams) and claims the next rows. Otherwise the queue is dealt
    // first and the sampler wave claims the next row before the roles start.
    const int64_t b0 = blockIdx.x;  // the grid is min(batch, CUs)
    // every length load in flight before the first is used
    const bool ordered = p.batch > (int64_t)gridDim.x && queue_ordered(p.batch);
    int64_t L0 = p.n_cols;
    int64_t lens[kLenPer];
#pragma unroll
    for (int j = 0; j < kLenPer; ++j) lens[j] = p.n_cols;
    if (p.lengths != nullptr) {  // unconditional loads (clamped rows), so that one wait covers all
        L0 = p.lengths[b0];
#pragma unroll
        for (int j = 0; j < kLenPer; ++j) {
            const int64_t b = threadIdx.x + (int64_t)j * kThreads;
            lens[j] = p.lengths[b < p.batch ? b : p.batch - 1];
        }
    }
    // Row 0's sample goes out with the lengths, by waves 0 and 1 (which load
    // no chunks), laid out over the full width n_cols; its runs that lie
    // inside the row are the sample, unless they are under half of what a
    // layout over the row's own length would hold (then it is loaded again).
    const bool maybe_sampled =
        p.force_path == TOPK_PATH_SAMPLED || (p.force_path == TOPK_PATH_AUTO && p.n_cols > (int64_t)cap);
    const bool spec = maybe_sampled && (ordered || p.batch <= (int64_t)gridDim.x);
    const SamplePlan wide(p.n_cols);
    if (spec && wave_id() < 2) sample_issue_pair(p, sm, b0, wide, wave_id());
    L0 = L0 < 0 ? 0 : (L0 > p.n_cols ? p.n_cols : L0);
#pragma unroll
    for (int j = 0; j < kLenPer; ++j) {
        const int64_t b = threadIdx.x + (int64_t)j * kThreads;
        const int64_t L = lens[j] < 0 ? 0 : (lens[j] > p.n_cols ? p.n_cols : lens[j]);
        lens[j] = ordered && b < p.batch ? L : 0;
    }
    const uint32_t kind0 = L0 > p.k ? row_kind(p, L0) : kKindFull;
    const bool stream0 = L0 > p.k && kind0 != kKindFull;  // row 0 is this workgroup's first streamed row
    // Its loads go out before the queue is built when that needs no more
    // length loads: one row per workgroup, or the ordered queue.
    const bool early = stream0 && (ordered || p.batch <= (int64_t)gridDim.x);
    const bool sampled0 = early && kind0 == kKindSampled;
    const bool queue_later = ordered;  // the table is made by the sampler wave once the roles start
    const int wide_runs = wide.runs_within(L0);
    const bool wide_ok = spec && wide_runs >= 2 && 2 * wide_runs >= SamplePlan(L0).runs;
    if (stream0 && threadIdx.x == 0) {
        fill_slot(sm.slot[0], p, b0, L0, kind0);
        if (wide_ok) sm.slot[0].nsv = (uint32_t)wide_runs * (kRunLen / 4);
        sm.chunk_next[0] = early ? 2u * (uint32_t)kStreamers : 0u;
    }
    // a sample not used: wave 0's loads land before the sampler wave loads
    // another into the same LDS (wave 1's own land in order)
    if (spec && !sampled0 && wave_id() == 0) __builtin_amdgcn_s_waitcnt(kWaitVm0);
    if (queue_later) {
        queue_count(p, sm, queue_lds(sm), L0, lens);
        if (threadIdx.x == 0) sm.n_claimed = stream0 ? 1u : 0u;
        if (wave_id() == 1 && L0 > p.k && kind0 == kKindFull)
            defer_row(p, sm, sampler_lds, &sm.semitted, b0, TOPK_ROW_FULL_FORCED);
    } else {
        build_queue(p, sm, L0);
        if (wave_id() == 1) {
            if (L0 > p.k && kind0 == kKindFull) defer_row(p, sm, sampler_lds, &sm.semitted, b0, TOPK_ROW_FULL_FORCED);
            if (!stream0) claim_row(p, sm, sm.slot[0], sampler_lds, &sm.semitted);
            claim_row(p, sm, sm.slot[1], sampler_lds, &sm.semitted);
            if (lane_id() == 0) sm.n_claimed = 2u;
        }
    }
    B::sync();
    Chunk a, b;
    Streamer st{p, sm, cap, 0, kNone, -1, -1, 0u, 0u, 0};
    if (early && wave_id() >= kFirstStreamer) {
        // Each streaming wave's first two chunks of row 0, from one load
        // site each (their registers then stay where the roles use them):
        // streaming wave s takes chunks s and s + kStreamers, and a wave
        // left without its first is done with row 0. Chunks past the row
        // issue loads that touch no memory. Only streaming waves load here:
        // a wave that issues loads waits until the compute unit's memory
        // queue takes them.
        const uint32_t c0 = wave_id() - kFirstStreamer;
        const uint32_t nc0 = nchunks_of(L0);
        const uint32_t c = c0 < nc0 ? c0 : kNone;
        const uint32_t c1 = c0 + kStreamers < nc0 ? c0 + kStreamers : kNone;
        const float* row0 = p.scores + b0 * p.row_stride;
        load_chunk(a, c < kNone ? row0 : p.scores, c < kNone ? L0 : 0, c);
        load_chunk(b, c1 < kNone ? row0 : p.scores, c1 < kNone ? L0 : 0, c1);
        st.c = c;
        st.pre = c1;
        if (c == kNone) {
            st.leave(0);
            st.i = 1;
        }
    }
    // Row 0 when it comes after a queue dealt in index order: its sample,
    // then its chunks.
    const bool late = !early && sm.slot[0].valid;
    const bool late_sampled = late && sm.slot[0].kind == kKindSampled;
    if (late_sampled) sample_load<B>(p, sm, sm.slot[0]);
    if (late && wave_id() >= kFirstStreamer) {
        // after the queue: each streaming wave's first chunk of rows 0-1
        // (later rows are not claimed yet)
        st.c = st.grab(st.i, 1, false);
        if (st.c < kNone) st.load(a, st.i, st.c);
    }
    if (late_sampled) {
        B::sync();
        sample_select<B>(sm, sm.slot[0], sampler_lds);
    }
    if (sampled0) {
        // row 0's cutoff from the sample by waves 0 and 1, while the
        // streaming waves issue their chunks' loads (a wave that issues
        // loads waits until the compute unit's memory queue takes them, so
        // a cutoff found by the whole workgroup would wait for the queue)
        if (wave_id() < 2) {
            if (!wide_ok) sample_issue_pair(p, sm, b0, SamplePlan(L0), wave_id());
            __builtin_amdgcn_s_waitcnt(kWaitVm0);
            sample_select_pair(sm, sm.slot[0], sampler_lds, wave_id());
        }
    } else {
        // row 0's cutoff is set (or there is no row 0), unless the sampler
        // wave is still to claim it from the table
        if (threadIdx.x == 0 && (stream0 || !queue_later)) sm.n_ready = 1u;
        B::sync();
    }

    if (wave_id() == 0) {
        // finisher: rows in order; the last row is left to the whole workgroup
        int last = -1;
        for (int i = 0;; ++i) {
            const int s = i % kSlots;
            if (!wait_for(sm, &sm.n_claimed, (uint32_t)i + 1u) || !sm.slot[s].valid) break;
            // row i's buffer is free (rows up to i - 1 are finished); its
            // tail is filtered once its cutoff is set
            const float tail = load_tail(p, sm.slot[s]);
            if (!wait_for(sm, &sm.n_ready, (uint32_t)i + 1u)) break;
            append_tail(sm, sm.slot[s], i & 1, cap, tail);
            if (!wait_for(sm, &sm.n_claimed, (uint32_t)i + 2u)) break;
            if (!sm.slot[(i + 1) % kSlots].valid) {
                last = i;
                break;
            }
            if (!wait_for(sm, &sm.left[s], (uint32_t)kStreamers)) break;
            finish_row<WaveScope>(p, sm, sm.slot[s], i & 1, cap);
            if (lane_id() == 0) sm.left[s] = 0u;
            publish(&sm.n_finished, (uint32_t)i + 1u);
        }
        if (lane_id() == 0) sm.last_row = last;
    } else if (wave_id() == 1) {
        // sampler: the queue's table if it is still to make, the claim of
        // rows 1 (and 0, if row w was not streamed) and that row 0's cutoff;
        // then the cutoff of row j, and the claim of row j + 1, whose slot
        // held row j - 3
        // The next row's sample goes out as soon as the table's first row is
        // known (its loads wait behind the streaming waves' loads); the row
        // claimed from the table is that row unless it is deferred.
        int64_t issued = -1;  // the row whose sample is in flight
        // ahead of the streaming waves on its SIMD: the next cutoff is due
        // before the current row is streamed
        __builtin_amdgcn_s_setprio(3);
        // row 0's sample is read until its cutoff is set
        const bool alive = !sampled0 || wait_for(sm, &sm.n_ready, 1u);
        if (alive && queue_later) {
            queue_table(p, sm, queue_lds(sm), [&](int64_t b, int64_t L) {
                if (row_kind(p, L) != kKindSampled) return;
                RowSlot R;
                R.b = b;
                R.L = L;
                sample_issue<WaveScope>(p, sm, R);
                issued = b;
            });
            if (!stream0) claim_row(p, sm, sm.slot[0], sampler_lds, &sm.semitted);
            claim_row(p, sm, sm.slot[1], sampler_lds, &sm.semitted);
            publish(&sm.n_claimed, 2u);
            if (!stream0) {
                RowSlot& R0 = sm.slot[0];
                if (R0.valid && R0.kind == kKindSampled) {
                    if (R0.b != issued) sample_issue<WaveScope>(p, sm, R0);
                    __builtin_amdgcn_s_waitcnt(kWaitVm0);
                    sample_select<WaveScope>(sm, R0, sampler_lds);
                    issued = -1;
                }
                publish(&sm.n_ready, 1u);
            }
        }
        for (int j = 1; alive; ++j) {
            const int s = j % kSlots;
            if (!sm.slot[s].valid) break;
            if (sm.slot[s].kind == kKindSampled) {
                if (sm.slot[s].b != issued) sample_issue<WaveScope>(p, sm, sm.slot[s]);
                __builtin_amdgcn_s_waitcnt(kWaitVm0);
                sample_select<WaveScope>(sm, sm.slot[s], sampler_lds);
                issued = -1;
            }
            publish(&sm.n_ready, (uint32_t)j + 1u);
            if (j >= 3 && !wait_for(sm, &sm.n_finished, (uint32_t)j - 2u)) break;
            const int sn = (j + 1) % kSlots;
            if (lane_id() == 0) sm.chunk_next[sn] = 0u;
            claim_row(p, sm, sm.slot[sn], sampler_lds, &sm.semitted);
            publish(&sm.n_claimed, (uint32_t)j + 2u);
        }
        __builtin_amdgcn_s_setprio(0);
    } else {
        // streaming waves ahead of the finisher on their SIMD: its long
        // dependent chains otherwise take issue cycles from the two
        // streaming waves beside it
        __builtin_amdgcn_s_setprio(2);
        bool more = st.c < kNone;  // a chunk of row 0 or 1 issued at the start
        if (!more && st.c != kEnd) {
            st.c = st.grab(st.i, INT32_MAX, false);
            st.load(a, st.i, st.c);
            more = st.c != kEnd;
        }
        while (more) {
            more = st.step(a, b);
            if (more) more = st.step(b, a);
        }
        __builtin_amdgcn_s_setprio(0);
    }
    B::sync();
    if (sm.abort != 0u && threadIdx.x == 0) atomicAdd(&g_watchdog_trips, 1u);
    bool full_rows = sm.ndeferred != 0u;  // rows deferred while the roles ran
    if (sm.last_row >= 0 && sm.abort == 0u) {
        const int r = sm.last_row;
        full_rows |= finish_row<B>(p, sm, sm.slot[r % kSlots], r & 1, cap);
    }
    if (!full_rows) return;
    B::sync();
    const uint32_t nd = sm.ndeferred < (uint32_t)kMaxDeferred ? sm.ndeferred : (uint32_t)kMaxDeferred;
    for (uint32_t j = 0; j < nd; ++j)
        full_row<B>(p, SelectLds{sm.hist[0], sm.found}, &sm.emitted, sm.deferred[j], sm.deferred_code[j]);
}

}  // namespace
}  // namespace topk

using namespace topk;

extern "C" {

const char* topk_status_string(int status) {
    switch (status) {
        case TOPK_OK: return "ok";
        case TOPK_ERR_ARG: return "invalid argument";
        case TOPK_ERR_K: return "k outside [1, 2048]";
        case TOPK_ERR_ALIGN: return "misaligned buffer or row stride";
        case TOPK_ERR_DEVICE: return "no gfx950 device is current";
        case TOPK_ERR_LAUNCH: return "kernel launch failed";
        default: return "unknown status";
    }
}

int32_t topk_max_capacity(void) { return kCapacity; }

int32_t topk_short_capacity(void) { return kShortCapacity; }

uint32_t topk_watchdog_trips(void) {
    unsigned int n = 0;
    if (hipMemcpyFromSymbol(&n, HIP_SYMBOL(g_watchdog_trips), sizeof(n), 0, hipMemcpyDeviceToHost) != hipSuccess)
        return 0xFFFFFFFFu;
    return n;
}

int topk_select_ex(const float* scores, int64_t batch, int64_t row_stride, int64_t n_cols,
                   const int32_t* lengths, int32_t k, int32_t* out_idx,
                   const int32_t* page_table, int64_t page_table_stride, int32_t page_size,
                   void* hip_stream, const topk_options* options) {
    if (batch < 0 || batch > INT32_MAX) return TOPK_ERR_ARG;
    if (k < 1 || k > TOPK_MAX_K) return TOPK_ERR_K;
    if (n_cols < 0 || n_cols > INT32_MAX || row_stride < n_cols) return TOPK_ERR_ARG;
    topk_options opt{TOPK_PATH_AUTO, 0, nullptr, TOPK_KERNEL_AUTO};
    if (options != nullptr) opt = *options;
    if (opt.force_path < TOPK_PATH_AUTO || opt.force_path > TOPK_PATH_FULLROW) return TOPK_ERR_ARG;
    if (opt.capacity < 0 || opt.capacity > kCapacity) return TOPK_ERR_ARG;
    if (opt.kernel < TOPK_KERNEL_AUTO || opt.kernel > TOPK_KERNEL_SHORT) return TOPK_ERR_ARG;
    if (page_table != nullptr) {
        if (page_size < 1) return TOPK_ERR_ARG;
        if (page_table_stride < (n_cols + page_size - 1) / page_size) return TOPK_ERR_ARG;
    }
    // the kernel: one workgroup per row for batches of short rows (the
    // hardware scheduler filling the compute units), else the persistent one;
    // a capacity above what the short-row kernel holds needs the persistent one
    int kernel = opt.kernel;
    if (kernel == TOPK_KERNEL_AUTO)
        kernel = n_cols <= kShortMaxCols && batch <= kShortMaxBatch && opt.capacity <= kShortCapacity
                     ? TOPK_KERNEL_SHORT
                     : TOPK_KERNEL_PERSISTENT;
    if (kernel == TOPK_KERNEL_SHORT && (opt.capacity > kShortCapacity || batch > kShortMaxBatch)) return TOPK_ERR_ARG;
    if (batch == 0) return TOPK_OK;
    if (scores == nullptr || out_idx == nullptr) return TOPK_ERR_ARG;
    if ((reinterpret_cast<uintptr_t>(scores) & 15u) != 0) return TOPK_ERR_ALIGN;
    if (batch > 1 && (row_stride & 3) != 0) return TOPK_ERR_ALIGN;
    const int cus = device_cus();
    if (cus <= 0) return TOPK_ERR_DEVICE;
    if (kernel == TOPK_KERNEL_SHORT)
        return launch_short_rows(scores, batch, row_stride, n_cols, lengths, k, out_idx, page_table,
                                 page_table_stride, page_size, opt, static_cast<hipStream_t>(hip_stream));

    if (opt.capacity == 0) opt.capacity = kCapacity;
    Params p{scores, row_stride, n_cols, lengths, out_idx, page_table, page_table_stride, page_size, k,
             opt.force_path, opt.capacity, opt.row_stats, batch};
    void* args[] = {&p};
    const int64_t grid = batch < cus ? batch : cus;
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&topk_rows_kernel), dim3((uint32_t)grid),
                                         dim3(kThreads), args, 0, static_cast<hipStream_t>(hip_stream));
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
