/*
 * CPU oracle: exact per-row top-k over ragged fp32 score rows, by full sort.
 *
 * Test infrastructure only. It is loaded by tests/, by __graft_entry__.smoke()
 * and by the cpu_baseline leg of bench.py, and by nothing in the product
 * library. It shares no source, header, table or helper with the GPU path: it
 * never forms an integer sort key from the float bits, builds no histogram and
 * takes no sample. It is the plain definition of the result, written out.
 *
 * What a row selects (sources, by page and section):
 *  - "dsv4.1: Top-k kernels and candidate selection" (sglang PR #39648
 *    report), code excerpts, docstring of the bf16 top-k entry: row b selects
 *    the k best of its first seq_lens[b] scores; -1 fills every slot past
 *    min(k, seq_lens[b]); a selected index i is written as
 *    page_table[b, i / page_size] * page_size + i % page_size in paged mode;
 *    the selection is exact and only the choice among scores equal to the
 *    k-th best is free.
 *  - same page, motivation: -inf is a legal score and must not lose its slot
 *    to padding; seq_lens must be non-negative, 0 meaning no tokens.
 *  - "Fix incorrect sparse-attention top-k selection when candidate bins
 *    overflow" (sglang PR #37625), comment thread, scope update: results are
 *    judged by their exact selected-value multiset; index swaps are allowed
 *    only among equal scores.
 *  - vLLM PR #56346 report, implementation item 4: lengths of -1 and of the
 *    row width + 17 are exercised; this oracle clamps a length to [0, n_cols].
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - order: IEEE ">" on the values, with +0 ranked above -0 (a total order on
 *    non-NaN floats, so the selected multiset is unique bit for bit);
 *  - ties (equal under that order): the lower index ranks first, so the
 *    selected index set is unique too;
 *  - NaN inside [0, L) is outside the contract: the call reports it;
 *  - output order within [0, m): best first (any order is acceptable to the
 *    checker, which sorts).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    float v;
    int32_t i;
} scored_pos;

/* qsort comparator: negative when a ranks before b. */
static int rank_before(const void* pa, const void* pb) {
    const scored_pos* a = (const scored_pos*)pa;
    const scored_pos* b = (const scored_pos*)pb;
    if (a->v > b->v) return -1;
    if (a->v < b->v) return 1;
    /* IEEE-equal: identical values, or +0 against -0 */
    int sa = signbit(a->v) ? 1 : 0;
    int sb = signbit(b->v) ? 1 : 0;
    if (sa != sb) return sa - sb; /* +0 (sign 0) ranks before -0 (sign 1) */
    return (a->i > b->i) - (a->i < b->i);
}

/* Return codes */
#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_NAN 2
#define ORACLE_ERR_NOMEM 3

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * scores      [batch, row_stride] fp32, host memory
 * lengths     [batch] int32, or NULL (every row has n_cols valid scores)
 * k           slots per row, >= 1
 * page_table  [batch, page_table_stride] int32, or NULL for raw indices
 * out         [batch, k] int32, written completely
 * threads     OpenMP threads over rows for this call (0: the runtime default)
 * Rows are independent; the parallel loop only splits rows over threads.
 */
int oracle_topk(const float* scores, int64_t batch, int64_t row_stride,
                int64_t n_cols, const int32_t* lengths, int32_t k,
                const int32_t* page_table, int64_t page_table_stride,
                int32_t page_size, int32_t* out, int32_t threads) {
    if (batch < 0 || k < 1 || n_cols < 0 || row_stride < n_cols) return ORACLE_ERR_ARG;
    if (batch > 0 && (scores == NULL || out == NULL)) return ORACLE_ERR_ARG;
    if (page_table != NULL && page_size < 1) return ORACLE_ERR_ARG;
    int status = ORACLE_OK;
#ifdef _OPENMP
    /* a clause, not omp_set_num_threads: a later call with 0 gets the default again */
    const int nt = threads > 0 ? threads : omp_get_max_threads();
#else
    (void)threads;
#endif

#pragma omp parallel for num_threads(nt) schedule(dynamic, 1)
    for (int64_t b = 0; b < batch; ++b) {
        int64_t L = lengths ? (int64_t)lengths[b] : n_cols;
        if (L < 0) L = 0;
        if (L > n_cols) L = n_cols;
        int64_t m = L < (int64_t)k ? L : (int64_t)k;
        int32_t* orow = out + b * (int64_t)k;
        for (int64_t j = 0; j < k; ++j) orow[j] = -1;
        if (L == 0) continue;

        scored_pos* pos = (scored_pos*)malloc((size_t)L * sizeof(scored_pos));
        if (pos == NULL) {
#pragma omp atomic write
            status = ORACLE_ERR_NOMEM;
            continue;
        }
        const float* x = scores + b * row_stride;
        int has_nan = 0;
        for (int64_t i = 0; i < L; ++i) {
            if (isnan(x[i])) has_nan = 1;
            pos[i].v = x[i];
            pos[i].i = (int32_t)i;
        }
        if (has_nan) {
            free(pos);
#pragma omp atomic write
            status = ORACLE_ERR_NAN;
            continue;
        }
        qsort(pos, (size_t)L, sizeof(scored_pos), rank_before);
        for (int64_t j = 0; j < m; ++j) {
            int64_t i = pos[j].i;
            if (page_table == NULL) {
                orow[j] = (int32_t)i;
            } else {
                int64_t page = page_table[b * page_table_stride + i / page_size];
                orow[j] = (int32_t)(page * page_size + i % page_size);
            }
        }
        free(pos);
    }
    return status;
}
