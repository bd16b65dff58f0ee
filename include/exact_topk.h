/*
 * exact_topk.h -- C ABI of the gfx950 library for exact per-row top-k over
 * long, ragged fp32 score rows (the decode-time selection of a sparse-
 * attention indexer).
 *
 * The operation (sources by page and section):
 *  - "dsv4.1: Top-k kernels and candidate selection" (sglang PR #39648
 *    report), code excerpts, docstring of the bf16 top-k entry: row b selects
 *    the k best of its first lengths[b] scores, in no particular order; -1
 *    fills every slot past min(k, lengths[b]); in paged mode a selected index
 *    i is written as page_table[b, i / page_size] * page_size + i % page_size;
 *    k is at most 2048.
 *  - same page, motivation: -inf is a legal score and is selected like any
 *    other; lengths are non-negative, 0 meaning an idle row.
 *  - "Fix incorrect sparse-attention top-k selection when candidate bins
 *    overflow" (sglang PR #37625), modifications and comment thread: the
 *    selected-value multiset is exact even when one coarse bin holds more
 *    candidates than any buffer; only equal scores may trade places.
 *  - vLLM PR #56346 report, implementation items 1-3: one launch serves long
 *    and short rows, and lengths stay on the device.
 *
 * Result, exactly: with L = clamp(lengths[b], 0, n_cols) and m = min(k, L),
 * slots [0, m) of out row b hold the m positions of [0, L) that rank first
 * by value (descending; +0 above -0; among equal values the lower index
 * first), in an unspecified order, and slots [m, k) hold -1. Because equal
 * values go to the lower index, the selected set is unique: every call, and
 * every internal path, returns the same set.
 *
 * Memory: every pointer argument is a DEVICE pointer owned by the caller.
 * The library allocates, frees and retains nothing (one device word counts
 * watchdog trips, see topk_watchdog_trips); it reads scores[b, 0:L),
 * lengths[0:batch) and the page-table entries of pages that hold a selected
 * position, and writes only out_idx[0:batch, 0:k) (and row_stats).
 *
 * Calls are asynchronous on `hip_stream` (a hipStream_t; NULL = the default
 * stream) and never synchronise. Each call of topk_select is one launch on
 * that stream: for n_cols <= 32768 (and no forced path or capacity), one
 * workgroup per row with the row's survivors in LDS; otherwise a persistent
 * kernel with one workgroup per compute unit, whose LDS (about 157 KB) leaves
 * room for no other workgroup on the unit while it runs.
 * Argument errors are returned synchronously
 * as a status code before anything is launched; device data (lengths, page
 * table contents) is never an error: lengths are clamped to [0, n_cols].
 * NaN inside [0, L) is outside the contract: the call stays memory-safe, but
 * which positions it selects is unspecified. Calls are safe from several host
 * threads.
 */
#ifndef EXACT_TOPK_H
#define EXACT_TOPK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define TOPK_OK 0
#define TOPK_ERR_ARG 1    /* negative or oversized size, row_stride < n_cols, NULL data pointer,
                             page_size < 1 or page_table_stride too small, bad option value */
#define TOPK_ERR_K 2      /* k outside [1, TOPK_MAX_K] */
#define TOPK_ERR_ALIGN 3  /* scores not 16-byte aligned, or row_stride % 4 != 0 with batch > 1 */
#define TOPK_ERR_DEVICE 4 /* no device is current, or the current one is not a gfx950 (the
                             library holds gfx950 code only); pointers are not inspected */
#define TOPK_ERR_LAUNCH 5 /* the HIP launch itself failed */

#define TOPK_MAX_K 2048

/* internal paths (for topk_options.force_path and row statistics) */
#define TOPK_PATH_AUTO 0
#define TOPK_PATH_LDS 1      /* every position kept in LDS, exact select there (rows <= capacity) */
#define TOPK_PATH_SAMPLED 2  /* sampled cutoff, one streaming pass, exact select on survivors */
#define TOPK_PATH_FULLROW 3  /* full-row exact: histogram-only passes, one emission pass */

/* kernels (for topk_options.kernel) */
#define TOPK_KERNEL_AUTO 0        /* topk_select's choice (see topk_select_ex) */
#define TOPK_KERNEL_PERSISTENT 1  /* one workgroup per compute unit, rows in turn */
#define TOPK_KERNEL_SHORT 2       /* one workgroup per row, survivors in LDS */

/* row statistics codes, written to row_stats[2*b] */
#define TOPK_ROW_EMPTY 0          /* m == 0: every slot -1 */
#define TOPK_ROW_ALL 1            /* L <= k: every position selected */
#define TOPK_ROW_LDS 2            /* every position held in LDS */
#define TOPK_ROW_SAMPLED 3        /* sampled cutoff, selected among the survivors */
#define TOPK_ROW_FULL_OVERFLOW 4  /* sampled survivors exceeded the capacity */
#define TOPK_ROW_FULL_UNDERFLOW 5 /* fewer sampled survivors than m */
#define TOPK_ROW_FULL_FORCED 6    /* full-row path chosen by the caller, or LDS forced on a row above capacity */

/*
 * topk_select -- exact top-k of every row.
 *
 *  scores             fp32 [batch, row_stride], row-major; 16-byte aligned base and
 *                     row_stride % 4 == 0 (when batch > 1)
 *  batch              rows, 0 <= batch <= INT32_MAX (0: no-op, TOPK_OK)
 *  row_stride         elements between row starts, >= n_cols
 *  n_cols             largest valid length, 0 <= n_cols <= INT32_MAX
 *  lengths            int32 [batch] valid scores per row, or NULL (all rows n_cols);
 *                     values are clamped to [0, n_cols]
 *  k                  slots per row, 1 <= k <= TOPK_MAX_K
 *  out_idx            int32 [batch, k], contiguous
 *  page_table         int32 [batch, page_table_stride] or NULL for raw positions
 *  page_table_stride  elements between page-table rows, >= ceil(n_cols / page_size)
 *  page_size          positions per page, >= 1 when page_table is given
 *  hip_stream         hipStream_t to launch on
 * Returns TOPK_OK or an error code (TOPK_ERR_ARG, TOPK_ERR_K, TOPK_ERR_ALIGN,
 * TOPK_ERR_DEVICE, TOPK_ERR_LAUNCH); on error nothing was launched.
 * The caller keeps slot values inside int32 (page * page_size + offset).
 */
int topk_select(const float* scores, int64_t batch, int64_t row_stride, int64_t n_cols,
                const int32_t* lengths, int32_t k, int32_t* out_idx,
                const int32_t* page_table, int64_t page_table_stride, int32_t page_size,
                void* hip_stream);

/*
 * Diagnostic and test controls for topk_select_ex. A zeroed struct (or a NULL
 * pointer) gives exactly topk_select. The selected set never depends on them:
 * every path of every kernel returns the same unique set, so they exist to
 * reach each path on chosen rows (the forced-backend audit of the vLLM PR
 * #56346 report, discussion).
 *  force_path  TOPK_PATH_* for every row with k < L (rows with L <= k take the
 *              direct path); LDS forced on a row longer than the capacity runs
 *              the full-row path instead (row code TOPK_ROW_FULL_FORCED);
 *              SAMPLED forced on a row too short to sample (fewer than 256
 *              scores) keeps every score under a cutoff of 0
 *  capacity    survivor capacity in entries (0 = the kernel's maximum):
 *              1..topk_max_capacity() for the persistent kernel,
 *              1..topk_short_capacity() for the short-row kernel; a small
 *              value makes the overflow fallback easy to reach, and rows of
 *              at most `capacity` scores keep every score on the automatic path
 *  row_stats   device int32 [batch, 2] or NULL: [2b] = TOPK_ROW_* code,
 *              [2b+1] = survivors of the streaming pass (or L on the other paths)
 *  kernel      TOPK_KERNEL_*: AUTO takes the short-row kernel when
 *              n_cols <= 32768 and capacity <= topk_short_capacity(), else the
 *              persistent kernel; SHORT with a capacity above
 *              topk_short_capacity() is TOPK_ERR_ARG. Either kernel takes any
 *              width; the short-row kernel sends rows whose survivors
 *              overflow its buffer to the full-row path.
 */
typedef struct topk_options {
    int32_t force_path;
    int32_t capacity;
    int32_t* row_stats;
    int32_t kernel;
} topk_options;

int topk_select_ex(const float* scores, int64_t batch, int64_t row_stride, int64_t n_cols,
                   const int32_t* lengths, int32_t k, int32_t* out_idx,
                   const int32_t* page_table, int64_t page_table_stride, int32_t page_size,
                   void* hip_stream, const topk_options* options);

/* Human-readable name of a status code (static storage, never NULL). */
const char* topk_status_string(int status);

/* Largest survivor capacity of the persistent kernel (entries held in one
 * LDS buffer). */
int32_t topk_max_capacity(void);

/* Largest survivor capacity of the short-row kernel (entries held in LDS per
 * row). */
int32_t topk_short_capacity(void);

/*
 * Workgroups that gave up a wait between their roles since the library was
 * loaded, on the current device. Each wait is bounded (10 s) so that a defect
 * ends the launch instead of hanging the GPU; a nonzero count means outputs
 * of that launch are wrong. Synchronous (copies one word from the device);
 * 0xFFFFFFFF if the copy fails.
 */
uint32_t topk_watchdog_trips(void);

/*
 * Split-row mode, for batches with fewer rows than the GPU has compute units
 * (the cluster-split rows of "dsv4.1: Top-k kernels and candidate selection",
 * implementation section 4, where several blocks share one long row).
 * Same result as topk_select, bit for bit and index for index; each row is
 * cut into pieces of equal size, one workgroup each, so a small batch still
 * reads with the whole chip. Three launches on `hip_stream`:
 *  1. one workgroup per row writes rows with L <= k directly and finds the
 *     other rows' sampled cutoff keys;
 *  2. one workgroup per piece appends the piece's scores at or above the
 *     cutoff to the row's area of `workspace`;
 *  3. one workgroup per row selects the exact top m from there, or runs the
 *     full-row exact selection when the survivors overflow the area (the
 *     capacity) or fall short of m.
 *
 *  workspace        device memory owned by the caller, 256-byte aligned,
 *                   at least topk_split_workspace_bytes(batch) bytes; its
 *                   contents need no initialisation and are scratch between
 *                   calls. Calls that overlap in time must not share one.
 *  workspace_bytes  its size in bytes
 *  pieces           workgroups per row wanted, 0 = about four workgroups per
 *                   compute unit over the batch, at most 256; each piece is a
 *                   whole number of 8192-score rounds, so short rows get
 *                   fewer pieces. With 0, a batch of at least four rows per
 *                   compute unit (one piece per row) runs as topk_select_ex
 *                   does, one workgroup per row in one launch, and the
 *                   workspace is not touched (unless options set a
 *                   capacity: then the split kernels run)
 *  options          as for topk_select_ex, with capacity up to
 *                   topk_split_capacity() and kernel TOPK_KERNEL_AUTO (this
 *                   entry has its own kernels); TOPK_PATH_LDS keeps every score of
 *                   rows up to the capacity (others take the full-row path);
 *                   row_stats codes as for topk_select_ex (TOPK_ROW_LDS: every
 *                   score was kept). NULL = automatic.
 * Other arguments, results and status codes as for topk_select;
 * TOPK_ERR_ARG also for a NULL or too small workspace, and TOPK_ERR_ALIGN for
 * a workspace that is not 256-byte aligned.
 */
int topk_select_split(const float* scores, int64_t batch, int64_t row_stride, int64_t n_cols,
                      const int32_t* lengths, int32_t k, int32_t* out_idx,
                      const int32_t* page_table, int64_t page_table_stride, int32_t page_size,
                      void* workspace, int64_t workspace_bytes, int32_t pieces, void* hip_stream,
                      const topk_options* options);

/*
 * topk_select_split for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same three launches and the same result, with the workspace taken from
 * a fixed device array inside the library instead of from the caller. The
 * array holds TOPK_SPLIT_NOALLOC_MAX_BATCH rows (about 16 MiB); each GPU the
 * library runs this entry on keeps its own copy until the process ends. The
 * entry allocates and frees nothing; its first call on a device looks the
 * array's address up once.
 *
 * Every call on one GPU shares that GPU's array: calls whose launches can
 * overlap in time on one GPU (other streams, other host threads) race and
 * give wrong results; calls ordered on one stream are safe. The array needs
 * no clearing: each call writes every word it later reads.
 *
 * Arguments, results and status codes as for topk_select_split, without
 * workspace and workspace_bytes; TOPK_ERR_ARG for batch above
 * TOPK_SPLIT_NOALLOC_MAX_BATCH, TOPK_ERR_DEVICE when no gfx950 device is
 * current or the array's address cannot be found.
 */
#define TOPK_SPLIT_NOALLOC_MAX_BATCH 256

int topk_select_split_noalloc(const float* scores, int64_t batch, int64_t row_stride, int64_t n_cols,
                              const int32_t* lengths, int32_t k, int32_t* out_idx,
                              const int32_t* page_table, int64_t page_table_stride, int32_t page_size,
                              int32_t pieces, void* hip_stream, const topk_options* options);

/* Workspace bytes topk_select_split needs for `batch` rows (-1 if batch is
 * negative or above INT32_MAX): a 16-byte header per row, then
 * topk_split_capacity() 8-byte survivor entries per row. */
int64_t topk_split_workspace_bytes(int64_t batch);

/* Survivor entries per row in the split-row workspace (8192). */
int32_t topk_split_capacity(void);

/*
 * Exact top-k of bf16 rows ("dsv4.1: Top-k kernels and candidate selection",
 * implementation section 2 and code excerpts, docstring of the bf16
 * small-row top-k: rows of at most 16384 scores, k at most 2048, selection
 * exact, -1 past min(k, lengths[b]), optional page-table transform, no NaN).
 * The result is topk_select's on the exactly widened fp32 rows: same order
 * (+0 above -0), same lowest-index ties, same set. One workgroup per row.
 *
 *  scores     bf16 bit patterns [batch, row_stride]; 16-byte aligned base
 *             and row_stride % 8 == 0 (when batch > 1)
 *  n_cols     at most 16384 (TOPK_ERR_ARG above)
 *  batch      at most 16777215 (one 256-thread workgroup per row; TOPK_ERR_ARG above)
 * Other arguments, results and status codes as for topk_select.
 */
int topk_select_bf16(const uint16_t* scores, int64_t batch, int64_t row_stride, int64_t n_cols,
                     const int32_t* lengths, int32_t k, int32_t* out_idx,
                     const int32_t* page_table, int64_t page_table_stride, int32_t page_size,
                     void* hip_stream);

/*
 * topk_select_bf16 with the diagnostic controls of topk_select_ex (the same
 * audit: every path of the bf16 kernel reached on chosen rows). kernel must
 * be TOPK_KERNEL_AUTO or TOPK_KERNEL_SHORT (bf16 rows have only the short-row
 * kernel); capacity up to topk_short_capacity(). Same result for any options.
 */
int topk_select_bf16_ex(const uint16_t* scores, int64_t batch, int64_t row_stride, int64_t n_cols,
                        const int32_t* lengths, int32_t k, int32_t* out_idx,
                        const int32_t* page_table, int64_t page_table_stride, int32_t page_size,
                        void* hip_stream, const topk_options* options);

/*
 * Block keys for the first stage of the two-level indexer (same page,
 * implementation section 2, the block-max kernel, and its amax8_varlen entry
 * among the code excerpts, whose name and argument order are kept).
 * For row b with L = clamp(lengths[b], 0, n_cols) and nb = ceil(L / 8):
 * out[b, i] = the largest of scores[b, 8i .. 8i+7] for i < nb - 1, NaN
 * ignored and +0 above -0 (a block of NaN only gives +qNaN 0x7FC00000);
 * out[b, nb - 1] = +inf (the newest block is always selected); nothing is
 * written past nb. With topk > 0 a row with nb <= topk is left untouched.
 *
 *  scores      fp32 [batch, row_stride]; 32-byte aligned base and
 *              row_stride % 8 == 0 (when batch > 1)
 *  lengths     int32 [batch] or NULL (every row n_cols)
 *  topk        0 (never skip) or the number of blocks the caller selects
 *  out         fp32 [batch, out_stride], out_stride >= ceil(n_cols / 8);
 *              device memory owned by the caller
 * Returns TOPK_OK, TOPK_ERR_ARG (sizes, topk < 0, NULL, out_stride too
 * small), TOPK_ERR_ALIGN, TOPK_ERR_DEVICE or TOPK_ERR_LAUNCH. Asynchronous
 * on hip_stream.
 */
int amax8_varlen(const float* scores, int64_t batch, int64_t row_stride, int64_t n_cols,
                 const int32_t* lengths, int32_t topk, float* out, int64_t out_stride,
                 void* hip_stream);

/*
 * Block table for the second stage of the two-level indexer (same page,
 * implementation section 2, the candidate-block-table kernel, and its
 * sort_candidate_blocks entry among the code excerpts). For row b with
 * nb = ceil(clamp(lengths[b], 0, n_cols) / 8) (a length past n_cols counts as
 * n_cols, as everywhere in this library):
 *  - nb <= k: blocks[b] becomes 0 .. nb-1, then INT32_MAX (input unread);
 *  - otherwise: the distinct ids among blocks[b, 0..k) that lie in [0, nb),
 *    ascending, then INT32_MAX (a top-k selection gives k distinct ids);
 *  - out_pages[b, j] = page_table[b, id / bpp] * bpp + id % bpp for each id of
 *    the table, bpp = page_size / 8, INT32_MAX where the table is padded.
 *
 *  blocks             int32 [batch, k] contiguous, rewritten in place
 *  n_cols             largest length in positions, at most 2^21
 *  page_table         int32 [batch, page_table_stride],
 *                     page_table_stride >= ceil(ceil(n_cols / 8) / bpp)
 *  page_size          a power of two, at least 8
 *  out_pages          int32 [batch, k] contiguous
 * Returns TOPK_OK, TOPK_ERR_ARG, TOPK_ERR_DEVICE or TOPK_ERR_LAUNCH.
 * Asynchronous on hip_stream. The caller keeps pool slots inside int32.
 */
int sort_candidate_blocks(int32_t* blocks, int64_t batch, int32_t k, const int32_t* lengths,
                          int64_t n_cols, const int32_t* page_table, int64_t page_table_stride,
                          int32_t page_size, int32_t* out_pages, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_TOPK_H */
