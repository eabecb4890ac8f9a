/*
 * topk_cols: column-wise top-k over a speculative drafter's vocabulary logits,
 * for AMD Instinct MI355X (gfx950).
 *
 * What it computes (ignis docs, page "DFlash2", section "How it works"):
 * for every column of a V-row logit matrix, select the k largest values and
 * their row ids, largest first, with ties broken toward the smaller row id.
 * The result is bit-identical to a plain per-column sort, so draft acceptance
 * cannot move.  A column is one draft position; the page's drafter proposes 7
 * per lane over a 248,046-token vocabulary (56 columns at eight lanes).
 *
 * The page leaves three points open.  This library reads them as follows.
 *   - Values compare as real numbers, so -0 equals +0 and a tie between them
 *     goes to the smaller row.  Subnormals compare exactly; nothing is flushed.
 *   - NaN of any sign or payload ranks above +Inf, and all NaNs tie with each
 *     other (the smaller row wins).
 *   - out_values holds the stored bit pattern of the selected element, so -0
 *     stays -0 and a NaN keeps its payload.
 *
 * Lifecycle: create a handle once per shape, run it any number of times,
 * destroy it.  All functions return a topk_status; none aborts or throws.
 */
#ifndef TOPK_COLS_H
#define TOPK_COLS_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TOPK_OK = 0,
    TOPK_ERR_INVALID_ARG = -1,  /* an argument is out of range, NULL or misaligned */
    TOPK_ERR_UNSUPPORTED = -2,  /* valid, but beyond this build's limits (k > TOPK_MAX_K, V > TOPK_MAX_V) */
    TOPK_ERR_HIP = -3,          /* a HIP runtime call failed (no device, launch error, ...) */
    TOPK_ERR_OUT_OF_MEMORY = -4, /* the workspace could not be allocated */
    TOPK_ERR_TIMEOUT = -5       /* reported by topk_cols_check: a run's cross-workgroup wait gave up */
} topk_status;

typedef enum {
    TOPK_BF16 = 0, /* bfloat16 stored as 16-bit patterns */
    TOPK_F32 = 1   /* IEEE binary32 */
} topk_dtype;

typedef enum {
    TOPK_COL_CONTIG = 0,     /* element (row r, column c) at x[c*ld + r], ld >= V */
    TOPK_ROW_INTERLEAVED = 1 /* element (row r, column c) at x[r*ld + c], ld >= C */
} topk_layout;

/* Largest k accepted. */
#define TOPK_MAX_K 64
/* Largest V accepted (row ids must fit in 24 bits). */
#define TOPK_MAX_V ((int64_t)((1 << 24) - 1))

typedef struct topk_cols *topk_cols_t;

/*
 * Create a handle for one shape on the current HIP device.
 *
 * V: rows (the vocabulary), 1 <= V <= TOPK_MAX_V.
 * C: columns (draft positions), >= 1.
 * k: 1 <= k <= V and k <= TOPK_MAX_K.
 * dtype, layout: see the enums.
 * ld: leading dimension in elements, ld >= V (column-contiguous) or ld >= C
 *     (row-interleaved).  Elements in the padding are never read.
 *
 * The handle owns a small device workspace: one partial list of k 8-byte
 * keys per column and vocabulary segment (C * segments * k keys), an error
 * word and, for the column-contiguous layout, one 128-byte line per column
 * holding a counter and the run count modulo 255, or, for the
 * row-interleaved layout, 32 4-byte bound words per column (C rounded up to
 * a multiple of 64) that the segments of a column share during a run.  Create allocates it on the
 * current device with hipMalloc, zeroes it and waits for the zeroing to
 * finish; create is not meant for the hot loop.  Every run leaves the
 * workspace ready for the next one; nothing is reset from the host.
 *
 * On any failure *out is set to NULL, and nothing stays allocated.
 * Returns TOPK_ERR_INVALID_ARG for a bad argument or a NULL out.
 * Returns TOPK_ERR_UNSUPPORTED when k > TOPK_MAX_K or V > TOPK_MAX_V, or
 * for the row-interleaved layout when C > 134,217,664.
 * Returns TOPK_ERR_HIP when there is no usable device.
 * Returns TOPK_ERR_OUT_OF_MEMORY when the allocation fails.
 */
int topk_cols_create(topk_cols_t *out, int64_t V, int64_t C, int32_t k, int32_t dtype,
                     int32_t layout, int64_t ld);

/*
 * Select the top k of every column.
 *
 * logits: device pointer to the matrix described at create.  It must be
 *         aligned to the element size.
 * out_values: device, C*k elements of the input dtype, aligned to the element
 *         size.  out_values[c*k + j] is the j-th largest of column c; j = 0 is
 *         the largest.
 * out_ids: device, C*k int32, 4-byte aligned.  out_ids[c*k + j] is the 0-based
 *         row of out_values[c*k + j].
 * stream: the HIP stream to enqueue on (0 = the null stream).
 *
 * Asynchronous: run only enqueues kernels.  It does not synchronize and does
 * not allocate.  The outputs are valid once the stream reaches this point.
 * The caller keeps ownership of all three buffers.  Runs on one handle must be
 * ordered on a single stream: the workspace serves one run at a time.  Use a
 * separate handle for each stream that runs concurrently.
 *
 * Graph capture: a run's enqueued work depends only on the handle's shape
 * and the arguments; the state that changes from run to run (the run count
 * that tags the column-contiguous layout's cross-workgroup lists) lives in
 * the workspace and is advanced by the kernels.  A run may therefore be
 * captured into a HIP graph and replayed (each replay is a run: replays
 * must not overlap each other or other runs on the handle).
 *
 * Cross-workgroup wait (column-contiguous layout): each column is merged by
 * the last of its workgroups to finish, which reads the others' lists and
 * waits, with a bound of tens of milliseconds, for any that has not landed
 * yet.  Every list was stored before its workgroup finished, so the wait
 * only covers stores still in flight and the bound is never reached in
 * normal operation.  If it were, that workgroup writes no output for the
 * column and sets the workspace's error word; topk_cols_check reports it.
 *
 * Returns TOPK_ERR_INVALID_ARG for a NULL or misaligned pointer, or a NULL
 * handle.  Returns TOPK_ERR_HIP when the launch fails.
 */
int topk_cols_run(topk_cols_t h, const void *logits, void *out_values, int32_t *out_ids,
                  hipStream_t stream);

/* Free the handle and its workspace.  NULL is accepted and returns TOPK_OK.
 * The caller must ensure no run on the handle is still in flight. */
int topk_cols_destroy(topk_cols_t h);

/*
 * Like topk_cols_run, over the first n_cols columns only (0 <= n_cols <= C):
 * a round in which fewer drafts are active than the handle was created for
 * (the "DFlash2" page, "How it works": the drafter proposes up to
 * spec.draft_tokens tokens per lane, so a round may carry fewer columns).
 * Lay the active columns out first; with a per-lane draft count, pack each
 * lane's active columns one after another and pass their total.
 *
 * Columns n_cols..C-1 of the matrix are not read, and out_values/out_ids are
 * written only in their first n_cols*k entries (same layout as
 * topk_cols_run).  n_cols = 0 enqueues nothing and returns TOPK_OK.  The
 * handle's launch decomposition (segments per column) stays the one chosen
 * at create, and the results are the same as a run on a matrix of n_cols
 * columns.  Ownership, ordering and capture rules are those of topk_cols_run.
 *
 * Returns TOPK_ERR_INVALID_ARG for n_cols < 0 or n_cols > C, and otherwise
 * as topk_cols_run.
 */
int topk_cols_run_n(topk_cols_t h, int64_t n_cols, const void *logits, void *out_values,
                    int32_t *out_ids, hipStream_t stream);

/*
 * Like topk_cols_run_n, with the row ids translated through a table: the
 * "DFlash2" page ("How it works") describes a "shortlist" head that scores
 * only the 131,072 most frequent tokens, so its row r stands for vocabulary
 * token row_to_id[r].  Selection is unchanged: values compare as for
 * topk_cols_run and ties go to the smaller ROW (shortlist position), not to
 * the smaller token id.  Only the reported id changes:
 * out_ids[c*k + j] = row_to_id[row of the j-th largest of column c].
 *
 * row_to_id: device, V int32 entries, 4-byte aligned, read-only, owned by
 *            the caller; any values (the table need not be a permutation).
 *
 * Returns TOPK_ERR_INVALID_ARG for a NULL or misaligned row_to_id, and
 * otherwise as topk_cols_run_n.
 */
int topk_cols_run_mapped(topk_cols_t h, int64_t n_cols, const void *logits, const int32_t *row_to_id,
                         void *out_values, int32_t *out_ids, hipStream_t stream);

/*
 * Sample one draft per column from its top-k list (the step after the
 * selection when the drafter samples: the "DFlash2" page measures sampled
 * drafting at temperature 1.0, top_p 0.95 and top_k 20, section "Greedy
 * coding is the best case" and the last row of "The numbers").  The page does
 * not spell out the sampler; this is the standard reading.  For column c with
 * top-k values v_0 >= ... >= v_{k-1} (values[c*k + j], largest first, as a
 * topk_cols run writes them):
 *   w_j = exp((v_j - v_0) / temperature),  S_m = w_0 + ... + w_{m-1},
 *   n   = the smallest m with S_m >= top_p * S_k   (the nucleus),
 *   u   = uniform in [0, 1) from Philox4x32-10 with counter
 *         (offset & 0xFFFFFFFF, offset >> 32, c, 0) and key
 *         (seed & 0xFFFFFFFF, seed >> 32): u = ((out0 << 32 | out1) >> 11) * 2^-53,
 *   j*  = the smallest j < n with S_{j+1} > u * S_n,
 * then out_ids[c] = ids[c*k + j*] and, if out_pos is not NULL,
 * out_pos[c] = j*.  A column whose v_0 is not finite (NaN, +Inf, -Inf) takes
 * j* = 0.  All arithmetic is IEEE double in the order written, with exp
 * evaluated by a fixed method (Cody-Waite reduction, degree-13 Taylor
 * polynomial by fused multiply-adds, ldexp), so the draw is reproducible
 * bit for bit by any implementation of these steps.  The same (seed,
 * offset, c) always gives the same u: advance offset between rounds.
 *
 * values: device, C*k elements of dtype (TOPK_BF16 or TOPK_F32), aligned to
 *         the element size; each row sorted largest first.
 * ids:    device, C*k int32 (rows, or token ids from topk_cols_run_mapped).
 * out_ids: device, C int32.  out_pos: device, C int32, or NULL.
 * All buffers are owned by the caller.  Asynchronous on stream; no
 * allocation, no synchronization, no handle.
 *
 * Returns TOPK_ERR_INVALID_ARG for a NULL or misaligned pointer, C < 1,
 * k < 1 or k > TOPK_MAX_K, an unknown dtype, temperature not finite and
 * positive, or top_p outside (0, 1]; TOPK_ERR_HIP when the launch fails.
 */
int topk_cols_sample(const void *values, const int32_t *ids, int64_t C, int32_t k, int32_t dtype,
                     double temperature, double top_p, uint64_t seed, uint64_t offset, int32_t *out_ids,
                     int32_t *out_pos, hipStream_t stream);

/* A static, human-readable name for a status code.  Never NULL. */
const char *topk_cols_status_string(int status);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the run of
 * topk_cols_run for the shape (V, C, k, dtype, layout, ld) of
 * topk_cols_create, with no handle.  Nothing is allocated: the workspace is
 * a static array of 8 MiB that each GPU the library runs on holds until the
 * process ends.  The first call on a device looks the array's address up
 * (hipGetSymbolAddress); later calls only launch kernels.
 *
 * Arguments as for topk_cols_create and topk_cols_run (all pointers device
 * pointers owned by the caller).  The launch decomposition is the one
 * topk_cols_create would choose; results are identical to a handle's.
 * Asynchronous on stream; no synchronization, no allocation.
 *
 * Every call on a GPU shares that GPU's array, which keeps what the last
 * call left: each call that completes leaves the parts that must start at
 * zero at zero, so calls of any shape and layout may follow each other on
 * one stream, or be captured and replayed.  Calls that overlap on one GPU
 * (unordered streams, overlapping replays) race: order them.  A
 * cross-workgroup wait that gives up (never in normal operation) leaves an
 * error in the array; topk_cols_check(NULL) reports it and clears the array.
 *
 * Returns the errors of topk_cols_create for a bad shape, and
 * TOPK_ERR_UNSUPPORTED when C > 4096 or the shape's workspace exceeds the
 * array (for example 248,046 x 448 bf16 rows with k = 16 needs 7.0 MiB and
 * fits); TOPK_ERR_INVALID_ARG for a NULL or misaligned pointer;
 * TOPK_ERR_HIP when there is no device or the launch fails.
 */
int topk_cols_run_noalloc(int64_t V, int64_t C, int32_t k, int32_t dtype, int32_t layout, int64_t ld,
                          const void *logits, void *out_values, int32_t *out_ids, hipStream_t stream);

/*
 * Report whether any run on the handle since the last check had a
 * cross-workgroup wait give up (see topk_cols_run).  Waits for all work on
 * the handle's device to finish (hipDeviceSynchronize) and reads the
 * handle's error word: not meant for the hot loop.  With h = NULL it checks
 * the workspace of topk_cols_run_noalloc on the current device instead.
 *
 * Returns TOPK_OK when no wait gave up.  Returns TOPK_ERR_TIMEOUT when one
 * did: the outputs of the runs since the last check are not valid, and the
 * workspace has been reset (zeroed, synchronously), so later runs are valid
 * again.  Returns TOPK_ERR_HIP when a HIP call fails (for h = NULL: also
 * when there is no device).
 */
int topk_cols_check(topk_cols_t h);

/*
 * For tests of the error path only: with on != 0, every later column-
 * contiguous run of the handle (with more than one segment per column) has
 * its merging workgroups treat every other list as not yet written and give
 * up after a few re-reads, as if a list never arrived.  Every kernel still
 * runs to completion.  topk_cols_check then returns TOPK_ERR_TIMEOUT and
 * resets the workspace.  on = 0 restores normal runs.  Returns
 * TOPK_ERR_INVALID_ARG for a NULL handle.
 */
int topk_cols_debug_fail_waits(topk_cols_t h, int32_t on);

/*
 * Like topk_cols_create, but with the vocabulary-axis split fixed to
 * `segments` workgroups per column (row segments for the interleaved layout)
 * instead of the automatic choice; 0 means automatic.  For tests and tuning:
 * the result is the same for every split.  For the column-contiguous
 * layout segments above 64, and for the row-interleaved layout segments * k
 * above 2048, return TOPK_ERR_UNSUPPORTED; negative values return
 * TOPK_ERR_INVALID_ARG.
 */
int topk_cols_create_with_segments(topk_cols_t *out, int64_t V, int64_t C, int32_t k,
                                   int32_t dtype, int32_t layout, int64_t ld, int64_t segments);

/* Kernel families of the column-contiguous layout (topk_cols_create_tuned). */
typedef enum {
    TOPK_ALGO_AUTO = 0,       /* chosen from the shape */
    TOPK_ALGO_WORKGROUP = 1,  /* a workgroup per vocabulary segment */
    TOPK_ALGO_ONE_WAVE = 3    /* one wave per column and no vocabulary split: the design that the
                                 "DFlash2" page ("How it works") replaced, kept as a baseline;
                                 never chosen automatically */
} topk_algo;

/*
 * Like topk_cols_create_with_segments, with the kernel family fixed as well
 * (column-contiguous layout; the row-interleaved layout accepts only
 * TOPK_ALGO_AUTO).  For tests and tuning: every family gives the same result.
 * TOPK_ALGO_ONE_WAVE accepts segments 0 or 1 only (else
 * TOPK_ERR_UNSUPPORTED).  An unknown algo returns TOPK_ERR_INVALID_ARG.
 */
int topk_cols_create_tuned(topk_cols_t *out, int64_t V, int64_t C, int32_t k, int32_t dtype,
                           int32_t layout, int64_t ld, int64_t segments, int32_t algo);

/*
 * Introspection for tests and benchmarks.  Writes the launch decomposition
 * chosen at create.
 * segments: workgroups per column (vocabulary-axis split) for the
 *           column-contiguous kernels, or row segments for the interleaved one.
 * blocks: total workgroups of the scan kernel (the row-interleaved layout
 *         adds a merge kernel of ceil(C / 4) workgroups).
 * workspace_bytes: device bytes owned by the handle.
 * algo: the topk_algo in use (TOPK_ALGO_AUTO for the row-interleaved layout).
 * Any output pointer may be NULL.
 */
int topk_cols_query(topk_cols_t h, int64_t *segments, int64_t *blocks, int64_t *workspace_bytes,
                    int32_t *algo);

#ifdef __cplusplus
}
#endif

#endif /* TOPK_COLS_H */
