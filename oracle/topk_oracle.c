/*
 * Oracle for column-wise vocabulary top-k -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the bench's CPU-baseline leg load
 * this file's library.  The GPU library never links, includes or calls it, and
 * it shares no code, header or table with the GPU kernels.
 *
 * What it computes (page "DFlash2" of the ignis docs, section "How it works":
 * the replacement top-k keeps the largest values first and breaks ties toward
 * the smaller row id, selecting bit-identically to the kernel it replaced):
 *
 *   For every column c, form the V pairs (x[r, c], r), r = 0 .. V-1, where
 *   x[r, c] is the stored element read as a real number.  Order the pairs by
 *     (a, ra) before (b, rb)  iff  a > b,  or  a == b and ra < rb.
 *   Row ids are distinct, so this order is strict and total and the answer is
 *   unique.  Emit the first k pairs: the stored bits of the element and its
 *   0-based row id.
 *
 * The page leaves three points open; the readings taken here are:
 *   - "a == b" is equality of real numbers: -0 equals +0 (the tie then goes
 *     to the smaller row) and subnormals compare exactly (no flushing).
 *   - NaN ranks above +Inf, and all NaNs are equal to one another (so the
 *     smaller row wins among NaNs), whatever their sign or payload.
 *   - The emitted value is the stored bit pattern, never a converted copy, so
 *     -0 stays -0 and a NaN keeps its payload.
 *
 * Method: widen every element of the column exactly to double (bf16 -> double
 * and fp32 -> double are exact), sort all V pairs with the order above using
 * the C library's qsort, keep the first k.  No blocking, no early exit, no
 * fusion: a full sort of every column, threaded over columns only.
 *
 * Layouts: column-contiguous (element (r, c) at x[c*ld + r], ld >= V) and
 * row-interleaved (element (r, c) at x[r*ld + c], ld >= C).  Elements outside
 * the V x C matrix (padding inside ld) are never read.
 *
 * Parity pins for this file live in tests/test_oracle.py.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_BF16 = 0, ORACLE_F32 = 1 };
enum { ORACLE_COL_CONTIG = 0, ORACLE_ROW_INTERLEAVED = 1 };

typedef struct {
    double value;  /* exact real value of the stored element (unused if NaN) */
    int is_nan;    /* 1 if the element is a NaN of either sign */
    int32_t row;   /* 0-based row id along the vocabulary axis */
} oracle_pair;

/* Exact real value of one stored element.  bf16 is the upper half of an IEEE
 * binary32, so shifting its 16 bits up by 16 gives the binary32 with the same
 * value; binary32 -> double is exact. */
static double element_value(const void *x, int dtype, int64_t index, int *is_nan) {
    uint32_t bits32;
    if (dtype == ORACLE_BF16) {
        uint16_t b = ((const uint16_t *)x)[index];
        bits32 = (uint32_t)b << 16;
    } else {
        bits32 = ((const uint32_t *)x)[index];
    }
    float f;
    memcpy(&f, &bits32, sizeof f);
    *is_nan = isnan(f) ? 1 : 0;
    return (double)f;
}

/* 1 if pair a comes strictly before pair b in the output order. */
static int comes_before(const oracle_pair *a, const oracle_pair *b) {
    if (a->is_nan || b->is_nan) {
        if (a->is_nan && b->is_nan) return a->row < b->row; /* NaNs tie */
        return a->is_nan;                                   /* NaN is largest */
    }
    if (a->value > b->value) return 1;
    if (a->value < b->value) return 0;
    return a->row < b->row; /* equal values (including -0 == +0) */
}

static int pair_cmp(const void *pa, const void *pb) {
    const oracle_pair *a = (const oracle_pair *)pa;
    const oracle_pair *b = (const oracle_pair *)pb;
    if (comes_before(a, b)) return -1;
    if (comes_before(b, a)) return 1;
    return 0; /* only when a and b are the same row */
}

typedef struct {
    int64_t V, C, ld;
    int32_t k;
    int dtype, layout;
    const void *x;
    void *out_values;
    int32_t *out_ids;
    int64_t col_begin, col_end;
    int failed;
} oracle_job;

static int64_t element_index(const oracle_job *j, int64_t r, int64_t c) {
    return j->layout == ORACLE_COL_CONTIG ? c * j->ld + r : r * j->ld + c;
}

static void *run_columns(void *arg) {
    oracle_job *j = (oracle_job *)arg;
    oracle_pair *pairs = (oracle_pair *)malloc((size_t)j->V * sizeof(oracle_pair));
    if (!pairs) {
        j->failed = 1;
        return NULL;
    }
    for (int64_t c = j->col_begin; c < j->col_end; ++c) {
        for (int64_t r = 0; r < j->V; ++r) {
            pairs[r].value = element_value(j->x, j->dtype, element_index(j, r, c), &pairs[r].is_nan);
            pairs[r].row = (int32_t)r;
        }
        qsort(pairs, (size_t)j->V, sizeof(oracle_pair), pair_cmp);
        for (int32_t t = 0; t < j->k; ++t) {
            int64_t src = element_index(j, pairs[t].row, c);
            int64_t dst = c * (int64_t)j->k + t;
            if (j->dtype == ORACLE_BF16)
                ((uint16_t *)j->out_values)[dst] = ((const uint16_t *)j->x)[src];
            else
                ((uint32_t *)j->out_values)[dst] = ((const uint32_t *)j->x)[src];
            j->out_ids[dst] = pairs[t].row;
        }
    }
    free(pairs);
    return NULL;
}

/*
 * Returns 0 on success, -1 on an invalid argument, -2 if memory or threads
 * could not be obtained.  Outputs: out_values[c*k + t] and out_ids[c*k + t],
 * t = 0 is the largest.  nthreads < 1 is treated as 1; threads split columns.
 */
int oracle_topk_cols(int64_t V, int64_t C, int32_t k, int dtype, int layout, int64_t ld,
                     const void *x, void *out_values, int32_t *out_ids, int nthreads) {
    if (V < 1 || C < 1 || k < 1 || (int64_t)k > V || V > INT32_MAX) return -1;
    if (dtype != ORACLE_BF16 && dtype != ORACLE_F32) return -1;
    if (layout != ORACLE_COL_CONTIG && layout != ORACLE_ROW_INTERLEAVED) return -1;
    if (layout == ORACLE_COL_CONTIG && ld < V) return -1;
    if (layout == ORACLE_ROW_INTERLEAVED && ld < C) return -1;
    if (!x || !out_values || !out_ids) return -1;
    if (nthreads < 1) nthreads = 1;
    if ((int64_t)nthreads > C) nthreads = (int)C;

    oracle_job *jobs = (oracle_job *)calloc((size_t)nthreads, sizeof(oracle_job));
    pthread_t *tids = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    char *joinable = (char *)calloc((size_t)nthreads, 1);
    if (!jobs || !tids || !joinable) {
        free(jobs);
        free(tids);
        free(joinable);
        return -2;
    }
    int status = 0;
    for (int t = 0; t < nthreads; ++t) {
        oracle_job *j = &jobs[t];
        j->V = V; j->C = C; j->ld = ld; j->k = k; j->dtype = dtype; j->layout = layout;
        j->x = x; j->out_values = out_values; j->out_ids = out_ids;
        j->col_begin = C * t / nthreads;
        j->col_end = C * (t + 1) / nthreads;
        if (nthreads == 1) {
            run_columns(j);
        } else if (pthread_create(&tids[t], NULL, run_columns, j) == 0) {
            joinable[t] = 1;
        } else {
            run_columns(j); /* could not start a thread: do the share here */
        }
    }
    for (int t = 0; t < nthreads; ++t)
        if (joinable[t]) pthread_join(tids[t], NULL);
    for (int t = 0; t < nthreads; ++t)
        if (jobs[t].failed) status = -2;
    free(jobs);
    free(tids);
    free(joinable);
    return status;
}
