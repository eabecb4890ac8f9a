/*
 * Oracle for sampling one draft token per column from its top-k -- TEST
 * INFRASTRUCTURE ONLY.  Like topk_oracle.c it is loaded only by the test
 * suite and the bench's CPU leg, and shares no code with the GPU library.
 *
 * What it computes.  The "DFlash2" page (section "Greedy coding is the best
 * case" and the last row of "The numbers") measures sampled drafting at
 * temperature 1.0, top_p 0.95 and top_k 20, but does not spell out the
 * sampler.  The reading taken is the standard one: softmax of the top-k
 * logits at temperature T, restricted to the smallest prefix of them (largest
 * first) whose probability mass reaches top_p, renormalised, then one draw by
 * inverse CDF with a uniform number from a counter-based generator.  For one
 * column, with v_0 >= v_1 >= ... >= v_{k-1} its top-k values (as the top-k
 * path emits them, largest first):
 *
 *   w_j = exp((v_j - v_0) / T)                  j = 0 .. k-1   (w_0 = 1)
 *   S_m = w_0 + w_1 + ... + w_{m-1}             summed in that order
 *   n   = the smallest m >= 1 with S_m >= top_p * S_k
 *   u   = uniform in [0, 1) from Philox4x32-10 (below)
 *   j*  = the smallest j < n with S_{j+1} > u * S_n
 *
 * and it emits j* (the position in the top-k list) and ids[j*].  If v_0 is
 * not finite (NaN, +Inf, or -Inf when the whole list is -Inf, so w is
 * undefined), j* = 0.  Every step is in IEEE double
 * with round-to-nearest; the operations and their order are fixed here so
 * that an implementation following the same steps lands on the same j*.
 *
 * exp.  The C library's exp is not used, because a last-bit difference from
 * another implementation could move j* when u * S_n falls on a boundary.
 * Instead exp(x), x <= 0, is evaluated by a fixed method: below -745 it is 0;
 * otherwise n = rint(x / ln 2) (x times the double nearest 1/ln 2),
 * r = x - n ln 2 with ln 2 split in two parts (Cody and Waite's reduction,
 * each step one fused multiply-add), the Taylor polynomial of e^r to degree
 * 13 by Horner's rule with fused multiply-adds (coefficients 1/i!, each the
 * double nearest), then ldexp by n.  Its accuracy is pinned against the
 * C library's exp in the tests (a few ulp).
 *
 * Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
 * easy as 1, 2, 3", SC 2011): a 4 x 32-bit counter and a 2 x 32-bit key; ten
 * rounds, each two 32 x 32 -> 64-bit products (multipliers 0xD2511F53 and
 * 0xCD9E8D57) whose high and low halves are mixed with the other words and
 * the key, the key bumped by the Weyl constants 0x9E3779B9 and 0xBB67AE85
 * between rounds.  Counter = (offset low, offset high, column, 0), key =
 * (seed low, seed high).  u = ((out0 << 32 | out1) >> 11) * 2^-53.
 * Pinned against the generator's published known-answer vectors.
 */
#include <math.h>
#include <stdint.h>

enum { SAMPLE_BF16 = 0, SAMPLE_F32 = 1 };

void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        const uint32_t n0 = hi1 ^ c1 ^ k0;
        const uint32_t n1 = lo1;
        const uint32_t n2 = hi0 ^ c3 ^ k1;
        const uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

double oracle_sample_exp(double x) {
    if (!(x >= -745.0)) return 0.0;  /* also -Inf */
    const double inv_ln2 = 1.4426950408889634;          /* nearest double to 1/ln 2 */
    const double ln2_hi = 6.93147180369123816490e-01;   /* ln 2, upper part */
    const double ln2_lo = 1.90821492927058770002e-10;   /* ln 2 - ln2_hi */
    const double n = rint(x * inv_ln2);
    double r = fma(-n, ln2_hi, x);
    r = fma(-n, ln2_lo, r);
    double p = 1.0 / 6227020800.0;                       /* 1/13! */
    p = fma(p, r, 1.0 / 479001600.0);                    /* 1/12! */
    p = fma(p, r, 1.0 / 39916800.0);
    p = fma(p, r, 1.0 / 3628800.0);
    p = fma(p, r, 1.0 / 362880.0);
    p = fma(p, r, 1.0 / 40320.0);
    p = fma(p, r, 1.0 / 5040.0);
    p = fma(p, r, 1.0 / 720.0);
    p = fma(p, r, 1.0 / 120.0);
    p = fma(p, r, 1.0 / 24.0);
    p = fma(p, r, 1.0 / 6.0);
    p = fma(p, r, 0.5);
    p = fma(p, r, 1.0);
    p = fma(p, r, 1.0);
    return ldexp(p, (int)n);
}

static double stored_value(const void *values, int dtype, int64_t i) {
    uint32_t b;
    float f;
    if (dtype == SAMPLE_BF16) {
        b = (uint32_t)((const uint16_t *)values)[i] << 16;
    } else {
        b = ((const uint32_t *)values)[i];
    }
    __builtin_memcpy(&f, &b, sizeof f);
    return (double)f;
}

/* One column: values[0..k) sorted largest first (stored bits of dtype). */
static int32_t sample_position(const void *values, int dtype, int64_t base, int32_t k, double temperature,
                               double top_p, uint64_t seed, uint64_t offset, uint32_t column) {
    const double v0 = stored_value(values, dtype, base);
    if (!isfinite(v0)) return 0;
    double w[64];
    double total = 0.0;
    for (int32_t j = 0; j < k; ++j) {
        const double z = (stored_value(values, dtype, base + j) - v0) / temperature;
        w[j] = oracle_sample_exp(z);
        total += w[j];
    }
    const double need = top_p * total;
    int32_t n = k;
    double s = 0.0;
    for (int32_t m = 1; m <= k; ++m) {
        s += w[m - 1];
        if (s >= need) {
            n = m;
            break;
        }
    }
    double sn = 0.0;
    for (int32_t j = 0; j < n; ++j) sn += w[j];
    const uint32_t ctr[4] = {(uint32_t)offset, (uint32_t)(offset >> 32), column, 0u};
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    oracle_philox4x32_10(ctr, key, out);
    const double u = (double)((((uint64_t)out[0] << 32) | out[1]) >> 11) * 0x1.0p-53;
    const double target = u * sn;
    double acc = 0.0;
    for (int32_t j = 0; j < n; ++j) {
        acc += w[j];
        if (acc > target) return j;
    }
    return n - 1;  /* not reached: acc reaches sn > target */
}

/* values: C*k stored elements (row c = column c's top-k, largest first);
 * ids: C*k int32.  Writes out_ids[c] = ids[c*k + j*] and out_pos[c] = j*.
 * Returns 0, or -1 for a bad argument. */
int oracle_sample_topk(const void *values, const int32_t *ids, int64_t C, int32_t k, int dtype,
                       double temperature, double top_p, uint64_t seed, uint64_t offset,
                       int32_t *out_ids, int32_t *out_pos) {
    if (!values || !ids || !out_ids || !out_pos || C < 1 || k < 1 || k > 64) return -1;
    if (dtype != SAMPLE_BF16 && dtype != SAMPLE_F32) return -1;
    if (!(temperature > 0.0) || isinf(temperature) || !(top_p > 0.0) || !(top_p <= 1.0)) return -1;
    for (int64_t c = 0; c < C; ++c) {
        const int32_t j = sample_position(values, dtype, c * k, k, temperature, top_p, seed, offset, (uint32_t)c);
        out_pos[c] = j;
        out_ids[c] = ids[c * k + j];
    }
    return 0;
}
