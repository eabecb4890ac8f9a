// Sampling one draft per column from its top-k list, for gfx950.
//
// The ignis "DFlash2" page measures sampled drafting at temperature 1.0,
// top_p 0.95 and top_k 20 ("Greedy coding is the best case"; last row of
// "The numbers") without spelling out the sampler.  This kernel implements
// the standard reading.  For a column whose top-k values are
// v_0 >= ... >= v_{k-1} (largest first, as the top-k kernels emit them):
//   w_j = exp((v_j - v_0) / T),  S_m = w_0 + ... + w_{m-1} (in that order),
//   n = the smallest m with S_m >= top_p * S_k,
//   u = a uniform in [0, 1) from Philox4x32-10,
//   j* = the smallest j < n with S_{j+1} > u * S_n,
// and the output is ids[j*] (and j*).  A column whose top value is not
// finite takes j* = 0.
//
// The draw is an integer decided by floating point, so every step is IEEE
// double in a fixed order, with no contraction of separate operations into
// fused ones, and exp is evaluated by a fixed method instead of the device
// library's: reduction x = n ln 2 + r (n = rint(x / ln 2), ln 2 in two
// parts, Cody and Waite's scheme with fused multiply-adds), the degree-13
// Taylor polynomial of e^r by Horner's rule with fused multiply-adds, then
// ldexp by n; 0 below -745.  Philox4x32-10 is the counter-based generator of
// Salmon, Moraes, Dror and Shaw ("Parallel random numbers: as easy as 1, 2,
// 3", SC 2011): counter (offset low, offset high, column, 0), key (seed low,
// seed high), ten rounds; u = ((out0 << 32 | out1) >> 11) * 2^-53.
//
// One wave per column.  Lane j computes w_j (one exp per lane, in
// parallel); the sums must keep the sequential order, so every lane then
// walks j = 0 .. k-1 with w_j broadcast from lane j and adds it when j <= its
// own index: lane m ends with S_{m+1}, summed in exactly the order above.
// Ballots find n and j*.
#include "topk_device.hpp"
#include "topk_internal.hpp"

namespace topk {

namespace {

constexpr int kSampleThreads = 256;
constexpr int kSampleWaves = kSampleThreads / 64;  // one column per wave

__device__ __forceinline__ void philox4x32_10(uint32_t (&c)[4], uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint32_t lo0 = 0xD2511F53u * c[0], hi0 = __umulhi(0xD2511F53u, c[0]);
        const uint32_t lo1 = 0xCD9E8D57u * c[2], hi1 = __umulhi(0xCD9E8D57u, c[2]);
        const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
        c[0] = n0;
        c[1] = lo1;
        c[2] = n2;
        c[3] = lo0;
    }
}

__device__ __forceinline__ double fixed_exp(double x) {
#pragma clang fp contract(off)
    if (!(x >= -745.0)) return 0.0;
    const double inv_ln2 = 1.4426950408889634;
    const double ln2_hi = 6.93147180369123816490e-01;
    const double ln2_lo = 1.90821492927058770002e-10;
    const double n = __builtin_rint(x * inv_ln2);
    double r = __builtin_fma(-n, ln2_hi, x);
    r = __builtin_fma(-n, ln2_lo, r);
    double p = 1.0 / 6227020800.0;
    p = __builtin_fma(p, r, 1.0 / 479001600.0);
    p = __builtin_fma(p, r, 1.0 / 39916800.0);
    p = __builtin_fma(p, r, 1.0 / 3628800.0);
    p = __builtin_fma(p, r, 1.0 / 362880.0);
    p = __builtin_fma(p, r, 1.0 / 40320.0);
    p = __builtin_fma(p, r, 1.0 / 5040.0);
    p = __builtin_fma(p, r, 1.0 / 720.0);
    p = __builtin_fma(p, r, 1.0 / 120.0);
    p = __builtin_fma(p, r, 1.0 / 24.0);
    p = __builtin_fma(p, r, 1.0 / 6.0);
    p = __builtin_fma(p, r, 0.5);
    p = __builtin_fma(p, r, 1.0);
    p = __builtin_fma(p, r, 1.0);
    return __builtin_ldexp(p, (int)n);
}

template <class DT>
__device__ __forceinline__ double stored_value(const typename DT::storage* v, int64_t i) {
    uint32_t b = (uint32_t)v[i];
    if constexpr (DT::kPerVec == 8) b <<= 16;  // bf16: the upper half of a binary32
    return (double)__builtin_bit_cast(float, b);
}

__device__ __forceinline__ double lane_value(double x, int lane) {
    const uint64_t b = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), lane);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ uint32_t first_lane(unsigned long long mask) {
    return (uint32_t)__builtin_ctzll(mask);
}

template <class DT>
__global__ __launch_bounds__(kSampleThreads) void topk_sample_kernel(SampleArgs a) {
#pragma clang fp contract(off)
    using storage = typename DT::storage;
    const uint32_t lane = threadIdx.x & 63u;
    const int64_t c = (int64_t)blockIdx.x * kSampleWaves + (threadIdx.x >> 6);
    if (c >= a.C) return;  // wave-uniform
    const int32_t k = a.k;
    const storage* v = static_cast<const storage*>(a.values) + c * k;
    uint32_t pick = 0;
    const double v0 = stored_value<DT>(v, 0);
    if (__builtin_isfinite(v0)) {
        const bool in = (int32_t)lane < k;
        const double w = in ? fixed_exp((stored_value<DT>(v, lane) - v0) / a.temperature) : 0.0;
        double acc = 0.0;  // S_{lane+1} (S_k for lanes >= k)
        for (int32_t j = 0; j < k; ++j) {
            const double wj = lane_value(w, j);
            if (j <= (int32_t)lane) acc = acc + wj;
        }
        const double total = lane_value(acc, k - 1);
        const double need = a.top_p * total;
        const unsigned long long reach = __ballot(in && acc >= need);
        const uint32_t n = reach ? first_lane(reach) + 1u : (uint32_t)k;  // lane k-1 always reaches
        const double sn = lane_value(acc, (int)n - 1);
        uint32_t ctr[4] = {(uint32_t)a.offset, (uint32_t)(a.offset >> 32), (uint32_t)c, 0u};
        philox4x32_10(ctr, (uint32_t)a.seed, (uint32_t)(a.seed >> 32));
        const double u = (double)((((uint64_t)ctr[0] << 32) | ctr[1]) >> 11) * 0x1.0p-53;
        const double target = u * sn;
        const unsigned long long above = __ballot(lane < n && acc > target);
        pick = above ? first_lane(above) : n - 1u;  // u < 1 makes lane n-1 pass
    }
    if (lane == 0) {
        a.out_ids[c] = a.ids[c * k + pick];
        if (a.out_pos) a.out_pos[c] = (int32_t)pick;
    }
}

}  // namespace

hipError_t launch_sample(int dtype, const SampleArgs& a, hipStream_t stream) {
    const dim3 grid((uint32_t)((a.C + kSampleWaves - 1) / kSampleWaves)), block(kSampleThreads);
    if (dtype == 0)
        hipLaunchKernelGGL(topk_sample_kernel<Bf16>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(topk_sample_kernel<F32>, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace topk
