// Helpers shared by the column-contiguous top-k kernels: 16-byte vector
// loads, element access within a vector, per-lane statistics of a pass and
// device-scope loads of published keys.
#pragma once

#include "topk_device.hpp"

namespace topk {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 load_vec(const u32x4* p) { return __builtin_nontemporal_load(p); }

// Raw pattern of element e (0 <= e < kPerVec, known at compile time).
template <class DT>
__device__ __forceinline__ uint32_t vec_elem(const u32x4& v, int e) {
    const uint32_t w = e < DT::kPerVec / 4 ? v.x
                     : e < 2 * DT::kPerVec / 4 ? v.y
                     : e < 3 * DT::kPerVec / 4 ? v.z : v.w;
    if constexpr (DT::kPerVec == 8) return (e & 1) ? (w >> 16) : (w & 0xFFFFu);
    else return w;
}

// Raw pattern of element e, e known only at run time.
template <class DT>
__device__ __forceinline__ uint32_t vec_elem_dyn(const u32x4& v, uint32_t e) {
    const uint32_t q = DT::kPerVec == 8 ? e >> 1 : e;
    const uint32_t wx = v.x, wy = v.y, wz = v.z, ww = v.w;
    const uint32_t w = q == 0 ? wx : q == 1 ? wy : q == 2 ? wz : ww;
    if constexpr (DT::kPerVec == 8) return (w >> ((e & 1u) * 16u)) & 0xFFFFu;
    else return w;
}

__device__ __forceinline__ s16x2 as_s16x2(uint32_t w) { return __builtin_bit_cast(s16x2, w); }
__device__ __forceinline__ u16x2 as_u16x2(uint32_t w) { return __builtin_bit_cast(u16x2, w); }

// Lane statistics of one pass (step 2).
//   vmax[i]: raw signed maximum of vector i (bf16: two 16-bit halves packed)
//   rep:     exact maximum order over the lane's elements, unless the lane
//            holds a negative NaN (then neg_nan is set and rep is unused)
// Invalid vector slots hold -Inf patterns, which never raise a maximum.
template <class DT, int NV>
__device__ __forceinline__ void lane_stats(const u32x4 (&d)[NV], uint32_t (&vmax)[NV],
                                           uint32_t& rep, bool& neg_nan) {
    if constexpr (DT::kPerVec == 8) {
        s16x2 smax = {-32768, -32768}, smin = {32767, 32767};
        u16x2 umax = {0, 0};
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            // Components go through scalars first: bit-casting a vector
            // component (d[i].y) directly reads the vector's first element.
            const uint32_t wx = d[i].x, wy = d[i].y, wz = d[i].z, ww = d[i].w;
            const s16x2 a = as_s16x2(wx), b = as_s16x2(wy), c = as_s16x2(wz), e = as_s16x2(ww);
            const s16x2 mx = __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                                       __builtin_elementwise_max(c, e));
            const s16x2 mn = __builtin_elementwise_min(__builtin_elementwise_min(a, b),
                                                       __builtin_elementwise_min(c, e));
            const u16x2 ux = __builtin_elementwise_max(
                __builtin_elementwise_max(as_u16x2(wx), as_u16x2(wy)),
                __builtin_elementwise_max(as_u16x2(wz), as_u16x2(ww)));
            vmax[i] = __builtin_bit_cast(uint32_t, mx);
            smax = __builtin_elementwise_max(smax, mx);
            smin = __builtin_elementwise_min(smin, mn);
            umax = __builtin_elementwise_max(umax, ux);
        }
        const int M = max_i32((int)smax.x, (int)smax.y);
        const int m = min_i32((int)smin.x, (int)smin.y);
        rep = M >= 0 ? order_bf16((uint32_t)M) : order_bf16((uint32_t)m & 0xFFFFu);
        neg_nan = max_u32((uint32_t)umax.x, (uint32_t)umax.y) > 0xFF80u;
    } else {
        int smax = INT32_MIN, smin = INT32_MAX;
        uint32_t umax = 0;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const uint32_t wx = d[i].x, wy = d[i].y, wz = d[i].z, ww = d[i].w;
            const int a = (int)wx, b = (int)wy, c = (int)wz, e = (int)ww;
            const int mx = max_i32(max_i32(a, b), max_i32(c, e));
            vmax[i] = (uint32_t)mx;
            smax = max_i32(smax, mx);
            smin = min_i32(smin, min_i32(min_i32(a, b), min_i32(c, e)));
            umax = max_u32(umax, max_u32(max_u32(wx, wy), max_u32(wz, ww)));
        }
        rep = smax >= 0 ? order_f32((uint32_t)smax) : order_f32((uint32_t)smin);
        neg_nan = umax > 0xFF800000u;
    }
}

// Signed maximum held in a vmax entry.
template <class DT>
__device__ __forceinline__ int vec_max_signed(uint32_t vm) {
    if constexpr (DT::kPerVec == 8) {
        const s16x2 h = as_s16x2(vm);
        return max_i32((int)h.x, (int)h.y);
    } else {
        return (int)vm;
    }
}

// Device-scope load of a published key (bypasses the non-coherent L2).
__device__ __forceinline__ uint64_t load_published(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A lower bound of the k-th largest of the lanes' orders for thresholds:
// exact for 16-bit orders; for 32-bit orders the search runs on the upper 16
// bits and the bound is rounded down to a multiple of 2^16 (half the rounds,
// and rounding down keeps it a lower bound).
template <class DT>
__device__ __forceinline__ uint32_t wave_kth_bound(uint32_t order, uint32_t k) {
    if (k == 1) return wave_max_u32(order);  // exact, every dtype
    if constexpr (DT::kOrderBits == 16) return wave_kth_largest<16>(order, k);
    else return wave_kth_largest<16>(order >> 16, k) << 16;
}

// Rank of two keys per lane among n <= 128 LDS keys (key a for slot lane,
// key b for slot lane + 64; n8 is n rounded up to 8, the padding zero): one
// pass over the keys counts, for both, how many are larger.
__device__ __forceinline__ void lds_rank2_of(const uint64_t* keys, uint32_t n8, uint64_t a, uint64_t b,
                                             uint32_t& ra, uint32_t& rb) {
    uint32_t a0 = 0, a1 = 0, b0 = 0, b1 = 0;
    for (uint32_t j = 0; j < n8; j += 8) {
        const u64x2 q0 = *reinterpret_cast<const u64x2*>(keys + j);
        const u64x2 q1 = *reinterpret_cast<const u64x2*>(keys + j + 2);
        const u64x2 q2 = *reinterpret_cast<const u64x2*>(keys + j + 4);
        const u64x2 q3 = *reinterpret_cast<const u64x2*>(keys + j + 6);
        a0 += (uint32_t)(q0.x > a) + (uint32_t)(q0.y > a) + (uint32_t)(q1.x > a) + (uint32_t)(q1.y > a);
        a1 += (uint32_t)(q2.x > a) + (uint32_t)(q2.y > a) + (uint32_t)(q3.x > a) + (uint32_t)(q3.y > a);
        b0 += (uint32_t)(q0.x > b) + (uint32_t)(q0.y > b) + (uint32_t)(q1.x > b) + (uint32_t)(q1.y > b);
        b1 += (uint32_t)(q2.x > b) + (uint32_t)(q2.y > b) + (uint32_t)(q3.x > b) + (uint32_t)(q3.y > b);
    }
    ra = a0 + a1;
    rb = b0 + b1;
}

// The j-th largest of one value per lane, j = 1 or 2, by wave maxima: the
// second is the maximum once one lane holding the first is set aside.
__device__ __forceinline__ uint32_t wave_top12(uint32_t v, uint32_t j) {
    const uint32_t m = wave_max_u32(v);
    if (j == 1) return m;
    const uint32_t first = (uint32_t)__builtin_ctzll(__ballot(v == m));
    return wave_max_u32((threadIdx.x & 63u) == first ? 0u : v);
}

}  // namespace topk
