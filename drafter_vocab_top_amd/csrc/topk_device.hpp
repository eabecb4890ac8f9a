// Device building blocks for column-wise top-k on gfx950 (CDNA4, wave64).
//
// The selection order is the one the ignis "DFlash2" page states for its
// top-k ("How it works"): larger value first, ties to the smaller row id.
// The library reads the open points as follows: -0 equals +0, subnormals are
// exact, and NaN of any sign ranks above +Inf with all NaNs tied.
//
// Every comparison is on integers.  A stored element maps to an unsigned
// "order" (16 bits for bf16, 32 for fp32) whose integer order is that real
// order.  A candidate is a 64-bit key:
//     [63:32] order of the value
//     [31: 8] 0xFFFFFF - row     (so the smaller row is the larger key)
//     [ 7: 0] run tag            (equal for every key of one run)
// Rows are distinct within a column, so keys of one column are distinct and
// the key order is strict and total: the top-k is unique.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace topk {

constexpr int kBlock = 256;              // threads per workgroup (4 waves of 64)
constexpr int kWaves = kBlock / 64;
constexpr int kMaxK = 64;                // largest k (the wave-wide k-th search needs k <= 64)
constexpr int kCandCap = 512;            // LDS candidate slots per workgroup
constexpr uint32_t kMaxRow = 0xFFFFFFu;  // rows must fit in 24 bits

typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ keys ---

__device__ __forceinline__ uint32_t order_bf16(uint32_t b) {
    const uint32_t m = b & 0x7FFFu;
    if (m > 0x7F80u) return 0xFFFFu;                   // NaN, any sign
    return (b & 0x8000u) ? 0x8000u - m : 0x8000u + m;  // -0 and +0 both -> 0x8000
}

__device__ __forceinline__ uint32_t order_f32(uint32_t b) {
    const uint32_t m = b & 0x7FFFFFFFu;
    if (m > 0x7F800000u) return 0xFFFFFFFFu;
    return (b & 0x80000000u) ? 0x80000000u - m : 0x80000000u + m;
}

__device__ __forceinline__ uint64_t make_key(uint32_t order, uint32_t row, uint32_t tag) {
    return ((uint64_t)order << 32) | ((uint64_t)(kMaxRow - row) << 8) | (uint64_t)tag;
}
__device__ __forceinline__ uint32_t key_order(uint64_t key) { return (uint32_t)(key >> 32); }
__device__ __forceinline__ uint32_t key_row(uint64_t key) {
    return kMaxRow - (uint32_t)((key >> 8) & kMaxRow);
}
__device__ __forceinline__ uint32_t key_tag(uint64_t key) { return (uint32_t)(key & 0xFFu); }

// Per-dtype constants and helpers.
struct Bf16 {
    using storage = uint16_t;
    static constexpr int kPerVec = 8;                 // elements per 16-byte vector
    static constexpr int kOrderBits = 16;
    static constexpr uint32_t kFillDword = 0xFF80FF80u;  // two -Inf: neutral for the lane maxima
    static constexpr uint32_t kZeroOrder = 0x8000u;
    static constexpr uint32_t kNanOrder = 0xFFFFu;
    static constexpr uint32_t kSignBit = 0x8000u;
    static constexpr uint32_t kFirstNan = 0x7F81u;     // smallest positive NaN pattern
    static constexpr uint32_t kRawMask = 0xFFFFu;
    __device__ static uint32_t order(uint32_t raw) { return order_bf16(raw); }
    // Stored bits of an order value; exact except for the zero and NaN classes.
    __device__ static uint32_t bits_from_order(uint32_t o) {
        return o > 0x8000u ? o - 0x8000u : (0x8000u | (0x8000u - o));
    }
};

struct F32 {
    using storage = uint32_t;
    static constexpr int kPerVec = 4;
    static constexpr int kOrderBits = 32;
    static constexpr uint32_t kFillDword = 0xFF800000u;
    static constexpr uint32_t kZeroOrder = 0x80000000u;
    static constexpr uint32_t kNanOrder = 0xFFFFFFFFu;
    static constexpr uint32_t kSignBit = 0x80000000u;
    static constexpr uint32_t kFirstNan = 0x7F800001u;
    static constexpr uint32_t kRawMask = 0xFFFFFFFFu;
    __device__ static uint32_t order(uint32_t raw) { return order_f32(raw); }
    __device__ static uint32_t bits_from_order(uint32_t o) {
        return o > 0x80000000u ? o - 0x80000000u : (0x80000000u | (0x80000000u - o));
    }
};

// Value filter "order(raw) >= T" without computing the order, for data with no
// negative NaN: a wrap-around interval test on the raw pattern,
// ((raw - lo) mod 2^bits) <= span.
//  T above the zero class: raw in [P, +max pattern], P the smallest positive
//    raw pattern with order >= T (positive NaNs are at the top of that range).
//  T at or below the zero class: all non-negative patterns, then negative
//    patterns up to the one of magnitude (zero order - T); -0 is included.
template <class DT>
struct RawFilter {
    uint32_t lo, span;
    bool positive;  // threshold strictly above the zero class
    __device__ void set(uint32_t T) {
        if (T == 0) {  // no threshold: everything passes
            lo = 0;
            span = DT::kRawMask;
            positive = false;
        } else if (T > DT::kZeroOrder) {
            lo = (T == DT::kNanOrder) ? DT::kFirstNan : T - DT::kZeroOrder;
            span = (DT::kSignBit - 1u) - lo;
            positive = true;
        } else {
            lo = 0;
            span = (uint32_t)((0x2ull * DT::kZeroOrder - T) & DT::kRawMask);  // sign | (zero - T)
            positive = false;
        }
    }
    __device__ bool pass(uint32_t raw) const { return ((raw - lo) & DT::kRawMask) <= span; }
};

// ------------------------------------------------------ wave primitives ---

// The k-th largest (1 <= k <= 64) of one unsigned value per lane of a full
// wave: the largest t with |{lanes: v >= t}| >= k, built bit by bit from a
// ballot and a population count.  The result is wave-uniform.
template <int BITS>
__device__ __forceinline__ uint32_t wave_kth_largest(uint32_t v, uint32_t k) {
    uint32_t t = 0;
#pragma unroll
    for (int b = BITS - 1; b >= 0; --b) {
        const uint32_t cand = t | (1u << b);
        const unsigned long long m = __ballot(v >= cand);
        if ((uint32_t)__popcll(m) >= k) t = cand;
    }
    return t;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// ------------------------------------------------------ block primitives ---

// Rank selection: cand[0..cnt) are distinct keys in LDS.  The key of rank r
// (r < k, rank 0 = largest) is written to best[r].  Each key's rank is the
// number of keys above it; every lane of a wave reads the same cand[j], so
// the LDS reads are broadcasts.
__device__ __forceinline__ void rank_select(const uint64_t* cand, uint32_t cnt, uint32_t k,
                                            uint64_t* best) {
    for (uint32_t t = threadIdx.x; t < cnt; t += kBlock) {
        const uint64_t key = cand[t];
        uint32_t r = 0;
        for (uint32_t j = 0; j < cnt; ++j) r += cand[j] > key ? 1u : 0u;
        if (r < k) best[r] = key;
    }
}

// Block-wide count reduction: every thread contributes `local`; all threads
// get the total.  `slot` is a 3-entry zeroed LDS array used in rotation
// (call n uses entry n % 3), so one barrier per call suffices: after call n's
// barrier every thread has finished reading entry (n-1) % 3, which is then
// cleared for call n+2, whose additions come after call n+1's barrier.
__device__ __forceinline__ uint32_t block_sum(uint32_t local, uint32_t* slot, uint32_t& phase) {
    const uint32_t w = wave_sum(local);
    if ((threadIdx.x & 63) == 0) atomicAdd(&slot[phase], w);
    __syncthreads();
    const uint32_t total = slot[phase];
    const uint32_t stale = phase == 0 ? 2u : phase - 1u;
    if (threadIdx.x == 0) slot[stale] = 0;
    phase = phase == 2 ? 0u : phase + 1u;
    return total;
}

}  // namespace topk
