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
//     [ 7: 0] run tag            (equal for every key of one run; the
//                                 column kernel's cross-workgroup lists)
// Rows are distinct within a column, so keys of one column are distinct and
// the key order is strict and total: the top-k is unique.  No element has
// order 0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace topk {

constexpr int kBlock = 256;              // threads per workgroup (4 waves of 64)
constexpr int kWaves = kBlock / 64;
constexpr int kMaxK = 64;                // largest k (the wave-wide k-th search needs k <= 64)
constexpr uint32_t kMaxRow = 0xFFFFFFu;  // rows must fit in 24 bits

typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Typed minimum/maximum.  (The generic max/min overloads can resolve mixed
// 64-bit integer arguments to the double-precision versions, which is slow
// and rounds 64-bit keys.)
__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t max_u32(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t min_u32(uint32_t a, uint32_t b) { return a < b ? a : b; }
__device__ __forceinline__ int max_i32(int a, int b) { return a > b ? a : b; }
__device__ __forceinline__ int min_i32(int a, int b) { return a < b ? a : b; }

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
            // above the order of +Inf only NaNs qualify (a rounded-down bound
            // may fall between the two)
            lo = (T > DT::kZeroOrder + (DT::kFirstNan - 1u)) ? DT::kFirstNan : T - DT::kZeroOrder;
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

// Maximum of one unsigned value per lane over a full wave, through DPP lane
// moves (row shifts within rows of 16, then row broadcasts): wave-uniform.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max_u32(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x111, 0xF, 0xF, false));  // row_shr:1
    v = max_u32(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x112, 0xF, 0xF, false));  // row_shr:2
    v = max_u32(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x114, 0xF, 0xF, false));  // row_shr:4
    v = max_u32(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x118, 0xF, 0xF, false));  // row_shr:8
    v = max_u32(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xA, 0xF, false));  // row_bcast:15
    v = max_u32(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xC, 0xF, false));  // row_bcast:31
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Number of lanes below this one whose bit is set in `mask`.
__device__ __forceinline__ uint32_t lanes_below(unsigned long long mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Wave-uniform append: every lane calls it; the lanes with `has` write their
// key to buf[cnt + (number of such lanes below)], positions at or past `cap`
// are dropped.  Returns the new count (which may exceed cap: overflow).
// A call in which no lane appends costs a ballot and a scalar branch.
template <class KeyT>
__device__ __forceinline__ uint32_t wave_append(KeyT* buf, uint32_t cnt, uint32_t cap, bool has, KeyT key) {
    const unsigned long long m = __ballot(has);
    if (m == 0ull) return cnt;  // wave-uniform
    if (has) {
        const uint32_t pos = cnt + lanes_below(m);
        if (pos < cap) buf[pos] = key;
    }
    return cnt + (uint32_t)__popcll(m);
}

typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

// Rank selection: keys[0..n) are distinct keys in LDS (16-byte aligned,
// readable up to n rounded up to 8).  For the key of rank r (r < k, rank 0 =
// largest) it calls f(r, key).  A key's rank is the number of keys above it.
// Threads first, first + stride, ... take one key each; all of them read the
// same eight keys per step with 16-byte LDS reads (broadcasts), so the count
// is not bound by the latency of one read per key.
template <class F>
__device__ __forceinline__ void rank_apply(const uint64_t* keys, uint32_t n, uint32_t k, uint32_t first,
                                           uint32_t stride, const F& f) {
    const uint32_t n8 = (n + 7u) & ~7u;
    for (uint32_t t = first; t < n; t += stride) {
        const uint64_t key = keys[t];
        uint32_t r = 0;
        for (uint32_t j = 0; j < n8; j += 8) {
            const u64x2 q0 = *reinterpret_cast<const u64x2*>(keys + j);
            const u64x2 q1 = *reinterpret_cast<const u64x2*>(keys + j + 2);
            const u64x2 q2 = *reinterpret_cast<const u64x2*>(keys + j + 4);
            const u64x2 q3 = *reinterpret_cast<const u64x2*>(keys + j + 6);
            const uint64_t v0 = q0.x, v1 = q0.y, v2 = q1.x, v3 = q1.y;
            const uint64_t v4 = q2.x, v5 = q2.y, v6 = q3.x, v7 = q3.y;
            r += (v0 > key && j + 0 < n) + (v1 > key && j + 1 < n) +
                 (v2 > key && j + 2 < n) + (v3 > key && j + 3 < n) +
                 (v4 > key && j + 4 < n) + (v5 > key && j + 5 < n) +
                 (v6 > key && j + 6 < n) + (v7 > key && j + 7 < n);
        }
        if (r < k) f(r, key);
    }
}

// rank_apply that writes the key of rank r to out[r]; returns min(n, k).
__device__ __forceinline__ uint32_t rank_select(const uint64_t* keys, uint32_t n, uint32_t k,
                                                uint64_t* out, uint32_t first, uint32_t stride) {
    rank_apply(keys, n, k, first, stride, [&](uint32_t r, uint64_t key) { out[r] = key; });
    return min_u32(n, k);
}

// Rank of each lane's key among the n <= 64 distinct keys in LDS, keys[0..n8)
// with n8 = n rounded up to 8 and the slots past n holding 0 (below every
// key): the number of them that are larger.  All lanes read the same 16 bytes
// at a time (a broadcast), and the eight comparisons of a step are
// independent of each other, so the cost is a few LDS reads and compares per
// eight keys rather than a dependent chain per key.  Lanes whose key is not
// one of the n get a rank as well; callers ignore it.
__device__ __forceinline__ uint32_t lds_rank_of(const uint64_t* keys, uint32_t n8, uint64_t key) {
    uint32_t r0 = 0, r1 = 0;
    for (uint32_t j = 0; j < n8; j += 8) {
        const u64x2 q0 = *reinterpret_cast<const u64x2*>(keys + j);
        const u64x2 q1 = *reinterpret_cast<const u64x2*>(keys + j + 2);
        const u64x2 q2 = *reinterpret_cast<const u64x2*>(keys + j + 4);
        const u64x2 q3 = *reinterpret_cast<const u64x2*>(keys + j + 6);
        r0 += (uint32_t)(q0.x > key) + (uint32_t)(q0.y > key) + (uint32_t)(q1.x > key) + (uint32_t)(q1.y > key);
        r1 += (uint32_t)(q2.x > key) + (uint32_t)(q2.y > key) + (uint32_t)(q3.x > key) + (uint32_t)(q3.y > key);
    }
    return r0 + r1;
}

// Rank selection by one wave (see rank_select).
__device__ __forceinline__ uint32_t wave_rank_select(const uint64_t* keys, uint32_t n, uint32_t k,
                                                     uint64_t* out) {
    return rank_select(keys, n, k, out, threadIdx.x & 63u, 64u);
}

// Exact top-k of the keys a wave holds, by a bit-by-bit search for the k-th
// largest key (the tag bits [7:0] are equal for all keys and skipped), then a
// rank count of the at most k keys at or above it.  visit(f) calls
// f(key, valid) for every key slot of the calling lane, in the same order on
// every lane.  Collects into buf (cap entries), writes the result sorted to
// out[0..n) and returns n = min(k, number of valid keys).  Valid keys must be
// distinct.
template <int OrderBits, class Visit>
__device__ __forceinline__ uint32_t wave_exact_topk(uint64_t* buf, uint32_t cap, uint64_t* out,
                                                    const Visit& visit, uint32_t k) {
    // counts are wave-wide: one ballot per key slot (visit is wave-uniform)
    uint32_t total = 0;
    visit([&](uint64_t, bool valid) { total += (uint32_t)__popcll(__ballot(valid)); });
    uint64_t thr = 0;
    if (total > k) {
        // a rare path: the rounds stay a loop, so the code stays small
#pragma unroll 1
        for (int b = 32 + OrderBits - 1; b >= 8; --b) {
            const uint64_t cand = thr | (1ull << b);
            uint32_t n = 0;
            visit([&](uint64_t key, bool valid) { n += (uint32_t)__popcll(__ballot(valid && key >= cand)); });
            if (n >= k) thr = cand;
        }
    }
    uint32_t cnt = 0;
    visit([&](uint64_t key, bool valid) { cnt = wave_append(buf, cnt, cap, valid && key >= thr, key); });
    return wave_rank_select(buf, min_u32(cnt, cap), k, out);
}

}  // namespace topk
