// Row-interleaved top-k kernels for gfx950: element (r, c) at x[r*ld + c].
//
// This layout holds many independent rounds side by side.  Each column (one
// draft position of one round) is spread over V rows, ld elements apart, and
// a 128-byte line holds 128 bytes of adjacent columns of one row.  Coalesced
// reads therefore touch many columns at once.  A workgroup owns a tile of
// columns (128 bytes of each row: 64 bf16 or 32 fp32 columns) over a segment
// of rows.  Each lane loads one 16-byte vector of a row per step (8 or 4
// columns): 8 lanes cover a row, a wave 8 rows, the workgroup 32 rows.  The
// selection order is the one of the column-contiguous kernel: larger value
// first, ties to the smaller row (ignis "DFlash2" page, "How it works").
//
// Scan kernel.  A pass is NV steps of 32 rows, and the next pass's loads are
// issued before the current pass is filtered.  In a whole tile of aligned
// rows every load is unconditional (rows past the segment are clamped and
// masked), so the compiler can count the loads in flight and filtering waits
// for the current pass only.  Every column keeps a running
// threshold T_c (an order that is at most the segment's k-th largest) and an
// LDS buffer of candidate keys that holds every element seen so far at or
// above T_c.
//  1. First pass only: packed 16-bit (bf16) or 32-bit integer max/min of the
//     raw patterns over the first two passes (both are loaded by then) give
//     each lane two exact group maxima per column, 64 per column in the
//     workgroup.  T_c starts as the k-th largest of them: k distinct
//     elements are at least that large.
//  2. Every pass: each 32-bit word of a row vector is tested against the
//     thresholds of its columns in the raw bit domain (one xor and one packed
//     signed max per word, see RowFilter).  A lane with a passing element
//     appends its whole row vector to its wave's LDS queue (ballot + mbcnt).
//     When the queue fills, and at the end of the pass, the wave turns the
//     queued vectors into keys, one vector per lane, and adds them to the
//     column buffers (an LDS atomic per key).
//  2b. Segments of one column share a lower bound on the column's k-th
//     largest order over all V rows.  After step 1 each workgroup publishes
//     its column maximum (an atomic max into slot s mod k of the column, in
//     the workspace); every pass reads the k slots before its prefetch and,
//     once all are filled, raises T_c to their minimum: k elements of
//     distinct segments are at least that large.  This bound is far above a
//     single segment's own, so after the first passes almost nothing passes
//     the filter.  The merge kernel clears the slots for the next run.
//  3. After a pass, a column holding more than max(2k, 24) keys is trimmed:
//     the threads of the column find the exact k-th largest order among its
//     candidates, which becomes the new T_c, and compact the buffer in place.
//     T_c then follows the segment's own k-th largest, so later passes add
//     few candidates.
//  4. At the end a rank count over each column's candidates (trimmed first
//     if many) writes the column's top k, sorted, to the segment's slot of
//     the partial lists.
// A column whose buffer overflows during a pass is rebuilt at the end of the
// pass: one wave re-reads the pass's rows of that column and keeps what is at
// or above the exact k-th largest order seen so far.  Negative NaNs never
// pass the raw filter; a lane notes them in a running unsigned maximum.  Such
// a column, like one that still overflows after a rebuild (massive ties), is
// re-read over the whole segment by one wave and selected by an exact search.
//
// Merge kernel: one workgroup per column selects the top k of its S sorted
// partial lists (its four waves read a quarter of the entries each with
// coalesced loads; the k-th largest of the S list heads is the threshold,
// then a rank count, by 16-byte LDS broadcasts when at most 64 entries pass)
// and writes the output.  The kernel boundary orders it after the scan.
#include <type_traits>

#include "topk_device.hpp"
#include "topk_internal.hpp"

namespace topk {

namespace {

constexpr int kRowLanesPerRow = 8;                      // 8 lanes x 16 bytes = one 128-byte row tile
constexpr int kRowsPerStep = kBlock / kRowLanesPerRow;  // 32 rows per workgroup step
constexpr int kRowTileBytes = 128;
constexpr int kRowReps = 2 * kRowsPerStep;              // group maxima per column (first pass)
constexpr int kRowQueue = 128;                          // queued row vectors per wave
// Candidate buffer per column: CAP keys.  A trim leaves about k of them and
// is due above max(2k, 24), so a pass may add at least CAP - max(2k, 24)
// (32 or more) before the buffer overflows.
constexpr int kRowCapSmall = 64;
constexpr int kRowCapLarge = 192;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <class DT>
struct RowTile {
    static constexpr int TW = kRowTileBytes / (int)sizeof(typename DT::storage);  // columns per tile
    static constexpr int CPV = DT::kPerVec;                                     // columns per lane
    static constexpr int TPC = kBlock / TW;                                     // threads per column
};

// Candidate keys of the scan.  RowKey64 is the library's 64-bit key.
// RowKey32 (bf16, segments of at most 65,536 rows) keeps the 16-bit order in
// bits 31..16 and 0xFFFF - (row - r_lo) in bits 15..0: the same order, half
// the LDS, so twice the candidates fit.  Keys are widened to 64 bits when a
// segment's list is written.  A zero key is never a real one.
struct RowKey64 {
    using T = uint64_t;
    static constexpr int kPad = 2;  // keeps rows 16-byte aligned, spreads banks
    __device__ __forceinline__ static T make(uint32_t order, uint32_t row, uint32_t) { return make_key(order, row, 0u); }
    __device__ __forceinline__ static uint32_t order(T key) { return key_order(key); }
    __device__ __forceinline__ static uint32_t row(T key, uint32_t) { return key_row(key); }
    __device__ __forceinline__ static uint64_t wide(T key, uint32_t) { return key; }
};
struct RowKey32 {
    using T = uint32_t;
    static constexpr int kPad = 4;
    __device__ __forceinline__ static T make(uint32_t order, uint32_t row, uint32_t r_lo) {
        return (order << 16) | (0xFFFFu - (row - r_lo));
    }
    __device__ __forceinline__ static uint32_t order(T key) { return key >> 16; }
    __device__ __forceinline__ static uint32_t row(T key, uint32_t r_lo) { return r_lo + 0xFFFFu - (key & 0xFFFFu); }
    __device__ __forceinline__ static uint64_t wide(T key, uint32_t r_lo) {
        return key ? make_key(key >> 16, row(key, r_lo), 0u) : 0ull;
    }
};

template <class DT, int CAP, class KT>
struct RowShared {
    static constexpr int TW = RowTile<DT>::TW;
    static constexpr int STRIDE = CAP + KT::kPad;  // keys per column row
    // The first pass's group maxima are read before any candidate is
    // appended (a barrier lies between), so they share the candidates' space.
    union {
        alignas(16) typename KT::T cand[TW][STRIDE];  // per-column candidate keys
        uint32_t reps[TW][kRowReps + 1];              // first-pass group maxima (orders)
    };
    alignas(16) uint64_t tmp[kWaves][kMaxK];     // exact-path output per wave
    alignas(16) u32x4 qdata[kWaves][kRowQueue];  // queued row vectors
    uint32_t qmeta[kWaves][kRowQueue];           // (row << 3) | lane group of each queued vector
    alignas(16) typename DT::storage fm[TW];     // raw-filter xor mask per column
    alignas(16) typename DT::storage fq[TW];     // raw-filter bound per column
    uint32_t thr[TW];                            // running threshold per column (order)
    uint32_t cnt[TW];                            // candidates per column (may exceed CAP)
    uint32_t flag[TW];                           // 1: candidates overflowed, 2: negative NaN seen
    uint32_t cm[TW];                             // first-pass maximum per column (order)
    uint32_t ovf;                                // some column overflowed in this pass
};

static_assert(sizeof(uint32_t[RowTile<Bf16>::TW][kRowReps + 1]) <=
                  sizeof(RowKey32::T[RowTile<Bf16>::TW][kRowCapSmall + RowKey32::kPad]) &&
              sizeof(uint32_t[RowTile<F32>::TW][kRowReps + 1]) <=
                  sizeof(RowKey64::T[RowTile<F32>::TW][kRowCapSmall + RowKey64::kPad]),
              "the group maxima fit in the candidate area");

__device__ __forceinline__ s16x2 as_s16x2_r(uint32_t w) { return __builtin_bit_cast(s16x2, w); }
__device__ __forceinline__ u16x2 as_u16x2_r(uint32_t w) { return __builtin_bit_cast(u16x2, w); }

// Raw-domain test "order(x) >= T" for every pattern except negative NaNs
// (which always fail; they are detected separately).  With y = x ^ m read as
// a signed integer, the element passes iff y > q:
//  - T above the zero class: m = 0 and q = (smallest positive pattern with
//    order >= T) - 1.  Negative patterns are negative integers and fail;
//    positive NaNs are the largest positive patterns and pass.
//  - T at or below the zero class: the passing patterns are the unsigned
//    range [0, R], R the negative pattern of order T (the zero class gives
//    R = -0).  x ^ 0x7FF..F maps unsigned patterns to signed integers in
//    decreasing order, so m = 0x7FF..F and q = (R ^ m) - 1.
//  - T at or below the order of -Inf: every pattern but the all-ones
//    negative NaN passes (q is the smallest signed integer).
template <class DT>
struct RowFilter;

template <>
struct RowFilter<Bf16> {
    __device__ __forceinline__ static void encode(uint32_t T, uint32_t& m, uint32_t& q) {
        if (T <= 0x80u) {
            m = 0x7FFFu;
            q = 0x8000u;
        } else if (T <= 0x8000u) {
            m = 0x7FFFu;
            q = (((0x10000u - T) ^ 0x7FFFu) - 1u) & 0xFFFFu;
        } else if (T <= 0xFF80u) {
            m = 0u;
            q = T - 0x8001u;
        } else {
            m = 0u;
            q = 0x7F80u;
        }
    }
    // A word holds two columns; a nonzero half of the result passes.
    __device__ __forceinline__ static uint32_t test(uint32_t x, uint32_t m, uint32_t q) {
        const s16x2 y = as_s16x2_r(x ^ m);
        return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(y, as_s16x2_r(q))) ^ q;
    }
    __device__ __forceinline__ static bool passes(uint32_t t, int half) { return ((t >> (16 * half)) & 0xFFFFu) != 0u; }
    // running unsigned maximum of the raw patterns, per half
    __device__ __forceinline__ static uint32_t umax(uint32_t acc, uint32_t x) {
        return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(as_u16x2_r(acc), as_u16x2_r(x)));
    }
    __device__ __forceinline__ static bool has_negative_nan(uint32_t acc, int half) {
        return ((acc >> (16 * half)) & 0xFFFFu) > 0xFF80u;
    }
    // running signed maximum per half of already-masked words (x ^ m)
    static constexpr uint32_t kSMin = 0x80008000u;
    __device__ __forceinline__ static uint32_t smax(uint32_t acc, uint32_t y) {
        return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(as_s16x2_r(acc), as_s16x2_r(y)));
    }
};

template <>
struct RowFilter<F32> {
    __device__ __forceinline__ static void encode(uint32_t T, uint32_t& m, uint32_t& q) {
        if (T <= 0x00800000u) {
            m = 0x7FFFFFFFu;
            q = 0x80000000u;
        } else if (T <= 0x80000000u) {
            m = 0x7FFFFFFFu;
            q = ((0u - T) ^ 0x7FFFFFFFu) - 1u;
        } else if (T <= 0xFF800000u) {
            m = 0u;
            q = T - 0x80000001u;
        } else {
            m = 0u;
            q = 0x7F800000u;
        }
    }
    __device__ __forceinline__ static uint32_t test(uint32_t x, uint32_t m, uint32_t q) {
        return (int)(x ^ m) > (int)q ? 1u : 0u;
    }
    __device__ __forceinline__ static bool passes(uint32_t t, int) { return t != 0u; }
    __device__ __forceinline__ static uint32_t umax(uint32_t acc, uint32_t x) { return max_u32(acc, x); }
    __device__ __forceinline__ static bool has_negative_nan(uint32_t acc, int) { return acc > 0xFF800000u; }
    static constexpr uint32_t kSMin = 0x80000000u;
    __device__ __forceinline__ static uint32_t smax(uint32_t acc, uint32_t y) { return (uint32_t)max_i32((int)acc, (int)y); }
};

__device__ __forceinline__ uint32_t word(const u32x4& v, int q) {
    const uint32_t wx = v.x, wy = v.y, wz = v.z, ww = v.w;
    return q == 0 ? wx : q == 1 ? wy : q == 2 ? wz : ww;
}

// Element j (column j of the lane's vector) of a loaded vector; j may vary.
template <class DT>
__device__ __forceinline__ uint32_t row_elem(const u32x4& v, uint32_t j) {
    const uint32_t wx = v.x, wy = v.y, wz = v.z, ww = v.w;
    if constexpr (DT::kPerVec == 8) {
        const uint32_t q = j >> 1;
        const uint32_t w = q == 0 ? wx : q == 1 ? wy : q == 2 ? wz : ww;
        return (w >> (16u * (j & 1u))) & 0xFFFFu;
    } else {
        return j == 0 ? wx : j == 1 ? wy : j == 2 ? wz : ww;
    }
}

// Exact maximum order per column of one lane over a group of row vectors,
// from the raw patterns: the signed maximum when some pattern is
// non-negative, else the signed minimum (the negative value nearest zero).
// A negative NaN may be missed, which leaves a lower bound: enough for a
// threshold.
template <class DT>
struct ColMax {
    uint32_t smax[4], smin[4];
    __device__ __forceinline__ void init() {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            smax[q] = DT::kPerVec == 8 ? 0x80008000u : 0x80000000u;
            smin[q] = DT::kPerVec == 8 ? 0x7FFF7FFFu : 0x7FFFFFFFu;
        }
    }
    __device__ __forceinline__ void add(const u32x4& v) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t w = word(v, q);
            if constexpr (DT::kPerVec == 8) {
                smax[q] = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(as_s16x2_r(smax[q]), as_s16x2_r(w)));
                smin[q] = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(as_s16x2_r(smin[q]), as_s16x2_r(w)));
            } else {
                smax[q] = (uint32_t)max_i32((int)smax[q], (int)w);
                smin[q] = (uint32_t)min_i32((int)smin[q], (int)w);
            }
        }
    }
    __device__ __forceinline__ uint32_t order(int j) const {
        if constexpr (DT::kPerVec == 8) {
            const int q = j >> 1, sh = (j & 1) * 16;
            const int M = (int)(int16_t)(smax[q] >> sh);
            const int m = (int)(int16_t)(smin[q] >> sh);
            return M >= 0 ? DT::order((uint32_t)M) : DT::order((uint32_t)m & 0xFFFFu);
        } else {
            return (int)smax[j] >= 0 ? DT::order(smax[j]) : DT::order(smin[j]);
        }
    }
};

// Value of v in a partner lane through a DPP lane permutation (no LDS
// round trip): 0xB1 swaps neighbours within a quad, 0x4E swaps the two lane
// pairs of a quad, 0x141 mirrors each half-row of 8 lanes.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// Sum, maximum and minimum of v over the TPC (4 or 8) consecutive lanes of
// one column's thread group, all of them active.
template <int TPC>
__device__ __forceinline__ uint32_t group_sum(uint32_t v) {
    static_assert(TPC == 4 || TPC == 8, "quads or half-rows");
    v += dpp_mov<0xB1>(v);
    v += dpp_mov<0x4E>(v);
    if constexpr (TPC == 8) v += dpp_mov<0x141>(v);
    return v;
}
template <int TPC>
__device__ __forceinline__ uint32_t group_max(uint32_t v) {
    v = max_u32(v, dpp_mov<0xB1>(v));
    v = max_u32(v, dpp_mov<0x4E>(v));
    if constexpr (TPC == 8) v = max_u32(v, dpp_mov<0x141>(v));
    return v;
}
template <int TPC>
__device__ __forceinline__ uint32_t group_min(uint32_t v) {
    v = min_u32(v, dpp_mov<0xB1>(v));
    v = min_u32(v, dpp_mov<0x4E>(v));
    if constexpr (TPC == 8) v = min_u32(v, dpp_mov<0x141>(v));
    return v;
}

// The k-th largest of the values a thread group holds (VPT per thread, empty
// slots 0), by bisection of [lo, hi] where at least k values are >= lo and
// hi is the largest value: about log2(hi - lo) counting rounds.  The upper
// midpoint is lo + ceil((hi - lo) / 2), written so that it does not wrap
// when hi - lo is 2^32 - 1 (lo = 0 and a NaN, order 0xFFFFFFFF): a wrapped
// midpoint equals lo and the bisection would never end.
template <int TPC, int VPT>
__device__ __forceinline__ uint32_t group_kth(const uint32_t (&v)[VPT], uint32_t k, uint32_t lo, uint32_t hi) {
    while (lo < hi) {
        const uint32_t d = hi - lo;
        const uint32_t mid = lo + (d >> 1) + (d & 1u);
        uint32_t m = 0;
#pragma unroll
        for (int j = 0; j < VPT; ++j) m += v[j] >= mid ? 1u : 0u;
        if (group_sum<TPC>(m) >= k) lo = mid;
        else hi = mid - 1u;
    }
    return lo;
}

// Bit i set for each column i < TW of the tile taken by wave w (columns w,
// w + kWaves, ...) that satisfies pred(column); wave-uniform.
template <int TW, class Pred>
__device__ __forceinline__ uint64_t wave_columns(uint32_t w, const Pred& pred) {
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t colx = w + lane * kWaves;
    return __ballot(colx < (uint32_t)TW && pred(colx));
}

// Exact path for one column of a segment: one wave re-reads the column's rows
// [r_lo, r_hi) (stride ld) at every step of an exact bit search and writes
// the column's top-k (sorted) to out; returns n.
template <class DT>
__device__ __noinline__ uint32_t exact_row_column(const typename DT::storage* x, int64_t ld, uint32_t col,
                                                  uint32_t r_lo, uint32_t r_hi, uint64_t* buf,
                                                  uint32_t cap, uint64_t* out, uint32_t k) {
    const uint32_t lane = threadIdx.x & 63u;
    auto visit = [&](auto&& f) {
#pragma unroll 1
        for (uint32_t r0 = r_lo; r0 < r_hi; r0 += 64u) {
            const uint32_t r = r0 + lane;
            const bool valid = r < r_hi;
            const uint32_t raw = valid ? (uint32_t)x[(int64_t)r * ld + col] : 0u;
            f(make_key(DT::order(raw), r, 0u), valid);
        }
    };
    return wave_exact_topk<DT::kOrderBits>(buf, cap, out, visit, k);
}

// Keeps the candidates of one column whose order is at least the k-th
// largest order among the n of them (all of them when n <= k), compacted in
// place.  Every candidate's order is at least thr.  Called by the column's
// TPC threads (consecutive lanes of one wave); thread q holds candidates q,
// q + TPC, ...  Returns the new count and sets T_out to that k-th largest
// order (thr when n <= k).
template <class DT, int CAP, class KT>
__device__ __forceinline__ uint32_t trim_column(typename KT::T* cand, uint32_t q, uint32_t n, uint32_t k,
                                                uint32_t thr, uint32_t* T_out) {
    constexpr int TPC = RowTile<DT>::TPC;
    constexpr int VPT = CAP / TPC;
    uint32_t o[VPT];
    uint32_t mx = 0;
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const uint32_t idx = q + (uint32_t)v * TPC;
        o[v] = idx < n ? KT::order(cand[idx]) : 0u;
        mx = max_u32(mx, o[v]);
    }
    uint32_t T = thr;
    if (n > k) T = group_kth<TPC, VPT>(o, k, thr, group_max<TPC>(mx));
    *T_out = T;
    // In-place stable compaction with the TPC threads in step: at step v
    // every index below (v + 1) * TPC has been read, and a kept key moves to
    // an index at or below its own.
    const uint32_t lane = threadIdx.x & 63u;
    const uint64_t gmask = ((1ull << TPC) - 1ull) << (lane & ~(uint32_t)(TPC - 1));
    const uint64_t below = (1ull << lane) - 1ull;
    uint32_t out = 0;
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const uint32_t idx = q + (uint32_t)v * TPC;
        const bool keep = idx < n && o[v] >= T;
        const uint64_t bal = __ballot(keep) & gmask;
        const typename KT::T key = keep ? cand[idx] : (typename KT::T)0;
        if (keep) cand[out + (uint32_t)__popcll(bal & below)] = key;
        out += (uint32_t)__popcll(bal);
    }
    return out;
}

// Drops the candidates of one column whose order is below T (a raised
// threshold), compacting the rest in place; the same thread layout as
// trim_column.  Returns the new count.  n is column-uniform, so the loop
// trip count is too.
template <class DT, class KT>
__device__ __forceinline__ uint32_t cull_column(typename KT::T* cand, uint32_t q, uint32_t n, uint32_t T) {
    constexpr int TPC = RowTile<DT>::TPC;
    const uint32_t lane = threadIdx.x & 63u;
    const uint64_t gmask = ((1ull << TPC) - 1ull) << (lane & ~(uint32_t)(TPC - 1));
    const uint64_t below = (1ull << lane) - 1ull;
    uint32_t out = 0;
    for (uint32_t base = 0; base < n; base += TPC) {
        const uint32_t idx = base + q;
        const typename KT::T key = idx < n ? cand[idx] : (typename KT::T)0;
        const bool keep = idx < n && KT::order(key) >= T;
        const uint64_t bal = __ballot(keep) & gmask;
        if (keep) cand[out + (uint32_t)__popcll(bal & below)] = key;
        out += (uint32_t)__popcll(bal);
    }
    return out;
}

// Rank count over the keys of one column (thread first, first + stride, ...
// each take a key; all read the same keys with 16-byte LDS reads): the key
// of rank r < k goes, widened, to dst[r * dstride].  Keys are readable up to
// n rounded up to 8.
template <class KT>
__device__ __forceinline__ void rank_keys(const typename KT::T* keys, uint32_t n, uint32_t k, uint64_t* dst,
                                          uint32_t dstride, uint32_t first, uint32_t stride, uint32_t r_lo) {
    using T = typename KT::T;
    typedef T vec2 __attribute__((ext_vector_type(16 / sizeof(T))));
    constexpr uint32_t PER = 16 / sizeof(T);  // keys per 16-byte read
    const uint32_t n8 = (n + 7u) & ~7u;
    for (uint32_t t = first; t < n; t += stride) {
        const T key = keys[t];
        uint32_t r = 0;
        for (uint32_t j = 0; j < n8; j += 8) {
#pragma unroll
            for (uint32_t h = 0; h < 8; h += PER) {
                const vec2 q = *reinterpret_cast<const vec2*>(keys + j + h);
#pragma unroll
                for (uint32_t e = 0; e < PER; ++e) r += (q[e] > key && j + h + e < n) ? 1u : 0u;
            }
        }
        if (r < k) dst[(int64_t)r * dstride] = KT::wide(key, r_lo);
    }
}

template <class DT, int NV, int CAP, class KT>
__device__ __noinline__ void rebuild_column(RowShared<DT, CAP, KT>& sh, const typename DT::storage* x, int64_t ld,
                                            uint32_t colx, uint32_t col, uint32_t r_lo, uint32_t pass_lo,
                                            uint32_t pass_hi, uint32_t k) {
    using F = RowFilter<DT>;
    using T = typename KT::T;
    constexpr int PRE = (CAP + 63) / 64;             // buffer keys per lane
    constexpr int PER = kRowsPerStep * NV / 64;      // pass rows per lane
    constexpr int OB = DT::kOrderBits;
    const uint32_t lane = threadIdx.x & 63u;
    T key[PRE + PER];
    bool valid[PRE + PER];
#pragma unroll
    for (int j = 0; j < PRE; ++j) {
        const uint32_t idx = (uint32_t)j * 64u + lane;
        key[j] = idx < (uint32_t)CAP ? sh.cand[colx][idx] : (T)0;
        valid[j] = idx < (uint32_t)CAP && KT::row(key[j], r_lo) < pass_lo;
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const uint32_t r = pass_lo + (uint32_t)j * 64u + lane;
        valid[PRE + j] = r < pass_hi;
        const uint32_t raw = r < pass_hi ? (uint32_t)x[(int64_t)r * ld + col] : 0u;
        key[PRE + j] = KT::make(DT::order(raw), r, r_lo);
    }
    uint32_t T_k = 0;
#pragma unroll 1
    for (int b = OB - 1; b >= 0; --b) {
        const uint32_t c = T_k | (1u << b);
        uint32_t n = 0;
#pragma unroll
        for (int j = 0; j < PRE + PER; ++j) n += (uint32_t)__popcll(__ballot(valid[j] && KT::order(key[j]) >= c));
        if (n >= k) T_k = c;
    }
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < PRE + PER; ++j)
        cnt = wave_append(sh.cand[colx], cnt, (uint32_t)CAP, valid[j] && KT::order(key[j]) >= T_k, key[j]);
    if (lane == 0) {
        sh.cnt[colx] = cnt;
        if (cnt > (uint32_t)CAP) sh.flag[colx] |= 1u;
        if (T_k > sh.thr[colx]) {
            uint32_t fmv, fqv;
            F::encode(T_k, fmv, fqv);
            sh.thr[colx] = T_k;
            sh.fm[colx] = (typename DT::storage)fmv;
            sh.fq[colx] = (typename DT::storage)fqv;
        }
    }
}

// Three workgroups per CU when the candidate area allows (k <= kRowSmallK:
// 47 KB of LDS); the register budget is then 168 per lane.  The larger
// candidate areas allow fewer workgroups whatever the registers, and the
// compiler says so (the build silences that note for this file).
template <class DT, int NV, int CAP, class KT>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(3))) void topk_row_scan(RowArgs a);

template <class DT, int NV, int CAP, class KT>
__global__ __launch_bounds__(kBlock) void topk_row_scan(RowArgs a) {
    using storage = typename DT::storage;
    using F = RowFilter<DT>;
    constexpr int TW = RowTile<DT>::TW;
    constexpr int CPV = RowTile<DT>::CPV;
    constexpr int TPC = RowTile<DT>::TPC;
    static_assert(NV % 2 == 0, "two row groups per pass");
    __shared__ RowShared<DT, CAP, KT> sh;

    const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
    const uint32_t k = (uint32_t)a.k;
    // trim a column above this many candidates (room for a pass's new ones)
    const uint32_t trim_at = max_u32(2u * k, max_u32(24u, (uint32_t)CAP - 32u));
    const uint32_t tiles = (uint32_t)a.tiles;
    const uint32_t S = (uint32_t)a.S;
    const uint32_t s = blockIdx.x / tiles;          // row segment
    const uint32_t tile = blockIdx.x - s * tiles;   // column tile
    const uint32_t V = (uint32_t)a.V, C = (uint32_t)a.C;
    const uint32_t c0 = tile * TW;
    const uint32_t r_lo = (uint32_t)((uint64_t)V * s / S), r_hi = (uint32_t)((uint64_t)V * (s + 1) / S);
    const storage* x = static_cast<const storage*>(a.x);

    const uint32_t rsub = tid / kRowLanesPerRow;     // row within a 32-row step
    const uint32_t g = tid % kRowLanesPerRow;        // 16-byte group within the tile
    const uint32_t cg = c0 + g * CPV;                // first column of this lane
    const uint32_t ncols = cg < C ? min_u32((uint32_t)CPV, C - cg) : 0u;
    const bool vec_ok = a.vec_loads != 0 && ncols == (uint32_t)CPV;

    // column-parallel steps: TPC consecutive threads per tile column
    const uint32_t pcol = tid / TPC, pq = tid % TPC;

    if (tid < (uint32_t)TW) {
        sh.thr[tid] = 0;
        sh.cnt[tid] = 0;
        sh.flag[tid] = 0;
        sh.cm[tid] = 0;
    }
    if (tid == 0) sh.ovf = 0;

    const uint32_t per_pass = (uint32_t)kRowsPerStep * NV;
    const uint32_t npass = r_hi > r_lo ? (r_hi - r_lo + per_pass - 1) / per_pass : 0u;

    auto load_pass = [&](u32x4(&d)[NV], uint32_t p) {
        const uint32_t rbase = r_lo + p * per_pass + rsub;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const uint32_t r = rbase + (uint32_t)i * kRowsPerStep;
            const storage* src = x + (int64_t)r * a.ld + cg;
            if (r < r_hi && vec_ok) {
                d[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
            } else {
                // a partial vector (row past the segment, columns past C, or
                // rows not 16-byte aligned): element loads, -Inf elsewhere
                uint32_t e[CPV];
#pragma unroll
                for (int j = 0; j < CPV; ++j)
                    e[j] = (r < r_hi && (uint32_t)j < ncols) ? (uint32_t)src[j] : (DT::kFillDword & DT::kRawMask);
                if constexpr (CPV == 8)
                    d[i] = u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
                else
                    d[i] = u32x4{e[0], e[1], e[2], e[3]};
            }
        }
    };

    // Turn the wave's queued row vectors into candidate keys, one vector per
    // lane (wave-uniform qcnt).
    auto flush = [&](uint32_t qcnt) {
        for (uint32_t b = 0; b < qcnt; b += 64u) {
            const uint32_t e = b + lane;
            if (e < qcnt) {
                const u32x4 d = sh.qdata[wave][e];
                const uint32_t meta = sh.qmeta[wave][e];
                const uint32_t row = meta >> 3, gg = meta & 7u;
                const uint32_t nc = min_u32((uint32_t)CPV, C - (c0 + gg * CPV));  // queued lanes have columns < C
                const u32x4 fmw = *reinterpret_cast<const u32x4*>(&sh.fm[gg * CPV]);
                const u32x4 fqw = *reinterpret_cast<const u32x4*>(&sh.fq[gg * CPV]);
                uint32_t mask = 0;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t t = F::test(word(d, q), word(fmw, q), word(fqw, q));
                    if constexpr (CPV == 8) {
                        mask |= (F::passes(t, 0) ? 1u : 0u) << (2 * q);
                        mask |= (F::passes(t, 1) ? 1u : 0u) << (2 * q + 1);
                    } else {
                        mask |= (F::passes(t, 0) ? 1u : 0u) << q;
                    }
                }
                mask &= (1u << nc) - 1u;
                while (mask) {
                    const uint32_t j = (uint32_t)__builtin_ctz(mask);
                    mask &= mask - 1u;
                    const uint32_t col = gg * CPV + j;
                    const uint32_t o = DT::order(row_elem<DT>(d, j));
                    const uint32_t pos = atomicAdd(&sh.cnt[col], 1u);
                    if (pos < (uint32_t)CAP) sh.cand[col][pos] = KT::make(o, row, r_lo);
                    else sh.ovf = 1u;
                }
            }
        }
    };

    // A whole tile of 16-byte aligned rows loads with no per-lane branch:
    // rows past the segment re-read its last row and are masked where they
    // are used, and after the last pass a dummy prefetch re-reads the
    // segment's first rows. With every load unconditional the compiler knows
    // how many loads are in flight, so filtering a pass waits for that pass
    // alone while the next one streams in.
    const bool full_tile = a.vec_loads != 0 && c0 + (uint32_t)TW <= C;
    // Byte offsets from the segment's first row fit 32 bits (and a 24 x 24-bit
    // multiply) in every realistic shape; the row address is then one 24-bit
    // multiply-add on a uniform base instead of 64-bit arithmetic per load.
    const uint64_t row_bytes = (uint64_t)a.ld * sizeof(storage);
    const bool off24 = row_bytes < (1u << 24) && (uint64_t)(r_hi - r_lo) * row_bytes + 128u < (1ull << 31);
    const char* seg_bytes = reinterpret_cast<const char*>(x + (int64_t)r_lo * a.ld + c0);
    const uint32_t lane_bytes = (cg - c0) * (uint32_t)sizeof(storage);
    auto load_full = [&](u32x4(&d)[NV], uint32_t p, uint32_t step) {
        const uint32_t rbase = r_lo + p * per_pass + rsub;
        if (off24) {
            const uint32_t rb = (uint32_t)row_bytes, rel = rbase - r_lo, last = r_hi - 1u - r_lo;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const uint32_t rr = min_u32(rel + (uint32_t)i * step, last);
                const uint32_t off = __umul24(rr, rb) + lane_bytes;
                d[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(seg_bytes + off));
            }
        } else {
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const uint32_t r = min_u32(rbase + (uint32_t)i * step, r_hi - 1u);
                d[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + (int64_t)r * a.ld + cg));
            }
        }
    };
    const u32x4 fill4 = u32x4{DT::kFillDword, DT::kFillDword, DT::kFillDword, DT::kFillDword};

    // Lower bound shared by the segments of a column: each segment s <
    // kRowBoundRows stores one element of each of its columns (its largest
    // group maximum) in row s of the bound area (bound_ld words a row).  A
    // wave's stores fill whole lines that no other workgroup writes: loads
    // of words that many workgroups write at once (atomics, or stores to
    // one line) wait behind those writes for microseconds.  Distinct
    // segments hold distinct elements, so the k-th largest of a column's
    // words (zero where no segment has stored yet) is at most the column's
    // k-th largest order over all V rows: no element below it can be in the
    // output, whatever segment it lies in.  The merge kernel zeroes the
    // words for the next run.
    constexpr int kBoundPerThread = kRowBoundRows / TPC;
    const uint32_t bld = (uint32_t)a.bound_ld;
    // 32-bit word indices from the area's base (plans keep the area below
    // 2^32 words): one register per thread, the rows' steps are uniform
    const uint32_t bound_i = min_u32(c0 + pcol, C - 1u) + pq * (uint32_t)kBoundPerThread * bld;
    auto load_bound = [&](uint32_t(&w)[kBoundPerThread]) {
        // opaque here, so that the addresses are formed at each read rather
        // than kept in registers across the pass loop
        uint32_t bi = bound_i;
        asm volatile("" : "+v"(bi));
#pragma unroll
        for (int j = 0; j < kBoundPerThread; ++j)
            w[j] = __hip_atomic_load(&a.bound[bi + (uint32_t)j * bld], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    // max(floor, the k-th largest word), for a floor that is already a
    // valid threshold: the bisection only searches above it, a far narrower
    // range than all the words'
    auto bound_kth = [&](const uint32_t(&w)[kBoundPerThread], uint32_t floor) {
        uint32_t wmax = w[0], n = 0;
#pragma unroll
        for (int j = 0; j < kBoundPerThread; ++j) {
            wmax = max_u32(wmax, w[j]);
            n += w[j] >= floor ? 1u : 0u;
        }
        if (group_sum<TPC>(n) < k) return floor;
        return group_kth<TPC, kBoundPerThread>(w, k, floor, group_max<TPC>(wmax));
    };

    uint32_t nanacc[4] = {0u, 0u, 0u, 0u};
    auto scan_passes = [&](auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    u32x4 cur[NV], nxt[NV];
    if (npass > 0) {
        if constexpr (FULL)
            load_full(cur, 0, kRowsPerStep);
        else
            load_pass(cur, 0);
    }
    __syncthreads();

    // The shared bound is read twice.  The first pass stores this segment's
    // maxima as soon as its data is in, reads the bound back while it
    // gathers the second pass's group maxima, and filters against it (where
    // it does not hold yet, against the local k-th group maximum).  The second
    // pass reads it again at its top (by then nearly every segment has
    // stored; the loads go before the prefetch, so that waiting for them
    // does not wait for it), and the third applies it at its end: two
    // passes' filtering hide the loads' latency, which is several
    // microseconds while every workgroup streams.
    uint32_t bw[kBoundPerThread];
    for (uint32_t p = 0; p < npass; ++p) {
        const bool bound_late = a.use_bound && p == 2u && npass > 3u;
        if (a.use_bound && p == 1u && npass > 3u) load_bound(bw);
        if constexpr (FULL) {
            const bool more = p + 1 < npass;
            load_full(nxt, more ? p + 1 : 0u, more ? (uint32_t)kRowsPerStep : 0u);
        } else {
            if (p + 1 < npass) load_pass(nxt, p + 1);
        }

        if (p == 0) {
            // (1) starting thresholds from 64 group maxima per column
            ColMax<DT> m0, m1;
            m0.init();
            m1.init();
            // rows past the segment count as -Inf (a full tile loaded copies of its last row)
            auto row_vec = [&](const u32x4& v, uint32_t pp, int i) {
                if constexpr (FULL)
                    return r_lo + pp * per_pass + rsub + (uint32_t)i * kRowsPerStep < r_hi ? v : fill4;
                else
                    return v;
            };
#pragma unroll
            for (int i = 0; i < NV; i += 2) {
                m0.add(row_vec(cur[i], 0u, i));
                m1.add(row_vec(cur[i + 1], 0u, i + 1));
            }
            if (a.use_bound) {
                // the first pass's maximum of each column (an element of the
                // segment) for the other segments, then the bound read back
#pragma unroll
                for (int j = 0; j < CPV; ++j) atomicMax(&sh.cm[g * CPV + j], max_u32(m0.order(j), m1.order(j)));
                __syncthreads();
                if (pq == 0 && c0 + pcol < C && s < (uint32_t)kRowBoundRows)
                    __hip_atomic_store(&a.bound[s * bld + c0 + pcol], sh.cm[pcol], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                load_bound(bw);
            }
            if (npass > 1) {  // the second pass is already loaded: group maxima over both
#pragma unroll
                for (int i = 0; i < NV; i += 2) {
                    m0.add(row_vec(nxt[i], 1u, i));
                    m1.add(row_vec(nxt[i + 1], 1u, i + 1));
                }
            }
#pragma unroll
            for (int j = 0; j < CPV; ++j) {
                sh.reps[g * CPV + j][rsub * 2] = m0.order(j);
                sh.reps[g * CPV + j][rsub * 2 + 1] = m1.order(j);
            }
            __syncthreads();
            constexpr int RPT = kRowReps / TPC;
            uint32_t v[RPT];
#pragma unroll
            for (int j = 0; j < RPT; ++j) v[j] = sh.reps[pcol][pq * RPT + j];
            uint32_t vmin = v[0], vmax = v[0];
#pragma unroll
            for (int j = 1; j < RPT; ++j) {
                vmin = min_u32(vmin, v[j]);
                vmax = max_u32(vmax, v[j]);
            }
            // all 64 are >= the minimum, and k <= 64
            const uint32_t cmax = group_max<TPC>(vmax);
            // The starting threshold: the bound where it holds (almost every
            // column), above the smallest group maximum (a valid threshold
            // by itself: 64 >= k elements reach it); the local k-th group
            // maximum only for the waves where some column has no bound yet.
            // (The local search is VALU work that the workgroups on a CU
            // would otherwise all do at once while the bound is in flight.)
            const uint32_t vlo = group_min<TPC>(vmin);
            uint32_t T;
            if (a.use_bound) {
                T = bound_kth(bw, vlo);
                if (__ballot(T <= vlo) != 0ull) T = max_u32(T, group_kth<TPC, RPT>(v, k, vlo, cmax));
            } else {
                T = group_kth<TPC, RPT>(v, k, vlo, cmax);
            }
            if (pq == 0) {
                uint32_t fmv, fqv;
                F::encode(T, fmv, fqv);
                sh.thr[pcol] = T;
                sh.fm[pcol] = (storage)fmv;
                sh.fq[pcol] = (storage)fqv;
                // a larger element of the segment (over both passes) for the
                // segments that read the bound later
                if (a.use_bound && c0 + pcol < C && s < (uint32_t)kRowBoundRows && cmax > sh.cm[pcol])
                    __hip_atomic_store(&a.bound[s * bld + c0 + pcol], cmax, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
            __syncthreads();
        }

        // (2) raw filter of every row vector; lanes with a passing element queue it
        {
            const u32x4 fmw = *reinterpret_cast<const u32x4*>(&sh.fm[g * CPV]);
            const u32x4 fqw = *reinterpret_cast<const u32x4*>(&sh.fq[g * CPV]);
            const uint32_t rbase = r_lo + p * per_pass + rsub;
            // A pass whose rows all lie in the segment is first filtered per
            // lane: the test is monotone, so the per-word maxima of the masked
            // patterns over the pass's rows pass iff some row does.  Only the
            // lanes that pass queue their row vectors, and the drain tests each
            // element exactly.  When more lanes pass than the queue holds, the
            // per-vector filter below runs instead.
            bool filtered = false;
            if (r_lo + (p + 1u) * per_pass <= r_hi) {  // the same for the whole workgroup
                auto lane_maxima = [&](auto masked_tag) {
                    constexpr bool MASKED = decltype(masked_tag)::value;
                    uint32_t wm[4] = {F::kSMin, F::kSMin, F::kSMin, F::kSMin};
#pragma unroll
                    for (int i = 0; i < NV; ++i) {
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const uint32_t w = word(cur[i], q);
                            wm[q] = F::smax(wm[q], MASKED ? w ^ word(fmw, q) : w);
                            nanacc[q] = F::umax(nanacc[q], w);
                        }
                    }
                    uint32_t any = 0;
#pragma unroll
                    for (int q = 0; q < 4; ++q) any |= F::test(wm[q], 0u, word(fqw, q));
                    return any;
                };
                // thresholds above the zero class need no mask (m = 0)
                const bool masked = __ballot((fmw.x | fmw.y | fmw.z | fmw.w) != 0u) != 0ull;
                const uint32_t any = masked ? lane_maxima(std::integral_constant<bool, true>{})
                                            : lane_maxima(std::integral_constant<bool, false>{});
                const bool has = any != 0u && ncols != 0u;
                const unsigned long long bal = __ballot(has);
                const uint32_t nq = (uint32_t)__popcll(bal) * (uint32_t)NV;
                if (nq <= (uint32_t)kRowQueue) {
                    if (has) {
                        const uint32_t base = lanes_below(bal) * (uint32_t)NV;
#pragma unroll
                        for (int i = 0; i < NV; ++i) {
                            sh.qdata[wave][base + (uint32_t)i] = cur[i];
                            sh.qmeta[wave][base + (uint32_t)i] = ((rbase + (uint32_t)i * kRowsPerStep) << 3) | g;
                        }
                    }
                    flush(nq);
                    filtered = true;
                }
            }
            uint32_t qcnt = 0;
#pragma unroll
            for (int i = 0; i < NV && !filtered; ++i) {
                const uint32_t r = rbase + (uint32_t)i * kRowsPerStep;
                uint32_t any = 0;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    any |= F::test(word(cur[i], q), word(fmw, q), word(fqw, q));
                    nanacc[q] = F::umax(nanacc[q], word(cur[i], q));
                }
                const bool has = any != 0u && r < r_hi && ncols != 0u;
                const unsigned long long bal = __ballot(has);
                if (bal) {
                    if (has) {
                        const uint32_t pos = qcnt + lanes_below(bal);
                        sh.qdata[wave][pos] = cur[i];
                        sh.qmeta[wave][pos] = (r << 3) | g;
                    }
                    qcnt += (uint32_t)__popcll(bal);
                    if (qcnt > (uint32_t)(kRowQueue - 64)) {
                        flush(qcnt);
                        qcnt = 0;
                    }
                }
            }
            if (!filtered) flush(qcnt);
        }
        __syncthreads();

        // (3) a column whose buffer overflowed in this pass is rebuilt from
        //     this pass's rows; before another pass, a column holding more
        //     than max(2k, 24) keys is trimmed to its running top-k
        {
            const uint32_t n = sh.cnt[pcol];
            if (p + 1 < npass && n <= (uint32_t)CAP && n > trim_at) {
                uint32_t T;
                const uint32_t kept = trim_column<DT, CAP, KT>(sh.cand[pcol], pq, n, k, sh.thr[pcol], &T);
                if (pq == 0) {
                    sh.cnt[pcol] = kept;
                    if (T > sh.thr[pcol]) {
                        uint32_t fmv, fqv;
                        F::encode(T, fmv, fqv);
                        sh.thr[pcol] = T;
                        sh.fm[pcol] = (storage)fmv;
                        sh.fq[pcol] = (storage)fqv;
                    }
                }
            }
            // the shared bound read at the top of the second pass;
            // candidates below it go at once (an overflowed column is left
            // to the rebuild below; the bound applies to it from the next
            // pass on)
            if (bound_late) {
                const uint32_t Tb = bound_kth(bw, sh.thr[pcol]);
                if (Tb > sh.thr[pcol] && sh.cnt[pcol] <= (uint32_t)CAP) {
                    const uint32_t kept = cull_column<DT, KT>(sh.cand[pcol], pq, sh.cnt[pcol], Tb);
                    if (pq == 0) {
                        uint32_t fmv, fqv;
                        F::encode(Tb, fmv, fqv);
                        sh.thr[pcol] = Tb;
                        sh.fm[pcol] = (storage)fmv;
                        sh.fq[pcol] = (storage)fqv;
                        sh.cnt[pcol] = kept;
                    }
                }
            }
            // sh.ovf was set before the barrier that ended (2), so every
            // thread reads the same value.  The rebuild of a column runs in
            // another wave than the threads that own its trim and bound step
            // above: a barrier separates the two.
            if (sh.ovf) {
                __syncthreads();
                if (tid == 0) sh.ovf = 0u;
                const uint32_t pass_lo = r_lo + p * per_pass;
                const uint32_t pass_hi = min_u32(pass_lo + per_pass, r_hi);
                uint64_t todo = wave_columns<TW>(wave, [&](uint32_t colx) {
                    return c0 + colx < C && sh.cnt[colx] > (uint32_t)CAP && (sh.flag[colx] & 1u) == 0u;
                });
                while (todo) {
                    const uint32_t colx = wave + (uint32_t)__builtin_ctzll(todo) * kWaves;
                    todo &= todo - 1ull;
                    rebuild_column<DT, NV, CAP, KT>(sh, x, a.ld, colx, c0 + colx, r_lo, pass_lo, pass_hi, k);
                }
            }
        }
        if (p + 1 < npass) {
            __syncthreads();
#pragma unroll
            for (int i = 0; i < NV; ++i) cur[i] = nxt[i];
        }
    }
    };
    if (full_tile)
        scan_passes(std::integral_constant<bool, true>{});
    else
        scan_passes(std::integral_constant<bool, false>{});

    // columns that hold a negative NaN take the exact path
#pragma unroll
    for (int j = 0; j < CPV; ++j)
        if ((uint32_t)j < ncols && F::has_negative_nan(nanacc[j * 4 / CPV], j % (CPV / 4)))
            atomicOr(&sh.flag[g * CPV + j], 2u);
    __syncthreads();

    // (4) the segment's top-k of every column, sorted
    uint64_t* lists = a.partials;
    {
        const uint32_t col = c0 + pcol;
        const uint32_t n = sh.cnt[pcol];
        if (col < C && sh.flag[pcol] == 0u && n <= (uint32_t)CAP) {
            typename KT::T* cand = sh.cand[pcol];
            uint32_t kept = n;
            if (n > max_u32(2u * k, 32u)) {  // many left: trim to k plus ties first
                uint32_t T;
                kept = trim_column<DT, CAP, KT>(cand, pq, n, k, sh.thr[pcol], &T);
            }
            // rank what is left and write the top k, sorted, to the segment's list
            uint64_t* dst = lists + ((int64_t)col * S + s) * k;
            rank_keys<KT>(cand, kept, k, dst, 1u, pq, TPC, r_lo);
            for (uint32_t t = kept + pq; t < k; t += TPC) dst[t] = 0ull;
        }
    }
    // flagged or overflowed columns: exact search over the segment, one wave per column
    uint64_t todo = wave_columns<TW>(wave, [&](uint32_t colx) {
        return c0 + colx < C && (sh.flag[colx] != 0u || sh.cnt[colx] > (uint32_t)CAP);
    });
    while (todo) {
        const uint32_t colx = wave + (uint32_t)__builtin_ctzll(todo) * kWaves;
        todo &= todo - 1ull;
        const uint32_t col = c0 + colx;
        // the wave's queue area (idle by now) is the exact search's scratch
        const uint32_t n = exact_row_column<DT>(x, a.ld, col, r_lo, r_hi, reinterpret_cast<uint64_t*>(sh.qdata[wave]),
                                                2u * kRowQueue, sh.tmp[wave], k);
        uint64_t* dst = lists + ((int64_t)col * S + s) * k;
        if (lane < k) dst[lane] = lane < n ? sh.tmp[wave][lane] : 0ull;
    }
}

// One workgroup per column: the top k of the column's S partial lists.  The
// four waves split the column's S*k list entries (coalesced: load j of wave
// w gives lane l entry (w*KW + j)*64 + l).  Each wave takes the same
// threshold, the k-th largest of the S list heads (each list is sorted, so k
// distinct entries reach it), and appends its entries at or above it to the
// workgroup's buffer behind the other waves' (one LDS atomic per wave).
// Wave 0 ranks them and writes the output.  A column whose candidates
// overflow the buffer (massive ties) is merged by wave 0 with the exact
// search over all entries, re-read from memory at each step.
template <class DT, int KPL>
__global__ __launch_bounds__(kBlock) void topk_row_merge(RowArgs a) {
    using storage = typename DT::storage;
    constexpr int OB = DT::kOrderBits;
    constexpr int KW = KPL / kWaves;  // loads per lane in each wave
    static_assert(KPL % kWaves == 0, "whole loads per wave");
    constexpr int kBuf = kMaxK + 192;
    __shared__ alignas(16) uint64_t cand[kBuf];
    __shared__ alignas(16) uint64_t best[kMaxK];
    __shared__ uint32_t ncand;
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    const uint32_t col = blockIdx.x;
    const uint32_t k = (uint32_t)a.k, S = (uint32_t)a.S, M = S * k;
    const uint64_t* src = a.partials + (int64_t)col * M;
    if (threadIdx.x == 0) ncand = 0;
    // The scan is over: clear the shared-bound words for the next run.  Row
    // r of the area is cleared by workgroup r mod C, in whole lines.
    if (a.use_bound) {
        for (uint32_t r = col; r < (uint32_t)kRowBoundRows; r += (uint32_t)a.C) {
            uint32_t* row = a.bound + (size_t)r * (uint32_t)a.bound_ld;
            for (uint32_t c = threadIdx.x; c < (uint32_t)a.C; c += kBlock) row[c] = 0u;
        }
    }
    uint64_t keys[KW];
#pragma unroll
    for (int j = 0; j < KW; ++j) {
        const uint32_t idx = (wave * (uint32_t)KW + (uint32_t)j) * 64u + lane;
        keys[j] = idx < M ? src[idx] : 0ull;
    }
    // the list heads, two per lane issued together (S <= 128 whenever
    // k >= 16), more in a loop
    const uint64_t h0 = lane < S ? src[lane * k] : 0ull;
    const uint64_t h1 = lane + 64u < S ? src[(lane + 64u) * k] : 0ull;
    uint64_t rep = max_u64(h0, h1);
    for (uint32_t sg = lane + 128u; sg < S; sg += 64u) rep = max_u64(rep, src[sg * k]);
    const uint32_t T = wave_kth_largest<OB>(key_order(rep), k);
    // sentinel entries (order 0, from segments with fewer than k rows) never qualify
    auto passes = [&](uint64_t key) { return key_order(key) != 0u && key_order(key) >= T; };
    uint32_t mine = 0;
#pragma unroll
    for (int j = 0; j < KW; ++j) mine += (uint32_t)__popcll(__ballot(passes(keys[j])));
    __syncthreads();  // ncand is zero
    uint32_t base = 0;
    if (lane == 0 && mine != 0u) base = atomicAdd(&ncand, mine);
    uint32_t cnt = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
#pragma unroll
    for (int j = 0; j < KW; ++j) cnt = wave_append(cand, cnt, (uint32_t)kBuf, passes(keys[j]), keys[j]);
    __syncthreads();
    if (wave != 0) return;

    const storage* x = static_cast<const storage*>(a.x);
    auto write_out = [&](uint32_t pos, uint64_t key) {
        const uint32_t row = key_row(key), o = key_order(key);
        static_cast<storage*>(a.out_values)[(int64_t)col * k + pos] =
            (storage)((o == DT::kZeroOrder || o == DT::kNanOrder) ? (uint32_t)x[(int64_t)row * a.ld + col]
                                                                  : DT::bits_from_order(o));
        a.out_ids[(int64_t)col * k + pos] = a.id_map ? a.id_map[row] : (int32_t)row;
    };
    const uint32_t n = ncand;
    if (n <= 64u) {
        // one candidate per lane: its rank decides its output slot
        const uint32_t n8 = (n + 7u) & ~7u;
        uint64_t key = 0;
        if (lane < n) key = cand[lane];
        else if (lane < n8) cand[lane] = 0;  // padding for the rank
        const uint32_t r = lds_rank_of(cand, n8, key);
        if (lane < n && r < k) write_out(r, key);
        return;
    }
    uint32_t m;
    if (n <= (uint32_t)kBuf) {
        m = wave_rank_select(cand, n, k, best);
    } else {
        auto visit = [&](auto&& f) {
#pragma unroll 1
            for (uint32_t i = lane; i < KPL * 64u; i += 64u) {
                const uint64_t key = i < M ? src[i] : 0ull;
                f(key, key_order(key) != 0u);
            }
        };
        m = wave_exact_topk<OB>(cand, (uint32_t)kBuf, best, visit, k);
    }
    if (lane < k && lane < m) write_out(lane, best[lane]);
}

template <class DT, int CAP, class KT>
hipError_t launch_scan(int nv, const RowArgs& a, hipStream_t stream) {
    const dim3 grid((uint32_t)((int64_t)a.tiles * a.S)), block(kBlock);
    switch (nv) {
        case 8: hipLaunchKernelGGL((topk_row_scan<DT, 8, CAP, KT>), grid, block, 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <class DT>
hipError_t launch_row_dt(int nv, const RowArgs& a, hipStream_t stream) {
    hipError_t e;
    if constexpr (DT::kOrderBits == 16) {
        if (a.key32)
            e = a.k <= kRowSmallK ? launch_scan<DT, 2 * kRowCapSmall, RowKey32>(nv, a, stream)
                                  : launch_scan<DT, kRowCapLarge, RowKey32>(nv, a, stream);
        else
            e = a.k <= kRowSmallK ? launch_scan<DT, kRowCapSmall, RowKey64>(nv, a, stream)
                                  : launch_scan<DT, kRowCapLarge, RowKey64>(nv, a, stream);
    } else {
        e = a.k <= kRowSmallK ? launch_scan<DT, kRowCapSmall, RowKey64>(nv, a, stream)
                              : launch_scan<DT, kRowCapLarge, RowKey64>(nv, a, stream);
    }
    if (e != hipSuccess) return e;
    // keys per lane: S*k entries over 64 lanes, in the smallest register
    // bucket that holds them (every slot is visited in the selection)
    const dim3 mgrid((uint32_t)a.C);
    const int64_t m = (int64_t)a.S * a.k;
    if (m <= 16 * 64)
        hipLaunchKernelGGL((topk_row_merge<DT, 16>), mgrid, dim3(kBlock), 0, stream, a);
    else if (m <= 20 * 64)
        hipLaunchKernelGGL((topk_row_merge<DT, 20>), mgrid, dim3(kBlock), 0, stream, a);
    else if (m <= 24 * 64)
        hipLaunchKernelGGL((topk_row_merge<DT, 24>), mgrid, dim3(kBlock), 0, stream, a);
    else
        hipLaunchKernelGGL((topk_row_merge<DT, kRowMaxMergeKeys / 64>), mgrid, dim3(kBlock), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

int row_tile_columns(int dtype) { return dtype == 0 ? RowTile<Bf16>::TW : RowTile<F32>::TW; }

hipError_t launch_row(int dtype, int nv, const RowArgs& a, hipStream_t stream) {
    return dtype == 0 ? launch_row_dt<Bf16>(nv, a, stream) : launch_row_dt<F32>(nv, a, stream);
}

}  // namespace topk
