// Row-interleaved top-k kernels for gfx950: element (r, c) at x[r*ld + c].
//
// This layout holds many independent rounds side by side: the column of each
// draft position is spread over V rows ld elements apart, and one 128-byte
// cache line holds 128 bytes of adjacent columns of one row.  Coalesced
// reads therefore see many columns at once, so a workgroup owns a tile of
// columns (128 bytes of each row: 64 bf16 or 32 fp32 columns) over a segment
// of rows, and each lane holds one 16-byte vector (8 or 4 columns) of a row
// per load.  A wave load covers 8 rows of the tile; the workgroup, 32 rows.
// The selection order is the same as for the column-contiguous kernel: larger
// value first, ties to the smaller row (ignis "DFlash2" page, "How it works").
//
// Scan kernel, one pass = NV row-steps of 32 rows:
//  1. Per lane and column, packed 16-bit (bf16) or 32-bit integer max/min of
//     the raw patterns over two interleaved row groups give two exact maxima
//     (the column's order at its largest element); 32 lanes hold each column,
//     so each column has 64 such representatives in the workgroup.
//  2. Four threads per column bit-search the k-th largest of the 64: a lower
//     bound on the column's k-th largest value in this pass, hence in the
//     segment.  The column's threshold T_c is the largest bound seen so far,
//     so it only rises.
//  3. Elements at or above T_c are appended, as 64-bit keys, to the column's
//     LDS buffer (a per-column LDS counter).  A lane compares its elements
//     only for columns whose lane maximum reaches T_c.
//  4. After the last pass each wave takes 1/4 of the tile's columns: the keys
//     still at or above the final T_c are rank-counted to the column's exact
//     top-k, which goes to the segment's slot of a partial list.
// A column whose buffer overflows (massive ties) is re-read from memory by
// one wave and selected by an exact wave-wide bit search.
//
// Merge kernel: one wave per column selects the top k of its S partial
// lists (k-th largest list maximum as threshold, then a rank count) and
// writes the output.  The kernel boundary orders it after the scan.
#include "topk_device.hpp"
#include "topk_internal.hpp"

namespace topk {

namespace {

constexpr int kRowLanesPerRow = 8;                    // 8 lanes x 16 bytes = one 128-byte line
constexpr int kRowsPerStep = kBlock / kRowLanesPerRow;  // 32 rows per workgroup load step
constexpr int kRowTileBytes = 128;
constexpr int kRowCap = 96;                           // candidate slots per column
constexpr int kRowRepsPerColumn = 2 * kRowsPerStep;   // two row groups per lane
constexpr int kRowMergeKeysPerLane = 16;              // S*k <= 1024 per column

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <class DT>
struct RowShape {
    static constexpr int kCols = kRowTileBytes / (int)sizeof(typename DT::storage);  // tile width
    static constexpr int kPerVec = DT::kPerVec;                                    // columns per lane
};

template <class DT>
struct RowShared {
    static constexpr int TW = RowShape<DT>::kCols;
    alignas(16) uint64_t cand[TW][kRowCap];   // per-column candidate keys
    alignas(16) uint64_t tmp[kWaves][kMaxK];   // per-wave selection output
    uint32_t reps[TW][kRowRepsPerColumn + 1];  // per-pass column maxima (orders); padded row
                                               // length spreads a column's reads over banks
    uint32_t thr[TW];                          // running column thresholds (orders)
    uint32_t cnt[TW];                          // candidates per column
};

__device__ __forceinline__ s16x2 as_s16x2_r(uint32_t w) { return __builtin_bit_cast(s16x2, w); }
__device__ __forceinline__ u16x2 as_u16x2_r(uint32_t w) { return __builtin_bit_cast(u16x2, w); }

// Element j (column) of a loaded vector, j known at compile time.
template <class DT>
__device__ __forceinline__ uint32_t row_elem(const u32x4& v, int j) {
    const uint32_t wx = v.x, wy = v.y, wz = v.z, ww = v.w;
    if constexpr (DT::kPerVec == 8) {
        const uint32_t w = j < 2 ? wx : j < 4 ? wy : j < 6 ? wz : ww;
        return (j & 1) ? (w >> 16) : (w & 0xFFFFu);
    } else {
        return j == 0 ? wx : j == 1 ? wy : j == 2 ? wz : ww;
    }
}

// Exact maximum order per column of one lane over a group of rows, from the
// raw patterns: the signed maximum when some pattern is non-negative, else the
// signed minimum (the least negative value); any negative NaN makes it the NaN
// class (which is the top of the order).
template <class DT>
struct ColMax {
    // bf16: two columns per packed register; fp32: one per register
    static constexpr int R = DT::kPerVec == 8 ? 4 : 4;
    uint32_t smax[R], smin[R], umax[R];
    __device__ void init() {
#pragma unroll
        for (int q = 0; q < R; ++q) {
            if constexpr (DT::kPerVec == 8) {
                smax[q] = 0x80008000u;  // two int16 minima
                smin[q] = 0x7FFF7FFFu;
                umax[q] = 0u;
            } else {
                smax[q] = 0x80000000u;
                smin[q] = 0x7FFFFFFFu;
                umax[q] = 0u;
            }
        }
    }
    __device__ void add(const u32x4& v) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < R; ++q) {
            if constexpr (DT::kPerVec == 8) {
                smax[q] = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(as_s16x2_r(smax[q]), as_s16x2_r(w[q])));
                smin[q] = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(as_s16x2_r(smin[q]), as_s16x2_r(w[q])));
                umax[q] = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(as_u16x2_r(umax[q]), as_u16x2_r(w[q])));
            } else {
                smax[q] = (uint32_t)max_i32((int)smax[q], (int)w[q]);
                smin[q] = (uint32_t)min_i32((int)smin[q], (int)w[q]);
                umax[q] = max_u32(umax[q], w[q]);
            }
        }
    }
    // exact maximum order of column j
    __device__ uint32_t order(int j) const {
        if constexpr (DT::kPerVec == 8) {
            const int q = j >> 1, sh = (j & 1) * 16;
            const int M = (int)(int16_t)(smax[q] >> sh);
            const int m = (int)(int16_t)(smin[q] >> sh);
            const uint32_t U = (umax[q] >> sh) & 0xFFFFu;
            if (U > 0xFF80u) return DT::kNanOrder;
            return M >= 0 ? DT::order((uint32_t)M) : DT::order((uint32_t)m & 0xFFFFu);
        } else {
            if (umax[j] > 0xFF800000u) return DT::kNanOrder;
            return (int)smax[j] >= 0 ? DT::order(smax[j]) : DT::order(smin[j]);
        }
    }
};

// Exact path for one column of a segment whose buffer overflowed: one wave
// re-reads the column's rows [r_lo, r_hi) (stride ld) at every step of an
// exact bit search.  Writes the column's top-k (sorted) to out, returns n.
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

template <class DT, int NV>
__global__ __launch_bounds__(kBlock) void topk_row_scan(RowArgs a) {
    using storage = typename DT::storage;
    constexpr int TW = RowShape<DT>::kCols;
    constexpr int CPV = DT::kPerVec;
    constexpr int OB = DT::kOrderBits;
    static_assert(NV % 2 == 0, "two row groups per pass");
    __shared__ RowShared<DT> sh;

    const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
    const uint32_t k = (uint32_t)a.k;
    const uint32_t tiles = (uint32_t)a.tiles;
    const uint32_t S = (uint32_t)a.S;
    const uint32_t s = blockIdx.x / tiles;          // row segment
    const uint32_t tile = blockIdx.x - s * tiles;   // column tile
    const uint32_t V = (uint32_t)a.V, C = (uint32_t)a.C;
    const uint32_t c0 = tile * TW;
    const uint32_t r_lo = (uint32_t)((uint64_t)V * s / S), r_hi = (uint32_t)((uint64_t)V * (s + 1) / S);
    const storage* x = static_cast<const storage*>(a.x);

    const uint32_t rsub = tid / kRowLanesPerRow;          // row within a 32-row step
    const uint32_t g = tid % kRowLanesPerRow;             // 16-byte group within the tile
    const uint32_t cg = c0 + g * CPV;                     // first column of this lane
    const uint32_t ncols = cg < C ? min_u32((uint32_t)CPV, C - cg) : 0u;  // valid columns of this lane
    const bool vec_ok = a.vec_loads != 0 && ncols == (uint32_t)CPV;

    for (uint32_t t = tid; t < (uint32_t)TW; t += kBlock) {
        sh.thr[t] = 0;
        sh.cnt[t] = 0;
    }
    __syncthreads();

    const uint32_t per_pass = (uint32_t)kRowsPerStep * NV;
    const uint32_t npass = r_hi > r_lo ? (r_hi - r_lo + per_pass - 1) / per_pass : 0u;
    for (uint32_t p = 0; p < npass; ++p) {
        const uint32_t rbase = r_lo + p * per_pass + rsub;
        u32x4 d[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const uint32_t r = rbase + (uint32_t)i * kRowsPerStep;
            const storage* src = x + (int64_t)r * a.ld + cg;
            if (r < r_hi && vec_ok) {
                d[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
            } else {
                // partial vector (row past the segment, columns past C, or an
                // unaligned layout): element loads, -Inf where nothing is read
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

        // (1) two representatives per column: even and odd row-steps
        ColMax<DT> m0, m1;
        m0.init();
        m1.init();
#pragma unroll
        for (int i = 0; i < NV; i += 2) {
            m0.add(d[i]);
            m1.add(d[i + 1]);
        }
        uint32_t lane_max[CPV];
#pragma unroll
        for (int j = 0; j < CPV; ++j) {
            const uint32_t o0 = m0.order(j), o1 = m1.order(j);
            lane_max[j] = max_u32(o0, o1);
            sh.reps[g * CPV + j][rsub * 2] = o0;
            sh.reps[g * CPV + j][rsub * 2 + 1] = o1;
        }
        __syncthreads();

        // (2) k-th largest of each column's 64 representatives; 4 threads per
        //     column, 16 representatives each, sums over the 4 with shuffles
        for (uint32_t col = tid / 4; col < (uint32_t)TW; col += kBlock / 4) {
            const uint32_t q = tid & 3u;
            uint32_t v[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) v[j] = sh.reps[col][q * 16 + j];
            uint32_t t = 0;
#pragma unroll 1
            for (int b = OB - 1; b >= 0; --b) {
                const uint32_t cand = t | (1u << b);
                uint32_t n = 0;
#pragma unroll
                for (int j = 0; j < 16; ++j) n += v[j] >= cand ? 1u : 0u;
                n += __shfl_xor(n, 1, 64);
                n += __shfl_xor(n, 2, 64);
                if (n >= k) t = cand;
            }
            if (q == 0 && t > sh.thr[col]) sh.thr[col] = t;
        }
        __syncthreads();

        // (3) append the elements at or above each column's threshold
        uint32_t thr[CPV];
#pragma unroll
        for (int j = 0; j < CPV; ++j) thr[j] = sh.thr[(g * CPV + j) % TW];
#pragma unroll
        for (int j = 0; j < CPV; ++j) {
            if ((uint32_t)j < ncols && lane_max[j] >= thr[j]) {
                const uint32_t colx = g * CPV + j;
#pragma unroll
                for (int i = 0; i < NV; ++i) {
                    const uint32_t r = rbase + (uint32_t)i * kRowsPerStep;
                    const uint32_t o = DT::order(row_elem<DT>(d[i], j));
                    if (r < r_hi && o >= thr[j]) {
                        const uint32_t pos = atomicAdd(&sh.cnt[colx], 1u);
                        if (pos < (uint32_t)kRowCap) sh.cand[colx][pos] = make_key(o, r, 0u);
                    }
                }
            }
        }
        __syncthreads();  // reps and thresholds are rewritten by the next pass
    }

    // (4) per column: exact top-k of the candidates still at or above T_c
    uint64_t* out_lists = a.partials;
    for (uint32_t colx = wave; colx < (uint32_t)TW; colx += kWaves) {
        const uint32_t col = c0 + colx;
        if (col >= C) break;
        uint64_t* dst = out_lists + ((int64_t)col * S + s) * k;
        const uint32_t total = sh.cnt[colx];
        uint32_t n;
        if (total > (uint32_t)kRowCap) {
            n = exact_row_column<DT>(x, a.ld, col, r_lo, r_hi, sh.cand[colx], kRowCap, sh.tmp[wave], k);
        } else {
            const uint64_t T = (uint64_t)sh.thr[colx] << 32;
            uint32_t m = 0;
            for (uint32_t b = 0; b < total; b += 64u) {
                const uint32_t t = b + lane;
                const uint64_t key = t < total ? sh.cand[colx][t] : 0ull;
                // compact in place (reads of this round precede its writes)
                m = wave_append(sh.cand[colx], m, kRowCap, t < total && key >= T, key);
            }
            n = wave_rank_select(sh.cand[colx], m, k, sh.tmp[wave]);
        }
        if (lane < k) dst[lane] = lane < n ? sh.tmp[wave][lane] : 0ull;
    }
}

// One wave per column: the top k of the column's S partial lists.
template <class DT>
__global__ __launch_bounds__(kBlock) void topk_row_merge(RowArgs a) {
    using storage = typename DT::storage;
    constexpr int OB = DT::kOrderBits;
    __shared__ alignas(16) uint64_t buf[kWaves][kMaxK + 192];
    __shared__ alignas(16) uint64_t tmp[kWaves][kMaxK];
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    const uint32_t col = blockIdx.x * kWaves + wave;
    if (col >= (uint32_t)a.C) return;
    const uint32_t k = (uint32_t)a.k, S = (uint32_t)a.S, M = S * k;
    const uint64_t* src = a.partials + (int64_t)col * M;
    uint64_t keys[kRowMergeKeysPerLane];
#pragma unroll
    for (int j = 0; j < kRowMergeKeysPerLane; ++j) {
        const uint32_t idx = (uint32_t)j * 64u + lane;
        keys[j] = idx < M ? src[idx] : 0ull;
    }
    uint64_t rep = 0;
#pragma unroll
    for (int j = 0; j < kRowMergeKeysPerLane; ++j) rep = max_u64(rep, keys[j]);
    const uint32_t T = wave_kth_largest<OB>(key_order(rep), k);
    auto visit = [&](auto&& f) {
#pragma unroll
        for (int j = 0; j < kRowMergeKeysPerLane; ++j) f(keys[j], key_order(keys[j]) != 0);
    };
    uint32_t cnt = 0;
    visit([&](uint64_t key, bool valid) { cnt = wave_append(buf[wave], cnt, kMaxK + 192, valid && key_order(key) >= T, key); });
    uint32_t n;
    if (cnt > (uint32_t)(kMaxK + 192))
        n = wave_exact_topk<OB>(buf[wave], kMaxK + 192, tmp[wave], visit, k);
    else
        n = wave_rank_select(buf[wave], cnt, k, tmp[wave]);
    if (lane < k && lane < n) {
        const uint64_t key = tmp[wave][lane];
        const uint32_t row = key_row(key), o = key_order(key);
        const storage* x = static_cast<const storage*>(a.x);
        static_cast<storage*>(a.out_values)[(int64_t)col * k + lane] =
            (storage)((o == DT::kZeroOrder || o == DT::kNanOrder) ? (uint32_t)x[(int64_t)row * a.ld + col]
                                                                  : DT::bits_from_order(o));
        a.out_ids[(int64_t)col * k + lane] = (int32_t)row;
    }
}

template <class DT>
hipError_t launch_row_dt(int nv, const RowArgs& a, hipStream_t stream) {
    const dim3 grid((uint32_t)((int64_t)a.tiles * a.S)), block(kBlock);
    switch (nv) {
        case 2: hipLaunchKernelGGL((topk_row_scan<DT, 2>), grid, block, 0, stream, a); break;
        case 4: hipLaunchKernelGGL((topk_row_scan<DT, 4>), grid, block, 0, stream, a); break;
        case 8: hipLaunchKernelGGL((topk_row_scan<DT, 8>), grid, block, 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((topk_row_merge<DT>), dim3((uint32_t)((a.C + kWaves - 1) / kWaves)), block, 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace

int row_tile_columns(int dtype) { return dtype == 0 ? RowShape<Bf16>::kCols : RowShape<F32>::kCols; }

hipError_t launch_row(int dtype, int nv, const RowArgs& a, hipStream_t stream) {
    return dtype == 0 ? launch_row_dt<Bf16>(nv, a, stream) : launch_row_dt<F32>(nv, a, stream);
}

}  // namespace topk
