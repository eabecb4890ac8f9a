// Column-contiguous top-k kernel for gfx950.
//
// The ignis "DFlash2" page ("How it works") explains why the replacement
// top-k was fast: it split each column's vocabulary rows across workgroups
// and kept k in registers.  This kernel keeps the split and does the rest
// differently.  Each column's V rows are cut into S segments, and one 256-lane
// workgroup scans each segment, so C*S workgroups fill the 256 CUs even at
// C = 7.  A workgroup reduces its segment to a sorted top-k; the last
// workgroup of each column to finish merges the S partial lists and writes
// the answer.
//
// A scan pass, per workgroup:
//  1. Every lane loads NV 16-byte vectors with coalesced loads.  Vectors are
//     aligned to 16 bytes; the unaligned head and tail rows of the column
//     (fewer than one vector each) go to a few lanes of the first and last
//     segment as single "edge" elements.
//  2. Each lane takes the exact maximum order of its elements with packed
//     16-bit (bf16) or 32-bit integer max/min on the raw bit patterns, never
//     on converted floats.  The signed-integer maximum of raw patterns is the
//     largest non-negative value; when a lane holds only negative patterns,
//     the signed minimum is its largest value.
//  3. Each wave finds the k-th largest lane maximum with a ballot bit-search,
//     and the workgroup takes the largest of those.  The result T is a lower
//     bound on the workgroup's k-th largest value.  Any element below T
//     cannot be in the top-k.
//  4. Elements whose value is at least T (usually about k to 2k of them) are
//     appended as 64-bit keys to an LDS buffer.  They are found with a
//     per-vector prefilter and an integer interval test on the raw pattern.
//  5. A rank count over the buffer picks the exact top-k.  It is carried as
//     a running threshold into the next pass, if the segment needs several.
// Negative NaNs, or more candidates than the buffer holds (massive ties),
// switch that pass to an exact block-wide bit search over the keys.
//
// Cross-workgroup merge without cache-flushing fences.  Each workgroup
// publishes its k keys with device-scope atomic stores, which write through
// the XCD's L2.  It then increments the column's ticket.  Every key carries
// the run's tag, so the workgroup that draws the last ticket reads the other
// lists with device-scope loads and re-reads any slot whose tag is stale
// until its store lands.  That workgroup merges the lists, writes the output
// and resets the ticket for the next run.
#include "topk_device.hpp"
#include "topk_internal.hpp"

namespace topk {

namespace {

struct ColShared {
    uint64_t cand[kCandCap];   // candidate keys
    uint64_t best[kMaxK];      // current top-k, sorted
    uint32_t wave_thr[kWaves];
    uint32_t red[3];           // block_sum rotation slots
    uint32_t flags[2];         // per-pass "exact path needed" flags, alternating
    uint32_t cnt;
    uint32_t is_last;
};

constexpr int kSpinLimit = 1 << 16;  // about 0.1 s: a store that has not landed by then never will
constexpr int kMergeKeysPerThread = kMaxMergeKeys / kBlock;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 load_vec(const u32x4* p) { return __builtin_nontemporal_load(p); }

// Raw pattern of element e (0 <= e < kPerVec) of a loaded vector.
template <class DT>
__device__ __forceinline__ uint32_t vec_elem(const u32x4& v, int e) {
    const uint32_t w = e < DT::kPerVec / 4 ? v.x
                     : e < 2 * DT::kPerVec / 4 ? v.y
                     : e < 3 * DT::kPerVec / 4 ? v.z : v.w;
    if constexpr (DT::kPerVec == 8) return (e & 1) ? (w >> 16) : (w & 0xFFFFu);
    else return w;
}

__device__ __forceinline__ s16x2 as_s16x2(uint32_t w) { return __builtin_bit_cast(s16x2, w); }
__device__ __forceinline__ u16x2 as_u16x2(uint32_t w) { return __builtin_bit_cast(u16x2, w); }

// Lane statistics of one pass (see step 2 above).
//   vmax[i]: raw signed maximum of vector i (bf16: two 16-bit halves packed)
//   rep:     exact maximum order over the lane's elements, unless the lane
//            holds a negative NaN (then neg_nan is set and rep is unused)
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
        const int M = max((int)smax.x, (int)smax.y);
        const int m = min((int)smin.x, (int)smin.y);
        rep = M >= 0 ? order_bf16((uint32_t)M) : order_bf16((uint32_t)m & 0xFFFFu);
        neg_nan = max((uint32_t)umax.x, (uint32_t)umax.y) > 0xFF80u;
    } else {
        int smax = INT32_MIN, smin = INT32_MAX;
        uint32_t umax = 0;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int a = (int)d[i].x, b = (int)d[i].y, c = (int)d[i].z, e = (int)d[i].w;
            const int mx = max(max(a, b), max(c, e));
            vmax[i] = (uint32_t)mx;
            smax = max(smax, mx);
            smin = min(smin, min(min(a, b), min(c, e)));
            umax = max(umax, max(max(d[i].x, d[i].y), max(d[i].z, d[i].w)));
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
        return max((int)h.x, (int)h.y);
    } else {
        return (int)vm;
    }
}

__device__ __forceinline__ void append(ColShared& sh, uint64_t key) {
    const uint32_t idx = atomicAdd(&sh.cnt, 1u);
    if (idx < (uint32_t)kCandCap) sh.cand[idx] = key;
}

// Exact top-k of the keys the threads hold: a block-wide bit search for the
// k-th largest key, then a rank count of the (at most k) keys at or above it.
// visit(f) calls f(key) for every key the calling thread holds.  Writes
// sh.best[0..n) sorted and returns n = min(k, number of keys).  Keys must be
// distinct, apart from identical sentinels that never reach the top k.
template <int OrderBits, class Visit>
__device__ uint32_t exact_topk(ColShared& sh, const Visit& visit, uint32_t k, uint32_t& phase) {
    uint32_t local = 0;
    visit([&](uint64_t) { ++local; });
    const uint32_t total = block_sum(local, sh.red, phase);
    uint64_t thr = 0;
    if (total > k) {
        for (int b = 32 + OrderBits - 1; b >= 8; --b) {
            const uint64_t cand = thr | (1ull << b);
            uint32_t n = 0;
            visit([&](uint64_t key) { n += key >= cand ? 1u : 0u; });
            if (block_sum(n, sh.red, phase) >= k) thr = cand;
        }
    }
    if (threadIdx.x == 0) sh.cnt = 0;
    __syncthreads();
    visit([&](uint64_t key) {
        if (key >= thr) append(sh, key);
    });
    __syncthreads();
    const uint32_t n = min(sh.cnt, (uint32_t)kCandCap);
    rank_select(sh.cand, n, k, sh.best);
    __syncthreads();
    return min(n, k);
}

// Device-scope load of a published key, re-read until it carries this run's tag.
__device__ __forceinline__ uint64_t load_published(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <class DT, int NV>
__global__ __launch_bounds__(kBlock) void topk_col_kernel(ColArgs a) {
    using storage = typename DT::storage;
    constexpr int EPV = DT::kPerVec;
    constexpr int OB = DT::kOrderBits;
    __shared__ ColShared sh;

    const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
    const uint32_t k = (uint32_t)a.k;
    const uint32_t tag = a.tag;
    const int64_t c = blockIdx.x / a.S;
    const int64_t s = blockIdx.x % a.S;
    const int64_t V = a.V;
    const storage* col = static_cast<const storage*>(a.x) + c * a.ld;

    // Split the column into an unaligned head, 16-byte vectors and a tail.
    int64_t head = (int64_t)(((16u - ((uint32_t)(uintptr_t)col & 15u)) & 15u) / sizeof(storage));
    if (head > V) head = V;
    const int64_t nvec = (V - head) / EPV;
    const int64_t tail0 = head + nvec * EPV;
    const int64_t vb = nvec * s / a.S, ve = nvec * (s + 1) / a.S;
    const u32x4* vec = reinterpret_cast<const u32x4*>(col + head);

    uint64_t edge = 0;  // this lane's edge element, or 0
    {
        int64_t row = -1;
        if (s == 0 && (int64_t)tid < head) row = tid;
        if (s == a.S - 1 && tid >= 32 && (int64_t)(tid - 32) < V - tail0) row = tail0 + (tid - 32);
        if (row >= 0) edge = make_key(DT::order(col[row]), (uint32_t)row, tag);
    }

    if (tid == 0) {
        sh.red[0] = sh.red[1] = sh.red[2] = 0;
        sh.flags[0] = sh.flags[1] = 0;
    }
    __syncthreads();
    uint32_t phase = 0;
    uint32_t nbest = 0;   // keys carried in sh.cand[0..nbest) from earlier passes
    uint64_t t_run = 0;   // carried k-th best key (valid when nbest == k)
    const int64_t per_pass = (int64_t)kBlock * NV;
    const int64_t span = ve - vb;
    const int64_t npass = span > 0 ? (span + per_pass - 1) / per_pass : 1;

    for (int64_t p = 0; p < npass; ++p) {
        const int64_t v0 = vb + p * per_pass + tid;
        u32x4 d[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int64_t vi = v0 + (int64_t)i * kBlock;
            d[i] = vi < ve ? load_vec(vec + vi)
                           : u32x4{DT::kFillDword, DT::kFillDword, DT::kFillDword, DT::kFillDword};
        }
        const int nvalid = ve > v0 ? (int)min((int64_t)NV, (ve - v0 + kBlock - 1) / kBlock) : 0;
        const uint64_t ex = p == 0 ? edge : 0;
        const uint32_t fl = (uint32_t)(p & 1);

        uint32_t vmax[NV];
        uint32_t rep;
        bool neg_nan;
        lane_stats<DT, NV>(d, vmax, rep, neg_nan);
        if (ex) rep = max(rep, key_order(ex));
        const uint32_t wt = wave_kth_largest<OB>(rep, k);
        const bool any_nan = __ballot(neg_nan) != 0ull;
        if (lane == 0) {
            sh.wave_thr[wave] = wt;
            if (any_nan) atomicOr(&sh.flags[fl], 1u);
        }
        if (tid == 0) {
            sh.cnt = nbest;
            sh.flags[fl ^ 1u] = 0;
        }
        __syncthreads();

        uint32_t T = sh.wave_thr[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) T = max(T, sh.wave_thr[w]);
        if (nbest == k) T = max(T, key_order(t_run));
        const uint64_t tc = max((uint64_t)T << 32, nbest == k ? t_run + 1 : 0ull);
        const bool exact = sh.flags[fl] != 0;
        if (!exact) {
            RawFilter<DT> f;
            f.set(T);
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                if (i < nvalid && (!f.positive || vec_max_signed<DT>(vmax[i]) >= (int)f.lo)) {
                    const int64_t row0 = head + (v0 + (int64_t)i * kBlock) * EPV;
#pragma unroll
                    for (int e = 0; e < EPV; ++e) {
                        const uint32_t raw = vec_elem<DT>(d[i], e);
                        if (f.pass(raw)) {
                            const uint64_t key = make_key(DT::order(raw), (uint32_t)(row0 + e), tag);
                            if (key >= tc) append(sh, key);
                        }
                    }
                }
            }
            if (ex != 0 && ex >= tc) append(sh, ex);
        }
        __syncthreads();

        const uint32_t cnt = sh.cnt;
        uint32_t nb;
        if (exact || cnt > (uint32_t)kCandCap) {
            const uint64_t carried = tid < nbest ? sh.cand[tid] : 0ull;
            auto visit = [&](auto&& f) {
#pragma unroll
                for (int i = 0; i < NV; ++i) {
                    if (i < nvalid) {
                        const int64_t row0 = head + (v0 + (int64_t)i * kBlock) * EPV;
#pragma unroll
                        for (int e = 0; e < EPV; ++e)
                            f(make_key(DT::order(vec_elem<DT>(d[i], e)), (uint32_t)(row0 + e), tag));
                    }
                }
                if (ex) f(ex);
                if (carried) f(carried);
            };
            nb = exact_topk<OB>(sh, visit, k, phase);
        } else {
            rank_select(sh.cand, cnt, k, sh.best);
            __syncthreads();
            nb = min(cnt, k);
        }
        if (p + 1 < npass && tid < nb) sh.cand[tid] = sh.best[tid];
        nbest = nb;
        if (nb == k) t_run = sh.best[k - 1];
    }

    // ---- publish ----
    storage* out_v = static_cast<storage*>(a.out_values) + c * k;
    int32_t* out_i = a.out_ids + c * k;
    if (a.S == 1) {
        if (tid < k) {
            const uint64_t key = sh.best[tid];
            const uint32_t row = key_row(key), o = key_order(key);
            out_v[tid] = (storage)((o == DT::kZeroOrder || o == DT::kNanOrder) ? (uint32_t)col[row]
                                                                               : DT::bits_from_order(o));
            out_i[tid] = (int32_t)row;
        }
        return;
    }
    const uint64_t sentinel = tag;  // order 0: below every real key
    uint64_t* col_parts = a.partials + c * a.S * (int64_t)k;
    if (tid < k)
        __hip_atomic_store(&col_parts[s * k + tid], tid < nbest ? sh.best[tid] : sentinel,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid == 0) {
        const uint32_t old = __hip_atomic_fetch_add(&a.tickets[c], 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        sh.is_last = old == (uint32_t)(a.S - 1) ? 1u : 0u;
    }
    __syncthreads();
    if (!sh.is_last) return;

    // ---- last workgroup of the column: merge the S lists ----
    const uint32_t total = (uint32_t)a.S * k;
    uint64_t keys[kMergeKeysPerThread];
#pragma unroll
    for (int j = 0; j < kMergeKeysPerThread; ++j) {
        const uint32_t idx = tid + (uint32_t)j * kBlock;
        keys[j] = 0;
        if (idx < total) {
            const uint32_t seg = idx / k, slot = idx - seg * k;
            if ((int64_t)seg == s) keys[j] = slot < nbest ? sh.best[slot] : sentinel;
            else keys[j] = load_published(&col_parts[idx]);
        }
    }
#pragma unroll
    for (int j = 0; j < kMergeKeysPerThread; ++j) {
        const uint32_t idx = tid + (uint32_t)j * kBlock;
        if (idx < total) {
            for (int spin = 0; key_tag(keys[j]) != tag && spin < kSpinLimit; ++spin) {
                __builtin_amdgcn_s_sleep(1);
                keys[j] = load_published(&col_parts[idx]);
            }
        }
    }
    uint64_t rep = 0;
#pragma unroll
    for (int j = 0; j < kMergeKeysPerThread; ++j) rep = max(rep, keys[j]);
    const uint32_t wt = wave_kth_largest<OB>(key_order(rep), k);
    if (lane == 0) sh.wave_thr[wave] = wt;
    if (tid == 0) sh.cnt = 0;
    __syncthreads();
    uint32_t T = sh.wave_thr[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) T = max(T, sh.wave_thr[w]);
#pragma unroll
    for (int j = 0; j < kMergeKeysPerThread; ++j)
        if (keys[j] != 0 && key_order(keys[j]) >= T) append(sh, keys[j]);
    __syncthreads();
    const uint32_t cnt = sh.cnt;
    if (cnt > (uint32_t)kCandCap) {
        auto visit = [&](auto&& f) {
#pragma unroll
            for (int j = 0; j < kMergeKeysPerThread; ++j)
                if (keys[j] != 0) f(keys[j]);
        };
        exact_topk<OB>(sh, visit, k, phase);
    } else {
        rank_select(sh.cand, cnt, k, sh.best);
        __syncthreads();
    }
    if (tid < k) {
        const uint64_t key = sh.best[tid];
        const uint32_t row = key_row(key), o = key_order(key);
        out_v[tid] = (storage)((o == DT::kZeroOrder || o == DT::kNanOrder) ? (uint32_t)col[row]
                                                                           : DT::bits_from_order(o));
        out_i[tid] = (int32_t)row;
    }
    if (tid == 0) __hip_atomic_store(&a.tickets[c], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

hipError_t launch_col_bf16(const ColArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((topk_col_kernel<Bf16, kColVecsPerThread>), dim3((uint32_t)(a.C * a.S)),
                       dim3(kBlock), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_col_f32(const ColArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((topk_col_kernel<F32, kColVecsPerThread>), dim3((uint32_t)(a.C * a.S)),
                       dim3(kBlock), 0, stream, a);
    return hipGetLastError();
}

}  // namespace topk
