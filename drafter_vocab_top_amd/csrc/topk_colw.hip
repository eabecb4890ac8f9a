// Column-contiguous top-k with one wave per vocabulary segment, for matrices
// with many columns.
//
// Each column's 16-byte vectors are split into Sw = 4 S segments, one per
// wave of S workgroups, and every wave works on its own: no workgroup
// barriers, no shared candidate area.  The selection order is the one of the
// other kernels: larger value first, ties to the smaller row (ignis "DFlash2"
// page, "How it works").
//
// A wave streams its segment in passes of NV vectors per lane, and loads the
// next pass before it filters the current one.  Per pass:
//  1. Lane statistics: the exact maximum order of the lane's elements from
//     packed integer max/min of the raw patterns, and each vector's raw
//     signed maximum.
//  2. T = the k-th largest lane maximum (a ballot bit-search), raised to the
//     wave's running k-th best key once it holds k keys.
//  3. A vector whose maximum reaches T is appended, as a whole, to the
//     wave's LDS queue (ballot + mbcnt); the queue is then drained one vector
//     per lane: elements at or above T (integer interval test on the raw
//     pattern) become keys in the wave's candidate area, behind the k best
//     keys carried from earlier passes.
//  4. A rank count over the carried keys and the new candidates gives the
//     wave's running top-k.
// A negative NaN, or more candidates than the area holds, sends the pass to
// an exact wave-wide bit search (rare).
//
// Merge: each wave publishes its sorted k keys with device-scope stores and
// takes the column's ticket; the wave that draws the last one selects the
// top k of the Sw lists (a contiguous run of them per lane, the k-th largest
// lane maximum as threshold, a rank count) and writes the output.  The run
// tag in every key exposes a store that has not landed yet, as in the
// workgroup-level kernel.
#include "topk_col_common.hpp"
#include "topk_device.hpp"
#include "topk_internal.hpp"

namespace topk {

namespace {

constexpr int kWQueue = 128;                   // queued vectors per wave
constexpr int kWCand = 256;                    // carried best + candidates per wave
constexpr int kWMergePerLane = kWaveSegMergeKeys / 64;
constexpr int kWSpinLimit = 1 << 16;           // about 0.1 s: a store that has not landed by then never will

struct WaveArea {
    alignas(16) u32x4 qdata[kWQueue];  // queued vectors
    uint32_t qvec[kWQueue];            // their vector indices
    alignas(16) uint64_t cand[kWCand]; // [0, nbest) carried best, then new candidates
    alignas(16) uint64_t best[kMaxK];  // rank-selection output, sorted
};

struct ColWShared {
    WaveArea w[kWaves];
};

// Exact top-k of one pass of one wave: its vectors, its edge element and the
// keys carried from earlier passes.  Rare, so out of line; it re-reads the
// vectors at every step of the search.
template <class DT, int NV>
__device__ __noinline__ uint32_t exact_wave_pass(uint64_t* buf, uint64_t* out, const u32x4* vec, uint32_t v0,
                                                 uint32_t ve, uint32_t head, uint64_t ex, uint64_t carried,
                                                 uint32_t k, uint32_t tag) {
    constexpr int EPV = DT::kPerVec;
    auto visit = [&](auto&& f) {
#pragma unroll 1
        for (int i = 0; i < NV; ++i) {
            const uint32_t vi = v0 + (uint32_t)i * 64u;
            const bool valid = vi < ve;
            const u32x4 v = valid ? vec[vi] : u32x4{0u, 0u, 0u, 0u};
            const uint32_t row0 = head + vi * EPV;
#pragma unroll
            for (int e = 0; e < EPV; ++e) f(make_key(DT::order(vec_elem<DT>(v, e)), row0 + e, tag), valid);
        }
        f(ex, ex != 0);
        f(carried, carried != 0);
    };
    return wave_exact_topk<DT::kOrderBits>(buf, kWCand, out, visit, k);
}

template <class DT, int NV>
__global__ __launch_bounds__(kBlock) void topk_colw_kernel(ColArgs a) {
    using storage = typename DT::storage;
    constexpr int EPV = DT::kPerVec;
    constexpr int OB = DT::kOrderBits;
    __shared__ ColWShared sh;

    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    const uint32_t k = (uint32_t)a.k, tag = a.tag;
    const uint32_t S = (uint32_t)a.S;             // workgroups per column
    const uint32_t Sw = S * kWaves;               // wave segments per column
    const uint32_t c = blockIdx.x / S;
    const uint32_t ws = (blockIdx.x - c * S) * kWaves + wave;
    const uint32_t V = (uint32_t)a.V;
    const storage* col = static_cast<const storage*>(a.x) + (int64_t)c * a.ld;

    // unaligned head, 16-byte vectors, tail
    uint32_t head = ((16u - ((uint32_t)(uintptr_t)col & 15u)) & 15u) / (uint32_t)sizeof(storage);
    if (head > V) head = V;
    const uint32_t nvec = (V - head) / EPV;
    const uint32_t tail0 = head + nvec * EPV;
    const uint32_t vb = (uint32_t)((uint64_t)nvec * ws / Sw), ve = (uint32_t)((uint64_t)nvec * (ws + 1) / Sw);
    const u32x4* vec = reinterpret_cast<const u32x4*>(col + head);

    // head rows go to the lanes of the first segment, tail rows to the last
    uint64_t edge = 0;
    {
        uint32_t row = 0xFFFFFFFFu;
        if (ws == 0 && lane < head) row = lane;
        if (ws == Sw - 1 && lane >= 32 && lane - 32 < V - tail0) row = tail0 + (lane - 32);
        if (row != 0xFFFFFFFFu) edge = make_key(DT::order(col[row]), row, tag);
    }

    WaveArea& W = sh.w[wave];
    uint32_t nbest = 0;   // carried best keys, in W.cand[0, nbest) at the start of a pass
    uint64_t t_run = 0;   // the k-th best key once nbest == k
    const uint32_t per_pass = 64u * NV;
    const uint32_t npass = ve > vb ? (ve - vb + per_pass - 1) / per_pass : 1u;

    auto load_pass = [&](u32x4(&d)[NV], uint32_t p) {
        const uint32_t v0 = vb + p * per_pass + lane;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const uint32_t vi = v0 + (uint32_t)i * 64u;
            d[i] = vi < ve ? load_vec(vec + vi)
                           : u32x4{DT::kFillDword, DT::kFillDword, DT::kFillDword, DT::kFillDword};
        }
    };

    u32x4 cur[NV], nxt[NV];
    load_pass(cur, 0);
    for (uint32_t p = 0; p < npass; ++p) {
        if (p + 1 < npass) load_pass(nxt, p + 1);
        const uint32_t v0 = vb + p * per_pass + lane;
        const int nvalid = ve > v0 ? (int)min_u32((uint32_t)NV, (ve - v0 + 63u) / 64u) : 0;
        const uint64_t ex = p == 0 ? edge : 0;

        uint32_t vmax[NV];
        uint32_t rep;
        bool neg_nan;
        lane_stats<DT, NV>(cur, vmax, rep, neg_nan);
        if (ex) rep = max_u32(rep, key_order(ex));
        uint32_t T = wave_kth_bound<DT>(rep, k);
        if (nbest == k) T = max_u32(T, key_order(t_run));
        const uint64_t tc = max_u64((uint64_t)T << 32, nbest == k ? t_run + 1 : (uint64_t)0);

        bool exact = __any(neg_nan);
        uint32_t cnt = 0;  // new candidates, in W.cand[nbest, nbest + cnt)
        if (!exact) {
            RawFilter<DT> f;
            f.set(T);
            uint32_t qcnt = 0;  // wave-uniform
            auto drain = [&]() {
                for (uint32_t b = 0; b < qcnt; b += 64u) {
                    const uint32_t e = b + lane;
                    u32x4 v = {0u, 0u, 0u, 0u};
                    uint32_t m = 0, row0 = 0;
                    if (e < qcnt) {
                        v = W.qdata[e];
                        row0 = head + W.qvec[e] * EPV;
#pragma unroll
                        for (int el = 0; el < EPV; ++el) m |= f.pass(vec_elem<DT>(v, el)) ? (1u << el) : 0u;
                    }
                    while (__any(m != 0)) {
                        const uint32_t el = m != 0 ? (uint32_t)__builtin_ctz(m) : 0u;
                        const uint64_t key = make_key(DT::order(vec_elem_dyn<DT>(v, el)), row0 + el, tag);
                        cnt = wave_append(W.cand + nbest, cnt, (uint32_t)kWCand - nbest, m != 0 && key >= tc, key);
                        m &= m - 1u;
                    }
                }
                qcnt = 0;
            };
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const bool pv = i < nvalid && (!f.positive || vec_max_signed<DT>(vmax[i]) >= (int)f.lo);
                const unsigned long long bal = __ballot(pv);
                if (bal) {
                    if (pv) {
                        const uint32_t pos = qcnt + lanes_below(bal);
                        W.qdata[pos] = cur[i];
                        W.qvec[pos] = v0 + (uint32_t)i * 64u;
                    }
                    qcnt += (uint32_t)__popcll(bal);
                    if (qcnt > (uint32_t)(kWQueue - 64)) drain();
                }
            }
            drain();
            cnt = wave_append(W.cand + nbest, cnt, (uint32_t)kWCand - nbest, ex != 0 && ex >= tc, ex);
            exact = nbest + cnt > (uint32_t)kWCand;
        }
        uint32_t n;
        if (exact) {
            const uint64_t carried = lane < nbest ? W.cand[lane] : 0ull;
            n = exact_wave_pass<DT, NV>(W.cand, W.best, vec, v0, ve, head, ex, carried, k, tag);
        } else {
            n = wave_rank_select(W.cand, nbest + cnt, k, W.best);
        }
        nbest = n;
        if (nbest == k) t_run = W.best[k - 1];
        if (p + 1 < npass) {
            if (lane < nbest) W.cand[lane] = W.best[lane];
#pragma unroll
            for (int i = 0; i < NV; ++i) cur[i] = nxt[i];
        }
    }

    // ---- publish the segment's sorted list, then take the column's ticket ----
    uint64_t* parts = a.partials + (int64_t)c * Sw * k;
    if (lane < k)
        __hip_atomic_store(&parts[ws * k + lane], lane < nbest ? W.best[lane] : (uint64_t)tag,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t last = 0;
    if (lane == 0) {
        const uint32_t old = __hip_atomic_fetch_add(&a.tickets[c * kTicketStride], 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        last = old == Sw - 1u ? 1u : 0u;
    }
    if (__builtin_amdgcn_readfirstlane(last) == 0u) return;

    // ---- the column's last wave: select from the Sw published lists ----
    const uint32_t M = Sw * k;
    const uint32_t R = (M + 63u) / 64u;  // keys per lane, a contiguous run (wave-uniform)
    uint64_t keys[kWMergePerLane];
#pragma unroll
    for (int j = 0; j < kWMergePerLane; ++j) {
        const uint32_t idx = lane * R + (uint32_t)j;
        keys[j] = 0;
        if ((uint32_t)j < R && idx < M) keys[j] = load_published(parts + idx);
    }
#pragma unroll
    for (int j = 0; j < kWMergePerLane; ++j) {
        const uint32_t idx = lane * R + (uint32_t)j;
        if ((uint32_t)j < R && idx < M) {
            for (int spin = 0; key_tag(keys[j]) != tag && spin < kWSpinLimit; ++spin) {
                __builtin_amdgcn_s_sleep(1);
                keys[j] = load_published(parts + idx);
            }
        }
    }
    uint64_t rep = 0;
#pragma unroll
    for (int j = 0; j < kWMergePerLane; ++j)
        if ((uint32_t)j < R) rep = max_u64(rep, keys[j]);
    const uint32_t T = wave_kth_bound<DT>(key_order(rep), k);
    // sentinel keys (order 0, from segments with fewer than k rows) never qualify
    auto visit = [&](auto&& f) {
#pragma unroll
        for (int j = 0; j < kWMergePerLane; ++j)
            if ((uint32_t)j < R) f(keys[j], key_order(keys[j]) != 0);
    };
    uint32_t cnt = 0;
    visit([&](uint64_t key, bool valid) {
        cnt = wave_append(W.cand, cnt, (uint32_t)kWCand, valid && key_order(key) >= T, key);
    });
    const uint32_t n = cnt > (uint32_t)kWCand ? wave_exact_topk<OB>(W.cand, kWCand, W.best, visit, k)
                                              : wave_rank_select(W.cand, cnt, k, W.best);
    if (lane < k && lane < n) {
        const uint64_t key = W.best[lane];
        const uint32_t row = key_row(key), o = key_order(key);
        static_cast<storage*>(a.out_values)[(int64_t)c * k + lane] =
            (storage)((o == DT::kZeroOrder || o == DT::kNanOrder) ? (uint32_t)col[row] : DT::bits_from_order(o));
        a.out_ids[(int64_t)c * k + lane] = a.id_map ? a.id_map[row] : (int32_t)row;
    }
    if (lane == 0)
        __hip_atomic_store(&a.tickets[c * kTicketStride], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <class DT>
hipError_t launch_w(int nv, const ColArgs& a, hipStream_t stream) {
    const dim3 grid((uint32_t)((int64_t)a.C * a.S)), block(kBlock);
    switch (nv) {
        case 2: hipLaunchKernelGGL((topk_colw_kernel<DT, 2>), grid, block, 0, stream, a); break;
        case 4: hipLaunchKernelGGL((topk_colw_kernel<DT, 4>), grid, block, 0, stream, a); break;
        case 8: hipLaunchKernelGGL((topk_colw_kernel<DT, 8>), grid, block, 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_colw(int dtype, int nv, const ColArgs& a, hipStream_t stream) {
    return dtype == 0 ? launch_w<Bf16>(nv, a, stream) : launch_w<F32>(nv, a, stream);
}

}  // namespace topk
