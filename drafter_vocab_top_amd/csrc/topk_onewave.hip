// One wave per column: the top-k design that the ignis "DFlash2" page
// ("How it works", and the first row of "The numbers") measured as the
// bottleneck before its replacement: a single warp walked each of the seven
// columns, so seven warps carried the whole 3.47 MB.  It is kept here, on
// gfx950, as a baseline that the vocabulary-split kernels are compared
// against on the same part; it is never chosen automatically.
//
// One 64-lane workgroup per column.  Lane l reads the 16-byte vectors l,
// l + 64, l + 128, ... of the column (coalesced per wave) and keeps a sorted
// list of its KL best keys in registers, KL the smallest bucket >= k; an
// element enters the list only when its key beats the list's last entry.
// The wave then pops k times: a wave-wide maximum of the lane list heads,
// and the lane that owns it shifts its list up.  Keys are distinct, so
// exactly one lane owns each maximum.  The unaligned head and tail of a
// column (fewer than one vector each) are single elements of lanes 0..7
// and 32..39.
#include "topk_col_common.hpp"
#include "topk_device.hpp"
#include "topk_internal.hpp"

namespace topk {

namespace {

constexpr int kOneWaveUnroll = 4;  // vectors in flight per lane

// Insert key into the descending list L[0..KL) if it beats L[KL-1].
template <int KL>
__device__ __forceinline__ void list_insert(uint64_t (&L)[KL], uint64_t key) {
    if (key > L[KL - 1]) {
#pragma unroll
        for (int j = KL - 1; j > 0; --j)
            L[j] = key > L[j - 1] ? L[j - 1] : max_u64(key, L[j]);
        L[0] = max_u64(L[0], key);
    }
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, off, 64);
        const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), off, 64);
        v = max_u64(v, ((uint64_t)hi << 32) | lo);
    }
    return v;
}

template <class DT, int KL>
__global__ __launch_bounds__(64) void topk_onewave_kernel(ColArgs a) {
    using storage = typename DT::storage;
    constexpr int EPV = DT::kPerVec;
    const uint32_t lane = threadIdx.x;
    const uint32_t c = blockIdx.x;
    const uint32_t V = (uint32_t)a.V, k = (uint32_t)a.k;
    const storage* col = static_cast<const storage*>(a.x) + (int64_t)c * a.ld;

    uint32_t head = ((16u - ((uint32_t)(uintptr_t)col & 15u)) & 15u) / (uint32_t)sizeof(storage);
    if (head > V) head = V;
    const uint32_t nvec = (V - head) / EPV;
    const uint32_t tail0 = head + nvec * EPV;
    const u32x4* vec = reinterpret_cast<const u32x4*>(col + head);

    uint64_t L[KL];
#pragma unroll
    for (int j = 0; j < KL; ++j) L[j] = 0;  // below every real key

    if (lane < head) list_insert(L, make_key(DT::order(col[lane]), lane, 0));
    if (lane >= 32 && lane - 32 < V - tail0) {
        const uint32_t row = tail0 + (lane - 32);
        list_insert(L, make_key(DT::order(col[row]), row, 0));
    }

    for (uint32_t v0 = lane; v0 < nvec; v0 += 64u * kOneWaveUnroll) {
        u32x4 d[kOneWaveUnroll];
#pragma unroll
        for (int u = 0; u < kOneWaveUnroll; ++u) {
            const uint32_t vi = v0 + 64u * (uint32_t)u;
            d[u] = vi < nvec ? load_vec(vec + vi)
                             : u32x4{DT::kFillDword, DT::kFillDword, DT::kFillDword, DT::kFillDword};
        }
#pragma unroll
        for (int u = 0; u < kOneWaveUnroll; ++u) {
            const uint32_t vi = v0 + 64u * (uint32_t)u;
            if (vi < nvec) {
                const uint32_t row0 = head + vi * EPV;
#pragma unroll
                for (int e = 0; e < EPV; ++e)
                    list_insert(L, make_key(DT::order(vec_elem<DT>(d[u], e)), row0 + (uint32_t)e, 0));
            }
        }
    }

    // k pops of the largest list head.
    for (uint32_t j = 0; j < k; ++j) {
        const uint64_t top = wave_max_u64(L[0]);
        if (L[0] == top) {
#pragma unroll
            for (int i = 0; i + 1 < KL; ++i) L[i] = L[i + 1];
            L[KL - 1] = 0;
        }
        if (lane == 0) {
            const uint32_t row = key_row(top), o = key_order(top);
            static_cast<storage*>(a.out_values)[(int64_t)c * k + j] =
                (storage)((o == DT::kZeroOrder || o == DT::kNanOrder) ? (uint32_t)col[row]
                                                                      : DT::bits_from_order(o));
            a.out_ids[(int64_t)c * k + j] = a.id_map ? a.id_map[row] : (int32_t)row;
        }
    }
}

template <class DT>
hipError_t launch_dt(int32_t k, const ColArgs& a, hipStream_t stream) {
    const dim3 grid((uint32_t)a.C), block(64);
    if (k <= 1) hipLaunchKernelGGL((topk_onewave_kernel<DT, 1>), grid, block, 0, stream, a);
    else if (k <= 8) hipLaunchKernelGGL((topk_onewave_kernel<DT, 8>), grid, block, 0, stream, a);
    else if (k <= 16) hipLaunchKernelGGL((topk_onewave_kernel<DT, 16>), grid, block, 0, stream, a);
    else if (k <= 32) hipLaunchKernelGGL((topk_onewave_kernel<DT, 32>), grid, block, 0, stream, a);
    else if (k <= kMaxK) hipLaunchKernelGGL((topk_onewave_kernel<DT, kMaxK>), grid, block, 0, stream, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace

hipError_t launch_onewave(int dtype, const ColArgs& a, hipStream_t stream) {
    return dtype == 0 ? launch_dt<Bf16>(a.k, a, stream) : launch_dt<F32>(a.k, a, stream);
}

}  // namespace topk
