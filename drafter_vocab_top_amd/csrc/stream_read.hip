// A plain streaming read of a buffer, for measurement only: the achievable
// HBM read rate on this part for a given number of bytes, read once, cold.
// It is not part of the top-k path and the top-k library does not use it;
// the benchmark times it beside the top-k over the same bytes.
//
// Each workgroup reads one contiguous chunk of the buffer; per step every
// lane issues eight 16-byte non-temporal loads, 256 lanes x 16 bytes apart
// (coalesced), and folds them with xor (one ALU op per dword), so the loads
// cannot be removed; one conditional store that practically never happens
// keeps the fold alive.  The benchmark tries a few workgroup counts and
// keeps the fastest, so the yardstick is the best this plain read achieves.
//
// C ABI (built into libstream_read.so, loaded only by the benchmark):
//   int stream_read_run(const void* x, int64_t bytes, int64_t blocks,
//                       uint32_t* sink, hipStream_t stream)
//     x: device pointer, 16-byte aligned; bytes: a multiple of 16, >= 16;
//     blocks: workgroups, 1 .. 65,536 (each reads a contiguous chunk);
//     sink: device, one uint32 that the kernel may write; returns 0, -1 for
//     a bad argument, -3 when the launch fails.
//   int stream_read_empty(hipStream_t stream)
//     launches one workgroup of an empty kernel: the launch floor under the
//     same eager launches as the top-k; returns 0, -3 when the launch fails.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;
constexpr int64_t kStep = (int64_t)kThreads * kUnroll;  // vectors per workgroup step

__device__ __forceinline__ uint32_t fold(const u32x4& v) {
    const uint32_t a = v.x, b = v.y, c = v.z, d = v.w;
    return a ^ b ^ c ^ d;
}

// Workgroup b reads vectors [b*chunk, min((b+1)*chunk, nvec)).
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* x, int64_t nvec, int64_t chunk,
                                                               uint32_t* sink) {
    const int64_t lo = (int64_t)blockIdx.x * chunk;
    const int64_t hi = lo + chunk < nvec ? lo + chunk : nvec;
    uint32_t acc = 0;
    // every step issues its (up to) eight loads together, the last one
    // predicated lane by lane
    for (int64_t i = lo + threadIdx.x; i < hi; i += kStep) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t j = i + u * kThreads;
            v[u] = j < hi ? __builtin_nontemporal_load(x + j) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= fold(v[u]);
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

__global__ __launch_bounds__(64) void empty_kernel() {}

}  // namespace

extern "C" int stream_read_empty(hipStream_t stream) {
    hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, stream);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

extern "C" int stream_read_run(const void* x, int64_t bytes, int64_t blocks, uint32_t* sink, hipStream_t stream) {
    if (!x || !sink || bytes < 16 || bytes % 16 != 0 || ((uintptr_t)x % 16) != 0) return -1;
    if (blocks < 1 || blocks > 65536) return -1;
    const int64_t nvec = bytes / 16;
    const int64_t chunk = (nvec + blocks - 1) / blocks;
    hipLaunchKernelGGL(stream_read_kernel, dim3((uint32_t)blocks), dim3(kThreads), 0, stream,
                       static_cast<const u32x4*>(x), nvec, chunk, sink);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}
