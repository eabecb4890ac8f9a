// A plain streaming read of a buffer, for measurement only: the achievable
// HBM read rate on this part for a given number of bytes, read once, cold.
// It is not part of the top-k path and the top-k library does not use it;
// the benchmark times it beside the top-k over the same bytes.
//
// Every lane reads four 16-byte vectors per step with non-temporal loads,
// grid-strided, and folds them with xor (one ALU op per dword), so the loads
// cannot be removed; one conditional store that practically never happens
// keeps the fold alive.
//
// C ABI (built into libstream_read.so, loaded only by the benchmark):
//   int stream_read_run(const void* x, int64_t bytes, uint32_t* sink,
//                       hipStream_t stream)
//     x: device pointer, 16-byte aligned; bytes: a multiple of 16, >= 16;
//     sink: device, one uint32 that the kernel may write; returns 0, -1 for
//     a bad argument, -3 when the launch fails.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr int64_t kMaxBlocks = 2048;

__device__ __forceinline__ uint32_t fold(const u32x4& v) {
    const uint32_t a = v.x, b = v.y, c = v.z, d = v.w;
    return a ^ b ^ c ^ d;
}

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* x, int64_t nvec, uint32_t* sink) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kUnroll - 1) * stride < nvec; i += kUnroll * stride) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(x + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= fold(v[u]);
    }
    for (; i < nvec; i += stride) acc ^= fold(__builtin_nontemporal_load(x + i));
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

extern "C" int stream_read_run(const void* x, int64_t bytes, uint32_t* sink, hipStream_t stream) {
    if (!x || !sink || bytes < 16 || bytes % 16 != 0 || ((uintptr_t)x % 16) != 0) return -1;
    const int64_t nvec = bytes / 16;
    int64_t blocks = (nvec + (int64_t)kThreads * kUnroll - 1) / ((int64_t)kThreads * kUnroll);
    if (blocks > kMaxBlocks) blocks = kMaxBlocks;
    hipLaunchKernelGGL(stream_read_kernel, dim3((uint32_t)blocks), dim3(kThreads), 0, stream,
                       static_cast<const u32x4*>(x), nvec, sink);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}
