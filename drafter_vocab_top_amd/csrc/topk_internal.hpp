// Shared between the host library and the kernels: launch arguments and the
// launch entry points of each kernel family.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace topk {

// Column-contiguous launch: element (r, c) at x[c*ld + r].
// The grid is C*S workgroups; workgroup b handles column b / S and vocabulary
// segment b % S.
struct ColArgs {
    const void* x;
    int64_t ld;
    int64_t V;
    int32_t C;
    int32_t k;
    int32_t S;            // vocabulary segments (workgroups) per column
    uint32_t tag;         // 1..255, differs between consecutive runs of a handle
    uint64_t* partials;   // C*S*k keys (unused when S == 1)
    uint32_t* tickets;    // C counters, zero between runs
    void* out_values;     // C*k elements of the input dtype
    int32_t* out_ids;     // C*k
};

hipError_t launch_col_bf16(const ColArgs& a, hipStream_t stream);
hipError_t launch_col_f32(const ColArgs& a, hipStream_t stream);

// Limit on S * k: the last workgroup of a column merges S lists of k keys,
// at most this many, held 16 per thread.
constexpr int kMaxMergeKeys = 4096;

// Elements each thread holds per pass of the column-contiguous kernel
// (NV 16-byte vectors per thread).
constexpr int kColVecsPerThread = 8;

}  // namespace topk
