// The entry point that allocates nothing: topk_cols_run_noalloc runs the
// same kernels as topk_cols_run, with the workspace in a static device array
// instead of a handle's allocation.  It serves callers that cannot allocate
// device memory: code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc.
//
// Every GPU the library runs on holds one copy of the array until the
// process ends.  Its layout is fixed, so calls of any shape and either
// layout can follow each other:
//   [0, 256)                 the error word of a merging workgroup's wait
//   tickets                  one 128-byte line per column (column layout):
//                            zero between calls
//   bound words              32 words per column (row layout): zero
//                            between calls (the row merge kernel clears them)
//   lists                    the partial lists of either layout.  Column
//                            lists are tagged 1 and the column's merger sets
//                            them back to zero; row lists are rewritten in
//                            full by each call and carry tag 0.
// The array starts zeroed, and every call that completes leaves the parts
// that must start at zero at zero, so no call clears anything before it
// runs.  Calls that overlap on one GPU (different streams, no ordering)
// share the array and race.
#include "topk_cols.h"

#include <atomic>

#include "topk_internal.hpp"

namespace topk {

namespace {

constexpr size_t kScratchBytes = size_t(8) << 20;
constexpr int64_t kNoallocMaxColumns = 4096;
constexpr size_t kTicketRegion = (size_t)kNoallocMaxColumns * kTicketStride * sizeof(uint32_t);
constexpr size_t kBoundRegion = (size_t)kNoallocMaxColumns * kRowBoundRows * sizeof(uint32_t);
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

// Per device: the array's device address and the CU count, looked up once
// (with that device current) on the device's first call.
std::atomic<void*> g_scratch[kMaxDevices];
std::atomic<int> g_cus[kMaxDevices];

int device_scratch(int device, void** ptr, int* cus) {
    if (device < 0 || device >= kMaxDevices) return TOPK_ERR_UNSUPPORTED;
    void* p = g_scratch[device].load(std::memory_order_acquire);
    int n = g_cus[device].load(std::memory_order_acquire);
    if (!p || n < 1) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return TOPK_ERR_HIP;
        }
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || n < 1)
            return TOPK_ERR_HIP;
        g_cus[device].store(n, std::memory_order_release);
        g_scratch[device].store(p, std::memory_order_release);
    }
    *ptr = p;
    *cus = n;
    return TOPK_OK;
}

}  // namespace

// The no-allocation workspace of the current device: address and size
// (for topk_cols_check with a NULL handle).
int noalloc_workspace(void** ptr, size_t* bytes) {
    int device = 0, cus = 0;
    if (hipGetDevice(&device) != hipSuccess) return TOPK_ERR_HIP;
    const int st = device_scratch(device, ptr, &cus);
    *bytes = kScratchBytes;
    return st;
}

}  // namespace topk

extern "C" int topk_cols_run_noalloc(int64_t V, int64_t C, int32_t k, int32_t dtype, int32_t layout, int64_t ld,
                                     const void* logits, void* out_values, int32_t* out_ids, hipStream_t stream) {
    using namespace topk;
    if (!logits || !out_values || !out_ids) return TOPK_ERR_INVALID_ARG;
    // the shape's rules are those of topk_cols_create
    Plan plan;
    int st = make_plan(&plan, V, C, k, dtype, layout, ld, 0, TOPK_ALGO_AUTO, 1);
    if (st != TOPK_OK) return st;
    const uintptr_t es = (uintptr_t)(dtype == TOPK_BF16 ? 2 : 4);
    if (((uintptr_t)logits % es) != 0 || ((uintptr_t)out_values % es) != 0 || ((uintptr_t)out_ids % 4) != 0)
        return TOPK_ERR_INVALID_ARG;
    if (C > kNoallocMaxColumns) return TOPK_ERR_UNSUPPORTED;
    int device = 0, cus = 0;
    void* ws = nullptr;
    if (hipGetDevice(&device) != hipSuccess) return TOPK_ERR_HIP;
    st = device_scratch(device, &ws, &cus);
    if (st != TOPK_OK) return st;
    st = make_plan(&plan, V, C, k, dtype, layout, ld, 0, TOPK_ALGO_AUTO, cus);
    if (st != TOPK_OK) return st;
    // the fixed layout of the array
    const size_t list_bytes = plan.bound_off - plan.list_off;
    plan.error_off = 0;
    plan.ticket_off = 256;
    plan.bound_off = plan.ticket_off + kTicketRegion;
    plan.list_off = plan.bound_off + kBoundRegion;
    plan.workspace_bytes = plan.list_off + list_bytes;
    if (plan.workspace_bytes > kScratchBytes) return TOPK_ERR_UNSUPPORTED;
    const hipError_t e = launch_plan(plan, ws, C, logits, nullptr, out_values, out_ids, kDefaultSpinLimit, 0u, 1u,
                                     stream);
    return e == hipSuccess ? TOPK_OK : TOPK_ERR_HIP;
}
