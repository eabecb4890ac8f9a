// C ABI of the column-wise top-k library (declared in include/topk_cols.h):
// argument checks, workspace ownership, launch decomposition and dispatch to
// the kernels.  No function here synchronizes the device except create,
// destroy and check, and no function aborts.
#include "topk_cols.h"

#include <stdlib.h>

#include <algorithm>

#include <new>

#include "topk_internal.hpp"

struct topk_cols {
    topk::Plan plan;
    int device;
    void* workspace;      // plan.workspace_bytes, zeroed at create
    uint32_t spin_limit;  // see topk::ColArgs
    uint32_t fail_waits;
};

namespace topk {

namespace {

constexpr int64_t kBlockThreads = 256;
// Do not split a column into segments smaller than this many vectors.
constexpr int64_t kMinVecsPerSegment = 64;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

int element_size(int32_t dtype) { return dtype == TOPK_BF16 ? 2 : 4; }

int64_t vectors_per_column(int64_t V, int dtype) { return V / (16 / element_size(dtype)); }

int64_t choose_col_segments(int64_t V, int64_t C, int32_t k, int dtype, int cu_count) {
    const int64_t nvec = vectors_per_column(V, dtype);
    const int64_t max_nv = kColVecChoices[3];
    int64_t s = ceil_div(nvec, kBlockThreads * max_nv);                 // one pass per workgroup
    // Fill the CUs, but with at most one workgroup per CU (a CU that runs
    // two holds up its columns' merges); for k > 1 also with no more
    // segments than one pass of 4 vectors per lane needs, since the merge
    // reads S*k keys.
    int64_t fill = (int64_t)cu_count / C;
    if (k > 1) fill = std::min(fill, ceil_div(nvec, kBlockThreads * kColVecChoices[1]));
    if (fill > s) s = fill;
    const int64_t most = nvec / kMinVecsPerSegment;                     // not too thin
    if (s > most) s = most;
    if (s > kMaxSegments) s = kMaxSegments;
    return s < 1 ? 1 : s;
}

// Row-interleaved: tiles of 128 bytes of a row; row segments so that as
// many workgroups run as fit at once (three per CU for k <= kRowSmallK, else
// two), each segment at least one 32-row step, and the merge input S*k
// within its limit.
int64_t choose_row_segments(int64_t V, int64_t tiles, int32_t k, int cu_count) {
    const int64_t per_cu = k <= kRowSmallK ? 3 : 2;
    int64_t s = (int64_t)cu_count * per_cu / tiles;  // no partial last wave
    const int64_t most_rows = V / 32;
    if (s > most_rows) s = most_rows;
    const int64_t merge_cap = kRowMaxMergeKeys / k;
    if (s > merge_cap) s = merge_cap;
    return s < 1 ? 1 : s;
}

// Row steps of 32 rows per pass: 8 (256 rows).  Twice that keeps twice the
// row vectors in registers and halves the scan's occupancy once the lane
// pre-filter is in (measured: 65 against 62 us at 248,046 x 448).
int choose_row_nv(int64_t, int64_t) { return 8; }

// Smallest vector count per lane that covers a segment in one pass.
int choose_col_nv(int64_t V, int64_t S, int dtype) {
    const int64_t per_block = ceil_div(vectors_per_column(V, dtype), S);
    for (int nv : kColVecChoices)
        if (per_block <= kBlockThreads * nv) return nv;
    return kColVecChoices[3];
}

}  // namespace

int make_plan(Plan* plan, int64_t V, int64_t C, int32_t k, int32_t dtype, int32_t layout, int64_t ld,
              int64_t forced_segments, int32_t algo, int cu_count) {
    if (V < 1 || C < 1 || k < 1 || (int64_t)k > V) return TOPK_ERR_INVALID_ARG;
    if (dtype != TOPK_BF16 && dtype != TOPK_F32) return TOPK_ERR_INVALID_ARG;
    if (layout != TOPK_COL_CONTIG && layout != TOPK_ROW_INTERLEAVED) return TOPK_ERR_INVALID_ARG;
    if (layout == TOPK_COL_CONTIG && ld < V) return TOPK_ERR_INVALID_ARG;
    if (layout == TOPK_ROW_INTERLEAVED && ld < C) return TOPK_ERR_INVALID_ARG;
    if (forced_segments < 0) return TOPK_ERR_INVALID_ARG;
    if (algo != TOPK_ALGO_AUTO && algo != TOPK_ALGO_WORKGROUP && algo != TOPK_ALGO_ONE_WAVE)
        return TOPK_ERR_INVALID_ARG;
    if (k > TOPK_MAX_K || V > TOPK_MAX_V) return TOPK_ERR_UNSUPPORTED;
    const bool row = layout == TOPK_ROW_INTERLEAVED;
    if (!row && forced_segments > kMaxSegments) return TOPK_ERR_UNSUPPORTED;
    if (row && algo != TOPK_ALGO_AUTO) return TOPK_ERR_UNSUPPORTED;
    if (row && forced_segments * k > kRowMaxMergeKeys) return TOPK_ERR_UNSUPPORTED;
    if (algo == TOPK_ALGO_ONE_WAVE && forced_segments > 1) return TOPK_ERR_UNSUPPORTED;  // no split
    if (C > 0x7FFFFFFF) return TOPK_ERR_UNSUPPORTED;
    // the row scan indexes the shared-bound area with 32-bit word indices
    if (row && row_bound_ld(C) * kRowBoundRows > 0xFFFFFFFFll) return TOPK_ERR_UNSUPPORTED;
    if (cu_count < 1) return TOPK_ERR_HIP;

    if (!row && algo == TOPK_ALGO_AUTO) algo = TOPK_ALGO_WORKGROUP;
    const bool one_wave = !row && algo == TOPK_ALGO_ONE_WAVE;
    const int64_t tiles = row ? ceil_div(C, row_tile_columns(dtype)) : 0;
    const int64_t S = one_wave ? 1
                      : forced_segments > 0 ? forced_segments
                      : row ? choose_row_segments(V, tiles, k, cu_count)
                            : choose_col_segments(V, C, k, dtype, cu_count);
    const int64_t blocks = row ? tiles * S : C * S;
    if (blocks > 0x7FFFFFFF) return TOPK_ERR_UNSUPPORTED;

    Plan p;
    p.V = V; p.C = C; p.ld = ld; p.k = k; p.dtype = dtype; p.layout = layout;
    p.algo = row ? (int32_t)TOPK_ALGO_AUTO : algo;
    p.segments = S; p.blocks = blocks; p.tiles = tiles;
    p.nv = row ? choose_row_nv(V, S) : choose_col_nv(V, S, dtype);
    p.error_off = 0;
    p.ticket_off = 256;
    const size_t ticket_bytes = row ? 0 : align256((size_t)C * kTicketStride * sizeof(uint32_t));
    p.list_off = p.ticket_off + ticket_bytes;
    // one list of k keys per segment and column
    const size_t list_bytes = align256((size_t)C * (size_t)S * (size_t)k * sizeof(uint64_t));
    p.bound_off = p.list_off + list_bytes;
    const size_t bound_bytes =
        row ? align256((size_t)row_bound_ld(C) * kRowBoundRows * sizeof(uint32_t)) : 0;
    p.workspace_bytes = p.bound_off + bound_bytes;
    *plan = p;
    return TOPK_OK;
}

hipError_t launch_plan(const Plan& h, void* ws, int64_t n_cols, const void* logits, const int32_t* id_map,
                       void* out_values, int32_t* out_ids, uint32_t spin_limit, uint32_t fail_waits,
                       uint32_t clear_lists, hipStream_t stream) {
    char* base = static_cast<char*>(ws);
    uint64_t* partials = reinterpret_cast<uint64_t*>(base + h.list_off);
    const uintptr_t es = (uintptr_t)element_size(h.dtype);
    if (h.layout == TOPK_ROW_INTERLEAVED) {
        RowArgs a;
        a.x = logits;
        a.ld = h.ld;
        a.V = h.V;
        a.C = (int32_t)n_cols;
        a.k = h.k;
        a.S = (int32_t)h.segments;
        a.tiles = (int32_t)ceil_div(n_cols, row_tile_columns(h.dtype));
        a.vec_loads = ((uintptr_t)logits % 16 == 0 && (h.ld * (int64_t)es) % 16 == 0) ? 1 : 0;
        a.key32 = (h.dtype == TOPK_BF16 && ceil_div(h.V, h.segments) <= 65536) ? 1 : 0;
        a.partials = partials;
        a.bound = reinterpret_cast<uint32_t*>(base + h.bound_off);
        a.bound_ld = (int32_t)row_bound_ld(h.C);
        a.use_bound = h.k <= kRowBoundMaxK && h.segments >= h.k ? 1 : 0;
        a.out_values = out_values;
        a.out_ids = out_ids;
        a.id_map = id_map;
        return launch_row(h.dtype, h.nv, a, stream);
    }
    ColArgs a;
    a.x = logits;
    a.ld = h.ld;
    a.V = h.V;
    a.C = (int32_t)n_cols;
    a.k = h.k;
    a.S = (int32_t)h.segments;
    // Segment s takes 16-byte vectors [s * seg_vecs, (s + 1) * seg_vecs) of
    // its column, cut at the column's vector count (the last segments may
    // hold fewer, or none); a column has at most V / (elements per vector).
    const int64_t elements_per_vector = h.dtype == TOPK_BF16 ? 8 : 4;
    a.seg_vecs = (uint32_t)ceil_div(h.V / elements_per_vector, h.segments);
    a.spin_limit = spin_limit;
    a.fail_waits = fail_waits;
    a.clear_lists = clear_lists;
    a.partials = partials;
    a.tickets = reinterpret_cast<uint32_t*>(base + h.ticket_off);
    a.error = reinterpret_cast<uint32_t*>(base + h.error_off);
    a.out_values = out_values;
    a.out_ids = out_ids;
    a.id_map = id_map;
    return h.algo == TOPK_ALGO_ONE_WAVE ? launch_onewave(h.dtype, a, stream)
                                        : launch_col(h.dtype, h.nv, a, stream);
}

}  // namespace topk

namespace {

int create_impl(topk_cols_t* out, int64_t V, int64_t C, int32_t k, int32_t dtype, int32_t layout,
                int64_t ld, int64_t forced_segments, int32_t algo) {
    if (!out) return TOPK_ERR_INVALID_ARG;
    *out = nullptr;
    int device = 0;
    int cu_count = 0;
    topk::Plan plan;
    // shape errors take precedence over device errors
    int st = topk::make_plan(&plan, V, C, k, dtype, layout, ld, forced_segments, algo, 1);
    if (st != TOPK_OK) return st;
    if (hipGetDevice(&device) != hipSuccess) return TOPK_ERR_HIP;
    if (hipDeviceGetAttribute(&cu_count, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
        cu_count < 1)
        return TOPK_ERR_HIP;
    st = topk::make_plan(&plan, V, C, k, dtype, layout, ld, forced_segments, algo, cu_count);
    if (st != TOPK_OK) return st;

    topk_cols* h = new (std::nothrow) topk_cols();
    if (!h) return TOPK_ERR_OUT_OF_MEMORY;
    h->plan = plan;
    h->device = device;
    h->spin_limit = topk::kDefaultSpinLimit;
    h->fail_waits = 0;
    hipError_t e = hipMalloc(&h->workspace, plan.workspace_bytes);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        delete h;
        return e == hipErrorOutOfMemory ? TOPK_ERR_OUT_OF_MEMORY : TOPK_ERR_HIP;
    }
    if (hipMemset(h->workspace, 0, plan.workspace_bytes) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
        (void)hipFree(h->workspace);
        delete h;
        return TOPK_ERR_HIP;
    }
    *out = h;
    return TOPK_OK;
}

int run_impl(topk_cols_t h, int64_t n_cols, const void* logits, const int32_t* id_map,
             void* out_values, int32_t* out_ids, hipStream_t stream) {
    if (!h || !logits || !out_values || !out_ids) return TOPK_ERR_INVALID_ARG;
    if (n_cols < 0 || n_cols > h->plan.C) return TOPK_ERR_INVALID_ARG;
    const uintptr_t es = (uintptr_t)(h->plan.dtype == TOPK_BF16 ? 2 : 4);
    if (((uintptr_t)logits % es) != 0 || ((uintptr_t)out_values % es) != 0 ||
        ((uintptr_t)out_ids % 4) != 0 || ((uintptr_t)id_map % 4) != 0)
        return TOPK_ERR_INVALID_ARG;
    if (n_cols == 0) return TOPK_OK;
    const hipError_t e = topk::launch_plan(h->plan, h->workspace, n_cols, logits, id_map, out_values, out_ids,
                                           h->spin_limit, h->fail_waits, 0u, stream);
    return e == hipSuccess ? TOPK_OK : TOPK_ERR_HIP;
}

}  // namespace

extern "C" {

int topk_cols_create(topk_cols_t* out, int64_t V, int64_t C, int32_t k, int32_t dtype,
                     int32_t layout, int64_t ld) {
    return create_impl(out, V, C, k, dtype, layout, ld, 0, TOPK_ALGO_AUTO);
}

int topk_cols_create_with_segments(topk_cols_t* out, int64_t V, int64_t C, int32_t k,
                                   int32_t dtype, int32_t layout, int64_t ld, int64_t segments) {
    return create_impl(out, V, C, k, dtype, layout, ld, segments, TOPK_ALGO_AUTO);
}

int topk_cols_create_tuned(topk_cols_t* out, int64_t V, int64_t C, int32_t k, int32_t dtype,
                           int32_t layout, int64_t ld, int64_t segments, int32_t algo) {
    return create_impl(out, V, C, k, dtype, layout, ld, segments, algo);
}

int topk_cols_run(topk_cols_t h, const void* logits, void* out_values, int32_t* out_ids,
                  hipStream_t stream) {
    return run_impl(h, h ? h->plan.C : 0, logits, nullptr, out_values, out_ids, stream);
}

int topk_cols_run_n(topk_cols_t h, int64_t n_cols, const void* logits, void* out_values,
                    int32_t* out_ids, hipStream_t stream) {
    return run_impl(h, n_cols, logits, nullptr, out_values, out_ids, stream);
}

int topk_cols_run_mapped(topk_cols_t h, int64_t n_cols, const void* logits, const int32_t* row_to_id,
                         void* out_values, int32_t* out_ids, hipStream_t stream) {
    if (!row_to_id) return TOPK_ERR_INVALID_ARG;
    return run_impl(h, n_cols, logits, row_to_id, out_values, out_ids, stream);
}

int topk_cols_check(topk_cols_t h) {
    if (!h) {
        // the no-allocation entry point's workspace on the current device
        void* ws = nullptr;
        size_t bytes = 0;
        const int st = topk::noalloc_workspace(&ws, &bytes);
        if (st != TOPK_OK) return st;
        uint32_t err = 0;
        if (hipDeviceSynchronize() != hipSuccess || hipMemcpy(&err, ws, sizeof(err), hipMemcpyDeviceToHost) != hipSuccess)
            return TOPK_ERR_HIP;
        if (err == 0) return TOPK_OK;
        if (hipMemset(ws, 0, bytes) != hipSuccess || hipDeviceSynchronize() != hipSuccess) return TOPK_ERR_HIP;
        return TOPK_ERR_TIMEOUT;
    }
    int prev = 0;
    if (hipGetDevice(&prev) != hipSuccess || hipSetDevice(h->device) != hipSuccess) return TOPK_ERR_HIP;
    int status = TOPK_OK;
    uint32_t err = 0;
    if (hipDeviceSynchronize() != hipSuccess ||
        hipMemcpy(&err, static_cast<char*>(h->workspace) + h->plan.error_off, sizeof(err),
                  hipMemcpyDeviceToHost) != hipSuccess) {
        status = TOPK_ERR_HIP;
    } else if (err != 0) {
        status = TOPK_ERR_TIMEOUT;
        if (hipMemset(h->workspace, 0, h->plan.workspace_bytes) != hipSuccess || hipDeviceSynchronize() != hipSuccess)
            status = TOPK_ERR_HIP;
    }
    (void)hipSetDevice(prev);
    return status;
}

int topk_cols_debug_fail_waits(topk_cols_t h, int32_t on) {
    if (!h) return TOPK_ERR_INVALID_ARG;
    h->fail_waits = on ? 1u : 0u;
    h->spin_limit = on ? 4u : topk::kDefaultSpinLimit;
    return TOPK_OK;
}

int topk_cols_sample(const void* values, const int32_t* ids, int64_t C, int32_t k, int32_t dtype,
                     double temperature, double top_p, uint64_t seed, uint64_t offset, int32_t* out_ids,
                     int32_t* out_pos, hipStream_t stream) {
    if (!values || !ids || !out_ids) return TOPK_ERR_INVALID_ARG;
    if (C < 1 || k < 1 || k > TOPK_MAX_K) return TOPK_ERR_INVALID_ARG;
    if (dtype != TOPK_BF16 && dtype != TOPK_F32) return TOPK_ERR_INVALID_ARG;
    if (!(temperature > 0.0) || temperature > 1.7976931348623157e308 || !(top_p > 0.0) || !(top_p <= 1.0))
        return TOPK_ERR_INVALID_ARG;
    const uintptr_t es = (uintptr_t)(dtype == TOPK_BF16 ? 2 : 4);
    if (((uintptr_t)values % es) != 0 || ((uintptr_t)ids % 4) != 0 || ((uintptr_t)out_ids % 4) != 0 ||
        ((uintptr_t)out_pos % 4) != 0)
        return TOPK_ERR_INVALID_ARG;
    if ((C + 3) / 4 > 0x7FFFFFFF) return TOPK_ERR_UNSUPPORTED;  // one column per wave, four per workgroup
    topk::SampleArgs a;
    a.values = values;
    a.ids = ids;
    a.C = C;
    a.k = k;
    a.temperature = temperature;
    a.top_p = top_p;
    a.seed = seed;
    a.offset = offset;
    a.out_ids = out_ids;
    a.out_pos = out_pos;
    return topk::launch_sample(dtype, a, stream) == hipSuccess ? TOPK_OK : TOPK_ERR_HIP;
}

int topk_cols_destroy(topk_cols_t h) {
    if (!h) return TOPK_OK;
    int status = TOPK_OK;
    if (h->workspace && hipFree(h->workspace) != hipSuccess) status = TOPK_ERR_HIP;
    delete h;
    return status;
}

const char* topk_cols_status_string(int status) {
    switch (status) {
        case TOPK_OK: return "TOPK_OK";
        case TOPK_ERR_INVALID_ARG: return "TOPK_ERR_INVALID_ARG: an argument is out of range, NULL or misaligned";
        case TOPK_ERR_UNSUPPORTED: return "TOPK_ERR_UNSUPPORTED: valid, but beyond this build's limits";
        case TOPK_ERR_HIP: return "TOPK_ERR_HIP: a HIP runtime call failed";
        case TOPK_ERR_OUT_OF_MEMORY: return "TOPK_ERR_OUT_OF_MEMORY: the workspace could not be allocated";
        case TOPK_ERR_TIMEOUT:
            return "TOPK_ERR_TIMEOUT: a merging workgroup gave up waiting for another workgroup's list; "
                   "outputs since the last check are not valid (the workspace has been reset)";
        default: return "unknown topk_cols status";
    }
}

int topk_cols_query(topk_cols_t h, int64_t* segments, int64_t* blocks, int64_t* workspace_bytes,
                    int32_t* algo) {
    if (!h) return TOPK_ERR_INVALID_ARG;
    if (algo) *algo = h->plan.algo;
    if (segments) *segments = h->plan.segments;
    if (blocks) *blocks = h->plan.blocks;
    if (workspace_bytes) *workspace_bytes = (int64_t)h->plan.workspace_bytes;
    return TOPK_OK;
}

}  // extern "C"
