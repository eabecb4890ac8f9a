// C ABI of the column-wise top-k library (declared in include/topk_cols.h):
// argument checks, workspace ownership, launch decomposition and dispatch to
// the kernels.  No function here synchronizes the device except create and
// destroy, and no function aborts.
#include "topk_cols.h"

#include <stdlib.h>

#include <new>

#include "topk_internal.hpp"

struct topk_cols {
    int64_t V, C, ld;
    int32_t k;
    int32_t dtype, layout;
    int device;
    int64_t segments;   // workgroups per column
    int64_t blocks;     // workgroups of the main kernel
    int64_t tiles;      // column tiles (row-interleaved layout)
    int32_t algo;       // topk_algo of the column-contiguous layout
    int nv;             // 16-byte vectors (row steps) per lane per pass
    void* workspace;    // tickets, then the published lists (C*S*k keys)
    size_t workspace_bytes;
    uint32_t* tickets;
    uint64_t* partials;
    uint32_t* bound;    // row layout: per-column lower bounds shared by the segments
    uint32_t runs;      // completed run() calls, for the run tag
    uint8_t* col_tag;   // column layout: the tag of the last run that wrote each column's lists
};

namespace {

constexpr int64_t kBlockThreads = 256;
// Scan workgroups the column-contiguous launch aims for: enough that every CU
// has work even when the matrix has few columns.
constexpr int64_t kTargetBlocksPerCU = 2;
// Do not split a column into segments smaller than this many vectors.
constexpr int64_t kMinVecsPerSegment = 64;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int element_size(int32_t dtype) { return dtype == TOPK_BF16 ? 2 : 4; }

int64_t vectors_per_column(int64_t V, int dtype) { return V / (16 / element_size(dtype)); }

int64_t choose_col_segments(int64_t V, int64_t C, int dtype, int cu_count) {
    const int64_t nvec = vectors_per_column(V, dtype);
    const int64_t max_nv = topk::kColVecChoices[2];
    int64_t s = ceil_div(nvec, kBlockThreads * max_nv);                 // one pass per workgroup
    // about one workgroup per CU: more segments make the merge longer than
    // they make the scan shorter
    const int64_t fill = ceil_div((int64_t)cu_count, C);
    if (fill > s) s = fill;
    const int64_t most = nvec / kMinVecsPerSegment;                     // not too thin
    if (s > most) s = most;
    if (s > topk::kMaxSegments) s = topk::kMaxSegments;
    return s < 1 ? 1 : s;
}

// Row-interleaved: tiles of 128 bytes of a row; row segments so that about
// kTargetBlocksPerCU workgroups run per CU, each segment at least one
// 32-row step, and the merge input S*k within its limit.
int64_t choose_row_segments(int64_t V, int64_t tiles, int32_t k, int cu_count) {
    int64_t s = (int64_t)cu_count * kTargetBlocksPerCU / tiles;  // no partial second wave
    const int64_t most_rows = V / 32;
    if (s > most_rows) s = most_rows;
    const int64_t merge_cap = topk::kRowMaxMergeKeys / k;
    if (s > merge_cap) s = merge_cap;
    return s < 1 ? 1 : s;
}

// Row steps of 32 rows per pass: 8 (256 rows).  Twice that keeps twice the
// row vectors in registers and halves the scan's occupancy once the lane
// pre-filter is in (measured: 65 against 62 us at 248,046 x 448).
int choose_row_nv(int64_t, int64_t) { return 8; }

// One wave per vocabulary segment pays off once the columns alone give every
// CU a workgroup or so: then no column needs a deep split, and waves that
// never wait for each other keep the memory system busy.
#ifndef TOPK_WAVE_MIN_COLUMNS
#define TOPK_WAVE_MIN_COLUMNS (1 << 30)
#endif

bool wave_fits(int64_t S, int32_t k) { return S * topk::kColWavesPerBlock * k <= topk::kWaveSegMergeKeys; }

// Workgroups per column for the wave-segment kernel: about one workgroup per
// CU overall, at least 64 vectors per wave, and the merge within its limit.
int64_t choose_wave_segments(int64_t V, int64_t C, int dtype, int32_t k, int cu_count) {
    const int64_t nvec = vectors_per_column(V, dtype);
    int64_t s = ceil_div(cu_count, C);
    const int64_t most = nvec / (kMinVecsPerSegment * topk::kColWavesPerBlock);
    if (s > most) s = most;
    while (s > 1 && !wave_fits(s, k)) --s;
    return s < 1 ? 1 : s;
}

// Smallest vector count per lane that covers a wave segment in one pass, else 8.
int choose_wave_nv(int64_t V, int64_t S, int dtype) {
    const int64_t per_wave = ceil_div(vectors_per_column(V, dtype), S * topk::kColWavesPerBlock);
    for (int nv : topk::kColVecChoices)
        if (per_wave <= 64 * nv) return nv;
    return topk::kColVecChoices[2];
}

// Smallest vector count per lane that covers a segment in one pass.
int choose_col_nv(int64_t V, int64_t S, int dtype) {
    const int64_t per_block = ceil_div(vectors_per_column(V, dtype), S);
    for (int nv : topk::kColVecChoices)
        if (per_block <= kBlockThreads * nv) return nv;
    return topk::kColVecChoices[2];
}

int create_impl(topk_cols_t* out, int64_t V, int64_t C, int32_t k, int32_t dtype, int32_t layout,
                int64_t ld, int64_t forced_segments, int32_t algo) {
    if (!out) return TOPK_ERR_INVALID_ARG;
    *out = nullptr;
    if (V < 1 || C < 1 || k < 1 || (int64_t)k > V) return TOPK_ERR_INVALID_ARG;
    if (dtype != TOPK_BF16 && dtype != TOPK_F32) return TOPK_ERR_INVALID_ARG;
    if (layout != TOPK_COL_CONTIG && layout != TOPK_ROW_INTERLEAVED) return TOPK_ERR_INVALID_ARG;
    if (layout == TOPK_COL_CONTIG && ld < V) return TOPK_ERR_INVALID_ARG;
    if (layout == TOPK_ROW_INTERLEAVED && ld < C) return TOPK_ERR_INVALID_ARG;
    if (forced_segments < 0) return TOPK_ERR_INVALID_ARG;
    if (algo != TOPK_ALGO_AUTO && algo != TOPK_ALGO_WORKGROUP && algo != TOPK_ALGO_WAVE &&
        algo != TOPK_ALGO_ONE_WAVE)
        return TOPK_ERR_INVALID_ARG;
    if (k > TOPK_MAX_K || V > TOPK_MAX_V) return TOPK_ERR_UNSUPPORTED;
    const bool row = layout == TOPK_ROW_INTERLEAVED;
    if (!row && forced_segments > topk::kMaxSegments) return TOPK_ERR_UNSUPPORTED;
    if (row && algo != TOPK_ALGO_AUTO) return TOPK_ERR_UNSUPPORTED;
    if (row && forced_segments * k > topk::kRowMaxMergeKeys) return TOPK_ERR_UNSUPPORTED;
    if (!row && algo == TOPK_ALGO_WAVE && forced_segments > 0 && !wave_fits(forced_segments, k))
        return TOPK_ERR_UNSUPPORTED;
    if (algo == TOPK_ALGO_ONE_WAVE && forced_segments > 1) return TOPK_ERR_UNSUPPORTED;  // no split
    if (C > 0x7FFFFFFF) return TOPK_ERR_UNSUPPORTED;

    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return TOPK_ERR_HIP;
    int cu_count = 0;
    if (hipDeviceGetAttribute(&cu_count, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
        cu_count < 1)
        return TOPK_ERR_HIP;

    if (!row && algo == TOPK_ALGO_AUTO) {
        algo = C >= TOPK_WAVE_MIN_COLUMNS ? TOPK_ALGO_WAVE : TOPK_ALGO_WORKGROUP;
        if (algo == TOPK_ALGO_WAVE && forced_segments > 0 && !wave_fits(forced_segments, k))
            algo = TOPK_ALGO_WORKGROUP;
    }
    const bool wave = !row && algo == TOPK_ALGO_WAVE;
    const bool one_wave = !row && algo == TOPK_ALGO_ONE_WAVE;
    const int64_t tiles = row ? ceil_div(C, topk::row_tile_columns(dtype)) : 0;
    const int64_t S = one_wave ? 1
                      : forced_segments > 0 ? forced_segments
                      : row  ? choose_row_segments(V, tiles, k, cu_count)
                      : wave ? choose_wave_segments(V, C, dtype, k, cu_count)
                             : choose_col_segments(V, C, dtype, cu_count);
    const int64_t blocks = row ? tiles * S : C * S;
    if (blocks > 0x7FFFFFFF) return TOPK_ERR_UNSUPPORTED;
    const int64_t lists = wave ? S * topk::kColWavesPerBlock : S;  // published lists per column

    const size_t ticket_bytes =
        row ? 0 : ((size_t)C * topk::kTicketStride * sizeof(uint32_t) + 255) & ~(size_t)255;
    const size_t list_bytes = ((size_t)C * (size_t)lists * (size_t)k * sizeof(uint64_t) + 255) & ~(size_t)255;
    const size_t bound_bytes = row ? (size_t)C * topk::kRowBoundSlots * sizeof(uint32_t) : 0;
    const size_t ws_bytes = ticket_bytes + list_bytes + bound_bytes;

    topk_cols* h = new (std::nothrow) topk_cols();
    if (!h) return TOPK_ERR_OUT_OF_MEMORY;
    h->col_tag = nullptr;
    if (!row) {
        h->col_tag = new (std::nothrow) uint8_t[(size_t)C]();  // 0: never written (no run uses tag 0)
        if (!h->col_tag) {
            delete h;
            return TOPK_ERR_OUT_OF_MEMORY;
        }
    }
    h->V = V; h->C = C; h->ld = ld; h->k = k; h->dtype = dtype; h->layout = layout;
    h->device = device; h->segments = S; h->blocks = blocks; h->tiles = tiles;
    h->algo = row ? (int32_t)TOPK_ALGO_AUTO : algo;
    h->nv = row ? choose_row_nv(V, S) : wave ? choose_wave_nv(V, S, dtype) : choose_col_nv(V, S, dtype);
    h->workspace_bytes = ws_bytes;
    hipError_t e = hipMalloc(&h->workspace, ws_bytes);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        delete[] h->col_tag;
        delete h;
        return e == hipErrorOutOfMemory ? TOPK_ERR_OUT_OF_MEMORY : TOPK_ERR_HIP;
    }
    h->tickets = row ? nullptr : static_cast<uint32_t*>(h->workspace);
    h->partials = reinterpret_cast<uint64_t*>(static_cast<char*>(h->workspace) + ticket_bytes);
    h->bound = row ? reinterpret_cast<uint32_t*>(static_cast<char*>(h->workspace) + ticket_bytes + list_bytes) : nullptr;
    if (hipMemset(h->workspace, 0, ws_bytes) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
        (void)hipFree(h->workspace);
        delete[] h->col_tag;
        delete h;
        return TOPK_ERR_HIP;
    }
    *out = h;
    return TOPK_OK;
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

}  // extern "C"

namespace {

// The run tag for the column layout: the first value in 1..255, starting
// from the handle's run count, that no active column's lists carry from an
// earlier run.  The last workgroup of a column tells a list slot written in
// this run from a stale one by its tag, so a column must never see its own
// previous tag again while its old lists are still there; with runs over
// fewer columns, a column's last write can be any number of runs back.
// Returns 0 when every tag is taken (then the caller clears the lists).
uint32_t choose_tag(const topk_cols* h, int64_t n) {
    uint64_t used[4] = {0, 0, 0, 0};
    for (int64_t c = 0; c < n; ++c) used[h->col_tag[c] >> 6] |= 1ull << (h->col_tag[c] & 63u);
    for (uint32_t i = 0; i < 255u; ++i) {
        const uint32_t t = 1u + ((h->runs + i) % 255u);
        if (!((used[t >> 6] >> (t & 63u)) & 1ull)) return t;
    }
    return 0;
}

int run_impl(topk_cols_t h, int64_t n_cols, const void* logits, const int32_t* id_map,
             void* out_values, int32_t* out_ids, hipStream_t stream) {
    if (!h || !logits || !out_values || !out_ids) return TOPK_ERR_INVALID_ARG;
    if (n_cols < 0 || n_cols > h->C) return TOPK_ERR_INVALID_ARG;
    const uintptr_t es = (uintptr_t)element_size(h->dtype);
    if (((uintptr_t)logits % es) != 0 || ((uintptr_t)out_values % es) != 0 ||
        ((uintptr_t)out_ids % 4) != 0 || ((uintptr_t)id_map % 4) != 0)
        return TOPK_ERR_INVALID_ARG;
    if (n_cols == 0) return TOPK_OK;

    hipError_t e;
    if (h->layout == TOPK_ROW_INTERLEAVED) {
        topk::RowArgs a;
        a.x = logits;
        a.ld = h->ld;
        a.V = h->V;
        a.C = (int32_t)n_cols;
        a.k = h->k;
        a.S = (int32_t)h->segments;
        a.tiles = (int32_t)ceil_div(n_cols, topk::row_tile_columns(h->dtype));
        a.vec_loads = ((uintptr_t)logits % 16 == 0 && (h->ld * (int64_t)es) % 16 == 0) ? 1 : 0;
        a.key32 = (h->dtype == TOPK_BF16 && ceil_div(h->V, h->segments) <= 65536) ? 1 : 0;
        a.partials = h->partials;
        a.bound = h->bound;
        a.use_bound = h->k <= topk::kRowBoundSlots ? 1 : 0;
        a.out_values = out_values;
        a.out_ids = out_ids;
        a.id_map = id_map;
        e = topk::launch_row(h->dtype, h->nv, a, stream);
    } else {
        topk::ColArgs a;
        a.x = logits;
        a.ld = h->ld;
        a.V = h->V;
        a.C = (int32_t)n_cols;
        a.k = h->k;
        a.S = (int32_t)h->segments;
        a.partials = h->partials;
        a.tickets = h->tickets;
        a.out_values = out_values;
        a.out_ids = out_ids;
        a.id_map = id_map;
        if (h->algo == TOPK_ALGO_ONE_WAVE) {
            a.tag = 0;
            e = topk::launch_onewave(h->dtype, a, stream);
        } else {
            uint32_t tag = choose_tag(h, n_cols);
            if (tag == 0) {
                // every tag is still held by some active column's lists: clear
                // them all (tag 0 is never a run's tag)
                const size_t list_bytes = (size_t)h->workspace_bytes -
                                          (size_t)((char*)h->partials - (char*)h->workspace);
                if (hipMemsetAsync(h->partials, 0, list_bytes, stream) != hipSuccess) return TOPK_ERR_HIP;
                for (int64_t c = 0; c < h->C; ++c) h->col_tag[c] = 0;
                tag = 1u + (h->runs % 255u);
            }
            a.tag = tag;
            e = h->algo == TOPK_ALGO_WAVE ? topk::launch_colw(h->dtype, h->nv, a, stream)
                                          : topk::launch_col(h->dtype, h->nv, a, stream);
            if (e == hipSuccess)
                for (int64_t c = 0; c < n_cols; ++c) h->col_tag[c] = (uint8_t)tag;
        }
    }
    if (e != hipSuccess) return TOPK_ERR_HIP;
    ++h->runs;
    return TOPK_OK;
}

}  // namespace

extern "C" {

int topk_cols_run(topk_cols_t h, const void* logits, void* out_values, int32_t* out_ids,
                  hipStream_t stream) {
    return run_impl(h, h ? h->C : 0, logits, nullptr, out_values, out_ids, stream);
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

int topk_cols_sample(const void* values, const int32_t* ids, int64_t C, int32_t k, int32_t dtype,
                     double temperature, double top_p, uint64_t seed, uint64_t offset, int32_t* out_ids,
                     int32_t* out_pos, hipStream_t stream) {
    if (!values || !ids || !out_ids) return TOPK_ERR_INVALID_ARG;
    if (C < 1 || k < 1 || k > TOPK_MAX_K) return TOPK_ERR_INVALID_ARG;
    if (dtype != TOPK_BF16 && dtype != TOPK_F32) return TOPK_ERR_INVALID_ARG;
    if (!(temperature > 0.0) || temperature > 1.7976931348623157e308 || !(top_p > 0.0) || !(top_p <= 1.0))
        return TOPK_ERR_INVALID_ARG;
    const uintptr_t es = (uintptr_t)element_size(dtype);
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
    delete[] h->col_tag;
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
        default: return "unknown topk_cols status";
    }
}

int topk_cols_query(topk_cols_t h, int64_t* segments, int64_t* blocks, int64_t* workspace_bytes,
                    int32_t* algo) {
    if (!h) return TOPK_ERR_INVALID_ARG;
    if (algo) *algo = h->algo;
    if (segments) *segments = h->segments;
    if (blocks) *blocks = h->blocks;
    if (workspace_bytes) *workspace_bytes = (int64_t)h->workspace_bytes;
    return TOPK_OK;
}

}  // extern "C"
