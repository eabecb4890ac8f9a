// Shared between the host library and the kernels: launch arguments and the
// launch entry points of each kernel family.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace topk {

// Column-contiguous launch: element (r, c) at x[c*ld + r].
// The grid is C*S workgroups; workgroup b handles column b / S and vocabulary
// segment b % S and publishes that segment's sorted top-k.  The last
// workgroup of a column to finish merges the column's S lists.
struct ColArgs {
    const void* x;
    int64_t ld;
    int64_t V;
    int32_t C;
    int32_t k;
    int32_t S;            // vocabulary segments (workgroups) per column, <= kMaxSegments
    uint32_t seg_vecs;    // 16-byte vectors per segment, ceil(floor(V / elements per vector) / S)
    uint32_t spin_limit;  // re-reads of a list slot before the merger gives up
    uint32_t fail_waits;  // tests only: the merger treats every list as not yet published
    uint32_t clear_lists; // 1: the workspace is shared between shapes (keep tag 1, zero the lists after a run)
    uint64_t* partials;   // C*S*k keys: one list of k per workgroup
    uint32_t* tickets;    // per column, kTicketStride apart: a counter (zero between runs) and the run count mod 255
    uint32_t* error;      // set nonzero when a merger's wait gave up
    void* out_values;     // C*k elements of the input dtype
    int32_t* out_ids;     // C*k
    const int32_t* id_map;  // NULL, or V entries: out_ids holds id_map[row] instead of row
};

// Waves per workgroup of the column-contiguous kernel.
constexpr int kColWavesPerBlock = 4;
// The last workgroup merges S*k <= 4096 keys, 16 per thread.
constexpr int kMaxSegments = 64;
// Per-column tickets sit 128 bytes apart: counters of different columns in
// one cache line serialize every workgroup's atomic on that line.
constexpr int kTicketStride = 32;
// Columns per launch of the column-contiguous kernel (the grid's y size).
constexpr int64_t kColGridY = 65535;
// 16-byte vectors per lane per pass: the kernel is instantiated for these.
constexpr int kColVecChoices[4] = {2, 4, 8, 16};

// dtype: TOPK_BF16 or TOPK_F32; nv: one of kColVecChoices.
hipError_t launch_col(int dtype, int nv, const ColArgs& a, hipStream_t stream);

// Column-contiguous, one wave per column and no vocabulary split (the
// baseline design): C workgroups of 64 lanes; S, partials, tickets and the
// wait fields are not used.
hipError_t launch_onewave(int dtype, const ColArgs& a, hipStream_t stream);

// Row-interleaved launch: element (r, c) at x[r*ld + c].  The scan grid is
// tiles*S workgroups: workgroup b handles row segment b / tiles and column
// tile b % tiles (128 bytes of each row); a second kernel merges each
// column's S partial lists.
struct RowArgs {
    const void* x;
    int64_t ld;
    int64_t V;
    int32_t C;
    int32_t k;
    int32_t S;            // row segments; S*k <= kRowMaxMergeKeys
    int32_t tiles;        // column tiles
    int32_t vec_loads;    // 1 if every row start of a tile is 16-byte aligned
    int32_t key32;        // 1: bf16 and segments of at most 65,536 rows (32-bit candidate keys)
    uint64_t* partials;   // C*S*k keys
    uint32_t* bound;      // kRowBoundRows rows of bound_ld orders, zero between runs (see the row scan)
    int32_t bound_ld;     // words per bound row: at least C, a multiple of 64
    int32_t use_bound;    // 1 if k <= kRowBoundMaxK and S >= k: segments share a lower bound per column
    void* out_values;     // C*k elements of the input dtype
    int32_t* out_ids;     // C*k
    const int32_t* id_map;  // NULL, or V entries: out_ids holds id_map[row] instead of row
};

constexpr int kRowMaxMergeKeys = 2048;
// Row scans with k <= kRowSmallK keep a smaller candidate area and run three
// workgroups per CU; larger k, two.
constexpr int kRowSmallK = 16;
// Row segments below kRowBoundRows store one element per column to the
// shared bound (one row of words each); scans with k <= kRowBoundMaxK use
// it.
constexpr int kRowBoundRows = 32;
constexpr int kRowBoundMaxK = 16;
// Words per bound row for C columns: whole 64-column tiles, so that a row of
// a tile fills whole lines.
inline int64_t row_bound_ld(int64_t C) { return (C + 63) / 64 * 64; }

// One sampled draft per column from its top-k list (values sorted largest
// first, C*k of the dtype; ids C*k): out_ids[c] = ids[c*k + j*], out_pos[c] =
// j* when out_pos is not NULL.
struct SampleArgs {
    const void* values;
    const int32_t* ids;
    int64_t C;
    int32_t k;
    double temperature;   // > 0, finite
    double top_p;         // in (0, 1]
    uint64_t seed;        // Philox key
    uint64_t offset;      // Philox counter words 0-1 (the column is word 2)
    int32_t* out_ids;
    int32_t* out_pos;     // may be NULL
};
hipError_t launch_sample(int dtype, const SampleArgs& a, hipStream_t stream);

// Columns per tile for a dtype (128 bytes of a row).
int row_tile_columns(int dtype);
hipError_t launch_row(int dtype, int nv, const RowArgs& a, hipStream_t stream);

// ------------------------------------------------------------ host side ---

// The launch decomposition of one shape and the layout of its workspace, as
// chosen for a device.  Built by make_plan; used by a handle and by the
// entry point that runs in a caller-free static workspace.
struct Plan {
    int64_t V, C, ld;
    int32_t k, dtype, layout;
    int32_t algo;          // topk_algo of the column-contiguous layout (AUTO for the row layout)
    int64_t segments;      // workgroups per column, or row segments
    int64_t blocks;        // workgroups of the main kernel
    int64_t tiles;         // column tiles (row layout)
    int nv;                // 16-byte vectors (row steps) per lane per pass
    // workspace: [error word][tickets][lists][bound], each part 256-byte aligned
    size_t error_off, ticket_off, list_off, bound_off, workspace_bytes;
};

// Validates a shape (the rules of topk_cols_create) and fills plan for a
// device with cu_count CUs.  Returns a topk_status.
int make_plan(Plan* plan, int64_t V, int64_t C, int32_t k, int32_t dtype, int32_t layout, int64_t ld,
              int64_t forced_segments, int32_t algo, int cu_count);

// Enqueues one run over the first n_cols columns (0 < n_cols <= plan.C)
// with the workspace at ws (plan.workspace_bytes, zero where the kernels
// expect zeros).  Pointers are checked by the caller.  Returns a HIP error.
hipError_t launch_plan(const Plan& plan, void* ws, int64_t n_cols, const void* logits, const int32_t* id_map,
                       void* out_values, int32_t* out_ids, uint32_t spin_limit, uint32_t fail_waits,
                       uint32_t clear_lists, hipStream_t stream);

// The no-allocation entry point's workspace on the current device (a
// static array): its device address and size.
int noalloc_workspace(void** ptr, size_t* bytes);

// Re-reads of a list slot before a merging workgroup gives up (each costs a
// device round trip of about a microsecond: tens of milliseconds in all).
constexpr uint32_t kDefaultSpinLimit = 1u << 16;

}  // namespace topk
