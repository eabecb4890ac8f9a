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
    uint32_t tag;         // 1..255, differs between consecutive runs of a handle
    uint64_t* partials;   // C*S*k keys: one list of k per workgroup
    uint32_t* tickets;    // C counters kTicketStride apart, zero between runs
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
// 16-byte vectors per lane per pass: the kernel is instantiated for these.
constexpr int kColVecChoices[3] = {2, 4, 8};

// dtype: TOPK_BF16 or TOPK_F32; nv: one of kColVecChoices.
hipError_t launch_col(int dtype, int nv, const ColArgs& a, hipStream_t stream);

// Column-contiguous, one wave per vocabulary segment: the same arguments,
// with S workgroups per column and 4*S wave segments, each publishing a list
// (partials holds C*4*S*k keys).  The last wave of a column merges
// 4*S*k <= kWaveSegMergeKeys keys.
constexpr int kWaveSegMergeKeys = 2048;
hipError_t launch_colw(int dtype, int nv, const ColArgs& a, hipStream_t stream);

// Column-contiguous, one wave per column and no vocabulary split (the
// baseline design): C workgroups of 64 lanes; S, tag, partials and tickets
// are not used.
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
    uint32_t* bound;      // C*kRowBoundSlots orders, zero between runs (see the row scan)
    int32_t use_bound;    // 1 if k <= kRowBoundSlots: segments share a lower bound per column
    void* out_values;     // C*k elements of the input dtype
    int32_t* out_ids;     // C*k
    const int32_t* id_map;  // NULL, or V entries: out_ids holds id_map[row] instead of row
};

constexpr int kRowMaxMergeKeys = 2048;
constexpr int kRowBoundSlots = 16;

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

}  // namespace topk
