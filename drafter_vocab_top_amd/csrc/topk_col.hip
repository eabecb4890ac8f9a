// Column-contiguous top-k kernel for gfx950.
//
// The ignis "DFlash2" page ("How it works") explains why the replacement
// top-k was fast: it split each column's vocabulary rows across workgroups
// and kept k in registers.  This kernel keeps that split.  Each column's V
// rows are cut into S segments, and one 256-lane workgroup scans each
// segment, so C*S workgroups fill the 256 CUs even at C = 7.  The rest is
// built for wave64 CDNA and for latency: at these sizes one round trip to
// memory costs about a microsecond and a lone wave about 3 ns per
// instruction, so the design minimises both on the critical path.
//
// One scan pass:
//  1. Each lane loads NV 16-byte vectors (coalesced: 64 lanes x 16 bytes),
//     NV in {2, 4, 8} picked so that a segment takes one pass when it can.
//     Vectors are aligned to 16 bytes.  The column's unaligned head and tail
//     rows, fewer than one vector each, go to lanes of wave 0 in the first
//     and last segment as single "edge" elements.
//  2. Each lane takes the exact maximum order of its elements.  It uses
//     packed 16-bit (bf16) or 32-bit integer max/min on the raw bit patterns,
//     never converted floats.  The signed maximum of raw patterns is the
//     largest non-negative value; when a lane holds only negative patterns,
//     the signed minimum is its largest value.
//  3. Each wave finds the k-th largest of its lanes' maxima with a ballot
//     bit-search: k lanes hold an element at or above it, so it bounds the
//     wave's, and the workgroup's, k-th largest element from below.  The
//     largest of the four waves' bounds is the workgroup's threshold T.
//  4. The elements at or above T (usually about k of them) are found with a
//     per-vector prefilter and an integer interval test on the raw pattern.
//     With two vectors per lane they are tested in place; with more, the
//     vectors that reach T are queued in LDS and drained one vector per lane.
//     Ballot/mbcnt compaction collects the passing elements as 64-bit keys
//     in the wave's LDS area; the wave then copies them after the carried
//     best keys in the workgroup area (one LDS atomic per wave).
//  5. After one workgroup barrier, a rank count over that area gives the
//     segment's exact top-k.  A segment that needs several passes carries it
//     into the next pass as a running threshold.
// Negative NaNs, more candidates than a wave's area holds, or more than the
// workgroup's (massive ties), send that pass to an exact path.  There, each
// wave finds its own top-k by a wave-wide bit search over the keys.
//
// Cross-workgroup merge without cache-flushing fences.  Each workgroup takes
// the column's ticket, a device-scope atomic on a 128-byte line of its own,
// and while the reply is in flight ranks its candidates and publishes its
// sorted k keys with device-scope atomic stores, which write through the
// XCD's L2.  Every key carries the run's tag in its low byte, so the
// workgroup that draws the last ticket reads the S lists with device-scope
// loads and re-reads any slot whose tag is not the run's (a list that
// another workgroup, or this one, has not yet published, or whose store has
// not landed) until it is.  All four of its waves then select from the S*k
// keys: per-wave thresholds, one barrier, one rank count.  It writes the
// output and sets the ticket back to zero.
//
// The run's tag lives in device memory, next to the column's ticket: every
// workgroup reads it as it starts (the read travels with the data), and the
// merger advances it (1, 2, ..., 255, 1, ...) when it resets the ticket.  A
// list slot not yet rewritten in a run still holds the previous run's tag,
// so the state a run starts from needs no reset, and a captured launch
// replays correctly.  When the workspace is shared by runs of different
// shapes (the entry point that allocates nothing), the tag stays 1 and the
// merger sets the column's list slots back to zero instead.  The merger's
// wait is bounded; if it gives up, it raises the workspace's error word,
// which the host reports, and writes no output.
#include "topk_col_common.hpp"
#include "topk_device.hpp"
#include "topk_internal.hpp"

namespace topk {

namespace {

static_assert(kWaves == kColWavesPerBlock, "host and kernel disagree on waves per workgroup");

constexpr int kWaveCap = 192;                // candidate slots per wave
constexpr int kBlockCap = 512;               // carried best + candidates per workgroup
constexpr int kMergeKeysPerThread = 16;      // S*k <= 4096 published keys, 16 per thread
constexpr int kQueue = 128;                  // queued vectors per wave
constexpr int kWaveMergeKeys = 256;          // wave 0 alone merges up to this many published keys

struct ColShared {
    alignas(16) uint64_t cand[kBlockCap];          // [0, nbest) carried best, then candidates
    alignas(16) uint64_t best[kMaxK];              // rank-selection output, sorted
    alignas(16) uint64_t wbuf[kWaves][kWaveCap];   // each wave's candidates
    alignas(16) uint64_t wtmp[kWaves][kMaxK];      // each wave's exact-path result
    alignas(16) u32x4 qdata[kWaves][kQueue];       // each wave's queued vectors
    uint32_t qvec[kWaves][kQueue];                 // their vector indices
    uint32_t wave_thr[kWaves];
    uint32_t ncand;
    uint32_t overflow;
    uint32_t is_last;
};

// Copy a wave's m keys (src, LDS) into the workgroup area behind what other
// waves have added (one LDS atomic for the wave's base).  Sets sh.overflow if
// they do not fit.
__device__ __forceinline__ void wave_to_block(ColShared& sh, const uint64_t* src, uint32_t m) {
    const uint32_t lane = threadIdx.x & 63u;
    uint32_t base = 0;
    if (lane == 0 && m != 0) {
        base = atomicAdd(&sh.ncand, m);
        if (base + m > (uint32_t)kBlockCap) sh.overflow = 1u;
    }
    base = __builtin_amdgcn_readfirstlane(base);
    for (uint32_t t = lane; t < m; t += 64u)
        if (base + t < (uint32_t)kBlockCap) sh.cand[base + t] = src[t];
}

// The exact path of one scan pass for one wave: its own top-k (at most k
// keys, sorted, in out) over the pass's elements and its edge element.  Rare,
// so it is kept out of line and re-reads the pass's vectors at every step of
// its search instead of holding 2*NV*EPV key registers across it.
template <class DT, int NV>
__device__ __noinline__ uint32_t exact_scan_wave(uint64_t* wb, uint64_t* out, const u32x4* vec,
                                                 uint32_t v0, uint32_t ve, uint32_t head, uint64_t ex,
                                                 uint32_t k, uint32_t tag) {
    constexpr int EPV = DT::kPerVec;
    auto visit = [&](auto&& f) {
#pragma unroll 1
        for (int i = 0; i < NV; ++i) {
            const uint32_t vi = v0 + (uint32_t)i * kBlock;
            const bool valid = vi < ve;
            const u32x4 v = valid ? vec[vi] : u32x4{0u, 0u, 0u, 0u};
            const uint32_t row0 = head + vi * EPV;
#pragma unroll
            for (int e = 0; e < EPV; ++e)
                f(make_key(DT::order(vec_elem<DT>(v, e)), row0 + e, tag), valid);
        }
        f(ex, ex != 0);
    };
    return wave_exact_topk<DT::kOrderBits>(wb, kWaveCap, out, visit, k);
}

// Re-reads a published slot until its key carries the run's tag (only the
// lanes still waiting take part, one read in flight each).  Returns true
// when the bounded wait gave up.
__device__ __forceinline__ bool wait_tag(const ColArgs& a, const uint64_t* p, uint32_t tag, uint64_t& key) {
    for (uint32_t spin = 0; key_tag(key) != tag || a.fail_waits != 0; ++spin) {
        if (spin >= a.spin_limit) return true;
        __builtin_amdgcn_s_sleep(1);
        key = load_published(p);
    }
    return false;
}

// Selection by the last workgroup of a column: the top k of the S*k
// published keys, into sh.best.
template <class DT>
__device__ __forceinline__ bool merge_lists(const ColArgs& a, ColShared& sh, const uint64_t* parts, uint32_t tag) {
    constexpr int OB = DT::kOrderBits;
    const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
    const uint32_t k = (uint32_t)a.k;
    const uint32_t M = (uint32_t)a.S * k;
    // slots j < J hold keys (J = M / 256 rounded up; the later slots are skipped
    // by a workgroup-uniform test)
    const uint32_t J = (M + kBlock - 1) / kBlock;
    uint64_t keys[kMergeKeysPerThread];
#pragma unroll
    for (int j = 0; j < kMergeKeysPerThread; ++j) {
        const uint32_t idx = tid + (uint32_t)j * kBlock;
        keys[j] = 0;
        if ((uint32_t)j < J && idx < M) keys[j] = load_published(parts + idx);
    }
    bool gave_up = false;
#pragma unroll
    for (int j = 0; j < kMergeKeysPerThread; ++j) {
        const uint32_t idx = tid + (uint32_t)j * kBlock;
        if ((uint32_t)j < J && idx < M) gave_up |= wait_tag(a, parts + idx, tag, keys[j]);
    }
    if (__syncthreads_or(gave_up)) {
        if (tid == 0) __hip_atomic_fetch_or(a.error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return false;
    }
    uint64_t rep = 0;
#pragma unroll
    for (int j = 0; j < kMergeKeysPerThread; ++j)
        if ((uint32_t)j < J) rep = max_u64(rep, keys[j]);
    const uint32_t wt = wave_kth_bound<DT>(key_order(rep), k);
    if (lane == 0) sh.wave_thr[wave] = wt;
    if (tid == 0) {
        sh.ncand = 0;
        sh.overflow = 0;
    }
    __syncthreads();
    uint32_t T = sh.wave_thr[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) T = max_u32(T, sh.wave_thr[w]);

    // sentinel keys (order 0, from segments with fewer than k rows) never qualify
    auto visit = [&](auto&& f) {
#pragma unroll
        for (int j = 0; j < kMergeKeysPerThread; ++j)
            if ((uint32_t)j < J) f(keys[j], key_order(keys[j]) != 0);
    };
    uint64_t* wb = sh.wbuf[wave];
    uint32_t cnt = 0;
    visit([&](uint64_t key, bool valid) {
        cnt = wave_append(wb, cnt, kWaveCap, valid && key_order(key) >= T, key);
    });
    if (cnt > (uint32_t)kWaveCap) {
        cnt = wave_exact_topk<OB>(wb, kWaveCap, sh.wtmp[wave], visit, k);
        wave_to_block(sh, sh.wtmp[wave], cnt);
    } else {
        wave_to_block(sh, wb, cnt);
    }
    __syncthreads();
    uint32_t n = sh.ncand;
    if (sh.overflow) {
        __syncthreads();
        if (tid == 0) {
            sh.ncand = 0;
            sh.overflow = 0;
        }
        __syncthreads();
        const uint32_t m = wave_exact_topk<OB>(wb, kWaveCap, sh.wtmp[wave], visit, k);
        wave_to_block(sh, sh.wtmp[wave], m);
        __syncthreads();
        n = sh.ncand;
    }
    rank_select(sh.cand, n, k, sh.best, tid, kBlock);
    __syncthreads();
    return true;
}

// Selection by wave 0 of the column's last workgroup when the S*k published
// keys fit 16 per lane (coalesced device-scope loads): the k-th largest lane
// maximum is the threshold, the keys at or above it are ranked (through
// 16-byte LDS broadcasts when at most 64), and out(position, key) writes each of
// the top k.
template <class DT, int RMAX, class Out>
__device__ __forceinline__ bool merge_lists_wave(const ColArgs& a, ColShared& sh, const uint64_t* parts,
                                                 uint32_t tag, const Out& out) {
    constexpr int OB = DT::kOrderBits;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t k = (uint32_t)a.k;
    const uint32_t M = (uint32_t)a.S * k;
    const uint32_t R = (M + 63u) / 64u;  // wave-uniform
    uint64_t keys[RMAX];
#pragma unroll
    for (int j = 0; j < RMAX; ++j) {
        const uint32_t idx = (uint32_t)j * 64u + lane;
        keys[j] = 0;
        if ((uint32_t)j < R && idx < M) keys[j] = load_published(parts + idx);
    }
    bool gave_up = false;
#pragma unroll
    for (int j = 0; j < RMAX; ++j) {
        const uint32_t idx = (uint32_t)j * 64u + lane;
        if ((uint32_t)j < R && idx < M) gave_up |= wait_tag(a, parts + idx, tag, keys[j]);
    }
    if (__any(gave_up)) {
        if (lane == 0) __hip_atomic_fetch_or(a.error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return false;
    }
    uint64_t rep = 0;
#pragma unroll
    for (int j = 0; j < RMAX; ++j)
        if ((uint32_t)j < R) rep = max_u64(rep, keys[j]);
    const uint32_t T = wave_kth_bound<DT>(key_order(rep), k);
    // sentinel keys (order 0, from segments with fewer than k rows) never qualify
    auto visit = [&](auto&& f) {
#pragma unroll
        for (int j = 0; j < RMAX; ++j)
            if ((uint32_t)j < R) f(keys[j], key_order(keys[j]) != 0);
    };
    uint32_t cnt = 0;
    visit([&](uint64_t key, bool valid) {
        cnt = wave_append(sh.cand, cnt, kBlockCap, valid && key_order(key) >= T, key);
    });
    if (cnt <= 64u) {
        const uint32_t n8 = (cnt + 7u) & ~7u;
        uint64_t key = 0;
        if (lane < cnt) key = sh.cand[lane];
        else if (lane < n8) sh.cand[lane] = 0;  // padding for the rank
        const uint32_t r = lds_rank_of(sh.cand, n8, key);
        if (lane < cnt && r < k) out(r, key);
        return true;
    }
    const uint32_t n = cnt > (uint32_t)kBlockCap ? wave_exact_topk<OB>(sh.wbuf[0], kWaveCap, sh.best, visit, k)
                                                 : wave_rank_select(sh.cand, cnt, k, sh.best);
    if (lane < n) out(lane, sh.best[lane]);
    return true;
}

// The fields the first loads need come first, as separate arguments, so that
// the hardware can place them in registers as the waves start (kernarg
// preload) instead of every workgroup reading them before its first load;
// the rest follow in ColArgs.  Column c0 + blockIdx.y, segment blockIdx.x.
template <class DT, int NV, bool kBigMerge>
__global__ __launch_bounds__(kBlock) void topk_col_kernel(const void* x, int64_t ld, uint32_t V, uint32_t S,
                                                          uint32_t seg_vecs, uint32_t c0, uint32_t* tickets,
                                                          ColArgs a) {
    using storage = typename DT::storage;
    constexpr int EPV = DT::kPerVec;
    __shared__ ColShared sh;

    const uint32_t tid = threadIdx.x, wave = tid >> 6;
    const uint32_t k = (uint32_t)a.k;
    // Rows and vector indices fit in 32 bits (V < 2^24); only the column
    // offset c * ld needs 64.
    const uint32_t c = c0 + blockIdx.y;
    const uint32_t s = blockIdx.x;
    const storage* col = static_cast<const storage*>(x) + (int64_t)c * ld;
    // The column's ticket and the run's tag share a 128-byte line: word 0
    // counts the workgroups that finished, word 1 holds the run count
    // modulo 255 (the tag is one more).  Read before any data load; the
    // read travels with the data.
    uint32_t* ticket = tickets + c * kTicketStride;
    const uint32_t epoch_v = __hip_atomic_load(ticket + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t epoch = 0, tag = 0;  // taken from epoch_v once the first pass's data are in

    // Split the column into an unaligned head, 16-byte vectors and a tail.
    uint32_t head = ((16u - ((uint32_t)(uintptr_t)col & 15u)) & 15u) / (uint32_t)sizeof(storage);
    if (head > V) head = V;
    const uint32_t nvec = (V - head) / EPV;
    const uint32_t tail0 = head + nvec * EPV;
    const uint32_t vb = min_u32(s * seg_vecs, nvec), ve = min_u32(vb + seg_vecs, nvec);
    const u32x4* vec = reinterpret_cast<const u32x4*>(col + head);

    // This lane's edge element (wave 0 only): its row, or all ones, and its
    // raw bits.  The load is issued here and its value first used in pass 0,
    // after the pass's own loads, so that nothing waits for it alone.
    uint32_t edge_row = 0xFFFFFFFFu;
    if (s == 0 && tid < head) edge_row = tid;
    if (s == S - 1 && tid >= 32 && tid - 32 < V - tail0) edge_row = tail0 + (tid - 32);
    uint32_t edge_raw = 0;
    if (edge_row != 0xFFFFFFFFu) edge_raw = (uint32_t)col[edge_row];

    // A pass's vectors (fill values past the segment's end).  The first
    // pass's loads go out here, before the loop's set-up, and the LDS init's
    // barrier waits while they are in flight.  With 8 or more vectors per
    // lane the loads are unconditional (a slot past the end re-reads the
    // segment's last vector) and the fill is chosen when the pass uses
    // them: cheaper than a branch per load there, dearer with fewer
    // (measured).
    u32x4 d[NV];
    auto load_pass = [&](uint32_t v0) {
        if constexpr (NV >= 8) {
            if (ve > vb) {
#pragma unroll
                for (int i = 0; i < NV; ++i) d[i] = load_vec(vec + min_u32(v0 + (uint32_t)i * kBlock, ve - 1u));
            }
        } else {
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const uint32_t vi = v0 + (uint32_t)i * kBlock;
                d[i] = vi < ve ? load_vec(vec + vi)
                               : u32x4{DT::kFillDword, DT::kFillDword, DT::kFillDword, DT::kFillDword};
            }
        }
    };
    load_pass(vb + tid);
    if (tid == 0) {
        sh.ncand = 0;
        sh.overflow = 0;
    }
    __syncthreads();

    uint64_t* wb = sh.wbuf[wave];
    uint32_t old = 0;  // the ticket's reply (thread 0)
    uint32_t nbest = 0;  // the segment's best so far, in sh.cand[0..nbest) at the start of a pass
    uint64_t t_run = 0;  // the k-th best key once nbest == k
    uint32_t n_last = 0; // candidates of the last pass, in sh.cand
    const uint32_t per_pass = (uint32_t)kBlock * NV;
    const uint32_t npass = ve > vb ? (ve - vb + per_pass - 1) / per_pass : 1u;

    for (uint32_t p = 0; p < npass; ++p) {
        const uint32_t v0 = vb + p * per_pass + tid;
        if (p > 0) load_pass(v0);
        // vector slots of this lane that hold data
        const int nvalid = ve > v0 ? (int)min_u32((uint32_t)NV, (ve - v0 + kBlock - 1) / kBlock) : 0;
        if constexpr (NV >= 8) {
#pragma unroll
            for (int i = 0; i < NV; ++i)
                if (i >= nvalid) d[i] = u32x4{DT::kFillDword, DT::kFillDword, DT::kFillDword, DT::kFillDword};
        }
        uint32_t vmax[NV];
        uint32_t rep;
        bool neg_nan;
        lane_stats<DT, NV>(d, vmax, rep, neg_nan);
        uint64_t ex = 0;
        if (p == 0) {
            epoch = (uint32_t)__builtin_amdgcn_readfirstlane((int)epoch_v);
            tag = epoch + 1u;
            // keeps the edge value's first use (and its wait) here
            asm volatile("" : "+v"(edge_raw));
            if (edge_row != 0xFFFFFFFFu) ex = make_key(DT::order((storage)edge_raw), edge_row, tag);
        }
        if (ex) rep = max_u32(rep, key_order(ex));
        // Each wave takes its kw-th largest lane maximum, kw = ceil(k / 4):
        // every wave then holds at least kw elements at or above the smallest
        // of the four, so that smallest bounds the workgroup's k-th largest
        // element from below.  (For k = 1 a wave's own maximum already leaves
        // only its ties.)
        uint32_t T;
        if (k == 1) {
            T = wave_max_u32(rep);
        } else {
            const uint32_t kw = (k + kWaves - 1) / kWaves;
            T = kw <= 2 ? wave_top12(rep, kw) : wave_kth_bound<DT>(rep, kw);
            if ((tid & 63u) == 0) sh.wave_thr[wave] = T;
            __syncthreads();
#pragma unroll
            for (int w = 0; w < kWaves; ++w) T = min_u32(T, sh.wave_thr[w]);
        }
        if (nbest == k) T = max_u32(T, key_order(t_run));
        const uint64_t tc = max_u64((uint64_t)T << 32, nbest == k ? t_run + 1 : (uint64_t)0);
        // The last pass takes the column's ticket as soon as its threshold
        // is known; the reply is read only after the list is published, so
        // the round trip hides the extraction and the rank.
        if (p + 1 == npass && tid == 0) old = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

        bool exact = __any(neg_nan);
        uint32_t cnt = 0;
        if (!exact) {
            RawFilter<DT> f;
            f.set(T);
          if constexpr (NV <= 2) {
            // few vectors per lane: test them in place
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const bool pv = i < nvalid && (!f.positive || vec_max_signed<DT>(vmax[i]) >= (int)f.lo);
                if (__any(pv)) {
                    // bit e set: element e is at or above the value threshold
                    uint32_t m = 0;
                    if (pv) {
#pragma unroll
                        for (int e = 0; e < EPV; ++e) m |= f.pass(vec_elem<DT>(d[i], e)) ? (1u << e) : 0u;
                    }
                    const uint32_t row0 = head + (v0 + (uint32_t)i * kBlock) * EPV;
                    while (__any(m != 0)) {
                        const uint32_t e = m != 0 ? (uint32_t)__builtin_ctz(m) : 0u;
                        const uint64_t key = make_key(DT::order(vec_elem_dyn<DT>(d[i], e)), row0 + e, tag);
                        cnt = wave_append(wb, cnt, kWaveCap, m != 0 && key >= tc, key);
                        m &= m - 1u;
                    }
                }
            }
          } else {
            // Vectors whose maximum reaches T go to the wave's queue; the
            // queue is drained one vector per lane, and the elements at or
            // above T become keys.
            u32x4* qd = sh.qdata[wave];
            uint32_t* qv = sh.qvec[wave];
            const uint32_t lane = tid & 63u;
            uint32_t qcnt = 0;  // wave-uniform
            auto drain = [&]() {
                for (uint32_t b = 0; b < qcnt; b += 64u) {
                    const uint32_t e = b + lane;
                    u32x4 v = {0u, 0u, 0u, 0u};
                    uint32_t m = 0, row0 = 0;
                    if (e < qcnt) {
                        v = qd[e];
                        row0 = head + qv[e] * EPV;
#pragma unroll
                        for (int el = 0; el < EPV; ++el) m |= f.pass(vec_elem<DT>(v, el)) ? (1u << el) : 0u;
                    }
                    while (__any(m != 0)) {
                        const uint32_t el = m != 0 ? (uint32_t)__builtin_ctz(m) : 0u;
                        const uint64_t key = make_key(DT::order(vec_elem_dyn<DT>(v, el)), row0 + el, tag);
                        cnt = wave_append(wb, cnt, kWaveCap, m != 0 && key >= tc, key);
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
                        qd[pos] = d[i];
                        qv[pos] = v0 + (uint32_t)i * kBlock;
                    }
                    qcnt += (uint32_t)__popcll(bal);
                    if (qcnt > (uint32_t)(kQueue - 64)) drain();
                }
            }
            drain();
          }
            if (wave == 0) cnt = wave_append(wb, cnt, kWaveCap, ex != 0 && ex >= tc, ex);
            exact = cnt > (uint32_t)kWaveCap;
        }
        if (exact) {
            cnt = exact_scan_wave<DT, NV>(wb, sh.wtmp[wave], vec, v0, ve, head, ex, k, tag);
            wave_to_block(sh, sh.wtmp[wave], cnt);
        } else {
            wave_to_block(sh, wb, cnt);
        }
        __syncthreads();
        uint32_t n = sh.ncand;
        if (sh.overflow) {
            // More candidates than the workgroup area holds (massive ties):
            // every wave reduces its share exactly, then the workgroup selects.
            __syncthreads();
            if (tid == 0) {
                sh.ncand = nbest;  // the carried best in cand[0..nbest) is intact
                sh.overflow = 0;
            }
            __syncthreads();
            const uint32_t m = exact_scan_wave<DT, NV>(wb, sh.wtmp[wave], vec, v0, ve, head, ex, k, tag);
            wave_to_block(sh, sh.wtmp[wave], m);
            __syncthreads();
            n = sh.ncand;
        }
        if (p + 1 < npass) {
            rank_select(sh.cand, n, k, sh.best, tid, kBlock);
            __syncthreads();
            nbest = min_u32(n, k);
            if (nbest == k) t_run = sh.best[k - 1];
            if (tid < nbest) sh.cand[tid] = sh.best[tid];
            if (tid == 0) sh.ncand = nbest;
            __syncthreads();
        } else {
            n_last = n;
        }
    }

    // ---- wave 0: rank the segment's candidates and publish the sorted list
    //      (the ticket was taken in the last pass); the list's slots carry
    //      the run tag, so the last ticket holder waits for any list not yet
    //      published ----
    const uint64_t sentinel = tag;  // order 0: below every real key
    uint64_t* parts = a.partials + (int64_t)c * S * k;
    if (wave == 0) {
        const uint32_t lane = tid;
        uint64_t* dst = parts + s * k;
        if (n_last <= 64u) {
            const uint32_t n8 = (n_last + 7u) & ~7u;
            uint64_t key = 0;
            if (lane < n_last) key = sh.cand[lane];
            else if (lane < n8) sh.cand[lane] = 0;  // padding for the rank
            const uint32_t r = lds_rank_of(sh.cand, n8, key);
            if (lane < n_last && r < k)
                __hip_atomic_store(&dst[r], key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else if (n_last <= 128u) {
            // two candidates per lane (common at k = 20): one pass ranks both
            const uint32_t n8 = (n_last + 7u) & ~7u;
            uint64_t ka = sh.cand[lane], kb = 0;
            if (lane + 64u < n_last) kb = sh.cand[lane + 64u];
            else if (lane + 64u < n8) sh.cand[lane + 64u] = 0;  // padding for the rank
            uint32_t ra, rb;
            lds_rank2_of(sh.cand, n8, ka, kb, ra, rb);
            if (ra < k) __hip_atomic_store(&dst[ra], ka, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (lane + 64u < n_last && rb < k)
                __hip_atomic_store(&dst[rb], kb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            const uint32_t m = wave_rank_select(sh.cand, n_last, k, sh.best);
            if (lane < m) __hip_atomic_store(&dst[lane], sh.best[lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (lane >= min_u32(n_last, k) && lane < k)
            __hip_atomic_store(&dst[lane], sentinel, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (lane == 0) sh.is_last = old == S - 1u ? 1u : 0u;
    }
    __syncthreads();
    if (!sh.is_last) return;

    // ---- the column's last workgroup: select from the S published lists ----
    auto write_out = [&](uint32_t pos, uint64_t key) {
        const uint32_t row = key_row(key), o = key_order(key);
        static_cast<storage*>(a.out_values)[(int64_t)c * k + pos] =
            (storage)((o == DT::kZeroOrder || o == DT::kNanOrder) ? (uint32_t)col[row]
                                                                  : DT::bits_from_order(o));
        a.out_ids[(int64_t)c * k + pos] = a.id_map ? a.id_map[row] : (int32_t)row;
    };
    bool ok;
    uint32_t first, stride;
    if constexpr (!kBigMerge) {
        if (wave != 0) return;
        // instantiated for the keys per lane the run needs: a larger
        // instance costs its guarded slots even where they are empty
        const uint32_t M = (uint32_t)a.S * k;
        ok = M <= 64u    ? merge_lists_wave<DT, 1>(a, sh, parts, tag, write_out)
             : M <= 128u ? merge_lists_wave<DT, 2>(a, sh, parts, tag, write_out)
                         : merge_lists_wave<DT, kWaveMergeKeys / 64>(a, sh, parts, tag, write_out);
        first = tid;
        stride = 64u;
    } else {
        ok = merge_lists<DT>(a, sh, parts, tag);
        if (ok && tid < k) write_out(tid, sh.best[tid]);
        first = tid;
        stride = kBlock;
    }
    // Every list of the run has landed (the merger saw all of them).  The
    // next run of the column starts from a zero ticket and the next tag; in
    // a workspace shared between shapes the lists go back to zero instead.
    // (After a wait that gave up, the host resets the workspace.)
    if (a.clear_lists && ok)
        for (uint32_t idx = first; idx < S * k; idx += stride) __hip_atomic_store(parts + idx, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid == 0) {
        const uint64_t next = a.clear_lists ? (uint64_t)epoch : (uint64_t)(epoch + 1u == 255u ? 0u : epoch + 1u);
        __hip_atomic_store(reinterpret_cast<uint64_t*>(ticket), next << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// One launch per kColGridY columns (the grid's y size is at most 65,535).
template <class DT, int NV, bool kBigMerge>
hipError_t launch_nv(const ColArgs& a, hipStream_t stream) {
    for (int64_t c0 = 0; c0 < a.C; c0 += kColGridY) {
        const int64_t n = a.C - c0 < kColGridY ? a.C - c0 : kColGridY;
        hipLaunchKernelGGL((topk_col_kernel<DT, NV, kBigMerge>), dim3((uint32_t)a.S, (uint32_t)n), dim3(kBlock), 0, stream,
                           a.x, a.ld, (uint32_t)a.V, (uint32_t)a.S, a.seg_vecs, (uint32_t)c0, a.tickets, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <class DT>
hipError_t launch_dt(int nv, const ColArgs& a, hipStream_t stream) {
    // the merge a column's last workgroup runs is chosen here, so that each
    // kernel holds the code of one
    const bool big = (int64_t)a.S * a.k > kWaveMergeKeys;
    switch (nv) {
        case 2: return big ? launch_nv<DT, 2, true>(a, stream) : launch_nv<DT, 2, false>(a, stream);
        case 4: return big ? launch_nv<DT, 4, true>(a, stream) : launch_nv<DT, 4, false>(a, stream);
        case 8: return big ? launch_nv<DT, 8, true>(a, stream) : launch_nv<DT, 8, false>(a, stream);
        case 16: return big ? launch_nv<DT, 16, true>(a, stream) : launch_nv<DT, 16, false>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_col(int dtype, int nv, const ColArgs& a, hipStream_t stream) {
    return dtype == 0 ? launch_dt<Bf16>(nv, a, stream) : launch_dt<F32>(nv, a, stream);
}

}  // namespace topk
