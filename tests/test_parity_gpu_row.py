"""GPU parity of the row-interleaved layout (element (r, c) at x[r*ld + c]):
the HIP library through its C ABI against the CPU oracle, bit-exact.

The cases cover partial column tiles (C not a multiple of the 128-byte tile),
padded and unaligned rows (element loads instead of 16-byte loads), ragged
row segments, every split of the vocabulary axis the merge accepts, ties that
overflow the candidate buffers (the exact fallback), and special values.
"""
import numpy as np
import pytest

from drafter_vocab_top_amd import workloads as W
from gpu_harness import assert_parity, run_oracle, to_device
from topk_checks import bits

pytestmark = pytest.mark.gpu


def test_full_width_padded_and_misaligned(gpu):
    """448 columns over a shorter vocabulary: a padded ld that keeps rows
    16-byte aligned, one that does not, and unaligned bases."""
    V, C, k = 60001, 448, 16
    for ld in (456, 451):
        x = W.random_matrix(31 + ld, V, C, W.BF16, W.ROW, ld=ld, kind="normal")
        for offset in (0, 1, 3):
            print(f"[parity-row] ld={ld} offset={offset}", flush=True)
            assert_parity(gpu, x, V, C, k, W.BF16, W.ROW, ld, offset=offset,
                          label=f"row ld={ld} offset={offset}")


SMALL_V = [1, 2, 7, 31, 32, 33, 63, 64, 65, 255, 257, 2049, 20011]
SMALL_C = [1, 5, 8, 33, 64, 65, 130]


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
@pytest.mark.parametrize("kind", ["normal", "alphabet", "special"])
def test_small_sweep(gpu, dtype, kind):
    for V in SMALL_V:
        for C in SMALL_C:
            for k in sorted({1, 8, 64, V}):
                if k > V or k > 64:
                    continue
                x = W.random_matrix(V * 257 + C * 7 + k, V, C, dtype, W.ROW, kind=kind)
                print(f"[parity-row] small V={V} C={C} k={k} {dtype} {kind}", flush=True)
                assert_parity(gpu, x, V, C, k, dtype, W.ROW, C, label=f"row V={V} C={C} k={k} {kind}")


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_every_segment_count(gpu, dtype):
    """Any split of the rows gives the same answer (S*k <= 2048; above 1024
    the merge holds 32 keys per lane)."""
    V, C = 50021, 70
    x = W.random_matrix(78, V, C, dtype, W.ROW, kind="normal")
    for k in (1, 16, 64):
        for seg in (1, 2, 3, 7, 16, 31, 64, 73, 128, 1024):
            if seg * k > 2048:
                continue
            print(f"[parity-row] segments={seg} k={k} {dtype}", flush=True)
            assert_parity(gpu, x, V, C, k, dtype, W.ROW, C, segments=seg, label=f"row segments={seg} k={k}")


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
@pytest.mark.parametrize("kind", ["equal", "asc", "desc", "alphabet"])
def test_ties_and_monotone_columns(gpu, dtype, kind):
    """All-equal columns overflow every candidate buffer (exact fallback);
    monotone columns move the running threshold at every pass."""
    V, C = 8000, 70
    x = W.random_matrix(6, V, C, dtype, W.ROW, kind=kind)
    for k in (1, 16, 64):
        for seg in (0, 1, 5):
            print(f"[parity-row] {kind} k={k} segments={seg} {dtype}", flush=True)
            assert_parity(gpu, x, V, C, k, dtype, W.ROW, C, segments=seg, label=f"row {kind} k={k} seg={seg}")


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_negative_and_nan_columns(gpu, dtype):
    V, C = 20000, 40
    rng = np.random.default_rng(10)
    base = (-10.0 + 3.0 * rng.standard_normal((V, C))).astype(np.float32)
    b = W.bf16_bits_from_f32(base) if dtype == W.BF16 else base.view(np.uint32).copy()
    nan_neg = 0xFFC0 if dtype == W.BF16 else 0xFFC00000
    nan_pos = 0x7FC0 if dtype == W.BF16 else 0x7FC00000
    for c in range(0, C, 3):
        b[rng.choice(V, 5, replace=False), c] = nan_neg
    for c in range(1, C, 3):
        b[rng.choice(V, 40, replace=False), c] = nan_pos
        b[rng.choice(V, 40, replace=False), c] = nan_neg
    x = W.storage_from_bits(b, dtype)
    for k in (1, 8, 64):
        for seg in (0, 1, 4):
            print(f"[parity-row] neg/nan k={k} segments={seg} {dtype}", flush=True)
            assert_parity(gpu, x, V, C, k, dtype, W.ROW, C, segments=seg, label=f"row neg/nan k={k} seg={seg}")


def test_exhaustive_small_alphabet_rows(gpu):
    # Every length-6 column over {-inf, -1, -0, +0, 1}, stored as 6 rows of 15,625 columns.
    cols = W.exhaustive_columns([0xFF80, 0xBF80, 0x8000, 0x0000, 0x3F80], 6).astype(np.uint16)
    n = cols.shape[0]
    x = np.ascontiguousarray(cols.T)
    for k in range(1, 7):
        assert_parity(gpu, x, 6, n, k, W.BF16, W.ROW, n, label=f"row exhaustive k={k}")


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_handle_reuse_across_inputs(gpu, dtype):
    """Segments of a column share a lower bound on its k-th largest element
    during a run.  One handle runs a matrix of large values, then matrices of
    small values: every run must match the oracle on its own input (nothing
    of an earlier run may carry over), including when the earlier run ended
    on a different input."""
    torch, T = gpu
    V, C = 120011, 96
    st = np.uint16 if dtype == W.BF16 else np.uint32
    high = W.random_matrix(91, V, C, dtype, W.ROW, kind="normal")
    low = W.random_matrix(92, V, C, dtype, W.ROW, kind="normal")
    hf = W.float_view(high, dtype) + np.float32(64.0)
    high = W.storage_from_bits(W.bf16_bits_from_f32(hf), dtype) if dtype == W.BF16 else hf.astype(np.float32)
    for k in (1, 4, 16):
        with T.TopkCols(V, C, k, dtype, W.ROW, C) as h:
            for name, x in (("high", high), ("low", low), ("high", high), ("low", low)):
                print(f"[parity-row] reuse k={k} {name} {dtype}", flush=True)
                v, i = h.run(to_device(torch, x))
                torch.cuda.synchronize()
                gv = v.cpu().numpy().view(st).reshape(C, k)
                gi = i.cpu().numpy().reshape(C, k)
                ov, oi = run_oracle(x, V, C, k, dtype, W.ROW, C)
                bad = np.flatnonzero((gi != oi).any(axis=1) | (bits(gv) != bits(ov)).any(axis=1))
                assert bad.size == 0, f"reuse k={k} {name}: {bad.size} columns differ, first {bad[0]}"


def test_graph_replay(gpu):
    """A captured row-interleaved run replays correctly: the shared-bound
    slots are cleared by the run's own merge kernel, and nothing else
    carries state between calls.  Replays alternate two inputs, with eager
    work and host syncs between them, and every replay is checked."""
    torch, T = gpu
    V, C, k = 60013, 130, 16
    st = np.uint16
    xs = [W.random_matrix(300 + i, V, C, W.BF16, W.ROW, kind="normal") for i in range(2)]
    ref = [run_oracle(x, V, C, k, W.BF16, W.ROW, C) for x in xs]
    src = to_device(torch, xs[0])
    staged = [to_device(torch, x) for x in xs]
    with T.TopkCols(V, C, k, W.BF16, W.ROW, C) as h:
        vals = torch.empty(C * k, dtype=torch.int16, device="cuda")
        ids = torch.empty(C * k, dtype=torch.int32, device="cuda")
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            h.run(src, vals, ids)          # warm the handle outside the capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            h.run(src, vals, ids, stream=stream)
        for rep in range(6):
            i = rep % 2
            src.copy_(staged[i])               # eager work between replays
            torch.cuda.synchronize()
            print(f"[parity-row] graph replay {rep} input {i}", flush=True)
            g.replay()
            torch.cuda.synchronize()
            gv = vals.cpu().numpy().view(st).reshape(C, k)
            gi = ids.cpu().numpy().reshape(C, k)
            ov, oi = ref[i]
            bad = np.flatnonzero((gi != oi).any(axis=1) | (bits(gv) != bits(ov)).any(axis=1))
            assert bad.size == 0, f"replay {rep}: {bad.size} columns differ, first {bad[0]}"


@pytest.mark.parametrize("kind,dtype,V,segments", [
    ("asc", W.BF16, 32639, 16),      # the longest strictly increasing bf16 column
    ("asc", W.F32, 248046, 0),
    ("equal", W.BF16, 248046, 0),
    ("desc", W.F32, 248046, 0),
    ("desc", W.BF16, 32639, 16),
])
def test_overflow_rebuild_with_shared_bound(gpu, kind, dtype, V, segments):
    """Long columns with several passes per segment and at least k segments,
    so the shared bound fills while columns overflow their buffers and are
    rebuilt: ascending columns overflow in every pass, all-equal ones end on
    the exact path, descending ones stop passing the filter at once."""
    C, k = 64, 16
    x = W.random_matrix(4321, V, C, dtype, W.ROW, kind=kind)
    print(f"[parity-row] overflow and rebuild, {kind} {dtype} V={V} C={C} k={k} segments={segments}", flush=True)
    assert_parity(gpu, x, V, C, k, dtype, W.ROW, C, segments=segments,
                  label=f"row {kind} {dtype} V={V} segments={segments}")


def test_merge_candidate_counts(gpu):
    """The merge kernel's three selection paths, at the full row count (109
    segments of 16-entry lists): a value above every other planted at N rows
    of a column makes about N list entries reach the merge's threshold.
    N = 30 ranks them in one wave (at most 64), N = 150 by the workgroup's
    rank selection, N = 600 overflows the candidate buffer (the exact search
    that re-reads the lists)."""
    V, C, k = 248046, 64, 16
    x = W.random_matrix(5150, V, C, W.BF16, W.ROW)
    rng = np.random.default_rng(5151)
    big = 0x4220  # bf16 40.0, above every N(0, 4^2) sample here
    for c in range(C):
        n = (30, 150, 600)[c % 3]
        rows = rng.choice(V, size=n, replace=False)
        x[rows, c] = big
    print(f"[parity-row] merge candidate counts 30/150/600, V={V} C={C} k={k}", flush=True)
    assert_parity(gpu, x, V, C, k, W.BF16, W.ROW, C, label="row merge candidate counts")


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_nan_columns_with_shared_bound(gpu, dtype):
    """NaNs at the full row count, with several passes per segment and more
    than k segments (128 at this shape), so both reads of the shared bound
    see them.  A column with positive NaNs in the first pass of more than k
    segments makes the bound itself the NaN order (0xFFFF or 0xFFFFFFFF)
    while words of segments that have not stored are still zero: the
    bisection then spans the whole order range.
    Negative NaNs send their segments to the exact path."""
    V, C, k = 248046, 64, 16
    x = W.random_matrix(6262, V, C, dtype, W.ROW)
    b = x.view(np.uint16 if dtype == W.BF16 else np.uint32)
    rng = np.random.default_rng(6263)
    if dtype == W.BF16:
        nan_pos, nan_neg, inf_pos, inf_neg = 0x7FC1, 0xFFC0, 0x7F80, 0xFF80
    else:
        nan_pos, nan_neg, inf_pos, inf_neg = 0x7FFFFFFF, 0xFFC00000, 0x7F800000, 0xFF800000
    for c in range(C):
        kind = c % 5
        if kind == 0:      # positive NaNs near the start of 40 of the 128 segments, and elsewhere
            b[[V * sg // 128 + 1 for sg in range(40)], c] = nan_pos
            b[rng.choice(V, 20, replace=False), c] = nan_pos
        elif kind == 1:    # a few negative NaNs
            b[rng.choice(V, 5, replace=False), c] = nan_neg
        elif kind == 2:    # both signs
            b[rng.choice(V, 20, replace=False), c] = nan_pos
            b[rng.choice(V, 20, replace=False), c] = nan_neg
        elif kind == 3:    # infinities
            b[rng.choice(V, 3, replace=False), c] = inf_pos
            b[rng.choice(V, 3000, replace=False), c] = inf_neg
    print(f"[parity-row] NaN columns with the shared bound, V={V} C={C} k={k} {dtype}", flush=True)
    assert_parity(gpu, x, V, C, k, dtype, W.ROW, C, label=f"row NaN columns shared bound {dtype}")


def test_random_shapes_with_shared_bound(gpu):
    """Seeded random shapes around the shared bound's cases: k <= 16 (the
    bound in use), segment counts on both sides of its 32 publishing
    segments and of k, one to several passes per segment, partial column
    tiles, padded rows and every value kind."""
    rng = np.random.default_rng(7070)
    kinds = ["normal", "alphabet", "special", "equal", "normal", "normal"]
    for case in range(24):
        dtype = (W.BF16, W.F32)[case % 2]
        kind = kinds[case % len(kinds)]
        V = int(rng.integers(300, 120001))
        C = int(rng.integers(1, 140))
        k = int(rng.integers(1, 17))
        k = min(k, V)
        seg = int(rng.choice([0, 0, k, max(k, 17), max(k, 31), max(k, 33), max(k, 64), 2048 // k]))
        seg = min(seg, 2048 // k)
        ld = C + int(rng.integers(0, 3))
        x = W.random_matrix(9000 + case, V, C, dtype, W.ROW, ld=ld, kind=kind)
        print(f"[parity-row] random case {case}: V={V} C={C} k={k} {dtype} {kind} segments={seg} ld={ld}", flush=True)
        assert_parity(gpu, x, V, C, k, dtype, W.ROW, ld, segments=seg,
                      label=f"row random case {case} V={V} C={C} k={k} seg={seg}")
