"""GPU parity of the column-contiguous layout, and of the seeded workloads in
both layouts: the HIP library (through its C ABI) against the CPU oracle.

The bar is bit-exact.  Output values are compared as raw bits and ids as
integers.  Every GPU output is also checked against the invariants in
topk_checks.check_invariants, which do not use the oracle.  The inputs are
the seeded workloads at full size, plus small and ragged cases that cover
many workgroup tiles, unaligned column starts, padded leading dimensions,
every split of the vocabulary axis, ties, signed zeros, subnormals, infinities
and NaNs.
"""
import hashlib

import numpy as np
import pytest

from drafter_vocab_top_amd import workloads as W
from gpu_harness import assert_parity, run_gpu, run_oracle, to_device
from topk_checks import bits, golden_names, read_golden

pytestmark = pytest.mark.gpu

# ------------------------------------------------------------ fixtures ---

@pytest.mark.parametrize("name", golden_names())
def test_golden_fixtures(gpu, name):
    g = read_golden(name)
    gv, gi = run_gpu(gpu, g["x"], g["V"], g["C"], g["k"], g["dtype"], g["layout"], g["ld"])
    assert np.array_equal(bits(gv), g["values"]) and np.array_equal(gi, g["ids"])


# ------------------------------------------------- full-size workloads ---

@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_workload_full_size(gpu, n):
    w = W.config(n)
    print(f"[parity] workload {w.name} seed {w.seed}", flush=True)
    assert_parity(gpu, w.x, w.V, w.C, w.k, w.dtype, w.layout, w.ld, label=w.name)


@pytest.mark.parametrize("n", [2, 3, 4, 5])
def test_workload_other_seeds(gpu, n):
    for seed in (2000 + n, 2001 + n):
        w = W.config(n, seed=seed)
        print(f"[parity] workload {w.name} seed {seed}", flush=True)
        assert_parity(gpu, w.x, w.V, w.C, w.k, w.dtype, w.layout, w.ld, label=f"{w.name} seed {seed}")


def test_workload_padded_and_misaligned(gpu):
    w = W.config(2)
    ld = (w.V + 63) // 64 * 64
    x = np.full((w.C, ld), 0x7F7F, dtype=np.uint16)
    x[:, :w.V] = w.x
    print("[parity] cfg2 padded ld, offsets 0..3", flush=True)
    for offset in (0, 1, 2, 3):
        assert_parity(gpu, x, w.V, w.C, w.k, w.dtype, W.COL, ld, offset=offset,
                      label=f"padded ld={ld} offset={offset}")


# ------------------------------------------------------- small and ragged ---

SMALL_V = [1, 2, 7, 8, 9, 63, 64, 65, 255, 256, 257, 2047, 2049, 4099, 20011]


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
@pytest.mark.parametrize("kind", ["normal", "alphabet", "special"])
def test_small_sweep(gpu, dtype, kind):
    for V in SMALL_V:
        for k in sorted({1, 2, 8, 20, 64, V}):
            if k > V or k > 64:
                continue
            C = 5
            for offset in (0, 1, 3):
                ld = V + (offset * 2 % 5)
                x = W.random_matrix(V * 131 + k, V, C, dtype, W.COL, ld=ld, kind=kind)
                print(f"[parity] small V={V} k={k} {dtype} {kind} offset={offset}", flush=True)
                assert_parity(gpu, x, V, C, k, dtype, W.COL, ld, offset=offset,
                              label=f"V={V} k={k} {kind} offset={offset}")


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_every_segment_count(gpu, dtype):
    """The answer does not depend on the vocabulary split: 1 workgroup per
    column (multi-pass), a ragged number, and many thin segments."""
    V, C = 100003, 3
    x = W.random_matrix(77, V, C, dtype, W.COL, kind="normal")
    for k in (1, 8, 64):
        for seg in (1, 2, 3, 7, 16, 31, 64):
            if seg > 64:
                continue
            print(f"[parity] segments={seg} k={k} {dtype}", flush=True)
            assert_parity(gpu, x, V, C, k, dtype, W.COL, V, segments=seg, label=f"segments={seg} k={k}")


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
@pytest.mark.parametrize("kind", ["equal", "asc", "desc", "alphabet"])
def test_ties_and_monotone_columns(gpu, dtype, kind):
    """Degenerate columns: all equal (candidate overflow, exact path), strictly
    monotone, and dense small-alphabet ties, across splits."""
    V, C = 30000, 4
    x = W.random_matrix(5, V, C, dtype, W.COL, kind=kind)
    for k in (1, 16, 64):
        for seg in (0, 1, 5):
            print(f"[parity] {kind} k={k} segments={seg}", flush=True)
            assert_parity(gpu, x, V, C, k, dtype, W.COL, V, segments=seg, label=f"{kind} k={k} seg={seg}")


@pytest.mark.parametrize("n_cols,k", [(7, 8), (56, 8), (56, 20)])
def test_tied_top_counts(gpu, n_cols, k):
    """The selection paths of a workgroup and of a column's merger at full
    column length: a value above every other, planted at N rows of a column,
    makes about N/S of each segment's elements and about N list entries tie
    at the top.  N = 20 and 100 keep each segment's candidates within one
    wave's LDS rank; N = 2,000 and 5,000 put 50-300 candidates in a segment
    and every list entry of the column in the merger's rank selection."""
    V = 248046
    x = W.random_matrix(6160 + n_cols + k, V, n_cols, W.BF16, W.COL)
    rng = np.random.default_rng(6161)
    big = 0x4220  # bf16 40.0, above every N(0, 4^2) sample here
    for c in range(n_cols):
        n = (20, 100, 2000, 5000)[c % 4]
        x[c, rng.choice(V, size=n, replace=False)] = big
    print(f"[parity] tied top counts 20/100/2000/5000, V={V} C={n_cols} k={k}", flush=True)
    assert_parity(gpu, x, V, n_cols, k, W.BF16, W.COL, V, label=f"tied top counts C={n_cols} k={k}")


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_negative_and_nan_columns(gpu, dtype):
    """All-negative columns (log-probability-like), columns with negative NaNs,
    and columns whose top-k is mostly NaN."""
    V, C = 50000, 3
    rng = np.random.default_rng(9)
    base = (-10.0 + 3.0 * rng.standard_normal((C, V))).astype(np.float32)
    b = W.bf16_bits_from_f32(base) if dtype == W.BF16 else base.view(np.uint32).copy()
    nan_neg = 0xFFC0 if dtype == W.BF16 else 0xFFC00000
    nan_pos = 0x7FC0 if dtype == W.BF16 else 0x7FC00000
    b[1, rng.choice(V, 5, replace=False)] = nan_neg
    b[2, rng.choice(V, 40, replace=False)] = nan_pos
    b[2, rng.choice(V, 40, replace=False)] = nan_neg
    x = W.storage_from_bits(b, dtype)
    for k in (1, 8, 64):
        for seg in (0, 1, 4):
            assert_parity(gpu, x, V, C, k, dtype, W.COL, V, segments=seg, label=f"neg/nan k={k} seg={seg}")


def test_more_columns_than_one_grid_row(gpu):
    """More columns than the launch grid's y size holds (65,535): the rest
    continue along z.  Every column is checked, with the automatic split
    and with two segments per column."""
    V, C = 40, 70003
    x = W.random_matrix(7003, V, C, W.BF16, W.COL, kind="normal")
    for k, seg in ((3, 0), (3, 2)):
        print(f"[parity] V={V} C={C} k={k} segments={seg}", flush=True)
        assert_parity(gpu, x, V, C, k, W.BF16, W.COL, V, segments=seg, label=f"C={C} k={k} seg={seg}")


def test_exhaustive_small_alphabet_columns(gpu):
    # Every length-6 column over {-inf, -1, -0, +0, 1}: 15,625 columns, every k.
    cols = W.exhaustive_columns([0xFF80, 0xBF80, 0x8000, 0x0000, 0x3F80], 6).astype(np.uint16)
    n = cols.shape[0]
    for k in range(1, 7):
        assert_parity(gpu, cols, 6, n, k, W.BF16, W.COL, 6, label=f"exhaustive k={k}")


# ---------------------------------------------------------- repeated runs ---

def test_back_to_back_runs_are_identical(gpu):
    """Many runs without a host sync on rotating inputs: the per-column tickets
    reset themselves and the run tags keep stale partial lists out."""
    torch, T = gpu
    w = W.config(3)
    xs = [w.x, W.config(3, seed=4242).x]
    dxs = [to_device(torch, x) for x in xs]
    ref = [run_oracle(x, w.V, w.C, w.k, w.dtype, w.layout, w.ld) for x in xs]
    digests = [hashlib.sha256(bits(r[0]).tobytes() + r[1].tobytes()).hexdigest() for r in ref]
    outs = []
    with T.TopkCols(w.V, w.C, w.k, w.dtype, w.layout, w.ld) as h:
        for it in range(300):
            v = torch.empty((w.C, w.k), dtype=torch.int16, device="cuda")
            i = torch.empty((w.C, w.k), dtype=torch.int32, device="cuda")
            h.run(dxs[it % 2], v, i)
            outs.append((v, i))
        torch.cuda.synchronize()
    for it, (v, i) in enumerate(outs):
        got = hashlib.sha256(v.cpu().numpy().view(np.uint16).tobytes() + i.cpu().numpy().tobytes()).hexdigest()
        assert got == digests[it % 2], f"run {it} differs"


def test_two_handles_on_two_streams(gpu):
    torch, T = gpu
    w = W.config(2)
    dx = to_device(torch, w.x)
    ov, oi = run_oracle(w.x, w.V, w.C, w.k, w.dtype, w.layout, w.ld)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    res = []
    with T.TopkCols(w.V, w.C, w.k) as h1, T.TopkCols(w.V, w.C, w.k) as h2:
        for it in range(100):
            for h, s in ((h1, s1), (h2, s2)):
                v = torch.empty((w.C, w.k), dtype=torch.int16, device="cuda")
                i = torch.empty((w.C, w.k), dtype=torch.int32, device="cuda")
                h.run(dx, v, i, stream=s)
                res.append((v, i))
        torch.cuda.synchronize()
    for v, i in res:
        assert np.array_equal(v.cpu().numpy().view(np.uint16), ov)
        assert np.array_equal(i.cpu().numpy(), oi)
