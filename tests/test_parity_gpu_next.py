"""GPU parity of the widened entry points, through the C ABI, against the
CPU oracle (bit-exact: values as raw bits, ids as integers).

- The one-wave-per-column kernel (TOPK_ALGO_ONE_WAVE), the baseline design
  that the "DFlash2" page ("How it works") replaced.
- topk_cols_run_n: rounds with fewer active columns than the handle was
  created for (up to spec.draft_tokens drafts per lane, same section),
  including runs whose column count changes from call to call without a
  host synchronization, and columns left idle for up to 255 runs.
- topk_cols_run_mapped: the shortlist head's row -> token translation
  (same section), ties to the smaller row.
"""
import numpy as np
import pytest

import oracle
from drafter_vocab_top_amd import workloads as W
from gpu_harness import ODT, OLY, assert_parity, run_oracle, to_device
from topk_checks import bits, check_invariants

pytestmark = pytest.mark.gpu

SENTINEL_ID = -7


def storage_type(dtype):
    return np.uint16 if dtype == W.BF16 else np.uint32


def run_n_gpu(gpu, h, dx, n_cols, id_map=None):
    """One run over n_cols columns into outputs prefilled with a sentinel."""
    torch, _ = gpu
    vals = torch.full((h.C, h.k), 0x5A5A, dtype=dx.dtype, device=dx.device)
    ids = torch.full((h.C, h.k), SENTINEL_ID, dtype=torch.int32, device=dx.device)
    h.run(dx, vals, ids, n_cols=n_cols, id_map=id_map)
    return vals, ids


def host(gpu, vals, ids, dtype):
    torch, _ = gpu
    torch.cuda.synchronize()
    return vals.cpu().numpy().view(storage_type(dtype)), ids.cpu().numpy()


def check_prefix(x, w_like, n, gv, gi, ov, oi):
    """The first n columns equal the oracle's; the rest are untouched."""
    V, k, dtype, layout, ld = w_like
    assert np.array_equal(gi[:n], oi), f"ids differ for n_cols={n}"
    assert np.array_equal(bits(gv[:n]), bits(ov)), f"values differ for n_cols={n}"
    assert (gi[n:] == SENTINEL_ID).all(), f"ids written past column {n}"
    if n:
        check_invariants(x, V, n, k, dtype, layout, ld, gv[:n], gi[:n])


# ------------------------------------------------------- one wave per column ---

@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_one_wave_full_size(gpu, n):
    w = W.config(n)
    print(f"[parity] one_wave {w.name}", flush=True)
    assert_parity(gpu, w.x, w.V, w.C, w.k, w.dtype, w.layout, w.ld, algo="one_wave",
                  label=f"one_wave {w.name}")


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
@pytest.mark.parametrize("kind", ["normal", "alphabet", "special", "asc", "equal"])
def test_one_wave_small(gpu, dtype, kind):
    for V in (1, 7, 9, 64, 65, 511, 4099):
        for k in sorted({1, 2, 8, 17, 33, 64, V}):
            if k > V or k > 64:
                continue
            for offset in (0, 3):
                ld = V + offset
                x = W.random_matrix(V * 7 + k, V, 3, dtype, W.COL, ld=ld, kind=kind)
                print(f"[parity] one_wave V={V} k={k} {dtype} {kind} offset={offset}", flush=True)
                assert_parity(gpu, x, V, 3, k, dtype, W.COL, ld, offset=offset, algo="one_wave",
                              label=f"one_wave V={V} k={k} {kind} offset={offset}")


# -------------------------------------------------------- active columns ---

@pytest.mark.parametrize("n,counts", [(2, [0, 1, 3, 6, 7]), (3, [1, 13, 55, 56]), (4, [1, 20, 56]),
                                      (5, [1, 63, 64, 65, 300, 448])])
def test_run_n_matches_the_first_columns(gpu, n, counts):
    torch, T = gpu
    w = W.config(n)
    dx = to_device(torch, w.x)
    print(f"[parity] run_n {w.name} counts {counts}", flush=True)
    with T.TopkCols(w.V, w.C, w.k, w.dtype, w.layout, w.ld) as h:
        for m in counts:
            gv, gi = host(gpu, *run_n_gpu(gpu, h, dx, m), w.dtype)
            ov, oi = run_oracle(w.x, w.V, m, w.k, w.dtype, w.layout, w.ld) if m else (gv[:0], gi[:0])
            check_prefix(w.x, (w.V, w.k, w.dtype, w.layout, w.ld), m, gv, gi, ov, oi)


@pytest.mark.parametrize("algo", ["auto", "one_wave"])
def test_run_n_changing_counts_without_sync(gpu, algo):
    # 600 runs back to back with the column count changing from call to call:
    # a column may sit idle for any number of runs before it is used again.
    torch, T = gpu
    w = W.config(2)
    dx = to_device(torch, w.x)
    rng = np.random.default_rng(17)
    counts = [int(c) for c in rng.integers(1, w.C + 1, size=600)]
    counts[100:360] = [1] * 255 + [7] * 5        # column 6 idle for 255 runs
    expect = {m: run_oracle(w.x, w.V, m, w.k, w.dtype, w.layout, w.ld) for m in set(counts)}
    print(f"[parity] run_n {algo} 600 runs without sync", flush=True)
    with T.TopkCols(w.V, w.C, w.k, w.dtype, w.layout, w.ld, algo=algo) as h:
        outs = [run_n_gpu(gpu, h, dx, m) for m in counts]
        torch.cuda.synchronize()
        for i, (m, (v, d)) in enumerate(zip(counts, outs)):
            gv, gi = host(gpu, v, d, w.dtype)
            ov, oi = expect[m]
            assert np.array_equal(gi[:m], oi) and np.array_equal(bits(gv[:m]), bits(ov)), (i, m)
            assert (gi[m:] == SENTINEL_ID).all(), (i, m)


def test_run_n_after_shrinking_counts(gpu):
    # Runs over 255, 254, ..., 1 columns, then runs over more columns again:
    # columns left idle for up to 255 runs come back with clean state.
    torch, T = gpu
    V, C, k = 3001, 256, 4
    x = W.random_matrix(77, V, C, W.BF16, W.COL, kind="alphabet")
    dx = to_device(torch, x)
    expect = {m: run_oracle(x, V, m, k, W.BF16, W.COL, V) for m in (1, 128, 255, 256)}
    print("[parity] run_n after shrinking counts", flush=True)
    with T.TopkCols(V, C, k, "bf16", "col", segments=4) as h:
        for m in range(255, 0, -1):
            h.run(dx, n_cols=m)
        for m in (255, 256, 128, 1, 256):
            gv, gi = host(gpu, *run_n_gpu(gpu, h, dx, m), W.BF16)
            ov, oi = expect[m]
            assert np.array_equal(gi[:m], oi) and np.array_equal(bits(gv[:m]), bits(ov)), m


def test_run_n_refuses_bad_counts(gpu):
    torch, T = gpu
    w = W.config(2)
    dx = to_device(torch, w.x)
    with T.TopkCols(w.V, w.C, w.k, w.dtype, w.layout, w.ld) as h:
        for bad in (-1, w.C + 1):
            with pytest.raises(T.TopkError) as e:
                h.run(dx, n_cols=bad)
            assert e.value.status == T.TOPK_ERR_INVALID_ARG


# ------------------------------------------------------------ shortlist ids ---

def shortlist_table(V, seed=9):
    """V distinct token ids out of the drafter's 248,046-token vocabulary."""
    return np.random.default_rng(seed).permutation(248046)[:V].astype(np.int32)


@pytest.mark.parametrize("n,algo", [(4, "auto"), (4, "one_wave"), (2, "auto"), (5, "auto")])
def test_run_mapped(gpu, n, algo):
    torch, T = gpu
    w = W.config(n)
    table = shortlist_table(w.V)
    dx = to_device(torch, w.x)
    dmap = torch.from_numpy(table).to("cuda")
    print(f"[parity] run_mapped {w.name} {algo}", flush=True)
    with T.TopkCols(w.V, w.C, w.k, w.dtype, w.layout, w.ld, algo=algo) as h:
        for m in sorted({w.C, max(1, w.C // 3)}):
            gv, gi = host(gpu, *run_n_gpu(gpu, h, dx, m, id_map=dmap), w.dtype)
            ov, oi = oracle.topk_cols_mapped(w.x, w.V, m, w.k, ODT[w.dtype], OLY[w.layout], w.ld, table)
            assert np.array_equal(gi[:m], oi) and np.array_equal(bits(gv[:m]), bits(ov)), m
            assert (gi[m:] == SENTINEL_ID).all()


def test_run_mapped_ties_follow_the_row(gpu):
    # A decreasing table on tie-dense columns: ties to the smaller row are
    # ties to the larger token.
    torch, T = gpu
    V, C, k = 131072, 8, 20
    x = W.random_matrix(91, V, C, W.F32, W.COL, kind="alphabet")
    table = (248045 - np.arange(V, dtype=np.int64)).astype(np.int32)
    dx = to_device(torch, x)
    dmap = torch.from_numpy(table).to("cuda")
    with T.TopkCols(V, C, k, "f32", "col") as h:
        gv, gi = host(gpu, *run_n_gpu(gpu, h, dx, C, id_map=dmap), W.F32)
    ov, oi = oracle.topk_cols_mapped(x, V, C, k, oracle.F32, oracle.COL_CONTIG, V, table)
    assert np.array_equal(gi, oi) and np.array_equal(bits(gv), bits(ov))
    assert (np.diff(gi, axis=1) < 0).all()   # all 2.0s: tokens strictly decrease


def test_run_mapped_refuses_a_null_table(gpu):
    torch, T = gpu
    w = W.config(2)
    dx = to_device(torch, w.x)
    vals = torch.empty((w.C, w.k), dtype=dx.dtype, device="cuda")
    ids = torch.empty((w.C, w.k), dtype=torch.int32, device="cuda")
    with T.TopkCols(w.V, w.C, w.k, w.dtype, w.layout, w.ld) as h:
        rc = T.load().topk_cols_run_mapped(h._h, w.C, dx.data_ptr(), None, vals.data_ptr(),
                                           ids.data_ptr(), None)
        assert rc == T.TOPK_ERR_INVALID_ARG
