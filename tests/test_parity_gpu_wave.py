"""GPU parity of the column-contiguous kernel with one wave per vocabulary
segment (topk_cols_create_tuned with TOPK_ALGO_WAVE), against the CPU oracle,
bit-exact.  The workgroup-segment kernel is covered by test_parity_gpu.py;
here the same kinds of inputs run through the other kernel family: all
column-contiguous workloads, ragged and tiny vocabularies, unaligned bases,
every split the wave merge accepts, ties, NaNs, and repeated runs.
"""
import hashlib

import numpy as np
import pytest

from drafter_vocab_top_amd import workloads as W
from gpu_harness import assert_parity, run_oracle, to_device
from topk_checks import bits

pytestmark = pytest.mark.gpu
ALGO = "wave"


@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_workload_full_size(gpu, n):
    w = W.config(n)
    print(f"[parity-wave] workload {w.name}", flush=True)
    assert_parity(gpu, w.x, w.V, w.C, w.k, w.dtype, w.layout, w.ld, label=w.name, algo=ALGO)


@pytest.mark.parametrize("n", [3, 4])
def test_workload_other_seed(gpu, n):
    w = W.config(n, seed=3000 + n)
    print(f"[parity-wave] workload {w.name} seed {w.seed}", flush=True)
    assert_parity(gpu, w.x, w.V, w.C, w.k, w.dtype, w.layout, w.ld, label=w.name, algo=ALGO)


def test_padded_and_misaligned(gpu):
    w = W.config(2)
    ld = (w.V + 63) // 64 * 64
    x = np.full((w.C, ld), 0x7F7F, dtype=np.uint16)
    x[:, :w.V] = w.x
    for offset in (0, 1, 2, 3):
        print(f"[parity-wave] padded offset {offset}", flush=True)
        assert_parity(gpu, x, w.V, w.C, w.k, w.dtype, W.COL, ld, offset=offset,
                      label=f"padded offset={offset}", algo=ALGO)


SMALL_V = [1, 2, 7, 8, 9, 63, 64, 65, 255, 256, 257, 2047, 2049, 4099, 20011]


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
@pytest.mark.parametrize("kind", ["normal", "alphabet", "special"])
def test_small_sweep(gpu, dtype, kind):
    for V in SMALL_V:
        for k in sorted({1, 8, 20, 64, V}):
            if k > V or k > 64:
                continue
            C = 5
            for offset in (0, 1):
                ld = V + offset * 3
                x = W.random_matrix(V * 113 + k, V, C, dtype, W.COL, ld=ld, kind=kind)
                print(f"[parity-wave] small V={V} k={k} {dtype} {kind} offset={offset}", flush=True)
                assert_parity(gpu, x, V, C, k, dtype, W.COL, ld, offset=offset,
                              label=f"V={V} k={k} {kind} offset={offset}", algo=ALGO)


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_every_segment_count(gpu, dtype):
    V, C = 100003, 3
    x = W.random_matrix(79, V, C, dtype, W.COL, kind="normal")
    for k in (1, 8, 64):
        for seg in (1, 2, 3, 5, 8, 16, 31, 64):
            if 4 * seg * k > 2048:
                continue
            print(f"[parity-wave] segments={seg} k={k} {dtype}", flush=True)
            assert_parity(gpu, x, V, C, k, dtype, W.COL, V, segments=seg,
                          label=f"segments={seg} k={k}", algo=ALGO)


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
@pytest.mark.parametrize("kind", ["equal", "asc", "desc", "alphabet"])
def test_ties_and_monotone_columns(gpu, dtype, kind):
    V, C = 30000, 4
    x = W.random_matrix(7, V, C, dtype, W.COL, kind=kind)
    for k in (1, 16, 64):
        for seg in (0, 1, 5):
            if seg and 4 * seg * k > 2048:
                continue
            print(f"[parity-wave] {kind} k={k} segments={seg}", flush=True)
            assert_parity(gpu, x, V, C, k, dtype, W.COL, V, segments=seg,
                          label=f"{kind} k={k} seg={seg}", algo=ALGO)


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_negative_and_nan_columns(gpu, dtype):
    V, C = 50000, 3
    rng = np.random.default_rng(11)
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
            if seg and 4 * seg * k > 2048:
                continue
            print(f"[parity-wave] neg/nan k={k} segments={seg}", flush=True)
            assert_parity(gpu, x, V, C, k, dtype, W.COL, V, segments=seg,
                          label=f"neg/nan k={k} seg={seg}", algo=ALGO)


def test_exhaustive_small_alphabet_columns(gpu):
    cols = W.exhaustive_columns([0xFF80, 0xBF80, 0x8000, 0x0000, 0x3F80], 6).astype(np.uint16)
    n = cols.shape[0]
    for k in range(1, 7):
        assert_parity(gpu, cols, 6, n, k, W.BF16, W.COL, 6, label=f"exhaustive k={k}", algo=ALGO)


def test_back_to_back_runs_are_identical(gpu):
    """Runs without a host sync on rotating inputs: the tickets reset
    themselves and the run tags keep stale published keys out."""
    torch, T = gpu
    w = W.config(3)
    xs = [w.x, W.config(3, seed=4343).x]
    dxs = [to_device(torch, x) for x in xs]
    ref = [run_oracle(x, w.V, w.C, w.k, w.dtype, w.layout, w.ld) for x in xs]
    digests = [hashlib.sha256(bits(r[0]).tobytes() + r[1].tobytes()).hexdigest() for r in ref]
    outs = []
    with T.TopkCols(w.V, w.C, w.k, w.dtype, w.layout, w.ld, algo=ALGO) as h:
        assert h.query()["algo"] == ALGO
        for it in range(300):
            v = torch.empty((w.C, w.k), dtype=torch.int16, device="cuda")
            i = torch.empty((w.C, w.k), dtype=torch.int32, device="cuda")
            h.run(dxs[it % 2], v, i)
            outs.append((v, i))
        torch.cuda.synchronize()
    for it, (v, i) in enumerate(outs):
        got = hashlib.sha256(v.cpu().numpy().view(np.uint16).tobytes() + i.cpu().numpy().tobytes()).hexdigest()
        assert got == digests[it % 2], f"run {it} differs"
