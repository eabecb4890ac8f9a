"""GPU parity at the library's limits: V = TOPK_MAX_V (2^24 - 1 rows, the
largest row id the 24-bit key field holds) with k = TOPK_MAX_K (64), in both
layouts, bit-exact against the CPU oracle.

At this size the column layout splits each column into 64 segments of many
passes (the multi-pass path with a carried running threshold), and the
row-interleaved layout's segments exceed 65,536 rows (64-bit candidate keys)
with the large candidate buffers of k > 16.  The maximum of each column is
planted in its last row, so the largest row id must come out first.
"""
import numpy as np
import pytest

from drafter_vocab_top_amd import workloads as W
from gpu_harness import assert_parity

pytestmark = pytest.mark.gpu

V_MAX = (1 << 24) - 1
K_MAX = 64


def plant_last_row_max(x, V, C, dtype, layout, ld):
    """Make row V-1 hold each column's unique maximum (a large finite value)."""
    big = np.uint16(0x7F00) if dtype == W.BF16 else np.uint32(0x7F000000)
    flat = x.reshape(-1)
    for c in range(C):
        idx = c * ld + (V - 1) if layout == W.COL else (V - 1) * ld + c
        flat[idx] = big
    return x


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_max_rows_column_layout(gpu, dtype):
    C = 3
    x = W.random_matrix(4242 + (dtype == W.F32), V_MAX, C, dtype, W.COL, kind="normal")
    x = plant_last_row_max(x, V_MAX, C, dtype, W.COL, V_MAX)
    print(f"[parity] V={V_MAX} C={C} k={K_MAX} {dtype} col", flush=True)
    assert_parity(gpu, x, V_MAX, C, K_MAX, dtype, W.COL, V_MAX, label=f"max V {dtype} col")


def test_max_rows_row_layout(gpu):
    C = 9   # one partial tile of 64 columns
    x = W.random_matrix(4343, V_MAX, C, W.BF16, W.ROW, kind="normal")
    x = plant_last_row_max(x, V_MAX, C, W.BF16, W.ROW, C)
    print(f"[parity] V={V_MAX} C={C} k={K_MAX} bf16 row", flush=True)
    assert_parity(gpu, x, V_MAX, C, K_MAX, W.BF16, W.ROW, C, label="max V bf16 row")
