"""Pins of the oracle's shortlist mapping (oracle.topk_cols_mapped), on the CPU.

The "DFlash2" page ("How it works") describes a "shortlist" output head over
the 131,072 most frequent tokens: its row r stands for a vocabulary token.
The reading taken is that selection is over shortlist rows (ties to the
smaller row) and only the reported id is translated.  The pins below do not
reuse the oracle's own route: they rank (value, token) pairs with numpy's
lexsort, a different library routine, under tables whose order either agrees
with the row order (increasing tables: ties by row and by token coincide) or
reverses it (decreasing tables: ties then go to the LARGER token).
"""
import numpy as np
import pytest

import oracle
from drafter_vocab_top_amd import workloads as W

ODT = {W.BF16: oracle.BF16, W.F32: oracle.F32}


def lexsort_topk(f, tokens, k, token_ascending=True):
    """Top k of (value desc, token asc|desc) over one NaN-free column."""
    t = tokens.astype(np.int64)
    order = np.lexsort((t if token_ascending else -t, -f.astype(np.float64)))
    return tokens[order[:k]]


def tie_dense_matrix(seed, V, C, dtype):
    return W.random_matrix(seed, V, C, dtype, W.COL, kind="alphabet")


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_increasing_table_equals_token_order(dtype):
    V, C = 4099, 6
    x = tie_dense_matrix(31, V, C, dtype)
    f = W.float_view(x, dtype)
    table = (np.arange(V, dtype=np.int64) * 3 + 11).astype(np.int32)   # increasing
    for k in (1, 8, 20, 64):
        _, ids = oracle.topk_cols_mapped(x, V, C, k, ODT[dtype], oracle.COL_CONTIG, V, table)
        for c in range(C):
            assert np.array_equal(ids[c], lexsort_topk(f[c], table, k)), (k, c)


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_decreasing_table_ties_follow_the_row_not_the_token(dtype):
    V, C = 4099, 6
    x = tie_dense_matrix(37, V, C, dtype)
    f = W.float_view(x, dtype)
    table = (248045 - np.arange(V, dtype=np.int64) * 5).astype(np.int32)   # decreasing
    differs = 0
    for k in (8, 20, 64):
        _, ids = oracle.topk_cols_mapped(x, V, C, k, ODT[dtype], oracle.COL_CONTIG, V, table)
        for c in range(C):
            # ties to the smaller row = ties to the larger token under this table
            assert np.array_equal(ids[c], lexsort_topk(f[c], table, k, token_ascending=False)), (k, c)
            differs += not np.array_equal(ids[c], lexsort_topk(f[c], table, k, token_ascending=True))
    assert differs > 0   # the inputs do tell the two tie rules apart


def test_identity_table_and_row_layout():
    V, C = 3001, 9
    ld = C + 3
    x = W.random_matrix(41, V, C, W.BF16, W.ROW, ld=ld, kind="special")
    ident = np.arange(V, dtype=np.int32)
    v0, i0 = oracle.topk_cols(x, V, C, 16, oracle.BF16, oracle.ROW_INTERLEAVED, ld)
    v1, i1 = oracle.topk_cols_mapped(x, V, C, 16, oracle.BF16, oracle.ROW_INTERLEAVED, ld, ident)
    assert np.array_equal(v0, v1) and np.array_equal(i0, i1)
    perm = np.random.default_rng(5).permutation(248046)[:V].astype(np.int32)
    v2, i2 = oracle.topk_cols_mapped(x, V, C, 16, oracle.BF16, oracle.ROW_INTERLEAVED, ld, perm)
    assert np.array_equal(v2, v0) and np.array_equal(i2, perm[i0])


def test_table_shape_is_checked():
    x = W.random_matrix(1, 10, 2, W.F32, W.COL)
    with pytest.raises(ValueError):
        oracle.topk_cols_mapped(x, 10, 2, 3, oracle.F32, oracle.COL_CONTIG, 10, np.arange(9))
