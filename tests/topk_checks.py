"""Shared test helpers: golden-file reader, library-routine reference and the
output invariants that hold for any correct column-wise top-k.

The order being checked: larger value first, ties to the smaller row id, with
-0 == +0 and NaN (any sign) above +Inf and tied with other NaNs (the readings
of the ignis "DFlash2" page, section "How it works").
"""
import os

import numpy as np
import torch

from drafter_vocab_top_amd import workloads as W

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name):
    """Parse one tests/golden/*.txt fixture into a dict."""
    fields = {"x": [], "values": [], "ids": []}
    with open(os.path.join(GOLDEN_DIR, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *rest = line.split()
            if key in ("x", "values"):
                fields[key].extend(int(t, 16) for t in rest)
            elif key == "ids":
                fields[key].extend(int(t) for t in rest)
            elif key in ("dtype", "layout"):
                fields[key] = rest[0]
            else:
                fields[key] = int(rest[0])
    dt = W.BF16 if fields["dtype"] == "bf16" else W.F32
    st = np.uint16 if dt == W.BF16 else np.uint32
    fields["dtype"] = dt
    fields["x"] = W.storage_from_bits(np.array(fields["x"], dtype=st), dt)
    fields["values"] = np.array(fields["values"], dtype=st).reshape(fields["C"], fields["k"])
    fields["ids"] = np.array(fields["ids"], dtype=np.int32).reshape(fields["C"], fields["k"])
    return fields


def golden_names():
    return sorted(n for n in os.listdir(GOLDEN_DIR) if n.endswith(".txt"))


def bits(a):
    """Raw bit patterns of a storage array (uint16 for bf16, uint32 for fp32)."""
    a = np.asarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a


def matrix_vc(x, V, C, layout, ld):
    """The V x C matrix (storage dtype) from its storage array."""
    flat = np.asarray(x).reshape(-1)
    if layout == W.COL:
        need = (C - 1) * ld + V
        m = np.lib.stride_tricks.as_strided(flat[:need], shape=(V, C),
                                            strides=(flat.itemsize, ld * flat.itemsize))
    else:
        need = (V - 1) * ld + C
        m = np.lib.stride_tricks.as_strided(flat[:need], shape=(V, C),
                                            strides=(ld * flat.itemsize, flat.itemsize))
    return np.ascontiguousarray(m)


def torch_reference(x, V, C, k, dtype, layout, ld):
    """First k of torch.sort(descending=True, stable=True) per column, on CPU.

    torch's sort puts NaN (any sign) first and keeps equal keys (including
    -0/+0 and NaN/NaN) in index order, which is exactly the order checked."""
    m = matrix_vc(x, V, C, layout, ld)
    f = torch.from_numpy(W.float_view(m, dtype).copy())
    _, idx = torch.sort(f, dim=0, descending=True, stable=True)
    ids = idx[:k].T.contiguous().numpy().astype(np.int32)
    vals = np.take_along_axis(m, ids.T.astype(np.int64), axis=0).T
    return np.ascontiguousarray(vals), ids


def _order_keys(vals_f32):
    """(is_nan, value with -0 folded into +0) for vectorised comparisons."""
    v = np.asarray(vals_f32, dtype=np.float64)
    nan = np.isnan(v)
    w = np.where(nan, 0.0, v) + 0.0  # -0 + 0.0 == +0
    return nan, w


def check_invariants(x, V, C, k, dtype, layout, ld, values, ids):
    """Properties of a correct answer that need no reference implementation."""
    m = matrix_vc(x, V, C, layout, ld)
    ids = np.asarray(ids)
    assert ids.shape == (C, k)
    assert ids.min() >= 0 and ids.max() < V, "ids out of range"
    for c in range(C):
        assert len(set(ids[c].tolist())) == k, f"column {c}: repeated ids"
    # (iv) values are the stored bits at the chosen rows
    stored = np.take_along_axis(m, ids.T.astype(np.int64), axis=0).T
    assert np.array_equal(bits(stored), bits(values)), "values are not the stored bits"
    fv = W.float_view(m, dtype)
    sel_nan, sel_val = _order_keys(np.take_along_axis(fv, ids.T.astype(np.int64), axis=0).T)
    # (i)+(ii): consecutive outputs are in strictly decreasing order
    a_nan, a_val, a_id = sel_nan[:, :-1], sel_val[:, :-1], ids[:, :-1]
    b_nan, b_val, b_id = sel_nan[:, 1:], sel_val[:, 1:], ids[:, 1:]
    before = np.where(a_nan & b_nan, a_id < b_id,
             np.where(a_nan | b_nan, a_nan,
             (a_val > b_val) | ((a_val == b_val) & (a_id < b_id))))
    assert before.all(), "outputs are not in order"
    # (v) every unselected row comes after the last selected one
    all_nan, all_val = _order_keys(fv)
    rows = np.arange(V)[:, None]
    last_nan, last_val, last_id = sel_nan[:, -1], sel_val[:, -1], ids[:, -1]
    after = np.where(all_nan & last_nan, rows > last_id,
            np.where(all_nan | last_nan, last_nan,
            (all_val < last_val) | ((all_val == last_val) & (rows > last_id))))
    chosen = np.zeros((V, C), dtype=bool)
    chosen[ids.T, np.arange(C)[None, :]] = True
    assert (after | chosen).all(), "an unselected row beats the k-th output"


def brute_force_column(vals_f32):
    """Full order of one column by pairwise counting (pure Python, tiny V):
    position of row r = number of rows that come before it."""
    v = [float(t) for t in vals_f32]
    n = len(v)

    def before(a, b):
        na, nb = v[a] != v[a], v[b] != v[b]
        if na or nb:
            return (na and nb and a < b) or (na and not nb)
        return v[a] > v[b] or (v[a] == v[b] and a < b)

    order = [None] * n
    for r in range(n):
        order[sum(1 for s in range(n) if s != r and before(s, r))] = r
    return order
