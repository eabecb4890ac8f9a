"""CPU oracle for column-wise top-k -- test infrastructure only.

Only tests/, the smoke check in __graft_entry__ and bench.py's CPU-baseline
leg import this package.  The GPU path never imports it and it imports
nothing from the GPU path.

`topk_cols` wraps the plain-C oracle in topk_oracle.c (a full qsort of every
column under the order "larger value first, ties to the smaller row id"; see
that file's header for the readings of -0, NaN and the emitted bits).
`sample_topk` wraps sample_oracle.c: one temperature / top-p draw per column
from its top-k, with a Philox4x32-10 uniform (see that file's header).
"""
import ctypes
import os

import numpy as np

from . import build as _build

BF16 = 0
F32 = 1
COL_CONTIG = 0
ROW_INTERLEAVED = 1

_lib = None


def load_library(path):
    """Load an oracle build (the default one, or a test's planted-mistake build)."""
    lib = ctypes.CDLL(path)
    lib.oracle_topk_cols.restype = ctypes.c_int
    lib.oracle_topk_cols.argtypes = [
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int, ctypes.c_int,
        ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    if not hasattr(lib, "oracle_sample_topk"):
        return lib   # a planted-mistake build of topk_oracle.c alone
    lib.oracle_sample_topk.restype = ctypes.c_int
    lib.oracle_sample_topk.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int,
        ctypes.c_double, ctypes.c_double, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
    lib.oracle_philox4x32_10.restype = None
    lib.oracle_philox4x32_10.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.oracle_sample_exp.restype = ctypes.c_double
    lib.oracle_sample_exp.argtypes = [ctypes.c_double]
    return lib


def _load():
    global _lib
    if _lib is None:
        path = _build.LIBRARY
        if not os.path.exists(path) or any(os.path.getmtime(path) < os.path.getmtime(src)
                                           for src in _build.SOURCES):
            _build.build()
        _lib = load_library(path)
    return _lib


def topk_cols(x, V, C, k, dtype, layout, ld, nthreads=1, lib=None):
    """Top-k of every column of the V x C matrix stored in `x`.

    x: a contiguous numpy array holding the raw storage (np.uint16 bit
       patterns for bf16, np.float32 or np.uint32 for fp32), element (r, c) at
       x.flat[c*ld + r] (column-contiguous) or x.flat[r*ld + c] (interleaved).
    Returns (values, ids): values has the storage dtype of x, shape (C, k),
    bit-copied from x; ids is int32 (C, k).  Entry [c, 0] is the largest.
    nthreads: worker threads, split over columns.  lib: an alternative build
    returned by load_library (default: oracle/liboracle_topk.so).
    """
    x = np.ascontiguousarray(x)
    if dtype == BF16 and x.dtype != np.uint16:
        raise TypeError("bf16 input must be given as np.uint16 bit patterns")
    if dtype == F32 and x.dtype not in (np.float32, np.uint32):
        raise TypeError("fp32 input must be np.float32 or np.uint32")
    need = (C - 1) * ld + V if layout == COL_CONTIG else (V - 1) * ld + C
    if x.size < need:
        raise ValueError(f"x holds {x.size} elements, the layout needs {need}")
    values = np.empty((C, k), dtype=x.dtype)
    ids = np.empty((C, k), dtype=np.int32)
    rc = (lib or _load()).oracle_topk_cols(V, C, k, dtype, layout, ld, x.ctypes.data,
                                  values.ctypes.data, ids.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_topk_cols failed with status {rc}")
    return values, ids


def topk_cols_mapped(x, V, C, k, dtype, layout, ld, row_to_id, nthreads=1, lib=None):
    """Top-k of every column with the row ids translated through a table.

    The "DFlash2" page ("How it works") describes a "shortlist" output head
    that scores only the 131,072 most frequent vocabulary tokens, so the
    head's row r stands for token row_to_id[r].  Reading taken: the selection
    is the one of topk_cols -- larger value first, ties to the smaller ROW
    (shortlist position) -- and only the reported id is translated afterwards.
    Returns (values, row_to_id[ids]).
    """
    row_to_id = np.asarray(row_to_id)
    if row_to_id.shape != (V,):
        raise ValueError("row_to_id must hold one id per row")
    values, ids = topk_cols(x, V, C, k, dtype, layout, ld, nthreads=nthreads, lib=lib)
    return values, row_to_id[ids].astype(np.int32)


def sample_topk(values, ids, C, k, dtype, temperature, top_p, seed, offset, lib=None):
    """One sampled draft per column from its top-k list (sample_oracle.c).

    values: (C, k) stored bits (np.uint16 for bf16, np.uint32/np.float32 for
    fp32), each row sorted largest first as the top-k path emits it; ids:
    (C, k) int32.  Returns (sampled ids, positions in the list), int32 (C,).
    """
    values = np.ascontiguousarray(values)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    if values.size != C * k or ids.size != C * k:
        raise ValueError("values and ids must hold C*k entries")
    out_ids = np.empty(C, dtype=np.int32)
    out_pos = np.empty(C, dtype=np.int32)
    rc = (lib or _load()).oracle_sample_topk(values.ctypes.data, ids.ctypes.data, C, k, dtype,
                                             float(temperature), float(top_p), int(seed), int(offset),
                                             out_ids.ctypes.data, out_pos.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_sample_topk failed with status {rc}")
    return out_ids, out_pos


def philox4x32_10(counter, key):
    """The oracle's Philox4x32-10 block: 4 counter words, 2 key words -> 4 words."""
    c = np.asarray(counter, dtype=np.uint32)
    kk = np.asarray(key, dtype=np.uint32)
    out = np.empty(4, dtype=np.uint32)
    _load().oracle_philox4x32_10(c.ctypes.data, kk.ctypes.data, out.ctypes.data)
    return out


def sample_exp(x):
    """The oracle's fixed-method exp (x <= 0) used by sample_topk."""
    return _load().oracle_sample_exp(float(x))
