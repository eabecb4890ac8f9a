"""ctypes binding of libtopk_cols.so, the HIP column-wise top-k library.

The binding only marshals arguments.  It passes raw device pointers and the
current HIP stream to the C ABI in include/topk_cols.h; every step of the
selection runs in the library's kernels.  PyTorch supplies the device buffers
and the stream.

    h = TopkCols(V, C, k, "bf16", "col", ld)
    values, ids = h.run(x)            # x: torch tensor on the GPU
    h.close()

Loading fails loudly when the library is missing or cannot be loaded.  There
is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

LIBRARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtopk_cols.so")

TOPK_OK = 0
TOPK_ERR_INVALID_ARG = -1
TOPK_ERR_UNSUPPORTED = -2
TOPK_ERR_HIP = -3
TOPK_ERR_OUT_OF_MEMORY = -4
TOPK_ERR_TIMEOUT = -5
TOPK_MAX_K = 64
TOPK_MAX_V = (1 << 24) - 1

DTYPES = {"bf16": 0, "f32": 1}
LAYOUTS = {"col": 0, "row": 1}

EXPORTED = ("topk_cols_create", "topk_cols_create_with_segments", "topk_cols_create_tuned",
            "topk_cols_run", "topk_cols_run_n", "topk_cols_run_mapped", "topk_cols_sample",
            "topk_cols_destroy", "topk_cols_status_string", "topk_cols_query", "topk_cols_check",
            "topk_cols_debug_fail_waits", "topk_cols_run_noalloc")
# kernel families of the column-contiguous layout ("one_wave": the baseline
# design with one wave per column and no vocabulary split)
ALGOS = {"auto": 0, "workgroup": 1, "one_wave": 3}

_lib = None


class TopkError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}")


def load(path: str = LIBRARY):
    """Load the library (once) and declare its C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise OSError(f"{path} is missing: build it with `python -m drafter_vocab_top_amd.build`")
    lib = ctypes.CDLL(path)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.topk_cols_create.argtypes = [ctypes.POINTER(p), i64, i64, i32, i32, i32, i64]
    lib.topk_cols_create.restype = ctypes.c_int
    lib.topk_cols_create_with_segments.argtypes = [ctypes.POINTER(p), i64, i64, i32, i32, i32, i64, i64]
    lib.topk_cols_create_with_segments.restype = ctypes.c_int
    lib.topk_cols_create_tuned.argtypes = [ctypes.POINTER(p), i64, i64, i32, i32, i32, i64, i64, i32]
    lib.topk_cols_create_tuned.restype = ctypes.c_int
    lib.topk_cols_run.argtypes = [p, p, p, p, p]
    lib.topk_cols_run.restype = ctypes.c_int
    lib.topk_cols_run_n.argtypes = [p, i64, p, p, p, p]
    lib.topk_cols_run_n.restype = ctypes.c_int
    lib.topk_cols_run_mapped.argtypes = [p, i64, p, p, p, p, p]
    lib.topk_cols_run_mapped.restype = ctypes.c_int
    lib.topk_cols_sample.argtypes = [p, p, i64, i32, i32, ctypes.c_double, ctypes.c_double,
                                     ctypes.c_uint64, ctypes.c_uint64, p, p, p]
    lib.topk_cols_sample.restype = ctypes.c_int
    lib.topk_cols_destroy.argtypes = [p]
    lib.topk_cols_destroy.restype = ctypes.c_int
    lib.topk_cols_status_string.argtypes = [ctypes.c_int]
    lib.topk_cols_status_string.restype = ctypes.c_char_p
    lib.topk_cols_query.argtypes = [p, ctypes.POINTER(i64), ctypes.POINTER(i64), ctypes.POINTER(i64),
                                    ctypes.POINTER(i32)]
    lib.topk_cols_query.restype = ctypes.c_int
    lib.topk_cols_check.argtypes = [p]
    lib.topk_cols_check.restype = ctypes.c_int
    lib.topk_cols_debug_fail_waits.argtypes = [p, i32]
    lib.topk_cols_debug_fail_waits.restype = ctypes.c_int
    lib.topk_cols_run_noalloc.argtypes = [i64, i64, i32, i32, i32, i64, p, p, p, p]
    lib.topk_cols_run_noalloc.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().topk_cols_status_string(int(status)).decode()


def _torch_dtype(dtype: str):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


class TopkCols:
    """One top-k shape on the current GPU (a handle of the C library)."""

    def __init__(self, V: int, C: int, k: int, dtype: str = "bf16", layout: str = "col",
                 ld: int | None = None, segments: int = 0, algo: str = "auto"):
        if dtype not in DTYPES or layout not in LAYOUTS or algo not in ALGOS:
            raise ValueError(f"dtype must be one of {list(DTYPES)}, layout one of {list(LAYOUTS)}, "
                             f"algo one of {list(ALGOS)}")
        self.V, self.C, self.k, self.dtype, self.layout = V, C, k, dtype, layout
        self.ld = ld if ld is not None else (V if layout == "col" else C)
        lib = load()
        self._h = ctypes.c_void_p()
        if segments == 0 and algo == "auto":
            rc = lib.topk_cols_create(ctypes.byref(self._h), V, C, k, DTYPES[dtype], LAYOUTS[layout], self.ld)
        else:
            rc = lib.topk_cols_create_tuned(ctypes.byref(self._h), V, C, k, DTYPES[dtype],
                                            LAYOUTS[layout], self.ld, segments, ALGOS[algo])
        if rc != TOPK_OK:
            raise TopkError(rc, "topk_cols_create")

    def query(self) -> dict:
        s, b, w, a = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
        rc = load().topk_cols_query(self._h, ctypes.byref(s), ctypes.byref(b), ctypes.byref(w), ctypes.byref(a))
        if rc != TOPK_OK:
            raise TopkError(rc, "topk_cols_query")
        names = {v: n for n, v in ALGOS.items()}
        return {"segments": s.value, "blocks": b.value, "workspace_bytes": w.value, "algo": names.get(a.value)}

    def check(self) -> int:
        """topk_cols_check: synchronizes the device; TOPK_OK, or TOPK_ERR_TIMEOUT
        when a run's cross-workgroup wait gave up (the workspace is then reset)."""
        rc = load().topk_cols_check(self._h)
        if rc not in (TOPK_OK, TOPK_ERR_TIMEOUT):
            raise TopkError(rc, "topk_cols_check")
        return rc

    def debug_fail_waits(self, on: bool) -> None:
        """Tests of the error path only (topk_cols_debug_fail_waits)."""
        rc = load().topk_cols_debug_fail_waits(self._h, 1 if on else 0)
        if rc != TOPK_OK:
            raise TopkError(rc, "topk_cols_debug_fail_waits")

    def run_ptr(self, x_ptr: int, values_ptr: int, ids_ptr: int, stream_ptr: int,
                n_cols: int | None = None, id_map_ptr: int | None = None) -> None:
        """Enqueue one run on raw device pointers and a raw HIP stream handle.

        n_cols: active columns (topk_cols_run_n); None runs all C columns.
        id_map_ptr: device row -> id table (topk_cols_run_mapped), or None.
        """
        lib = load()
        if id_map_ptr is not None:
            rc = lib.topk_cols_run_mapped(self._h, self.C if n_cols is None else n_cols, x_ptr, id_map_ptr,
                                          values_ptr, ids_ptr, stream_ptr)
            what = "topk_cols_run_mapped"
        elif n_cols is not None:
            rc = lib.topk_cols_run_n(self._h, n_cols, x_ptr, values_ptr, ids_ptr, stream_ptr)
            what = "topk_cols_run_n"
        else:
            rc = lib.topk_cols_run(self._h, x_ptr, values_ptr, ids_ptr, stream_ptr)
            what = "topk_cols_run"
        if rc != TOPK_OK:
            raise TopkError(rc, what)

    def run(self, x, values=None, ids=None, stream=None, n_cols: int | None = None, id_map=None):
        """Enqueue one run on torch tensors (on the current stream by default).

        x: GPU tensor holding the matrix (bf16 or fp32, or int16/uint16/int32
           bit patterns of the same width), laid out as given at creation.
        values/ids: optional preallocated outputs (C*k elements each).
        n_cols: select over the first n_cols columns only (None: all C).
        id_map: optional int32 GPU tensor of V entries; the ids returned are
           id_map[row] (selection and tie order are unchanged).
        Returns (values, ids) shaped (C, k); with n_cols, rows n_cols.. of
        freshly allocated outputs are left uninitialised.
        """
        import torch
        if not x.is_cuda:
            raise ValueError("x must be a GPU tensor")
        need = (self.C - 1) * self.ld + self.V if self.layout == "col" else (self.V - 1) * self.ld + self.C
        if x.numel() < need or x.element_size() != (2 if self.dtype == "bf16" else 4):
            raise ValueError("x does not hold the matrix described at creation")
        if not x.is_contiguous():
            raise ValueError("x must be contiguous")
        if values is None:
            values = torch.empty((self.C, self.k), dtype=x.dtype, device=x.device)
        if ids is None:
            ids = torch.empty((self.C, self.k), dtype=torch.int32, device=x.device)
        if values.numel() < self.C * self.k or ids.numel() < self.C * self.k:
            raise ValueError("output buffers are too small")
        map_ptr = None
        if id_map is not None:
            if not id_map.is_cuda or id_map.dtype != torch.int32 or id_map.numel() < self.V \
                    or not id_map.is_contiguous():
                raise ValueError("id_map must be a contiguous int32 GPU tensor of V entries")
            map_ptr = id_map.data_ptr()
        s = stream if stream is not None else torch.cuda.current_stream(x.device)
        self.run_ptr(x.data_ptr(), values.data_ptr(), ids.data_ptr(), s.cuda_stream, n_cols, map_ptr)
        return values, ids

    def close(self) -> None:
        if getattr(self, "_h", None) and self._h.value:
            rc = load().topk_cols_destroy(self._h)
            self._h = ctypes.c_void_p()
            if rc != TOPK_OK:
                raise TopkError(rc, "topk_cols_destroy")

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def sample(values, ids, temperature: float = 1.0, top_p: float = 0.95, seed: int = 0, offset: int = 0,
           out_ids=None, out_pos=None, stream=None):
    """One sampled draft per column from top-k outputs (topk_cols_sample).

    values: (C, k) GPU tensor as a run wrote it (bf16 or fp32, or 16/32-bit
    patterns); ids: (C, k) int32 GPU tensor.  Returns (ids, positions), each
    (C,) int32 on the GPU; enqueued on the current stream by default.
    """
    import torch
    if values.dim() != 2 or ids.shape != values.shape or ids.dtype != torch.int32:
        raise ValueError("values and ids must be (C, k) tensors, ids int32")
    if not (values.is_cuda and ids.is_cuda and values.is_contiguous() and ids.is_contiguous()):
        raise ValueError("values and ids must be contiguous GPU tensors")
    C, k = values.shape
    dtype = 0 if values.element_size() == 2 else 1
    if out_ids is None:
        out_ids = torch.empty(C, dtype=torch.int32, device=values.device)
    if out_pos is None:
        out_pos = torch.empty(C, dtype=torch.int32, device=values.device)
    s = stream if stream is not None else torch.cuda.current_stream(values.device)
    rc = load().topk_cols_sample(values.data_ptr(), ids.data_ptr(), C, k, dtype, float(temperature),
                                 float(top_p), int(seed), int(offset), out_ids.data_ptr(), out_pos.data_ptr(),
                                 s.cuda_stream)
    if rc != TOPK_OK:
        raise TopkError(rc, "topk_cols_sample")
    return out_ids, out_pos


def run_noalloc(x, V: int, C: int, k: int, dtype: str = "bf16", layout: str = "col", ld=None,
                values=None, ids=None, stream=None):
    """topk_cols_run_noalloc: one run with no handle and no device allocation
    by the library (the outputs are allocated here when not given).  Returns
    (values, ids) shaped (C, k); enqueued on the current stream by default."""
    import torch
    if dtype not in DTYPES or layout not in LAYOUTS:
        raise ValueError(f"dtype must be one of {list(DTYPES)}, layout one of {list(LAYOUTS)}")
    ld = ld if ld is not None else (V if layout == "col" else C)
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous GPU tensor")
    need = (C - 1) * ld + V if layout == "col" else (V - 1) * ld + C
    if x.numel() < need or x.element_size() != (2 if dtype == "bf16" else 4):
        raise ValueError("x does not hold the matrix described")
    if values is None:
        values = torch.empty((C, k), dtype=x.dtype, device=x.device)
    if ids is None:
        ids = torch.empty((C, k), dtype=torch.int32, device=x.device)
    if values.numel() < C * k or ids.numel() < C * k:
        raise ValueError("output buffers are too small")
    s = stream if stream is not None else torch.cuda.current_stream(x.device)
    rc = load().topk_cols_run_noalloc(V, C, k, DTYPES[dtype], LAYOUTS[layout], ld, x.data_ptr(), values.data_ptr(),
                                      ids.data_ptr(), s.cuda_stream)
    if rc != TOPK_OK:
        raise TopkError(rc, "topk_cols_run_noalloc")
    return values, ids


def topk_cols(x, V: int, C: int, k: int, dtype: str = "bf16", layout: str = "col", ld=None):
    """One-shot convenience: create, run, synchronize, destroy."""
    import torch
    with TopkCols(V, C, k, dtype, layout, ld) as h:
        v, i = h.run(x)
        torch.cuda.current_stream(x.device).synchronize()
        return v, i
