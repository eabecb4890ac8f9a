"""The C ABI on a host without a GPU: the library loads, exports every function
include/topk_cols.h declares, refuses invalid arguments before touching a
device, and fails cleanly (TOPK_ERR_HIP, NULL handle) when no device exists."""
import ctypes
import os
import re
import subprocess

import pytest

from drafter_vocab_top_amd import topk_cols as T

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", n) for n in os.listdir(os.path.join(ROOT, "include"))
           if n.endswith(".h")]


def declared_functions():
    names = []
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(topk_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(T.LIBRARY):
        pytest.fail("libtopk_cols.so is not built (run __graft_entry__.build())")
    return T.load()


def test_header_declares_the_expected_entry_points():
    assert set(declared_functions()) == set(T.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", T.LIBRARY], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (\w+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_status_strings_cover_every_code(lib):
    for code in (T.TOPK_OK, T.TOPK_ERR_INVALID_ARG, T.TOPK_ERR_UNSUPPORTED, T.TOPK_ERR_HIP,
                 T.TOPK_ERR_OUT_OF_MEMORY, T.TOPK_ERR_TIMEOUT):
        s = T.status_string(code)
        assert s and "unknown" not in s
    assert "unknown" in T.status_string(12345)


def _create(lib, *args, segments=None):
    h = ctypes.c_void_p(0xDEAD)
    if segments is None:
        rc = lib.topk_cols_create(ctypes.byref(h), *args)
    else:
        rc = lib.topk_cols_create_with_segments(ctypes.byref(h), *args, segments)
    return rc, h


@pytest.mark.parametrize("args,expect", [
    ((0, 7, 1, 0, 0, 1), T.TOPK_ERR_INVALID_ARG),            # V < 1
    ((10, 0, 1, 0, 0, 10), T.TOPK_ERR_INVALID_ARG),          # C < 1
    ((10, 7, 0, 0, 0, 10), T.TOPK_ERR_INVALID_ARG),          # k < 1
    ((10, 7, 11, 0, 0, 10), T.TOPK_ERR_INVALID_ARG),         # k > V
    ((10, 7, 1, 2, 0, 10), T.TOPK_ERR_INVALID_ARG),          # unknown dtype
    ((10, 7, 1, 0, 2, 10), T.TOPK_ERR_INVALID_ARG),          # unknown layout
    ((10, 7, 1, 0, 0, 9), T.TOPK_ERR_INVALID_ARG),           # ld < V (column-contiguous)
    ((10, 7, 1, 0, 1, 6), T.TOPK_ERR_INVALID_ARG),           # ld < C (row-interleaved)
    ((100, 7, 65, 0, 0, 100), T.TOPK_ERR_UNSUPPORTED),       # k > TOPK_MAX_K
    ((1 << 24, 7, 8, 0, 0, 1 << 24), T.TOPK_ERR_UNSUPPORTED),  # V > TOPK_MAX_V
    ((10, 1 << 27, 1, 0, 1, 1 << 27), T.TOPK_ERR_UNSUPPORTED),  # row bound area past 2^32 words
])
def test_invalid_arguments_refused_without_a_device(lib, args, expect):
    rc, h = _create(lib, *args)
    assert rc == expect
    assert h.value is None          # *out is NULL after any failure


def test_negative_segments_refused(lib):
    rc, h = _create(lib, 100, 7, 8, 0, 0, 100, segments=-1)
    assert rc == T.TOPK_ERR_INVALID_ARG and h.value is None
    rc, h = _create(lib, 100000, 7, 64, 0, 0, 100000, segments=65)
    assert rc == T.TOPK_ERR_UNSUPPORTED and h.value is None
    # row-interleaved: the merge takes at most 2048 keys per column
    rc, h = _create(lib, 100000, 448, 64, 0, 1, 448, segments=33)
    assert rc == T.TOPK_ERR_UNSUPPORTED and h.value is None


def test_tuned_create_checks_its_arguments(lib):
    def tuned(*args):
        h = ctypes.c_void_p(0xDEAD)
        rc = lib.topk_cols_create_tuned(ctypes.byref(h), *args)
        return rc, h
    rc, h = tuned(100, 7, 8, 0, 0, 100, 0, 4)           # unknown algorithm
    assert rc == T.TOPK_ERR_INVALID_ARG and h.value is None
    rc, h = tuned(100, 7, 8, 0, 0, 100, 2, 3)           # one wave per column: no split
    assert rc == T.TOPK_ERR_UNSUPPORTED and h.value is None
    rc, h = tuned(100, 448, 8, 0, 1, 448, 0, 3)         # ... and column-contiguous only
    assert rc == T.TOPK_ERR_UNSUPPORTED and h.value is None
    rc, h = tuned(100, 448, 8, 0, 1, 448, 0, 1)         # row-interleaved takes only "auto"
    assert rc == T.TOPK_ERR_UNSUPPORTED and h.value is None
    rc, h = tuned(100, 7, 8, 0, 0, 100, 0, 2)           # 2: the removed wave-per-segment family
    assert rc == T.TOPK_ERR_INVALID_ARG and h.value is None


def test_null_out_pointer_refused(lib):
    assert lib.topk_cols_create(None, 10, 7, 1, 0, 0, 10) == T.TOPK_ERR_INVALID_ARG


def test_null_handle_calls(lib):
    assert lib.topk_cols_destroy(None) == T.TOPK_OK
    assert lib.topk_cols_run(None, 16, 16, 16, None) == T.TOPK_ERR_INVALID_ARG
    assert lib.topk_cols_run_n(None, 1, 16, 16, 16, None) == T.TOPK_ERR_INVALID_ARG
    assert lib.topk_cols_run_mapped(None, 1, 16, 16, 16, 16, None) == T.TOPK_ERR_INVALID_ARG
    assert lib.topk_cols_debug_fail_waits(None, 1) == T.TOPK_ERR_INVALID_ARG
    for args in ((None, 16, 16), (16, None, 16), (16, 16, None)):      # NULL logits, values, ids
        assert lib.topk_cols_run_noalloc(1000, 7, 8, 0, 0, 1000, *args, None) == T.TOPK_ERR_INVALID_ARG
    assert lib.topk_cols_run_noalloc(1000, 7, 8, 0, 0, 1000, 17, 16, 16, None) == T.TOPK_ERR_INVALID_ARG  # misaligned
    assert lib.topk_cols_run_noalloc(1000, 7, 65, 0, 0, 1000, 16, 16, 16, None) == T.TOPK_ERR_UNSUPPORTED
    assert lib.topk_cols_run_noalloc(1000, 7, 8, 0, 0, 999, 16, 16, 16, None) == T.TOPK_ERR_INVALID_ARG  # ld < V


def test_sample_checks_its_arguments_before_any_launch(lib):
    # pointers are never dereferenced on the host; every case fails validation
    good = (16, 16, 4, 8, 1, 1.0, 0.95, 0, 0, 16, None, None)
    def call(**kw):
        a = list(good)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return lib.topk_cols_sample(*a)
    assert call(a0=None) == T.TOPK_ERR_INVALID_ARG           # values
    assert call(a1=None) == T.TOPK_ERR_INVALID_ARG           # ids
    assert call(a9=None) == T.TOPK_ERR_INVALID_ARG           # out_ids
    assert call(a2=0) == T.TOPK_ERR_INVALID_ARG              # C < 1
    assert call(a3=0) == T.TOPK_ERR_INVALID_ARG              # k < 1
    assert call(a3=65) == T.TOPK_ERR_INVALID_ARG             # k > TOPK_MAX_K
    assert call(a4=2) == T.TOPK_ERR_INVALID_ARG              # dtype
    assert call(a5=0.0) == T.TOPK_ERR_INVALID_ARG            # temperature
    assert call(a5=float("inf")) == T.TOPK_ERR_INVALID_ARG
    assert call(a6=0.0) == T.TOPK_ERR_INVALID_ARG            # top_p
    assert call(a6=1.5) == T.TOPK_ERR_INVALID_ARG
    assert call(a0=17) == T.TOPK_ERR_INVALID_ARG             # misaligned fp32 values
    assert call(a10=18) == T.TOPK_ERR_INVALID_ARG            # misaligned out_pos
    assert lib.topk_cols_query(None, None, None, None, None) == T.TOPK_ERR_INVALID_ARG


def test_valid_create_without_a_device_fails_cleanly(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    rc, h = _create(lib, 248046, 7, 8, 0, 0, 248046)
    assert rc == T.TOPK_ERR_HIP
    assert h.value is None
    # the no-allocation entry point and its check need a device as well
    assert lib.topk_cols_run_noalloc(248046, 7, 8, 0, 0, 248046, 16, 16, 16, None) == T.TOPK_ERR_HIP
    assert lib.topk_cols_check(None) == T.TOPK_ERR_HIP
