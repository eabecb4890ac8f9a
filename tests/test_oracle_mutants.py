"""Planted mistakes in the oracle must fail its pins (CPU only).

Each case copies oracle/topk_oracle.c and changes one expression into a
plausible mistake: a flipped comparison, a wrong shift, a transposed index,
a wrong output slot.  It builds the copy with gcc in a temporary directory and
runs the pins from tests/test_oracle.py against that build.  If every pin
still passes, the pins cannot see that kind of mistake, and the test fails.
The oracle itself is never modified.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from drafter_vocab_top_amd import workloads as W
from topk_checks import bits, golden_names, read_golden, torch_reference

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "topk_oracle.c")

MUTANTS = {
    "tie_to_larger_row": ("return a->row < b->row; /* equal values", "return a->row > b->row; /* equal values"),
    "nan_smallest": ("return a->is_nan;                                   /* NaN is largest */",
                     "return b->is_nan;"),
    "nan_ties_reversed": ("if (a->is_nan && b->is_nan) return a->row < b->row;",
                          "if (a->is_nan && b->is_nan) return a->row > b->row;"),
    "ascending_values": ("if (a->value > b->value) return 1;\n    if (a->value < b->value) return 0;",
                         "if (a->value < b->value) return 1;\n    if (a->value > b->value) return 0;"),
    "bf16_wrong_shift": ("bits32 = (uint32_t)b << 16;", "bits32 = (uint32_t)b << 15;"),
    "layout_transposed": ("return j->layout == ORACLE_COL_CONTIG ? c * j->ld + r : r * j->ld + c;",
                          "return j->layout == ORACLE_COL_CONTIG ? r * j->ld + c : c * j->ld + r;"),
    "value_from_rank_not_row": ("int64_t src = element_index(j, pairs[t].row, c);",
                                "int64_t src = element_index(j, t, c);"),
    "output_slot_transposed": ("int64_t dst = c * (int64_t)j->k + t;",
                               "int64_t dst = t * j->C + c;"),
    "plus_zero_above_minus_zero": ("return a->row < b->row; /* equal values",
                                   "if (signbit(a->value) != signbit(b->value)) return !signbit(a->value);\n    return a->row < b->row; /* equal values"),
    "last_row_skipped": ("for (int64_t r = 0; r < j->V; ++r) {", "for (int64_t r = 0; r + 1 < j->V; ++r) {"),
    "nan_as_value": ("*is_nan = isnan(f) ? 1 : 0;", "*is_nan = 0;"),
}


def _build_mutant(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-D_POSIX_C_SOURCE=200809L", "-fPIC", "-shared",
                    "-pthread", "-o", str(lib), str(path), "-lm"], check=True)
    return oracle.load_library(str(lib))


def _pins_pass(lib):
    """True if the build passes every pin below; False at the first failure."""
    odt = {W.BF16: oracle.BF16, W.F32: oracle.F32}
    oly = {W.COL: oracle.COL_CONTIG, W.ROW: oracle.ROW_INTERLEAVED}
    for name in golden_names():
        g = read_golden(name)
        try:
            v, i = oracle.topk_cols(g["x"], g["V"], g["C"], g["k"], odt[g["dtype"]],
                                    oly[g["layout"]], g["ld"], lib=lib)
        except ValueError:
            return False
        if not (np.array_equal(bits(v), g["values"]) and np.array_equal(i, g["ids"])):
            return False
    for dtype in (W.BF16, W.F32):
        for layout in (W.COL, W.ROW):
            for kind in ("alphabet", "special", "normal"):
                V, C = 301, 3
                ld = V + 2 if layout == W.COL else C + 1
                x = W.random_matrix(5, V, C, dtype, layout, ld=ld, kind=kind)
                for k in (1, 5):
                    v, i = oracle.topk_cols(x, V, C, k, odt[dtype], oly[layout], ld, lib=lib)
                    rv, ri = torch_reference(x, V, C, k, dtype, layout, ld)
                    if not (np.array_equal(i, ri) and np.array_equal(bits(v), bits(rv))):
                        return False
    return True


def test_unmodified_oracle_passes_the_pin_battery():
    assert _pins_pass(None)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    lib = _build_mutant(tmp_path, name)
    assert not _pins_pass(lib), f"the pins did not catch the planted mistake '{name}'"
