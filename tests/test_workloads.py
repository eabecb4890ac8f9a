"""The seeded generators: determinism and the tie structure each workload claims."""
import hashlib

import numpy as np
import pytest

from drafter_vocab_top_amd import workloads as W


def _digest(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


@pytest.mark.parametrize("n", [1, 2])
def test_same_seed_same_bytes(n):
    a, b = W.config(n), W.config(n)
    assert _digest(a.x) == _digest(b.x)
    assert _digest(W.config(n, seed=77).x) != _digest(a.x)


def test_shapes_match_the_parameters():
    for n in range(1, 6):
        s = W.config_shape(n)
        assert s["ld"] == (s["V"] if s["layout"] == W.COL else s["C"])
    assert W.config_shape(1)["V"] * 7 * 2 == 3_472_644   # 3.47 MB per lane-round


def test_bf16_rounding_is_nearest_even():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1e-40, 3.4e38], dtype=np.float32)
    b = W.bf16_bits_from_f32(f)
    assert b.tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x0001, 0x7F80]
    assert np.array_equal(W.f32_from_bf16_bits(np.array([0x3F82], np.uint16)),
                          np.array([1.015625], np.float32))


def test_config1_has_four_copies_of_each_max():
    w = W.config(1)
    f = W.float_view(w.x, w.dtype)
    for c in range(w.C):
        assert (f[c] == f[c].max()).sum() >= 4


def test_config2_spikes_and_duplicates():
    w = W.config(2)
    assert len(w.notes["spike_copies"]) == 11
    for c, src, dst in w.notes["spike_copies"]:
        assert w.x[c, src] == w.x[c, dst] and src != dst
    f = W.float_view(w.x, w.dtype)
    assert ((f >= 12.0).sum(axis=1) >= 32).all()


@pytest.mark.slow
def test_configs_3_to_5_plant_ties():
    for n in (3, 4):
        w = W.config(n)
        st = W.float_view(w.x, w.dtype) if w.layout == W.COL else None
        for c, pairs in w.notes["copies"].items():
            assert len(pairs) == 4
            for src, dst in pairs:
                assert w.x[c, src].tobytes() == w.x[c, dst].tobytes()
        assert len(w.notes["straddle_columns"]) == 8
        del st
