"""Pins of the sampling oracle (oracle.sample_topk), on the CPU.

The reading (oracle/sample_oracle.c): softmax of the top-k logits at
temperature T, the smallest largest-first prefix whose mass reaches top_p,
one inverse-CDF draw with a Philox4x32-10 uniform.  The pins:
  - Philox4x32-10 against the known-answer vectors published with the
    generator (Salmon et al., SC 2011; the Random123 distribution);
  - the fixed-method exp against the C library's exp (a few ulp);
  - the whole draw against a second route written here with numpy (np.exp,
    np.cumsum, searchsorted): equal positions on thousands of columns;
  - closed forms (k = 1, tiny top_p, equal logits, a dominant logit,
    non-finite tops) and the sampled frequencies against the renormalised
    probabilities (a chi-square bound).
"""
import math

import numpy as np
import pytest

import oracle
from drafter_vocab_top_amd import workloads as W

M0, M1, W0, W1 = 0xD2511F53, 0xCD9E8D57, 0x9E3779B9, 0xBB67AE85


# Known-answer vectors of Philox4x32-10: (counter, key) -> output.
KAT = [
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
    ((0xffffffff, 0xffffffff, 0xffffffff, 0xffffffff), (0xffffffff, 0xffffffff),
     (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
    ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
     (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
]


@pytest.mark.parametrize("ctr,key,expect", KAT)
def test_philox_known_answers(ctr, key, expect):
    assert tuple(int(v) for v in oracle.philox4x32_10(ctr, key)) == expect


def philox_np(ctr, key):
    """Philox4x32-10 over arrays of counters (numpy, uint64 arithmetic)."""
    c = [np.asarray(x, dtype=np.uint64) for x in ctr]
    k0, k1 = np.uint64(key[0]), np.uint64(key[1])
    mask = np.uint64(0xFFFFFFFF)
    for rnd in range(10):
        if rnd:
            k0, k1 = (k0 + np.uint64(W0)) & mask, (k1 + np.uint64(W1)) & mask
        p0, p1 = np.uint64(M0) * c[0], np.uint64(M1) * c[2]
        c = [((p1 >> np.uint64(32)) ^ c[1] ^ k0) & mask, p1 & mask,
             ((p0 >> np.uint64(32)) ^ c[3] ^ k1) & mask, p0 & mask]
    return c


def test_numpy_philox_agrees_with_the_oracle():
    rng = np.random.default_rng(2)
    for _ in range(50):
        ctr = [int(v) for v in rng.integers(0, 2**32, size=4)]
        key = [int(v) for v in rng.integers(0, 2**32, size=2)]
        got = [int(v[()]) for v in philox_np(ctr, key)]
        assert got == [int(v) for v in oracle.philox4x32_10(ctr, key)]
    for ctr, key, expect in KAT:
        assert tuple(int(v[()]) for v in philox_np(ctr, key)) == expect


def test_exp_against_the_c_library():
    xs = np.concatenate([-np.geomspace(1e-12, 745.0, 20000), np.linspace(-40.0, 0.0, 5001)])
    worst = 0.0
    for x in xs:
        got, ref = oracle.sample_exp(float(x)), math.exp(float(x))
        if ref >= 2.2250738585072014e-308:                  # normal results: relative error in ulp
            worst = max(worst, abs(got - ref) / math.ulp(ref))
        else:                                               # subnormal results: a few ulp of 2^-1074
            assert abs(got - ref) <= 4 * 5e-324, x
    assert worst <= 4.0, worst
    assert oracle.sample_exp(0.0) == 1.0
    assert oracle.sample_exp(-math.inf) == 0.0 and oracle.sample_exp(-746.0) == 0.0


def uniforms(C, seed, offset):
    out = philox_np([np.full(C, offset & 0xFFFFFFFF), np.full(C, offset >> 32), np.arange(C), np.zeros(C)],
                    [seed & 0xFFFFFFFF, seed >> 32])
    bits = (out[0] << np.uint64(32)) | out[1]
    return (bits >> np.uint64(11)).astype(np.float64) * 2.0 ** -53


def numpy_route(vals_f, T, p, seed, offset):
    """The draw written independently: np.exp, np.cumsum, searchsorted."""
    C, k = vals_f.shape
    u = uniforms(C, seed, offset)
    pos = np.empty(C, dtype=np.int64)
    for c in range(C):
        w = np.exp((vals_f[c].astype(np.float64) - float(vals_f[c, 0])) / T)
        cs = np.cumsum(w)
        n = int(np.searchsorted(cs, p * cs[-1], side="left")) + 1
        pos[c] = int(np.searchsorted(cs[:n], u[c] * cs[n - 1], side="right"))
    return pos


def sorted_topk(seed, C, k, dtype, kind="normal"):
    """A (C, k) matrix of stored bits, each row sorted largest first (real values)."""
    x = W.random_matrix(seed, 4 * k + 3, C, dtype, W.COL, kind=kind)
    v, i = oracle.topk_cols(x, 4 * k + 3, C, k, oracle.BF16 if dtype == W.BF16 else oracle.F32,
                            oracle.COL_CONTIG, 4 * k + 3)
    return v, i


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
@pytest.mark.parametrize("T,p", [(1.0, 0.95), (0.5, 0.9), (2.0, 1.0), (1.0, 0.5), (0.05, 0.95)])
def test_matches_the_numpy_route(dtype, T, p):
    C, k = 3000, 20
    v, ids = sorted_topk(int(T * 100 + p * 10), C, k, dtype)
    odt = oracle.BF16 if dtype == W.BF16 else oracle.F32
    f = W.float_view(v, dtype)
    for seed, offset in ((1, 0), (2**40 + 7, 3), (0xDEADBEEF, 2**33 + 1)):
        sid, pos = oracle.sample_topk(v, ids, C, k, odt, T, p, seed, offset)
        ref = numpy_route(f, T, p, seed, offset)
        assert np.array_equal(pos, ref), (seed, offset, np.flatnonzero(pos != ref)[:5])
        assert np.array_equal(sid, ids[np.arange(C), pos])


def test_closed_forms():
    C = 500
    # k = 1: always the top
    v, ids = sorted_topk(3, C, 1, W.F32)
    _, pos = oracle.sample_topk(v, ids, C, 1, oracle.F32, 1.0, 0.95, 5, 0)
    assert (pos == 0).all()
    # a tiny top_p keeps only the top
    v, ids = sorted_topk(4, C, 20, W.BF16)
    _, pos = oracle.sample_topk(v, ids, C, 20, oracle.BF16, 1.0, 1e-9, 5, 0)
    assert (pos == 0).all()
    # equal logits with top_p = 1: position floor(u * k)
    k = 20
    v = np.full((C, k), 0x3FC0, dtype=np.uint16)             # 1.5 everywhere
    ids = np.tile(np.arange(k, dtype=np.int32), (C, 1))
    _, pos = oracle.sample_topk(v, ids, C, k, oracle.BF16, 1.0, 1.0, 11, 7)
    u = uniforms(C, 11, 7)
    assert np.array_equal(pos, np.floor(u * k).astype(np.int64))
    # one logit 1000 above the rest: always the top
    f = np.full((C, k), -500.0, dtype=np.float32)
    f[:, 0] = 500.0
    _, pos = oracle.sample_topk(f.view(np.uint32), ids, C, k, oracle.F32, 1.0, 0.95, 13, 0)
    assert (pos == 0).all()
    # a non-finite top: position 0
    for top in (np.inf, np.nan, -np.inf):
        f = np.full((C, k), -np.inf if top == -np.inf else 1.0, dtype=np.float32)
        f[:, 0] = top
        _, pos = oracle.sample_topk(f.view(np.uint32), ids, C, k, oracle.F32, 1.0, 0.95, 13, 0)
        assert (pos == 0).all(), top


def test_frequencies_follow_the_renormalised_probabilities():
    k, T, p = 8, 1.0, 0.95
    logits = np.array([2.0, 1.5, 1.0, 0.5, 0.0, -0.5, -1.0, -4.0], dtype=np.float32)
    w = np.exp((logits.astype(np.float64) - logits[0]) / T)
    cs = np.cumsum(w)
    n = int(np.searchsorted(cs, p * cs[-1])) + 1
    prob = w[:n] / cs[n - 1]
    C, rounds = 4000, 10
    v = np.tile(logits, (C, 1))
    ids = np.tile(np.arange(k, dtype=np.int32), (C, 1))
    counts = np.zeros(k)
    for offset in range(rounds):
        _, pos = oracle.sample_topk(v.view(np.uint32), ids, C, k, oracle.F32, T, p, 99, offset)
        counts += np.bincount(pos, minlength=k)
    assert counts[n:].sum() == 0          # nothing outside the nucleus
    expect = prob * C * rounds
    chi2 = float(((counts[:n] - expect) ** 2 / expect).sum())
    assert chi2 < 40.0, (chi2, counts, expect)   # n - 1 <= 7 degrees of freedom; p ~ 1e-6


def test_bad_arguments_are_refused():
    v, ids = sorted_topk(1, 4, 8, W.F32)
    for T, p in ((0.0, 0.9), (-1.0, 0.9), (math.inf, 0.9), (1.0, 0.0), (1.0, 1.5), (math.nan, 0.9)):
        with pytest.raises(ValueError):
            oracle.sample_topk(v, ids, 4, 8, oracle.F32, T, p, 1, 0)
