"""Seeded synthetic logit matrices: the five benchmark workloads and test inputs.

This module only builds inputs.  It never computes a top-k result and holds
no expected outputs.  The GPU path, the tests, the bench and the oracle all
take their inputs from here, so every side reads the same bytes.

Storage conventions:
  * bf16 matrices are numpy ``uint16`` arrays of bit patterns.  The generator
    draws in float64, casts to float32, then rounds to bf16 with
    round-to-nearest-even.
  * fp32 matrices are numpy ``float32`` arrays.
  * Column-contiguous ("col") matrices have shape (C, ld): element (r, c) is
    at [c, r].  Row-interleaved ("row") matrices have shape (V, ld): element
    (r, c) is at [r, c].

The shapes come from the speculative-drafter setting on the ignis "DFlash2"
page.  That page describes a 248,046-token vocabulary, 7 draft columns per
lane, 56 at eight lanes, a 131,072-row shortlist head, and top_k 20 under
sampling (sections "How it works" and "The numbers").  The pages publish no
logits, so every value here is synthetic.

Several tie recipes pick which values to duplicate ("4 of the 16 largest").
To find those values they use numpy's partition and sort on the float values.
That only shapes the input; the top-k answer is never recorded here.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BF16 = "bf16"
F32 = "f32"
COL = "col"
ROW = "row"

NUM_CONFIGS = 5
VOCAB = 248_046
SHORTLIST_VOCAB = 131_072


@dataclass
class Workload:
    """A logit matrix plus the parameters of the top-k call it feeds."""
    name: str
    V: int
    C: int
    k: int
    dtype: str          # "bf16" (x is uint16 bit patterns) or "f32" (x is float32)
    layout: str         # "col": x[c, r];  "row": x[r, c]
    ld: int
    x: np.ndarray
    seed: int
    notes: dict = field(default_factory=dict)

    @property
    def element_bytes(self) -> int:
        return 2 if self.dtype == BF16 else 4

    @property
    def matrix_bytes(self) -> int:
        """Bytes of the V x C matrix itself (padding excluded)."""
        return self.V * self.C * self.element_bytes


# ---------------------------------------------------------------- rounding ---

def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return bits.

    The input must be free of NaN (the generators never make one).
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def float_view(x: np.ndarray, dtype: str) -> np.ndarray:
    """The stored values as float32 (exact for both dtypes)."""
    return f32_from_bf16_bits(x) if dtype == BF16 else np.asarray(x, dtype=np.float32)


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _normal_bf16(rng: np.random.Generator, shape, sigma: float, mean=0.0) -> np.ndarray:
    """Draw N(mean, sigma^2) in float64, cast to float32, round to bf16 bits."""
    out = np.empty(shape, dtype=np.uint16)
    flat = out.reshape(shape[0], -1)
    chunk = max(1, (1 << 23) // max(1, flat.shape[1]))
    for i in range(0, flat.shape[0], chunk):
        rows = slice(i, min(flat.shape[0], i + chunk))
        draw = rng.standard_normal((rows.stop - rows.start, flat.shape[1]))
        m = mean[rows, None] if isinstance(mean, np.ndarray) else mean
        flat[rows] = bf16_bits_from_f32((draw * sigma + m).astype(np.float32))
    return out


# ------------------------------------------------------------ tie injection ---

def _top_rows(values: np.ndarray, n: int) -> np.ndarray:
    """Rows of the n largest values of one column, largest first (input shaping only)."""
    part = np.argpartition(-values, n - 1)[:n]
    order = np.lexsort((part, -values[part]))
    return part[order]


def _copy_top_values(rng, col_vals: np.ndarray, col_bits: np.ndarray, top: int, ncopy: int,
                     force_rank: int | None) -> list:
    """Copy `ncopy` of the `top` largest values of one column exactly to random
    rows outside those `top` rows.  If `force_rank` is given, the value at that
    0-based rank is among the copies (a tie straddling rank k).  Returns the
    (source_row, dest_row) pairs."""
    V = col_vals.shape[0]
    top_rows = _top_rows(col_vals, top)
    ranks = rng.choice(top, size=ncopy, replace=False)
    if force_rank is not None and force_rank not in ranks:
        ranks[0] = force_rank
    taken = set(int(r) for r in top_rows)
    pairs = []
    for rank in ranks:
        src = int(top_rows[rank])
        while True:
            dst = int(rng.integers(0, V))
            if dst not in taken:
                break
        taken.add(dst)
        col_bits[dst] = col_bits[src]
        pairs.append((src, dst))
    return pairs


# --------------------------------------------------------------- workloads ---

def config(n: int, seed: int | None = None) -> Workload:
    """Benchmark workload n (1..5); default seed 1000 + n."""
    if seed is None:
        seed = 1000 + n
    builders = {1: _config1, 2: _config2, 3: _config3, 4: _config4, 5: _config5}
    if n not in builders:
        raise ValueError(f"workload {n} does not exist (1..{NUM_CONFIGS})")
    return builders[n](seed)


def config_shape(n: int) -> dict:
    """The parameters of workload n without generating its data."""
    shapes = {
        1: dict(V=VOCAB, C=7, k=1, dtype=BF16, layout=COL, ld=VOCAB),
        2: dict(V=VOCAB, C=7, k=8, dtype=BF16, layout=COL, ld=VOCAB),
        3: dict(V=VOCAB, C=56, k=8, dtype=BF16, layout=COL, ld=VOCAB),
        4: dict(V=SHORTLIST_VOCAB, C=56, k=20, dtype=F32, layout=COL, ld=SHORTLIST_VOCAB),
        5: dict(V=VOCAB, C=448, k=16, dtype=BF16, layout=ROW, ld=448),
    }
    return dict(shapes[n])


def _config1(seed: int) -> Workload:
    """One lane, argmax: 248,046 x 7 bf16 N(0, 4^2), each column's maximum
    copied exactly to 3 further random rows."""
    s = config_shape(1)
    rng = _rng(seed)
    x = _normal_bf16(rng, (s["C"], s["V"]), 4.0)
    copies = []
    for c in range(s["C"]):
        vals = f32_from_bf16_bits(x[c])
        peak = vals.max()
        holders = set(int(r) for r in np.flatnonzero(vals == peak))
        src = min(holders)
        dst = []
        while len(dst) < 3:
            r = int(rng.integers(0, s["V"]))
            if r not in holders and r not in dst:
                dst.append(r)
        x[c, dst] = x[c, src]
        copies.append(dst)
    return Workload("cfg1 V=248046 C=7 k=1 bf16 col", x=x, seed=seed,
                    notes={"max_copies": copies}, **s)


def _config2(seed: int) -> Workload:
    """One lane, k=8: N(0, 4^2) plus 32 spikes per column (12 + 3*Exp(1)) at
    distinct rows drawn from a Zipf law over the row id (P(r) ~ 1/(r+1));
    5% of all spikes copied exactly to another non-spike row of their column."""
    s = config_shape(2)
    V, C = s["V"], s["C"]
    rng = _rng(seed)
    x = _normal_bf16(rng, (C, V), 4.0)
    zipf = 1.0 / np.arange(1, V + 1, dtype=np.float64)
    zipf /= zipf.sum()
    spikes = []
    for c in range(C):
        rows = rng.choice(V, size=32, replace=False, p=zipf)
        vals = 12.0 + 3.0 * rng.standard_exponential(32)
        x[c, rows] = bf16_bits_from_f32(vals.astype(np.float32))
        spikes.append(rows)
    n_dup = int(round(0.05 * 32 * C))
    chosen = rng.choice(32 * C, size=n_dup, replace=False)
    dups = []
    for idx in chosen:
        c, j = divmod(int(idx), 32)
        taken = set(int(r) for r in spikes[c])
        while True:
            dst = int(rng.integers(0, V))
            if dst not in taken:
                break
        spikes[c] = np.append(spikes[c], dst)
        x[c, dst] = x[c, spikes[c][j]]
        dups.append((c, int(spikes[c][j]), dst))
    return Workload("cfg2 V=248046 C=7 k=8 bf16 col", x=x, seed=seed,
                    notes={"spike_copies": dups}, **s)


def _config3(seed: int) -> Workload:
    """Eight lanes: 248,046 x 56 bf16, per-column mean U(-2, 2) plus N(0, 4^2);
    per column 4 of the 16 largest values copied exactly to rows outside the
    top 16; 8 columns always copy their rank-8 value (a tie straddling k=8)."""
    s = config_shape(3)
    V, C = s["V"], s["C"]
    rng = _rng(seed)
    mu = rng.uniform(-2.0, 2.0, size=C)
    x = _normal_bf16(rng, (C, V), 4.0, mean=mu)
    straddle = set(int(c) for c in rng.choice(C, size=8, replace=False))
    copies = {}
    for c in range(C):
        copies[c] = _copy_top_values(rng, f32_from_bf16_bits(x[c]), x[c], 16, 4,
                                     7 if c in straddle else None)
    return Workload("cfg3 V=248046 C=56 k=8 bf16 col", x=x, seed=seed,
                    notes={"copies": copies, "straddle_columns": sorted(straddle)}, **s)


def _config4(seed: int) -> Workload:
    """Shortlist head: 131,072 x 56 fp32 N(0, 3^2); 5% of the rows (the same
    rows in every column) drawn instead from 3 * Student-t(df=2); per column 4
    of the 24 largest values copied exactly to other rows; 8 columns always
    copy their rank-20 value (a tie straddling k=20)."""
    s = config_shape(4)
    V, C = s["V"], s["C"]
    rng = _rng(seed)
    x = (rng.standard_normal((C, V)) * 3.0).astype(np.float32)
    heavy = rng.choice(V, size=int(round(0.05 * V)), replace=False)
    x[:, heavy] = (3.0 * rng.standard_t(2.0, size=(C, heavy.size))).astype(np.float32)
    straddle = set(int(c) for c in rng.choice(C, size=8, replace=False))
    copies = {}
    for c in range(C):
        copies[c] = _copy_top_values(rng, x[c], x[c], 24, 4, 19 if c in straddle else None)
    return Workload("cfg4 V=131072 C=56 k=20 f32 col", x=x, seed=seed,
                    notes={"copies": copies, "heavy_rows": heavy.size,
                           "straddle_columns": sorted(straddle)}, **s)


def _config5(seed: int) -> Workload:
    """64 rounds x 7 drafts: 248,046 x 448 bf16 N(0, 4^2) stored row-interleaved
    [V][C]; per column 4 of the 32 largest values copied exactly to other rows;
    32 columns always copy their rank-16 value (a tie straddling k=16)."""
    s = config_shape(5)
    V, C = s["V"], s["C"]
    rng = _rng(seed)
    x = _normal_bf16(rng, (V, C), 4.0)
    straddle = set(int(c) for c in rng.choice(C, size=32, replace=False))
    copies = {}
    for c in range(C):
        col = np.ascontiguousarray(x[:, c])
        copies[c] = _copy_top_values(rng, f32_from_bf16_bits(col), col, 32, 4,
                                     15 if c in straddle else None)
        x[:, c] = col
    return Workload("cfg5 V=248046 C=448 k=16 bf16 row", x=x, seed=seed,
                    notes={"copies": copies, "straddle_columns": sorted(straddle)}, **s)


# ------------------------------------------------------------- test inputs ---

SPECIAL_BF16 = {
    "+0": 0x0000, "-0": 0x8000, "+inf": 0x7F80, "-inf": 0xFF80,
    "+nan": 0x7FC0, "-nan": 0xFFC0, "+nan_payload": 0x7F81, "-nan_payload": 0xFFFF,
    "+min_sub": 0x0001, "-min_sub": 0x8001, "+max": 0x7F7F, "-max": 0xFF7F, "1": 0x3F80,
}
SPECIAL_F32 = {
    "+0": 0x00000000, "-0": 0x80000000, "+inf": 0x7F800000, "-inf": 0xFF800000,
    "+nan": 0x7FC00000, "-nan": 0xFFC00000, "+nan_payload": 0x7F800001,
    "-nan_payload": 0xFFFFFFFF, "+min_sub": 0x00000001, "-min_sub": 0x80000001,
    "+max": 0x7F7FFFFF, "-max": 0xFF7FFFFF, "1": 0x3F800000,
}


def storage_from_bits(bits, dtype: str) -> np.ndarray:
    """Turn raw bit patterns into the storage array of `dtype`."""
    if dtype == BF16:
        return np.asarray(bits, dtype=np.uint16)
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


def random_matrix(seed: int, V: int, C: int, dtype: str, layout: str, ld: int | None = None,
                  kind: str = "normal", pad_bits: int | None = None) -> np.ndarray:
    """A seeded test matrix in the given layout.

    kind: "normal"   N(0, 4^2)
          "alphabet" values drawn from {-2, -1, -0, +0, 1, 2} (dense ties)
          "special"  a mix of normals, +-0, +-Inf, subnormals and NaNs
          "equal"    every element 1.5
          "asc"/"desc" strictly increasing/decreasing with the row id
    Padding (elements inside ld but outside the matrix) is set to pad_bits
    (default: the largest finite value), so a kernel that reads padding shows up.
    """
    rng = _rng(seed)
    if ld is None:
        ld = V if layout == COL else C
    specials = SPECIAL_BF16 if dtype == BF16 else SPECIAL_F32
    if kind == "normal":
        vals = (rng.standard_normal((V, C)) * 4.0).astype(np.float32)
    elif kind == "alphabet":
        alphabet = np.array([-2.0, -1.0, -0.0, 0.0, 1.0, 2.0], dtype=np.float32)
        vals = alphabet[rng.integers(0, alphabet.size, size=(V, C))]
    elif kind == "equal":
        vals = np.full((V, C), 1.5, dtype=np.float32)
    elif kind in ("asc", "desc"):
        # strictly increasing positive bit patterns (hence values) down the rows
        base = 0x0001 if dtype == BF16 else 0x3F800000
        limit = 0x7F7F if dtype == BF16 else 0x7F7FFFFF
        if base + V - 1 > limit:
            raise ValueError("V too large for a strictly monotone column")
        b = (base + np.arange(V, dtype=np.uint64))
        bits = np.repeat(b[:, None], C, axis=1)
        if kind == "desc":
            bits = bits[::-1].copy()
        return _place(bits, V, C, ld, layout, dtype, pad_bits, specials)
    elif kind == "special":
        vals = (rng.standard_normal((V, C)) * 4.0).astype(np.float32)
        bits = (bf16_bits_from_f32(vals) if dtype == BF16 else vals.view(np.uint32)).astype(np.uint64)
        names = list(specials)
        mask = rng.random((V, C)) < 0.25
        picks = rng.integers(0, len(names), size=(V, C))
        table = np.array([specials[nm] for nm in names], dtype=np.uint64)
        bits = np.where(mask, table[picks], bits)
        return _place(bits, V, C, ld, layout, dtype, pad_bits, specials)
    else:
        raise ValueError(kind)
    bits = bf16_bits_from_f32(vals) if dtype == BF16 else vals.view(np.uint32)
    return _place(bits, V, C, ld, layout, dtype, pad_bits, specials)


def _place(bits_vc, V, C, ld, layout, dtype, pad_bits, specials):
    """Lay a (V, C) array of bit patterns out in storage with padding."""
    if pad_bits is None:
        pad_bits = specials["+max"]
    st = np.uint16 if dtype == BF16 else np.uint32
    if layout == COL:
        out = np.full((C, ld), pad_bits, dtype=st)
        out[:, :V] = np.asarray(bits_vc, dtype=np.uint64).T.astype(st)
    else:
        out = np.full((V, ld), pad_bits, dtype=st)
        out[:, :C] = np.asarray(bits_vc, dtype=np.uint64).astype(st)
    return storage_from_bits(out, dtype)


def exhaustive_columns(alphabet_bits, V: int) -> np.ndarray:
    """Every length-V column over the given bit patterns: shape (len^V, V)."""
    a = np.asarray(alphabet_bits, dtype=np.uint64)
    n = a.size
    idx = np.indices((n,) * V).reshape(V, -1).T
    return a[idx]
