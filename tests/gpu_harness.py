"""Shared helpers of the GPU parity tests: device copies, one run of the HIP
library through its C ABI, one run of the oracle, and the bit-exact check."""
import numpy as np

import oracle
from drafter_vocab_top_amd import workloads as W
from topk_checks import bits, check_invariants

ODT = {W.BF16: oracle.BF16, W.F32: oracle.F32}
OLY = {W.COL: oracle.COL_CONTIG, W.ROW: oracle.ROW_INTERLEAVED}


def to_device(torch, x, offset=0):
    """Copy a storage array to the GPU, starting `offset` elements into a fresh
    buffer (offset > 0 gives a base that is not 16-byte aligned).  The words
    around the copy hold the largest finite value, so stray reads show up."""
    flat = np.ascontiguousarray(x).reshape(-1)
    if flat.dtype == np.uint16:
        host = torch.from_numpy(flat.view(np.int16))
    else:
        host = torch.from_numpy(flat.view(np.int32))
    buf = torch.empty(flat.size + offset + 8, dtype=host.dtype, device="cuda")
    buf.fill_(0x7F7F if flat.dtype == np.uint16 else 0x7F7FFFFF)
    buf[offset:offset + flat.size].copy_(host)
    return buf[offset:offset + flat.size]


def run_gpu(gpu, x, V, C, k, dtype, layout, ld, segments=0, offset=0, repeat=1, algo="auto"):
    torch, T = gpu
    dx = to_device(torch, x, offset)
    with T.TopkCols(V, C, k, dtype, layout, ld, segments=segments, algo=algo) as h:
        for _ in range(repeat):
            v, i = h.run(dx)
        torch.cuda.synchronize()
    st = np.uint16 if dtype == W.BF16 else np.uint32
    return v.cpu().numpy().view(st).reshape(C, k), i.cpu().numpy().reshape(C, k)


def run_oracle(x, V, C, k, dtype, layout, ld, nthreads=8):
    return oracle.topk_cols(x, V, C, k, ODT[dtype], OLY[layout], ld, nthreads=nthreads)


def assert_parity(gpu, x, V, C, k, dtype, layout, ld, segments=0, offset=0, label="", algo="auto"):
    gv, gi = run_gpu(gpu, x, V, C, k, dtype, layout, ld, segments=segments, offset=offset, algo=algo)
    ov, oi = run_oracle(x, V, C, k, dtype, layout, ld)
    bad = np.flatnonzero((gi != oi).any(axis=1) | (bits(gv) != bits(ov)).any(axis=1))
    assert bad.size == 0, (f"{label}: {bad.size} of {C} columns differ; first column {bad[0]}: "
                           f"gpu ids {gi[bad[0]][:8]} oracle ids {oi[bad[0]][:8]}")
    check_invariants(x, V, C, k, dtype, layout, ld, gv, gi)
