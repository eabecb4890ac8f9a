"""GPU parity of topk_cols_sample (through the C ABI) with the sampling
oracle: the sampled positions and ids must be equal, column by column.

The top-k lists come from the library's own runs on the seeded workloads
(bit-exact with the oracle's, checked here again), and from constructed
lists with ties, special values and every k up to 64.
"""
import math

import numpy as np
import pytest

import oracle
from drafter_vocab_top_amd import workloads as W
from gpu_harness import ODT, OLY, run_oracle, to_device
from topk_checks import bits

pytestmark = pytest.mark.gpu

SETTINGS = [(1.0, 0.95, 1, 0), (1.0, 0.95, 1, 1), (0.7, 0.9, 12345, 2**33 + 5), (2.0, 1.0, 2**63 + 9, 77),
            (0.05, 0.5, 3, 4)]


def gpu_sample(gpu, vals, ids, T, p, seed, offset):
    torch, T_ = gpu
    sid, pos = T_.sample(vals, ids, T, p, seed, offset)
    torch.cuda.synchronize()
    return sid.cpu().numpy(), pos.cpu().numpy()


@pytest.mark.parametrize("n", [2, 3, 4, 5])
def test_sample_after_workload_topk(gpu, n):
    torch, T = gpu
    w = W.config(n)
    dx = to_device(torch, w.x)
    print(f"[parity] sample after {w.name}", flush=True)
    with T.TopkCols(w.V, w.C, w.k, w.dtype, w.layout, w.ld) as h:
        vals, ids = h.run(dx)
        torch.cuda.synchronize()
    ov, oi = run_oracle(w.x, w.V, w.C, w.k, w.dtype, w.layout, w.ld)
    st = np.uint16 if w.dtype == W.BF16 else np.uint32
    assert np.array_equal(ids.cpu().numpy(), oi) and np.array_equal(vals.cpu().numpy().view(st), bits(ov))
    for temp, p, seed, offset in SETTINGS:
        sid, pos = gpu_sample(gpu, vals, ids, temp, p, seed, offset)
        eid, epos = oracle.sample_topk(ov, oi, w.C, w.k, ODT[w.dtype], temp, p, seed, offset)
        assert np.array_equal(pos, epos), (temp, p, seed, offset, np.flatnonzero(pos != epos)[:5])
        assert np.array_equal(sid, eid)


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
@pytest.mark.parametrize("k", [1, 2, 8, 20, 33, 64])
def test_sample_constructed_lists(gpu, dtype, k):
    torch, T = gpu
    C = 5003
    V = 4 * k + 3
    x = W.random_matrix(k * 31 + (dtype == W.F32), V, C, dtype, W.COL, kind="special" if k % 2 else "alphabet")
    ov, oi = oracle.topk_cols(x, V, C, k, ODT[dtype], oracle.COL_CONTIG, V)
    tdt = torch.int16 if dtype == W.BF16 else torch.int32
    vals = torch.from_numpy(ov.view(np.int16 if dtype == W.BF16 else np.int32)).to("cuda")
    ids = torch.from_numpy(oi).to("cuda")
    assert vals.dtype == tdt
    print(f"[parity] sample constructed k={k} {dtype}", flush=True)
    for temp, p, seed, offset in SETTINGS:
        sid, pos = gpu_sample(gpu, vals, ids, temp, p, seed, offset)
        eid, epos = oracle.sample_topk(ov, oi, C, k, ODT[dtype], temp, p, seed, offset)
        assert np.array_equal(pos, epos), (k, temp, p, np.flatnonzero(pos != epos)[:5])
        assert np.array_equal(sid, eid)


def test_sample_mapped_ids_and_non_finite_tops(gpu):
    torch, T = gpu
    C, k = 300, 20
    f = np.random.default_rng(5).standard_normal((C, k)).astype(np.float32) * 3
    f = -np.sort(-f, axis=1)
    f[0, 0], f[1, 0], f[2, :] = np.inf, np.nan, -np.inf
    tokens = np.random.default_rng(6).permutation(248046)[:C * k].astype(np.int32).reshape(C, k)
    vals = torch.from_numpy(f.view(np.int32)).to("cuda")
    ids = torch.from_numpy(tokens).to("cuda")
    sid, pos = gpu_sample(gpu, vals, ids, 1.0, 0.95, 8, 0)
    eid, epos = oracle.sample_topk(f.view(np.uint32), tokens, C, k, oracle.F32, 1.0, 0.95, 8, 0)
    assert np.array_equal(pos, epos) and np.array_equal(sid, eid)
    assert pos[0] == 0 and pos[1] == 0 and pos[2] == 0


def test_sample_refuses_bad_arguments(gpu):
    torch, T = gpu
    vals = torch.zeros((4, 8), dtype=torch.float32, device="cuda")
    ids = torch.zeros((4, 8), dtype=torch.int32, device="cuda")
    out = torch.empty(4, dtype=torch.int32, device="cuda")
    lib = T.load()
    for temp, p in ((0.0, 0.9), (math.inf, 0.9), (math.nan, 0.9), (1.0, 0.0), (1.0, 1.01)):
        rc = lib.topk_cols_sample(vals.data_ptr(), ids.data_ptr(), 4, 8, 1, temp, p, 0, 0, out.data_ptr(), None, None)
        assert rc == T.TOPK_ERR_INVALID_ARG, (temp, p)
    assert lib.topk_cols_sample(vals.data_ptr(), ids.data_ptr(), 4, 65, 1, 1.0, 0.9, 0, 0, out.data_ptr(),
                                None, None) == T.TOPK_ERR_INVALID_ARG
    assert lib.topk_cols_sample(None, ids.data_ptr(), 4, 8, 1, 1.0, 0.9, 0, 0, out.data_ptr(),
                                None, None) == T.TOPK_ERR_INVALID_ARG


def test_graph_replay_of_topk_and_sample(gpu):
    """A row-interleaved top-k followed by the sampler, captured in one graph
    and replayed with alternating inputs (eager copies and host syncs between
    replays): every replay's draws equal the oracle's.  The sampler keeps no
    state, and the row layout's run clears what it shares."""
    torch, T = gpu
    V, C, k = 40009, 70, 16
    temp, p, seed, offset = 1.0, 0.95, 77, 5
    xs = [W.random_matrix(500 + i, V, C, W.BF16, W.ROW, kind="normal") for i in range(2)]
    expect = []
    for x in xs:
        ov, oi = run_oracle(x, V, C, k, W.BF16, W.ROW, C)
        expect.append(oracle.sample_topk(ov, oi, C, k, oracle.BF16, temp, p, seed, offset))
    src = to_device(torch, xs[0])
    staged = [to_device(torch, x) for x in xs]
    with T.TopkCols(V, C, k, W.BF16, W.ROW, C) as h:
        vals = torch.empty((C, k), dtype=torch.int16, device="cuda")
        ids = torch.empty((C, k), dtype=torch.int32, device="cuda")
        sid = torch.empty(C, dtype=torch.int32, device="cuda")
        pos = torch.empty(C, dtype=torch.int32, device="cuda")
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            h.run(src, vals, ids)
            T.sample(vals, ids, temp, p, seed, offset, sid, pos)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            h.run(src, vals, ids, stream=stream)
            T.sample(vals, ids, temp, p, seed, offset, sid, pos, stream=stream)
        for rep in range(6):
            i = rep % 2
            src.copy_(staged[i])
            torch.cuda.synchronize()
            print(f"[parity] graph replay {rep} input {i}", flush=True)
            g.replay()
            torch.cuda.synchronize()
            eid, epos = expect[i]
            assert np.array_equal(pos.cpu().numpy(), epos), rep
            assert np.array_equal(sid.cpu().numpy(), eid), rep
