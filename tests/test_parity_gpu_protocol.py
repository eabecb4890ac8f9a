"""GPU tests of the column-contiguous layout's cross-workgroup protocol,
through the C ABI, against the CPU oracle (bit-exact).

Each column is merged in the same launch by the workgroup that takes the
column's last ticket; the others publish their lists into zeroed slots that
the merger clears again.  A run therefore leaves the workspace as it found
it, which is what makes a captured run replay correctly.  The merger's wait
is bounded; when it gives up, topk_cols_check reports it.  The error path is
forced from the host (topk_cols_debug_fail_waits): the merger's wait gives
up after a few re-reads and every kernel still ends normally.
"""
import ctypes

import numpy as np
import pytest

from drafter_vocab_top_amd import workloads as W
from gpu_harness import run_oracle, to_device
from topk_checks import bits, check_invariants

pytestmark = pytest.mark.gpu

MARK_ID = -7


def host(v, d, dtype, C, k):
    st = np.uint16 if dtype == W.BF16 else np.uint32
    return v.cpu().numpy().view(st).reshape(C, k), d.cpu().numpy().reshape(C, k)


def same(gv, gi, ov, oi):
    return np.array_equal(gi, oi) and np.array_equal(bits(gv), bits(ov))


@pytest.mark.parametrize("n", [3, 4])
def test_plain_create_entry_point_full_size(gpu, n):
    """topk_cols_create itself (the entry point callers use), called through
    ctypes with the workload's own arguments."""
    torch, T = gpu
    lib = T.load()
    w = W.config(n)
    dx = to_device(torch, w.x)
    h = ctypes.c_void_p()
    rc = lib.topk_cols_create(ctypes.byref(h), w.V, w.C, w.k, T.DTYPES[w.dtype], T.LAYOUTS[w.layout], w.ld)
    assert rc == T.TOPK_OK
    try:
        vals = torch.empty((w.C, w.k), dtype=dx.dtype, device="cuda")
        ids = torch.empty((w.C, w.k), dtype=torch.int32, device="cuda")
        print(f"[protocol] topk_cols_create + run {w.name}", flush=True)
        for _ in range(3):
            assert lib.topk_cols_run(h, dx.data_ptr(), vals.data_ptr(), ids.data_ptr(),
                                     torch.cuda.current_stream().cuda_stream) == T.TOPK_OK
        assert lib.topk_cols_check(h) == T.TOPK_OK
        gv, gi = host(vals, ids, w.dtype, w.C, w.k)
    finally:
        assert lib.topk_cols_destroy(h) == T.TOPK_OK
    ov, oi = run_oracle(w.x, w.V, w.C, w.k, w.dtype, w.layout, w.ld)
    assert same(gv, gi, ov, oi)
    check_invariants(w.x, w.V, w.C, w.k, w.dtype, w.layout, w.ld, gv, gi)


@pytest.mark.parametrize("n", [2, 1])
def test_graph_replay_column_layout(gpu, n):
    """A captured column-contiguous run replays correctly: replays alternate
    two inputs, with eager work and host syncs between them, and every
    replay is checked; then an eager run on the same handle."""
    torch, T = gpu
    w0 = W.config(n)
    xs = [w0.x, W.config(n, seed=4000 + n).x]
    ref = [run_oracle(x, w0.V, w0.C, w0.k, w0.dtype, w0.layout, w0.ld) for x in xs]
    src = to_device(torch, xs[0])
    staged = [to_device(torch, x) for x in xs]
    with T.TopkCols(w0.V, w0.C, w0.k, w0.dtype, w0.layout, w0.ld) as h:
        vals = torch.empty(w0.C * w0.k, dtype=src.dtype, device="cuda")
        ids = torch.empty(w0.C * w0.k, dtype=torch.int32, device="cuda")
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            h.run(src, vals, ids)          # warm the handle outside the capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            h.run(src, vals, ids, stream=stream)
        for rep in range(8):
            i = rep % 2
            src.copy_(staged[i])           # eager work between replays
            torch.cuda.synchronize()
            print(f"[protocol] graph replay {w0.name} {rep} input {i}", flush=True)
            g.replay()
            torch.cuda.synchronize()
            gv, gi = host(vals, ids, w0.dtype, w0.C, w0.k)
            assert same(gv, gi, *ref[i]), f"replay {rep}"
        src.copy_(staged[1])
        h.run(src, vals, ids)
        assert h.check() == T.TOPK_OK
        gv, gi = host(vals, ids, w0.dtype, w0.C, w0.k)
        assert same(gv, gi, *ref[1])


def test_graph_replay_many_back_to_back(gpu):
    """Twenty replays of one captured run without a host sync between them,
    then the output of the last one."""
    torch, T = gpu
    w = W.config(3)
    ov, oi = run_oracle(w.x, w.V, w.C, w.k, w.dtype, w.layout, w.ld)
    src = to_device(torch, w.x)
    with T.TopkCols(w.V, w.C, w.k, w.dtype, w.layout, w.ld) as h:
        vals = torch.empty(w.C * w.k, dtype=src.dtype, device="cuda")
        ids = torch.empty(w.C * w.k, dtype=torch.int32, device="cuda")
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            h.run(src, vals, ids)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            h.run(src, vals, ids, stream=stream)
        print("[protocol] 20 replays back to back", flush=True)
        for _ in range(20):
            g.replay()
        torch.cuda.synchronize()
        assert h.check() == T.TOPK_OK
        gv, gi = host(vals, ids, w.dtype, w.C, w.k)
    assert same(gv, gi, ov, oi)


@pytest.mark.parametrize("n,segments", [(2, 0), (3, 0), (4, 0), (2, 64)])
def test_forced_wait_failure_is_reported(gpu, n, segments):
    """With the merger's wait forced to give up, no output is written, the
    check reports TOPK_ERR_TIMEOUT and resets the workspace, and the next
    runs are exact again."""
    torch, T = gpu
    w = W.config(n)
    ov, oi = run_oracle(w.x, w.V, w.C, w.k, w.dtype, w.layout, w.ld)
    dx = to_device(torch, w.x)
    with T.TopkCols(w.V, w.C, w.k, w.dtype, w.layout, w.ld, segments=segments) as h:
        assert h.query()["segments"] > 1
        vals = torch.zeros((w.C, w.k), dtype=dx.dtype, device="cuda")
        ids = torch.full((w.C, w.k), MARK_ID, dtype=torch.int32, device="cuda")
        assert h.check() == T.TOPK_OK
        h.debug_fail_waits(True)
        print(f"[protocol] forced wait failure {w.name} segments={segments}", flush=True)
        h.run(dx, vals, ids)
        torch.cuda.synchronize()
        assert (ids.cpu().numpy() == MARK_ID).all()      # the mergers wrote nothing
        assert h.check() == T.TOPK_ERR_TIMEOUT
        assert h.check() == T.TOPK_OK                    # the check cleared it
        h.debug_fail_waits(False)
        for _ in range(3):
            h.run(dx, vals, ids)
        assert h.check() == T.TOPK_OK
        gv, gi = host(vals, ids, w.dtype, w.C, w.k)
    assert same(gv, gi, ov, oi)


def test_two_handles_interleaved_on_one_stream(gpu):
    """Two handles of different shapes used alternately on one stream: each
    keeps its own state."""
    torch, T = gpu
    wa, wb = W.config(2), W.config(4)
    ra = run_oracle(wa.x, wa.V, wa.C, wa.k, wa.dtype, wa.layout, wa.ld)
    rb = run_oracle(wb.x, wb.V, wb.C, wb.k, wb.dtype, wb.layout, wb.ld)
    da, db = to_device(torch, wa.x), to_device(torch, wb.x)
    with T.TopkCols(wa.V, wa.C, wa.k, wa.dtype, wa.layout, wa.ld) as ha, \
            T.TopkCols(wb.V, wb.C, wb.k, wb.dtype, wb.layout, wb.ld) as hb:
        outs = []
        print("[protocol] two handles interleaved", flush=True)
        for _ in range(50):
            outs.append(("a",) + ha.run(da))
            outs.append(("b",) + hb.run(db))
        torch.cuda.synchronize()
        for which, v, d in outs:
            w, r = (wa, ra) if which == "a" else (wb, rb)
            assert same(*host(v, d, w.dtype, w.C, w.k), *r)
