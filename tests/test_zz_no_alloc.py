"""GPU tests of topk_cols_run_noalloc, the entry point that allocates
nothing: through the C ABI, its output is compared with the handle entry
point's (topk_cols_create + topk_cols_run) and with the CPU oracle, bit-exact,
on calls in a row whose shapes shrink, change layout, repeat without a host
synchronization, and replay from a captured graph."""
import ctypes

import numpy as np
import pytest

from drafter_vocab_top_amd import workloads as W
from gpu_harness import run_oracle, to_device
from topk_checks import bits

pytestmark = pytest.mark.gpu


def host(v, d, dtype, C, k):
    st = np.uint16 if dtype == W.BF16 else np.uint32
    return v.cpu().numpy().view(st).reshape(C, k), d.cpu().numpy().reshape(C, k)


def noalloc(gpu, dx, w, values=None, ids=None, stream=None):
    torch, T = gpu
    return T.run_noalloc(dx, w.V, w.C, w.k, w.dtype, w.layout, w.ld, values=values, ids=ids, stream=stream)


def with_handle(gpu, dx, w):
    torch, T = gpu
    with T.TopkCols(w.V, w.C, w.k, w.dtype, w.layout, w.ld) as h:
        v, i = h.run(dx)
        torch.cuda.synchronize()
    return host(v, i, w.dtype, w.C, w.k)


def check_same(gpu, dx, w, got):
    gv, gi = got
    hv, hi = with_handle(gpu, dx, w)
    assert np.array_equal(gi, hi) and np.array_equal(bits(gv), bits(hv)), f"{w.name}: differs from the handle's run"
    ov, oi = run_oracle(w.x, w.V, w.C, w.k, w.dtype, w.layout, w.ld)
    assert np.array_equal(gi, oi) and np.array_equal(bits(gv), bits(ov)), f"{w.name}: differs from the oracle"


def small(seed, V, C, k, dtype, layout):
    x = W.random_matrix(seed, V, C, dtype, layout, kind="normal")
    ld = V if layout == W.COL else C
    return W.Workload(name=f"V={V} C={C} k={k} {dtype} {layout}", V=V, C=C, k=k, dtype=dtype, layout=layout,
                      ld=ld, x=x, seed=seed)


@pytest.mark.parametrize("first,second", [(3, 2), (4, 1), (5, None)])
def test_two_calls_second_smaller(gpu, first, second):
    torch, T = gpu
    wa = W.config(first)
    wb = W.config(second) if second else small(55, 60013, 130, 16, W.BF16, W.ROW)
    for w in (wa, wb):
        dx = to_device(torch, w.x)
        print(f"[noalloc] {w.name}", flush=True)
        v, i = noalloc(gpu, dx, w)
        torch.cuda.synchronize()
        check_same(gpu, dx, w, host(v, i, w.dtype, w.C, w.k))
    assert T.load().topk_cols_check(None) == T.TOPK_OK


def test_layouts_and_shapes_alternate_without_sync(gpu):
    """Column and row calls of several shapes, 60 in a row with no host
    synchronization: each call finds the shared array as the last left it."""
    torch, T = gpu
    ws = [W.config(2), small(71, 60013, 130, 16, W.BF16, W.ROW), W.config(1),
          small(72, 20011, 9, 64, W.F32, W.COL), small(73, 4099, 448, 8, W.F32, W.ROW)]
    dxs = [to_device(torch, w.x) for w in ws]
    refs = [run_oracle(w.x, w.V, w.C, w.k, w.dtype, w.layout, w.ld) for w in ws]
    print("[noalloc] 60 calls of alternating shapes and layouts", flush=True)
    outs = []
    for rep in range(60):
        j = (rep * 3) % len(ws)
        outs.append((j,) + noalloc(gpu, dxs[j], ws[j]))
    torch.cuda.synchronize()
    for n, (j, v, i) in enumerate(outs):
        w = ws[j]
        gv, gi = host(v, i, w.dtype, w.C, w.k)
        ov, oi = refs[j]
        assert np.array_equal(gi, oi) and np.array_equal(bits(gv), bits(ov)), f"call {n}: {w.name}"
    assert T.load().topk_cols_check(None) == T.TOPK_OK


@pytest.mark.parametrize("n", [2, 5])
def test_graph_replay(gpu, n):
    """A captured no-allocation call replays correctly with alternating
    inputs and eager work between replays."""
    torch, T = gpu
    w0 = W.config(n)
    xs = [w0.x, W.config(n, seed=5000 + n).x]
    ref = [run_oracle(x, w0.V, w0.C, w0.k, w0.dtype, w0.layout, w0.ld) for x in xs]
    src = to_device(torch, xs[0])
    staged = [to_device(torch, x) for x in xs]
    vals = torch.empty((w0.C, w0.k), dtype=src.dtype, device="cuda")
    ids = torch.empty((w0.C, w0.k), dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        noalloc(gpu, src, w0, vals, ids, stream)      # first call on the device outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        noalloc(gpu, src, w0, vals, ids, stream)
    for rep in range(6):
        i = rep % 2
        src.copy_(staged[i])
        torch.cuda.synchronize()
        print(f"[noalloc] graph replay {w0.name} {rep}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        gv, gi = host(vals, ids, w0.dtype, w0.C, w0.k)
        ov, oi = ref[i]
        assert np.array_equal(gi, oi) and np.array_equal(bits(gv), bits(ov)), f"replay {rep}"
    assert T.load().topk_cols_check(None) == T.TOPK_OK


def test_sizes_beyond_the_array_are_refused(gpu):
    torch, T = gpu
    lib = T.load()
    buf = torch.zeros(64, dtype=torch.int32, device="cuda")
    p = buf.data_ptr()
    # more columns than the array's fixed ticket and bound regions hold
    assert lib.topk_cols_run_noalloc(1000, 4097, 8, 0, 0, 1000, p, p, p, None) == T.TOPK_ERR_UNSUPPORTED
    # lists larger than the array (row layout, 4,096 columns, k = 64)
    assert lib.topk_cols_run_noalloc(248046, 4096, 64, 0, 1, 4096, p, p, p, None) == T.TOPK_ERR_UNSUPPORTED
    torch.cuda.synchronize()
