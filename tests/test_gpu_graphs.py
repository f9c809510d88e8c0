"""Every dense entry point can be captured in a HIP graph: the library
allocates nothing, never synchronizes and records no memset. Each graph
replays several times with eager work between the replays, and every replay
equals the eager result bit for bit (the batch-1 kernels, the tall batch-1
shape, the matrix-core batched kernels, the outlier epilogue and the fused
argmax)."""
import numpy as np
import pytest

import quantized_decode_matvec_amd as qmv
from quantized_decode_matvec_amd import workloads as wl
from tests.gpu_helpers import dev, host

pytestmark = pytest.mark.gpu

FMTS = ["int4", "fp4", "int8", "km4", "int4aff", "int8km", "km4o"]


def _packed(fmt, W):
    if fmt == "km4o":
        return qmv.qpack_km4o(W, 8)
    return qmv.qpack(fmt, W)


def _call(fmt, packed, x, y):
    if fmt == "km4o":
        return qmv.qmatvec_km4o(*packed, x, y=y)
    return qmv.qmatvec(fmt, packed[0], packed[1], x, y=y)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K,B", [(4096, 1024, 1), (40000, 512, 1), (2048, 2048, 8)])
def test_matvec_graph_replays_equal_eager(fmt, N, K, B):
    import torch
    print("graph", fmt, N, K, B, flush=True)
    c = wl.small_dense("km4", N, K, batch=B, seed=N + B)
    W = dev(c.W)
    packed = _packed(fmt, W)
    xs = [dev(np.random.default_rng(i).standard_normal((B, K)).astype(np.float16)) for i in range(3)]
    eager = [host(_call(fmt, packed, x, None)) for x in xs]
    ys = [torch.empty((B, N), dtype=torch.float32, device="cuda") for _ in xs]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _call(fmt, packed, xs[0], ys[0])   # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for x, y in zip(xs, ys):
                _call(fmt, packed, x, y)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        for y in ys:
            y.fill_(float("nan"))
        junk = _call(fmt, packed, xs[(rep + 1) % 3], None)   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for y, want in zip(ys, eager):
            assert np.array_equal(host(y), want), (fmt, rep)
        assert np.array_equal(host(junk), eager[(rep + 1) % 3])


@pytest.mark.parametrize("fmt", ["km4", "int8km", "int4aff"])
def test_argmax_graph_replays_equal_eager(fmt):
    import torch
    N, K, B = 40000 if fmt != "int8km" else 40000 - 40000 % 32, 1024, 2
    c = wl.small_dense("km4", N, K, batch=B, seed=5)
    codes, plane = qmv.qpack(fmt, dev(c.W))
    x = dev(c.x)
    i0, v0 = qmv.qmatvec_argmax(fmt, codes, plane, x)
    want = (host(i0), host(v0))
    ws = torch.empty((qmv.qmatvec_argmax_workspace_bytes(N, B),), dtype=torch.uint8, device="cuda")
    idx = torch.empty((B,), dtype=torch.int32, device="cuda")
    val = torch.empty((B,), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        qmv.qmatvec_argmax(fmt, codes, plane, x, idx=idx, val=val, workspace=ws)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            qmv.qmatvec_argmax(fmt, codes, plane, x, idx=idx, val=val, workspace=ws)
    for rep in range(3):
        idx.fill_(-1)
        val.fill_(float("nan"))
        ws.fill_(255)    # the partial keys must be rewritten, not read stale
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(idx), want[0]) and np.array_equal(host(val), want[1])


@pytest.mark.parametrize("fmt", ["km4", "fp4", "int8km"])
@pytest.mark.parametrize("B", [1, 8])
def test_prepared_call_equals_matvec(fmt, B):
    """qmatvec_call checks once and relaunches the same matvec: each call equals
    qmatvec on the same inputs bit for bit, also after x is rewritten in place
    and when called on another stream."""
    import torch
    N, K = 8192, 2048
    print("prepared", fmt, B, flush=True)
    c = wl.small_dense("km4", N, K, batch=B, seed=7 + B)
    codes, plane = qmv.qpack(fmt, dev(c.W))
    x = dev(c.x[:B])
    y = torch.empty((B, N), dtype=torch.float32, device="cuda")
    call = qmv.qmatvec_call(fmt, codes, plane, x, y=y)
    for i in range(3):
        x.copy_(dev(np.random.default_rng(i).standard_normal((B, K)).astype(np.float16)))
        want = host(qmv.qmatvec(fmt, codes, plane, x))
        y.fill_(float("nan"))
        assert call() is y
        assert np.array_equal(host(y), want), (fmt, B, i)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    y.fill_(float("nan"))
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        call()
    torch.cuda.synchronize()
    assert np.array_equal(host(y), want)
