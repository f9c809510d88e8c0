"""GPU parity of the ops on either side of the lm_head matvec: the fused
matvec + argmax, and the int8 embedding table (per-row packer and
dequant-gather).

Argmax: where several rows are within rounding of the largest value, fp32
and fp64 sums may pick different ones, so the check is that the returned
row's oracle value is within the matvec tolerance of the oracle maximum and
the returned value matches that row; rows planted with a clear margin must
be found exactly, and identical winning rows give the lowest index."""
import numpy as np
import pytest

import oracle
import quantized_decode_matvec_amd as qmv
from quantized_decode_matvec_amd import workloads as wl
from tests.gpu_helpers import RTOL, dev, host

pytestmark = pytest.mark.gpu

FMTS = ["int4", "fp4", "int8", "km4", "int4aff"]


def _check_argmax(idx, val, ref):
    ref = np.atleast_2d(ref)
    for b in range(ref.shape[0]):
        scale = np.abs(ref[b]).max()
        i = int(idx[b])
        assert 0 <= i < ref.shape[1]
        assert ref[b, i] >= ref[b].max() - RTOL * scale, (b, i, ref[b, i], ref[b].max())
        assert abs(val[b] - ref[b, i]) <= RTOL * scale


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K,Bs", [(3000, 2048, (1, 2, 3, 4, 8)), (517, 1024, (1, 5)), (65, 96, (1, 2, 8)),
                                    (1, 64, (1, 3))])
def test_matvec_argmax_parity(fmt, N, K, Bs):
    print("argmax", fmt, N, K, Bs, flush=True)
    c = wl.small_dense(fmt, N, K, batch=8, seed=N + K)
    W = c.W.copy()
    x = c.x
    # a clear winner for token 0 and two identical winners for token 1
    if N >= 40:
        W[N // 3] = (np.sign(x[0]) * 0.06).astype(W.dtype)
        W[N - 7] = W[11] = (np.sign(x[1]) * 0.06).astype(W.dtype)
    codes, plane = oracle.pack(fmt, W)
    dc, dp = dev(codes), dev(plane)
    for B in Bs:
        ref = oracle.matvec(fmt, codes, plane, x[:B])
        idx, val = qmv.qmatvec_argmax(fmt, dc, dp, dev(x[:B]))
        idx, val = host(idx), host(val)
        _check_argmax(idx, val, ref)
        if N >= 40:
            assert idx[0] == N // 3
            if B > 1:
                assert idx[1] == 11
        # the fused call runs the plain matvec's kernel for the shape (dot2 or
        # matrix cores), so it gives the same winner and value
        y = host(qmv.qmatvec(fmt, dc, dp, dev(x[:B])))
        assert np.array_equal(idx, np.argmax(y, axis=1))
        assert np.array_equal(val, y[np.arange(B), idx])


def test_lm_head_argmax_full_size_fp4():
    """248320 x 2048 (the lm_head shape), fp4, batch 1 (dot2 matvec), 4 and 8
    (matrix-core matvec)."""
    c = wl.lm_head_km4()
    codes, plane = oracle.pack("fp4", c.W)
    dc, dp = dev(codes), dev(plane)
    for B in (1, 4, 8):
        print("lm_head argmax fp4 B", B, flush=True)
        ref = oracle.matvec("fp4", codes, plane, c.x[:B])
        idx, val = qmv.qmatvec_argmax("fp4", dc, dp, dev(c.x[:B]))
        _check_argmax(host(idx), host(val), ref)


def test_argmax_past_the_first_stretch_of_each_workgroup():
    """270000 rows: more than 64 x 4096, so reduction workgroups take several
    stretches. Token 0 wins at row 263000 (a later stretch of the first
    workgroup), token 1 ties between rows 5 and 269990 (lowest row wins),
    token 2 wins at the last row."""
    N, K = 270000, 64
    rng = np.random.default_rng(31)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    x = rng.standard_normal((3, K)).astype(np.float16)
    W[263000] = (np.sign(x[0]) * 0.06).astype(np.float16)
    W[5] = W[269990] = (np.sign(x[1]) * 0.07).astype(np.float16)
    W[N - 1] = (np.sign(x[2]) * 0.08).astype(np.float16)
    codes, plane = oracle.pack("fp4", W)
    ref = oracle.matvec("fp4", codes, plane, x)
    idx, val = qmv.qmatvec_argmax("fp4", dev(codes), dev(plane), dev(x))
    idx, val = host(idx), host(val)
    _check_argmax(idx, val, ref)
    assert idx.tolist() == [263000, 5, N - 1]


@pytest.mark.parametrize("B", [2, 6])
def test_argmax_replays_in_a_hip_graph(B):
    """Batch 2 (the dot2 matvec zeroes the reduction header) and 6 (the
    matrix-core matvec zeroes it)."""
    import torch
    c = wl.small_dense("km4", 4000, 2048, batch=B, seed=9)
    codes, plane = oracle.pack("km4", c.W)
    dc, dp, xd = dev(codes), dev(plane), dev(c.x)
    idx = torch.empty((B,), dtype=torch.int32, device="cuda")
    val = torch.empty((B,), dtype=torch.float32, device="cuda")
    ws = torch.empty((qmv.qmatvec_argmax_workspace_bytes(4000, B),), dtype=torch.uint8, device="cuda")
    qmv.qmatvec_argmax("km4", dc, dp, xd, idx=idx, val=val, workspace=ws)
    torch.cuda.synchronize()
    ref = (host(idx).copy(), host(val).copy())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qmv.qmatvec_argmax("km4", dc, dp, xd, idx=idx, val=val, workspace=ws)
    for r in range(3):
        idx.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(idx), ref[0]) and np.array_equal(host(val), ref[1]), r
        qmv.qmatvec_argmax("km4", dc, dp, xd, idx=idx, val=val, workspace=ws)
        torch.cuda.synchronize()


@pytest.mark.parametrize("V,H,dtype", [(300, 64, np.float16), (257, 1544, np.float32), (70, 2048, np.float16)])
def test_int8_rows_pack_bit_exact(V, H, dtype):
    rng = np.random.default_rng(V + H)
    W = (rng.standard_normal((V, H)) * 0.03).astype(dtype)
    W[3] = 0
    W[4, 5] = 2.5
    want_q, want_s = oracle.pack_int8_rows(W)
    q, s = qmv.qpack_int8_rows(dev(W))
    assert np.array_equal(host(q), want_q)
    assert np.array_equal(host(s), want_s)


def test_embed_gather_bit_exact_and_out_of_range_ids():
    import torch
    rng = np.random.default_rng(5)
    V, H = 1000, 1536
    W = (rng.standard_normal((V, H)) * 0.03).astype(np.float16)
    q, s = oracle.pack_int8_rows(W)
    dq, ds = dev(q), dev(s)
    ids = np.array([0, 999, 17, 17, 500, 3], np.int32)
    out = qmv.qembed_gather_int8(dq, ds, dev(ids))
    want = oracle.embed_gather_int8(q, s, ids)
    assert np.array_equal(host(out).view(np.uint16), want)
    bad = np.array([5, -1, 1000, 7], np.int32)
    out = qmv.qembed_gather_int8(dq, ds, dev(bad))
    o = host(out).view(np.uint16)
    assert np.array_equal(o, oracle.embed_gather_int8(q, s, bad))   # ids outside [0, V): zero rows
    assert not o[[1, 2]].any()
    empty = qmv.qembed_gather_int8(dq, ds, torch.empty((0,), dtype=torch.int32, device="cuda"))
    assert empty.shape == (0, H)


def test_embed_gather_large_table():
    """262144 x 1536 (the pages' example head/table shape), 8 tokens."""
    rng = np.random.default_rng(6)
    V, H = 262144, 1536
    W = (rng.standard_normal((V, H), dtype=np.float32) * 0.03).astype(np.float16)
    q, s = oracle.pack_int8_rows(W)
    del W
    ids = rng.integers(0, V, size=8).astype(np.int32)
    ids[0], ids[1] = 0, V - 1
    out = qmv.qembed_gather_int8(dev(q), dev(s), dev(ids))
    assert np.array_equal(host(out).view(np.uint16), oracle.embed_gather_int8(q, s, ids))


@pytest.mark.parametrize("N,K,Bs", [(3000, 2048, (1, 2, 4)), (70000, 2048, (1, 2, 3)), (517, 1024, (1,)),
                                    (1, 512, (1, 2)), (700, 4096, (1, 3, 4)), (66001, 1024, (2, 4)),
                                    (1100, 1536, (1, 2, 4)), (800, 3072, (1, 3))])
def test_argmax_km4_tiled_parity(N, K, Bs):
    """The fused argmax from the row-tiled plane (one key per workgroup, then
    the largest): same winner and value as the argmax of qmatvec_km4_tiled's
    y, within tolerance of the oracle maximum, planted winners exact, identical
    winners to the lowest row; one and two tiles per workgroup, the dot2 and
    matrix-core kernels, a ragged last tile."""
    print("argmax km4 tiled", N, K, Bs, flush=True)
    c = wl.small_dense("km4", N, K, batch=4, seed=N + K + 1)
    W = c.W.copy()
    x = c.x
    if N >= 40:
        W[N // 3] = (np.sign(x[0]) * 0.06).astype(W.dtype)
        W[N - 7] = W[11] = (np.sign(x[1]) * 0.06).astype(W.dtype)
    codes, lut = oracle.pack("km4", W)
    dt, dl = qmv.qtile_km4(dev(codes)), dev(lut)
    for B in Bs:
        ref = oracle.matvec("km4", codes, lut, x[:B])
        idx, val = qmv.qmatvec_argmax_km4_tiled(dt, dl, dev(x[:B]))
        idx, val = host(idx), host(val)
        _check_argmax(idx, val, ref)
        if N >= 40:
            assert idx[0] == N // 3
            if B > 1:
                assert idx[1] == 11
        y = host(qmv.qmatvec_km4_tiled(dt, dl, dev(x[:B])))
        assert np.array_equal(idx, np.argmax(y, axis=1))
        assert np.array_equal(val, y[np.arange(B), idx])
