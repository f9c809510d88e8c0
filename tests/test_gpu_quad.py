"""The 4x4x4-block matrix-core kernels: km4 at batch 3 to 8 (K of 512, 1024,
2048 or 4096) and int4 / affine int4 at batch 2 to 8 (K of 512, 1024, 2048,
and 4096 for int4); one token quad up to batch 4, two above. They take
matrices from 8192 rows at batch 3-8 (affine int4 from 4096 rows at batch
5-8) and at batch 2 from 16384 (int4) or 32768 rows (affine int4); rows per
wave grow with the matrix (one row quad per wave below 32768 rows, two above,
four for km4 at batch <= 4 from 196608 rows; scale formats at batch <= 4 take
two from 65536). Every launch branch runs on a ragged matrix (rows not a multiple of the
wave's rows). The GPU packs and multiplies the whole matrix; the oracle packs
and multiplies sampled rows, the last 16 rows of the ragged tail included.
The 248320 x 2048 km4 head at batch 4 is compared on every row in
test_gpu_configs.py."""
import numpy as np
import pytest

import oracle
import quantized_decode_matvec_amd as qmv
from quantized_decode_matvec_amd import workloads as wl
from tests.gpu_helpers import RTOL, dev, host, rel_err, sample_rows

pytestmark = pytest.mark.gpu

CASES = [
    (8192 + 7, 1024),      # one quad, two chunks per lane
    (32768 + 9, 2048),     # two quads, four chunks
    (16384 + 13, 512),     # one quad, one chunk per lane
    (16384 + 2, 2048),     # one quad, four chunks
    (16384 + 1, 4096),     # one quad, eight chunks
    (196608 + 37, 512),    # four quads, one chunk
    (196608 + 6, 1024),    # four quads, two chunks
    (196608 + 3, 4096),    # two quads, eight chunks
]


@pytest.mark.parametrize("N,K", CASES)
def test_km4_quad_kernel_on_sampled_rows(N, K):
    c = wl.small_dense("km4", N, K, batch=8, seed=N + K)
    print("km4 quad", N, K, flush=True)
    codes, lut = qmv.qpack_km4(dev(c.W))
    rows = np.unique(np.concatenate([sample_rows(N, n=64, seed=K), np.arange(N - 16, N)]))
    oc, ol = oracle.pack_km4(c.W[rows])
    for B in (3, 4, 5, 8):
        y = host(qmv.qmatvec_km4(codes, lut, dev(c.x[:B])))
        assert y.shape == (B, N)
        assert np.all(np.isfinite(y))
        assert rel_err(y[:, rows], oracle.matvec("km4", oc, ol, c.x[:B])) <= RTOL, B


@pytest.mark.parametrize("N,K", [(16384 + 13, 2048), (32768 + 5, 1024), (196608 + 3, 512), (65536 + 9, 2048)])
def test_km4_quad_argmax_matches_its_matvec(N, K):
    """The fused argmax runs the same matvec kernel, so its index is the
    argmax of the plain call's output and its value that output's maximum;
    two identical planted rows tie and the lower wins. One, two and four row
    quads per wave, one and two token quads."""
    print("km4 quad argmax", N, K, flush=True)
    c = wl.small_dense("km4", N, K, batch=8, seed=5)
    W = c.W.copy()
    W[N - 3] = W[7] = (np.sign(c.x[0]) * 0.06).astype(W.dtype)
    codes, lut = qmv.qpack_km4(dev(W))
    for B in (3, 4, 5, 8):
        x = dev(c.x[:B])
        y = host(qmv.qmatvec_km4(codes, lut, x))
        idx, val = qmv.qmatvec_argmax("km4", codes, lut, x)
        assert host(idx).tolist() == np.argmax(y, axis=1).tolist()
        assert np.array_equal(host(val), y.max(axis=1))
        assert host(idx)[0] == 7


SCALED_CASES = [
    ("int4", 8192 + 5, 2048),       # one row quad
    ("int4", 65536 + 3, 512),       # two row quads at every batch
    ("int4aff", 4096 + 3, 1024),    # batch 5-8 only (batch 2-4 keep the dot2 kernels)
    ("int4", 16384 + 13, 512),
    ("int4", 16384 + 2, 2048),
    ("int4", 16384 + 1, 4096),
    ("int4aff", 16384 + 5, 512),
    ("int4aff", 16384 + 3, 2048),
    ("int4aff", 32768 + 7, 1024),   # batch 2 takes the 4x4x4 kernel from 32768 rows
]


@pytest.mark.parametrize("fmt,N,K", SCALED_CASES)
def test_scaled_quad_kernel_on_sampled_rows(fmt, N, K):
    c = wl.small_dense(fmt, N, K, batch=8, seed=N + K, outlier_frac=0.01)
    print("scaled quad", fmt, N, K, flush=True)
    codes, plane = qmv.qpack(fmt, dev(c.W))
    rows = np.unique(np.concatenate([sample_rows(N, n=64, seed=K), np.arange(N - 16, N)]))
    oc, op = oracle.pack(fmt, c.W[rows])
    for B in (2, 3, 4, 5, 8):
        y = host(qmv.qmatvec(fmt, codes, plane, dev(c.x[:B])))
        assert y.shape == (B, N)
        assert np.all(np.isfinite(y))
        assert rel_err(y[:, rows], oracle.matvec(fmt, oc, op, c.x[:B])) <= RTOL, B


@pytest.mark.parametrize("fmt", ["int4", "int4aff"])
def test_scaled_quad_argmax_matches_its_matvec(fmt):
    N, K = 16384 + 13, 2048
    c = wl.small_dense(fmt, N, K, batch=8, seed=7)
    codes, plane = qmv.qpack(fmt, dev(c.W))
    for B in (3, 8):
        x = dev(c.x[:B])
        y = host(qmv.qmatvec(fmt, codes, plane, x))
        idx, val = qmv.qmatvec_argmax(fmt, codes, plane, x)
        assert host(idx).tolist() == np.argmax(y, axis=1).tolist()
        assert np.array_equal(host(val), y.max(axis=1))
