"""Batch 2-8 matvec on matrices short of the tall shape with long rows, the
shapes that take the kernel with x staged once per workgroup in LDS (int4,
fp4, int8; rows of whole 64-chunk strides: 4-bit K = 2048, 4096, 8192, int8
K = 1024, 2048, 4096; at most 64 KiB of staged x): full output against the
oracle, row counts that leave a partial last workgroup, a single row, and the
batch widths between the compiled ones (B = 3 runs the B = 4 kernel with a
zero row, B = 5-7 the B = 8 one; at K = 2048 B = 5-8 stays on this kernel up
to 8192 rows instead of the matrix cores). The fused argmax on the same kernel zeroes
its reduction header there; its result must equal the argmax of the matvec."""
import numpy as np
import pytest

import oracle
import quantized_decode_matvec_amd as qmv
from quantized_decode_matvec_amd import workloads as wl
from tests.gpu_helpers import RTOL, dev, host, rel_err

pytestmark = pytest.mark.gpu

CASES = [("int4", 4097, 4096), ("fp4", 4097, 4096), ("int4", 1, 4096), ("fp4", 2051, 8192), ("int4", 2051, 8192),
         ("int8", 4097, 2048), ("int8", 2051, 4096), ("int8", 3, 1024), ("fp4", 4101, 2048), ("int4", 4101, 2048),
         ("fp4", 8191, 2048), ("int8", 8185, 2048)]


@pytest.mark.parametrize("fmt,N,K", CASES)
def test_staged_x_matvec_full_output(fmt, N, K):
    print("xstage", fmt, N, K, flush=True)
    c = wl.small_dense(fmt, N, K, batch=8, seed=N + K, outlier_frac=0.01)
    gc, gp = qmv.qpack(fmt, dev(c.W))
    codes, plane = host(gc), host(gp)
    for B in (2, 3, 4, 5, 7, 8):
        y = host(qmv.qmatvec(fmt, gc, gp, dev(c.x[:B])))
        err = rel_err(y, oracle.matvec(fmt, codes, plane, c.x[:B]))
        assert err <= RTOL, (fmt, N, K, B, err)


@pytest.mark.parametrize("fmt", ["int4", "fp4", "int8"])
def test_staged_x_argmax_equals_matvec_argmax(fmt):
    N, K = 3001, 2048 if fmt == "int8" else 4096
    c = wl.small_dense(fmt, N, K, batch=8, seed=5, outlier_frac=0.01)
    gc, gp = qmv.qpack(fmt, dev(c.W))
    for B in (2, 4):
        x = dev(c.x[:B])
        y = host(qmv.qmatvec(fmt, gc, gp, x))
        idx, val = qmv.qmatvec_argmax(fmt, gc, gp, x)
        want = np.argmax(y, axis=1)
        assert np.array_equal(host(idx), want), (fmt, B)
        assert np.array_equal(host(val), y[np.arange(B), want]), (fmt, B)
