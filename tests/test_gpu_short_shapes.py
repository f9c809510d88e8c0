"""Batch 2-8 matvec on short matrices (2048 to 8192 rows), full output against
the oracle, in every format. These shapes take the dot-product kernel at one
iteration per wave with 1, 2 or 4 rows per wave, or the matrix-core kernel,
depending on rows, batch and K; K = 2048 fills the lanes exactly and K = 1056
leaves a ragged last chunk per row."""
import numpy as np
import pytest

import oracle
import quantized_decode_matvec_amd as qmv
from quantized_decode_matvec_amd import workloads as wl
from tests.gpu_helpers import RTOL, bits_equal, dev, host, rel_err

pytestmark = pytest.mark.gpu

FORMATS = ["int4", "fp4", "int8", "km4", "int4aff", "int8km"]


@pytest.mark.parametrize("K", [2048, 1056])
@pytest.mark.parametrize("fmt", FORMATS)
def test_short_matrices_batched_full_output(fmt, K):
    for N in (2048, 3000, 4096, 8192):
        if fmt == "int8km" and N % 32:
            N = 3008                                   # int8 k-means tables cover groups of 32 rows
        c = wl.small_dense(fmt, N, K, batch=8, seed=N + K, outlier_frac=0.01)
        codes, plane = oracle.pack(fmt, c.W)
        gc, gp = qmv.qpack(fmt, dev(c.W))
        assert np.array_equal(host(gc), codes), (fmt, N, K)
        assert bits_equal(host(gp), plane), (fmt, N, K)
        for B in (2, 4, 5, 8):
            y = host(qmv.qmatvec(fmt, gc, gp, dev(c.x[:B])))
            err = rel_err(y, oracle.matvec(fmt, codes, plane, c.x[:B]))
            assert err <= RTOL, (fmt, N, K, B, err)
