"""GPU parity of 4-bit k-means rows plus int8 outliers: the packer (outlier
selection, int8 values and the k-means of the zeroed row) bit-exact against
the oracle, and the matvec with the outlier epilogue within the relative-error
bound on the register path (K <= 4096) and the generic path (longer rows,
fp32 x). Rows beyond the packer's K limit use seeded synthetic codes, tables
and outliers."""
import numpy as np
import pytest

import oracle
import quantized_decode_matvec_amd as qmv
from quantized_decode_matvec_amd import workloads as wl
from tests.gpu_helpers import RTOL, dev, host, rel_err

pytestmark = pytest.mark.gpu


def _weights(N, K, seed):
    c = wl.small_dense("km4", N, K, batch=8, seed=seed, outlier_frac=0.01)
    W = c.W.astype(np.float16)
    rng = np.random.default_rng(seed)
    W[rng.integers(0, N, 3 * N), rng.integers(0, K, 3 * N)] *= np.float16(12)
    return W, c.x


def _synthetic(N, K, nout, seed):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    lut = np.sort(rng.standard_normal((N, 16)) * 0.02, axis=1).astype(np.float16).view(np.uint16)
    ocol = np.stack([np.sort(rng.choice(K, nout, replace=False)) for _ in range(N)]).astype(np.uint16)
    oval = rng.integers(-127, 128, size=(N, nout), dtype=np.int8)
    oscale = (np.abs(rng.standard_normal(N)) * 0.002).astype(np.float16).view(np.uint16)
    return codes, lut, ocol.reshape(N, nout), oval, oscale


@pytest.mark.parametrize("N,K,nout", [(37, 96, 1), (50, 512, 8), (65, 1024, 16), (129, 2048, 16), (33, 4096, 64),
                                      (9, 256, 256), (20, 512, 0)])
def test_pack_bit_exact(N, K, nout):
    print("km4o pack", N, K, nout, flush=True)
    W, _ = _weights(N, K, seed=N + K)
    W[0] = 0
    W[1, [3, 9, 17]] = np.float16(0.75)          # equal magnitudes
    W[1, [5, 11]] = np.float16(-0.75)
    want = oracle.pack_km4o(W, nout)
    got = qmv.qpack_km4o(dev(W), nout)
    for name, a, b in zip(("codes", "lut", "ocol", "oval", "oscale"), want, got):
        assert np.array_equal(a, host(b)), name


@pytest.mark.parametrize("N,K,nout", [(37, 96, 4), (65, 1024, 16), (129, 2048, 16), (300, 2048, 64),
                                      (33, 4096, 32), (20, 512, 0)])
@pytest.mark.parametrize("B", [1, 2, 3, 4, 8])
def test_matvec_parity(N, K, nout, B):
    print("km4o matvec", N, K, nout, B, flush=True)
    W, x = _weights(N, K, seed=N + nout)
    packed = oracle.pack_km4o(W, nout, max_iter=4)
    want = oracle.matvec_km4o(*packed, x[:B])
    y = host(qmv.qmatvec_km4o(*[dev(a) for a in packed], dev(x[:B])))
    assert rel_err(y, want) <= RTOL


@pytest.mark.parametrize("N,K,nout", [(40, 8192, 100), (17, 6144, 256)])
@pytest.mark.parametrize("B", [1, 5])
def test_matvec_long_rows_and_fp32_x(N, K, nout, B):
    packed = _synthetic(N, K, nout, seed=K + B)
    x = np.random.default_rng(B).standard_normal((B, K))
    for xs in (x.astype(np.float16), x.astype(np.float32)):
        want = oracle.matvec_km4o(*packed, xs)
        y = host(qmv.qmatvec_km4o(*[dev(a) for a in packed], dev(xs)))
        assert rel_err(y, want) <= RTOL


def test_matvec_unit_vectors_pick_columns():
    """A unit vector returns the column: table value plus outlier, rounded
    once to fp32."""
    W, _ = _weights(64, 2048, seed=3)
    packed = oracle.pack_km4o(W, 16)
    ks = sorted(set([0, 1, 2047] + [int(c) for c in packed[2][5][:3]]))
    x = np.zeros((len(ks), 2048), np.float16)
    for i, k in enumerate(ks):
        x[i, k] = 1.0
    want = oracle.matvec_km4o(*packed, x).astype(np.float32)
    y = host(qmv.qmatvec_km4o(*[dev(a) for a in packed], dev(x)))
    assert np.array_equal(y, want)


def test_gpu_pack_then_gpu_matvec_end_to_end():
    W, x = _weights(500, 2048, seed=8)
    packed = qmv.qpack_km4o(dev(W), 16)
    y = host(qmv.qmatvec_km4o(*packed, dev(x[:2])))
    want = oracle.matvec_km4o(*oracle.pack_km4o(W, 16), x[:2])
    assert rel_err(y, want) <= RTOL


@pytest.mark.parametrize("N,K,nout,B", [(1037, 2048, 16, 1), (1037, 2048, 16, 2), (3000, 1024, 5, 4),
                                        (700, 512, 40, 1), (66001, 2048, 16, 1), (100, 4096, 0, 3),
                                        (257, 2048, 1, 2), (900, 1536, 16, 1), (500, 2560, 20, 2),
                                        (800, 1024, 40, 3), (66001, 2048, 16, 4)])
def test_km4o_tiled_matches_oracle(N, K, nout, B):
    """The outlier format from the row-tiled codes: the 16 lanes that sum a
    row take its outliers (one each, more past 16)."""
    print("km4o tiled", N, K, nout, B, flush=True)
    c = wl.small_dense("km4", N, K, batch=4, seed=N + nout)
    packed = oracle.pack_km4o(c.W, nout, max_iter=4)
    want = oracle.matvec_km4o(*packed, c.x[:B])
    codes, lut, ocol, oval, oscale = (dev(a) for a in packed)
    y = host(qmv.qmatvec_km4o_tiled(qmv.qtile_km4(codes), lut, ocol, oval, oscale, dev(c.x[:B])))
    assert rel_err(y, want) <= RTOL
