"""GPU parity of the int8 k-means format (one 256-entry fp16 table per group
of 32 rows): the packer bit-exact against the oracle, dequant exact, the
matvec within the relative-error bound at every kernel shape and batch
width, the fused argmax, and sampled groups of the full lm_head shape.

Matvec cases beyond the packer's K limit (2048) use seeded random indices
and random ascending tables: the matvec reads any valid codes and tables."""
import numpy as np
import pytest

import oracle
import quantized_decode_matvec_amd as qmv
from quantized_decode_matvec_amd import workloads as wl
from tests.gpu_helpers import RTOL, dev, host, rel_err

pytestmark = pytest.mark.gpu


def _weights(N, K, seed, outliers=True):
    c = wl.small_dense("km4", N, K, batch=8, seed=seed, outlier_frac=0.01 if outliers else 0.0)
    return c.W.astype(np.float16), c.x


def _random_codes(N, K, seed):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    lut = np.sort(rng.standard_normal((N // 32, 256)) * 0.02, axis=1).astype(np.float16).view(np.uint16)
    return codes, lut


@pytest.mark.parametrize("N,K", [(32, 32), (32, 96), (64, 512), (96, 1024), (32, 2048)])
def test_pack_bit_exact(N, K):
    print("int8km pack", N, K, flush=True)
    W, _ = _weights(N, K, seed=N + K)
    W[0] = 0
    W[1, ::3] = np.float16(-0.0)
    want = oracle.pack_int8km(W)
    got = qmv.qpack_int8km(dev(W))
    assert np.array_equal(want[1], host(got[1]))
    assert np.array_equal(want[0], host(got[0]))


@pytest.mark.parametrize("max_iter", [1, 2, 7, 60])
def test_pack_iterations_bit_exact(max_iter):
    W, _ = _weights(64, 256, seed=5)
    want = oracle.pack_int8km(W, max_iter=max_iter)
    got = qmv.qpack_int8km(dev(W), max_iter=max_iter)
    assert np.array_equal(want[1], host(got[1]))
    assert np.array_equal(want[0], host(got[0]))


def test_pack_few_distinct_and_hand_worked_groups():
    """Groups with <= 256 distinct values (exact tables), one with exactly 257,
    and the hand-worked fixed point of the oracle pins (even integers)."""
    rng = np.random.default_rng(7)
    vals = np.unique(rng.standard_normal(2000).astype(np.float16))
    W = np.empty((128, 64), np.float16)
    W[:32] = rng.choice(vals[:256], size=(32, 64))
    W[32:64] = rng.choice(vals[:3], size=(32, 64))
    g = rng.choice(vals[:257], size=(32, 64))
    g.reshape(-1)[:257] = vals[:257]
    W[64:96] = g
    ev = np.repeat(np.arange(0, 1024, 2), 4)
    W[96:] = ev[rng.permutation(ev.size)].reshape(32, 64)
    want = oracle.pack_int8km(W)
    got = qmv.qpack_int8km(dev(W))
    assert np.array_equal(want[1], host(got[1]))
    assert np.array_equal(want[0], host(got[0]))


def test_dequant_exact():
    W, _ = _weights(96, 512, seed=9)
    codes, lut = oracle.pack_int8km(W)
    D = host(qmv.qdequant("int8km", dev(codes), dev(lut)))
    assert np.array_equal(D.astype(np.float64), oracle.dequant("int8km", codes, lut))


SHAPES = [(32, 96), (64, 256), (96, 512), (160, 1024), (64, 2048), (32, 2560), (96, 4096), (32, 6144), (64, 8192)]


@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("B", [1, 2, 3, 4, 8])
def test_matvec_parity(N, K, B):
    print("int8km matvec", N, K, B, flush=True)
    codes, lut = _random_codes(N, K, seed=N + K + B)
    x = np.random.default_rng(B).standard_normal((B, K)).astype(np.float16)
    want = oracle.matvec("int8km", codes, lut, x)
    y = host(qmv.qmatvec("int8km", dev(codes), dev(lut), dev(x)))
    assert rel_err(y, want) <= RTOL


def test_matvec_fp32_x_and_packed_weights():
    W, x = _weights(128, 1024, seed=11)
    codes, lut = oracle.pack_int8km(W)
    for xs in (x[:1].astype(np.float32), x[:5].astype(np.float32), x[:3]):
        want = oracle.matvec("int8km", codes, lut, xs)
        y = host(qmv.qmatvec("int8km", dev(codes), dev(lut), dev(xs)))
        assert rel_err(y, want) <= RTOL


def test_matvec_unit_vectors_pick_columns_exactly():
    codes, lut = _random_codes(64, 2048, seed=12)
    D = oracle.dequant("int8km", codes, lut)
    ks = [0, 1, 15, 16, 1000, 2047]
    x = np.zeros((len(ks), 2048), np.float16)
    for i, k in enumerate(ks):
        x[i, k] = 1.0
    y = host(qmv.qmatvec("int8km", dev(codes), dev(lut), dev(x)))
    for i, k in enumerate(ks):
        assert np.array_equal(y[i].astype(np.float64), D[:, k])


@pytest.mark.parametrize("N,K,Bs", [(3008, 2048, (1, 2, 4, 8)), (64, 96, (1, 3))])
def test_matvec_argmax(N, K, Bs):
    codes, lut = _random_codes(N, K, seed=13)
    rng = np.random.default_rng(14)
    x = rng.standard_normal((8, K)).astype(np.float16)
    # rows 40 and 45 (one group) are identical, largest for token 0
    codes[40] = codes[45] = np.where(x[0] > 0, 255, 0).astype(np.uint8)
    dc, dl = dev(codes), dev(lut)
    for B in Bs:
        ref = oracle.matvec("int8km", codes, lut, x[:B])
        idx, val = qmv.qmatvec_argmax("int8km", dc, dl, dev(x[:B]))
        idx, val = host(idx), host(val)
        assert idx[0] == 40
        for b in range(B):
            scale = np.abs(ref[b]).max()
            assert ref[b, idx[b]] >= ref[b].max() - RTOL * scale
            assert abs(val[b] - ref[b, idx[b]]) <= RTOL * scale


def test_lm_head_shape_sampled_groups():
    """248320 x 2048: the GPU packs every group; sampled groups (first, last,
    random) equal the oracle's bit for bit, and the matvec on sampled rows at
    B = 2, 3, 4 is within the bound."""
    c = wl.lm_head_km4(batch=4)
    W = dev(c.W)
    codes, lut = qmv.qpack_int8km(W)
    del W
    N = c.W.shape[0]
    groups = [0, N // 32 - 1, 1234, 5000]
    for g in groups:
        oc, ol = oracle.pack_int8km(c.W[32 * g:32 * g + 32])
        assert np.array_equal(ol[0], host(lut[g]))
        assert np.array_equal(oc, host(codes[32 * g:32 * g + 32]))
    rows = np.concatenate([np.arange(32 * g, 32 * g + 32) for g in groups])
    hl = host(lut)
    want = oracle.matvec("int8km", host(codes[rows]), np.concatenate([hl[g:g + 1] for g in groups]), c.x)
    for B in (2, 3, 4):   # dot2 at B = 2, the matrix cores at B = 3, 4
        y = host(qmv.qmatvec("int8km", codes, lut, dev(c.x[:B])))
        assert rel_err(y[:, rows], want[:B]) <= RTOL, B


@pytest.mark.parametrize("fmt", ["km4", "int8km"])
def test_pack_heavily_repeated_value_bit_exact(fmt):
    """Half of every row is one value: repeated starting entries, empty
    clusters that keep their value (both k-means packers)."""
    rng = np.random.default_rng(60)
    W = (rng.standard_normal((64, 512)) * 0.3).astype(np.float16)
    W[:, ::2] = np.float16(0.5)
    want = oracle.pack(fmt, W)
    got = qmv.qpack(fmt, dev(W))
    assert np.array_equal(want[1], host(got[1]))
    assert np.array_equal(want[0], host(got[0]))
