"""GPU parity against the CPU oracle at sizes the oracle finishes in seconds:
packing bit-exact, dequant exact, matvec within the relative-error bound,
across every kernel variant (lanes per row, chunks per lane, batch width),
ragged row counts and the special blocks of each format."""
import numpy as np
import pytest

import oracle
import quantized_decode_matvec_amd as qmv
from quantized_decode_matvec_amd import workloads as wl
from tests.gpu_helpers import RTOL, bits_equal, dev, host, rel_err

pytestmark = pytest.mark.gpu

FMTS = ["int4", "fp4", "int8", "km4", "int4aff"]
# (N, K): short K (16 lanes per row), 32 lanes, one chunk per lane at 64 lanes,
# two/three/four chunks per lane, a K beyond the register fast path, ragged N
SHAPES = [(37, 96), (50, 512), (65, 1024), (129, 2048), (33, 2560), (47, 4096), (21, 6144), (8, 8192)]


def _special_rows(K, dtype):
    """Rows that hit the formats' corner cases: all zero, tiny values, exact
    E2M1 ties at E = 0, a single outlier per block, negative zeros."""
    rows = np.zeros((6, K), np.float32)
    rows[1, :] = 2.0 ** -24
    ties = np.array([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, -0.25, -2.5, -5.0], np.float32)
    rows[2, :] = np.resize(ties, K)
    rows[2, ::32] = 6.0
    rows[3, ::32] = 1.0
    rows[4, :] = -0.0
    rows[4, 1::2] = np.linspace(-1, 1, K // 2)
    rows[5, :] = np.resize(np.array([-0.5, 0.0, 0.25, 1.0], np.float32), K)
    return rows.astype(dtype)


def _case(fmt, N, K, B=1, dtype=np.float16, seed=0):
    c = wl.small_dense(fmt, N, K, batch=B, seed=seed, dtype=dtype, outlier_frac=0.01)
    W = c.W.copy()
    sp = _special_rows(K, dtype)
    W[: min(len(sp), N)] = sp[: min(len(sp), N)]
    return W, c.x


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", SHAPES[:6])
def test_pack_bit_exact(fmt, N, K):
    W, _ = _case(fmt, N, K)
    if fmt == "km4" and K > 4096:
        pytest.skip("km4 packing takes K <= 4096")
    want = oracle.pack(fmt, W)
    got = qmv.qpack(fmt, dev(W))
    for a, b in zip(want, got):
        assert bits_equal(a, host(b)), fmt


@pytest.mark.parametrize("fmt", ["int4", "fp4", "int8", "int4aff"])
def test_pack_fp32_input_bit_exact(fmt):
    c = wl.tiny_int4()
    W = c.W.copy()
    W[:6] = _special_rows(W.shape[1], np.float32)
    W[6, :32] = np.float32(0.99999994)
    W[7, :32] = np.float32(2.0 ** -130)
    want = oracle.pack(fmt, W)
    got = qmv.qpack(fmt, dev(W))
    for a, b in zip(want, got):
        assert bits_equal(a, host(b))


@pytest.mark.parametrize("max_iter", [1, 3, 20])
def test_km4_pack_iterations_bit_exact(max_iter):
    W, _ = _case("km4", 96, 512, seed=3)
    want = oracle.pack_km4(W, max_iter=max_iter)
    got = qmv.qpack_km4(dev(W), max_iter=max_iter)
    assert np.array_equal(want[0], host(got[0]))
    assert np.array_equal(want[1], host(got[1]))


def test_km4_pack_midpoint_means():
    """Rows whose cluster means fall on fp16 midpoints (ties to even)."""
    ints = [v for v in range(-8, 8) if v != 1]
    rows = []
    for pair in [(1.0, 1.0 + 2 ** -10), (1.0 + 2 ** -10, 1.0 + 2 ** -9)]:
        r = np.array(sorted(ints * 2 + list(pair)), np.float16)
        rows.append(r[np.random.default_rng(len(rows)).permutation(32)])
    W = np.stack(rows)
    want = oracle.pack_km4(W)
    got = qmv.qpack_km4(dev(W))
    assert np.array_equal(want[1], host(got[1]))
    assert np.array_equal(want[0], host(got[0]))


@pytest.mark.parametrize("fmt", FMTS)
def test_dequant_exact(fmt):
    W, _ = _case(fmt, 41, 2560 if fmt != "km4" else 2048)
    codes, plane = oracle.pack(fmt, W)
    D = host(qmv.qdequant(fmt, dev(codes), dev(plane)))
    want = oracle.dequant(fmt, codes, plane)
    if fmt == "int4aff":
        # s * u + b is exact in fp64 and rounded once to fp32 on the device
        want = want.astype(np.float32).astype(np.float64)
    assert np.array_equal(D.astype(np.float64), want)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("B", [1, 2, 3, 4, 8])
def test_matvec_parity(fmt, N, K, B):
    W, x = _case(fmt, N, K, B=B, seed=N + B)
    if fmt == "km4":
        codes, plane = oracle.pack_km4(W, max_iter=4)
    else:
        codes, plane = oracle.pack(fmt, W)
    want = oracle.matvec(fmt, codes, plane, x)
    y = host(qmv.qmatvec(fmt, dev(codes), dev(plane), dev(x)))
    assert rel_err(y, want) <= RTOL


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K,Bs", [(1000, 2048, (3, 5, 6, 7, 8)), (16, 512, (8,)), (17, 1536, (4, 8)),
                                    (600, 4096, (3,)), (300, 3584, (8,)), (517, 640, (4,)), (260, 256, (8,)),
                                    (4113, 2048, (5, 8)), (4113, 1536, (8,))])
def test_batched_matvec_parity(fmt, N, K, Bs):
    """The matrix-core batched path: several workgroups and a ragged last row
    group, every batch width it takes, a single row group (N = 16), one load
    step per row (K = 512) and three (K = 1536, past 4096 rows), the largest K
    it stages (4096, at B = 3); and shapes it hands to the dot2 path (up to
    4096 rows of K 1025..2048 at B = 5-8, x too
    large for its LDS stage at K = 3584, K = 640 not a multiple of 512, int8
    K = 256 taken but the 4-bit formats not)."""
    W, x = _case(fmt, N, K, B=8, seed=N + K)
    codes, plane = oracle.pack(fmt, W)
    dc, dp = dev(codes), dev(plane)
    for B in Bs:
        print("batched", fmt, N, K, B, flush=True)
        want = oracle.matvec(fmt, codes, plane, x[:B])
        y = host(qmv.qmatvec(fmt, dc, dp, dev(x[:B])))
        assert rel_err(y, want) <= RTOL


@pytest.mark.parametrize("fmt", ["int4", "int8", "int4aff"])
def test_batched_matvec_with_unaligned_scale_plane(fmt):
    """A scale plane aligned to its element size only (2 bytes; 4 for the
    affine words) is valid input; the batched path, which reads a group's
    scales as 16-byte pieces, leaves it to the dot2 path."""
    import torch
    N, K, B = 96, 1024, 8
    W, x = _case(fmt, N, K, B=B, seed=3)
    codes, plane = oracle.pack(fmt, W)
    want = oracle.matvec(fmt, codes, plane, x)
    flat = np.concatenate([np.zeros(1, plane.dtype), plane.reshape(-1)])
    dflat = dev(flat)
    dp = dflat[1:].view(plane.shape)
    assert dp.data_ptr() % 16 != 0
    y = host(qmv.qmatvec(fmt, dev(codes), dp, dev(x)))
    assert rel_err(y, want) <= RTOL


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("B", [1, 5])
def test_matvec_fp32_x(fmt, B):
    W, x = _case(fmt, 70, 512, B=B, dtype=np.float32, seed=7)
    if fmt == "km4":
        W = W.astype(np.float16)
    codes, plane = oracle.pack(fmt, W)
    want = oracle.matvec(fmt, codes, plane, x)
    y = host(qmv.qmatvec(fmt, dev(codes), dev(plane), dev(x.astype(np.float32))))
    assert rel_err(y, want) <= RTOL


@pytest.mark.parametrize("fmt", FMTS)
def test_matvec_unit_vectors_pick_columns_exactly(fmt):
    W, _ = _case(fmt, 64, 2048, seed=5)
    codes, plane = oracle.pack(fmt, W)
    D = oracle.dequant(fmt, codes, plane)
    if fmt == "int4aff":
        D = D.astype(np.float32).astype(np.float64)   # s * u + b rounded once to fp32
    ks = [0, 1, 31, 32, 1000, 2047]
    x = np.zeros((len(ks), 2048), np.float16)
    for i, k in enumerate(ks):
        x[i, k] = 1.0
    y = host(qmv.qmatvec(fmt, dev(codes), dev(plane), dev(x)))
    for i, k in enumerate(ks):
        assert np.array_equal(y[i].astype(np.float64), D[:, k])


@pytest.mark.parametrize("fmt", FMTS)
def test_matvec_deterministic(fmt):
    W, x = _case(fmt, 300, 2048, B=2, seed=9)
    codes, plane = oracle.pack(fmt, W) if fmt != "km4" else oracle.pack_km4(W, max_iter=2)
    c, p, xx = dev(codes), dev(plane), dev(x)
    y1 = host(qmv.qmatvec(fmt, c, p, xx))
    y2 = host(qmv.qmatvec(fmt, c, p, xx))
    assert np.array_equal(y1, y2)


def test_gpu_pack_then_gpu_matvec_matches_oracle_end_to_end():
    for fmt in FMTS:
        W, x = _case(fmt, 200, 2048, B=1, seed=11)
        codes, plane = qmv.qpack(fmt, dev(W))
        y = host(qmv.qmatvec(fmt, codes, plane, dev(x)))
        oc, op = oracle.pack(fmt, W)
        assert rel_err(y, oracle.matvec(fmt, oc, op, x)) <= RTOL


def test_stream_read_checksum():
    rng = np.random.default_rng(0)
    a = rng.integers(0, 2 ** 32, size=(1 << 20) + 4, dtype=np.uint32)
    sink = host(qmv.qmv_stream_read(dev(a.view(np.int32))))
    assert np.bitwise_xor.reduce(sink.view(np.uint32)) == np.bitwise_xor.reduce(a)


@pytest.mark.parametrize("fmt", ["int4", "fp4", "int8", "km4", "int4aff", "km4o"])
def test_tall_batch1_shape_on_sampled_rows(fmt):
    """At batch 1 a matrix of at least 32768 rows takes the tall launch shape
    (8 rows per wave for most formats). The GPU packs and multiplies the whole
    ragged matrix; the oracle packs the sampled rows (rows are packed
    independently) and computes their outputs."""
    from tests.gpu_helpers import sample_rows
    N, K = 32768 + 37, 1024
    c = wl.small_dense("km4", N, K, batch=1, seed=21, outlier_frac=0.01)
    W, x = c.W, c.x
    rows = sample_rows(N, n=96, seed=4)
    print("tall", fmt, N, K, flush=True)
    if fmt == "km4o":
        y = host(qmv.qmatvec_km4o(*qmv.qpack_km4o(dev(W), 8), dev(x)))
        want = oracle.matvec_km4o(*oracle.pack_km4o(W[rows], 8), x)
    else:
        codes, plane = qmv.qpack(fmt, dev(W))
        y = host(qmv.qmatvec(fmt, codes, plane, dev(x)))
        oc, op = oracle.pack(fmt, W[rows])
        want = oracle.matvec(fmt, oc, op, x)
    assert rel_err(y[:, rows], want) <= RTOL


@pytest.mark.parametrize("fmt", ["int4", "fp4", "int8", "km4", "int4aff", "int8km"])
@pytest.mark.parametrize("N,Bs", [(16416, (3, 4, 8)), (49184, (5,)), (98336, (8,))])
def test_batched_large_matrices_on_sampled_rows(fmt, N, Bs):
    """The matrix-core path at B = 3 and 4 takes matrices of at least 16384
    rows, and its rows per wave grow with N (one, two, four row groups here):
    the GPU packs and multiplies the whole matrix, the oracle packs and
    multiplies sampled rows (whole 32-row groups for int8 k-means)."""
    from tests.gpu_helpers import sample_rows
    K = 1024
    c = wl.small_dense("km4", N, K, batch=8, seed=N, outlier_frac=0.01)
    W, x = c.W, c.x
    print("large batched", fmt, N, Bs, flush=True)
    codes, plane = qmv.qpack(fmt, dev(W))
    if fmt == "int8km":
        groups = np.unique(sample_rows(N // 32, n=6, seed=2))
        rows = np.concatenate([np.arange(32 * g, 32 * g + 32) for g in groups])
    else:
        rows = sample_rows(N, n=96, seed=2)
    oc, op = oracle.pack(fmt, W[rows])
    for B in Bs:
        y = host(qmv.qmatvec(fmt, codes, plane, dev(x[:B])))
        assert rel_err(y[:, rows], oracle.matvec(fmt, oc, op, x[:B])) <= RTOL, B
