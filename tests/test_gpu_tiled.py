"""km4 on the row-tiled code plane (qtile_km4 + qmatvec_km4_tiled) against the
oracle: the relayout is checked byte for byte against the layout's definition
applied (in numpy) to the canonical codes, and the batch-1 matvec against the
oracle's fp64 matvec of the canonical codes and tables.

Codes are random bytes (every index pair occurs) and tables random fp16 values
~N(0, 0.02); the matvec's definition does not require them to come from
k-means. Shapes: every supported K (512 .. 4096), row counts that fill no tile,
one tile, a ragged last tile, and enough tiles for the two-tiles-per-workgroup
launch (including an odd tile count, whose last workgroup has a second tile
past the end); batch 1 to 4."""
import numpy as np
import pytest

import oracle
import quantized_decode_matvec_amd as qmv
from tests.gpu_helpers import RTOL, dev, host, rel_err

pytestmark = pytest.mark.gpu


def tiled_reference(codes: np.ndarray) -> np.ndarray:
    """The row-tiled byte order: chunk q (16 bytes) of row 64 t + r at byte
    ((t * Q + q) * 64 + r) * 16; rows past N zero."""
    N, half = codes.shape
    Q = half // 16
    T = (N + 63) // 64
    pad = np.zeros((T * 64, half), np.uint8)
    pad[:N] = codes
    return pad.reshape(T, 64, Q, 16).transpose(0, 2, 1, 3).reshape(-1)


def case(N, K, seed, B=1):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    lut = (rng.standard_normal((N, 16)) * 0.02).astype(np.float16).view(np.uint16)
    x = rng.standard_normal((B, K)).astype(np.float16)
    return codes, lut, x


def test_tiled_reference_is_a_permutation():
    codes, _, _ = case(100, 512, 0)
    t = tiled_reference(codes)
    assert t.size == 128 * 256
    assert np.array_equal(np.sort(t), np.sort(np.concatenate([codes.reshape(-1), np.zeros(28 * 256, np.uint8)])))
    # row 70, chunk 3 -> tile 1, r = 6
    assert np.array_equal(t[((1 * 16 + 3) * 64 + 6) * 16:][:16], codes[70, 48:64])


@pytest.mark.parametrize("N,K", [(1, 2048), (64, 512), (100, 1024), (4097, 2048), (3000, 4096),
                                 (70000, 2048), (65600, 1024), (66000, 512), (2000, 1536), (66000, 1536),
                                 (1500, 2560), (700, 3072), (900, 3584)])
def test_tiled_matvec_matches_oracle(N, K):
    print("tiled km4 N=%d K=%d" % (N, K), flush=True)
    codes, lut, x = case(N, K, seed=N + K)
    gt = qmv.qtile_km4(dev(codes))
    assert np.array_equal(host(gt), tiled_reference(codes))
    y = host(qmv.qmatvec_km4_tiled(gt, dev(lut), dev(x)))
    assert rel_err(y, oracle.matvec("km4", codes, lut, x)) <= RTOL


@pytest.mark.parametrize("B", [2, 3, 4])
@pytest.mark.parametrize("N,K", [(100, 512), (4097, 2048), (3000, 4096), (66001, 1024), (70000, 2048),
                                 (66001, 1536), (1500, 2560), (700, 3584)])
def test_tiled_matvec_batches_match_oracle(N, K, B):
    print("tiled km4 N=%d K=%d B=%d" % (N, K, B), flush=True)
    codes, lut, x = case(N, K, seed=N + K + B, B=B)
    y = host(qmv.qmatvec_km4_tiled(qmv.qtile_km4(dev(codes)), dev(lut), dev(x)))
    assert rel_err(y, oracle.matvec("km4", codes, lut, x)) <= RTOL


def test_tiled_matvec_repeat_is_bitwise_stable():
    """Fixed summation order: two calls give the same bits."""
    codes, lut, x = case(5000, 2048, 7)
    gt, gl, gx = qmv.qtile_km4(dev(codes)), dev(lut), dev(x)
    a = host(qmv.qmatvec_km4_tiled(gt, gl, gx))
    b = host(qmv.qmatvec_km4_tiled(gt, gl, gx))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_tiled_call_launcher():
    codes, lut, x = case(700, 1024, 3)
    gt = qmv.qtile_km4(dev(codes))
    call = qmv.qmatvec_km4_tiled_call(gt, dev(lut), dev(x))
    y = host(call())
    assert rel_err(y, oracle.matvec("km4", codes, lut, x)) <= RTOL
