"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names what fixes the expected answer: a hand-worked block from the
pages' definitions (tests/golden), a closed form, an invariant that
characterises the result, a special case that reduces to a textbook or library
routine (numpy), or brute force on tiny inputs.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _records(name):
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                yield [p.strip() for p in line.rstrip("\n").split(";")]


def _f16(bits):
    return np.array(bits, np.uint16).view(np.float16)


# --------------------------------------------------------------------------
# binary16 helpers against numpy's float16 conversion (library routine)
# --------------------------------------------------------------------------

def test_f16_round_trip_all_finite_codes():
    bits = np.arange(0x10000, dtype=np.uint16)
    vals = bits.view(np.float16)
    finite = np.isfinite(vals)
    for b, v in zip(bits[finite][::37], vals[finite][::37]):
        assert oracle.f16_to_f64(int(b)) == float(v)
        back = oracle.f64_to_f16(float(v))
        assert back == int(b) or (float(v) == 0.0 and back == int(b))


def test_f16_rounding_matches_numpy():
    rng = np.random.default_rng(1)
    mags = np.concatenate([
        rng.uniform(0, 2 ** -14, 2000),            # subnormal range
        np.exp(rng.uniform(-20, 11, 4000)),        # normal range
        np.array([65504.0, 65519.99, 65520.0, 1e6, 2 ** -25, 3 * 2 ** -26, 2 ** -26]),
    ])
    # exact ties: midpoints between adjacent fp16 numbers
    f = np.arange(0x0001, 0x7bff, 97, dtype=np.uint16).view(np.float16).astype(np.float64)
    g = (np.arange(0x0001, 0x7bff, 97, dtype=np.uint16) + 1).view(np.float16).astype(np.float64)
    vals = np.concatenate([mags, -mags, (f + g) / 2])
    for v in vals:
        want = int(np.array(v, np.float64).astype(np.float16).view(np.uint16))
        assert oracle.f64_to_f16(float(v)) == want, v


# --------------------------------------------------------------------------
# FP4 E2M1 / e8m0
# --------------------------------------------------------------------------

def _e2m1_closed_form(code):
    """Decode from the bit fields: sign, 2 exponent bits (bias 1), 1 mantissa bit."""
    s = -1.0 if code & 8 else 1.0
    e = (code >> 1) & 3
    m = code & 1
    mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
    return s * mag


def test_e2m1_grid_closed_form():
    # scale byte 127 is 2^0, so dequant returns the raw grid values
    codes = np.array([[c | (c2 << 4) for c, c2 in zip(range(0, 16, 2), range(1, 16, 2))] + [0] * 8], np.uint8)
    scale = np.array([[127]], np.uint8)
    deq = oracle.dequant("fp4", codes, scale)[0, :16]
    want = [_e2m1_closed_form(c) for c in range(16)]
    assert list(deq) == want
    assert sorted(set(abs(v) for v in want)) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def test_fp4_golden_blocks():
    n = 0
    for name, dt, nz, sbyte, bytes_hex, deq in _records("fp4_blocks.txt"):
        if dt == "f16":
            w = np.zeros(32, np.float16)
            for item in filter(None, nz.split(",")):
                i, h = item.split("=")
                w[int(i)] = _f16(int(h, 16))
        else:
            w = np.zeros(32, np.float32)
            for item in filter(None, nz.split(",")):
                i, h = item.split("=")
                w[int(i)] = np.array(int(h, 16), np.uint32).view(np.float32)
        codes, scale = oracle.pack_fp4(w[None, :])
        assert scale[0, 0] == int(sbyte, 16), name
        want = bytes.fromhex(bytes_hex)
        assert codes[0, :len(want)].tobytes() == want, name
        d = oracle.dequant("fp4", codes, scale)[0]
        idx = [int(it.split("=")[0]) for it in filter(None, nz.split(","))]
        if deq:
            assert [d[i] for i in idx] == [float(v) for v in deq.split(",")], name
        n += 1
    assert n == 8


def _fp4_random_blocks(seed=3):
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((64, 256)).astype(np.float32) * np.float32(0.02)
    W[:, ::17] *= 40.0
    W[3, :] = 0.0
    W[5, 32:64] = np.float32(2 ** -130)              # subnormal fp32 block
    W[6, 64:96] = rng.standard_normal(32).astype(np.float32) * np.float32(1e-38)
    W[7, :32] *= np.float32(1e4)
    return W


def test_fp4_scale_invariant():
    """E is the unique exponent with amax / 2^E in [4, 8) (clamped to e8m0)."""
    W = _fp4_random_blocks()
    codes, scale = oracle.pack_fp4(W)
    blocks = W.reshape(W.shape[0], -1, 32)
    amax = np.abs(blocks.astype(np.float64)).max(-1)
    E = scale.astype(np.int64) - 127
    for a, e in zip(amax.ravel(), E.ravel()):
        if a == 0:
            assert e == -127
        elif math.ldexp(4.0, int(e)) <= a < math.ldexp(8.0, int(e)):
            pass
        else:
            assert e == -127 and a < math.ldexp(4.0, -127)


def test_fp4_codes_are_nearest_grid_points():
    """Every dequantized value is a nearest point of the scaled grid to w;
    on an exact tie it is the even-mantissa point; above 6 it saturates."""
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    W = _fp4_random_blocks()
    codes, scale = oracle.pack_fp4(W)
    D = oracle.dequant("fp4", codes, scale)
    for n in range(W.shape[0]):
        for k in range(W.shape[1]):
            E = int(scale[n, k // 32]) - 127
            v = math.ldexp(abs(float(W[n, k])), -E)
            got = math.ldexp(abs(D[n, k]), -E)
            dmin = min(abs(v - g) for g in grid)
            assert abs(v - got) == dmin
            ties = [i for i, g in enumerate(grid) if abs(v - g) == dmin]
            if len(ties) == 2:
                assert grid.index(got) % 2 == 0
            byte = codes[n, k // 2]
            c = byte & 15 if k % 2 == 0 else byte >> 4
            assert bool(c & 8) == bool(np.signbit(W[n, k]))


def test_fp4_tie_points():
    # ties of the E2M1 grid at scale 2^0 (block amax 6 sets E = 0)
    ties = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0, 7.0: 6.0}
    w = np.zeros((1, 32), np.float32)
    w[0, 0] = 6.0
    for i, v in enumerate(ties):
        w[0, 1 + i] = v
        w[0, 16 + i] = -v
    codes, scale = oracle.pack_fp4(w)
    assert scale[0, 0] == 127
    d = oracle.dequant("fp4", codes, scale)[0]
    for i, v in enumerate(ties):
        assert d[1 + i] == ties[v] and d[16 + i] == -ties[v]


# --------------------------------------------------------------------------
# int4 / int8 symmetric blocks
# --------------------------------------------------------------------------

def _golden_int_blocks():
    for name, fmt, clip, nz, s16, bytes_hex in _records("int_blocks.txt"):
        w = np.zeros((1, 32), np.float32)
        for item in nz.split(","):
            i, h = item.split("=")
            w[0, int(i)] = np.array(int(h, 16), np.uint32).view(np.float32)
        yield name, fmt, clip == "1", w, int(s16, 16), bytes.fromhex(bytes_hex)


def test_int_golden_blocks():
    seen = 0
    for name, fmt, clip, w, s16, want in _golden_int_blocks():
        if fmt == "int4":
            codes, scale = oracle.pack_int4(w, clip_search=clip)
            got = codes[0, :len(want)].tobytes()
        else:
            codes, scale = oracle.pack_int8(w)
            got = codes[0, :len(want)].view(np.uint8).tobytes()
        assert scale[0, 0] == s16, name
        assert got == want, name
        seen += 1
    assert seen == 3


def _numpy_absmax(W, qmax):
    """Textbook symmetric absmax quantization per block of 32 with numpy's
    float32 operations and float16 cast (library routines)."""
    B = W.reshape(W.shape[0], -1, 32).astype(np.float32)
    amax = np.abs(B).max(-1, keepdims=True)
    s = (amax / np.float32(qmax)).astype(np.float16)
    sf = s.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(sf == 0, 0, np.clip(np.rint(B / sf), -qmax, qmax))
    return q.astype(np.int64).reshape(W.shape), s[..., 0].view(np.uint16)


def _unpack_nibbles(codes):
    lo = (codes & 15).astype(np.int64)
    hi = (codes >> 4).astype(np.int64)
    return np.stack([lo, hi], -1).reshape(codes.shape[0], -1)


@pytest.mark.parametrize("seed", [0, 1])
def test_int8_is_textbook_absmax(seed):
    rng = np.random.default_rng(seed)
    W = (rng.standard_t(3, (48, 256)) * 0.02).astype(np.float32)
    W[2] = 0
    W[4, :32] = np.float32(1e-9)
    codes, scale = oracle.pack_int8(W)
    q, s = _numpy_absmax(W, 127)
    assert np.array_equal(scale, s)
    assert np.array_equal(codes.astype(np.int64), q)
    # the block's largest element always lands on +-127
    B = W.reshape(48, -1, 32)
    arg = np.abs(B).argmax(-1)
    cb = codes.reshape(48, -1, 32)
    for n in range(48):
        for b in range(B.shape[1]):
            if np.abs(B[n, b]).max() > 1e-6:
                assert abs(int(cb[n, b, arg[n, b]])) == 127


def test_int4_without_clip_search_is_textbook_absmax():
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((40, 512)) * 0.02).astype(np.float32)
    W[:, ::13] *= 20
    W[7] = 0
    codes, scale = oracle.pack_int4(W, clip_search=False)
    q, s = _numpy_absmax(W, 7)
    assert np.array_equal(scale, s)
    assert np.array_equal(_unpack_nibbles(codes) - 8, q)


def _block_sse64(w, s16, qmax):
    s = float(_f16(s16))
    if s == 0:
        return float(np.sum(w.astype(np.float64) ** 2))
    q = np.clip(np.rint(w.astype(np.float32) / np.float32(s)), -qmax, qmax)
    return float(np.sum((w.astype(np.float64) - s * q) ** 2))


def test_int4_clip_choice_is_the_error_minimum():
    """Against an independent fp64 evaluation of the seven clip candidates:
    the stored scale is one of them, its error is the minimum (within fp32
    summation noise), and never above the plain absmax error."""
    clips = [1.0, 0.95, 0.9, 0.85, 0.8, 0.75, 0.7]
    rng = np.random.default_rng(11)
    W = (rng.standard_normal((32, 256)) * 0.02).astype(np.float32)
    W[:, ::29] *= 20
    codes, scale = oracle.pack_int4(W)
    D = oracle.dequant("int4", codes, scale)
    chosen_any_clip = 0
    for n in range(W.shape[0]):
        for b in range(W.shape[1] // 32):
            w = W[n, 32 * b:32 * b + 32]
            amax = np.float32(np.abs(w).max())
            cands = [int(np.array(np.float32(np.float32(c) * amax) / np.float32(7)).astype(np.float16).view(np.uint16))
                     for c in clips]
            sse = [_block_sse64(w, s, 7) for s in cands]
            got = int(scale[n, b])
            assert got in cands
            got_sse = float(np.sum((w.astype(np.float64) - D[n, 32 * b:32 * b + 32]) ** 2))
            assert got_sse <= min(sse) * (1 + 1e-5) + 1e-30
            assert got_sse <= sse[0] * (1 + 1e-6) + 1e-30
            chosen_any_clip += got != cands[0]
    assert chosen_any_clip > 0   # the search is not a no-op on such data


def test_pack_layout_round_trip_all_bytes():
    """Every byte value decodes to (low nibble, high nibble) as elements (2j, 2j+1)."""
    codes = np.arange(256, dtype=np.uint8).reshape(16, 16)      # 16 rows, K = 32
    one = np.full((16, 1), 0x3C00, np.uint16)                   # fp16 1.0
    d = oracle.dequant("int4", codes, one)
    for r in range(16):
        for j in range(16):
            b = 16 * r + j
            assert d[r, 2 * j] == (b & 15) - 8 and d[r, 2 * j + 1] == (b >> 4) - 8
    lut = np.tile(np.arange(16, dtype=np.float16).view(np.uint16), (16, 1))
    d = oracle.dequant("km4", codes, lut)
    for r in range(16):
        for j in range(16):
            b = 16 * r + j
            assert d[r, 2 * j] == (b & 15) and d[r, 2 * j + 1] == (b >> 4)


def test_weight_error_levels_are_sane():
    """Soft check: per-32 block error levels on Gaussian weights sit near the
    pages' reported relative errors (int8 ~0.0055, int4 MSE-clip ~0.095, fp4
    ~0.117 on real weights; Gaussian int4 absmax is ~0.097)."""
    rng = np.random.default_rng(2)
    W = (rng.standard_normal((256, 1024)) * 0.02).astype(np.float32)

    def rel(fmt, **kw):
        c, s = oracle.pack(fmt, W, **kw)
        D = oracle.dequant(fmt, c, s)
        return np.linalg.norm(D - W) / np.linalg.norm(W)

    assert 0.004 < rel("int8") < 0.007
    assert 0.08 < rel("int4") < 0.10
    assert rel("int4") < rel("int4", clip_search=False)
    assert 0.09 < rel("fp4") < 0.13


# --------------------------------------------------------------------------
# km4 (k-means palettization)
# --------------------------------------------------------------------------

def test_km4_golden_rows():
    n = 0
    for name, pattern, lut_hex, bytes_hex in _records("km4_rows.txt"):
        pat = [int(h, 16) for h in pattern.split(",")]
        row = _f16(pat * 8)[None, :]
        codes, lut = oracle.pack_km4(row)
        assert [int(v) for v in lut[0]] == [int(h, 16) for h in lut_hex.split(",")], name
        want = bytes.fromhex(bytes_hex)
        assert codes[0, :len(want)].tobytes() == want, name
        n += 1
    assert n == 2


def test_km4_few_distinct_values_are_exact():
    rng = np.random.default_rng(4)
    for d in (1, 2, 5, 16):
        vals = rng.standard_normal(d).astype(np.float16)
        row = rng.choice(vals, size=(3, 256)).astype(np.float16)
        codes, lut = oracle.pack_km4(row)
        D = oracle.dequant("km4", codes, lut)
        assert np.array_equal(D, row.astype(np.float64))
        assert np.all(np.diff(lut.view(np.float16).astype(np.float64), axis=1) >= 0)


def _km4_check_invariants(W, codes, lut, iters, max_iter):
    Lf = lut.view(np.float16).astype(np.float64)
    idx = _unpack_nibbles(codes)
    Wf = W.astype(np.float64)
    assert np.all(np.diff(Lf, axis=1) >= 0), "table ascending"
    for n in range(W.shape[0]):
        dist = np.abs(Wf[n][:, None] - Lf[n][None, :])
        best = dist.min(1)
        # nearest entry, lowest index among equals
        first = np.argmax(dist == best[:, None], axis=1)
        assert np.array_equal(idx[n], first)
        if iters[n] < max_iter:
            # converged: every used entry is its members' mean rounded to fp16
            for j in np.unique(idx[n]):
                mem = W[n][idx[n] == j].astype(np.float64)
                mean = sum(Fraction(float(v)) for v in mem) / len(mem)
                c = Fraction(float(Lf[n, j]))
                lo = Fraction(float(np.nextafter(np.float16(Lf[n, j]), np.float16(-np.inf))))
                hi = Fraction(float(np.nextafter(np.float16(Lf[n, j]), np.float16(np.inf))))
                assert abs(mean - c) <= abs(mean - lo) and abs(mean - c) <= abs(mean - hi)


def test_km4_lloyd_invariants():
    rng = np.random.default_rng(6)
    W = (rng.standard_normal((12, 512)) * 0.02).astype(np.float16)
    W[3, ::7] *= 30
    codes, lut, iters = oracle.pack_km4(W, max_iter=200, return_iters=True)
    assert np.all(iters < 200)
    _km4_check_invariants(W, codes, lut, iters, 200)
    # with the default 20 steps, the nearest-entry invariant still holds
    codes, lut, iters = oracle.pack_km4(W, return_iters=True)
    _km4_check_invariants(W, codes, lut, iters, 20)


def test_km4_starting_table_is_order_statistics():
    """With no Lloyd step the table of a row with more than 16 distinct values
    is the row's order statistics at ranks (2j+1)K/32 (numpy sort), and every
    weight takes its nearest entry (ties to the lower index)."""
    rng = np.random.default_rng(44)
    for K in (32, 96, 2048):
        W = (rng.standard_normal((6, K)) * 0.02).astype(np.float16)
        W[2, ::5] *= 25
        codes, lut, iters = oracle.pack_km4(W, max_iter=0, return_iters=True)
        assert np.all(iters == 0)
        ranks = (2 * np.arange(16) + 1) * K // 32
        S = np.sort(W.astype(np.float64), axis=1)
        assert np.array_equal(lut.view(np.float16).astype(np.float64), S[:, ranks]), K
        _km4_check_invariants(W, codes, lut, iters, 0)


# A row of 32 distinct integers worked through the Lloyd steps by hand with the
# midpoint rule (a weight goes to the number of adjacent entry pairs whose sum
# is strictly below twice the weight) and exact member means (all fp16 numbers).
_KM4_HAND_ROW = list(range(24)) + [33, 37, 38, 39, 48, 49, 62, 63]
_KM4_HAND_HEAD = [1.0] + [2 * j + 1.5 for j in range(1, 11)] + [23.0]   # entries 0..11 after step 1
_KM4_HAND_TABLES = {
    # start: ranks 1, 3, ..., 31 of the sorted row
    0: [2 * j + 1.0 for j in range(12)] + [37.0, 39.0, 49.0, 63.0],
    # step 1 (midpoints 2, 4, .., 22, 30, 38, 44, 56): {0,1,2} {3,4} .. {21,22} {23}
    # {33,37,38} {39} {48,49} {62,63}
    1: _KM4_HAND_HEAD + [36.0, 39.0, 48.5, 62.5],
    # step 2 (midpoints .., 29.5, 37.5, 43.75, 55.5): 38 moves up: {33,37} {38,39}
    2: _KM4_HAND_HEAD + [35.0, 38.5, 48.5, 62.5],
    # step 3 (midpoints .., 29, 36.75, 43.5, 55.5): 37 moves up: {33} {37,38,39}
    3: _KM4_HAND_HEAD + [33.0, 38.0, 48.5, 62.5],
    # step 4 (midpoints .., 28, 35.5, 43.25, 55.5) moves nothing: stop
}


def _km4_hand_codes(table):
    t = np.array(table)
    v = np.array(_KM4_HAND_ROW, np.float64)
    return np.sum((t[:-1] + t[1:])[None, :] < 2 * v[:, None], axis=1)


@pytest.mark.parametrize("max_iter", [0, 1, 2, 3, 4, 20])
def test_km4_hand_worked_lloyd_steps(max_iter):
    perm = np.random.default_rng(45).permutation(32)          # weights in a scrambled order
    row = np.array(_KM4_HAND_ROW, np.float16)[perm][None, :]
    codes, lut, iters = oracle.pack_km4(row, max_iter=max_iter, return_iters=True)
    table = _KM4_HAND_TABLES[min(max_iter, 3)]
    assert iters[0] == min(max_iter, 4)
    assert lut[0].view(np.float16).astype(np.float64).tolist() == table
    assert np.array_equal(_unpack_nibbles(codes)[0], _km4_hand_codes(table)[perm])


def test_km4_default_is_twenty_lloyd_steps():
    """The default table is the one after at most 20 steps: on rows that need
    more, it equals max_iter=20 and differs from 19 and 21."""
    rng = np.random.default_rng(46)
    W = rng.standard_normal((64, 2048)).astype(np.float16)
    _, _, iters = oracle.pack_km4(W, max_iter=500, return_iters=True)
    slow = np.nonzero(iters > 22)[0][:4]
    assert slow.size > 0
    W = W[slow]
    c, l = oracle.pack_km4(W)
    c20, l20 = oracle.pack_km4(W, max_iter=20)
    assert np.array_equal(c, c20) and np.array_equal(l, l20)
    for m in (19, 21):
        cm, lm = oracle.pack_km4(W, max_iter=m)
        assert not np.array_equal(lm, l20), m


def test_km4_gaussian_reaches_lloyd_max_levels():
    """A long Gaussian row converges to the 16-level Lloyd-Max quantizer of
    N(0, 1) (Max, 1960: levels +-0.1284, 0.3881, 0.6568, 0.9424, 1.2562, 1.6181,
    2.0690, 2.7326 sigma; normalised error 0.00950)."""
    levels = np.array([0.1284, 0.3881, 0.6568, 0.9424, 1.2562, 1.6181, 2.0690, 2.7326])
    want = np.concatenate([-levels[::-1], levels])
    rng = np.random.default_rng(7)
    row = rng.standard_normal((1, 32768)).astype(np.float16)
    codes, lut, iters = oracle.pack_km4(row, max_iter=500, return_iters=True)
    got = lut.view(np.float16).astype(np.float64)[0]
    assert np.max(np.abs(got - want)) < 0.06
    D = oracle.dequant("km4", codes, lut)
    mse = np.mean((D - row.astype(np.float64)) ** 2) / np.var(row.astype(np.float64))
    assert abs(mse - 0.0095) < 0.0006


# --------------------------------------------------------------------------
# matvec
# --------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", ["int4", "fp4", "int8", "km4", "int4aff"])
def test_matvec_equals_dense_fp64_matmul(fmt):
    rng = np.random.default_rng(8)
    W = (rng.standard_normal((37, 96)) * 0.02).astype(np.float16)
    x = rng.standard_normal((3, 96)).astype(np.float16)
    codes, plane = oracle.pack(fmt, W)
    D = oracle.dequant(fmt, codes, plane)
    y = oracle.matvec(fmt, codes, plane, x)
    ref = x.astype(np.float64) @ D.T           # numpy fp64 GEMM (library routine)
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-15)
    # unit vectors pick columns exactly
    k = 41
    e = np.zeros((1, 96), np.float16)
    e[0, k] = 1
    assert np.array_equal(oracle.matvec(fmt, codes, plane, e)[0], D[:, k])
    # row subset agrees with the full result
    rows = np.array([36, 0, 17])
    assert np.array_equal(oracle.matvec(fmt, codes, plane, x, rows=rows), y[:, rows])


def test_matvec_linearity():
    rng = np.random.default_rng(9)
    W = (rng.standard_normal((16, 64)) * 0.02).astype(np.float32)
    codes, plane = oracle.pack_int4(W)
    a = rng.standard_normal((1, 64))
    b = rng.standard_normal((1, 64))
    ya = oracle.matvec("int4", codes, plane, a)
    yb = oracle.matvec("int4", codes, plane, b)
    yab = oracle.matvec("int4", codes, plane, 2 * a - 3 * b)
    assert np.allclose(yab, 2 * ya - 3 * yb, rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------
# mixture of experts
# --------------------------------------------------------------------------

def test_moe_route_matches_numpy_sort_and_softmax():
    rng = np.random.default_rng(10)
    L = rng.standard_normal((8, 256)).astype(np.float32)
    L[2, 10] = L[2, 200] = L[2].max() + 1          # equal logits: lower id first
    ids, w = oracle.moe_route(L, 8)
    for t in range(8):
        order = np.argsort(-L[t].astype(np.float64), kind="stable")[:8]
        assert np.array_equal(ids[t], order)
        z = np.exp(L[t, order].astype(np.float64) - L[t, order].max())
        assert np.allclose(w[t], z / z.sum(), rtol=1e-14)
    assert ids[2, 0] == 10 and ids[2, 1] == 200


def _small_moe(seed=12, E=6, H=64, I=32, fmt="int4"):
    rng = np.random.default_rng(seed)
    gu = (rng.standard_normal((E * 2 * I, H)) * 0.02).astype(np.float16)
    dn = (rng.standard_normal((E * H, I)) * 0.02).astype(np.float16)
    guc, gus = oracle.pack(fmt, gu)
    dnc, dns = oracle.pack(fmt, dn)
    return (guc.reshape(E, 2 * I, -1), gus.reshape(E, 2 * I, -1),
            dnc.reshape(E, H, -1), dns.reshape(E, H, -1), rng)


@pytest.mark.parametrize("fmt", ["int4", "fp4", "int8", "km4", "int4aff"])
def test_moe_top1_reduces_to_one_expert_ffn(fmt):
    """One slot of weight 1 is that expert's SwiGLU FFN (numpy GEMVs over the
    dequantized slabs); the last expert catches a wrong per-expert stride, and
    two slots give the weighted sum of the two one-expert results."""
    E, H, I = 6, 64, 32
    guc, gus, dnc, dns, rng = _small_moe(E=E, H=H, I=I, fmt=fmt)
    x = rng.standard_normal((1, H)).astype(np.float16)
    refs = {}
    for e in (1, E - 1):
        y = oracle.moe_ffn(guc, gus, dnc, dns, x, np.array([[e]]), np.array([[1.0]]), fmt=fmt)
        Wg = oracle.dequant(fmt, guc[e], gus[e])
        Wd = oracle.dequant(fmt, dnc[e], dns[e])
        g = Wg @ x[0].astype(np.float64)                  # numpy GEMV
        h = (g[:I] / (1 + np.exp(-g[:I])) * g[I:]).astype(np.float16).astype(np.float64)
        refs[e] = Wd @ h
        assert np.allclose(y[0], refs[e], rtol=1e-12, atol=1e-12)
    y2 = oracle.moe_ffn(guc, gus, dnc, dns, x, np.array([[E - 1, 1]]), np.array([[0.75, 0.25]]), fmt=fmt)
    assert np.allclose(y2[0], 0.75 * refs[E - 1] + 0.25 * refs[1], rtol=1e-12, atol=1e-15)


def test_moe_token_order_and_shared_experts():
    guc, gus, dnc, dns, rng = _small_moe(seed=13)
    H = 2 * guc.shape[2]
    x = rng.standard_normal((4, H)).astype(np.float16)
    L = rng.standard_normal((4, guc.shape[0])).astype(np.float32)
    ids, w = oracle.moe_route(L, 3)
    y = oracle.moe_ffn(guc, gus, dnc, dns, x, ids, w)
    perm = np.array([2, 0, 3, 1])
    yp = oracle.moe_ffn(guc, gus, dnc, dns, x[perm], ids[perm], w[perm])
    assert np.array_equal(yp, y[perm])
    # every token sending weight 1 to one shared expert: a batched single-expert FFN
    ids1 = np.full((4, 1), 2, np.int32)
    y1 = oracle.moe_ffn(guc, gus, dnc, dns, x, ids1, np.ones((4, 1)))
    for t in range(4):
        yt = oracle.moe_ffn(guc, gus, dnc, dns, x[t:t + 1], ids1[:1], np.ones((1, 1)))
        assert np.array_equal(yt[0], y1[t])


@pytest.mark.parametrize("pair,kept,other", [
    ((1.0, 1.0 + 2 ** -10), 0x3C00, 0x3C01),                 # lower neighbour even
    ((1.0 + 2 ** -10, 1.0 + 2 ** -9), 0x3C02, 0x3C01),       # upper neighbour even
])
def test_km4_mean_on_an_fp16_midpoint_rounds_to_even(pair, kept, other):
    """Two members whose mean lies halfway between two fp16 numbers: the one
    with the even significand is kept. Fifteen well-separated integer values
    (each twice) occupy the other fifteen entries."""
    ints = [v for v in range(-8, 8) if v != 1]
    row = np.array(sorted(ints * 2 + list(pair)), np.float16)[None, :]
    rng = np.random.default_rng(0)
    row = row[:, rng.permutation(32)]
    codes, lut, iters = oracle.pack_km4(row, return_iters=True)
    L = [int(v) for v in lut[0]]
    assert kept in L and other not in L
    D = oracle.dequant("km4", codes, lut)[0]
    kept_val = float(_f16(kept))
    assert np.all(D[np.isin(row[0], np.array(pair, np.float16))] == kept_val)
    for v in ints:
        assert np.all(D[row[0] == v] == v)


# --- embedding table (int8, one scale per row) and fused argmax ---

def test_int8_rows_hand_worked():
    """Row [1.27, -0.005, -0.635, 0, ...]: amax 1.27 gives the fp16 scale
    0x211F (0.0100021); 1.27/s = 126.97 -> 127, -0.005/s = -0.4999 -> 0,
    -0.635/s = -63.49 -> -63. The gathered values are fp16(q * s)."""
    w = np.zeros((1, 64), np.float32)
    w[0, :3] = [1.27, -0.005, -0.635]
    q, s = oracle.pack_int8_rows(w)
    assert s[0] == 0x211F
    assert list(q[0, :3]) == [127, 0, -63] and not q[0, 3:].any()
    out = oracle.embed_gather_int8(q, s, [0])
    sv = np.array([0x211F], np.uint16).view(np.float16)[0]
    assert out[0, 0] == (np.float16(127) * sv).view(np.uint16)
    assert out[0, 2] == (np.float16(-63) * sv).view(np.uint16)
    assert out[0, 1] == 0


def test_int8_rows_equal_textbook_absmax():
    """Per-row symmetric int8 equals the textbook recipe computed with numpy in
    fp32 (amax, fp16 scale, rint, clamp), an all-zero row included."""
    rng = np.random.default_rng(31)
    W = (rng.standard_normal((40, 300)) * 0.05).astype(np.float32)
    W[5] = 0.0
    W[6, 17] = -3.0
    q, s = oracle.pack_int8_rows(W)
    amax = np.abs(W).max(axis=1)
    s_np = (amax / np.float32(127)).astype(np.float16)
    assert np.array_equal(s, s_np.view(np.uint16))
    sf = s_np.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q_np = np.clip(np.rint(W / sf[:, None]), -127, 127)
    q_np[sf == 0] = 0
    assert np.array_equal(q, q_np.astype(np.int8))


def test_embed_gather_equals_numpy_fp16_product():
    rng = np.random.default_rng(32)
    W = (rng.standard_normal((70, 96)) * 0.02).astype(np.float16)
    q, s = oracle.pack_int8_rows(W)
    ids = np.array([0, 69, 5, 5, 33, 0], np.int32)
    out = oracle.embed_gather_int8(q, s, ids)
    want = q[ids].astype(np.float16) * s.view(np.float16)[ids][:, None]
    assert np.array_equal(out, want.view(np.uint16))
    # ids that name no row (below 0, at or past V) give zero rows, the others as above
    bad = np.array([-1, 3, 70, 1 << 30, 69], np.int32)
    out = oracle.embed_gather_int8(q, s, bad)
    assert not out[[0, 2, 3]].any()
    assert np.array_equal(out[[1, 4]], oracle.embed_gather_int8(q, s, bad[[1, 4]]))


@pytest.mark.parametrize("fmt", ["int4", "fp4", "int8", "km4", "int4aff"])
def test_matvec_argmax_picks_the_lowest_index_among_equal_maxima(fmt):
    """The argmax of the fp64 products equals numpy's on a numpy GEMM of the
    dequantized matrix; two identical winning rows give the lower index."""
    rng = np.random.default_rng(33)
    W = (rng.standard_normal((50, 128)) * 0.02).astype(np.float16)
    x = rng.standard_normal((3, 128)).astype(np.float16)
    W[41] = W[17] = np.sign(x[0]).astype(np.float16) * 0.05   # rows 17 and 41: the largest for token 0
    codes, plane = oracle.pack(fmt, W)
    idx, val = oracle.matvec_argmax(fmt, codes, plane, x)
    ref = x.astype(np.float64) @ oracle.dequant(fmt, codes, plane).T
    assert idx[0] == 17
    assert np.array_equal(idx, np.argmax(ref, axis=1))
    assert np.allclose(val, ref.max(axis=1), rtol=1e-12, atol=0)


# --- affine int4 (scale and bias per 32-block) ---

def test_int4aff_golden_blocks():
    seen = 0
    for name, nz, word, bytes_hex in _records("int4aff_blocks.txt"):
        w = np.zeros((1, 32), np.float32)
        for item in nz.split(","):
            i, h = item.split("=")
            v = np.array(int(h, 16), np.uint32).view(np.float32)
            if i == "all":
                w[0, :] = v
            else:
                w[0, int(i)] = v
        codes, plane = oracle.pack_int4aff(w)
        assert plane[0, 0] == int(word, 16), name
        want = bytes.fromhex(bytes_hex)
        assert codes[0, :len(want)].tobytes() == want, name
        seen += 1
    assert seen == 2
    w = np.zeros((1, 32), np.float32)
    w[0, :3] = [-0.5, 0.25, 1.0]
    d = oracle.dequant("int4aff", *oracle.pack_int4aff(w))[0]
    s = np.float64(np.array(0x2E66, np.uint16).view(np.float16))
    assert d[0] == -0.5 and d[1] == 8 * s - 0.5 and d[2] == 15 * s - 0.5 and d[3] == 5 * s - 0.5


def test_int4aff_equals_numpy_minmax():
    """The packer equals the min-max affine recipe computed with numpy's fp32
    operations and fp16 casts, over random blocks, a constant block and
    blocks with a large outlier."""
    rng = np.random.default_rng(41)
    W = (rng.standard_normal((30, 256)) * 0.03).astype(np.float32)
    W[2, :32] = 0.125
    W[3, 40] = 5.0
    B = W.reshape(30, -1, 32)
    mn, mx = B.min(-1, keepdims=True), B.max(-1, keepdims=True)
    s = ((mx - mn) / np.float32(15)).astype(np.float16)
    b = mn.astype(np.float16)
    sf, bf = s.astype(np.float32), b.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        u = np.where(sf == 0, 0, np.clip(np.rint((B - bf) / sf), 0, 15)).astype(np.int64).reshape(30, 256)
    codes, plane = oracle.pack_int4aff(W)
    assert np.array_equal(_unpack_nibbles(codes), u)
    word = s[..., 0].view(np.uint16).astype(np.uint32) | (b[..., 0].view(np.uint16).astype(np.uint32) << 16)
    assert np.array_equal(plane, word)


def test_int4aff_reconstruction_error_is_half_a_step():
    """Every reconstructed value lies within half a step (plus the fp16
    rounding of the bias) of its input."""
    rng = np.random.default_rng(42)
    W = (rng.standard_normal((20, 512)) * 0.05).astype(np.float32)
    codes, plane = oracle.pack_int4aff(W)
    D = oracle.dequant("int4aff", codes, plane)
    s = (plane & 0xFFFF).astype(np.uint16).view(np.float16).astype(np.float64)
    b = (plane >> 16).astype(np.uint16).view(np.float16).astype(np.float64)
    mn = W.reshape(20, -1, 32).min(-1).astype(np.float64)
    bound = 0.5 * s + np.abs(b - mn) + 1e-6 * s
    err = np.abs(D - W).reshape(20, -1, 32).max(-1)
    assert np.all(err <= bound)


# --- int8 k-means: one 256-entry table per group of 32 rows ---

def test_int8km_few_distinct_values_are_exact():
    """At most 256 distinct numbers in a group: they are the table (ascending,
    padded with the largest), so dequant reproduces the weights exactly."""
    rng = np.random.default_rng(40)
    for d in (1, 3, 200, 256):
        vals = np.unique(rng.standard_normal(4 * d).astype(np.float16))[:d]
        assert len(vals) == d
        W = rng.choice(vals, size=(64, 96)).astype(np.float16)
        W[32:] = (W[:32][::-1] * np.float16(-3)).astype(np.float16)   # second group: its own values
        codes, lut = oracle.pack_int8km(W)
        assert codes.shape == (64, 96) and lut.shape == (2, 256)
        assert np.array_equal(oracle.dequant("int8km", codes, lut), W.astype(np.float64))
        Lf = lut.view(np.float16).astype(np.float64)
        for g in range(2):
            used = np.unique(W[32 * g:32 * g + 32].astype(np.float64))
            assert np.array_equal(Lf[g, :len(used)], used)
            assert np.all(Lf[g, len(used):] == used[-1])


def test_int8km_starting_table_is_order_statistics():
    """With no Lloyd step the table is the group's order statistics at ranks
    (2j+1)M/512 (numpy sort), and every weight takes its nearest entry."""
    rng = np.random.default_rng(41)
    W = (rng.standard_normal((64, 128)) * 0.02).astype(np.float16)
    codes, lut, iters = oracle.pack_int8km(W, max_iter=0, return_iters=True)
    assert np.all(iters == 0)
    M = 32 * 128
    ranks = (2 * np.arange(256) + 1) * M // 512
    for g in range(2):
        S = np.sort(W[32 * g:32 * g + 32].reshape(-1).astype(np.float64))
        assert np.array_equal(lut[g].view(np.float16).astype(np.float64), S[ranks])
    _int8km_check_nearest(W, codes, lut)


def test_int8km_hand_worked_fixed_point():
    """Even integers 0..1022, four copies each, in one group: the starting
    entries are 4j+2; one Lloyd step moves entry 0 to 2 (members 0, 2, 4),
    entry j to 4j+3 (members 4j+2, 4j+4) and keeps 1022 in the last; the next
    step moves nothing. Worked by hand from the midpoint rule."""
    vals = np.repeat(np.arange(0, 1024, 2), 4)
    rng = np.random.default_rng(42)
    W = vals[rng.permutation(vals.size)].reshape(32, 64).astype(np.float16)
    codes, lut, iters = oracle.pack_int8km(W, return_iters=True)
    want = np.array([2] + [4 * j + 3 for j in range(1, 255)] + [1022], np.float64)
    assert np.array_equal(lut[0].view(np.float16).astype(np.float64), want)
    assert iters[0] == 2
    v = W.astype(np.int64)
    want_codes = np.where(v <= 4, 0, (v - 2) // 4)
    assert np.array_equal(codes.astype(np.int64), want_codes)


def _int8km_check_nearest(W, codes, lut):
    Lf = lut.view(np.float16).astype(np.float64)
    for g in range(W.shape[0] // 32):
        w = W[32 * g:32 * g + 32].reshape(-1).astype(np.float64)
        c = codes[32 * g:32 * g + 32].reshape(-1).astype(np.int64)
        assert np.all(np.diff(Lf[g]) >= 0), "table ascending"
        dist = np.abs(w[:, None] - Lf[g][None, :])
        assert np.array_equal(dist[np.arange(w.size), c], dist.min(1)), "nearest entry"
        # among distinct entries at equal distance the lower one is taken
        best = dist.min(1)
        first = np.argmax(dist == best[:, None], axis=1)
        assert np.all((Lf[g][first] == Lf[g][c]) | (first == c))
        tie = np.isclose(dist[np.arange(w.size), first], dist[np.arange(w.size), c]) & (Lf[g][first] != Lf[g][c])
        assert not np.any(tie & (Lf[g][c] > Lf[g][first]))


def test_int8km_lloyd_invariants():
    """Converged groups: every weight takes its nearest entry and every used
    entry is its members' exact mean rounded to the nearest fp16 number."""
    rng = np.random.default_rng(43)
    W = (rng.standard_normal((64, 64)) * 0.02).astype(np.float16)
    W[40, ::5] *= 25                                 # outliers in the second group
    codes, lut, iters = oracle.pack_int8km(W, max_iter=2000, return_iters=True)
    assert np.all(iters < 2000)
    _int8km_check_nearest(W, codes, lut)
    Lf = lut.view(np.float16).astype(np.float64)
    for g in range(2):
        w = W[32 * g:32 * g + 32].reshape(-1)
        c = codes[32 * g:32 * g + 32].reshape(-1)
        for j in np.unique(c):
            mem = w[c == j].astype(np.float64)
            mean = sum(Fraction(float(v)) for v in mem) / len(mem)
            e = np.float16(Lf[g, j])
            lo = Fraction(float(np.nextafter(e, np.float16(-np.inf))))
            hi = Fraction(float(np.nextafter(e, np.float16(np.inf))))
            assert abs(mean - Fraction(float(e))) <= min(abs(mean - lo), abs(mean - hi))
    # the default 20 steps keep the nearest-entry property
    codes, lut = oracle.pack_int8km(W)
    _int8km_check_nearest(W, codes, lut)


def test_int8km_uniform_group_reaches_the_uniform_quantizer():
    """256-level k-means of a uniform group: the optimal quantizer has equal
    cells, with squared error (2/L)^2/12 for U(-1, 1), i.e. var/L^2; the
    entries sit at the cell centres (2j+1)/L - 1."""
    rng = np.random.default_rng(44)
    W = rng.uniform(-1, 1, (32, 1024)).astype(np.float16)
    codes, lut = oracle.pack_int8km(W)
    D = oracle.dequant("int8km", codes, lut)
    w = W.astype(np.float64)
    mse = np.mean((D - w) ** 2)
    want = (2 / 256) ** 2 / 12
    assert abs(mse / want - 1) < 0.05, (mse, want)
    centres = (2 * np.arange(256) + 1) / 256 - 1
    # sampling noise moves the cell edges by a fraction of a cell, never by one
    assert np.max(np.abs(lut[0].view(np.float16).astype(np.float64) - centres)) < 2 / 256


def test_int8km_matvec_moe_and_argmax():
    """Matvec equals a numpy GEMM of the dequantized rows (groups of 32 rows
    sharing a table), the one-expert MoE reduces to numpy GEMVs, and equal
    winning rows of one group give the lower index."""
    rng = np.random.default_rng(45)
    W = (rng.standard_normal((64, 96)) * 0.02).astype(np.float16)
    x = rng.standard_normal((3, 96)).astype(np.float16)
    W[20] = W[17] = np.sign(x[0]).astype(np.float16) * 0.05
    codes, lut = oracle.pack_int8km(W)
    D = oracle.dequant("int8km", codes, lut)
    assert np.array_equal(D[33], lut[1].view(np.float16).astype(np.float64)[codes[33]])
    y = oracle.matvec("int8km", codes, lut, x)
    assert np.allclose(y, x.astype(np.float64) @ D.T, rtol=1e-13, atol=1e-15)
    idx, val = oracle.matvec_argmax("int8km", codes, lut, x)
    assert idx[0] == 17
    E, H, I = 6, 64, 32
    guc, gus, dnc, dns, rng = _small_moe(E=E, H=H, I=I, fmt="int8km")
    xt = rng.standard_normal((1, H)).astype(np.float16)
    e = E - 1
    y = oracle.moe_ffn(guc, gus, dnc, dns, xt, np.array([[e]]), np.array([[1.0]]), fmt="int8km")
    Wg = oracle.dequant("int8km", guc[e], gus[e])
    Wd = oracle.dequant("int8km", dnc[e], dns[e])
    g = Wg @ xt[0].astype(np.float64)
    h = (g[:I] / (1 + np.exp(-g[:I])) * g[I:]).astype(np.float16).astype(np.float64)
    assert np.allclose(y[0], Wd @ h, rtol=1e-12, atol=1e-12)


# --- 4-bit k-means rows plus int8 outliers ---

def _km4o_dense_numpy(codes, lut, ocol, oval, oscale):
    """W_hat assembled with numpy from the packed pieces: table lookups plus the
    scattered int8 outliers times the row scale."""
    idx = _unpack_nibbles(codes)
    L = lut.view(np.float16).astype(np.float64)
    W = np.take_along_axis(L, idx.astype(np.int64), axis=1)
    s = oscale.view(np.float16).astype(np.float64)
    for n in range(W.shape[0]):
        W[n, ocol[n].astype(np.int64)] += s[n] * oval[n].astype(np.float64)
    return W


def test_km4o_without_outliers_is_km4():
    rng = np.random.default_rng(50)
    W = (rng.standard_normal((9, 256)) * 0.02).astype(np.float16)
    codes, lut, ocol, oval, oscale = oracle.pack_km4o(W, 0)
    c4, l4 = oracle.pack_km4(W)
    assert np.array_equal(codes, c4) and np.array_equal(lut, l4)
    assert ocol.shape == (9, 0) and np.all(oscale == 0)


def test_km4o_outliers_are_the_largest_magnitudes_as_textbook_int8():
    """Selection equals a numpy lexsort on (-|w|, column); the values are the
    absmax int8 recipe on them (numpy); the 4-bit part is the k-means of the
    row with the outliers zeroed."""
    rng = np.random.default_rng(51)
    W = (rng.standard_normal((12, 512)) * 0.02).astype(np.float16)
    W[:, ::37] *= 8
    W[3, [10, 20, 30]] = np.float16(0.5)          # equal magnitudes: lower columns first
    W[3, [15, 25]] = np.float16(-0.5)
    W[5] = 0                                       # all-zero row: scale 0, q 0
    P = 6
    codes, lut, ocol, oval, oscale = oracle.pack_km4o(W, P)
    for n in range(W.shape[0]):
        a = np.abs(W[n].astype(np.float64))
        order = np.lexsort((np.arange(512), -a))[:P]
        cols = np.sort(order)
        assert np.array_equal(ocol[n], cols)
        amax = np.float32(a[cols].max())
        s = np.float16(amax / np.float32(127))
        assert oscale[n] == s.view(np.uint16)
        if s == 0:
            q = np.zeros(P)
        else:
            q = np.clip(np.rint(W[n, cols].astype(np.float32) / np.float32(s)), -127, 127)
        assert np.array_equal(oval[n].astype(np.float64), q.astype(np.float64))
        res = W[n].copy()
        res[cols] = 0
        c4, l4 = oracle.pack_km4(res[None, :])
        assert np.array_equal(codes[n], c4[0]) and np.array_equal(lut[n], l4[0])
    assert list(ocol[3][:5]) == [10, 15, 20, 25, 30]


def test_km4o_matvec_equals_numpy_gemm_and_outliers_help():
    rng = np.random.default_rng(52)
    W = (rng.standard_normal((40, 256)) * 0.02).astype(np.float16)
    big = rng.choice(256, size=4, replace=False)
    W[:, big] = (rng.standard_normal((40, 4)) * 0.5).astype(np.float16)   # heavy columns
    x = rng.standard_normal((3, 256)).astype(np.float16)
    packed = oracle.pack_km4o(W, 4)
    D = _km4o_dense_numpy(*packed)
    y = oracle.matvec_km4o(*packed, x)
    assert np.allclose(y, x.astype(np.float64) @ D.T, rtol=1e-13, atol=1e-15)
    # outliers taken out of the table lower the weight error against plain km4
    c4, l4 = oracle.pack_km4(W)
    e4 = np.abs(oracle.dequant("km4", c4, l4) - W.astype(np.float64)).mean()
    eo = np.abs(D - W.astype(np.float64)).mean()
    assert eo < 0.75 * e4


@pytest.mark.parametrize("fmt", ["km4", "int8km"])
def test_kmeans_empty_entries_stay_in_place(fmt):
    """Half the values equal 0.5: the starting order statistics repeat 0.5 many
    times, the repeated entries above the first get no members (the midpoint
    rule sends 0.5 to the lowest of them) and must keep their value, so the
    table stays ascending and (in some row) still holds 0.5 more than once."""
    rng = np.random.default_rng(60)
    rows = 32 if fmt == "int8km" else 4
    W = (rng.standard_normal((rows, 512)) * 0.3).astype(np.float16)
    W[:, ::2] = np.float16(0.5)
    codes, lut = oracle.pack(fmt, W)
    L = lut.view(np.float16).astype(np.float64)
    assert np.all(np.diff(L, axis=-1) >= 0)
    assert max(np.sum(L[r] == 0.5) for r in range(L.shape[0])) >= 2
    if fmt == "int8km":
        _int8km_check_nearest(W, codes, lut)
