"""Oracle: plain CPU reference for block-quantized decode matvec.

TEST INFRASTRUCTURE ONLY. Only the test suite, ``__graft_entry__.smoke()`` and
the benchmark's CPU-baseline leg may import this package. The GPU library under
``quantized_decode_matvec_amd`` never imports it, and this package imports
nothing from there: the two share no code. The arithmetic lives in
``oracle.c`` (plain C, one IEEE operation per step, fp64 accumulation); this
module only builds it with gcc and marshals numpy arrays through ctypes.

Formats (codes and planes as numpy arrays; W is N x K row-major, K % 32 == 0):

* int4: codes uint8 [N, K/2] (u = q + 8, element 2j in the low nibble),
  scale uint16 [N, K/32] (fp16 bits).
* fp4:  codes uint8 [N, K/2] (E2M1, sign in bit 3), scale uint8 [N, K/32] (e8m0).
* int8: codes int8 [N, K], scale uint16 [N, K/32].
* km4:  codes uint8 [N, K/2] (4-bit indices), lut uint16 [N, 16] (fp16 bits).
* int4aff: codes uint8 [N, K/2] (u in 0..15), plane uint32 [N, K/32] (fp16 scale | fp16 bias << 16).
* int8km: codes uint8 [N, K] (8-bit indices), lut uint16 [N/32, 256] (fp16 bits), N % 32 == 0.
* km4 + int8 outliers: km4 codes and tables of the row with its P largest-magnitude
  entries zeroed, plus ocol uint16 [N, P] (increasing), oval int8 [N, P], oscale uint16 [N].
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

FMT_INT4, FMT_FP4, FMT_INT8, FMT_KM4, FMT_INT4AFF, FMT_INT8KM = 0, 1, 2, 3, 4, 5
FORMATS = {"int4": FMT_INT4, "fp4": FMT_FP4, "int8": FMT_INT8, "km4": FMT_KM4, "int4aff": FMT_INT4AFF,
           "int8km": FMT_INT8KM}

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
               "-fopenmp", "-shared", "-fPIC", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        ci = ctypes.c_int
        L.orc_f16_to_f64.restype = ctypes.c_double
        L.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_f64_to_f16.restype = ctypes.c_uint16
        L.orc_f64_to_f16.argtypes = [ctypes.c_double]
        L.orc_pack_fp4.argtypes = [P, i64, i64, P, P]
        L.orc_pack_int4.argtypes = [P, i64, i64, ci, P, P]
        L.orc_pack_int8.argtypes = [P, i64, i64, P, P]
        L.orc_pack_int4aff.argtypes = [P, i64, i64, P, P]
        L.orc_pack_km4.argtypes = [P, i64, i64, ci, P, P, P]
        L.orc_pack_int8km.argtypes = [P, i64, i64, ci, P, P, P]
        L.orc_pack_km4o.argtypes = [P, i64, i64, ci, ci, P, P, P, P, P]
        L.orc_matvec_km4o.argtypes = [P, P, P, P, P, i64, i64, ci, P, ci, P]
        L.orc_dequant.argtypes = [ci, P, P, i64, i64, P]
        L.orc_matvec.argtypes = [ci, P, P, i64, i64, P, ci, P, i64, P]
        L.orc_moe_route.argtypes = [P, ci, ci, ci, P, P]
        L.orc_pack_int8_rows.argtypes = [P, i64, i64, P, P]
        L.orc_embed_gather_int8.argtypes = [P, P, i64, i64, P, i64, P]
        L.orc_moe_ffn.argtypes = [ci, P, P, P, P, ci, i64, i64, P, ci, ci, P, P, P, P]
        L.orc_num_threads.argtypes = []
        L.orc_num_threads.restype = ci
        L.orc_set_num_threads.argtypes = [ci]
        L.orc_set_num_threads.restype = None
        for f in ("orc_pack_fp4", "orc_pack_int4", "orc_pack_int8", "orc_pack_km4",
                  "orc_dequant", "orc_matvec", "orc_moe_route", "orc_moe_ffn"):
            getattr(L, f).restype = None
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _as_f32(W) -> np.ndarray:
    """fp16 and fp32 weights both enter the packers as exact fp32 values."""
    return np.ascontiguousarray(np.asarray(W).astype(np.float32))


def _check_shape(W):
    N, K = W.shape
    if K % 32 != 0:
        raise ValueError("K must be a multiple of 32")
    return N, K


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().orc_num_threads())


def set_num_threads(n: int) -> None:
    """Set the OpenMP thread count (results do not depend on it)."""
    lib().orc_set_num_threads(int(n))


# --- scalar fp16 helpers (written from the binary16 definition in oracle.c) ---

def f16_to_f64(bits: int) -> float:
    return lib().orc_f16_to_f64(int(bits) & 0xFFFF)


def f64_to_f16(v: float) -> int:
    return int(lib().orc_f64_to_f16(float(v)))


# --- packers ---

def pack_fp4(W):
    W = _as_f32(W)
    N, K = _check_shape(W)
    codes = np.zeros((N, K // 2), np.uint8)
    scale = np.zeros((N, K // 32), np.uint8)
    lib().orc_pack_fp4(_p(W), N, K, _p(codes), _p(scale))
    return codes, scale


def pack_int4(W, clip_search: bool = True):
    W = _as_f32(W)
    N, K = _check_shape(W)
    codes = np.zeros((N, K // 2), np.uint8)
    scale = np.zeros((N, K // 32), np.uint16)
    lib().orc_pack_int4(_p(W), N, K, 7 if clip_search else 1, _p(codes), _p(scale))
    return codes, scale


def pack_int8(W):
    W = _as_f32(W)
    N, K = _check_shape(W)
    codes = np.zeros((N, K), np.int8)
    scale = np.zeros((N, K // 32), np.uint16)
    lib().orc_pack_int8(_p(W), N, K, _p(codes), _p(scale))
    return codes, scale


def pack_int4aff(W):
    """codes [N, K/2] uint8 (u in 0..15, element 2j low nibble), plane [N, K/32]
    uint32 (fp16 scale low half, fp16 bias high half)."""
    W = _as_f32(W)
    N, K = _check_shape(W)
    codes = np.zeros((N, K // 2), np.uint8)
    plane = np.zeros((N, K // 32), np.uint32)
    lib().orc_pack_int4aff(_p(W), N, K, _p(codes), _p(plane))
    return codes, plane


def pack_km4(W_f16, max_iter: int = 20, return_iters: bool = False):
    W = np.ascontiguousarray(np.asarray(W_f16, dtype=np.float16)).view(np.uint16)
    N, K = _check_shape(W)
    codes = np.zeros((N, K // 2), np.uint8)
    lut = np.zeros((N, 16), np.uint16)
    iters = np.zeros((N,), np.int32)
    lib().orc_pack_km4(_p(W), N, K, int(max_iter), _p(codes), _p(lut), _p(iters))
    if return_iters:
        return codes, lut, iters
    return codes, lut


def pack_int8km(W_f16, max_iter: int = 20, return_iters: bool = False):
    """W [N, K] fp16 (N % 32 == 0) -> codes uint8 [N, K] (indices), lut uint16
    [N/32, 256] (fp16 bits): one 256-entry table per group of 32 rows."""
    W = np.ascontiguousarray(np.asarray(W_f16, dtype=np.float16)).view(np.uint16)
    N, K = _check_shape(W)
    assert N % 32 == 0, "int8km groups 32 rows"
    codes = np.zeros((N, K), np.uint8)
    lut = np.zeros((N // 32, 256), np.uint16)
    iters = np.zeros((N // 32,), np.int32)
    lib().orc_pack_int8km(_p(W), N, K, int(max_iter), _p(codes), _p(lut), _p(iters))
    if return_iters:
        return codes, lut, iters
    return codes, lut


def pack_km4o(W_f16, P: int, max_iter: int = 20):
    """4-bit k-means rows plus P int8 outliers per row. Returns (codes uint8
    [N, K/2], lut uint16 [N, 16], ocol uint16 [N, P], oval int8 [N, P],
    oscale uint16 [N] fp16 bits)."""
    W = np.ascontiguousarray(np.asarray(W_f16, dtype=np.float16)).view(np.uint16)
    N, K = _check_shape(W)
    assert 0 <= P <= K
    codes = np.zeros((N, K // 2), np.uint8)
    lut = np.zeros((N, 16), np.uint16)
    ocol = np.zeros((N, P), np.uint16)
    oval = np.zeros((N, P), np.int8)
    oscale = np.zeros((N,), np.uint16)
    lib().orc_pack_km4o(_p(W), N, K, int(P), int(max_iter), _p(codes), _p(lut), _p(ocol), _p(oval), _p(oscale))
    return codes, lut, ocol, oval, oscale


def matvec_km4o(codes, lut, ocol, oval, oscale, x) -> np.ndarray:
    """y [B, N] = W_hat x in fp64, W_hat = table value + outlier (if any)."""
    codes, lut = np.ascontiguousarray(codes), np.ascontiguousarray(lut, dtype=np.uint16)
    ocol = np.ascontiguousarray(ocol, dtype=np.uint16)
    oval = np.ascontiguousarray(oval, dtype=np.int8)
    oscale = np.ascontiguousarray(oscale, dtype=np.uint16)
    N, K = codes.shape[0], codes.shape[1] * 2
    P = ocol.shape[1]
    x = np.ascontiguousarray(np.atleast_2d(np.asarray(x)).astype(np.float64))
    assert x.shape[1] == K and ocol.shape == (N, P) and oval.shape == (N, P)
    B = x.shape[0]
    y = np.zeros((B, N), np.float64)
    lib().orc_matvec_km4o(_p(codes), _p(lut), _p(ocol), _p(oval), _p(oscale), N, K, int(P), _p(x), B, _p(y))
    return y


def pack(fmt: str, W, **kw):
    return {"int4": pack_int4, "fp4": pack_fp4, "int8": pack_int8, "km4": pack_km4,
            "int4aff": pack_int4aff, "int8km": pack_int8km}[fmt](W, **kw)


# --- dequant and matvec ---

def _kdim(fmt: str, codes: np.ndarray) -> int:
    return codes.shape[1] if fmt in ("int8", "int8km") else codes.shape[1] * 2


def dequant(fmt: str, codes, plane) -> np.ndarray:
    codes = np.ascontiguousarray(codes)
    plane = np.ascontiguousarray(plane)
    N, K = codes.shape[0], _kdim(fmt, codes)
    out = np.zeros((N, K), np.float64)
    lib().orc_dequant(FORMATS[fmt], _p(codes), _p(plane), N, K, _p(out))
    return out


def matvec(fmt: str, codes, plane, x, rows=None) -> np.ndarray:
    """y[b, i] = sum_k dequant(W)[row_i, k] * x[b, k], fp64 sequential sum.

    x: [B, K] (any float dtype, converted exactly to fp64). rows: optional
    index array; then y is [B, len(rows)].
    """
    codes = np.ascontiguousarray(codes)
    plane = np.ascontiguousarray(plane)
    N, K = codes.shape[0], _kdim(fmt, codes)
    x = np.ascontiguousarray(np.atleast_2d(np.asarray(x)).astype(np.float64))
    assert x.shape[1] == K
    B = x.shape[0]
    if rows is None:
        M, rp, nr = N, None, 0
    else:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        assert rows.min() >= 0 and rows.max() < N
        M, rp, nr = len(rows), _p(rows), len(rows)
    y = np.zeros((B, M), np.float64)
    lib().orc_matvec(FORMATS[fmt], _p(codes), _p(plane), N, K, _p(x), B, rp, nr, _p(y))
    return y


def matvec_argmax(fmt: str, codes, plane, x):
    """Largest entry of each batch row of matvec(...) and its row index (the
    lowest index among equal largest values), from the fp64 products."""
    y = matvec(fmt, codes, plane, x)
    idx = np.argmax(y, axis=1)   # first occurrence of the maximum
    return idx.astype(np.int64), y[np.arange(y.shape[0]), idx]


# --- embedding table: int8 per-row scale, dequant-gather ---

def pack_int8_rows(W):
    """W [V, H] (fp16 or fp32, converted exactly to fp32) -> codes int8 [V, H],
    scale fp16 bits uint16 [V]."""
    W = np.ascontiguousarray(np.asarray(W).astype(np.float32))
    V, H = W.shape
    codes = np.zeros((V, H), np.int8)
    scale = np.zeros(V, np.uint16)
    lib().orc_pack_int8_rows(_p(W), V, H, _p(codes), _p(scale))
    return codes, scale


def embed_gather_int8(codes, scale, ids):
    """out [T, H] fp16 bits (uint16) = fp16(codes[ids] * scale[ids]); an id
    outside [0, V) gives a zero row."""
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    scale = np.ascontiguousarray(scale, dtype=np.uint16)
    ids = np.ascontiguousarray(np.asarray(ids).reshape(-1), dtype=np.int32)
    V, H = codes.shape
    out = np.zeros((len(ids), H), np.uint16)
    lib().orc_embed_gather_int8(_p(codes), _p(scale), V, H, _p(ids), len(ids), _p(out))
    return out


# --- mixture of experts ---

def moe_route(logits, topk: int):
    logits = np.ascontiguousarray(np.asarray(logits, dtype=np.float32))
    T, E = logits.shape
    ids = np.zeros((T, topk), np.int32)
    w = np.zeros((T, topk), np.float64)
    lib().orc_moe_route(_p(logits), T, E, topk, _p(ids), _p(w))
    return ids, w


def moe_ffn(gu_codes, gu_plane, dn_codes, dn_plane, x, ids, weights, return_h: bool = False, fmt: str = "int4"):
    """gu_*: E stacked [2I, H] matrices packed in `fmt` (codes [E, 2I, ...],
    plane [E, 2I, ...]); dn_*: E stacked [H, I] matrices."""
    gu_codes = np.ascontiguousarray(gu_codes)
    gu_plane = np.ascontiguousarray(gu_plane)
    dn_codes = np.ascontiguousarray(dn_codes)
    dn_plane = np.ascontiguousarray(dn_plane)
    E, I2 = gu_codes.shape[:2]
    I, H = I2 // 2, _kdim(fmt, gu_codes[0])
    assert dn_codes.shape[:2] == (E, H) and _kdim(fmt, dn_codes[0]) == I
    x = np.ascontiguousarray(np.atleast_2d(np.asarray(x)).astype(np.float64))
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    weights = np.ascontiguousarray(weights, dtype=np.float64)
    T, topk = ids.shape
    assert ids.min() >= 0 and ids.max() < E
    y = np.zeros((T, H), np.float64)
    h = np.zeros((T, topk, I), np.float64)
    lib().orc_moe_ffn(FORMATS[fmt], _p(gu_codes), _p(gu_plane), _p(dn_codes), _p(dn_plane), E, H, I,
                      _p(x), T, topk, _p(ids), _p(weights), _p(h), _p(y))
    return (y, h) if return_h else y
