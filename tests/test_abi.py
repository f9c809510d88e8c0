"""The C ABI library loads, exports every symbol include/qmv.h declares, and
refuses invalid arguments before anything is launched (no GPU needed: every
call below fails validation, so no device memory is touched)."""
import ctypes
import os
import re

import pytest

import quantized_decode_matvec_amd as qmv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmv.h")

OK, E_NULL, E_SHAPE, E_ALIGN, E_DTYPE, E_WORKSPACE = 0, 1, 2, 3, 4, 5


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(qmv.LIB_PATH):
        import quantized_decode_matvec_amd.build as b
        b.build()
    return qmv.lib()


def test_header_declares_exactly_the_exports():
    assert _declared() == sorted(qmv.EXPORTS)


def test_every_declared_symbol_is_exported(L):
    for name in _declared():
        assert hasattr(L, name), name


def test_status_strings(L):
    for s in range(7):
        assert L.qmv_status_string(s).decode().startswith("QMV_")
    assert L.qmv_status_string(99) == b"unknown qmv_status"


FAKE = ctypes.c_void_p(0x10000)       # aligned, never dereferenced
ODD = ctypes.c_void_p(0x10001)        # misaligned
NUL = ctypes.c_void_p(0)
S = ctypes.c_void_p(0)


def test_pack_validation(L):
    assert L.qpack_int4(NUL, 1, 4, 64, FAKE, FAKE, S) == E_NULL
    assert L.qpack_int4(FAKE, 1, 4, 48, FAKE, FAKE, S) == E_SHAPE      # K % 32
    assert L.qpack_int4(FAKE, 1, 0, 64, FAKE, FAKE, S) == E_SHAPE      # N < 1
    assert L.qpack_int4(FAKE, 7, 4, 64, FAKE, FAKE, S) == E_DTYPE
    assert L.qpack_int4(ODD, 1, 4, 64, FAKE, FAKE, S) == E_ALIGN
    assert L.qpack_fp4(FAKE, 1, 4, 64, NUL, FAKE, S) == E_NULL
    assert L.qpack_int8(FAKE, 0, 4, 64, ODD, FAKE, S) == E_ALIGN
    assert L.qpack_km4(FAKE, 4, 8192, 20, FAKE, FAKE, S) == E_SHAPE    # K too large for the row sort
    assert L.qpack_km4(FAKE, 4, 64, 0, FAKE, FAKE, S) == E_SHAPE       # max_iter < 1
    half = ctypes.c_void_p(0x10002)   # 2-byte aligned: too little for the 32-bit scale + bias words
    assert L.qpack_int4aff(FAKE, 1, 4, 48, FAKE, FAKE, S) == E_SHAPE
    assert L.qpack_int4aff(FAKE, 1, 4, 64, FAKE, half, S) == E_ALIGN
    assert L.qmatvec_int4aff(FAKE, half, 8, 64, FAKE, 1, 1, FAKE, S) == E_ALIGN
    assert L.qdequant(6, FAKE, FAKE, 4, 64, FAKE, S) == E_DTYPE        # one past the last format
    # int8km: rows in groups of 32, K <= 2048 for the packer, max_iter >= 1, 4-byte tables
    assert L.qpack_int8km(FAKE, 48, 64, 20, FAKE, FAKE, S) == E_SHAPE
    assert L.qpack_int8km(FAKE, 64, 4096, 20, FAKE, FAKE, S) == E_SHAPE
    assert L.qpack_int8km(FAKE, 64, 64, 0, FAKE, FAKE, S) == E_SHAPE
    assert L.qpack_int8km(FAKE, 64, 64, 20, FAKE, half, S) == E_ALIGN
    assert L.qpack_int8km(NUL, 64, 64, 20, FAKE, FAKE, S) == E_NULL
    assert L.qmatvec_int8km(FAKE, FAKE, 40, 64, FAKE, 1, 1, FAKE, S) == E_SHAPE
    assert L.qmatvec_int8km(FAKE, half, 64, 64, FAKE, 1, 1, FAKE, S) == E_ALIGN
    assert L.qdequant(5, FAKE, FAKE, 40, 64, FAKE, S) == E_SHAPE
    # km4 + outliers: nout range, K limit for packing, NULL outlier arrays only with nout == 0
    assert L.qpack_km4o(FAKE, 8, 64, 300, 20, FAKE, FAKE, FAKE, FAKE, FAKE, S) == E_SHAPE
    assert L.qpack_km4o(FAKE, 8, 64, 65, 20, FAKE, FAKE, FAKE, FAKE, FAKE, S) == E_SHAPE
    assert L.qpack_km4o(FAKE, 8, 8192, 4, 20, FAKE, FAKE, FAKE, FAKE, FAKE, S) == E_SHAPE
    assert L.qpack_km4o(FAKE, 8, 64, 4, 20, FAKE, FAKE, NUL, FAKE, FAKE, S) == E_NULL
    assert L.qmatvec_km4o(FAKE, FAKE, FAKE, FAKE, FAKE, 8, 64, -1, FAKE, 1, 1, FAKE, S) == E_SHAPE
    assert L.qmatvec_km4o(FAKE, FAKE, NUL, NUL, NUL, 8, 64, 0, FAKE, 1, 1, FAKE, S) == E_NULL   # oscale needed
    assert L.qmatvec_km4o(FAKE, FAKE, ODD, FAKE, FAKE, 8, 64, 2, FAKE, 1, 1, FAKE, S) == E_ALIGN
    TWO = ctypes.c_void_p(0x10002)    # 2-byte aligned table: read as 32-bit words, refused
    assert L.qmatvec_km4o(FAKE, TWO, FAKE, FAKE, FAKE, 8, 64, 2, FAKE, 1, 1, FAKE, S) == E_ALIGN
    assert L.qmatvec_km4(FAKE, TWO, 8, 64, FAKE, 1, 1, FAKE, S) == E_ALIGN


@pytest.mark.parametrize("name", ["qmatvec_int4", "qmatvec_fp4", "qmatvec_int8", "qmatvec_km4", "qmatvec_int4aff",
                                  "qmatvec_int8km"])
def test_matvec_validation(L, name):
    f = getattr(L, name)
    assert f(NUL, FAKE, 8, 64, FAKE, 1, 1, FAKE, S) == E_NULL
    assert f(FAKE, FAKE, 8, 64, FAKE, 1, 0, FAKE, S) == E_SHAPE        # B = 0
    assert f(FAKE, FAKE, 8, 64, FAKE, 1, 9, FAKE, S) == E_SHAPE        # B = 9
    assert f(FAKE, FAKE, 8, 80, FAKE, 1, 1, FAKE, S) == E_SHAPE        # K % 32
    assert f(FAKE, FAKE, 8, 64, FAKE, 5, 1, FAKE, S) == E_DTYPE
    assert f(ODD, FAKE, 8, 64, FAKE, 1, 1, FAKE, S) == E_ALIGN
    assert f(FAKE, FAKE, 8, 64, ODD, 1, 1, FAKE, S) == E_ALIGN


def test_dequant_and_moe_validation(L):
    assert L.qdequant(9, FAKE, FAKE, 4, 64, FAKE, S) == E_DTYPE
    assert L.qdequant(0, FAKE, FAKE, 4, 33, FAKE, S) == E_SHAPE
    assert L.qmoe_route(FAKE, 2, 256, 0, FAKE, FAKE, S) == E_SHAPE
    assert L.qmoe_route(FAKE, 2, 4, 8, FAKE, FAKE, S) == E_SHAPE       # topk > E
    assert L.qmoe_route(NUL, 2, 256, 8, FAKE, FAKE, S) == E_NULL
    # gather: T > 8, combine without weights, int8 K > 4096, bad epilogue, fp32 x
    g = L.gather_qmatvec
    assert g(0, FAKE, FAKE, 256, 2048, 512, FAKE, 1, 1, 9, 8, FAKE, FAKE, 2, FAKE, NUL, 0, S) == E_SHAPE
    assert g(0, FAKE, FAKE, 256, 2048, 512, FAKE, 1, 1, 4, 8, FAKE, NUL, 2, FAKE, NUL, 0, S) == E_NULL
    assert g(2, FAKE, FAKE, 256, 2048, 8192, FAKE, 1, 1, 4, 8, FAKE, FAKE, 0, FAKE, NUL, 0, S) == E_SHAPE
    assert g(0, FAKE, FAKE, 256, 2048, 512, FAKE, 1, 1, 4, 8, FAKE, FAKE, 7, FAKE, NUL, 0, S) == E_DTYPE
    assert g(0, FAKE, FAKE, 256, 2048, 512, FAKE, 0, 1, 4, 8, FAKE, FAKE, 0, FAKE, NUL, 0, S) == E_DTYPE
    assert g(0, FAKE, FAKE, 256, 1023, 512, FAKE, 1, 0, 4, 8, FAKE, FAKE, 1, FAKE, NUL, 0, S) == E_SHAPE  # odd N
    for epi in (0, 1, 2):
        assert L.gather_qmatvec_workspace_bytes(4, 8, 256, 2048, epi) == 0
    # fused MoE layer: fmt, null output, T > 8, topk > E, H not a multiple of 32, int8 I > 4096, misaligned h
    f = L.qmoe_ffn
    args = [0, FAKE, FAKE, FAKE, FAKE, 256, 2048, 512, FAKE, FAKE, 4, 8, FAKE, FAKE, FAKE, FAKE, S]

    def call(**kw):
        a = list(args)
        for k, v in kw.items():
            a[int(k[1:])] = v
        return f(*a)
    assert call(a0=7) == E_DTYPE
    assert call(a15=NUL) == E_NULL
    assert call(a10=9) == E_SHAPE
    assert call(a5=4) == E_SHAPE
    assert call(a6=2047) == E_SHAPE
    assert call(a0=2, a7=8192) == E_SHAPE
    assert call(a14=ODD) == E_ALIGN
    assert L.qmv_stream_read(FAKE, 24, FAKE, S) == E_SHAPE


def test_argmax_and_embedding_validation(L):
    A = L.qmatvec_argmax
    ws = L.qmatvec_argmax_workspace_bytes(1000, 2)
    assert ws >= 128 + 1000 * 2 * 4   # header + y [2][1000] fp32
    assert L.qmatvec_argmax_workspace_bytes(1000, 9) == 0
    # B > 8, K = 8192 int4 at B = 8 (beyond the dot-path register budget), missing workspace, misaligned x
    assert A(0, FAKE, FAKE, 1000, 2048, FAKE, 9, FAKE, FAKE, FAKE, ws, S) == E_SHAPE
    assert A(0, FAKE, FAKE, 1000, 8192, FAKE, 8, FAKE, FAKE, FAKE, 1 << 30, S) == E_SHAPE
    assert A(3, FAKE, FAKE, 1000, 2048, FAKE, 2, FAKE, FAKE, NUL, 0, S) == E_WORKSPACE
    assert A(3, FAKE, FAKE, 1000, 2048, FAKE, 2, FAKE, FAKE, FAKE, ws - 8, S) == E_WORKSPACE
    assert A(3, FAKE, FAKE, 1000, 2048, ODD, 2, FAKE, FAKE, FAKE, ws, S) == E_ALIGN
    assert A(3, FAKE, FAKE, 1000, 2048, NUL, 2, FAKE, FAKE, FAKE, ws, S) == E_NULL
    # embedding: H not a multiple of 8, negative T, misaligned out, null scale
    G = L.qembed_gather_int8
    assert G(FAKE, FAKE, 100, 12, FAKE, 3, FAKE, S) == E_SHAPE
    assert G(FAKE, FAKE, 100, 16, FAKE, -1, FAKE, S) == E_SHAPE
    assert G(FAKE, FAKE, 100, 16, FAKE, 3, ODD, S) == E_ALIGN
    assert G(FAKE, NUL, 100, 16, FAKE, 3, FAKE, S) == E_NULL
    assert G(FAKE, FAKE, 100, 16, NUL, 3, FAKE, S) == E_NULL
    assert G(FAKE, FAKE, 100, 16, NUL, 0, NUL, S) == 0          # T = 0: nothing to do
    assert L.qpack_int8_rows(FAKE, 5, 10, 16, FAKE, FAKE, S) == E_DTYPE
    assert L.qpack_int8_rows(FAKE, 0, 0, 16, FAKE, FAKE, S) == E_SHAPE


def test_tiled_km4_validation(L):
    half = ctypes.c_void_p(0x10002)
    assert L.qtile_km4_bytes(100, 2048) == 128 * 1024        # rows padded to whole 64-row tiles
    assert L.qtile_km4_bytes(64, 512) == 64 * 256
    assert L.qtile_km4_bytes(0, 2048) == 0 and L.qtile_km4_bytes(4, 48) == 0
    assert L.qtile_km4(NUL, 4, 64, FAKE, S) == E_NULL
    assert L.qtile_km4(FAKE, 4, 48, FAKE, S) == E_SHAPE
    assert L.qtile_km4(FAKE, 4, 64, ODD, S) == E_ALIGN
    assert L.qmatvec_km4_tiled(NUL, FAKE, 64, 2048, FAKE, 1, 1, FAKE, S) == E_NULL
    assert L.qmatvec_km4_tiled(FAKE, FAKE, 64, 2048, FAKE, 0, 1, FAKE, S) == E_DTYPE   # fp32 x
    assert L.qmatvec_km4_tiled(FAKE, FAKE, 64, 2048, FAKE, 1, 5, FAKE, S) == E_SHAPE   # batch 1..4
    assert L.qmatvec_km4_tiled(FAKE, FAKE, 64, 2048, FAKE, 1, 0, FAKE, S) == E_SHAPE
    assert L.qmatvec_km4_tiled(FAKE, FAKE, 64, 1280, FAKE, 1, 1, FAKE, S) == E_SHAPE   # K not a tile width
    assert L.qmatvec_km4_tiled(FAKE, FAKE, 64, 4608, FAKE, 1, 1, FAKE, S) == E_SHAPE   # K past 4096
    assert L.qmatvec_km4_tiled(FAKE, FAKE, 64, 8192, FAKE, 1, 1, FAKE, S) == E_SHAPE
    assert L.qmatvec_km4_tiled(FAKE, half, 64, 2048, FAKE, 1, 1, FAKE, S) == E_ALIGN   # 32-bit table words


def test_tiled_argmax_validation(L):
    ws = ctypes.c_size_t(1 << 20)
    assert L.qmatvec_argmax_km4_tiled(NUL, FAKE, 64, 2048, FAKE, 1, FAKE, FAKE, FAKE, ws, S) == E_NULL
    assert L.qmatvec_argmax_km4_tiled(FAKE, FAKE, 64, 1280, FAKE, 1, FAKE, FAKE, FAKE, ws, S) == E_SHAPE
    assert L.qmatvec_argmax_km4_tiled(FAKE, FAKE, 64, 2048, FAKE, 5, FAKE, FAKE, FAKE, ws, S) == E_SHAPE
    assert L.qmatvec_argmax_km4_tiled(FAKE, FAKE, 64, 2048, FAKE, 1, FAKE, FAKE, FAKE, ctypes.c_size_t(64), S) \
        == E_WORKSPACE
    assert L.qmatvec_argmax_km4_tiled(FAKE, FAKE, 64, 2048, FAKE, 1, FAKE, FAKE, NUL, ws, S) == E_WORKSPACE
    assert L.qmatvec_argmax_km4_tiled(ODD, FAKE, 64, 2048, FAKE, 1, FAKE, FAKE, FAKE, ws, S) == E_ALIGN


def test_tiled_km4o_validation(L):
    assert L.qmatvec_km4o_tiled(FAKE, FAKE, FAKE, FAKE, NUL, 64, 2048, 4, FAKE, 1, 1, FAKE, S) == E_NULL
    assert L.qmatvec_km4o_tiled(FAKE, FAKE, NUL, FAKE, FAKE, 64, 2048, 4, FAKE, 1, 1, FAKE, S) == E_NULL
    assert L.qmatvec_km4o_tiled(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 2048, 4, FAKE, 0, 1, FAKE, S) == E_DTYPE
    assert L.qmatvec_km4o_tiled(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 2048, 300, FAKE, 1, 1, FAKE, S) == E_SHAPE
    assert L.qmatvec_km4o_tiled(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 1280, 4, FAKE, 1, 1, FAKE, S) == E_SHAPE
    assert L.qmatvec_km4o_tiled(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 2048, 4, FAKE, 1, 5, FAKE, S) == E_SHAPE
    assert L.qmatvec_km4o_tiled(FAKE, FAKE, ODD, FAKE, FAKE, 64, 2048, 4, FAKE, 1, 1, FAKE, S) == E_ALIGN
