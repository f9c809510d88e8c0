"""The Python binding refuses tensors whose shape, dtype, layout or device the
C ABI cannot see, before any pointer reaches the library (CPU only: every case
here raises before the library is loaded)."""
import pytest
import torch

import quantized_decode_matvec_amd as qmv

f16, f32, u8, u16, i32 = torch.float16, torch.float32, torch.uint8, torch.uint16, torch.int32


def z(*shape, dtype=f16):
    return torch.zeros(shape, dtype=dtype)


def raises(exc, match, fn, *a, **kw):
    with pytest.raises(exc, match=match):
        fn(*a, **kw)


# --------------------------------------------------------------- packers

@pytest.mark.parametrize("name", ["qpack_int4", "qpack_fp4", "qpack_int8", "qpack_int4aff", "qpack_km4"])
def test_packers_check_weights(name):
    fn = getattr(qmv, name)
    raises(ValueError, "GPU memory", fn, z(64, 64))                      # valid shapes, CPU tensor
    raises(ValueError, "multiple of 32", fn, z(64, 48))
    raises(ValueError, r"\[N, K\]", fn, z(64))
    raises(ValueError, "contiguous", fn, z(64, 128)[:, ::2])
    raises(TypeError, "dtype", fn, z(64, 64, dtype=torch.float64))


def test_packers_check_outputs():
    raises(ValueError, "codes has shape", qmv.qpack_int4, z(64, 64), codes=z(64, 16, dtype=u8))
    raises(ValueError, "plane has shape", qmv.qpack_int4, z(64, 64), scale=z(64, 1, dtype=u16))
    raises(TypeError, "1-byte|2-byte|elements", qmv.qpack_int4, z(64, 64), scale=z(64, 2, dtype=u8))
    raises(ValueError, "plane has shape", qmv.qpack_km4, z(8, 64), lut=z(8, 15, dtype=u16))
    raises(TypeError, "dtype", qmv.qpack_km4, z(8, 64, dtype=f32))
    raises(ValueError, "multiple of 32", qmv.qpack_int8km, z(40, 64))
    raises(ValueError, "lut has shape", qmv.qpack_int8km, z(64, 64), lut=z(1, 256, dtype=u16))
    raises(ValueError, "scale has shape", qmv.qpack_int8_rows, z(10, 16), scale=z(9, dtype=u16))


# --------------------------------------------------------------- matvec

PLANES = {"int4": (lambda N, K: z(N, K // 32, dtype=u16)), "fp4": (lambda N, K: z(N, K // 32, dtype=u8)),
          "int8": (lambda N, K: z(N, K // 32, dtype=u16)), "km4": (lambda N, K: z(N, 16, dtype=u16)),
          "int4aff": (lambda N, K: z(N, K // 32, dtype=i32)), "int8km": (lambda N, K: z(N // 32, 256, dtype=u16))}


def codes_for(fmt, N, K):
    return z(N, K if fmt in ("int8", "int8km") else K // 2, dtype=u8)


@pytest.mark.parametrize("fmt", sorted(PLANES))
def test_matvec_checks(fmt):
    N, K = 64, 128
    c, p = codes_for(fmt, N, K), PLANES[fmt](N, K)
    x = z(2, K)
    raises(ValueError, "GPU memory", qmv.qmatvec, fmt, c, p, x)           # everything right but the device
    raises(ValueError, "x has shape", qmv.qmatvec, fmt, c, p, z(2, K - 32))
    raises(ValueError, "x has shape", qmv.qmatvec, fmt, c, p, z(2, 1, K))
    raises(ValueError, "contiguous", qmv.qmatvec, fmt, c, p, z(K, 2).t())
    raises(TypeError, "dtype", qmv.qmatvec, fmt, c, p, z(2, K, dtype=torch.bfloat16))
    raises(ValueError, "plane holds", qmv.qmatvec, fmt, c, PLANES[fmt](N // 2, K), x)
    raises(ValueError, "contiguous", qmv.qmatvec, fmt, c, torch.cat([p, p], 1)[:, ::2], x)
    raises(ValueError, "codes has 1 dimensions", qmv.qmatvec, fmt, c.reshape(-1), p, x)
    raises(ValueError, "y has shape", qmv.qmatvec, fmt, c, p, x, y=z(2, N - 1, dtype=f32))
    raises(TypeError, "dtype", qmv.qmatvec, fmt, c, p, x, y=z(2, N, dtype=f16))
    raises(ValueError, "contiguous", qmv.qmatvec, fmt, c, p, x, y=z(N, 2, dtype=f32).t())
    raises(ValueError, "plane holds", qmv.qdequant, fmt, c, PLANES[fmt](N // 2, K))
    raises(ValueError, "out has shape", qmv.qdequant, fmt, c, p, out=z(N, K - 1, dtype=f32))


@pytest.mark.parametrize("fmt", ["km4", "int4"])
def test_prepared_matvec_checks_once_like_matvec(fmt):
    N, K = 64, 128
    c, p = codes_for(fmt, N, K), PLANES[fmt](N, K)
    x = z(2, K)
    raises(ValueError, "GPU memory", qmv.qmatvec_call, fmt, c, p, x)
    raises(ValueError, "plane holds", qmv.qmatvec_call, fmt, c, PLANES[fmt](N // 2, K), x)
    raises(ValueError, "y has shape", qmv.qmatvec_call, fmt, c, p, x, y=z(2, N - 1, dtype=f32))
    raises(ValueError, "x has shape", qmv.qmatvec_call, fmt, c, p, z(2, K - 32))


def test_km4o_checks():
    N, K, P = 16, 64, 4
    c, l = codes_for("km4", N, K), PLANES["km4"](N, K)
    oc, ov, os_ = z(N, P, dtype=u16), z(N, P, dtype=torch.int8), z(N, dtype=u16)
    raises(ValueError, "GPU memory", qmv.qmatvec_km4o, c, l, oc, ov, os_, z(1, K))
    raises(ValueError, "oval has shape", qmv.qmatvec_km4o, c, l, oc, z(N, P + 1, dtype=torch.int8), os_, z(1, K))
    raises(ValueError, "oscale has shape", qmv.qmatvec_km4o, c, l, oc, ov, z(N - 1, dtype=u16), z(1, K))
    raises(ValueError, "x has shape", qmv.qmatvec_km4o, c, l, oc, ov, os_, z(1, K + 32))


def test_argmax_checks():
    N, K = 64, 128
    c, p = codes_for("fp4", N, K), PLANES["fp4"](N, K)
    raises(ValueError, "GPU memory", qmv.qmatvec_argmax, "fp4", c, p, z(2, K))
    raises(TypeError, "dtype", qmv.qmatvec_argmax, "fp4", c, p, z(2, K, dtype=f32))   # fp16 x only
    raises(ValueError, "x has shape", qmv.qmatvec_argmax, "fp4", c, p, z(2, K // 2))
    raises(ValueError, "idx has shape", qmv.qmatvec_argmax, "fp4", c, p, z(2, K), idx=z(3, dtype=i32))
    raises(ValueError, "unknown format", qmv.qmatvec_argmax, "fp5", c, p, z(2, K))


# --------------------------------------------------------------- MoE and embedding

def test_moe_checks():
    E, N, K, T, topk = 8, 64, 128, 2, 2
    c, p = z(E, N, K // 2, dtype=u8), z(E, N, K // 32, dtype=u16)
    ids, w = z(T, topk, dtype=i32), z(T, topk, dtype=f32)
    x = z(T, K)
    raises(ValueError, "GPU memory", qmv.gather_qmatvec, "int4", c, p, x, ids)
    raises(ValueError, "x has shape", qmv.gather_qmatvec, "int4", c, p, z(T, K - 32), ids)
    raises(ValueError, "x has shape", qmv.gather_qmatvec, "int4", c, p, x, ids, x_per_slot=True)
    raises(TypeError, "dtype", qmv.gather_qmatvec, "int4", c, p, x, ids.long())
    raises(ValueError, "plane holds", qmv.gather_qmatvec, "int4", c, z(E, N // 2, K // 32, dtype=u16), x, ids)
    raises(ValueError, "first dimension", qmv.gather_qmatvec, "int4", c, p[:4], x, ids)
    raises(ValueError, "needs weights", qmv.gather_qmatvec, "int4", c, p, x, ids, epi="combine")
    raises(ValueError, "weights has shape", qmv.gather_qmatvec, "int4", c, p, x, ids, weights=z(T, 1, dtype=f32),
           epi="combine")
    raises(ValueError, "y has shape", qmv.gather_qmatvec, "int4", c, p, x, ids, epi="swiglu",
           y=z(T, topk, N, dtype=f16))
    raises(ValueError, "unknown epilogue", qmv.gather_qmatvec, "int4", c, p, x, ids, epi="gelu")
    # the layer
    H, I = 128, 64
    guc, gup = z(E, 2 * I, H // 2, dtype=u8), z(E, 2 * I, H // 32, dtype=u16)
    dnc, dnp = z(E, H, I // 2, dtype=u8), z(E, H, I // 32, dtype=u16)
    lg = z(T, E, dtype=f32)
    raises(ValueError, "GPU memory", qmv.qmoe_ffn, "int4", guc, gup, dnc, dnp, z(T, H), lg, topk)
    raises(ValueError, "x has shape", qmv.qmoe_ffn, "int4", guc, gup, dnc, dnp, z(T, H + 32), lg, topk)
    raises(ValueError, "logits has shape", qmv.qmoe_ffn, "int4", guc, gup, dnc, dnp, z(T, H), z(T, E - 1, dtype=f32),
           topk)
    raises(ValueError, "do not match|must hold", qmv.qmoe_ffn, "int4", guc, gup, z(E, H, I, dtype=u8), dnp, z(T, H),
           lg, topk)
    raises(ValueError, "dn_plane holds", qmv.qmoe_ffn, "int4", guc, gup, dnc, z(E, H, 1, dtype=u16), z(T, H), lg, topk)
    raises(ValueError, "h has shape", qmv.qmoe_ffn, "int4", guc, gup, dnc, dnp, z(T, H), lg, topk,
           h=z(T, topk, I + 1))
    raises(TypeError, "dtype", qmv.qmoe_route, z(T, E), topk)             # fp32 logits only


def test_embedding_and_stream_checks():
    q, s = z(100, 64, dtype=torch.int8), z(100, dtype=u16)
    raises(ValueError, "GPU memory", qmv.qembed_gather_int8, q, s, z(3, dtype=i32))
    raises(ValueError, "scale has shape", qmv.qembed_gather_int8, q, z(99, dtype=u16), z(3, dtype=i32))
    raises(TypeError, "dtype", qmv.qembed_gather_int8, q, s, z(3, dtype=torch.int64))
    raises(ValueError, "out has shape", qmv.qembed_gather_int8, q, s, z(3, dtype=i32), out=z(3, 63))


def test_tiled_km4_checks():
    N, K = 100, 2048
    t, lut, x = z(128 * K // 2, dtype=u8), z(N, 16, dtype=u16), z(1, K)
    assert qmv.qtile_km4_bytes(N, K) == 128 * K // 2
    raises(ValueError, "GPU memory", qmv.qmatvec_km4_tiled, t, lut, x)            # all right but the device
    raises(ValueError, "GPU memory", qmv.qmatvec_km4_tiled, t, lut, z(4, K))      # batch 4 is accepted too
    raises(ValueError, "tiled has shape", qmv.qmatvec_km4_tiled, z(N * K // 2, dtype=u8), lut, x)   # unpadded
    raises(ValueError, "lut has shape", qmv.qmatvec_km4_tiled, t, z(N, 15, dtype=u16), x)
    raises(TypeError, "dtype", qmv.qmatvec_km4_tiled, t, lut, z(1, K, dtype=f32))
    raises(ValueError, r"1 <= B <= 4", qmv.qmatvec_km4_tiled, t, lut, z(5, K))
    raises(ValueError, "K = 1280", qmv.qmatvec_km4_tiled, z(128 * 640, dtype=u8), lut, z(1, 1280))
    raises(ValueError, "contiguous", qmv.qmatvec_km4_tiled, t, lut, z(1, 2 * K)[:, ::2])
    raises(ValueError, "GPU memory", qmv.qtile_km4, z(N, K // 2, dtype=u8))
    raises(ValueError, "tiled has shape", qmv.qtile_km4, z(N, K // 2, dtype=u8), tiled=z(N * K // 2, dtype=u8))


def test_tiled_argmax_checks():
    N, K = 100, 2048
    t, lut = z(128 * K // 2, dtype=u8), z(N, 16, dtype=u16)
    raises(ValueError, "GPU memory", qmv.qmatvec_argmax_km4_tiled, t, lut, z(1, K))
    raises(ValueError, "1 <= B <= 4", qmv.qmatvec_argmax_km4_tiled, t, lut, z(6, K))
    raises(ValueError, "tiled has shape", qmv.qmatvec_argmax_km4_tiled, z(N * K // 2, dtype=u8), lut, z(1, K))
