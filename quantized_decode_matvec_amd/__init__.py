"""Block-quantized decode matvec for AMD MI355X (gfx950).

Thin ctypes binding over ``libqmv.so`` (the C ABI declared in
``include/qmv.h``). Every function has the C entry point's name and does
argument marshalling only: torch tensors supply device memory and the current
HIP stream; all arithmetic runs in the library's kernels. There is no CPU
fallback: if the library is missing or a call fails, an exception is raised.

Build the library with ``python -m quantized_decode_matvec_amd.build``.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqmv.so")

QMV_F32, QMV_F16 = 0, 1
QMV_INT4, QMV_FP4, QMV_INT8, QMV_KM4, QMV_INT4AFF, QMV_INT8KM = 0, 1, 2, 3, 4, 5
QMV_EPI_NONE, QMV_EPI_SWIGLU, QMV_EPI_COMBINE = 0, 1, 2
FORMATS = {"int4": QMV_INT4, "fp4": QMV_FP4, "int8": QMV_INT8, "km4": QMV_KM4, "int4aff": QMV_INT4AFF,
           "int8km": QMV_INT8KM}
EPILOGUES = {"none": QMV_EPI_NONE, "swiglu": QMV_EPI_SWIGLU, "combine": QMV_EPI_COMBINE}

# every symbol include/qmv.h declares
EXPORTS = ("qmv_status_string", "qpack_int4", "qpack_fp4", "qpack_int8", "qpack_km4", "qpack_int4aff",
           "qpack_int8km", "qmatvec_int4", "qmatvec_fp4", "qmatvec_int8", "qmatvec_km4", "qmatvec_int4aff",
           "qmatvec_int8km", "qpack_km4o", "qmatvec_km4o", "qdequant",
           "qmoe_route", "gather_qmatvec_workspace_bytes", "gather_qmatvec", "qmoe_ffn",
           "qmatvec_argmax_workspace_bytes", "qmatvec_argmax", "qpack_int8_rows", "qembed_gather_int8",
           "qmv_stream_read_sink_words", "qmv_stream_read")


class QmvError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__("%s failed: %s" % (fn, msg))
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libqmv.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libqmv.so not found at %s; build it with "
                              "`python -m quantized_decode_matvec_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, i64, ci, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        sigs = {
            "qmv_status_string": ([ci], ctypes.c_char_p),
            "qpack_int4": ([P, ci, i64, i64, P, P, P], ci),
            "qpack_fp4": ([P, ci, i64, i64, P, P, P], ci),
            "qpack_int8": ([P, ci, i64, i64, P, P, P], ci),
            "qpack_km4": ([P, i64, i64, ci, P, P, P], ci),
            "qpack_int4aff": ([P, ci, i64, i64, P, P, P], ci),
            "qpack_int8km": ([P, i64, i64, ci, P, P, P], ci),
            "qmatvec_int4": ([P, P, i64, i64, P, ci, ci, P, P], ci),
            "qmatvec_fp4": ([P, P, i64, i64, P, ci, ci, P, P], ci),
            "qmatvec_int8": ([P, P, i64, i64, P, ci, ci, P, P], ci),
            "qmatvec_km4": ([P, P, i64, i64, P, ci, ci, P, P], ci),
            "qmatvec_int4aff": ([P, P, i64, i64, P, ci, ci, P, P], ci),
            "qmatvec_int8km": ([P, P, i64, i64, P, ci, ci, P, P], ci),
            "qpack_km4o": ([P, i64, i64, ci, ci, P, P, P, P, P, P], ci),
            "qmatvec_km4o": ([P, P, P, P, P, i64, i64, ci, P, ci, ci, P, P], ci),
            "qdequant": ([ci, P, P, i64, i64, P, P], ci),
            "qmoe_route": ([P, ci, ci, ci, P, P, P], ci),
            "gather_qmatvec_workspace_bytes": ([ci, ci, ci, i64, ci], sz),
            "gather_qmatvec": ([ci, P, P, ci, i64, i64, P, ci, ci, ci, ci, P, P, ci, P, P, sz, P], ci),
            "qmoe_ffn": ([ci, P, P, P, P, ci, i64, i64, P, P, ci, ci, P, P, P, P, P], ci),
            "qmatvec_argmax_workspace_bytes": ([i64, ci], sz),
            "qmatvec_argmax": ([ci, P, P, i64, i64, P, ci, P, P, P, sz, P], ci),
            "qpack_int8_rows": ([P, ci, i64, i64, P, P, P], ci),
            "qembed_gather_int8": ([P, P, i64, i64, P, i64, P, P], ci),
            "qmv_stream_read_sink_words": ([sz], sz),
            "qmv_stream_read": ([P, sz, P, P], ci),
        }
        for name, (args, res) in sigs.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _check(fn, status):
    if status != 0:
        msg = lib().qmv_status_string(status).decode()
        raise QmvError(fn, status, msg)


def _torch():
    import torch
    return torch


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _dt(t):
    torch = _torch()
    if t.dtype == torch.float16:
        return QMV_F16
    if t.dtype == torch.float32:
        return QMV_F32
    raise TypeError("expected an fp16 or fp32 tensor, got %s" % t.dtype)


def _empty(shape, dtype, like):
    return _torch().empty(shape, dtype=dtype, device=like.device)


# ---------------------------------------------------------------- packing

def qpack_int4(W, codes=None, scale=None, stream=None):
    torch = _torch()
    N, K = W.shape
    codes = _empty((N, K // 2), torch.uint8, W) if codes is None else codes
    scale = _empty((N, K // 32), torch.uint16, W) if scale is None else scale
    _check("qpack_int4", lib().qpack_int4(_ptr(W), _dt(W), N, K, _ptr(codes), _ptr(scale), _stream(stream)))
    return codes, scale


def qpack_fp4(W, codes=None, scale=None, stream=None):
    torch = _torch()
    N, K = W.shape
    codes = _empty((N, K // 2), torch.uint8, W) if codes is None else codes
    scale = _empty((N, K // 32), torch.uint8, W) if scale is None else scale
    _check("qpack_fp4", lib().qpack_fp4(_ptr(W), _dt(W), N, K, _ptr(codes), _ptr(scale), _stream(stream)))
    return codes, scale


def qpack_int8(W, codes=None, scale=None, stream=None):
    torch = _torch()
    N, K = W.shape
    codes = _empty((N, K), torch.int8, W) if codes is None else codes
    scale = _empty((N, K // 32), torch.uint16, W) if scale is None else scale
    _check("qpack_int8", lib().qpack_int8(_ptr(W), _dt(W), N, K, _ptr(codes), _ptr(scale), _stream(stream)))
    return codes, scale


def qpack_km4(W, max_iter=20, codes=None, lut=None, stream=None):
    torch = _torch()
    if W.dtype != torch.float16:
        raise TypeError("qpack_km4 takes fp16 weights")
    N, K = W.shape
    codes = _empty((N, K // 2), torch.uint8, W) if codes is None else codes
    lut = _empty((N, 16), torch.uint16, W) if lut is None else lut
    _check("qpack_km4", lib().qpack_km4(_ptr(W), N, K, int(max_iter), _ptr(codes), _ptr(lut), _stream(stream)))
    return codes, lut


def qpack_int4aff(W, codes=None, plane=None, stream=None):
    """W [N, K] -> (codes uint8 [N, K/2], plane uint32-as-int32 [N, K/32]: fp16 scale | fp16 bias << 16)."""
    torch = _torch()
    N, K = W.shape
    codes = _empty((N, K // 2), torch.uint8, W) if codes is None else codes
    plane = _empty((N, K // 32), torch.int32, W) if plane is None else plane
    _check("qpack_int4aff", lib().qpack_int4aff(_ptr(W), _dt(W), N, K, _ptr(codes), _ptr(plane), _stream(stream)))
    return codes, plane


def qpack_int8km(W, max_iter=20, codes=None, lut=None, stream=None):
    """W fp16 [N, K], N % 32 == 0 -> (codes uint8 [N, K], lut uint16 [N/32, 256])."""
    torch = _torch()
    if W.dtype != torch.float16:
        raise TypeError("qpack_int8km takes fp16 weights")
    N, K = W.shape
    codes = _empty((N, K), torch.uint8, W) if codes is None else codes
    lut = _empty((N // 32, 256), torch.uint16, W) if lut is None else lut
    _check("qpack_int8km", lib().qpack_int8km(_ptr(W), N, K, int(max_iter), _ptr(codes), _ptr(lut), _stream(stream)))
    return codes, lut


def qpack(fmt, W, **kw):
    return {"int4": qpack_int4, "fp4": qpack_fp4, "int8": qpack_int8, "km4": qpack_km4,
            "int4aff": qpack_int4aff, "int8km": qpack_int8km}[fmt](W, **kw)


# ---------------------------------------------------------------- matvec

def _kdim(fmt, codes):
    return codes.shape[-1] if fmt in ("int8", "int8km") else codes.shape[-1] * 2


def _matvec(name, fmt, codes, plane, x, y, stream):
    torch = _torch()
    N, K = codes.shape[0], _kdim(fmt, codes)
    x2 = x if x.dim() == 2 else x.view(1, -1)
    B = x2.shape[0]
    y = _empty((B, N), torch.float32, codes) if y is None else y
    fn = getattr(lib(), name)
    _check(name, fn(_ptr(codes), _ptr(plane), N, K, _ptr(x2), _dt(x2), B, _ptr(y), _stream(stream)))
    return y


def qmatvec_int4(codes, scale, x, y=None, stream=None):
    return _matvec("qmatvec_int4", "int4", codes, scale, x, y, stream)


def qmatvec_fp4(codes, scale, x, y=None, stream=None):
    return _matvec("qmatvec_fp4", "fp4", codes, scale, x, y, stream)


def qmatvec_int8(codes, scale, x, y=None, stream=None):
    return _matvec("qmatvec_int8", "int8", codes, scale, x, y, stream)


def qmatvec_km4(codes, lut, x, y=None, stream=None):
    return _matvec("qmatvec_km4", "km4", codes, lut, x, y, stream)


def qmatvec_int4aff(codes, plane, x, y=None, stream=None):
    return _matvec("qmatvec_int4aff", "int4aff", codes, plane, x, y, stream)


def qmatvec_int8km(codes, lut, x, y=None, stream=None):
    return _matvec("qmatvec_int8km", "int8km", codes, lut, x, y, stream)


def qpack_km4o(W, nout, max_iter=20, stream=None):
    """W fp16 [N, K] -> (codes [N, K/2] uint8, lut [N, 16] uint16, ocol [N, nout]
    uint16, oval [N, nout] int8, oscale [N] uint16): 4-bit k-means rows plus
    nout int8 outliers per row."""
    torch = _torch()
    if W.dtype != torch.float16:
        raise TypeError("qpack_km4o takes fp16 weights")
    N, K = W.shape
    codes = _empty((N, K // 2), torch.uint8, W)
    lut = _empty((N, 16), torch.uint16, W)
    ocol = _empty((N, nout), torch.uint16, W)
    oval = _empty((N, nout), torch.int8, W)
    oscale = _empty((N,), torch.uint16, W)
    _check("qpack_km4o", lib().qpack_km4o(_ptr(W), N, K, int(nout), int(max_iter), _ptr(codes), _ptr(lut),
                                          _ptr(ocol), _ptr(oval), _ptr(oscale), _stream(stream)))
    return codes, lut, ocol, oval, oscale


def qmatvec_km4o(codes, lut, ocol, oval, oscale, x, y=None, stream=None):
    torch = _torch()
    N, K = codes.shape[0], codes.shape[1] * 2
    nout = ocol.shape[1]
    x2 = x if x.dim() == 2 else x.view(1, -1)
    B = x2.shape[0]
    y = _empty((B, N), torch.float32, codes) if y is None else y
    _check("qmatvec_km4o", lib().qmatvec_km4o(_ptr(codes), _ptr(lut), _ptr(ocol), _ptr(oval), _ptr(oscale), N, K,
                                              int(nout), _ptr(x2), _dt(x2), B, _ptr(y), _stream(stream)))
    return y


def qmatvec(fmt, codes, plane, x, y=None, stream=None):
    return _matvec("qmatvec_" + fmt, fmt, codes, plane, x, y, stream)


def qdequant(fmt, codes, plane, out=None, stream=None):
    torch = _torch()
    N, K = codes.shape[0], _kdim(fmt, codes)
    out = _empty((N, K), torch.float32, codes) if out is None else out
    _check("qdequant", lib().qdequant(FORMATS[fmt], _ptr(codes), _ptr(plane), N, K, _ptr(out), _stream(stream)))
    return out


# ---------------------------------------------------------------- MoE

def qmoe_route(logits, topk, ids=None, weights=None, stream=None):
    torch = _torch()
    T, E = logits.shape
    ids = _empty((T, topk), torch.int32, logits) if ids is None else ids
    weights = _empty((T, topk), torch.float32, logits) if weights is None else weights
    _check("qmoe_route", lib().qmoe_route(_ptr(logits), T, E, topk, _ptr(ids), _ptr(weights), _stream(stream)))
    return ids, weights


def gather_qmatvec_workspace_bytes(T, topk, E, N, epi):
    return int(lib().gather_qmatvec_workspace_bytes(T, topk, E, N, EPILOGUES.get(epi, epi)))


def gather_qmatvec(fmt, codes, plane, x, ids, weights=None, epi="none", x_per_slot=False,
                   y=None, workspace=None, stream=None):
    """codes/plane: [E, N, ...] stacked experts; x [T, K] or [T, topk, K] (fp16)."""
    torch = _torch()
    E, N = codes.shape[0], codes.shape[1]
    K = _kdim(fmt, codes)
    T, topk = ids.shape
    e = EPILOGUES[epi]
    if y is None:
        if e == QMV_EPI_NONE:
            y = _empty((T, topk, N), torch.float32, codes)
        elif e == QMV_EPI_SWIGLU:
            y = _empty((T, topk, N // 2), torch.float16, codes)
        else:
            y = _empty((T, N), torch.float32, codes)
    need = gather_qmatvec_workspace_bytes(T, topk, E, N, e)
    if need and workspace is None:
        workspace = _empty((need,), torch.uint8, codes)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("gather_qmatvec", lib().gather_qmatvec(
        FORMATS[fmt], _ptr(codes), _ptr(plane), E, N, K, _ptr(x), _dt(x), 1 if x_per_slot else 0,
        T, topk, _ptr(ids), _ptr(weights), e, _ptr(y), _ptr(workspace), ws_bytes, _stream(stream)))
    return y


def qmoe_ffn(fmt, gu_codes, gu_plane, dn_codes, dn_plane, x, logits, topk, ids=None, weights=None, h=None,
             y=None, stream=None):
    """One decode MoE layer (routing, gate/up + SwiGLU, down + weighted combine).

    gu_codes/gu_plane: [E, 2I, ...]; dn_codes/dn_plane: [E, H, ...]; x [T, H]
    fp16; logits [T, E] fp32. Returns (y [T, H] fp32, ids, weights, h).
    """
    torch = _torch()
    E, I2 = gu_codes.shape[0], gu_codes.shape[1]
    H = dn_codes.shape[1]
    I = I2 // 2
    T = x.shape[0]
    ids = _empty((T, topk), torch.int32, x) if ids is None else ids
    weights = _empty((T, topk), torch.float32, x) if weights is None else weights
    h = _empty((T, topk, I), torch.float16, x) if h is None else h
    y = _empty((T, H), torch.float32, x) if y is None else y
    _check("qmoe_ffn", lib().qmoe_ffn(
        FORMATS[fmt], _ptr(gu_codes), _ptr(gu_plane), _ptr(dn_codes), _ptr(dn_plane), E, H, I,
        _ptr(logits), _ptr(x), T, topk, _ptr(ids), _ptr(weights), _ptr(h), _ptr(y), _stream(stream)))
    return y, ids, weights, h


def moe_ffn(gu_codes, gu_scale, dn_codes, dn_scale, x, logits, topk, fmt="int4", stream=None):
    """The same layer as three separate calls: route, gate/up + SwiGLU gather, down + combine gather."""
    ids, w = qmoe_route(logits, topk, stream=stream)
    h = gather_qmatvec(fmt, gu_codes, gu_scale, x, ids, epi="swiglu", stream=stream)
    return gather_qmatvec(fmt, dn_codes, dn_scale, h, ids, weights=w, epi="combine", x_per_slot=True,
                          stream=stream), ids, w


# ---------------------------------------------------------------- around the lm_head

def qmatvec_argmax_workspace_bytes(N, B):
    return int(lib().qmatvec_argmax_workspace_bytes(N, B))


def qmatvec_argmax(fmt, codes, plane, x, idx=None, val=None, workspace=None, stream=None):
    """Fused matvec + argmax: (idx int32 [B], val fp32 [B]) of the largest y per batch row."""
    torch = _torch()
    N, K = codes.shape[0], _kdim(fmt, codes)
    x2 = x if x.dim() == 2 else x.view(1, -1)
    B = x2.shape[0]
    idx = _empty((B,), torch.int32, codes) if idx is None else idx
    val = _empty((B,), torch.float32, codes) if val is None else val
    if workspace is None:
        workspace = _empty((qmatvec_argmax_workspace_bytes(N, B),), torch.uint8, codes)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("qmatvec_argmax", lib().qmatvec_argmax(
        FORMATS[fmt], _ptr(codes), _ptr(plane), N, K, _ptr(x2), B, _ptr(idx), _ptr(val),
        _ptr(workspace), ws_bytes, _stream(stream)))
    return idx, val


def qpack_int8_rows(W, codes=None, scale=None, stream=None):
    """Embedding table W [V, H] -> (codes int8 [V, H], scale fp16 bits uint16 [V])."""
    torch = _torch()
    V, H = W.shape
    codes = _empty((V, H), torch.int8, W) if codes is None else codes
    scale = _empty((V,), torch.uint16, W) if scale is None else scale
    _check("qpack_int8_rows", lib().qpack_int8_rows(_ptr(W), _dt(W), V, H, _ptr(codes), _ptr(scale),
                                                    _stream(stream)))
    return codes, scale


def qembed_gather_int8(codes, scale, ids, out=None, stream=None):
    """out fp16 [T, H] = fp16(codes[ids] * scale[ids])."""
    torch = _torch()
    V, H = codes.shape
    T = ids.numel()
    out = _empty((T, H), torch.float16, codes) if out is None else out
    _check("qembed_gather_int8", lib().qembed_gather_int8(_ptr(codes), _ptr(scale), V, H, _ptr(ids), T,
                                                          _ptr(out), _stream(stream)))
    return out


# ---------------------------------------------------------------- measurement aid

def qmv_stream_read(buf, sink=None, stream=None):
    torch = _torch()
    nbytes = buf.numel() * buf.element_size()
    words = int(lib().qmv_stream_read_sink_words(nbytes))
    sink = _empty((words,), torch.int32, buf) if sink is None else sink
    _check("qmv_stream_read", lib().qmv_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(stream)))
    return sink
