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
           "qmatvec_argmax_workspace_bytes", "qmatvec_argmax", "qmatvec_argmax_noalloc",
           "qmatvec_argmax_noalloc_max_bytes", "qpack_int8_rows", "qembed_gather_int8",
           "qmv_stream_read_sink_words", "qmv_stream_read", "qtile_km4_bytes", "qtile_km4",
           "qmatvec_km4_tiled", "qmatvec_argmax_km4_tiled", "qmatvec_km4o_tiled")


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
        # torch carries its own HIP runtime (libamdhip64.so, soname libamdhip64.so.7).
        # Load it first, so that our library's dependency on that soname binds to
        # the runtime torch uses: loaded the other way round, the process holds two
        # HIP runtimes and ours finds no device.
        _torch()
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
            "qmatvec_argmax_noalloc": ([ci, P, P, i64, i64, P, ci, P, P, P], ci),
            "qmatvec_argmax_noalloc_max_bytes": ([], sz),
            "qpack_int8_rows": ([P, ci, i64, i64, P, P, P], ci),
            "qembed_gather_int8": ([P, P, i64, i64, P, i64, P, P], ci),
            "qmv_stream_read_sink_words": ([sz], sz),
            "qmv_stream_read": ([P, sz, P, P], ci),
            "qtile_km4_bytes": ([i64, i64], sz),
            "qtile_km4": ([P, i64, i64, P, P], ci),
            "qmatvec_km4_tiled": ([P, P, i64, i64, P, ci, ci, P, P], ci),
            "qmatvec_argmax_km4_tiled": ([P, P, i64, i64, P, ci, P, P, P, sz, P], ci),
            "qmatvec_km4o_tiled": ([P, P, P, P, P, i64, i64, ci, P, ci, ci, P, P], ci),
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


# ---------------------------------------------------------------- argument checks
#
# The C ABI receives bare pointers and sizes, so it cannot see a tensor's shape,
# strides, dtype or device. Every wrapper checks those here, before any pointer
# reaches the library: a short or strided buffer would otherwise be read or
# written past its end on the GPU.

def _bad(fn, msg):
    raise ValueError("%s: %s" % (fn, msg))


def _tensor(fn, name, t, shape=None, itemsize=None, dtypes=None, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s: %s must be a torch.Tensor, got %s" % (fn, name, type(t).__name__))
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError("%s: %s has dtype %s, expected one of %s" % (fn, name, t.dtype, ", ".join(map(str, dtypes))))
    if itemsize is not None and t.element_size() != itemsize:
        raise TypeError("%s: %s has %d-byte elements, expected %d" % (fn, name, t.element_size(), itemsize))
    if ndim is not None and t.dim() != ndim:
        _bad(fn, "%s has %d dimensions, expected %d" % (name, t.dim(), ndim))
    if shape is not None and tuple(t.shape) != tuple(shape):
        _bad(fn, "%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if not t.is_contiguous():
        _bad(fn, "%s must be contiguous" % name)
    return t


def _nbytes(t):
    return t.numel() * t.element_size()


def _plane_bytes(fn, name, t, want):
    if _nbytes(t) != want:
        _bad(fn, "%s holds %d bytes, expected %d" % (name, _nbytes(t), want))


def _on_gpu(fn, *ts):
    devs = {t.device for t in ts if t is not None}
    if len(devs) != 1:
        _bad(fn, "tensors are on different devices: %s" % sorted(map(str, devs)))
    d = devs.pop()
    if d.type != "cuda":
        _bad(fn, "tensors must be in GPU memory, got device %s" % d)


def _fp(fn, name, t, allow_f32=True):
    torch = _torch()
    ok = (torch.float16, torch.float32) if allow_f32 else (torch.float16,)
    return _tensor(fn, name, t, dtypes=ok)


def _plane_row_bytes(fmt, K):
    """Bytes of the scale/table plane per row of K weights."""
    return {"int4": K // 16, "fp4": K // 32, "int8": K // 16, "km4": 32, "int4aff": K // 8,
            "int8km": 16}[fmt]


def _as_batch(fn, x, K, allow_f32=True):
    """x [K] or [B, K] -> [B, K] view."""
    _fp(fn, "x", x, allow_f32)
    if x.dim() == 1:
        x = x.view(1, -1)
    if x.dim() != 2 or x.shape[1] != K:
        _bad(fn, "x has shape %s, expected [B, %d] or [%d]" % (tuple(x.shape), K, K))
    return x


def _codes2d(fn, fmt, codes):
    _tensor(fn, "codes", codes, itemsize=1, ndim=2)
    K = codes.shape[1] if fmt in ("int8", "int8km") else codes.shape[1] * 2
    return codes.shape[0], K


# ---------------------------------------------------------------- packing

def _pack_args(fn, W, codes, plane, code_cols, plane_cols, plane_item, code_dtype, plane_dtype, allow_f32=True):
    torch = _torch()
    _fp(fn, "W", W, allow_f32)
    if W.dim() != 2:
        _bad(fn, "W must be [N, K], got shape %s" % (tuple(W.shape),))
    N, K = W.shape
    if K % 32 != 0:
        _bad(fn, "K = %d is not a multiple of 32" % K)
    codes = _empty((N, code_cols(K)), code_dtype, W) if codes is None else codes
    plane = _empty((N, plane_cols(K)), plane_dtype, W) if plane is None else plane
    _tensor(fn, "codes", codes, shape=(N, code_cols(K)), itemsize=1)
    _tensor(fn, "plane", plane, shape=(N, plane_cols(K)), itemsize=plane_item)
    _on_gpu(fn, W, codes, plane)
    return N, K, codes, plane


def qpack_int4(W, codes=None, scale=None, stream=None):
    torch = _torch()
    N, K, codes, scale = _pack_args("qpack_int4", W, codes, scale, lambda K: K // 2, lambda K: K // 32, 2,
                                    torch.uint8, torch.uint16)
    _check("qpack_int4", lib().qpack_int4(_ptr(W), _dt(W), N, K, _ptr(codes), _ptr(scale), _stream(stream)))
    return codes, scale


def qpack_fp4(W, codes=None, scale=None, stream=None):
    torch = _torch()
    N, K, codes, scale = _pack_args("qpack_fp4", W, codes, scale, lambda K: K // 2, lambda K: K // 32, 1,
                                    torch.uint8, torch.uint8)
    _check("qpack_fp4", lib().qpack_fp4(_ptr(W), _dt(W), N, K, _ptr(codes), _ptr(scale), _stream(stream)))
    return codes, scale


def qpack_int8(W, codes=None, scale=None, stream=None):
    torch = _torch()
    N, K, codes, scale = _pack_args("qpack_int8", W, codes, scale, lambda K: K, lambda K: K // 32, 2,
                                    torch.int8, torch.uint16)
    _check("qpack_int8", lib().qpack_int8(_ptr(W), _dt(W), N, K, _ptr(codes), _ptr(scale), _stream(stream)))
    return codes, scale


def qpack_km4(W, max_iter=20, codes=None, lut=None, stream=None):
    torch = _torch()
    N, K, codes, lut = _pack_args("qpack_km4", W, codes, lut, lambda K: K // 2, lambda K: 16, 2,
                                  torch.uint8, torch.uint16, allow_f32=False)
    _check("qpack_km4", lib().qpack_km4(_ptr(W), N, K, int(max_iter), _ptr(codes), _ptr(lut), _stream(stream)))
    return codes, lut


def qpack_int4aff(W, codes=None, plane=None, stream=None):
    """W [N, K] -> (codes uint8 [N, K/2], plane uint32-as-int32 [N, K/32]: fp16 scale | fp16 bias << 16)."""
    torch = _torch()
    N, K, codes, plane = _pack_args("qpack_int4aff", W, codes, plane, lambda K: K // 2, lambda K: K // 32, 4,
                                    torch.uint8, torch.int32)
    _check("qpack_int4aff", lib().qpack_int4aff(_ptr(W), _dt(W), N, K, _ptr(codes), _ptr(plane), _stream(stream)))
    return codes, plane


def qpack_int8km(W, max_iter=20, codes=None, lut=None, stream=None):
    """W fp16 [N, K], N % 32 == 0 -> (codes uint8 [N, K], lut uint16 [N/32, 256])."""
    torch = _torch()
    _fp("qpack_int8km", "W", W, allow_f32=False)
    if W.dim() != 2 or W.shape[0] % 32 != 0:
        _bad("qpack_int8km", "W must be [N, K] with N a multiple of 32, got shape %s" % (tuple(W.shape),))
    N, K = W.shape
    codes = _empty((N, K), torch.uint8, W) if codes is None else codes
    lut = _empty((N // 32, 256), torch.uint16, W) if lut is None else lut
    _tensor("qpack_int8km", "codes", codes, shape=(N, K), itemsize=1)
    _tensor("qpack_int8km", "lut", lut, shape=(N // 32, 256), itemsize=2)
    _on_gpu("qpack_int8km", W, codes, lut)
    _check("qpack_int8km", lib().qpack_int8km(_ptr(W), N, K, int(max_iter), _ptr(codes), _ptr(lut), _stream(stream)))
    return codes, lut


def qpack(fmt, W, **kw):
    return {"int4": qpack_int4, "fp4": qpack_fp4, "int8": qpack_int8, "km4": qpack_km4,
            "int4aff": qpack_int4aff, "int8km": qpack_int8km}[fmt](W, **kw)


# ---------------------------------------------------------------- matvec

def _kdim(fmt, codes):
    return codes.shape[-1] if fmt in ("int8", "int8km") else codes.shape[-1] * 2


def _dense_plane(fn, fmt, plane, N, K):
    _tensor(fn, "plane", plane)
    if fmt == "int8km" and N % 32 != 0:
        _bad(fn, "int8km needs N % 32 == 0, got N = %d" % N)
    _plane_bytes(fn, "plane", plane, N * _plane_row_bytes(fmt, K))


def _y_out(fn, y, shape, dtype, like, name="y"):
    if y is None:
        return _empty(shape, dtype, like)
    _tensor(fn, name, y, shape=shape, dtypes=(dtype,))
    return y


def _matvec_args(name, fmt, codes, plane, x, y):
    """Checked arguments of a matvec call (all but the stream) and its output."""
    torch = _torch()
    N, K = _codes2d(name, fmt, codes)
    _dense_plane(name, fmt, plane, N, K)
    x2 = _as_batch(name, x, K)
    B = x2.shape[0]
    y = _y_out(name, y, (B, N), torch.float32, codes)
    _on_gpu(name, codes, plane, x2, y)
    return (_ptr(codes), _ptr(plane), N, K, _ptr(x2), _dt(x2), B, _ptr(y)), (codes, plane, x2), y


def _matvec(name, fmt, codes, plane, x, y, stream):
    args, _, y = _matvec_args(name, fmt, codes, plane, x, y)
    _check(name, getattr(lib(), name)(*args, _stream(stream)))
    return y


def qmatvec_call(fmt, codes, plane, x, y=None, stream=None):
    """Check the arguments of qmatvec(fmt, codes, plane, x, y) once and return a
    function of no arguments that launches that same matvec (same buffers,
    output y) each time it is called, on `stream` or else on the current
    stream: for a decode loop that calls one matvec many times, without the
    per-call checks. The returned function keeps the tensors alive; their
    contents may change between calls, their storage must not."""
    name = "qmatvec_" + fmt
    args, keep, y = _matvec_args(name, fmt, codes, plane, x, y)
    fn = getattr(lib(), name)
    st = None if stream is None else ctypes.c_void_p(stream)
    torch = _torch()

    def call():
        _check(name, fn(*args, st if st is not None else ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)))
        return y

    call.tensors = keep + (y,)
    return call


def qmatvec_int4(codes, scale, x, y=None, stream=None):
    return _matvec("qmatvec_int4", "int4", codes, scale, x, y, stream)


def qmatvec_fp4(codes, scale, x, y=None, stream=None):
    return _matvec("qmatvec_fp4", "fp4", codes, scale, x, y, stream)


def qmatvec_int8(codes, scale, x, y=None, stream=None):
    return _matvec("qmatvec_int8", "int8", codes, scale, x, y, stream)


def qmatvec_km4(codes, lut, x, y=None, stream=None):
    return _matvec("qmatvec_km4", "km4", codes, lut, x, y, stream)


def qtile_km4_bytes(N, K):
    """Bytes of the row-tiled km4 code plane: whole 64-row tiles of K/2 bytes
    per row (the size qtile_km4_bytes in the C ABI returns)."""
    if N < 1 or K < 32 or K % 32:
        _bad("qtile_km4_bytes", "N = %d, K = %d is out of range" % (N, K))
    return (N + 63) // 64 * 64 * (K // 2)


def qtile_km4(codes, tiled=None, stream=None):
    """km4 codes [N, K/2] -> the row-tiled plane (uint8, qtile_km4_bytes(N, K)
    bytes) that qmatvec_km4_tiled reads."""
    torch = _torch()
    fn = "qtile_km4"
    N, K = _codes2d(fn, "km4", codes)
    nb = qtile_km4_bytes(N, K)
    tiled = _empty((nb,), torch.uint8, codes) if tiled is None else tiled
    _tensor(fn, "tiled", tiled, shape=(nb,), itemsize=1)
    _on_gpu(fn, codes, tiled)
    _check(fn, lib().qtile_km4(_ptr(codes), N, K, _ptr(tiled), _stream(stream)))
    return tiled


_NO_Y = object()   # _tiled_args: the caller has no y (the fused argmax)


def _tiled_args(fn, tiled, lut, x, y):
    torch = _torch()
    _tensor(fn, "lut", lut, itemsize=2, ndim=2)
    N = lut.shape[0]
    _tensor(fn, "lut", lut, shape=(N, 16))
    _fp(fn, "x", x, allow_f32=False)
    x2 = x.view(1, -1) if x.dim() == 1 else x
    if x2.dim() != 2 or not 1 <= x2.shape[0] <= 4:
        _bad(fn, "x must be [K] or [B, K] with 1 <= B <= 4, got shape %s" % (tuple(x.shape),))
    B, K = x2.shape
    if K < 512 or K > 4096 or K % 512:
        _bad(fn, "K = %d: the tiled kernel takes K a multiple of 512 up to 4096" % K)
    _tensor(fn, "tiled", tiled, shape=(qtile_km4_bytes(N, K),), itemsize=1)
    if y is _NO_Y:
        _on_gpu(fn, tiled, lut, x2)
        return (_ptr(tiled), _ptr(lut), N, K, _ptr(x2), QMV_F16, B, None), (tiled, lut, x2), None
    y = _y_out(fn, y, (B, N), torch.float32, tiled)
    _on_gpu(fn, tiled, lut, x2, y)
    return (_ptr(tiled), _ptr(lut), N, K, _ptr(x2), QMV_F16, B, _ptr(y)), (tiled, lut, x2), y


def qmatvec_km4_tiled(tiled, lut, x, y=None, stream=None):
    """km4 matvec from the row-tiled plane: x fp16 [K] or [B, K], 1 <= B <= 4 -> y fp32 [B, N]."""
    fn = "qmatvec_km4_tiled"
    args, _, y = _tiled_args(fn, tiled, lut, x, y)
    _check(fn, lib().qmatvec_km4_tiled(*args, _stream(stream)))
    return y


def qmatvec_km4_tiled_call(tiled, lut, x, y=None, stream=None):
    """qmatvec_km4_tiled with the argument checks done once: returns a function
    of no arguments that launches the same call (see qmatvec_call)."""
    fn = "qmatvec_km4_tiled"
    args, keep, y = _tiled_args(fn, tiled, lut, x, y)
    f = lib().qmatvec_km4_tiled
    st = None if stream is None else ctypes.c_void_p(stream)
    torch = _torch()

    def call():
        _check(fn, f(*args, st if st is not None else ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)))
        return y

    call.tensors = keep + (y,)
    return call


def qmatvec_int4aff(codes, plane, x, y=None, stream=None):
    return _matvec("qmatvec_int4aff", "int4aff", codes, plane, x, y, stream)


def qmatvec_int8km(codes, lut, x, y=None, stream=None):
    return _matvec("qmatvec_int8km", "int8km", codes, lut, x, y, stream)


def qpack_km4o(W, nout, max_iter=20, stream=None):
    """W fp16 [N, K] -> (codes [N, K/2] uint8, lut [N, 16] uint16, ocol [N, nout]
    uint16, oval [N, nout] int8, oscale [N] uint16): 4-bit k-means rows plus
    nout int8 outliers per row."""
    torch = _torch()
    _fp("qpack_km4o", "W", W, allow_f32=False)
    if W.dim() != 2:
        _bad("qpack_km4o", "W must be [N, K], got shape %s" % (tuple(W.shape),))
    _on_gpu("qpack_km4o", W)
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
    fn = "qmatvec_km4o"
    N, K = _codes2d(fn, "km4", codes)
    _dense_plane(fn, "km4", lut, N, K)
    _tensor(fn, "ocol", ocol, itemsize=2, ndim=2)
    nout = ocol.shape[1]
    _tensor(fn, "ocol", ocol, shape=(N, nout))
    _tensor(fn, "oval", oval, shape=(N, nout), itemsize=1)
    _tensor(fn, "oscale", oscale, shape=(N,), itemsize=2)
    x2 = _as_batch(fn, x, K)
    B = x2.shape[0]
    y = _y_out(fn, y, (B, N), torch.float32, codes)
    _on_gpu(fn, codes, lut, ocol, oval, oscale, x2, y)
    _check("qmatvec_km4o", lib().qmatvec_km4o(_ptr(codes), _ptr(lut), _ptr(ocol), _ptr(oval), _ptr(oscale), N, K,
                                              int(nout), _ptr(x2), _dt(x2), B, _ptr(y), _stream(stream)))
    return y


def qmatvec_km4o_tiled(tiled, lut, ocol, oval, oscale, x, y=None, stream=None):
    """qmatvec_km4o from the row-tiled plane (qtile_km4 of qpack_km4o's codes):
    x fp16 [K] or [B, K], 1 <= B <= 4 -> y fp32 [B, N]."""
    fn = "qmatvec_km4o_tiled"
    (pt, pl, N, K, px, dt, B, py), _, y = _tiled_args(fn, tiled, lut, x, y)
    _tensor(fn, "ocol", ocol, itemsize=2, ndim=2)
    nout = ocol.shape[1]
    _tensor(fn, "ocol", ocol, shape=(N, nout))
    _tensor(fn, "oval", oval, shape=(N, nout), itemsize=1)
    _tensor(fn, "oscale", oscale, shape=(N,), itemsize=2)
    _on_gpu(fn, tiled, ocol, oval, oscale)
    _check(fn, lib().qmatvec_km4o_tiled(pt, pl, _ptr(ocol), _ptr(oval), _ptr(oscale), N, K, int(nout), px, dt, B, py,
                                        _stream(stream)))
    return y


def qmatvec(fmt, codes, plane, x, y=None, stream=None):
    return _matvec("qmatvec_" + fmt, fmt, codes, plane, x, y, stream)


def qdequant(fmt, codes, plane, out=None, stream=None):
    torch = _torch()
    if fmt not in FORMATS:
        raise ValueError("qdequant: unknown format %r" % (fmt,))
    N, K = _codes2d("qdequant", fmt, codes)
    _dense_plane("qdequant", fmt, plane, N, K)
    out = _y_out("qdequant", out, (N, K), torch.float32, codes, "out")
    _on_gpu("qdequant", codes, plane, out)
    _check("qdequant", lib().qdequant(FORMATS[fmt], _ptr(codes), _ptr(plane), N, K, _ptr(out), _stream(stream)))
    return out


# ---------------------------------------------------------------- MoE

def qmoe_route(logits, topk, ids=None, weights=None, stream=None):
    torch = _torch()
    fn = "qmoe_route"
    _tensor(fn, "logits", logits, dtypes=(torch.float32,), ndim=2)
    T, E = logits.shape
    ids = _y_out(fn, ids, (T, topk), torch.int32, logits, "ids")
    weights = _y_out(fn, weights, (T, topk), torch.float32, logits, "weights")
    _on_gpu(fn, logits, ids, weights)
    _check("qmoe_route", lib().qmoe_route(_ptr(logits), T, E, topk, _ptr(ids), _ptr(weights), _stream(stream)))
    return ids, weights


def gather_qmatvec_workspace_bytes(T, topk, E, N, epi):
    return int(lib().gather_qmatvec_workspace_bytes(T, topk, E, N, EPILOGUES.get(epi, epi)))


def gather_qmatvec(fmt, codes, plane, x, ids, weights=None, epi="none", x_per_slot=False,
                   y=None, workspace=None, stream=None):
    """codes/plane: [E, N, ...] stacked experts; x [T, K] or [T, topk, K] (fp16)."""
    torch = _torch()
    fn = "gather_qmatvec"
    if fmt not in FORMATS:
        raise ValueError("%s: unknown format %r" % (fn, fmt))
    if epi not in EPILOGUES:
        raise ValueError("%s: unknown epilogue %r" % (fn, epi))
    _tensor(fn, "codes", codes, itemsize=1, ndim=3)
    E, N = codes.shape[0], codes.shape[1]
    K = _kdim(fmt, codes)
    _tensor(fn, "plane", plane)
    if plane.dim() < 1 or plane.shape[0] != E:
        _bad(fn, "plane must have E = %d as its first dimension, got shape %s" % (E, tuple(plane.shape)))
    if fmt == "int8km" and N % 32 != 0:
        _bad(fn, "int8km needs N % 32 == 0, got N = %d" % N)
    _plane_bytes(fn, "plane", plane, E * N * _plane_row_bytes(fmt, K))
    _tensor(fn, "ids", ids, dtypes=(torch.int32,), ndim=2)
    T, topk = ids.shape
    _tensor(fn, "x", x, dtypes=(torch.float16,))
    xs = (T, topk, K) if x_per_slot else (T, K)
    if tuple(x.shape) != xs:
        _bad(fn, "x has shape %s, expected %s" % (tuple(x.shape), xs))
    e = EPILOGUES[epi]
    if e == QMV_EPI_COMBINE:
        if weights is None:
            _bad(fn, "the combine epilogue needs weights")
        _tensor(fn, "weights", weights, shape=(T, topk), dtypes=(torch.float32,))
    if e == QMV_EPI_NONE:
        y = _y_out(fn, y, (T, topk, N), torch.float32, codes)
    elif e == QMV_EPI_SWIGLU:
        if N % 2 != 0:
            _bad(fn, "the SwiGLU epilogue needs an even N, got %d" % N)
        y = _y_out(fn, y, (T, topk, N // 2), torch.float16, codes)
    else:
        y = _y_out(fn, y, (T, N), torch.float32, codes)
    _on_gpu(fn, codes, plane, x, ids, y, weights if e == QMV_EPI_COMBINE else None)
    need = gather_qmatvec_workspace_bytes(T, topk, E, N, e)
    if need and workspace is None:
        workspace = _empty((need,), torch.uint8, codes)
    if workspace is not None:
        _tensor(fn, "workspace", workspace)
        _on_gpu(fn, codes, workspace)
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
    fn = "qmoe_ffn"
    if fmt not in FORMATS:
        raise ValueError("%s: unknown format %r" % (fn, fmt))
    _tensor(fn, "gu_codes", gu_codes, itemsize=1, ndim=3)
    _tensor(fn, "dn_codes", dn_codes, itemsize=1, ndim=3)
    E, I2 = gu_codes.shape[0], gu_codes.shape[1]
    H = dn_codes.shape[1]
    I = I2 // 2
    if I2 % 2 != 0 or dn_codes.shape[0] != E:
        _bad(fn, "gu_codes [E, 2I, ..] and dn_codes [E, H, ..] do not match: %s, %s"
             % (tuple(gu_codes.shape), tuple(dn_codes.shape)))
    if _kdim(fmt, gu_codes) != H or _kdim(fmt, dn_codes) != I:
        _bad(fn, "gate/up rows must hold H = %d weights and down rows I = %d weights" % (H, I))
    for name, pl, rows, k in (("gu_plane", gu_plane, I2, H), ("dn_plane", dn_plane, H, I)):
        _tensor(fn, name, pl)
        if pl.dim() < 1 or pl.shape[0] != E:
            _bad(fn, "%s must have E = %d as its first dimension" % (name, E))
        _plane_bytes(fn, name, pl, E * rows * _plane_row_bytes(fmt, k))
    _tensor(fn, "x", x, dtypes=(torch.float16,), ndim=2)
    T = x.shape[0]
    if x.shape[1] != H:
        _bad(fn, "x has shape %s, expected [T, %d]" % (tuple(x.shape), H))
    _tensor(fn, "logits", logits, shape=(T, E), dtypes=(torch.float32,))
    ids = _y_out(fn, ids, (T, topk), torch.int32, x, "ids")
    weights = _y_out(fn, weights, (T, topk), torch.float32, x, "weights")
    h = _y_out(fn, h, (T, topk, I), torch.float16, x, "h")
    y = _y_out(fn, y, (T, H), torch.float32, x)
    _on_gpu(fn, gu_codes, gu_plane, dn_codes, dn_plane, x, logits, ids, weights, h, y)
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
    fn = "qmatvec_argmax"
    if fmt not in FORMATS:
        raise ValueError("%s: unknown format %r" % (fn, fmt))
    N, K = _codes2d(fn, fmt, codes)
    _dense_plane(fn, fmt, plane, N, K)
    x2 = _as_batch(fn, x, K, allow_f32=False)
    B = x2.shape[0]
    idx = _y_out(fn, idx, (B,), torch.int32, codes, "idx")
    val = _y_out(fn, val, (B,), torch.float32, codes, "val")
    if workspace is None:
        workspace = _empty((qmatvec_argmax_workspace_bytes(N, B),), torch.uint8, codes)
    _tensor(fn, "workspace", workspace)
    _on_gpu(fn, codes, plane, x2, idx, val, workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("qmatvec_argmax", lib().qmatvec_argmax(
        FORMATS[fmt], _ptr(codes), _ptr(plane), N, K, _ptr(x2), B, _ptr(idx), _ptr(val),
        _ptr(workspace), ws_bytes, _stream(stream)))
    return idx, val


def qmatvec_argmax_km4_tiled(tiled, lut, x, idx=None, val=None, workspace=None, stream=None):
    """qmatvec_argmax for km4 from the row-tiled plane (qtile_km4): x fp16 [K] or
    [B, K], 1 <= B <= 4 -> (idx int32 [B], val fp32 [B])."""
    torch = _torch()
    fn = "qmatvec_argmax_km4_tiled"
    (pt, pl, N, K, px, _, B, _), keep, _ = _tiled_args(fn, tiled, lut, x, _NO_Y)
    idx = _y_out(fn, idx, (B,), torch.int32, tiled, "idx")
    val = _y_out(fn, val, (B,), torch.float32, tiled, "val")
    if workspace is None:
        workspace = _empty((qmatvec_argmax_workspace_bytes(N, B),), torch.uint8, tiled)
    _tensor(fn, "workspace", workspace)
    _on_gpu(fn, tiled, idx, val, workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(fn, lib().qmatvec_argmax_km4_tiled(pt, pl, N, K, px, B, _ptr(idx), _ptr(val), _ptr(workspace), ws_bytes,
                                              _stream(stream)))
    return idx, val


def qmatvec_argmax_noalloc(fmt, codes, plane, x, idx=None, val=None, stream=None):
    """qmatvec_argmax with its workspace in the library's fixed device array
    (no device allocation by the library; idx and val may be passed in so the
    call allocates nothing at all). Overlapping calls on one GPU race."""
    torch = _torch()
    fn = "qmatvec_argmax_noalloc"
    if fmt not in FORMATS:
        raise ValueError("%s: unknown format %r" % (fn, fmt))
    N, K = _codes2d(fn, fmt, codes)
    _dense_plane(fn, fmt, plane, N, K)
    x2 = _as_batch(fn, x, K, allow_f32=False)
    B = x2.shape[0]
    idx = _y_out(fn, idx, (B,), torch.int32, codes, "idx")
    val = _y_out(fn, val, (B,), torch.float32, codes, "val")
    _on_gpu(fn, codes, plane, x2, idx, val)
    _check(fn, lib().qmatvec_argmax_noalloc(FORMATS[fmt], _ptr(codes), _ptr(plane), N, K, _ptr(x2), B, _ptr(idx),
                                            _ptr(val), _stream(stream)))
    return idx, val


def qpack_int8_rows(W, codes=None, scale=None, stream=None):
    """Embedding table W [V, H] -> (codes int8 [V, H], scale fp16 bits uint16 [V])."""
    torch = _torch()
    fn = "qpack_int8_rows"
    _fp(fn, "W", W)
    if W.dim() != 2:
        _bad(fn, "W must be [V, H], got shape %s" % (tuple(W.shape),))
    V, H = W.shape
    codes = _empty((V, H), torch.int8, W) if codes is None else codes
    scale = _empty((V,), torch.uint16, W) if scale is None else scale
    _tensor(fn, "codes", codes, shape=(V, H), itemsize=1)
    _tensor(fn, "scale", scale, shape=(V,), itemsize=2)
    _on_gpu(fn, W, codes, scale)
    _check("qpack_int8_rows", lib().qpack_int8_rows(_ptr(W), _dt(W), V, H, _ptr(codes), _ptr(scale),
                                                    _stream(stream)))
    return codes, scale


def qembed_gather_int8(codes, scale, ids, out=None, stream=None):
    """out fp16 [T, H] = fp16(codes[ids] * scale[ids])."""
    torch = _torch()
    fn = "qembed_gather_int8"
    _tensor(fn, "codes", codes, itemsize=1, ndim=2)
    V, H = codes.shape
    _tensor(fn, "scale", scale, shape=(V,), itemsize=2)
    _tensor(fn, "ids", ids, dtypes=(torch.int32,))
    T = ids.numel()
    out = _y_out(fn, out, (T, H), torch.float16, codes, "out")
    _on_gpu(fn, codes, scale, ids, out)
    _check("qembed_gather_int8", lib().qembed_gather_int8(_ptr(codes), _ptr(scale), V, H, _ptr(ids), T,
                                                          _ptr(out), _stream(stream)))
    return out


# ---------------------------------------------------------------- measurement aid

def qmv_stream_read(buf, sink=None, stream=None):
    torch = _torch()
    fn = "qmv_stream_read"
    _tensor(fn, "buf", buf)
    nbytes = buf.numel() * buf.element_size()
    words = int(lib().qmv_stream_read_sink_words(nbytes))
    sink = _empty((words,), torch.int32, buf) if sink is None else sink
    _tensor(fn, "sink", sink, itemsize=4)
    if sink.numel() < words:
        _bad(fn, "sink holds %d words, needs %d" % (sink.numel(), words))
    _on_gpu(fn, buf, sink)
    _check("qmv_stream_read", lib().qmv_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(stream)))
    return sink
