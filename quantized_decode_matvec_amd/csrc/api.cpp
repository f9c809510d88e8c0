// C ABI of the library: argument validation, then one or two kernel launches
// on the caller's stream. Nothing here allocates, frees or synchronizes.
// The contract of each entry point is documented in include/qmv.h.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <mutex>

#include "qmv.h"
#include "qmv_launch.h"

namespace qmv {

int device_cu_count() {
    static std::mutex mu;
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> lk(mu);
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

}  // namespace qmv

namespace {

inline bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

// QMV_DEBUG_SYNC=1 in the environment: name the HIP error behind every
// QMV_E_LAUNCH on stderr, and after every launch wait for the stream and report
// any error the work itself raised (a debugging aid; off by default).
inline bool debug_sync() {
    static const bool on = [] {
        const char *v = getenv("QMV_DEBUG_SYNC");
        return v != nullptr && v[0] != '\0' && v[0] != '0';
    }();
    return on;
}

inline qmv_status launch_status_at(const char *fn, hipError_t e, void *stream) {
    if (e == hipSuccess && debug_sync()) e = hipStreamSynchronize(reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess && debug_sync()) fprintf(stderr, "qmv: %s: %s (%s)\n", fn, hipGetErrorName(e), hipGetErrorString(e));
    return e == hipSuccess ? QMV_OK : QMV_E_LAUNCH;
}
#define launch_status(call) launch_status_at(__func__, (call), stream)

// HIP keeps one last-error slot per host thread, and the launchers read it
// after their launches. Other code on the thread can leave a non-fatal error
// there (an allocator polling an event that is not ready yet, say), which
// would then be reported as a failed launch of ours: clear it just before
// launching. Errors that make the device unusable persist regardless.
inline void forget_earlier_errors() { (void)hipGetLastError(); }

qmv_status check_wk(const void *W, qmv_dtype wdt, int64_t N, int64_t K) {
    if (!W) return QMV_E_NULL;
    if (wdt != QMV_F16 && wdt != QMV_F32) return QMV_E_DTYPE;
    if (N < 1 || K < 32 || K % 32 != 0) return QMV_E_SHAPE;
    if (N > (int64_t(1) << 40) / K) return QMV_E_SHAPE;
    if (!aligned(W, 16)) return QMV_E_ALIGN;
    return QMV_OK;
}

qmv_status check_mv(const void *codes, const void *plane, size_t plane_align, int64_t N, int64_t K, const void *x,
                    qmv_dtype xdt, int B, const float *y) {
    if (!codes || !plane || !x || !y) return QMV_E_NULL;
    if (xdt != QMV_F16 && xdt != QMV_F32) return QMV_E_DTYPE;
    if (N < 1 || K < 32 || K % 32 != 0 || K > 65536 || B < 1 || B > 8) return QMV_E_SHAPE;
    if (N > (int64_t(1) << 40) / K) return QMV_E_SHAPE;
    if (!aligned(codes, 16) || !aligned(x, 16) || !aligned(plane, plane_align) || !aligned(y, 4)) return QMV_E_ALIGN;
    return QMV_OK;
}

// int8km tables cover groups of 32 rows: other row counts are refused
inline bool rows_fit(qmv_format f, int64_t N) { return f != QMV_INT8KM || N % 32 == 0; }

// largest K the expert gather handles: 256 chunks per row of codes
int64_t gather_max_k(qmv_format f) { return (f == QMV_INT8 || f == QMV_INT8KM) ? 4096 : 8192; }

size_t plane_alignment(qmv_format f) {
    switch (f) {
    case QMV_FP4: return 1;
    case QMV_KM4: return 4;       // tables are read as 32-bit words
    case QMV_INT4AFF: return 4;   // one 32-bit scale + bias word per block
    case QMV_INT8KM: return 4;    // tables are read as 32-bit words
    default: return 2;
    }
}

}  // namespace

extern "C" {

const char *qmv_status_string(qmv_status s) {
    switch (s) {
    case QMV_OK: return "QMV_OK";
    case QMV_E_NULL: return "QMV_E_NULL: a required pointer is NULL";
    case QMV_E_SHAPE: return "QMV_E_SHAPE: a size is out of range";
    case QMV_E_ALIGN: return "QMV_E_ALIGN: a pointer is misaligned";
    case QMV_E_DTYPE: return "QMV_E_DTYPE: unknown dtype, format or epilogue";
    case QMV_E_WORKSPACE: return "QMV_E_WORKSPACE: workspace missing or too small";
    case QMV_E_LAUNCH: return "QMV_E_LAUNCH: the HIP runtime failed a launch";
    }
    return "unknown qmv_status";
}

qmv_status qpack_int4(const void *W, qmv_dtype wdt, int64_t N, int64_t K, uint8_t *codes, uint16_t *scale,
                      void *stream) {
    qmv_status s = check_wk(W, wdt, N, K);
    if (s != QMV_OK) return s;
    if (!codes || !scale) return QMV_E_NULL;
    if (!aligned(codes, 16) || !aligned(scale, 2)) return QMV_E_ALIGN;
    forget_earlier_errors();
    return launch_status(qmv::launch_pack_int4(W, wdt, N, K, codes, scale, as_stream(stream)));
}

qmv_status qpack_fp4(const void *W, qmv_dtype wdt, int64_t N, int64_t K, uint8_t *codes, uint8_t *scale,
                     void *stream) {
    qmv_status s = check_wk(W, wdt, N, K);
    if (s != QMV_OK) return s;
    if (!codes || !scale) return QMV_E_NULL;
    if (!aligned(codes, 16)) return QMV_E_ALIGN;
    forget_earlier_errors();
    return launch_status(qmv::launch_pack_fp4(W, wdt, N, K, codes, scale, as_stream(stream)));
}

qmv_status qpack_int8(const void *W, qmv_dtype wdt, int64_t N, int64_t K, int8_t *codes, uint16_t *scale,
                      void *stream) {
    qmv_status s = check_wk(W, wdt, N, K);
    if (s != QMV_OK) return s;
    if (!codes || !scale) return QMV_E_NULL;
    if (!aligned(codes, 16) || !aligned(scale, 2)) return QMV_E_ALIGN;
    forget_earlier_errors();
    return launch_status(qmv::launch_pack_int8(W, wdt, N, K, codes, scale, as_stream(stream)));
}

qmv_status qpack_int4aff(const void *W, qmv_dtype wdt, int64_t N, int64_t K, uint8_t *codes, uint32_t *plane,
                         void *stream) {
    qmv_status s = check_wk(W, wdt, N, K);
    if (s != QMV_OK) return s;
    if (!codes || !plane) return QMV_E_NULL;
    if (!aligned(codes, 16) || !aligned(plane, 4)) return QMV_E_ALIGN;
    forget_earlier_errors();
    return launch_status(qmv::launch_pack_int4aff(W, wdt, N, K, codes, plane, as_stream(stream)));
}

qmv_status qpack_km4(const uint16_t *W_f16, int64_t N, int64_t K, int max_iter, uint8_t *codes, uint16_t *lut,
                     void *stream) {
    qmv_status s = check_wk(W_f16, QMV_F16, N, K);
    if (s != QMV_OK) return s;
    if (!codes || !lut) return QMV_E_NULL;
    if (K > 4096 || max_iter < 1 || max_iter > 1000) return QMV_E_SHAPE;
    if (!aligned(codes, 16) || !aligned(lut, 2)) return QMV_E_ALIGN;
    forget_earlier_errors();
    return launch_status(qmv::launch_pack_km4(W_f16, N, K, max_iter, codes, lut, as_stream(stream)));
}

qmv_status qmatvec_int4(const uint8_t *codes, const uint16_t *scale, int64_t N, int64_t K, const void *x,
                        qmv_dtype xdt, int B, float *y, void *stream) {
    qmv_status s = check_mv(codes, scale, 2, N, K, x, xdt, B, y);
    if (s != QMV_OK) return s;
    forget_earlier_errors();
    return launch_status(qmv::launch_matvec(QMV_INT4, codes, scale, N, K, x, xdt, B, y, as_stream(stream)));
}

qmv_status qmatvec_fp4(const uint8_t *codes, const uint8_t *scale, int64_t N, int64_t K, const void *x,
                       qmv_dtype xdt, int B, float *y, void *stream) {
    qmv_status s = check_mv(codes, scale, 1, N, K, x, xdt, B, y);
    if (s != QMV_OK) return s;
    forget_earlier_errors();
    return launch_status(qmv::launch_matvec(QMV_FP4, codes, scale, N, K, x, xdt, B, y, as_stream(stream)));
}

qmv_status qmatvec_int8(const int8_t *codes, const uint16_t *scale, int64_t N, int64_t K, const void *x,
                        qmv_dtype xdt, int B, float *y, void *stream) {
    qmv_status s = check_mv(codes, scale, 2, N, K, x, xdt, B, y);
    if (s != QMV_OK) return s;
    forget_earlier_errors();
    return launch_status(qmv::launch_matvec(QMV_INT8, codes, scale, N, K, x, xdt, B, y, as_stream(stream)));
}

qmv_status qmatvec_km4(const uint8_t *codes, const uint16_t *lut, int64_t N, int64_t K, const void *x,
                       qmv_dtype xdt, int B, float *y, void *stream) {
    qmv_status s = check_mv(codes, lut, 4, N, K, x, xdt, B, y);
    if (s != QMV_OK) return s;
    forget_earlier_errors();
    return launch_status(qmv::launch_matvec(QMV_KM4, codes, lut, N, K, x, xdt, B, y, as_stream(stream)));
}

size_t qtile_km4_bytes(int64_t N, int64_t K) {
    if (N < 1 || K < 32 || K % 32 != 0 || N > (int64_t(1) << 40) / K) return 0;
    return qmv::km4_tiled_bytes(N, K);
}

qmv_status qtile_km4(const uint8_t *codes, int64_t N, int64_t K, uint8_t *tiled, void *stream) {
    if (!codes || !tiled) return QMV_E_NULL;
    if (N < 1 || K < 32 || K % 32 != 0 || N > (int64_t(1) << 40) / K) return QMV_E_SHAPE;
    if (!aligned(codes, 16) || !aligned(tiled, 16)) return QMV_E_ALIGN;
    forget_earlier_errors();
    return launch_status(qmv::launch_tile_km4(codes, N, K, tiled, as_stream(stream)));
}

qmv_status qmatvec_km4_tiled(const uint8_t *tiled, const uint16_t *lut, int64_t N, int64_t K, const void *x,
                             qmv_dtype xdt, int B, float *y, void *stream) {
    qmv_status s = check_mv(tiled, lut, 4, N, K, x, xdt, B, y);
    if (s != QMV_OK) return s;
    if (xdt != QMV_F16) return QMV_E_DTYPE;
    if (!qmv::km4_tiled_supported(K, B)) return QMV_E_SHAPE;
    forget_earlier_errors();
    return launch_status(qmv::launch_matvec_km4_tiled(tiled, lut, N, K, reinterpret_cast<const _Float16 *>(x), B, y,
                                                      as_stream(stream)));
}

qmv_status qmatvec_km4o_tiled(const uint8_t *tiled, const uint16_t *lut, const uint16_t *ocol, const int8_t *oval,
                              const uint16_t *oscale, int64_t N, int64_t K, int nout, const void *x, qmv_dtype xdt,
                              int B, float *y, void *stream) {
    qmv_status s = check_mv(tiled, lut, 4, N, K, x, xdt, B, y);
    if (s != QMV_OK) return s;
    if (!oscale || (nout > 0 && (!ocol || !oval))) return QMV_E_NULL;
    if (xdt != QMV_F16) return QMV_E_DTYPE;
    if (!qmv::km4_tiled_supported(K, B) || nout < 0 || nout > 256 || nout > K) return QMV_E_SHAPE;
    if (!aligned(ocol, 2) || !aligned(oscale, 2)) return QMV_E_ALIGN;
    forget_earlier_errors();
    const _Float16 *xh = reinterpret_cast<const _Float16 *>(x);
    if (nout == 0) return launch_status(qmv::launch_matvec_km4_tiled(tiled, lut, N, K, xh, B, y, as_stream(stream)));
    return launch_status(
        qmv::launch_matvec_km4o_tiled(tiled, lut, ocol, oval, oscale, N, K, nout, xh, B, y, as_stream(stream)));
}

qmv_status qmatvec_int4aff(const uint8_t *codes, const uint32_t *plane, int64_t N, int64_t K, const void *x,
                           qmv_dtype xdt, int B, float *y, void *stream) {
    qmv_status s = check_mv(codes, plane, 4, N, K, x, xdt, B, y);
    if (s != QMV_OK) return s;
    forget_earlier_errors();
    return launch_status(qmv::launch_matvec(QMV_INT4AFF, codes, plane, N, K, x, xdt, B, y, as_stream(stream)));
}

qmv_status qpack_km4o(const uint16_t *W_f16, int64_t N, int64_t K, int nout, int max_iter, uint8_t *codes,
                      uint16_t *lut, uint16_t *ocol, int8_t *oval, uint16_t *oscale, void *stream) {
    qmv_status s = check_wk(W_f16, QMV_F16, N, K);
    if (s != QMV_OK) return s;
    if (!codes || !lut || !oscale || (nout > 0 && (!ocol || !oval))) return QMV_E_NULL;
    if (K > 4096 || max_iter < 1 || max_iter > 1000 || nout < 0 || nout > 256 || nout > K) return QMV_E_SHAPE;
    if (N > INT32_MAX) return QMV_E_SHAPE;
    if (!aligned(codes, 16) || !aligned(lut, 2) || !aligned(ocol, 2) || !aligned(oscale, 2)) return QMV_E_ALIGN;
    forget_earlier_errors();
    return launch_status(
        qmv::launch_pack_km4o(W_f16, N, K, nout, max_iter, codes, lut, ocol, oval, oscale, as_stream(stream)));
}

qmv_status qmatvec_km4o(const uint8_t *codes, const uint16_t *lut, const uint16_t *ocol, const int8_t *oval,
                        const uint16_t *oscale, int64_t N, int64_t K, int nout, const void *x, qmv_dtype xdt, int B,
                        float *y, void *stream) {
    qmv_status s = check_mv(codes, lut, 4, N, K, x, xdt, B, y);   // tables are read as 32-bit words
    if (s != QMV_OK) return s;
    if (!oscale || (nout > 0 && (!ocol || !oval))) return QMV_E_NULL;
    if (nout < 0 || nout > 256 || nout > K) return QMV_E_SHAPE;   // columns fit uint16: K <= 65536
    if (!aligned(ocol, 2) || !aligned(oscale, 2)) return QMV_E_ALIGN;
    forget_earlier_errors();
    return launch_status(
        qmv::launch_matvec_km4o(codes, lut, ocol, oval, oscale, N, K, nout, x, xdt, B, y, as_stream(stream)));
}

qmv_status qpack_int8km(const uint16_t *W_f16, int64_t N, int64_t K, int max_iter, uint8_t *codes, uint16_t *lut,
                        void *stream) {
    if (!W_f16 || !codes || !lut) return QMV_E_NULL;
    if (N < 32 || N % 32 != 0 || K < 32 || K % 32 != 0 || K > 2048 || max_iter < 1) return QMV_E_SHAPE;
    if (N / 32 > INT32_MAX) return QMV_E_SHAPE;
    if (!aligned(W_f16, 16) || !aligned(codes, 16) || !aligned(lut, 4)) return QMV_E_ALIGN;
    forget_earlier_errors();
    return launch_status(qmv::launch_pack_int8km(W_f16, N, K, max_iter, codes, lut, as_stream(stream)));
}

qmv_status qmatvec_int8km(const uint8_t *codes, const uint16_t *lut, int64_t N, int64_t K, const void *x,
                          qmv_dtype xdt, int B, float *y, void *stream) {
    qmv_status s = check_mv(codes, lut, 4, N, K, x, xdt, B, y);
    if (s != QMV_OK) return s;
    if (N % 32 != 0) return QMV_E_SHAPE;
    forget_earlier_errors();
    return launch_status(qmv::launch_matvec(QMV_INT8KM, codes, lut, N, K, x, xdt, B, y, as_stream(stream)));
}

qmv_status qdequant(qmv_format fmt, const void *codes, const void *plane, int64_t N, int64_t K, float *W_hat,
                    void *stream) {
    if (fmt < QMV_INT4 || fmt > QMV_INT8KM) return QMV_E_DTYPE;
    if (!codes || !plane || !W_hat) return QMV_E_NULL;
    if (N < 1 || K < 32 || K % 32 != 0 || N > (int64_t(1) << 40) / K || !rows_fit(fmt, N)) return QMV_E_SHAPE;
    if (!aligned(codes, 16) || !aligned(plane, plane_alignment(fmt)) || !aligned(W_hat, 16)) return QMV_E_ALIGN;
    forget_earlier_errors();
    return launch_status(qmv::launch_dequant(fmt, codes, plane, N, K, W_hat, as_stream(stream)));
}

qmv_status qmoe_route(const float *logits, int T, int E, int topk, int32_t *ids, float *weights, void *stream) {
    if (!logits || !ids || !weights) return QMV_E_NULL;
    if (T < 1 || T > 64 || E < 1 || E > 4096 || topk < 1 || topk > 64 || topk > E) return QMV_E_SHAPE;
    if (!aligned(logits, 4) || !aligned(ids, 4) || !aligned(weights, 4)) return QMV_E_ALIGN;
    forget_earlier_errors();
    return launch_status(qmv::launch_moe_route(logits, T, E, topk, ids, weights, as_stream(stream)));
}

size_t gather_qmatvec_workspace_bytes(int T, int topk, int E, int64_t N, qmv_epilogue epi) {
    if (T < 1 || topk < 1 || N < 1) return 0;
    return qmv::gather_workspace_bytes(T, topk, E, N, epi);
}

qmv_status gather_qmatvec(qmv_format fmt, const void *codes, const void *plane, int E, int64_t N, int64_t K,
                          const void *x, qmv_dtype xdt, int x_per_slot, int T, int topk, const int32_t *ids,
                          const float *weights, qmv_epilogue epi, void *y, void *workspace, size_t ws_bytes,
                          void *stream) {
    if (fmt < QMV_INT4 || fmt > QMV_INT8KM) return QMV_E_DTYPE;
    if (epi != QMV_EPI_NONE && epi != QMV_EPI_SWIGLU && epi != QMV_EPI_COMBINE) return QMV_E_DTYPE;
    if (xdt != QMV_F16) return QMV_E_DTYPE;
    if (!codes || !plane || !x || !ids || !y) return QMV_E_NULL;
    if (epi == QMV_EPI_COMBINE && !weights) return QMV_E_NULL;
    if (E < 1 || E > 4096 || N < 1 || K < 32 || K % 32 != 0 || K > gather_max_k(fmt)) return QMV_E_SHAPE;
    if (T < 1 || T > 8 || topk < 1 || topk > 64 || topk > E) return QMV_E_SHAPE;
    if (x_per_slot != 0 && x_per_slot != 1) return QMV_E_SHAPE;
    if (epi == QMV_EPI_SWIGLU && N % 2 != 0) return QMV_E_SHAPE;
    // int8km tables cover 32 rows: whole groups, and gate and up halves of whole groups
    if (!rows_fit(fmt, N) || (fmt == QMV_INT8KM && epi == QMV_EPI_SWIGLU && (N / 2) % 32 != 0)) return QMV_E_SHAPE;
    if (N > (int64_t(1) << 40) / K / E) return QMV_E_SHAPE;
    size_t need = qmv::gather_workspace_bytes(T, topk, E, N, epi);
    if (need > 0 && (!workspace || ws_bytes < need)) return QMV_E_WORKSPACE;
    if (need > 0 && !aligned(workspace, 256)) return QMV_E_ALIGN;
    if (!aligned(codes, 16) || !aligned(plane, plane_alignment(fmt)) || !aligned(x, 16) || !aligned(ids, 4) ||
        !aligned(y, epi == QMV_EPI_SWIGLU ? 2 : 4) || (weights && !aligned(weights, 4)))
        return QMV_E_ALIGN;
    forget_earlier_errors();
    return launch_status(qmv::launch_gather(fmt, codes, plane, E, N, K, x, xdt, x_per_slot, T, topk, ids, weights,
                                            epi, y, workspace, as_stream(stream)));
}

qmv_status qmoe_ffn(qmv_format fmt, const void *gu_codes, const void *gu_plane, const void *dn_codes,
                    const void *dn_plane, int E, int64_t H, int64_t I, const float *logits, const void *x, int T,
                    int topk, int32_t *ids, float *weights, void *h, float *y, void *stream) {
    if (fmt < QMV_INT4 || fmt > QMV_INT8KM) return QMV_E_DTYPE;
    if (!gu_codes || !gu_plane || !dn_codes || !dn_plane || !logits || !x || !ids || !weights || !h || !y)
        return QMV_E_NULL;
    if (E < 1 || E > 4096 || T < 1 || T > 8 || topk < 1 || topk > 64 || topk > E) return QMV_E_SHAPE;
    const int64_t kmax = gather_max_k(fmt);
    if (H < 32 || H % 32 != 0 || H > kmax || I < 32 || I % 32 != 0 || I > kmax) return QMV_E_SHAPE;
    const size_t pa = plane_alignment(fmt);
    if (!aligned(gu_codes, 16) || !aligned(dn_codes, 16) || !aligned(gu_plane, pa) || !aligned(dn_plane, pa) ||
        !aligned(logits, 4) || !aligned(x, 16) || !aligned(ids, 4) || !aligned(weights, 4) || !aligned(h, 16) ||
        !aligned(y, 4))
        return QMV_E_ALIGN;
    forget_earlier_errors();
    return launch_status(qmv::launch_moe_ffn(fmt, gu_codes, gu_plane, dn_codes, dn_plane, E, H, I, logits, x, T,
                                             topk, ids, weights, h, y, as_stream(stream)));
}

size_t qmatvec_argmax_workspace_bytes(int64_t N, int B) {
    if (N < 1 || B < 1 || B > 8) return 0;
    return qmv::argmax_workspace_bytes(N, B);
}

qmv_status qmatvec_argmax(qmv_format fmt, const void *codes, const void *plane, int64_t N, int64_t K, const void *x,
                          int B, int32_t *idx, float *val, void *workspace, size_t ws_bytes, void *stream) {
    if (fmt < QMV_INT4 || fmt > QMV_INT8KM) return QMV_E_DTYPE;
    if (!codes || !plane || !x || !idx || !val) return QMV_E_NULL;
    if (N < 1 || N > INT32_MAX || K < 32 || K % 32 != 0 || B < 1 || B > 8 || !rows_fit(fmt, N)) return QMV_E_SHAPE;
    if (N > (int64_t(1) << 40) / K || !qmv::argmax_supported(fmt, K, B)) return QMV_E_SHAPE;
    if (!workspace || ws_bytes < qmv::argmax_workspace_bytes(N, B)) return QMV_E_WORKSPACE;
    if (!aligned(codes, 16) || !aligned(plane, plane_alignment(fmt)) || !aligned(x, 16) || !aligned(idx, 4) ||
        !aligned(val, 4) || !aligned(workspace, 8))
        return QMV_E_ALIGN;
    forget_earlier_errors();
    return launch_status(qmv::launch_matvec_argmax(fmt, codes, plane, N, K, x, B, idx, val, workspace,
                                                   as_stream(stream)));
}

qmv_status qmatvec_argmax_km4_tiled(const uint8_t *tiled, const uint16_t *lut, int64_t N, int64_t K, const void *x,
                                    int B, int32_t *idx, float *val, void *workspace, size_t ws_bytes,
                                    void *stream) {
    if (!tiled || !lut || !x || !idx || !val) return QMV_E_NULL;
    if (N < 1 || N > INT32_MAX || N > (int64_t(1) << 40) / (K > 0 ? K : 1) || !qmv::km4_tiled_supported(K, B))
        return QMV_E_SHAPE;
    if (!workspace || ws_bytes < qmv::argmax_workspace_bytes(N, B)) return QMV_E_WORKSPACE;
    if (!aligned(tiled, 16) || !aligned(lut, 4) || !aligned(x, 16) || !aligned(idx, 4) || !aligned(val, 4) ||
        !aligned(workspace, 8))
        return QMV_E_ALIGN;
    forget_earlier_errors();
    return launch_status(qmv::launch_argmax_km4_tiled(tiled, lut, N, K, reinterpret_cast<const _Float16 *>(x), B,
                                                      idx, val, workspace, as_stream(stream)));
}

qmv_status qmatvec_argmax_noalloc(qmv_format fmt, const void *codes, const void *plane, int64_t N, int64_t K,
                                  const void *x, int B, int32_t *idx, float *val, void *stream) {
    if (fmt < QMV_INT4 || fmt > QMV_INT8KM) return QMV_E_DTYPE;
    if (!codes || !plane || !x || !idx || !val) return QMV_E_NULL;
    if (N < 1 || N > INT32_MAX || K < 32 || K % 32 != 0 || B < 1 || B > 8 || !rows_fit(fmt, N)) return QMV_E_SHAPE;
    if (N > (int64_t(1) << 40) / K || !qmv::argmax_supported(fmt, K, B)) return QMV_E_SHAPE;
    if (qmv::argmax_workspace_bytes(N, B) > qmv::scratch_bytes()) return QMV_E_WORKSPACE;
    if (!aligned(codes, 16) || !aligned(plane, plane_alignment(fmt)) || !aligned(x, 16) || !aligned(idx, 4) ||
        !aligned(val, 4))
        return QMV_E_ALIGN;
    void *ws = nullptr;
    forget_earlier_errors();
    if (qmv::scratch_address(&ws) != hipSuccess) return QMV_E_LAUNCH;
    return launch_status(qmv::launch_matvec_argmax(fmt, codes, plane, N, K, x, B, idx, val, ws, as_stream(stream)));
}

size_t qmatvec_argmax_noalloc_max_bytes(void) { return qmv::scratch_bytes(); }

qmv_status qpack_int8_rows(const void *W, qmv_dtype wdt, int64_t V, int64_t H, int8_t *codes, uint16_t *scale,
                           void *stream) {
    if (!W || !codes || !scale) return QMV_E_NULL;
    if (wdt != QMV_F16 && wdt != QMV_F32) return QMV_E_DTYPE;
    if (V < 1 || V > INT32_MAX || H < 1 || V > (int64_t(1) << 40) / H) return QMV_E_SHAPE;
    if (!aligned(W, wdt == QMV_F16 ? 2 : 4) || !aligned(scale, 2)) return QMV_E_ALIGN;
    forget_earlier_errors();
    return launch_status(qmv::launch_pack_int8_rows(W, wdt, V, H, codes, scale, as_stream(stream)));
}

qmv_status qembed_gather_int8(const int8_t *codes, const uint16_t *scale, int64_t V, int64_t H, const int32_t *ids,
                              int64_t T, void *out, void *stream) {
    if (!codes || !scale) return QMV_E_NULL;
    if (V < 1 || H < 8 || H % 8 != 0 || T < 0 || T > 65535 || V > (int64_t(1) << 40) / H) return QMV_E_SHAPE;
    if (T == 0) return QMV_OK;   // nothing to gather; ids and out may be NULL
    if (!ids || !out) return QMV_E_NULL;
    if (!aligned(codes, 8) || !aligned(scale, 2) || !aligned(ids, 4) || !aligned(out, 16)) return QMV_E_ALIGN;
    forget_earlier_errors();
    return launch_status(qmv::launch_embed_gather_int8(codes, scale, V, H, ids, T, out, as_stream(stream)));
}

size_t qmv_stream_read_sink_words(size_t bytes) { return qmv::stream_read_grid(bytes); }

qmv_status qmv_stream_read(const void *buf, size_t bytes, uint32_t *sink, void *stream) {
    if (!buf || !sink) return QMV_E_NULL;
    if (bytes == 0 || bytes % 16 != 0) return QMV_E_SHAPE;
    if (!aligned(buf, 16) || !aligned(sink, 4)) return QMV_E_ALIGN;
    forget_earlier_errors();
    return launch_status(qmv::launch_stream_read(buf, bytes, sink, as_stream(stream)));
}

}  // extern "C"
