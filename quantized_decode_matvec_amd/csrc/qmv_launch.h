// Internal host-side interface between the C ABI (api.cpp) and the kernel
// translation units. Every launcher enqueues on `st` and returns the HIP
// runtime's launch status; arguments are validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "qmv.h"

namespace qmv {

int device_cu_count();   // compute units of the current device (cached per device)

hipError_t launch_matvec(int fmt, const void *codes, const void *plane, int64_t N, int64_t K, const void *x,
                         qmv_dtype xdt, int B, float *y, hipStream_t st);
// batched matrix-core path; *handled is false when the shape is not one it takes
// Fused argmax workspace header: 64-bit words, the maxima of batch rows 0..7
// then one workgroup counter per batch row; a matvec given `hdr` zeroes them.
constexpr int kArgmaxHeader = 16;
hipError_t launch_matvec_mfma(int fmt, const uint8_t *codes, const void *plane, int64_t N, int64_t K, const void *x,
                              int B, float *y, hipStream_t st, bool *handled, uint64_t *hdr = nullptr);
// km4 at batch 1-4 on the row-tiled code plane (matvec_km4_rows.hip)
bool km4_tiled_supported(int64_t K, int B);
size_t km4_tiled_bytes(int64_t N, int64_t K);
hipError_t launch_tile_km4(const uint8_t *codes, int64_t N, int64_t K, uint8_t *out, hipStream_t st);
hipError_t launch_matvec_km4_tiled(const uint8_t *codes, const uint16_t *lut, int64_t N, int64_t K,
                                   const _Float16 *x, int B, float *y, hipStream_t st);
// the same with the int8 outliers of the km4 + outlier format (nout >= 1)
hipError_t launch_matvec_km4o_tiled(const uint8_t *codes, const uint16_t *lut, const uint16_t *ocol,
                                    const int8_t *oval, const uint16_t *oscale, int64_t N, int64_t K, int nout,
                                    const _Float16 *x, int B, float *y, hipStream_t st);
// the argmax of each batch row of y [B][N] into idx/val, reduced through the
// zeroed header hdr (matvec.hip)
hipError_t launch_argmax_rows(const float *y, int64_t N, int B, uint64_t *hdr, int32_t *idx, float *val,
                              hipStream_t st);
// greedy token from the tiled km4 plane: the matvec writes one argmax key per
// workgroup and batch row into the workspace (km4_tiled_argmax_keys_bytes at
// most, no logits), then one small launch takes the largest
size_t km4_tiled_argmax_keys_bytes(int64_t N, int B);
hipError_t launch_argmax_km4_tiled(const uint8_t *codes, const uint16_t *lut, int64_t N, int64_t K,
                                   const _Float16 *x, int B, int32_t *idx, float *val, void *workspace,
                                   hipStream_t st);
bool argmax_supported(int fmt, int64_t K, int B);
size_t argmax_workspace_bytes(int64_t N, int B);
hipError_t launch_matvec_argmax(int fmt, const void *codes, const void *plane, int64_t N, int64_t K, const void *x,
                                int B, int32_t *idx, float *val, void *workspace, hipStream_t st);
// the fixed device scratch of the allocation-free argmax (scratch.hip)
size_t scratch_bytes();
hipError_t scratch_address(void **out);
hipError_t launch_pack_int8_rows(const void *W, qmv_dtype wdt, int64_t V, int64_t H, int8_t *codes, uint16_t *scale,
                                 hipStream_t st);
hipError_t launch_embed_gather_int8(const int8_t *codes, const uint16_t *scale, int64_t V, int64_t H,
                                    const int32_t *ids, int64_t T, void *out, hipStream_t st);
hipError_t launch_dequant(int fmt, const void *codes, const void *plane, int64_t N, int64_t K, float *out,
                          hipStream_t st);
size_t stream_read_grid(size_t bytes);
hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t st);

hipError_t launch_pack_int4(const void *W, qmv_dtype wdt, int64_t N, int64_t K, uint8_t *codes, uint16_t *scale,
                            hipStream_t st);
hipError_t launch_pack_int8(const void *W, qmv_dtype wdt, int64_t N, int64_t K, int8_t *codes, uint16_t *scale,
                            hipStream_t st);
hipError_t launch_pack_fp4(const void *W, qmv_dtype wdt, int64_t N, int64_t K, uint8_t *codes, uint8_t *scale,
                           hipStream_t st);
hipError_t launch_pack_int4aff(const void *W, qmv_dtype wdt, int64_t N, int64_t K, uint8_t *codes, uint32_t *plane,
                               hipStream_t st);
hipError_t launch_pack_km4(const uint16_t *W, int64_t N, int64_t K, int max_iter, uint8_t *codes, uint16_t *lut,
                           hipStream_t st, const uint16_t *ocol = nullptr, int nout = 0);
hipError_t launch_pack_km4o(const uint16_t *W, int64_t N, int64_t K, int nout, int max_iter, uint8_t *codes,
                            uint16_t *lut, uint16_t *ocol, int8_t *oval, uint16_t *oscale, hipStream_t st);
hipError_t launch_matvec_km4o(const uint8_t *codes, const uint16_t *lut, const uint16_t *ocol, const int8_t *oval,
                              const uint16_t *oscale, int64_t N, int64_t K, int nout, const void *x, qmv_dtype xdt,
                              int B, float *y, hipStream_t st);
hipError_t launch_pack_int8km(const uint16_t *W, int64_t N, int64_t K, int max_iter, uint8_t *codes, uint16_t *lut,
                              hipStream_t st);

hipError_t launch_moe_route(const float *logits, int T, int E, int topk, int32_t *ids, float *weights,
                            hipStream_t st);
size_t gather_workspace_bytes(int T, int topk, int E, int64_t N, int epi);
hipError_t launch_gather(int fmt, const void *codes, const void *plane, int E, int64_t N, int64_t K, const void *x,
                         qmv_dtype xdt, int x_per_slot, int T, int topk, const int32_t *ids, const float *weights,
                         int epi, void *y, void *workspace, hipStream_t st);
hipError_t launch_moe_ffn(int fmt, const void *gu_codes, const void *gu_plane, const void *dn_codes,
                          const void *dn_plane, int E, int64_t H, int64_t I, const float *logits, const void *x, int T,
                          int topk, int32_t *ids, float *weights, void *h, float *y, hipStream_t st);

}  // namespace qmv
