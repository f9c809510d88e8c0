/*
 * qmv.h - block-quantized decode matvec on AMD Instinct MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels: quantize-and-pack fp16/fp32 weights
 * into four block formats, and the fused dequantize-matvec y = dequant(Wq) x
 * for decode batches of 1 to 8, plus the mixture-of-experts routed-expert
 * gather used for expert FFNs.
 *
 * Sources (web pages of the "Core AI model zoo" knowledge base) cited below:
 *  [S1] "Stream D - Quantization (FP4 + QAT-int4): feasibility, first result,
 *       and plan", section 1 "Toolchain reality" and section 2 "The de-risk
 *       experiment".
 *  [S2] "Dense-path int4km coverage + flagship Qwen3.6-35B - session findings
 *       & methods", sections 1 "The lever", 8 "FP4 (E2M1) dense matvec", 8b.
 *  [S3] "coreai-optimization (coreai-opt) reference - quantization &
 *       palettization", sections "Quantization", "Palettization",
 *       "Pitfalls", "Theoretical size".
 *  [S5] "Compression (palettization & quantization)", section "Per-channel
 *       int8 on a big-vocab LM head: use per-block-32".
 *
 * Conventions shared by every entry point
 *  - Layout. W is [N][K] row-major (N output rows, K inputs; the nn.Linear
 *    out x in convention), blocks of 32 run along K [S1 sec. 1, S3
 *    "Quantization"]. K must be a multiple of 32; a K that is not is refused
 *    with QMV_E_SHAPE rather than skipped [S3 "Pitfalls"].
 *    4-bit code planes are [N][K/2] bytes, element 2j in the low nibble of
 *    byte j (the same bytes as eight codes per little-endian 32-bit word)
 *    [S1 sec. 1, S2 sec. 8]. Scale and table planes are separate arrays.
 *  - Memory. Every pointer argument is device memory owned by the caller.
 *    The library never allocates, frees or synchronizes, and keeps no state
 *    between calls other than a cached device-property query.
 *  - Alignment. codes, W and x: 16 bytes. Planes, y, ids and weights: their
 *    element size. A misaligned pointer returns QMV_E_ALIGN.
 *  - Execution. Work is enqueued on `stream` (a hipStream_t; NULL is the
 *    default stream) and runs asynchronously. Calls are thread-safe; on one
 *    stream they run in order. Entry points taking a workspace may be
 *    captured in a HIP graph.
 *  - Errors. Arguments are validated before anything is enqueued; on any
 *    error nothing is launched. A failure reported by the HIP runtime at
 *    launch returns QMV_E_LAUNCH. Faults inside kernels surface on the
 *    caller's next synchronization. Non-finite weights or logits and
 *    out-of-range expert ids give unspecified results (not checked).
 */
#ifndef QMV_H
#define QMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QMV_OK = 0,
    QMV_E_NULL = 1,      /* a required pointer is NULL */
    QMV_E_SHAPE = 2,     /* a size is out of range (see each entry point) */
    QMV_E_ALIGN = 3,     /* a pointer breaks the alignment rule above */
    QMV_E_DTYPE = 4,     /* unknown dtype, format or epilogue value */
    QMV_E_WORKSPACE = 5, /* workspace missing or smaller than required */
    QMV_E_LAUNCH = 6     /* the HIP runtime refused or failed a launch */
} qmv_status;

typedef enum { QMV_F32 = 0, QMV_F16 = 1 } qmv_dtype;
typedef enum { QMV_INT4 = 0, QMV_FP4 = 1, QMV_INT8 = 2, QMV_KM4 = 3, QMV_INT4AFF = 4, QMV_INT8KM = 5 } qmv_format;
typedef enum { QMV_EPI_NONE = 0, QMV_EPI_SWIGLU = 1, QMV_EPI_COMBINE = 2 } qmv_epilogue;

/* Static string naming a status (never NULL). */
const char *qmv_status_string(qmv_status s);

/* ---------------------------------------------------------------------- */
/* Quantize and pack. W: [N][K], wdt QMV_F16 or QMV_F32 (fp32 values must  */
/* lie in the fp16 finite range for int4/int8). 1 <= N, K % 32 == 0.       */
/* ---------------------------------------------------------------------- */

/* Symmetric int4 per block of 32 with an MSE-chosen clip ratio and an fp16
 * scale [S1 sec. 1 "Convert invocation" (the default 4-bit recipe), sec. 2
 * (clip ratio per block chosen by squared error)]. For each clip c in
 * 1.0, 0.95, ..., 0.7 (in that order): s = fp16(fp32(c*amax)/7), q =
 * clamp(rint(w/s), -7, 7), err = sequential fmaf sum of (w - s*q)^2; the
 * first strictly smallest err wins. Outputs: codes [N][K/2] of u = q + 8,
 * scale [N][K/32] fp16 bits. Dequant: fp16(scale) * (u - 8). */
qmv_status qpack_int4(const void *W, qmv_dtype wdt, int64_t N, int64_t K,
                      uint8_t *codes, uint16_t *scale, void *stream);

/* FP4 E2M1 with an e8m0 scale per block of 32 [S1 sec. 1: E2M1 of the OCP MX
 * family, scale 2^(floor(log2 amax) - 2), two codes per byte; S2 sec. 8].
 * E = clamp(floor(log2 amax) - 2, -127, 127) (an all-zero block takes -127);
 * the code is the nearest of {0, .5, 1, 1.5, 2, 3, 4, 6} to |w| * 2^-E (ties
 * to the even mantissa, above 6 saturates) with the input's sign bit in bit
 * 3. Outputs: codes [N][K/2]; scale [N][K/32] bytes E + 127. */
qmv_status qpack_fp4(const void *W, qmv_dtype wdt, int64_t N, int64_t K,
                     uint8_t *codes, uint8_t *scale, void *stream);

/* Symmetric int8 per block of 32 with an fp16 scale, no clipping [S5]:
 * s = fp16(amax/127), q = clamp(rint(w/s), -127, 127). Outputs: codes
 * [N][K] int8, scale [N][K/32] fp16 bits. Dequant: fp16(scale) * q. */
qmv_status qpack_int8(const void *W, qmv_dtype wdt, int64_t N, int64_t K,
                      int8_t *codes, uint16_t *scale, void *stream);

/* 4-bit k-means palettization, one 16-entry fp16 table per output row
 * [S2 secs. 1, 8, 8b (palettize_grouped, n_bits = 4); S3 "Palettization"
 * (scalar k-means, per-channel grouping)]. W_f16: [N][K] fp16 bits,
 * 32 <= K <= 8192. Exact integer arithmetic on w * 2^24: a row with at most
 * 16 distinct values keeps them (ascending, padded with the largest);
 * otherwise centroids start at the order statistics of rank (2j+1)K/32 and
 * take at most max_iter (1..1000) Lloyd steps (nearest centroid, ties to the
 * lower index; each non-empty centroid moves to its members' mean rounded
 * to the nearest fp16, ties to even; stop when nothing moves); a final
 * assignment gives the indices. Outputs: codes [N][K/2] of indices; lut
 * [N][16] fp16 bits, ascending. */
qmv_status qpack_km4(const uint16_t *W_f16, int64_t N, int64_t K, int max_iter,
                     uint8_t *codes, uint16_t *lut, void *stream);

/* Affine int4 per block of 32 with an fp16 scale and an fp16 bias [S1 sec. 1:
 * affine int4, block 32, among the production MoE gather formats; S2 sec. 8:
 * fp4 is that affine structure without the bias]. Min-max, fp32 steps:
 * b = fp16(min), s = fp16((max - min) / 15), u = clamp(rint((w - b)/s), 0, 15)
 * (s == 0: u = 0). Outputs: codes [N][K/2] of u (element 2j in the low
 * nibble); plane [N][K/32] 32-bit words, fp16 scale in the low half and fp16
 * bias in the high half. Dequant: s * u + b. */
qmv_status qpack_int4aff(const void *W, qmv_dtype wdt, int64_t N, int64_t K,
                         uint8_t *codes, uint32_t *plane, void *stream);

/* 8-bit k-means palettization with one 256-entry fp16 table per group of 32
 * consecutive rows [S3 "Palettization": 2^n_bits centroids, 1-D k-means,
 * per-grouped-channel granularity; S5 "int8 k-means > whole-model int4":
 * int8 k-means, group 32]. The 4-bit table procedure above on the 32 * K
 * values of each group: exact integer arithmetic on units of 2^-24; at most
 * 256 distinct values form the table (ascending, padded with the largest);
 * otherwise start from the order statistics at ranks (2j+1)M/512 (M = 32K)
 * and take at most max_iter Lloyd steps (a value goes to the index equal to
 * the number of adjacent entry pairs whose midpoint lies strictly below it;
 * non-empty entries move to their members' mean rounded to the nearest fp16,
 * ties to even; stop when none moves). Outputs: codes [N][K] byte indices,
 * lut [N/32][256] fp16 bits ascending. N % 32 == 0 (a row count that is not
 * a multiple of the group is refused rather than left unpacked, [S3]
 * "Pitfalls"); K <= 2048 (a group's sorted values are held on chip);
 * max_iter >= 1; W, codes 16-byte aligned, lut 4-byte aligned. */
qmv_status qpack_int8km(const uint16_t *W_f16, int64_t N, int64_t K, int max_iter,
                        uint8_t *codes, uint16_t *lut, void *stream);

/* ---------------------------------------------------------------------- */
/* Fused dequantize-matvec [S2 secs. 1 and 8: the fused 4-bit decode       */
/* matvec; the same kernel structure for every format, only the dequant    */
/* differs]. y[b][n] = sum_k dequant(W)[n][k] * x[b][k] with fp32          */
/* accumulation. x: [B][K] (QMV_F16 or QMV_F32), y: [B][N] fp32            */
/* (overwritten). 1 <= B <= 8, 1 <= N, K % 32 == 0, K <= 65536.            */
/* ---------------------------------------------------------------------- */

qmv_status qmatvec_int4(const uint8_t *codes, const uint16_t *scale, int64_t N, int64_t K,
                        const void *x, qmv_dtype xdt, int B, float *y, void *stream);
qmv_status qmatvec_fp4(const uint8_t *codes, const uint8_t *scale, int64_t N, int64_t K,
                       const void *x, qmv_dtype xdt, int B, float *y, void *stream);
qmv_status qmatvec_int8(const int8_t *codes, const uint16_t *scale, int64_t N, int64_t K,
                        const void *x, qmv_dtype xdt, int B, float *y, void *stream);
qmv_status qmatvec_km4(const uint8_t *codes, const uint16_t *lut, int64_t N, int64_t K,
                       const void *x, qmv_dtype xdt, int B, float *y, void *stream);
/* ---------------------------------------------------------------------- */
/* 4-bit k-means rows on a row-tiled code plane [S2 secs. 1, 8: the lm_head */
/* is the largest per-token matvec, its int4km form read once per token;   */
/* S3 "Palettization": one 16-entry table per output row]. The same bytes  */
/* as qpack_km4's code plane, reordered once (at weight load) so that a    */
/* kernel can give each lane its own row: tile t holds rows 64t..64t+63    */
/* and chunk q (16 bytes = codes 32q..32q+31) of row 64t + r sits at byte  */
/* ((t * (K/32) + q) * 64 + r) * 16. Rows past N in the last tile are zero.*/
/* ---------------------------------------------------------------------- */

/* Bytes of the row-tiled plane: ceil(N / 64) * 64 * K / 2 (0 for sizes
 * qtile_km4 refuses). */
size_t qtile_km4_bytes(int64_t N, int64_t K);

/* codes [N][K/2] (as qpack_km4 writes them) -> tiled [qtile_km4_bytes(N, K)]
 * bytes; K % 32 == 0; both 16-byte aligned; the two must not overlap. */
qmv_status qtile_km4(const uint8_t *codes, int64_t N, int64_t K, uint8_t *tiled, void *stream);

/* y[b][n] = sum_k lut[n][code(n, k)] * x[b][k], fp32 accumulation, from the
 * tiled plane and qpack_km4's lut [N][16] (4-byte aligned). 1 <= B <= 4, x fp16
 * [B][K], K a multiple of 512 up to 4096 (QMV_E_SHAPE otherwise, QMV_E_DTYPE
 * for fp32 x); y fp32 [B][N]. */
qmv_status qmatvec_km4_tiled(const uint8_t *tiled, const uint16_t *lut, int64_t N, int64_t K,
                             const void *x, qmv_dtype xdt, int B, float *y, void *stream);

qmv_status qmatvec_int4aff(const uint8_t *codes, const uint32_t *plane, int64_t N, int64_t K,
                           const void *x, qmv_dtype xdt, int B, float *y, void *stream);
/* int8km: N % 32 == 0; lut as qpack_int8km writes it (4-byte aligned). */
qmv_status qmatvec_int8km(const uint8_t *codes, const uint16_t *lut, int64_t N, int64_t K,
                          const void *x, qmv_dtype xdt, int B, float *y, void *stream);

/* ---------------------------------------------------------------------- */
/* 4-bit k-means rows plus int8 outliers ["Kernel campaign - session       */
/* handoff", NEXT per lever, Stream D: a mixed int4 + int8-outlier matvec  */
/* on the int4 k-means linear, bridging the int4 quality cliff at about    */
/* int4 bandwidth]. Per row, the nout entries of largest magnitude (ties  */
/* to the lower column) are outliers, listed by increasing column: ocol    */
/* uint16 [N][nout], oval int8 [N][nout], and one fp16 scale per row       */
/* oscale [N] = fp16(max |w| of the outliers / 127), oval = clamp(rint(w / */
/* scale), -127, 127) (scale 0: 0). The row with its outliers set to +0 is */
/* palettized exactly as qpack_km4 (codes [N][K/2], lut [N][16]). The     */
/* weight is lut[n][code] + (k an outlier ? oscale[n] * oval : 0).        */
/* 0 <= nout <= min(256, K); K <= 4096 (packing) / 65536 (matvec); with   */
/* nout == 0, ocol and oval may be NULL and oscale is written as zeros.   */
/* ---------------------------------------------------------------------- */
qmv_status qpack_km4o(const uint16_t *W_f16, int64_t N, int64_t K, int nout, int max_iter,
                      uint8_t *codes, uint16_t *lut, uint16_t *ocol, int8_t *oval, uint16_t *oscale,
                      void *stream);

/* y[b][n] = sum_k W_hat[n][k] * x[b][k] with the outliers added in fp32;
 * x fp16 or fp32 [B][K], B <= 8, y fp32 [B][N]; the tables and codes as
 * qmatvec_km4 (lut 4-byte aligned: the tables are read as 32-bit words). */
qmv_status qmatvec_km4o(const uint8_t *codes, const uint16_t *lut, const uint16_t *ocol,
                        const int8_t *oval, const uint16_t *oscale, int64_t N, int64_t K, int nout,
                        const void *x, qmv_dtype xdt, int B, float *y, void *stream);

/* qmatvec_km4o from the row-tiled code plane (qtile_km4 of qpack_km4o's
 * codes): the tables and outlier arrays as qmatvec_km4o, x fp16 [B][K],
 * 1 <= B <= 4, K a multiple of 512 up to 4096, 0 <= nout <= 256. */
qmv_status qmatvec_km4o_tiled(const uint8_t *tiled, const uint16_t *lut, const uint16_t *ocol,
                              const int8_t *oval, const uint16_t *oscale, int64_t N, int64_t K, int nout,
                              const void *x, qmv_dtype xdt, int B, float *y, void *stream);

/* Reconstruct W_hat [N][K] fp32 from codes and plane (every reconstructed
 * weight is exact in fp32, except affine int4, where s * u + b is rounded
 * once to the nearest fp32) [S3 "Theoretical size" for the plane shapes].
 * QMV_INT8KM: N % 32 == 0. */
qmv_status qdequant(qmv_format fmt, const void *codes, const void *plane, int64_t N, int64_t K,
                    float *W_hat, void *stream);

/* ---------------------------------------------------------------------- */
/* Mixture of experts: routed-expert gather [S1 sec. 1 (gather_qmm over    */
/* expert slabs blocked along K, [1,1,1,32]); S2 sec. 1 (only routed       */
/* experts are kernelized)].                                              */
/* ---------------------------------------------------------------------- */

/* Top-k routing: logits [T][E] fp32 -> ids [T][topk] int32 (largest logit
 * first, equal logits in increasing id order) and weights [T][topk] fp32,
 * the softmax over the selected logits. 1 <= T <= 64, 1 <= topk <= min(E, 64),
 * E <= 4096. NaN logits rank below every number (ids stay valid expert
 * indices; the weights of such a token are then unspecified). */
qmv_status qmoe_route(const float *logits, int T, int E, int topk,
                      int32_t *ids, float *weights, void *stream);

/* Bytes of workspace gather_qmatvec needs for these sizes (0 if none; the
 * current kernels need none for any epilogue). */
size_t gather_qmatvec_workspace_bytes(int T, int topk, int E, int64_t N, qmv_epilogue epi);

/* Matvec against the experts chosen in ids, reading each chosen expert's
 * weights once however many tokens chose it.
 *  codes/plane: E stacked expert matrices [E][N][...] in `fmt`'s layout.
 *  x: x_per_slot == 0: [T][K] (one input per token, shared by its slots);
 *     x_per_slot == 1: [T][topk][K] (one input per token and slot).
 *  ids [T][topk] int32 in [0, E) (an id below 0 or at least E is read as 0
 *  or E - 1: never a memory access outside the slabs); weights [T][topk]
 *  fp32 (COMBINE only).
 *  epi == QMV_EPI_NONE:    y fp32 [T][topk][N].
 *  epi == QMV_EPI_SWIGLU:  rows [0, N/2) are gate, [N/2, N) up; y fp16
 *                          [T][topk][N/2] = fp16(silu(gate) * up); N even.
 *  epi == QMV_EPI_COMBINE: y fp32 [T][N] = sum over slots of
 *                          weights[t][slot] * (W[ids[t][slot]] x)[n].
 * 1 <= T <= 8, 1 <= topk <= min(E, 64), E <= 4096; 32 <= K <= 8192 (4096
 * for INT8 and INT8KM), K % 32 == 0. INT8KM: N % 32 == 0 (each expert's
 * tables cover groups of 32 rows; with SWIGLU, N % 64 == 0 so the gate and up
 * halves are whole groups). COMBINE sums the slots of a token in slot order,
 * so the result does not depend on scheduling. The workspace, if
 * gather_qmatvec_workspace_bytes(...) is nonzero, must hold that many
 * bytes, 256-byte aligned; otherwise it may be NULL. */
qmv_status gather_qmatvec(qmv_format fmt, const void *codes, const void *plane,
                          int E, int64_t N, int64_t K,
                          const void *x, qmv_dtype xdt, int x_per_slot,
                          int T, int topk, const int32_t *ids, const float *weights,
                          qmv_epilogue epi, void *y, void *workspace, size_t ws_bytes,
                          void *stream);

/* One decode MoE FFN layer: top-k routing (fused into the gate/up gather
 * for T == 1, its own launch otherwise), the gate/up gather with the SwiGLU
 * epilogue, then the down gather with the weighted combine [S1 sec. 1: routed experts' gather_qmm; S2 sec. 1:
 * gate/up and down of the routed experts only; the SwiGLU FFN of the
 * expert, silu(gate) * up, then down].
 *  gu_codes/gu_plane: [E][2I][H] in `fmt`'s layout, gate rows [0, I) and
 *                     up rows [I, 2I) of each expert.
 *  dn_codes/dn_plane: [E][H][I].
 *  logits [T][E] fp32; x [T][H] fp16.
 *  Outputs: ids [T][topk] int32 and weights [T][topk] fp32 exactly as
 *  qmoe_route; h [T][topk][I] fp16 = fp16(silu(gate) * up) per slot; y
 *  [T][H] fp32 = sum over slots (in slot order) of weights * (W_down h).
 * 1 <= T <= 8, 1 <= topk <= min(E, 64), E <= 4096; H and I multiples of 32
 * in [32, 8192] (4096 for INT8 and INT8KM; the int8 k-means tables then
 * cover 32-row groups of every expert matrix). Buffers must not overlap. */
qmv_status qmoe_ffn(qmv_format fmt, const void *gu_codes, const void *gu_plane,
                    const void *dn_codes, const void *dn_plane, int E, int64_t H, int64_t I,
                    const float *logits, const void *x, int T, int topk,
                    int32_t *ids, float *weights, void *h, float *y, void *stream);

/* ---------------------------------------------------------------------- */
/* Around the lm_head matvec ["coreai-optimization reference", "The LM     */
/* head + embeddings": the fused int8 head + argmax kernel path, and the  */
/* front-end embedding table as a plain int8 per-row dequant-gather].     */
/* ---------------------------------------------------------------------- */

/* Bytes of workspace qmatvec_argmax needs for N rows and batch B (0 for
 * invalid sizes). */
size_t qmatvec_argmax_workspace_bytes(int64_t N, int B);

/* Fused matvec + argmax: for each batch row b, idx[b] = the row n with the
 * largest y[b][n] = sum_k dequant(W)[n][k] * x[b][k] (fp32 accumulation, as
 * qmatvec_*), the lowest n among equal largest values, and val[b] = that
 * y[b][n]. The matvec (the kernel qmatvec_* runs for the shape, so y is
 * bit-identical to its output) writes y into the workspace (the caller
 * allocates no logits) and a second launch takes each row's argmax. codes/plane as for
 * qmatvec_* of `fmt`; x fp16 [B][K]; idx int32 [B]; val fp32 [B]; NaN
 * values are not ordered. 1 <= B <= 8; the shapes of the batch-1..8 dot
 * product path (K multiple of 32, up to 8192 for 4-bit formats and 4096
 * for int8 and int8 k-means, and at B > 2 the register budget of that path;
 * QMV_INT8KM also N % 32 == 0; QMV_E_SHAPE otherwise). workspace >=
 * qmatvec_argmax_workspace_bytes(N, B) (128 bytes + B * N fp32), 8-byte
 * aligned; calls sharing a workspace must not overlap. */
qmv_status qmatvec_argmax(qmv_format fmt, const void *codes, const void *plane, int64_t N, int64_t K,
                          const void *x, int B, int32_t *idx, float *val,
                          void *workspace, size_t ws_bytes, void *stream);

/* qmatvec_argmax for a km4 head on the row-tiled code plane (qtile_km4):
 * the qmatvec_km4_tiled kernels write no logits; each workgroup stores the
 * largest (value, lowest row) key of its rows per batch row into the
 * workspace (8 * B * ceil(N / 64) bytes at most), and one small launch takes
 * the largest key. tiled/lut/x/B/K as qmatvec_km4_tiled (1 <= B <= 4, x
 * fp16); idx, val, the workspace size and alignment, and the tie and NaN
 * rules as qmatvec_argmax. */
qmv_status qmatvec_argmax_km4_tiled(const uint8_t *tiled, const uint16_t *lut, int64_t N, int64_t K,
                                    const void *x, int B, int32_t *idx, float *val,
                                    void *workspace, size_t ws_bytes, void *stream);

/* qmatvec_argmax without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, results and kernels as
 * qmatvec_argmax; the workspace is a fixed device array of
 * qmatvec_argmax_noalloc_max_bytes() bytes (16 MiB) inside the library, one
 * copy per GPU, held until the process ends. Sizes whose workspace
 * (qmatvec_argmax_workspace_bytes(N, B)) would not fit return
 * QMV_E_WORKSPACE before anything is launched (the 248320-row head fits up
 * to B = 8). Nothing is allocated or freed. Every call on one GPU uses that
 * GPU's array: calls that overlap on one GPU (other streams, other host
 * threads) race and must be serialized by the caller. The first call on a
 * device looks up the array's address (QMV_E_LAUNCH if that fails). */
qmv_status qmatvec_argmax_noalloc(qmv_format fmt, const void *codes, const void *plane, int64_t N, int64_t K,
                                  const void *x, int B, int32_t *idx, float *val, void *stream);
size_t qmatvec_argmax_noalloc_max_bytes(void);

/* Embedding table packer: W [V][H] (fp16 or fp32) -> codes int8 [V][H] and
 * one fp16 scale per row: s = fp16(amax / 127), q = clamp(rint(w / s),
 * -127, 127) (an all-zero row has s = 0, q = 0). */
qmv_status qpack_int8_rows(const void *W, qmv_dtype wdt, int64_t V, int64_t H,
                           int8_t *codes, uint16_t *scale, void *stream);

/* Embedding dequant-gather: out fp16 [T][H], out[t][h] = fp16(codes[ids[t]][h]
 * * scale[ids[t]]) (exact product, one rounding to nearest even). An id
 * outside [0, V) yields a zero row. H % 8 == 0, 0 <= T <= 65535 (T == 0 does
 * nothing; ids and out may then be NULL); codes 8-byte, out 16-byte aligned. */
qmv_status qembed_gather_int8(const int8_t *codes, const uint16_t *scale, int64_t V, int64_t H,
                              const int32_t *ids, int64_t T, void *out, void *stream);

/* ---------------------------------------------------------------------- */
/* Measurement aid: read `bytes` (a multiple of 16) from buf with 128-bit   */
/* loads and write one checksum word per workgroup to sink[0..grid); the   */
/* practical HBM read ceiling for the kernels above. sink must hold        */
/* qmv_stream_read_sink_words(bytes) uint32 words.                          */
/* ---------------------------------------------------------------------- */
size_t qmv_stream_read_sink_words(size_t bytes);
qmv_status qmv_stream_read(const void *buf, size_t bytes, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QMV_H */
