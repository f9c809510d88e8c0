// Fused dequantize-matvec y[b][n] = sum_k dequant(W)[n][k] * x[b][k]
// ("Dense-path int4km coverage + flagship Qwen3.6-35B - session findings &
// methods", sections 1 and 8: one fused decode matvec whose structure is the
// same for every 4-bit format, only the dequant differs).
//
// gfx950 design. The op reads each packed weight byte once and is bound by
// HBM bandwidth at small batch. A wavefront owns whole rows: lane l of a row
// group loads 16-byte chunks l, l + LPR, ... of the row's code plane, so one
// wave-wide load instruction covers 64 x 16 B of contiguous bytes. The x
// slices that belong to the lane's chunks are loaded into registers once and
// reused for every row the wave visits. Decoding happens in registers (or
// from a 32-byte per-row table in LDS for km4), products accumulate in fp32
// via v_dot2_f32_f16 and the block scale multiplies the block sum. Row
// groups are reduced across their lanes with cross-lane shuffles.
#include "qmv_device.h"
#include "qmv_launch.h"

namespace qmv {

// ---------------------------------------------------------------------------
// Fast path: x fp16 in registers.
//   FMT  format, BT batch width compiled (runtime B <= BT, extra rows zero),
//   LPR  lanes per row (64, 32 or 16), CPL chunks per lane, R row groups per
//   iteration, ITERS iterations per wave, WAVES waves per workgroup.
// Each wave handles ITERS * R * (64 / LPR) consecutive rows and exits; a
// workgroup's rows are consecutive, so every workgroup streams one contiguous
// stretch of the code plane. The x slices are loaded once per wave, so ITERS
// grows with the batch width to amortize them.
// ---------------------------------------------------------------------------
// argmax workspace: the kArgmaxHeader-word header, then y [B][N] fp32

// int8 outliers added to 4-bit k-means rows ("Kernel campaign - session
// handoff", NEXT per lever, Stream D): per row, n columns (increasing), int8
// values and one fp16 scale; the row's weight is the table value plus the
// outlier, so y gains scale * q * x[col] per outlier.
struct OutlierArgs {
    const uint16_t *col = nullptr;   // [N][n]
    const int8_t *val = nullptr;     // [N][n]
    const uint16_t *scale = nullptr; // [N]
    int n = 0;
};

// hdr: if not null, the first wave zeroes kArgmaxHeader words there (the
// per-row maxima and the workgroup counter of the argmax launch that follows
// this matvec in the fused lm_head + argmax).
// OUTL: add the int8 outliers of each row (4-bit k-means rows only).
template <int FMT, int BT, int LPR, int CPL, int R, int ITERS, int WAVES, bool FULLK,
          bool OUTL = false>
__global__ __launch_bounds__(64 * WAVES) void mv_fast(const uint8_t *__restrict__ codes,
                                                      const void *__restrict__ plane, int64_t N, int K,
                                                      const _Float16 *__restrict__ x, int B,
                                                      float *__restrict__ y, uint64_t *__restrict__ hdr,
                                                      OutlierArgs ol) {
    constexpr int RPW = kWave / LPR;            // rows per row group
    constexpr int XW = ChunkTraits<FMT>::kXWords;
    constexpr int ROWS_IT = R * RPW;            // rows per iteration
    // with one wave per workgroup and one row per row group the km4 tables sit
    // at compile-time LDS offsets
    constexpr bool KM4_IMM = (FMT == KM4) && WAVES == 1 && RPW == 1;
    // int8 k-means: an iteration's rows share one 256-entry table (rows come in
    // groups of 32 and an iteration's rows never straddle two groups); one wave
    // per workgroup keeps the table at a compile-time LDS address
    constexpr bool KM8 = (FMT == INT8KM);
    static_assert(!KM8 || (WAVES == 1 && 32 % ROWS_IT == 0), "int8km: one wave, rows within a group");
    constexpr int LUT_WORDS = KM8 ? 128 : ROWS_IT * 8;   // table dwords per iteration
    constexpr int LUT_PER_LANE = (LUT_WORDS + kWave - 1) / kWave;
    __shared__ __align__(16) _Float16 lut_lds[(FMT == KM4) ? WAVES * ROWS_IT * 16 : (KM8 ? 256 : 1)];

    const int lane = threadIdx.x & 63;
    const int wave = (WAVES == 1) ? 0 : (threadIdx.x >> 6);
    const int sub = lane % LPR;
    const int rsub = lane / LPR;
    // FULLK: K fills the lanes exactly (chunks per row == LPR * CPL)
    const int cpr = FULLK ? LPR * CPL : ((FMT == INT8 || KM8) ? K / 16 : K / 32);   // chunks per row
    const int nb = K / 32;                                                          // blocks per row
    const uint32_t row_bytes = (FMT == INT8 || KM8) ? (uint32_t)K : (uint32_t)K / 2;
    const int64_t wrow0 = ((int64_t)blockIdx.x * WAVES + wave) * ROWS_IT * ITERS;
    if (hdr != nullptr && blockIdx.x == 0 && threadIdx.x < kArgmaxHeader) hdr[threadIdx.x] = 0;
    if (wrow0 >= N) return;

    // Loads of one iteration. Wave-uniform bases, 32-bit per-lane offsets.
    // Loads are unconditional: a row past the end reads row N-1 and a chunk
    // past the end of the row reads chunk 0; their x slices are zero and their
    // rows are never stored, so they contribute nothing.
    constexpr bool AFF = (FMT == INT4AFF);
    uint4 cw[R][CPL];
    float sc[R][CPL];
    float bi[AFF ? R : 1][AFF ? CPL : 1];   // affine bias per block
    uint32_t lutv[LUT_PER_LANE];
    // outliers (n >= 1): lane `sub` prefetches outlier min(sub, n - 1) of each row
    uint32_t ocol_r[OUTL ? R : 1];
    int32_t oval_r[OUTL ? R : 1];
    uint32_t osc_r[OUTL ? R : 1];
    auto issue_loads = [&](int64_t row0) {
        const int last = (int)((N - 1 - row0) < ROWS_IT ? (N - 1 - row0) : ROWS_IT);   // last valid row offset
        const uint8_t *cbase = codes + row0 * (int64_t)row_bytes;
#pragma unroll
        for (int g = 0; g < R; g++) {
            int rr = g * RPW + rsub;
            rr = rr <= last ? rr : last;
#pragma unroll
            for (int j = 0; j < CPL; j++) {
                int c = sub + LPR * j;
                int cc = (FULLK || c < cpr) ? c : 0;
                cw[g][j] = load_stream16(cbase + ((uint32_t)rr * row_bytes + (uint32_t)cc * 16u));
                if constexpr (FMT == INT4 || FMT == INT8) {
                    const uint16_t *s = reinterpret_cast<const uint16_t *>(plane) + row0 * nb;
                    int blk = (FMT == INT8) ? cc / 2 : cc;
                    sc[g][j] = f16_bits_to_f32(s[(uint32_t)rr * (uint32_t)nb + (uint32_t)blk]);
                } else if constexpr (FMT == FP4) {
                    const uint8_t *s = reinterpret_cast<const uint8_t *>(plane) + row0 * nb;
                    sc[g][j] = e8m0_to_f32(s[(uint32_t)rr * (uint32_t)nb + (uint32_t)cc]);
                } else if constexpr (AFF) {
                    const uint32_t *s = reinterpret_cast<const uint32_t *>(plane) + row0 * nb;
                    const uint32_t wd = s[(uint32_t)rr * (uint32_t)nb + (uint32_t)cc];
                    sc[g][j] = f16_bits_to_f32((uint16_t)(wd & 0xFFFFu));
                    bi[g][j] = f16_bits_to_f32((uint16_t)(wd >> 16));
                } else {
                    sc[g][j] = 1.f;
                }
            }
        }
        if constexpr (FMT == KM4) {
            // this iteration's tables: 8 dwords per row, LUT_PER_LANE dwords per lane
            const uint32_t *lsrc = reinterpret_cast<const uint32_t *>(plane) + row0 * 8;
#pragma unroll
            for (int q = 0; q < LUT_PER_LANE; q++) {
                int i = q * kWave + lane;
                int rr = (i < LUT_WORDS ? i : LUT_WORDS - 1) / 8;
                rr = rr <= last ? rr : last;
                lutv[q] = lsrc[rr * 8 + (i % 8)];
            }
        } else if constexpr (KM8) {
            const uint32_t *lsrc = reinterpret_cast<const uint32_t *>(plane) + (row0 / 32) * 128;
#pragma unroll
            for (int q = 0; q < LUT_PER_LANE; q++) lutv[q] = lsrc[q * kWave + lane];
        }
        if constexpr (OUTL) {
            const int o = sub < ol.n ? sub : ol.n - 1;
#pragma unroll
            for (int g = 0; g < R; g++) {
                int rr = g * RPW + rsub;
                rr = rr <= last ? rr : last;
                const int64_t row = row0 + rr;
                ocol_r[g] = ol.col[row * ol.n + o];
                oval_r[g] = ol.val[row * ol.n + o];
                osc_r[g] = ol.scale[row];
            }
        }
    };

    // x slices for this lane's chunks, every batch row (rows b >= B are zero)
    uint32_t xr[CPL][BT][XW];
#pragma unroll
    for (int j = 0; j < CPL; j++) {
        int c = sub + LPR * j;
#pragma unroll
        for (int b = 0; b < BT; b++)
            load_x_slice<FMT>(x + (size_t)(b < B ? b : 0) * K, c, (FULLK || c < cpr) && (BT == 1 || b < B),
                              xr[j][b]);
    }
    // affine blocks add bias * (sum of the block's x)
    float xsum[AFF ? CPL : 1][AFF ? BT : 1];
    if constexpr (AFF) {
#pragma unroll
        for (int j = 0; j < CPL; j++)
#pragma unroll
            for (int b = 0; b < BT; b++) xsum[j][b] = x_slice_sum<XW>(xr[j][b]);
    }

    issue_loads(wrow0);
#pragma unroll 1
    for (int it = 0; it < ITERS; it++) {
        const int64_t row0 = wrow0 + (int64_t)it * ROWS_IT;
        if (row0 >= N) break;
        // take this iteration's data, then start the next iteration's loads so
        // they are in flight while this one computes
        uint4 cwc[R][CPL];
        float scc[R][CPL];
        float bic[AFF ? R : 1][AFF ? CPL : 1];
#pragma unroll
        for (int g = 0; g < R; g++)
#pragma unroll
            for (int j = 0; j < CPL; j++) {
                cwc[g][j] = cw[g][j];
                scc[g][j] = sc[g][j];
                if constexpr (AFF) bic[g][j] = bi[g][j];
            }
        _Float16 *lut_w = lut_lds + wave * ROWS_IT * 16;
        if constexpr (FMT == KM4 || KM8) {
            uint32_t *ldst = reinterpret_cast<uint32_t *>(lut_w);
#pragma unroll
            for (int q = 0; q < LUT_PER_LANE; q++) {
                int i = q * kWave + lane;
                if (LUT_WORDS % kWave == 0 || i < LUT_WORDS) ldst[i] = lutv[q];
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        // outliers: this iteration's x values at the outlier columns, gathered
        // now so the loads are in flight during the dot products
        float ot[OUTL ? R : 1];
        _Float16 ox[OUTL ? R : 1][OUTL ? BT : 1];
        if constexpr (OUTL) {
#pragma unroll
            for (int g = 0; g < R; g++) {
                ot[g] = sub < ol.n ? (float)oval_r[g] * f16_bits_to_f32((uint16_t)osc_r[g]) : 0.f;   // exact
#pragma unroll
                for (int b = 0; b < BT; b++) ox[g][b] = x[(size_t)(b < B ? b : 0) * K + ocol_r[g]];
            }
        }
        if (ITERS > 1 && it + 1 < ITERS && row0 + ROWS_IT < N) issue_loads(row0 + ROWS_IT);

        float acc[R * BT];
#pragma unroll
        for (int g = 0; g < R; g++) {
#pragma unroll
            for (int b = 0; b < BT; b++) {
                float a = 0.f;
#pragma unroll
                for (int j = 0; j < CPL; j++) {
                    float d;
                    if constexpr (FMT == INT4) d = chunk_dot_int4(cwc[g][j], xr[j][b]);
                    else if constexpr (AFF) d = chunk_dot_int4<true>(cwc[g][j], xr[j][b]);
                    else if constexpr (FMT == FP4) d = chunk_dot_fp4(cwc[g][j], xr[j][b]);
                    else if constexpr (FMT == INT8) d = chunk_dot_int8(cwc[g][j], xr[j][b]);
                    else if constexpr (KM8)
                        d = chunk_dot_int8km_imm(cwc[g][j], reinterpret_cast<const char *>(lut_lds), xr[j][b]);
                    else if constexpr (KM4_IMM)
                        d = chunk_dot_km4_imm(cwc[g][j], reinterpret_cast<const char *>(lut_lds) + g * 32, xr[j][b]);
                    else d = chunk_dot_km4(cwc[g][j], lut_w + (g * RPW + rsub) * 16, xr[j][b]);
                    a = (FMT == KM4 || KM8) ? a + d : __builtin_fmaf(d, scc[g][j], a);
                    if constexpr (AFF) a = __builtin_fmaf(xsum[j][b], bic[g][j], a);
                }
                acc[g * BT + b] = a;
            }
        }
        if constexpr (OUTL) {
            // lane `sub` of a row takes its outliers sub (prefetched), sub + LPR, ...
#pragma unroll
            for (int g = 0; g < R; g++)
#pragma unroll
                for (int b = 0; b < BT; b++)
                    if (BT == 1 || b < B) acc[g * BT + b] = __builtin_fmaf(ot[g], (float)ox[g][b], acc[g * BT + b]);
            const int last = (int)((N - 1 - row0) < ROWS_IT ? (N - 1 - row0) : ROWS_IT);
#pragma unroll
            for (int g = 0; g < R; g++) {
                int rr = g * RPW + rsub;
                rr = rr <= last ? rr : last;
                const int64_t row = row0 + rr;
                const float so = f16_bits_to_f32(ol.scale[row]);
                for (int o = sub + LPR; o < ol.n; o += LPR) {
                    const float t = (float)ol.val[row * ol.n + o] * so;   // exact: 8 x 11 significant bits
                    const int col = ol.col[row * ol.n + o];
#pragma unroll
                    for (int b = 0; b < BT; b++)
                        if (BT == 1 || b < B)
                            acc[g * BT + b] = __builtin_fmaf(t, (float)x[(size_t)b * K + col], acc[g * BT + b]);
                }
            }
        }
        if constexpr ((FMT == KM4 || KM8) && ITERS > 1) {
            // the next iteration rewrites the tables: keep this iteration's reads above it
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        using Red = GroupReduce<R * BT, LPR>;
        Red::run(acc, lane);
        if (Red::writer(lane)) {
            const int base = Red::base(lane);
#pragma unroll
            for (int j = 0; j < Red::live; j++) {
                int idx = base + j, g = idx / BT, b = idx % BT;
                int64_t row = row0 + g * RPW + rsub;
                if (row < N && b < B) y[(size_t)b * N + row] = acc[j];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Batch 2-8 on matrices short of the tall shape, scale formats (int4, fp4,
// int8), rows of whole 64-chunk strides: x staged once per workgroup in LDS.
// mv_fast holds every x slice a lane needs in registers (CPL * BT * XW words,
// 128 at fp4 4096 x 4096 and B = 4, one wave per SIMD) and every wave loads
// its own copy of x from L2, four times its code bytes there. Here the eight
// waves of a workgroup share one LDS copy of x ([BT][chunk] slots of XW words
// plus 4 words of padding, so the 16-byte reads of consecutive lanes hit
// distinct banks), each wave owns one row, and a lane reads each x slice just
// before the chunks that use it. The arithmetic and its order per row are
// mv_fast's, so results are bit-identical to it.
// ---------------------------------------------------------------------------
constexpr int kXsWaves = 8;   // waves per workgroup, one row each

template <int FMT>
__host__ __device__ constexpr int xstage_pitch() { return ChunkTraits<FMT>::kXWords + 4; }   // words per x slot

template <int FMT, int BT, int CPL>
__global__ __launch_bounds__(64 * kXsWaves) void mv_xstage(const uint8_t *__restrict__ codes,
                                                           const void *__restrict__ plane, int64_t N, int K,
                                                           const _Float16 *__restrict__ x, int B,
                                                           float *__restrict__ y, uint64_t *__restrict__ hdr) {
    static_assert(FMT == INT4 || FMT == FP4 || FMT == INT8, "scale formats only");
    extern __shared__ __align__(16) uint32_t xl[];
    constexpr int XW = ChunkTraits<FMT>::kXWords;
    constexpr int PITCH = xstage_pitch<FMT>();
    constexpr int CPR = 64 * CPL;   // chunks per row (the launch checks K)
    const int nb = K / 32;
    const uint32_t row_bytes = (FMT == INT8) ? (uint32_t)K : (uint32_t)K / 2;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (hdr != nullptr && blockIdx.x == 0 && tid < kArgmaxHeader) hdr[tid] = 0;
    for (int i = tid; i < BT * CPR; i += 64 * kXsWaves) {
        const int b = i / CPR, c = i - b * CPR;
        uint32_t w[XW];
        load_x_slice<FMT>(x + (size_t)(b < B ? b : 0) * K, c, b < B, w);   // rows b >= B are zero
        uint4 *dst = reinterpret_cast<uint4 *>(xl + i * PITCH);
#pragma unroll
        for (int q = 0; q < XW / 4; q++) dst[q] = make_uint4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
    }
    __syncthreads();
    const int64_t row = (int64_t)blockIdx.x * kXsWaves + wave;
    if (row >= N) return;
    uint4 cw[CPL];
    float sc[CPL];
#pragma unroll
    for (int j = 0; j < CPL; j++) {
        const int c = lane + 64 * j;
        cw[j] = load_stream16(codes + row * (int64_t)row_bytes + (uint32_t)c * 16u);
        if constexpr (FMT == FP4)
            sc[j] = e8m0_to_f32(reinterpret_cast<const uint8_t *>(plane)[row * nb + c]);
        else
            sc[j] = f16_bits_to_f32(reinterpret_cast<const uint16_t *>(plane)[row * nb + (FMT == INT8 ? c / 2 : c)]);
    }
    float acc[BT];
#pragma unroll
    for (int b = 0; b < BT; b++) acc[b] = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; j++) {
#pragma unroll
        for (int b = 0; b < BT; b++) {
            uint32_t xs[XW];
            const uint4 *src = reinterpret_cast<const uint4 *>(xl + (b * CPR + lane + 64 * j) * PITCH);
#pragma unroll
            for (int q = 0; q < XW / 4; q++) {
                const uint4 v = src[q];
                xs[4 * q] = v.x;
                xs[4 * q + 1] = v.y;
                xs[4 * q + 2] = v.z;
                xs[4 * q + 3] = v.w;
            }
            float d;
            if constexpr (FMT == FP4) d = chunk_dot_fp4(cw[j], xs);
            else if constexpr (FMT == INT4) d = chunk_dot_int4(cw[j], xs);
            else d = chunk_dot_int8(cw[j], xs);
            acc[b] = __builtin_fmaf(d, sc[j], acc[b]);
        }
    }
    using Red = GroupReduce<BT, 64>;
    Red::run(acc, lane);
    if (Red::writer(lane)) {
        const int base = Red::base(lane);
#pragma unroll
        for (int j = 0; j < Red::live; j++) {
            const int b = base + j;
            if (b < B) y[(size_t)b * N + row] = acc[j];
        }
    }
}

// LDS bytes of mv_xstage's x copy; 0 where the kernel does not take the shape
// (formats with tables or a bias, rows not a whole number of 64-chunk strides,
// more than 64 KiB of x).
template <int FMT, int BT, int CPL>
static size_t xstage_lds(int K) {
    if constexpr (FMT != INT4 && FMT != FP4 && FMT != INT8) return 0;
    else {
        const int cpr = (FMT == INT8) ? K / 16 : K / 32;
        if (cpr != 64 * CPL) return 0;
        const size_t b = (size_t)BT * cpr * xstage_pitch<FMT>() * 4;
        return b <= 64 * 1024 ? b : 0;
    }
}

// Argmax over each batch row of y [B][N] -> (index, value). A grid of (G, B)
// workgroups, G <= kArgmaxGroups: each takes every G-th stretch of
// kArgmaxStretch values of its row, sixteen independent loads per thread in
// flight, keeps the largest key (value order, then the lower row), and merges
// it into the header word of its row with a 64-bit atomic max. The last of a
// row's G workgroups to finish (by the row's header counter, zeroed by the
// matvec launch before) turns that row's maximum into (index, value). Few
// workgroups per row keep the same-address atomics short: with 61 workgroups
// per row of the 248320-row head, their serialised acquire-release updates
// cost more than reading the 8 MB of logits at batch 8.
constexpr int kArgmaxStretch = 16384;   // values per workgroup and pass (16 per thread)
constexpr int kArgmaxGroups = 16;       // most workgroups per batch row

__global__ __launch_bounds__(1024) void argmax_rows_kernel(const float *__restrict__ y, int64_t N, int B,
                                                           uint64_t *__restrict__ hdr, int32_t *__restrict__ idx,
                                                           float *__restrict__ val) {
    const int b = blockIdx.y;
    const int G = gridDim.x;
    const float *yr = y + (int64_t)b * N;
    uint64_t k = 0;
    for (int64_t i0 = (int64_t)blockIdx.x * kArgmaxStretch + threadIdx.x; i0 < N; i0 += (int64_t)G * kArgmaxStretch) {
        float v[kArgmaxStretch / 1024];
#pragma unroll
        for (int u = 0; u < kArgmaxStretch / 1024; u++) {
            const int64_t i = i0 + u * 1024;
            v[u] = yr[i < N ? i : 0];
        }
#pragma unroll
        for (int u = 0; u < kArgmaxStretch / 1024; u++) {
            const int64_t i = i0 + u * 1024;
            const uint64_t key = i < N ? argmax_key(v[u], i) : 0;
            k = key > k ? key : k;
        }
    }
    k = wave_max_u64(k);
    __shared__ uint64_t red[16];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = k;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 0; w < 16; w++) k = red[w] > k ? red[w] : k;
        __hip_atomic_fetch_max(&hdr[b], k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t done = __hip_atomic_fetch_add(&hdr[8 + b], (uint64_t)1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (done + 1 == (uint64_t)G) {
            const uint64_t kk = __hip_atomic_load(&hdr[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            idx[b] = argmax_key_row(kk);
            val[b] = argmax_key_value(kk);
        }
    }
}

// ---------------------------------------------------------------------------
// Generic path: any K % 32 == 0, B <= 8, x fp16 or fp32. One wave per row,
// decode to fp32 and fma against x read through the cache.
// ---------------------------------------------------------------------------
template <int FMT>
__device__ __forceinline__ void decode_chunk_f32(const uint8_t *__restrict__ codes, const void *__restrict__ plane,
                                                 int64_t row, int K, int c, float (&w)[32]) {
    const int nb = K / 32;
    if constexpr (FMT == INT8KM) {
        const uint8_t *p = codes + row * (int64_t)K + (int64_t)c * 16;
        const uint16_t *lut = reinterpret_cast<const uint16_t *>(plane) + (row / 32) * 256;
#pragma unroll
        for (int i = 0; i < 16; i++) w[i] = f16_bits_to_f32(lut[p[i]]);
    } else if constexpr (FMT == INT8) {
        const int8_t *p = reinterpret_cast<const int8_t *>(codes) + row * (int64_t)K + (int64_t)c * 16;
        float s = f16_bits_to_f32(reinterpret_cast<const uint16_t *>(plane)[row * nb + c / 2]);
#pragma unroll
        for (int i = 0; i < 16; i++) w[i] = s * (float)p[i];
    } else {
        uint4 cw = *reinterpret_cast<const uint4 *>(codes + row * (int64_t)(K / 2) + (int64_t)c * 16);
        uint32_t wd[4] = {cw.x, cw.y, cw.z, cw.w};
        if constexpr (FMT == FP4) {
            float s = e8m0_to_f32(reinterpret_cast<const uint8_t *>(plane)[row * nb + c]);
#pragma unroll
            for (int d = 0; d < 4; d++) {
                h2 v[4] = {__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd[d], 1.0f, 0),
                           __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd[d], 1.0f, 1),
                           __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd[d], 1.0f, 2),
                           __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd[d], 1.0f, 3)};
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    w[8 * d + 2 * i] = (float)v[i].x * s;
                    w[8 * d + 2 * i + 1] = (float)v[i].y * s;
                }
            }
        } else if constexpr (FMT == INT4) {
            float s = f16_bits_to_f32(reinterpret_cast<const uint16_t *>(plane)[row * nb + c]);
#pragma unroll
            for (int d = 0; d < 4; d++)
#pragma unroll
                for (int i = 0; i < 8; i++) w[8 * d + i] = s * (float)((int)((wd[d] >> (4 * i)) & 15u) - 8);
        } else if constexpr (FMT == INT4AFF) {
            // s * u + b with one rounding (the fp32 value nearest the exact one)
            const uint32_t sb = reinterpret_cast<const uint32_t *>(plane)[row * nb + c];
            const float s = f16_bits_to_f32((uint16_t)(sb & 0xFFFFu)), b = f16_bits_to_f32((uint16_t)(sb >> 16));
#pragma unroll
            for (int d = 0; d < 4; d++)
#pragma unroll
                for (int i = 0; i < 8; i++) w[8 * d + i] = __builtin_fmaf(s, (float)((wd[d] >> (4 * i)) & 15u), b);
        } else {
            const uint16_t *lut = reinterpret_cast<const uint16_t *>(plane) + row * 16;
#pragma unroll
            for (int d = 0; d < 4; d++)
#pragma unroll
                for (int i = 0; i < 8; i++) w[8 * d + i] = f16_bits_to_f32(lut[(wd[d] >> (4 * i)) & 15u]);
        }
    }
}

template <typename XT>
__device__ __forceinline__ float load_x(const XT *p) { return (float)*p; }

template <int FMT, typename XT, bool OUTL = false>
__global__ __launch_bounds__(256) void mv_generic(const uint8_t *__restrict__ codes,
                                                  const void *__restrict__ plane, int64_t N, int K,
                                                  const XT *__restrict__ x, int B, float *__restrict__ y,
                                                  OutlierArgs ol) {
    constexpr int E = ChunkTraits<FMT>::kElems;
    const int lane = threadIdx.x & 63;
    const int64_t waves_total = (int64_t)gridDim.x * (blockDim.x >> 6);
    const int cpr = K / E;
    for (int64_t row = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); row < N; row += waves_total) {
        float acc[8];
#pragma unroll
        for (int b = 0; b < 8; b++) acc[b] = 0.f;
        for (int c = lane; c < cpr; c += kWave) {
            float w[32];
            decode_chunk_f32<FMT>(codes, plane, row, K, c, w);
#pragma unroll
            for (int b = 0; b < 8; b++) {
                if (b < B) {
                    const XT *xp = x + (size_t)b * K + (size_t)c * E;
#pragma unroll
                    for (int i = 0; i < E; i++) acc[b] = __builtin_fmaf(w[i], load_x(xp + i), acc[b]);
                }
            }
        }
        if constexpr (OUTL) {
            const float so = f16_bits_to_f32(ol.scale[row]);
            for (int o = lane; o < ol.n; o += kWave) {
                const float t = (float)ol.val[row * ol.n + o] * so;
                const int col = ol.col[row * ol.n + o];
#pragma unroll
                for (int b = 0; b < 8; b++)
                    if (b < B) acc[b] = __builtin_fmaf(t, load_x(x + (size_t)b * K + col), acc[b]);
            }
        }
#pragma unroll
        for (int b = 0; b < 8; b++) {
            if (b < B) {
                float s = group_sum<64>(acc[b]);
                if (lane == 0) y[(size_t)b * N + row] = s;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Dequant (test support): one thread per 32-element block.
// ---------------------------------------------------------------------------
template <int FMT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t *__restrict__ codes, const void *__restrict__ plane,
                                                      int64_t N, int K, float *__restrict__ out) {
    const int nb = K / 32;
    int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= N * nb) return;
    int64_t row = gid / nb;
    int blk = (int)(gid % nb);
    float w[32];
    if constexpr (FMT == INT8 || FMT == INT8KM) {
        decode_chunk_f32<FMT>(codes, plane, row, K, 2 * blk, w);
        float w2[32];
        decode_chunk_f32<FMT>(codes, plane, row, K, 2 * blk + 1, w2);
#pragma unroll
        for (int i = 0; i < 16; i++) w[16 + i] = w2[i];
    } else {
        decode_chunk_f32<FMT>(codes, plane, row, K, blk, w);
    }
    float4 *o = reinterpret_cast<float4 *>(out + row * (int64_t)K + (int64_t)blk * 32);
#pragma unroll
    for (int i = 0; i < 8; i++) o[i] = make_float4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
}

// ---------------------------------------------------------------------------
// Host-side dispatch (called from the C ABI after validation).
// ---------------------------------------------------------------------------
static int grid_for_waves(int64_t waves_needed) {
    int64_t cap = (int64_t)device_cu_count() * 32;   // 8 WGs x 4 waves per CU
    int64_t waves = waves_needed < cap ? waves_needed : cap;
    if (waves < 1) waves = 1;
    return (int)((waves + 3) / 4);
}

// Launch shape per format and batch width (rows per iteration R, iterations
// per wave ITERS, waves per workgroup WAVES), chosen by measurement on MI355X
// at the lm_head shape (248320 x 2048) under sustained load. km4 needs one
// wave per workgroup for its compile-time table offsets; more batch rows need
// more rows per wave to amortize the x slices held in registers. TALL (batch
// 1, at least kTallRows rows): 8 rows per wave for the table formats and
// affine int4, which halves the x slice loads per row; shorter matrices keep
// 4 so that enough waves fill the chip, and fewer as rows get longer (RS,
// see short_rows).
constexpr int64_t kTallRows = 32768;
template <int FMT, int BT, bool TALL = false, int RS = 0, int IT = 0> struct LaunchShape {
    static constexpr int R = (RS > 0) ? RS
                           : (BT == 1) ? ((FMT == INT4 || (TALL && FMT != FP4 && FMT != INT8)) ? 8 : 4)
                                       : (BT == 2 ? 4 : (BT == 4 ? ((FMT == KM4) ? 4 : 2) : 1));
    static constexpr int ITERS = (IT > 0) ? IT
                               : (FMT == KM4 || FMT == INT8KM) ? ((BT == 1) ? 1 : (BT == 8 ? 16 : 2))
                                              : ((BT == 1) ? 1 : (BT == 2 ? 2 : (BT == 4 ? 4 : 8)));
    static constexpr int WAVES = (FMT == KM4 || FMT == INT8KM) ? 1 : 4;
};

// Batch 1, fewer than kTallRows rows of at least 1 KiB (4-bit K >= 2048): rows
// per wave by row length, measured on q/o-projection shapes in HIP graphs
// (2048 x 4096: km4 3.75 us at 1 row against 4.89 at 4; fp4 2.78 at 2 against
// 3.75; int4 3.19 at 1 against 4.45 at 8. 4096 x 2048: km4 3.56 at 2 against
// 3.85; int4 3.01 at 4 against 3.32). 0 keeps the LaunchShape default.
template <int FMT>
static int short_rows(int64_t row_bytes) {
    if constexpr (FMT == KM4) return row_bytes >= 2048 ? 1 : (row_bytes >= 1024 ? 2 : 0);
    else if constexpr (FMT == FP4) return row_bytes >= 2048 ? 2 : 0;
    else if constexpr (FMT == INT4 || FMT == INT4AFF) return row_bytes >= 2048 ? 1 : (row_bytes >= 1024 ? 4 : 0);
    else return 0;
}

template <int FMT, int BT, int LPR, int CPL, bool OUTL, bool TALL, int RS = 0, int IT = 0>
static hipError_t launch_shape(const uint8_t *codes, const void *plane, int64_t N, int K, const void *x, int B,
                               float *y, hipStream_t st, uint64_t *hdr, OutlierArgs ol) {
    using S = LaunchShape<FMT, BT, TALL, RS, IT>;
    constexpr int ROWS_WG = S::WAVES * S::R * S::ITERS * (kWave / LPR);
    int64_t grid = (N + ROWS_WG - 1) / ROWS_WG;
    const int cpr = (FMT == INT8 || FMT == INT8KM) ? K / 16 : K / 32;
    if (cpr == LPR * CPL)
        hipLaunchKernelGGL((mv_fast<FMT, BT, LPR, CPL, S::R, S::ITERS, S::WAVES, true, OUTL>),
                           dim3((unsigned)grid), dim3(64 * S::WAVES), 0, st, codes, plane, N, K,
                           reinterpret_cast<const _Float16 *>(x), B, y, hdr, ol);
    else
        hipLaunchKernelGGL((mv_fast<FMT, BT, LPR, CPL, S::R, S::ITERS, S::WAVES, false, OUTL>),
                           dim3((unsigned)grid), dim3(64 * S::WAVES), 0, st, codes, plane, N, K,
                           reinterpret_cast<const _Float16 *>(x), B, y, hdr, ol);
    return hipGetLastError();
}

template <int FMT, int BT, int LPR, int CPL, bool OUTL = false>
static hipError_t launch_fast(const uint8_t *codes, const void *plane, int64_t N, int K, const void *x, int B,
                              float *y, hipStream_t st, uint64_t *hdr = nullptr, OutlierArgs ol = OutlierArgs()) {
    if constexpr (BT == 1) {
        if (N >= kTallRows) return launch_shape<FMT, BT, LPR, CPL, OUTL, true>(codes, plane, N, K, x, B, y, st, hdr, ol);
        if constexpr (LPR == 64) {
            const int rs = short_rows<FMT>((FMT == INT8 || FMT == INT8KM) ? (int64_t)K : (int64_t)K / 2);
            if (rs == 1) return launch_shape<FMT, BT, LPR, CPL, OUTL, false, 1>(codes, plane, N, K, x, B, y, st, hdr, ol);
            if (rs == 2) return launch_shape<FMT, BT, LPR, CPL, OUTL, false, 2>(codes, plane, N, K, x, B, y, st, hdr, ol);
            if (rs == 4) return launch_shape<FMT, BT, LPR, CPL, OUTL, false, 4>(codes, plane, N, K, x, B, y, st, hdr, ol);
        }
    }
    constexpr bool TABLE = (FMT == KM4 || FMT == INT8KM);
    if constexpr ((BT == 2 || BT == 4 || BT == 8) && LPR == 64) {
        // Batch 2-4 on fewer than kTallRows rows: one iteration per wave and
        // about 1024 waves, measured in HIP graphs against the tall-matrix
        // shape (fp4 4096 x 4096 at B = 4: 6.2 us with 4 rows per wave against
        // 9.8 us at 2 rows x 4 iterations; fp4 2048 x 4096: 4.7 us with 2 rows
        // against 9.5; int4 4096 x 2048 at B = 2: 3.5 us against 5.0). The
        // table formats (one wave per workgroup) take 2 rows: km4 2048 x 4096
        // at B = 4: 6.0 us against 8.8; int8 k-means 4096 x 2048: 5.1 against 6.5.
        // Batch 5-8 (matrices the matrix-core path leaves here) takes 2 rows,
        // km4 4 from 4096 rows (4096 x 2048 at B = 8: 6.4 us against 7.2).
        if (N < kTallRows) {
            // x staged in LDS (measured on MI355X in HIP graphs, against this
            // function's register-x shapes below: fp4 4096 x 4096 at B = 2 / 3 / 4:
            // 4.31 / 5.08 / 5.17 us against 4.77 / 5.96 / 6.12; int4 8192 x 4096
            // at B = 4: 8.43 against 13.07; fp4 4096 x 2048 at B = 8: 4.80
            // against 6.40; int8 within 2% either way at 2048 rows)
            if constexpr (!OUTL && (CPL == 1 || CPL == 2 || CPL == 4) && (FMT == INT4 || FMT == FP4 || FMT == INT8)) {
                const size_t lds = xstage_lds<FMT, BT, CPL>(K);
                if (lds > 0) {
                    const int64_t grid = (N + kXsWaves - 1) / kXsWaves;
                    hipLaunchKernelGGL((mv_xstage<FMT, BT, CPL>), dim3((unsigned)grid), dim3(64 * kXsWaves), lds, st,
                                       codes, plane, N, K, reinterpret_cast<const _Float16 *>(x), B, y, hdr);
                    return hipGetLastError();
                }
            }
            if (N >= 4096 && ((!TABLE && BT <= 4) || (FMT == KM4 && BT == 8)))
                return launch_shape<FMT, BT, LPR, CPL, OUTL, false, 4, 1>(codes, plane, N, K, x, B, y, st, hdr, ol);
            if (N >= 2048) return launch_shape<FMT, BT, LPR, CPL, OUTL, false, 2, 1>(codes, plane, N, K, x, B, y, st, hdr, ol);
            return launch_shape<FMT, BT, LPR, CPL, OUTL, false, 1, 1>(codes, plane, N, K, x, B, y, st, hdr, ol);
        }
    }
    return launch_shape<FMT, BT, LPR, CPL, OUTL, false>(codes, plane, N, K, x, B, y, st, hdr, ol);
}

// Register budget for the x slices held per lane (CPL * BT * XW words): the
// batch widths each (LPR, CPL) shape takes on the dot2 path.
template <int FMT, int CPL>
constexpr bool dot2_takes(int B) {
    constexpr int XW = ChunkTraits<FMT>::kXWords;
    return B <= 2 || (B <= 4 && CPL * 4 * XW <= 128) || (B <= 8 && CPL * 8 * XW <= 128);
}

template <int FMT, int LPR, int CPL, bool OUTL = false>
static hipError_t dispatch_b(const uint8_t *codes, const void *plane, int64_t N, int K, const void *x, int B,
                             float *y, hipStream_t st, bool *handled, uint64_t *hdr = nullptr,
                             OutlierArgs ol = OutlierArgs()) {
    *handled = true;
    constexpr int XW = ChunkTraits<FMT>::kXWords;
    if (B == 1) return launch_fast<FMT, 1, LPR, CPL, OUTL>(codes, plane, N, K, x, B, y, st, hdr, ol);
    if (B == 2) return launch_fast<FMT, 2, LPR, CPL, OUTL>(codes, plane, N, K, x, B, y, st, hdr, ol);
    if constexpr (CPL * 4 * XW <= 128) {
        if (B <= 4) return launch_fast<FMT, 4, LPR, CPL, OUTL>(codes, plane, N, K, x, B, y, st, hdr, ol);
    }
    if constexpr (CPL * 8 * XW <= 128) {
        if (B <= 8) return launch_fast<FMT, 8, LPR, CPL, OUTL>(codes, plane, N, K, x, B, y, st, hdr, ol);
    }
    *handled = false;
    return hipSuccess;
}

template <int FMT>
static hipError_t matvec_fmt(const uint8_t *codes, const void *plane, int64_t N, int K, const void *x,
                             qmv_dtype xdt, int B, float *y, hipStream_t st) {
    constexpr int E = ChunkTraits<FMT>::kElems;
    const int cpr = K / E;
    bool handled = false;
    hipError_t err = hipSuccess;
    if (xdt == QMV_F16) {
        err = launch_matvec_mfma(FMT, codes, plane, N, K, x, B, y, st, &handled);
        if (handled) return err;
        if (cpr <= 16) err = dispatch_b<FMT, 16, 1>(codes, plane, N, K, x, B, y, st, &handled);
        else if (cpr <= 32) err = dispatch_b<FMT, 32, 1>(codes, plane, N, K, x, B, y, st, &handled);
        else if (cpr <= 64) err = dispatch_b<FMT, 64, 1>(codes, plane, N, K, x, B, y, st, &handled);
        else if (cpr <= 128) err = dispatch_b<FMT, 64, 2>(codes, plane, N, K, x, B, y, st, &handled);
        else if (cpr <= 192) err = dispatch_b<FMT, 64, 3>(codes, plane, N, K, x, B, y, st, &handled);
        else if (cpr <= 256) err = dispatch_b<FMT, 64, 4>(codes, plane, N, K, x, B, y, st, &handled);
        if (handled) return err;
    }
    int grid = grid_for_waves(N);
    if (xdt == QMV_F16)
        hipLaunchKernelGGL((mv_generic<FMT, _Float16>), dim3(grid), dim3(256), 0, st, codes, plane, N, K,
                           reinterpret_cast<const _Float16 *>(x), B, y, OutlierArgs());
    else
        hipLaunchKernelGGL((mv_generic<FMT, float>), dim3(grid), dim3(256), 0, st, codes, plane, N, K,
                           reinterpret_cast<const float *>(x), B, y, OutlierArgs());
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fused matvec + argmax: the matvec writes y into the workspace and zeroes
// the header, then a grid of workgroups takes the argmax of each row. The
// matvec is the one the plain entry point would run for the shape (dot2 or
// matrix cores).
// ---------------------------------------------------------------------------
template <int FMT>
static bool argmax_shape(int K, int B, int *lpr, int *cpl) {
    const int cpr = K / ChunkTraits<FMT>::kElems;
    int l, c;
    if (cpr <= 16) l = 16, c = 1;
    else if (cpr <= 32) l = 32, c = 1;
    else if (cpr <= 64) l = 64, c = 1;
    else if (cpr <= 128) l = 64, c = 2;
    else if (cpr <= 192) l = 64, c = 3;
    else if (cpr <= 256) l = 64, c = 4;
    else return false;
    const bool ok = c == 1 ? dot2_takes<FMT, 1>(B) : c == 2 ? dot2_takes<FMT, 2>(B)
                  : c == 3 ? dot2_takes<FMT, 3>(B) : dot2_takes<FMT, 4>(B);
    if (lpr) *lpr = l;
    if (cpl) *cpl = c;
    return ok;
}

bool argmax_supported(int fmt, int64_t K, int B) {
    switch (fmt) {
    case INT4: return argmax_shape<INT4>((int)K, B, nullptr, nullptr);
    case INT4AFF: return argmax_shape<INT4AFF>((int)K, B, nullptr, nullptr);
    case INT8KM: return argmax_shape<INT8KM>((int)K, B, nullptr, nullptr);
    case FP4: return argmax_shape<FP4>((int)K, B, nullptr, nullptr);
    case INT8: return argmax_shape<INT8>((int)K, B, nullptr, nullptr);
    default: return argmax_shape<KM4>((int)K, B, nullptr, nullptr);
    }
}

// the header, then y [B][N] fp32 of the dot2 matvec
size_t argmax_workspace_bytes(int64_t N, int B) {
    return (size_t)kArgmaxHeader * sizeof(uint64_t) + (((size_t)N * (size_t)B * sizeof(float) + 15) / 16) * 16;
}

template <int FMT>
static hipError_t argmax_fmt(const uint8_t *codes, const void *plane, int64_t N, int K, const void *x, int B,
                             int32_t *idx, float *val, uint64_t *ws, hipStream_t st) {
    float *yw = reinterpret_cast<float *>(ws + kArgmaxHeader);
    int lpr = 0, cpl = 0;
    if (!argmax_shape<FMT>(K, B, &lpr, &cpl)) return hipErrorInvalidValue;
    bool handled = false;
    hipError_t err = launch_matvec_mfma(FMT, codes, plane, N, K, x, B, yw, st, &handled, ws);
    if (handled) {
        if (err != hipSuccess) return err;
    } else if (lpr == 16) err = dispatch_b<FMT, 16, 1>(codes, plane, N, K, x, B, yw, st, &handled, ws);
    else if (lpr == 32) err = dispatch_b<FMT, 32, 1>(codes, plane, N, K, x, B, yw, st, &handled, ws);
    else if (cpl == 1) err = dispatch_b<FMT, 64, 1>(codes, plane, N, K, x, B, yw, st, &handled, ws);
    else if (cpl == 2) err = dispatch_b<FMT, 64, 2>(codes, plane, N, K, x, B, yw, st, &handled, ws);
    else if (cpl == 3) err = dispatch_b<FMT, 64, 3>(codes, plane, N, K, x, B, yw, st, &handled, ws);
    else err = dispatch_b<FMT, 64, 4>(codes, plane, N, K, x, B, yw, st, &handled, ws);
    if (err != hipSuccess) return err;
    if (!handled) return hipErrorInvalidValue;
    if ((err = hipGetLastError()) != hipSuccess) return err;
    return launch_argmax_rows(yw, N, B, ws, idx, val, st);
}

hipError_t launch_argmax_rows(const float *y, int64_t N, int B, uint64_t *hdr, int32_t *idx, float *val,
                              hipStream_t st) {
    const int64_t g = (N + kArgmaxStretch - 1) / kArgmaxStretch;
    const dim3 grid((unsigned)(g < 1 ? 1 : (g > kArgmaxGroups ? kArgmaxGroups : g)), (unsigned)B);
    hipLaunchKernelGGL(argmax_rows_kernel, grid, dim3(1024), 0, st, y, N, B, hdr, idx, val);
    return hipGetLastError();
}

hipError_t launch_matvec_argmax(int fmt, const void *codes, const void *plane, int64_t N, int64_t K, const void *x,
                                int B, int32_t *idx, float *val, void *workspace, hipStream_t st) {
    const uint8_t *c = reinterpret_cast<const uint8_t *>(codes);
    uint64_t *ws = reinterpret_cast<uint64_t *>(workspace);
    switch (fmt) {
    case INT4: return argmax_fmt<INT4>(c, plane, N, (int)K, x, B, idx, val, ws, st);
    case INT4AFF: return argmax_fmt<INT4AFF>(c, plane, N, (int)K, x, B, idx, val, ws, st);
    case INT8KM: return argmax_fmt<INT8KM>(c, plane, N, (int)K, x, B, idx, val, ws, st);
    case FP4: return argmax_fmt<FP4>(c, plane, N, (int)K, x, B, idx, val, ws, st);
    case INT8: return argmax_fmt<INT8>(c, plane, N, (int)K, x, B, idx, val, ws, st);
    default: return argmax_fmt<KM4>(c, plane, N, (int)K, x, B, idx, val, ws, st);
    }
}

hipError_t launch_matvec(int fmt, const void *codes, const void *plane, int64_t N, int64_t K, const void *x,
                         qmv_dtype xdt, int B, float *y, hipStream_t st) {
    const uint8_t *c = reinterpret_cast<const uint8_t *>(codes);
    switch (fmt) {
    case INT4: return matvec_fmt<INT4>(c, plane, N, (int)K, x, xdt, B, y, st);
    case INT4AFF: return matvec_fmt<INT4AFF>(c, plane, N, (int)K, x, xdt, B, y, st);
    case INT8KM: return matvec_fmt<INT8KM>(c, plane, N, (int)K, x, xdt, B, y, st);
    case FP4: return matvec_fmt<FP4>(c, plane, N, (int)K, x, xdt, B, y, st);
    case INT8: return matvec_fmt<INT8>(c, plane, N, (int)K, x, xdt, B, y, st);
    default: return matvec_fmt<KM4>(c, plane, N, (int)K, x, xdt, B, y, st);
    }
}

hipError_t launch_matvec_km4o(const uint8_t *codes, const uint16_t *lut, const uint16_t *ocol, const int8_t *oval,
                              const uint16_t *oscale, int64_t N, int64_t K, int nout, const void *x, qmv_dtype xdt,
                              int B, float *y, hipStream_t st) {
    if (nout == 0) return launch_matvec(KM4, codes, lut, N, K, x, xdt, B, y, st);
    OutlierArgs ol;
    ol.col = ocol;
    ol.val = oval;
    ol.scale = oscale;
    ol.n = nout;
    const int k = (int)K;
    const int cpr = k / 32;
    bool handled = false;
    hipError_t err = hipSuccess;
    if (xdt == QMV_F16) {
        if (cpr <= 16) err = dispatch_b<KM4, 16, 1, true>(codes, lut, N, k, x, B, y, st, &handled, nullptr, ol);
        else if (cpr <= 32) err = dispatch_b<KM4, 32, 1, true>(codes, lut, N, k, x, B, y, st, &handled, nullptr, ol);
        else if (cpr <= 64) err = dispatch_b<KM4, 64, 1, true>(codes, lut, N, k, x, B, y, st, &handled, nullptr, ol);
        else if (cpr <= 128) err = dispatch_b<KM4, 64, 2, true>(codes, lut, N, k, x, B, y, st, &handled, nullptr, ol);
        if (handled) return err;
    }
    const int grid = grid_for_waves(N);
    if (xdt == QMV_F16)
        hipLaunchKernelGGL((mv_generic<KM4, _Float16, true>), dim3(grid), dim3(256), 0, st, codes, lut, N, k,
                           reinterpret_cast<const _Float16 *>(x), B, y, ol);
    else
        hipLaunchKernelGGL((mv_generic<KM4, float, true>), dim3(grid), dim3(256), 0, st, codes, lut, N, k,
                           reinterpret_cast<const float *>(x), B, y, ol);
    return hipGetLastError();
}

hipError_t launch_dequant(int fmt, const void *codes, const void *plane, int64_t N, int64_t K, float *out,
                          hipStream_t st) {
    const uint8_t *c = reinterpret_cast<const uint8_t *>(codes);
    int64_t blocks = N * (K / 32);
    int grid = (int)((blocks + 255) / 256);
    switch (fmt) {
    case INT4: hipLaunchKernelGGL(dequant_kernel<INT4>, dim3(grid), dim3(256), 0, st, c, plane, N, (int)K, out); break;
    case INT4AFF:
        hipLaunchKernelGGL(dequant_kernel<INT4AFF>, dim3(grid), dim3(256), 0, st, c, plane, N, (int)K, out);
        break;
    case INT8KM:
        hipLaunchKernelGGL(dequant_kernel<INT8KM>, dim3(grid), dim3(256), 0, st, c, plane, N, (int)K, out);
        break;
    case FP4: hipLaunchKernelGGL(dequant_kernel<FP4>, dim3(grid), dim3(256), 0, st, c, plane, N, (int)K, out); break;
    case INT8: hipLaunchKernelGGL(dequant_kernel<INT8>, dim3(grid), dim3(256), 0, st, c, plane, N, (int)K, out); break;
    default: hipLaunchKernelGGL(dequant_kernel<KM4>, dim3(grid), dim3(256), 0, st, c, plane, N, (int)K, out); break;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Streaming-read ceiling: the matvec's access pattern with no arithmetic.
// One-wave workgroups, each reading one contiguous stretch of kReadPerWave
// 1 KiB pieces: every lane issues all of its non-temporal 16-byte loads
// before it uses any, then the wave writes one xor checksum. (Measured on
// MI355X over 254 MB: 6.75 TB/s, against 6.52 TB/s for 256-thread
// workgroups reading 16 KiB with four loads per lane.)
// ---------------------------------------------------------------------------
constexpr int kReadPerWave = 8;   // 1 KiB pieces per wave

__global__ __launch_bounds__(64) void stream_read_kernel(const uint4 *__restrict__ p, int64_t n16,
                                                         uint32_t *__restrict__ sink) {
    const int64_t beg = (int64_t)blockIdx.x * (kReadPerWave * 64) + threadIdx.x;
    uint4 v[kReadPerWave];
#pragma unroll
    for (int u = 0; u < kReadPerWave; u++) {
        const int64_t i = beg + 64 * u;
        v[u] = load_stream16(p + (i < n16 ? i : 0));   // a piece past the end re-reads the first
    }
    uint32_t acc = 0;
#pragma unroll
    for (int u = 0; u < kReadPerWave; u++)
        if (beg + 64 * u < n16) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc ^= __shfl_xor(acc, m);
    if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

size_t stream_read_grid(size_t bytes) { return (bytes / 16 + kReadPerWave * 64 - 1) / (kReadPerWave * 64); }

hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t st) {
    size_t grid = stream_read_grid(bytes);
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(64), 0, st, reinterpret_cast<const uint4 *>(buf),
                       (int64_t)(bytes / 16), sink);
    return hipGetLastError();
}

}  // namespace qmv
