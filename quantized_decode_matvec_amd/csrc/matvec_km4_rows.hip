// Batch 1-4 k-means palettized matvec on a row-tiled code plane, one row per
// lane, two codes per table lookup ("Dense-path int4km coverage + flagship
// Qwen3.6-35B - session findings & methods", sections 1 and 8: the lm_head is
// the largest per-token matvec and its 4-bit palettized form is read once per
// token; "coreai-optimization (coreai-opt) reference", "Palettization": a
// 16-entry table per output row, 4-bit indices).
//
// A 16-entry table lookup per code costs an address, an LDS read and half of
// a merge + v_dot2, which keeps the row-per-wave kernel bound by instruction
// issue. Here every byte of codes (two indices) is looked up at once in a
// 256-entry table of fp16 pairs:
//   pair[e] = (lut[e & 15], lut[e >> 4])   (low nibble = even element)
// so one lookup yields the half2 operand of one v_dot2 per batch row. A 1 KiB pair table per
// row cannot be shared by the lanes of a wave without bank conflicts, so each
// lane owns one row: a 64-row tile's tables are stored transposed, entry e of
// row r at dword 64 e + r, and lane r only touches LDS bank r mod 32 (64 KiB
// per tile). The byte address 256 e + 4 r is one v_perm of the code word and
// the lane's 4 r. Per code: half a v_perm, half an LDS read and half a v_dot2,
// plus the table build (256 entries per row: one v_perm and one LDS write
// each, 1/8 of the lookups).
//
// Work split: a 16-wave workgroup takes a 64-row tile; wave w takes the code
// chunks (16 bytes = 32 codes of a row) CPW w .. CPW w + CPW - 1, so the x
// slice it multiplies is the same for all of its lanes and is read with
// scalar loads, the SGPR operand of v_dot2. Wave w builds the 16 table entries
// with low nibble in 4a..4a+3 and high nibble in 4b..4b+3 (a = w & 3,
// b = w >> 2), which needs 16 bytes of its row's table. The 16 partial sums of
// a row meet in LDS and are added by a fixed DPP tree, every wave taking 4 rows
// (deterministic; no wave is left alone at the end of a workgroup's life).
//
// Row-tiled code layout (tile t = rows 64 t .. 64 t + 63, Q = K / 32 chunks
// per row): chunk q of row 64 t + r is the 16 bytes at ((t Q + q) 64 + r) 16,
// so a wave-wide 16-byte load reads 1 KiB of consecutive bytes and a wave's
// CPW chunks of a tile are CPW consecutive KiB. Rows past N in the last tile
// are zero.
//
// Each workgroup takes TPW consecutive tiles; the table words of a tile are
// issued before its codes, so the pair table is built while the codes are
// still arriving, and tile i + 1's loads are in flight while tile i is built
// and looked up.
#include "qmv_device.h"
#include "qmv_launch.h"

namespace qmv {

constexpr int kRowsTile = 64;                                    // rows per tile (one per lane)
constexpr int kPairEntries = 256;                                // table entries per row
constexpr int kTileWaves = 16;                                   // waves per workgroup

// read-only memory in the constant address space: uniform loads from it are
// scalar loads into SGPRs
typedef __attribute__((address_space(4))) const uint32_t kconst_u32;

// dword at byte offset `a` of LDS (a is 4-aligned and below the allocation)
__device__ __forceinline__ uint32_t lds_word(const uint32_t *base, uint32_t a) {
    return *reinterpret_cast<const uint32_t *>(reinterpret_cast<const char *>(base) + a);
}

// int8 outliers added to the rows (the 4-bit k-means + int8 outlier format):
// per row, n columns (increasing), int8 values and one fp16 scale; the row's
// weight at an outlier column is the table value plus scale * q.
struct TiledOutliers {
    const uint16_t *col = nullptr;   // [N][n]
    const int8_t *val = nullptr;     // [N][n]
    const uint16_t *scale = nullptr; // [N]
    int n = 0;
};

// BT batch rows (x [BT][K], y [BT][N]); two workgroups per CU need at most
// 80 KiB of LDS each: 64 KiB of pair tables + 4 KiB of partial sums per batch
// row. OUTL: add the int8 outliers; the 16 lanes that sum a row's partial
// sums take its outliers ww, ww + 16, ... (the first one's column, value and
// scale loaded with the codes, its x gathered after the table build).
// KEYS (greedy decoding): no y; the workgroup writes the largest argmax key
// of its rows per batch row, keys[b][blockIdx.x], for argmax_keys_kernel.
template <int CPW, int TPW, int BT, bool OUTL = false, bool KEYS = false>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(8, 8))) void mv_km4_tiled(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ lut, int64_t N, const _Float16 *__restrict__ x,
    float *__restrict__ y, int64_t tiles, uint64_t *__restrict__ keys, TiledOutliers ol) {
    constexpr int W = kTileWaves;
    constexpr int Q = W * CPW;   // chunks per row
    constexpr int K = Q * 32;
    // pair tables at LDS address 0 (a static array: table addresses need no
    // base added), then the partial sums [BT][W][64]: wave w's sum for row r
    // at [w][r ^ w ^ 16 (r & 1)], so that both the writes (one wave, 64 rows)
    // and the reads (16 waves' sums of two rows per half-wave) fall on
    // distinct banks
    // OUTL: x [BT][K] after them where it fits in 80 KiB (the outliers'
    // x values are read from there, not gathered from global memory)
    constexpr bool XL = OUTL && (kPairEntries + BT * W) * kRowsTile * 4 + BT * K * 2 <= 80 * 1024;
    __shared__ __align__(16) uint32_t lds[kPairEntries * kRowsTile + BT * W * kRowsTile + (XL ? BT * K / 2 : 0)];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int la = (wave & 3) * 2, hb = (wave >> 2) * 2;   // table words of this wave's build share
    const uint32_t roff = (uint32_t)lane * 4u;
    float *part = reinterpret_cast<float *>(lds + kPairEntries * kRowsTile);
    // x[b][c] for the outliers: from the LDS copy where there is one
    auto xval = [&](int b, int c) -> float {
        if constexpr (XL)
            return (float)reinterpret_cast<const _Float16 *>(lds + (kPairEntries + BT * W) * kRowsTile)[b * K + c];
        else
            return (float)x[(size_t)b * K + c];
    };
    uint64_t kmax[BT];   // KEYS: this lane's largest key per batch row
#pragma unroll
    for (int bb = 0; bb < BT; bb++) kmax[bb] = 0;

    uint4 cw[TPW > 1 ? 2 : 1][CPW];
    uint2 lo[TPW > 1 ? 2 : 1], hi[TPW > 1 ? 2 : 1];
    // outliers: this lane sums row 4 wave + (lane >> 4) and takes its outlier
    // lane & 15 (column, value, row scale), prefetched per tile
    const int orr = 4 * wave + (lane >> 4), oww = lane & 15;
    uint32_t ocol_r[OUTL ? (TPW > 1 ? 2 : 1) : 1], oval_r[OUTL ? (TPW > 1 ? 2 : 1) : 1],
        osc_r[OUTL ? (TPW > 1 ? 2 : 1) : 1];
    // loads of tile t into buffer k; a tile past the end reads tile 0 again
    // (read by the first workgroups: a cache hit, no HBM traffic)
    auto load = [&](int64_t t, int k) {
        const int64_t tt = t < tiles ? t : 0;   // wave-uniform: a scalar select, no branch
        const int64_t row = tt * kRowsTile + lane;
        const uint32_t *lr = reinterpret_cast<const uint32_t *>(lut + (size_t)(row < N ? row : N - 1) * 16);
        lo[k] = *reinterpret_cast<const uint2 *>(lr + la);
        hi[k] = *reinterpret_cast<const uint2 *>(lr + hb);
        const uint8_t *tb = codes + ((size_t)tt * Q + CPW * wave) * (kRowsTile * 16) + lane * 16;
#pragma unroll
        for (int j = 0; j < CPW; j++) cw[k][j] = load_stream16(tb + j * (kRowsTile * 16));
        if constexpr (OUTL) {
            const int64_t orow = tt * kRowsTile + orr;
            const int64_t rc = orow < N ? orow : N - 1;
            const int o = oww < ol.n ? oww : 0;   // a lane without an outlier reads outlier 0 and drops it
            ocol_r[k] = ol.n > 0 ? ol.col[rc * ol.n + o] : 0u;
            oval_r[k] = ol.n > 0 ? (uint32_t)(int32_t)ol.val[rc * ol.n + o] : 0u;
            osc_r[k] = ol.scale[rc];
        }
    };
    auto step = [&](int64_t t, int k) {
        {
            // entries (lo = 4a + l, hi = 4b + h): low half from the word pair
            // lo[k], high half from hi[k]
            const uint32_t lw[2] = {lo[k].x, lo[k].y}, hw[2] = {hi[k].x, hi[k].y};
#pragma unroll
            for (int h = 0; h < 4; h++)
#pragma unroll
                for (int l = 0; l < 4; l++) {
                    const uint32_t sel =
                        ((l & 1) ? 0x00000706u : 0x00000504u) | ((h & 1) ? 0x03020000u : 0x01000000u);
                    const int e = ((hb * 2 + h) << 4) + (la * 2 + l);
                    lds[e * kRowsTile + lane] = __builtin_amdgcn_perm(lw[l >> 1], hw[h >> 1], sel);
                }
        }
        __syncthreads();
        // outliers: x at this lane's outlier column, gathered now that the
        // column has arrived (with the table words)
        float oterm[BT];
        if constexpr (OUTL) {
            const float sc = f16_bits_to_f32((uint16_t)osc_r[k]);
            const float tq = oww < ol.n ? (float)(int32_t)oval_r[k] * sc : 0.f;   // exact: 8 x 11 bits
#pragma unroll
            for (int bb = 0; bb < BT; bb++) oterm[bb] = tq * xval(bb, (int)ocol_r[k]);
        }
        float acc[BT][2];
#pragma unroll
        for (int bb = 0; bb < BT; bb++) acc[bb][0] = acc[bb][1] = 0.f;
        // x is re-read per tile (scalar cache hits) rather than held in SGPRs
        // from one tile to the next, which would spill them
        const kconst_u32 *xw = (const kconst_u32 *)x;
        asm volatile("" : "+s"(xw));
#pragma unroll
        for (int j = 0; j < CPW; j++) {
            const kconst_u32 *xq = xw + (size_t)(CPW * wave + j) * 16;   // wave-uniform
            const uint32_t w4[4] = {cw[k][j].x, cw[k][j].y, cw[k][j].z, cw[k][j].w};
#pragma unroll
            for (int d = 0; d < 4; d++)
#pragma unroll
                for (int b = 0; b < 4; b++) {
                    // byte b of code word d -> table address 256 * byte + 4 * lane
                    const uint32_t a = __builtin_amdgcn_perm(w4[d], roff, 0x0C0C0000u | ((4u + b) << 8));
                    const h2 v = as_h2(lds_word(lds, a));
#pragma unroll
                    for (int bb = 0; bb < BT; bb++)
                        acc[bb][b & 1] = dot2(v, as_h2(xq[bb * (K / 2) + 4 * d + b]), acc[bb][b & 1]);
                }
        }
#pragma unroll
        for (int bb = 0; bb < BT; bb++)
            part[(bb * W + wave) * kRowsTile + (lane ^ wave ^ ((lane & 1) << 4))] = acc[bb][0] + acc[bb][1];
        __syncthreads();
        // every wave sums 4 rows: lane l takes wave (l & 15)'s sum of row
        // 4 wave + (l >> 4), then a fixed DPP tree over each 16-lane row
        const int rr = 4 * wave + (lane >> 4), ww = lane & 15;
        const int64_t row = t * kRowsTile + rr;
        if constexpr (OUTL) {
            // outliers past the first 16 of a row (the prefetched one is ww)
            const int64_t rc = row < N ? row : N - 1;
            const float sc = f16_bits_to_f32(ol.scale[rc]);
            for (int o = ww + 16; o < ol.n; o += 16) {
                const float tq = (float)ol.val[rc * ol.n + o] * sc;
                const int col = ol.col[rc * ol.n + o];
#pragma unroll
                for (int bb = 0; bb < BT; bb++) oterm[bb] = __builtin_fmaf(tq, xval(bb, col), oterm[bb]);
            }
        }
#pragma unroll
        for (int bb = 0; bb < BT; bb++) {
            float pv = part[(bb * W + ww) * kRowsTile + (rr ^ ww ^ ((rr & 1) << 4))];
            if constexpr (OUTL) pv += oterm[bb];
            const float s = row16_sum(pv);
            if (ww == 0 && t < tiles && row < N) {
                if constexpr (KEYS) {
                    const uint64_t kk = argmax_key(s, row);
                    kmax[bb] = kk > kmax[bb] ? kk : kmax[bb];
                } else {
                    y[(size_t)bb * N + row] = s;
                }
            }
        }
    };
    const int64_t t0 = (int64_t)blockIdx.x * TPW;
    if constexpr (XL) {
        // x into LDS (visible after the first tile's build barrier)
        uint32_t *xl = lds + (kPairEntries + BT * W) * kRowsTile;
        for (int i = threadIdx.x; i < BT * K / 2; i += 64 * W) xl[i] = reinterpret_cast<const uint32_t *>(x)[i];
    }
    load(t0, 0);
    if constexpr (TPW == 1) {
        step(t0, 0);
    } else {
        // straight-line code: in a loop the compiler waits for every
        // outstanding load at the back edge, the prefetch included
        load(t0 + 1, 1);
        step(t0, 0);
        step(t0 + 1, 1);
    }
    if constexpr (KEYS) {
        // one key per wave and batch row, in the table region: the last
        // tile's lookups are done (barrier before its partial sums were read)
        uint64_t *kl = reinterpret_cast<uint64_t *>(lds);
#pragma unroll
        for (int bb = 0; bb < BT; bb++) {
            const uint64_t k = wave_max_u64(kmax[bb]);
            if (lane == 0) kl[bb * W + wave] = k;
        }
        __syncthreads();
        if (threadIdx.x < BT) {
            uint64_t k = 0;
            for (int w = 0; w < W; w++) k = kl[threadIdx.x * W + w] > k ? kl[threadIdx.x * W + w] : k;
            keys[(size_t)threadIdx.x * gridDim.x + blockIdx.x] = k;
        }
    }
}

// Batch 2-4 on the same tiles with the products on the matrix cores:
// v_mfma_f32_4x4x4_16b_f16 runs 16 blocks of D[4 tokens][4 rows] +=
// A[4 tokens][4 k] B[4 k][4 rows]; lane 4b + j supplies column j of block b's
// B, i.e. 4 k-values of its own row 4b + j (the two pair-table lookups of two
// code bytes), and row j of its A, 4 k-values of x for token j, and receives
// the 4 tokens' sums of its own row. All 16 blocks take the same 4 k, so the
// whole wave multiplies 64 rows by 4 tokens per instruction: per code byte one
// v_perm and one LDS read, and no VALU multiply.
// x [4][K] (token rows past B zero) is staged once per workgroup in LDS after
// the pair tables, 16-byte unit u of token j at unit u ^ j (the 4 tokens a
// read serves fall on distinct banks); 64 KiB + K / 2 KiB <= 80 KiB keeps two
// workgroups per CU, so K <= 2048, and the partial sums [4][W][64] go to the
// table region once a tile's lookups are done (two more barriers per tile).
// KEYS: as in mv_km4_tiled (the wave keys go to the x stage, free by then).
// OUTL: the int8 outliers, added as in mv_km4_tiled.
template <int CPW, bool KEYS = false, bool OUTL = false>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(8, 8))) void mv_km4_tiled_mfma(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ lut, int64_t N, const _Float16 *__restrict__ x,
    int B, float *__restrict__ y, int64_t tiles, uint64_t *__restrict__ keys, TiledOutliers ol) {
    constexpr int W = kTileWaves;
    constexpr int Q = W * CPW;   // chunks per row
    constexpr int K = Q * 32;
    constexpr int XU = K / 8;    // 16-byte units of x per token
    static_assert(kPairEntries * kRowsTile * 4 + 4 * K * 2 <= 80 * 1024, "two workgroups per CU");
    __shared__ __align__(16) uint32_t lds[kPairEntries * kRowsTile + 4 * K / 2];
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    typedef float f4v __attribute__((ext_vector_type(4)));
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int la = (wave & 3) * 2, hb = (wave >> 2) * 2;
    const uint32_t roff = (uint32_t)lane * 4u;
    float *part = reinterpret_cast<float *>(lds);
    uint4 *xs = reinterpret_cast<uint4 *>(lds + kPairEntries * kRowsTile);

    const int64_t t = blockIdx.x;
    // loads: table words first, then the codes, then this thread's x units
    const int64_t row = t * kRowsTile + lane;
    const uint32_t *lr = reinterpret_cast<const uint32_t *>(lut + (size_t)(row < N ? row : N - 1) * 16);
    const uint2 lo = *reinterpret_cast<const uint2 *>(lr + la);
    const uint2 hi = *reinterpret_cast<const uint2 *>(lr + hb);
    uint4 cw[CPW];
    const uint8_t *tb = codes + ((size_t)t * Q + CPW * wave) * (kRowsTile * 16) + lane * 16;
#pragma unroll
    for (int j = 0; j < CPW; j++) cw[j] = load_stream16(tb + j * (kRowsTile * 16));
    // outliers: this lane sums row rr = 4 wave + (lane >> 4) below and takes
    // its outlier ww = lane & 15 (column, value, row scale)
    const int rr = 4 * wave + (lane >> 4), ww = lane & 15;
    const int64_t orow = t * kRowsTile + rr;
    uint32_t ocol = 0, oval = 0, osc = 0;
    if constexpr (OUTL) {
        const int64_t rc = orow < N ? orow : N - 1;
        const int o = ww < ol.n ? ww : 0;   // a lane without an outlier reads outlier 0 and drops it
        ocol = ol.n > 0 ? ol.col[rc * ol.n + o] : 0u;
        oval = ol.n > 0 ? (uint32_t)(int32_t)ol.val[rc * ol.n + o] : 0u;
        osc = ol.scale[rc];
    }
    constexpr int XPT = (4 * XU + 1023) / 1024;   // x units per thread
    uint4 xv[XPT];
#pragma unroll
    for (int i = 0; i < XPT; i++) {
        const int u = threadIdx.x + 1024 * i, tok = u / XU;
        const bool ok = u < 4 * XU && tok < B;
        xv[i] = reinterpret_cast<const uint4 *>(x)[ok ? u : 0];
        if (!ok) xv[i] = make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < XPT; i++) {
        const int u = threadIdx.x + 1024 * i, tok = u / XU;
        if (u < 4 * XU) xs[tok * XU + ((u - tok * XU) ^ tok)] = xv[i];
    }
    {
        const uint32_t lw[2] = {lo.x, lo.y}, hw[2] = {hi.x, hi.y};
#pragma unroll
        for (int h = 0; h < 4; h++)
#pragma unroll
            for (int l = 0; l < 4; l++) {
                const uint32_t sel = ((l & 1) ? 0x00000706u : 0x00000504u) | ((h & 1) ? 0x03020000u : 0x01000000u);
                const int e = ((hb * 2 + h) << 4) + (la * 2 + l);
                lds[e * kRowsTile + lane] = __builtin_amdgcn_perm(lw[l >> 1], hw[h >> 1], sel);
            }
    }
    __syncthreads();
    // outliers: x at this lane's outlier column, read from the x stage
    // (element c of token b at half 8 (b XU + ((c >> 3) ^ b)) + (c & 7); the
    // rows past B are zero)
    const _Float16 *xsh = reinterpret_cast<const _Float16 *>(xs);
    auto xat = [&](int b, int c) { return (float)xsh[8 * (b * XU + ((c >> 3) ^ b)) + (c & 7)]; };
    float oterm[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (OUTL) {
        const float tq = ww < ol.n ? (float)(int32_t)oval * f16_bits_to_f32((uint16_t)osc) : 0.f;   // exact
#pragma unroll
        for (int b = 0; b < 4; b++) oterm[b] = tq * xat(b, (int)ocol);
    }
    const int tj = lane & 3;   // this lane's token in the A operand
    const uint4 *xj = xs + tj * XU;
    f4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < CPW; j++) {
        const int q = CPW * wave + j;
        const uint32_t w4[4] = {cw[j].x, cw[j].y, cw[j].z, cw[j].w};
#pragma unroll
        for (int d = 0; d < 4; d++) {
            // x of codes 8d .. 8d + 7 of chunk q: unit 4q + d of token tj
            const uint4 xu = xj[(4 * q + d) ^ tj];
#pragma unroll
            for (int s2 = 0; s2 < 2; s2++) {
                const uint32_t a0 = __builtin_amdgcn_perm(w4[d], roff, 0x0C0C0000u | ((4u + 2 * s2) << 8));
                const uint32_t a1 = __builtin_amdgcn_perm(w4[d], roff, 0x0C0C0000u | ((5u + 2 * s2) << 8));
                typedef uint32_t u2 __attribute__((ext_vector_type(2)));
                const u2 wv = {lds_word(lds, a0), lds_word(lds, a1)};
                const u2 xx = {s2 ? xu.z : xu.x, s2 ? xu.w : xu.y};
                acc = __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(h4, xx), __builtin_bit_cast(h4, wv), acc,
                                                         0, 0, 0);
            }
        }
    }
    __syncthreads();   // every wave's lookups are done: the table region takes the partial sums
#pragma unroll
    for (int b = 0; b < 4; b++) part[(b * W + wave) * kRowsTile + (lane ^ wave ^ ((lane & 1) << 4))] = acc[b];
    __syncthreads();
    if constexpr (OUTL) {
        // outliers past the first 16 of a row
        const int64_t rc = orow < N ? orow : N - 1;
        const float sc = f16_bits_to_f32(ol.scale[rc]);
        for (int o = ww + 16; o < ol.n; o += 16) {
            const float tq = (float)ol.val[rc * ol.n + o] * sc;
            const int col = ol.col[rc * ol.n + o];
#pragma unroll
            for (int b = 0; b < 4; b++) oterm[b] = __builtin_fmaf(tq, xat(b, col), oterm[b]);
        }
    }
    uint64_t km[4];
#pragma unroll
    for (int b = 0; b < 4; b++) {
        const float sum = row16_sum(part[(b * W + ww) * kRowsTile + (rr ^ ww ^ ((rr & 1) << 4))] + oterm[b]);
        km[b] = 0;
        if (ww == 0 && b < B && orow < N) {
            if constexpr (KEYS) km[b] = argmax_key(sum, orow);
            else y[(size_t)b * N + orow] = sum;
        }
    }
    if constexpr (KEYS) {
        uint64_t *kl = reinterpret_cast<uint64_t *>(xs);   // x is no longer read
#pragma unroll
        for (int b = 0; b < 4; b++) {
            const uint64_t k = wave_max_u64(km[b]);
            if (lane == 0) kl[b * W + wave] = k;
        }
        __syncthreads();
        if (threadIdx.x < B) {
            uint64_t k = 0;
            for (int w = 0; w < W; w++) k = kl[threadIdx.x * W + w] > k ? kl[threadIdx.x * W + w] : k;
            keys[(size_t)threadIdx.x * gridDim.x + blockIdx.x] = k;
        }
    }
}

// The launchers below take `keys` (null: write y) and return the grid size
// (the number of keys per batch row) in *grid when grid is not null.
template <int CPW>
static hipError_t launch_tiled_mfma(const uint8_t *codes, const uint16_t *lut, int64_t N, const _Float16 *x, int B,
                                    float *y, hipStream_t st, uint64_t *keys, int64_t *grid, const TiledOutliers *ol) {
    const int64_t tiles = (N + kRowsTile - 1) / kRowsTile;
    if (grid != nullptr) *grid = tiles;
    const dim3 g((unsigned)tiles), blk(64 * kTileWaves);
    if (ol != nullptr)
        hipLaunchKernelGGL((mv_km4_tiled_mfma<CPW, false, true>), g, blk, 0, st, codes, lut, N, x, B, y, tiles, nullptr,
                           *ol);
    else if (keys != nullptr)
        hipLaunchKernelGGL((mv_km4_tiled_mfma<CPW, true>), g, blk, 0, st, codes, lut, N, x, B, y, tiles, keys,
                           TiledOutliers());
    else
        hipLaunchKernelGGL((mv_km4_tiled_mfma<CPW>), g, blk, 0, st, codes, lut, N, x, B, y, tiles, nullptr,
                           TiledOutliers());
    return hipGetLastError();
}

static hipError_t launch_km4_tiled_mfma(const uint8_t *codes, const uint16_t *lut, int64_t N, int64_t K,
                                        const _Float16 *x, int B, float *y, hipStream_t st, uint64_t *keys,
                                        int64_t *grid, const TiledOutliers *ol) {
    switch (K) {
    case 512: return launch_tiled_mfma<1>(codes, lut, N, x, B, y, st, keys, grid, ol);
    case 1024: return launch_tiled_mfma<2>(codes, lut, N, x, B, y, st, keys, grid, ol);
    case 1536: return launch_tiled_mfma<3>(codes, lut, N, x, B, y, st, keys, grid, ol);
    case 2048: return launch_tiled_mfma<4>(codes, lut, N, x, B, y, st, keys, grid, ol);
    default: return hipErrorInvalidValue;
    }
}

template <int CPW, int TPW, int BT>
static hipError_t launch_tiled(const uint8_t *codes, const uint16_t *lut, int64_t N, const _Float16 *x, float *y,
                               hipStream_t st, uint64_t *keys, int64_t *gridp, const TiledOutliers *ol) {
    const int64_t tiles = (N + kRowsTile - 1) / kRowsTile;
    const int64_t grid = (tiles + TPW - 1) / TPW;
    if (gridp != nullptr) *gridp = grid;
    const dim3 g((unsigned)grid), blk(64 * kTileWaves);
    if (ol != nullptr)
        hipLaunchKernelGGL((mv_km4_tiled<CPW, TPW, BT, true>), g, blk, 0, st, codes, lut, N, x, y, tiles, nullptr, *ol);
    else if (keys != nullptr)
        hipLaunchKernelGGL((mv_km4_tiled<CPW, TPW, BT, false, true>), g, blk, 0, st, codes, lut, N, x, y, tiles, keys,
                           TiledOutliers());
    else
        hipLaunchKernelGGL((mv_km4_tiled<CPW, TPW, BT>), g, blk, 0, st, codes, lut, N, x, y, tiles, nullptr,
                           TiledOutliers());
    return hipGetLastError();
}

// K = 512 CPW (CPW = 1..8). Two tiles per workgroup once there are enough
// workgroups to keep two on every CU; fewer tiles spread one per workgroup;
// from K = 2560 a tile holds 20 or more code registers and a workgroup takes one
template <int BT>
static hipError_t launch_tiled_b(const uint8_t *codes, const uint16_t *lut, int64_t N, int64_t K, const _Float16 *x,
                                 float *y, bool two, hipStream_t st, uint64_t *keys, int64_t *grid,
                                 const TiledOutliers *ol) {
    switch (K) {
    case 512: return two ? launch_tiled<1, 2, BT>(codes, lut, N, x, y, st, keys, grid, ol)
                         : launch_tiled<1, 1, BT>(codes, lut, N, x, y, st, keys, grid, ol);
    case 1024: return two ? launch_tiled<2, 2, BT>(codes, lut, N, x, y, st, keys, grid, ol)
                          : launch_tiled<2, 1, BT>(codes, lut, N, x, y, st, keys, grid, ol);
    case 1536: return two ? launch_tiled<3, 2, BT>(codes, lut, N, x, y, st, keys, grid, ol)
                          : launch_tiled<3, 1, BT>(codes, lut, N, x, y, st, keys, grid, ol);
    case 2048: return two ? launch_tiled<4, 2, BT>(codes, lut, N, x, y, st, keys, grid, ol)
                          : launch_tiled<4, 1, BT>(codes, lut, N, x, y, st, keys, grid, ol);
    case 2560: return launch_tiled<5, 1, BT>(codes, lut, N, x, y, st, keys, grid, ol);
    case 3072: return launch_tiled<6, 1, BT>(codes, lut, N, x, y, st, keys, grid, ol);
    case 3584: return launch_tiled<7, 1, BT>(codes, lut, N, x, y, st, keys, grid, ol);
    case 4096: return launch_tiled<8, 1, BT>(codes, lut, N, x, y, st, keys, grid, ol);
    default: return hipErrorInvalidValue;
    }
}

bool km4_tiled_supported(int64_t K, int B) {
    return K >= 512 && K <= 4096 && K % 512 == 0 && B >= 1 && B <= 4;
}

static hipError_t launch_km4_tiled(const uint8_t *codes, const uint16_t *lut, int64_t N, int64_t K,
                                   const _Float16 *x, int B, float *y, hipStream_t st, uint64_t *keys,
                                   int64_t *grid, const TiledOutliers *ol) {
    const int64_t tiles = (N + kRowsTile - 1) / kRowsTile;
    const bool two = tiles >= 4 * (int64_t)device_cu_count();
    // batch 2-4: products on the matrix cores (the x stage fits up to K = 2048;
    // 248320 x 2048: 51 us against 53 / 61-70 us for B = 2 / 3-4 v_dot2 per
    // lookup)
    if (B >= 2 && K <= 2048) return launch_km4_tiled_mfma(codes, lut, N, K, x, B, y, st, keys, grid, ol);
    switch (B) {
    case 1: return launch_tiled_b<1>(codes, lut, N, K, x, y, two, st, keys, grid, ol);
    case 2: return launch_tiled_b<2>(codes, lut, N, K, x, y, two, st, keys, grid, ol);
    case 3: return launch_tiled_b<3>(codes, lut, N, K, x, y, two, st, keys, grid, ol);
    case 4: return launch_tiled_b<4>(codes, lut, N, K, x, y, two, st, keys, grid, ol);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_matvec_km4_tiled(const uint8_t *codes, const uint16_t *lut, int64_t N, int64_t K,
                                   const _Float16 *x, int B, float *y, hipStream_t st) {
    return launch_km4_tiled(codes, lut, N, K, x, B, y, st, nullptr, nullptr, nullptr);
}

hipError_t launch_matvec_km4o_tiled(const uint8_t *codes, const uint16_t *lut, const uint16_t *ocol,
                                    const int8_t *oval, const uint16_t *oscale, int64_t N, int64_t K, int nout,
                                    const _Float16 *x, int B, float *y, hipStream_t st) {
    TiledOutliers ol;
    ol.col = ocol;
    ol.val = oval;
    ol.scale = oscale;
    ol.n = nout;
    return launch_km4_tiled(codes, lut, N, K, x, B, y, st, nullptr, nullptr, &ol);
}

// The greedy token from the workgroup keys: one workgroup per batch row takes
// the largest of its G keys (order-independent, so the result does not depend
// on which workgroup finished first).
__global__ __launch_bounds__(1024) void argmax_keys_kernel(const uint64_t *__restrict__ keys, int G,
                                                           int32_t *__restrict__ idx, float *__restrict__ val) {
    const int b = blockIdx.x;
    const uint64_t *kb = keys + (size_t)b * G;
    uint64_t k = 0;
    for (int i0 = threadIdx.x; i0 < G; i0 += 4 * 1024) {
        uint64_t v[4];
#pragma unroll
        for (int u = 0; u < 4; u++) v[u] = i0 + 1024 * u < G ? kb[i0 + 1024 * u] : 0;
#pragma unroll
        for (int u = 0; u < 4; u++) k = v[u] > k ? v[u] : k;
    }
    k = wave_max_u64(k);
    __shared__ uint64_t red[16];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = k;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 0; w < 16; w++) k = red[w] > k ? red[w] : k;
        idx[b] = argmax_key_row(k);
        val[b] = argmax_key_value(k);
    }
}

size_t km4_tiled_argmax_keys_bytes(int64_t N, int B) {
    return (size_t)B * (size_t)((N + kRowsTile - 1) / kRowsTile) * sizeof(uint64_t);
}

hipError_t launch_argmax_km4_tiled(const uint8_t *codes, const uint16_t *lut, int64_t N, int64_t K,
                                   const _Float16 *x, int B, int32_t *idx, float *val, void *workspace,
                                   hipStream_t st) {
    uint64_t *keys = reinterpret_cast<uint64_t *>(workspace);
    int64_t grid = 0;
    hipError_t err = launch_km4_tiled(codes, lut, N, K, x, B, nullptr, st, keys, &grid, nullptr);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(argmax_keys_kernel, dim3((unsigned)B), dim3(1024), 0, st, keys, (int)grid, idx, val);
    return hipGetLastError();
}

// Row-tiled copy of a canonical [N][K/2] code plane (rows past N are zero).
// Workgroup b takes chunks 4 yb .. 4 yb + 3 of the 64 rows of tile t
// (t, yb from b, one division per workgroup): lane r of each wave copies row
// r's chunk, so a workgroup writes 4 KiB of consecutive destination bytes and
// the next workgroup reads the rest of the same rows' cache lines.
__global__ __launch_bounds__(256) void tile_codes_kernel(const uint4 *__restrict__ src, uint4 *__restrict__ dst,
                                                         int64_t N, int Q, int nb) {
    const uint32_t b = blockIdx.x;
    const uint32_t t = b / (uint32_t)nb, yb = b - t * (uint32_t)nb;   // uniform
    const int r = threadIdx.x & 63;
    const int q = 4 * (int)yb + (threadIdx.x >> 6);
    if (q >= Q) return;
    const int64_t n = (int64_t)t * kRowsTile + r;
    const uint4 v = n < N ? src[n * Q + q] : make_uint4(0u, 0u, 0u, 0u);
    dst[((int64_t)t * Q + q) * kRowsTile + r] = v;
}

size_t km4_tiled_bytes(int64_t N, int64_t K) {
    return (size_t)((N + kRowsTile - 1) / kRowsTile) * kRowsTile * (size_t)(K / 2);
}

hipError_t launch_tile_km4(const uint8_t *codes, int64_t N, int64_t K, uint8_t *out, hipStream_t st) {
    const int Q = (int)(K / 32);
    const int64_t tiles = (N + kRowsTile - 1) / kRowsTile;
    const int nb = (Q + 3) / 4;   // workgroups per tile
    const int64_t grid = tiles * nb;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(tile_codes_kernel, dim3((unsigned)grid), dim3(256), 0, st,
                       reinterpret_cast<const uint4 *>(codes), reinterpret_cast<uint4 *>(out), N, Q, nb);
    return hipGetLastError();
}

}  // namespace qmv
