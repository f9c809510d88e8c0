// Quantize-and-pack kernels for the four block formats.
//
// Definitions: "Stream D - Quantization (FP4 + QAT-int4): feasibility, first
// result, and plan" section 1 (E2M1 with e8m0 scale 2^(floor(log2 amax)-2),
// blocks of 32 along K, two codes per byte; the default 4-bit recipe is int4
// per-block-32 symmetric with clipping) and section 2 (MSE-optimal clip ratio
// per block); "Compression (palettization & quantization)", int8 per-block-32
// head; "coreai-optimization (coreai-opt) reference", "Palettization"
// (2^n_bits-entry table per output channel from scalar k-means) and
// "Dense-path int4km coverage + flagship Qwen3.6-35B", sections 8 and 8b
// (16-entry fp16 codebook per row, palettize_grouped with n_bits = 4).
//
// These kernels must reproduce the packing bit for bit, so every float
// operation is written as one IEEE operation with an explicit rounding and
// FP contraction is off in this file.
#include "qmv_device.h"
#include "qmv_launch.h"

#pragma clang fp contract(off)

namespace qmv {

template <typename WT>
__device__ __forceinline__ void load_block_f32(const WT *__restrict__ W, int64_t off, float (&w)[32]);

template <>
__device__ __forceinline__ void load_block_f32<_Float16>(const _Float16 *__restrict__ W, int64_t off, float (&w)[32]) {
    const uint4 *p = reinterpret_cast<const uint4 *>(W + off);
#pragma unroll
    for (int i = 0; i < 4; i++) {
        uint4 v = p[i];
        uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; j++) {
            h2 h = as_h2(d[j]);
            w[8 * i + 2 * j] = (float)h.x;
            w[8 * i + 2 * j + 1] = (float)h.y;
        }
    }
}

template <>
__device__ __forceinline__ void load_block_f32<float>(const float *__restrict__ W, int64_t off, float (&w)[32]) {
    const float4 *p = reinterpret_cast<const float4 *>(W + off);
#pragma unroll
    for (int i = 0; i < 8; i++) {
        float4 v = p[i];
        w[4 * i] = v.x;
        w[4 * i + 1] = v.y;
        w[4 * i + 2] = v.z;
        w[4 * i + 3] = v.w;
    }
}

// ---------------------------------------------------------------------------
// Symmetric integer blocks (int4 with clip search, int8 absmax).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float clip_ratio(int i) {
    // 1.0, 0.95, ..., 0.7 as fp32 literals
    switch (i) {
    case 0: return 1.0f;
    case 1: return 0.95f;
    case 2: return 0.9f;
    case 3: return 0.85f;
    case 4: return 0.8f;
    case 5: return 0.75f;
    default: return 0.7f;
    }
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float v) {
    return __builtin_bit_cast(uint16_t, (_Float16)v);   // v_cvt_f16_f32, round to nearest even
}

template <int QMAX>
__device__ __forceinline__ float quant_q(float w, float s) {
    if (s == 0.0f) return 0.0f;
    float r = __builtin_rintf(__fdiv_rn(w, s));
    return __builtin_fminf(__builtin_fmaxf(r, (float)-QMAX), (float)QMAX);
}

template <int QMAX, int NCLIPS, typename WT>
__global__ __launch_bounds__(256) void pack_sym_kernel(const WT *__restrict__ W, int64_t N, int K,
                                                       uint8_t *__restrict__ codes, uint16_t *__restrict__ scale) {
    const int nb = K / 32;
    int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= N * nb) return;
    int64_t row = gid / nb;
    int blk = (int)(gid % nb);
    float w[32];
    load_block_f32<WT>(W, row * K + (int64_t)blk * 32, w);
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 32; k++) amax = __builtin_fmaxf(amax, __builtin_fabsf(w[k]));

    float best_err = __builtin_inff();
    uint16_t best_s16 = 0;
#pragma unroll 1
    for (int ci = 0; ci < NCLIPS; ci++) {
        float t = __fmul_rn(clip_ratio(ci), amax);
        uint16_t s16 = f32_to_f16_bits(__fdiv_rn(t, (float)QMAX));
        float s = f16_bits_to_f32(s16);
        float err = 0.0f;
#pragma unroll
        for (int k = 0; k < 32; k++) {
            float q = quant_q<QMAX>(w[k], s);
            float d = __fsub_rn(w[k], __fmul_rn(s, q));
            err = __fmaf_rn(d, d, err);
        }
        if (err < best_err) {
            best_err = err;
            best_s16 = s16;
        }
    }
    const float s = f16_bits_to_f32(best_s16);
    scale[row * nb + blk] = best_s16;
    if constexpr (QMAX == 7) {
        uint32_t out[4];
#pragma unroll
        for (int d = 0; d < 4; d++) {
            uint32_t v = 0;
#pragma unroll
            for (int i = 0; i < 8; i++) v |= (uint32_t)((int)quant_q<QMAX>(w[8 * d + i], s) + 8) << (4 * i);
            out[d] = v;
        }
        *reinterpret_cast<uint4 *>(codes + row * (int64_t)(K / 2) + (int64_t)blk * 16) =
            make_uint4(out[0], out[1], out[2], out[3]);
    } else {
        uint32_t out[8];
#pragma unroll
        for (int d = 0; d < 8; d++) {
            uint32_t v = 0;
#pragma unroll
            for (int i = 0; i < 4; i++) v |= ((uint32_t)(int)quant_q<QMAX>(w[4 * d + i], s) & 0xFFu) << (8 * i);
            out[d] = v;
        }
        uint4 *o = reinterpret_cast<uint4 *>(codes + row * (int64_t)K + (int64_t)blk * 32);
        o[0] = make_uint4(out[0], out[1], out[2], out[3]);
        o[1] = make_uint4(out[4], out[5], out[6], out[7]);
    }
}

// ---------------------------------------------------------------------------
// FP4 E2M1 with e8m0 scale.
// ---------------------------------------------------------------------------
// Magnitude code of m >= 0 by the decision points between adjacent grid
// values {0, .5, 1, 1.5, 2, 3, 4, 6}; a midpoint goes to the even code.
__device__ __forceinline__ uint32_t e2m1_code(float m) {
    uint32_t c = (m > 0.25f) + (m >= 0.75f) + (m > 1.25f) + (m >= 1.75f) + (m > 2.5f) + (m >= 3.5f) + (m > 5.0f);
    return c;
}

template <typename WT>
__global__ __launch_bounds__(256) void pack_fp4_kernel(const WT *__restrict__ W, int64_t N, int K,
                                                       uint8_t *__restrict__ codes, uint8_t *__restrict__ scale) {
    const int nb = K / 32;
    int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= N * nb) return;
    int64_t row = gid / nb;
    int blk = (int)(gid % nb);
    float w[32];
    load_block_f32<WT>(W, row * K + (int64_t)blk * 32, w);
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 32; k++) amax = __builtin_fmaxf(amax, __builtin_fabsf(w[k]));
    int E = -127;
    if (amax > 0.0f) {
        int ex;
        __builtin_frexpf(amax, &ex);   // amax = f * 2^ex, f in [0.5, 1): floor(log2 amax) = ex - 1
        E = ex - 1 - 2;
        E = E < -127 ? -127 : (E > 127 ? 127 : E);
    }
    scale[row * nb + blk] = (uint8_t)(E + 127);
    uint32_t out[4];
#pragma unroll
    for (int d = 0; d < 4; d++) {
        uint32_t v = 0;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            float x = w[8 * d + i];
            float m = __builtin_ldexpf(__builtin_fabsf(x), -E);   // exact
            uint32_t c = e2m1_code(m) | ((__builtin_bit_cast(uint32_t, x) >> 31) << 3);
            v |= c << (4 * i);
        }
        out[d] = v;
    }
    *reinterpret_cast<uint4 *>(codes + row * (int64_t)(K / 2) + (int64_t)blk * 16) =
        make_uint4(out[0], out[1], out[2], out[3]);
}

// ---------------------------------------------------------------------------
// km4: per-row k-means on exact integers (value * 2^24), one workgroup per row.
//   sort the row (bitonic, LDS), prefix sums of the sorted values, then Lloyd
//   steps where every cluster is a contiguous range of the sorted row, so its
//   count and sum come from two binary searches and two prefix-sum reads.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int64_t units_of_f16(uint32_t h) {
    uint32_t e = (h >> 10) & 31u, f = h & 1023u;
    int64_t mag = e ? ((int64_t)(1024 + f) << (e - 1)) : (int64_t)f;
    return (h & 0x8000u) ? -mag : mag;
}

__device__ __forceinline__ uint16_t f16_of_units(int64_t v) {
    uint64_t a = v < 0 ? (uint64_t)(-v) : (uint64_t)v;
    uint32_t bits;
    if (a < 2048) {
        bits = (uint32_t)a;                     // subnormals and the first binade
    } else {
        int s = 63 - __builtin_clzll(a) - 10;   // a = M * 2^s, M in [1024, 2048)
        bits = ((uint32_t)s << 10) + (uint32_t)(a >> s);
    }
    return (uint16_t)(bits | (v < 0 ? 0x8000u : 0u));
}

// nearest fp16 number (as units) to sum/cnt, ties to the even significand
__device__ __forceinline__ int64_t mean_to_f16_units(int64_t sum, int64_t cnt) {
    uint64_t a = sum < 0 ? (uint64_t)(-sum) : (uint64_t)sum;
    uint64_t n = (uint64_t)cnt;
    uint64_t q = 1;
    while (a >= 2048ull * q * n) q <<= 1;
    uint64_t qn = q * n;
    uint64_t m = a / qn;
    uint64_t r = a - m * qn;
    if (2 * r > qn || (2 * r == qn && (m & 1))) m += 1;
    int64_t v = (int64_t)(m * q);
    return sum < 0 ? -v : v;
}

__device__ __forceinline__ uint16_t sort_key(uint16_t h) {
    return (h & 0x8000u) ? (uint16_t)~h : (uint16_t)(h | 0x8000u);
}
__device__ __forceinline__ uint16_t unsort_key(uint16_t k) {
    return (k & 0x8000u) ? (uint16_t)(k & 0x7FFFu) : (uint16_t)~k;
}

constexpr int kKmThreads = 256;

// With outliers (nout > 0, columns ocol[row][.]) the row is palettized with
// those entries taken as +0; they are stored apart (pack_outliers_kernel).
__global__ __launch_bounds__(kKmThreads) void pack_km4_kernel(const uint16_t *__restrict__ W, int64_t N, int K,
                                                              int P, int max_iter, uint8_t *__restrict__ codes,
                                                              uint16_t *__restrict__ lut,
                                                              const uint16_t *__restrict__ ocol, int nout) {
    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t *keys = reinterpret_cast<uint16_t *>(smem);                        // P keys
    int64_t *ps = reinterpret_cast<int64_t *>(smem + ((2 * P + 15) & ~15));     // K + 1 prefix sums
    __shared__ int64_t tsum[kKmThreads];
    __shared__ int tcnt[kKmThreads];
    __shared__ int64_t cent[16];
    __shared__ int ndistinct;
    __shared__ uint32_t omask[128];   // outlier columns (K <= 4096)

    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    const uint16_t *wr = W + row * (int64_t)K;

    for (int i = tid; i < P; i += kKmThreads) keys[i] = i < K ? sort_key(wr[i]) : (uint16_t)0xFFFFu;
    if (nout > 0) {
        for (int i = tid; i < 128; i += kKmThreads) omask[i] = 0;
        __syncthreads();
        for (int o = tid; o < nout; o += kKmThreads) {
            const int col = ocol[row * nout + o];
            keys[col] = sort_key(0);
            atomicOr(&omask[col >> 5], 1u << (col & 31));
        }
    }
    __syncthreads();
    // bitonic sort, ascending
    for (int k = 2; k <= P; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = tid; i < P; i += kKmThreads) {
                int ixj = i ^ j;
                if (ixj > i) {
                    uint16_t a = keys[i], b = keys[ixj];
                    bool up = (i & k) == 0;
                    if ((a > b) == up) {
                        keys[i] = b;
                        keys[ixj] = a;
                    }
                }
            }
            __syncthreads();
        }
    }
    // per-thread segments: sums and distinct-value starts
    const int seg = (K + kKmThreads - 1) / kKmThreads;
    const int lo = tid * seg < K ? tid * seg : K;
    const int hi = lo + seg < K ? lo + seg : K;
    int64_t s = 0;
    int cnt = 0;
    for (int i = lo; i < hi; i++) {
        int64_t xv = units_of_f16(unsort_key(keys[i]));
        s += xv;
        cnt += (i == 0) || xv != units_of_f16(unsort_key(keys[i - 1]));
    }
    tsum[tid] = s;
    tcnt[tid] = cnt;
    __syncthreads();
    // inclusive scan over the thread totals (Hillis-Steele)
    for (int off = 1; off < kKmThreads; off <<= 1) {
        int64_t a = tid >= off ? tsum[tid - off] : 0;
        int c = tid >= off ? tcnt[tid - off] : 0;
        __syncthreads();
        tsum[tid] += a;
        tcnt[tid] += c;
        __syncthreads();
    }
    int64_t base = tid ? tsum[tid - 1] : 0;
    int rank = tid ? tcnt[tid - 1] : 0;
    if (tid == kKmThreads - 1) ndistinct = tcnt[tid];
    if (tid == 0) ps[0] = 0;
    __syncthreads();
    const bool few = ndistinct <= 16;
    for (int i = lo; i < hi; i++) {
        int64_t xv = units_of_f16(unsort_key(keys[i]));
        base += xv;
        ps[i + 1] = base;
        if (few && ((i == 0) || xv != units_of_f16(unsort_key(keys[i - 1])))) {
            cent[rank] = xv;
            rank++;
        }
    }
    __syncthreads();
    if (tid < 16) {
        if (few) {
            if (tid >= ndistinct) cent[tid] = units_of_f16(unsort_key(keys[K - 1]));
        } else {
            cent[tid] = units_of_f16(unsort_key(keys[(2 * tid + 1) * (K / 32)]));
        }
    }
    __syncthreads();
    // Lloyd steps in the first wave; lane j owns centroid j
    if (!few && tid < kWave) {
        int64_t c = tid < 16 ? cent[tid] : 0;
        for (int it = 0; it < max_iter; it++) {
            int64_t nxt = __shfl_down(c, 1);
            int b = K;   // lane 15: end of the row
            if (tid < 15) {
                // first sorted index whose doubled value exceeds c_j + c_{j+1}
                int64_t t = c + nxt;
                int l = 0, h = K;
                while (l < h) {
                    int mid = (l + h) >> 1;
                    if (2 * units_of_f16(unsort_key(keys[mid])) > t) h = mid;
                    else l = mid + 1;
                }
                b = l;
            }
            int bprev = __shfl_up(b, 1);
            if (tid == 0) bprev = 0;
            int64_t cn = c;
            if (tid < 16) {
                int64_t n = b - bprev;
                if (n > 0) cn = mean_to_f16_units(ps[b] - ps[bprev], n);
            }
            bool moved = __any(tid < 16 && cn != c);
            c = cn;
            if (!moved) break;
        }
        if (tid < 16) cent[tid] = c;
    }
    __syncthreads();
    // thresholds and final nearest-centroid indices in the row's own order
    int64_t thr[15];
#pragma unroll
    for (int i = 0; i < 15; i++) thr[i] = cent[i] + cent[i + 1];
    uint32_t *crow = reinterpret_cast<uint32_t *>(codes + row * (int64_t)(K / 2));
    for (int g = tid; g < K / 8; g += kKmThreads) {
        uint4 raw = *reinterpret_cast<const uint4 *>(wr + 8 * g);
        uint32_t d[4] = {raw.x, raw.y, raw.z, raw.w};
        uint32_t v = 0;
#pragma unroll
        for (int e = 0; e < 8; e++) {
            uint32_t h = (d[e / 2] >> (16 * (e & 1))) & 0xFFFFu;
            if (nout > 0) {
                const int col = 8 * g + e;
                if ((omask[col >> 5] >> (col & 31)) & 1u) h = 0;
            }
            int64_t x2 = 2 * units_of_f16(h);
            uint32_t a = 0;
#pragma unroll
            for (int i = 0; i < 15; i++) a += thr[i] < x2;
            v |= a << (4 * e);
        }
        crow[g] = v;
    }
    if (tid < 16) lut[row * 16 + tid] = f16_of_units(cent[tid]);
}

// ---------------------------------------------------------------------------
// Outliers of a 4-bit k-means row ("Kernel campaign - session handoff", NEXT
// per lever, Stream D: int4 plus int8 outliers): the nout entries of largest
// magnitude (ties to the lower column), listed by increasing column, as int8
// with one fp16 scale per row (s = fp16(max |w| / 127), q = rint(w / s)).
// One workgroup per row: magnitude/column keys sorted in LDS (descending),
// the chosen columns sorted again (ascending).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kKmThreads) void pack_outliers_kernel(const uint16_t *__restrict__ W, int K, int P,
                                                                   int nout, uint16_t *__restrict__ ocol,
                                                                   int8_t *__restrict__ oval,
                                                                   uint16_t *__restrict__ oscale) {
    extern __shared__ __align__(16) unsigned char smem[];
    uint32_t *keys = reinterpret_cast<uint32_t *>(smem);   // P keys (P a power of two >= K)
    __shared__ uint32_t cols[256];
    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    const uint16_t *wr = W + row * (int64_t)K;
    // larger magnitude first; equal magnitudes: the lower column first
    for (int i = tid; i < P; i += kKmThreads)
        keys[i] = i < K ? (((uint32_t)wr[i] & 0x7FFFu) << 16) | (0xFFFFu - (uint32_t)i) : 0u;
    __syncthreads();
    for (int k = 2; k <= P; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int p = tid; p < P / 2; p += kKmThreads) {
                const int i = 2 * p - (p & (j - 1));
                const int ixj = i + j;
                const uint32_t a = keys[i], b = keys[ixj];
                if ((a < b) == ((i & k) == 0)) {
                    keys[i] = b;
                    keys[ixj] = a;
                }
            }
            __syncthreads();
        }
    }
    // the chosen columns, ascending (256 slots, unused ones sort last)
    cols[tid] = tid < nout ? 0xFFFFu - (keys[tid] & 0xFFFFu) : 0xFFFFFFFFu;
    __syncthreads();
    for (int k = 2; k <= 256; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            const int ixj = tid ^ j;
            uint32_t a = 0, b = 0;
            const bool act = ixj > tid;
            if (act) {
                a = cols[tid];
                b = cols[ixj];
            }
            __syncthreads();
            if (act && ((a > b) == ((tid & k) == 0))) {
                cols[tid] = b;
                cols[ixj] = a;
            }
            __syncthreads();
        }
    }
    const float amax = f16_bits_to_f32((uint16_t)(keys[0] >> 16));
    const uint16_t s16 = f32_to_f16_bits(__fdiv_rn(amax, 127.0f));
    const float sc = f16_bits_to_f32(s16);
    if (tid == 0) oscale[row] = s16;
    if (tid < nout) {
        const int col = (int)cols[tid];
        const float w = f16_bits_to_f32(wr[col]);
        float q = 0.f;
        if (sc != 0.f) q = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(__fdiv_rn(w, sc)), -127.f), 127.f);
        ocol[row * nout + tid] = (uint16_t)col;
        oval[row * nout + tid] = (int8_t)q;
    }
}

// ---------------------------------------------------------------------------
// int8km: one 256-entry table per group of 32 rows ("coreai-optimization
// reference", Palettization: 2^n_bits centroids, per-grouped-channel; the
// "Compression" page's recipe: int8 k-means, group 32). The km4 procedure on
// the group's M = 32 K values, one 1024-thread workgroup per group:
//   the keys are sorted in LDS (bitonic over P = M rounded up to a power of
//   two); the sorted values' prefix sums are kept every 64 keys (a full prefix
//   array would not fit next to the keys), so the prefix at any position is
//   one of them plus at most 63 keys; in each Lloyd step thread j < 256 owns
//   entry j, finds its cluster's upper edge by binary search and takes the
//   exact mean from two prefixes.
// ---------------------------------------------------------------------------
constexpr int kKm8Threads = 1024;
constexpr int kKm8MaxKeys = 65536;   // M <= 65536: K <= 2048

// inclusive prefix sum over the 1024 threads of the workgroup
__device__ __forceinline__ int64_t block_scan_1024(int64_t v, int64_t *wtot) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int64_t t = __shfl_up(v, o);
        if (lane >= o) v += t;
    }
    if (lane == 63) wtot[w] = v;
    __syncthreads();
    int64_t add = 0;
    for (int i = 0; i < w; i++) add += wtot[i];
    __syncthreads();
    return v + add;
}

__global__ __launch_bounds__(kKm8Threads) void pack_int8km_kernel(const uint16_t *__restrict__ W, int K, int P,
                                                                  int max_iter, uint8_t *__restrict__ codes,
                                                                  uint16_t *__restrict__ lut) {
    __shared__ uint16_t keys[kKm8MaxKeys];
    __shared__ int64_t ps64[kKm8MaxKeys / 64 + 1];   // sum of the sorted values before key 64 c
    __shared__ int64_t cent[256];
    __shared__ int64_t pre[256];                      // prefix at each cluster's upper edge; then thresholds
    __shared__ int bnd[256];
    __shared__ int64_t wtot[16];
    __shared__ int ndistinct;

    const int tid = threadIdx.x;
    const int M = 32 * K;
    const int NC = M / 64;
    const int64_t g = blockIdx.x;
    const uint16_t *wg = W + g * (int64_t)M;

    for (int v = tid; v < M / 8; v += kKm8Threads) {
        const uint4 raw = reinterpret_cast<const uint4 *>(wg)[v];
        const uint32_t d[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e = 0; e < 8; e++) keys[8 * v + e] = sort_key((uint16_t)(d[e / 2] >> (16 * (e & 1))));
    }
    for (int i = M + tid; i < P; i += kKm8Threads) keys[i] = 0xFFFFu;
    __syncthreads();
    // bitonic sort, ascending; every thread takes compare-exchange pairs
    for (int k = 2; k <= P; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int p = tid; p < P / 2; p += kKm8Threads) {
                const int i = 2 * p - (p & (j - 1));
                const int ixj = i + j;
                const uint16_t a = keys[i], b = keys[ixj];
                if ((a > b) == ((i & k) == 0)) {
                    keys[i] = b;
                    keys[ixj] = a;
                }
            }
            __syncthreads();
        }
    }
    // 64-key chunks: sums and distinct-value starts, then their prefix sums
    int64_t csum = 0;
    int ccnt = 0;
    if (tid < NC) {
        int64_t prev = tid ? units_of_f16(unsort_key(keys[64 * tid - 1])) : 0;
        for (int i = 64 * tid; i < 64 * tid + 64; i++) {
            const int64_t xv = units_of_f16(unsort_key(keys[i]));
            csum += xv;
            ccnt += (i == 0) || xv != prev;
            prev = xv;
        }
    }
    const int64_t sincl = block_scan_1024(csum, wtot);
    const int64_t cincl = block_scan_1024(ccnt, wtot);
    if (tid < NC) ps64[tid] = sincl - csum;
    if (tid == NC - 1) {
        ps64[NC] = sincl;
        ndistinct = (int)cincl;
    }
    __syncthreads();
    const bool few = ndistinct <= 256;
    if (few) {
        if (tid < NC) {
            int rank = (int)(cincl - ccnt);
            int64_t prev = tid ? units_of_f16(unsort_key(keys[64 * tid - 1])) : 0;
            for (int i = 64 * tid; i < 64 * tid + 64; i++) {
                const int64_t xv = units_of_f16(unsort_key(keys[i]));
                if (i == 0 || xv != prev) cent[rank++] = xv;
                prev = xv;
            }
        }
        __syncthreads();
        if (tid >= ndistinct && tid < 256) cent[tid] = units_of_f16(unsort_key(keys[M - 1]));
    } else if (tid < 256) {
        cent[tid] = units_of_f16(unsort_key(keys[(2 * tid + 1) * (M / 512)]));
    }
    __syncthreads();
    if (!few) {
        for (int it = 0; it < max_iter; it++) {
            if (tid < 256) {
                int b = M;
                if (tid < 255) {
                    // first sorted index whose doubled value exceeds c_j + c_{j+1}
                    const int64_t t = cent[tid] + cent[tid + 1];
                    int l = 0, h = M;
                    while (l < h) {
                        const int mid = (l + h) >> 1;
                        if (2 * units_of_f16(unsort_key(keys[mid])) > t) h = mid;
                        else l = mid + 1;
                    }
                    b = l;
                }
                int64_t pb = ps64[b >> 6];
                for (int i = b & ~63; i < b; i++) pb += units_of_f16(unsort_key(keys[i]));
                bnd[tid] = b;
                pre[tid] = pb;
            }
            __syncthreads();
            int64_t cn = 0;
            bool moved = false;
            if (tid < 256) {
                const int lo = tid ? bnd[tid - 1] : 0;
                const int64_t plo = tid ? pre[tid - 1] : 0;
                const int64_t n = bnd[tid] - lo;
                cn = n > 0 ? mean_to_f16_units(pre[tid] - plo, n) : cent[tid];
                moved = cn != cent[tid];
            }
            __syncthreads();
            if (tid < 256) cent[tid] = cn;
            if (!__syncthreads_or(moved)) break;
        }
    }
    // thresholds c_j + c_{j+1}; a value's index is how many lie below twice it
    if (tid < 255) pre[tid] = cent[tid] + cent[tid + 1];
    __syncthreads();
    uint8_t *cg = codes + g * (int64_t)M;
    for (int u = tid; u < M / 16; u += kKm8Threads) {
        const uint4 r0 = reinterpret_cast<const uint4 *>(wg)[2 * u];
        const uint4 r1 = reinterpret_cast<const uint4 *>(wg)[2 * u + 1];
        const uint32_t d[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
        uint32_t out[4] = {0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 16; e++) {
            const int64_t x2 = 2 * units_of_f16((d[e / 2] >> (16 * (e & 1))) & 0xFFFFu);
            int l = 0, h = 255;
            while (l < h) {
                const int mid = (l + h) >> 1;
                if (pre[mid] < x2) l = mid + 1;
                else h = mid;
            }
            out[e / 4] |= (uint32_t)l << (8 * (e & 3));
        }
        reinterpret_cast<uint4 *>(cg)[u] = make_uint4(out[0], out[1], out[2], out[3]);
    }
    if (tid < 256) lut[g * 256 + tid] = f16_of_units(cent[tid]);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static int blocks_grid(int64_t N, int64_t K) { return (int)((N * (K / 32) + 255) / 256); }

hipError_t launch_pack_int4(const void *W, qmv_dtype wdt, int64_t N, int64_t K, uint8_t *codes, uint16_t *scale,
                            hipStream_t st) {
    if (wdt == QMV_F16)
        hipLaunchKernelGGL((pack_sym_kernel<7, 7, _Float16>), dim3(blocks_grid(N, K)), dim3(256), 0, st,
                           reinterpret_cast<const _Float16 *>(W), N, (int)K, codes, scale);
    else
        hipLaunchKernelGGL((pack_sym_kernel<7, 7, float>), dim3(blocks_grid(N, K)), dim3(256), 0, st,
                           reinterpret_cast<const float *>(W), N, (int)K, codes, scale);
    return hipGetLastError();
}

hipError_t launch_pack_int8(const void *W, qmv_dtype wdt, int64_t N, int64_t K, int8_t *codes, uint16_t *scale,
                            hipStream_t st) {
    uint8_t *c = reinterpret_cast<uint8_t *>(codes);
    if (wdt == QMV_F16)
        hipLaunchKernelGGL((pack_sym_kernel<127, 1, _Float16>), dim3(blocks_grid(N, K)), dim3(256), 0, st,
                           reinterpret_cast<const _Float16 *>(W), N, (int)K, c, scale);
    else
        hipLaunchKernelGGL((pack_sym_kernel<127, 1, float>), dim3(blocks_grid(N, K)), dim3(256), 0, st,
                           reinterpret_cast<const float *>(W), N, (int)K, c, scale);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Affine int4 blocks ("Stream D - Quantization", section 1: affine int4 with
// block 32 among the MoE gather formats). Min-max: b = fp16(min),
// s = fp16((max - min) / 15), u = clamp(rint((w - b) / s), 0, 15); plane
// word = scale | bias << 16. One thread per block, one IEEE op per step.
// ---------------------------------------------------------------------------
template <typename WT>
__global__ __launch_bounds__(256) void pack_int4aff_kernel(const WT *__restrict__ W, int64_t N, int K,
                                                           uint8_t *__restrict__ codes, uint32_t *__restrict__ plane) {
    const int nb = K / 32;
    int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= N * nb) return;
    int64_t row = gid / nb;
    int blk = (int)(gid % nb);
    float w[32];
    load_block_f32<WT>(W, row * K + (int64_t)blk * 32, w);
    float mn = w[0], mx = w[0];
#pragma unroll
    for (int k = 1; k < 32; k++) {
        mn = w[k] < mn ? w[k] : mn;
        mx = w[k] > mx ? w[k] : mx;
    }
    const uint16_t s16 = f32_to_f16_bits(__fdiv_rn(__fsub_rn(mx, mn), 15.0f));
    const uint16_t b16 = f32_to_f16_bits(mn);
    const float s = f16_bits_to_f32(s16), b = f16_bits_to_f32(b16);
    plane[row * nb + blk] = (uint32_t)s16 | ((uint32_t)b16 << 16);
    uint32_t out[4];
#pragma unroll
    for (int d = 0; d < 4; d++) {
        uint32_t v = 0;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            float u = 0.0f;
            if (s != 0.0f)
                u = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(__fdiv_rn(__fsub_rn(w[8 * d + i], b), s)), 0.0f),
                                    15.0f);
            v |= (uint32_t)u << (4 * i);
        }
        out[d] = v;
    }
    *reinterpret_cast<uint4 *>(codes + row * (int64_t)(K / 2) + (int64_t)blk * 16) =
        make_uint4(out[0], out[1], out[2], out[3]);
}

hipError_t launch_pack_int4aff(const void *W, qmv_dtype wdt, int64_t N, int64_t K, uint8_t *codes, uint32_t *plane,
                               hipStream_t st) {
    if (wdt == QMV_F16)
        hipLaunchKernelGGL((pack_int4aff_kernel<_Float16>), dim3(blocks_grid(N, K)), dim3(256), 0, st,
                           reinterpret_cast<const _Float16 *>(W), N, (int)K, codes, plane);
    else
        hipLaunchKernelGGL((pack_int4aff_kernel<float>), dim3(blocks_grid(N, K)), dim3(256), 0, st,
                           reinterpret_cast<const float *>(W), N, (int)K, codes, plane);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Embedding table: int8 with one fp16 scale per row ("coreai-optimization
// reference", "The LM head + embeddings": plain int8 per-row dequant-gather).
// One workgroup per row: amax over the row, s = fp16(amax / 127), q =
// clamp(rint(w / s), -127, 127), each step one IEEE operation.
// ---------------------------------------------------------------------------
template <typename WT>
__global__ __launch_bounds__(256) void pack_int8_rows_kernel(const WT *__restrict__ W, int64_t H,
                                                             int8_t *__restrict__ codes, uint16_t *__restrict__ scale) {
    const int64_t v = blockIdx.x;
    const WT *w = W + v * H;
    float amax = 0.0f;
    for (int64_t h = threadIdx.x; h < H; h += 256) amax = __builtin_fmaxf(amax, __builtin_fabsf((float)w[h]));
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, m));
    __shared__ float red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
    const uint16_t s16 = f32_to_f16_bits(__fdiv_rn(amax, 127.0f));
    const float s = f16_bits_to_f32(s16);
    if (threadIdx.x == 0) scale[v] = s16;
    for (int64_t h = threadIdx.x; h < H; h += 256) codes[v * H + h] = (int8_t)quant_q<127>((float)w[h], s);
}

hipError_t launch_pack_int8_rows(const void *W, qmv_dtype wdt, int64_t V, int64_t H, int8_t *codes, uint16_t *scale,
                                 hipStream_t st) {
    if (wdt == QMV_F16)
        hipLaunchKernelGGL(pack_int8_rows_kernel<_Float16>, dim3((unsigned)V), dim3(256), 0, st,
                           reinterpret_cast<const _Float16 *>(W), H, codes, scale);
    else
        hipLaunchKernelGGL(pack_int8_rows_kernel<float>, dim3((unsigned)V), dim3(256), 0, st,
                           reinterpret_cast<const float *>(W), H, codes, scale);
    return hipGetLastError();
}

hipError_t launch_pack_fp4(const void *W, qmv_dtype wdt, int64_t N, int64_t K, uint8_t *codes, uint8_t *scale,
                           hipStream_t st) {
    if (wdt == QMV_F16)
        hipLaunchKernelGGL((pack_fp4_kernel<_Float16>), dim3(blocks_grid(N, K)), dim3(256), 0, st,
                           reinterpret_cast<const _Float16 *>(W), N, (int)K, codes, scale);
    else
        hipLaunchKernelGGL((pack_fp4_kernel<float>), dim3(blocks_grid(N, K)), dim3(256), 0, st,
                           reinterpret_cast<const float *>(W), N, (int)K, codes, scale);
    return hipGetLastError();
}

hipError_t launch_pack_km4(const uint16_t *W, int64_t N, int64_t K, int max_iter, uint8_t *codes, uint16_t *lut,
                           hipStream_t st, const uint16_t *ocol, int nout) {
    int P = 32;
    while (P < K) P <<= 1;
    size_t shmem = (size_t)((2 * P + 15) & ~15) + sizeof(int64_t) * (size_t)(K + 1);
    // one workgroup per row; rows beyond the grid limit are covered by chunks
    const int64_t chunk = 1 << 30;
    for (int64_t r0 = 0; r0 < N; r0 += chunk) {
        int64_t rows = N - r0 < chunk ? N - r0 : chunk;
        hipLaunchKernelGGL(pack_km4_kernel, dim3((unsigned)rows), dim3(kKmThreads), shmem, st, W + r0 * K, rows,
                           (int)K, P, max_iter, codes + r0 * (K / 2), lut + r0 * 16,
                           ocol ? ocol + r0 * nout : nullptr, nout);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

__global__ __launch_bounds__(256) void zero_u16_kernel(uint16_t *__restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0;
}

hipError_t launch_pack_km4o(const uint16_t *W, int64_t N, int64_t K, int nout, int max_iter, uint8_t *codes,
                            uint16_t *lut, uint16_t *ocol, int8_t *oval, uint16_t *oscale, hipStream_t st) {
    if (nout > 0) {
        int P = 32;
        while (P < K) P <<= 1;
        const int64_t chunk = 1 << 30;
        for (int64_t r0 = 0; r0 < N; r0 += chunk) {
            int64_t rows = N - r0 < chunk ? N - r0 : chunk;
            hipLaunchKernelGGL(pack_outliers_kernel, dim3((unsigned)rows), dim3(kKmThreads), sizeof(uint32_t) * P, st,
                               W + r0 * K, (int)K, P, nout, ocol + r0 * nout, oval + r0 * nout, oscale + r0);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    } else {
        hipLaunchKernelGGL(zero_u16_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, st, oscale, N);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return launch_pack_km4(W, N, K, max_iter, codes, lut, st, nout > 0 ? ocol : nullptr, nout);
}

hipError_t launch_pack_int8km(const uint16_t *W, int64_t N, int64_t K, int max_iter, uint8_t *codes, uint16_t *lut,
                              hipStream_t st) {
    int P = 1024;
    while (P < 32 * K) P <<= 1;
    hipLaunchKernelGGL(pack_int8km_kernel, dim3((unsigned)(N / 32)), dim3(kKm8Threads), 0, st, W, (int)K, P, max_iter,
                       codes, lut);
    return hipGetLastError();
}

}  // namespace qmv
