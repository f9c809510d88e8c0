/*
 * Oracle for block-quantized decode matvec.
 *
 * TEST INFRASTRUCTURE ONLY. This file is a plain, slow, deliberately simple CPU
 * statement of what the quantizers and the dequantize-matvec compute. Only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg may load it.
 * The GPU library never links, includes or calls it, and it includes nothing
 * from the GPU library.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no fast-math), so
 * every float operation below is one IEEE-754 operation rounded to nearest even.
 *
 * Sources (web pages of the "Core AI model zoo" knowledge base):
 *  [S1] "Stream D - Quantization (FP4 + QAT-int4): feasibility, first result,
 *       and plan": section 1 "Toolchain reality" (FP4 E2M1 dtype, block 32 along
 *       K, e8m0 scale formula, two values per byte, the default 4-bit recipe is
 *       int4 per-block-32 symmetric-with-clipping on axis 1, MoE expert slabs use
 *       a [1,1,1,32] block); section 2 "The de-risk experiment" (int4/int8
 *       symmetric-with-clipping with an MSE-optimal clip ratio per block from a
 *       grid that starts at 1.0 and ends at 0.7).
 *  [S2] "Dense-path int4km coverage + flagship Qwen3.6-35B - session findings &
 *       methods": section 1 "The lever" (fused int4km matvec for lm_head and
 *       attention q/o), section 8 "FP4 (E2M1) dense matvec" (codes packed 8 per
 *       32-bit word, per-row 16-entry k-means codebook, fixed E2M1 grid times a
 *       per-K-block e8m0 scale), section 8b (int4km is palettize_grouped with
 *       n_bits=4).
 *  [S3] "coreai-optimization (coreai-opt) reference - quantization &
 *       palettization": "Quantization" (symmetric schemes, per-block along the
 *       in-features axis), "Palettization" (2^n_bits centroids, scalar 1-D
 *       k-means, per-channel grouping), "Theoretical size".
 *  [S5] "Compression (palettization & quantization)": section "Per-channel int8
 *       on a big-vocab LM head: use per-block-32" (int8 per-block-32 head).
 *
 * Where the pages leave a step open, the reading taken is stated next to the
 * code that implements it.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* IEEE-754 binary16, written out from the format definition:               */
/* 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; exponent field 0 */
/* holds zero and subnormals (fraction * 2^-24).                              */
/* ------------------------------------------------------------------------ */

double orc_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* Encode a value that is already exactly representable in binary16. */
static uint16_t f16_encode_exact(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return sign | 0x7c00;
    int ex;
    frexp(a, &ex);          /* a = m * 2^ex, m in [0.5, 1) */
    int e = ex - 1;         /* floor(log2 a) */
    if (e < -14)            /* subnormal: a = f * 2^-24 */
        return sign | (uint16_t)ldexp(a, 24);
    uint16_t frac = (uint16_t)(ldexp(a, 10 - e) - 1024.0);
    return sign | (uint16_t)((e + 15) << 10) | frac;
}

/* Round a double to the nearest binary16 value, ties to even; overflow
   (magnitude >= 65520) gives infinity. */
uint16_t orc_f64_to_f16(double v)
{
    if (isnan(v))
        return 0x7e00;
    double a = fabs(v);
    double r;
    if (a == 0.0) {
        r = 0.0;
    } else {
        int ex;
        frexp(a, &ex);
        int e = ex - 1;
        int qexp = (e < -14) ? -24 : e - 10;       /* spacing of the grid at a */
        r = ldexp(nearbyint(ldexp(a, -qexp)), qexp); /* scaling by 2^k is exact */
        if (r >= 65520.0)
            r = INFINITY;
    }
    return f16_encode_exact(signbit(v) ? -r : r);
}

/* ------------------------------------------------------------------------ */
/* FP4 E2M1 with an e8m0 block scale [S1 section 1; S2 section 8].           */
/* ------------------------------------------------------------------------ */

/* Magnitudes of the eight E2M1 codes, code = (exponent << 1) | mantissa:
   exponent 0 is subnormal (mantissa * 0.5), otherwise 2^(exponent-1)*(1+m/2). */
static const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* floor(log2(a)) for finite a > 0, exact: read off frexp, never a rounded log2. */
static int floor_log2(double a)
{
    int ex;
    frexp(a, &ex);
    return ex - 1;
}

/* Nearest E2M1 magnitude index for m >= 0; ties go to the even index (even
   mantissa bit); anything above the largest value saturates to 6. */
static int e2m1_round_magnitude(double m)
{
    int best = 0;
    for (int i = 1; i < 8; i++) {
        double dbest = fabs(m - kE2M1[best]);
        double di = fabs(m - kE2M1[i]);
        if (di < dbest || (di == dbest && (i % 2) == 0 && (best % 2) != 0))
            best = i;
    }
    return best;
}

/* W: N x K values (fp32 or fp16 inputs, given here as fp32), row-major.
   codes: N x K/2 bytes, element 2j in the low nibble of byte j.
   scale: N x K/32 e8m0 bytes (value 2^(byte-127)). */
void orc_pack_fp4(const float *W, int64_t N, int64_t K, uint8_t *codes, uint8_t *scale)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        for (int64_t b = 0; b < K / 32; b++) {
            const float *w = W + n * K + b * 32;
            double amax = 0.0;
            for (int k = 0; k < 32; k++)
                if (fabs((double)w[k]) > amax)
                    amax = fabs((double)w[k]);
            /* scale = 2^(floor(log2 amax) - 2), the exponent clamped to the e8m0
               range; an all-zero block takes the smallest scale (byte 0). */
            int E = (amax == 0.0) ? -127 : floor_log2(amax) - 2;
            if (E < -127) E = -127;
            if (E > 127) E = 127;
            scale[n * (K / 32) + b] = (uint8_t)(E + 127);
            for (int k = 0; k < 32; k++) {
                double v = ldexp((double)w[k], -E);   /* exact */
                int idx = e2m1_round_magnitude(fabs(v));
                /* the code's sign bit is the input's sign bit */
                int c = (signbit(w[k]) ? 8 : 0) | idx;
                uint8_t *byte = codes + n * (K / 2) + b * 16 + k / 2;
                if (k % 2 == 0)
                    *byte = (uint8_t)c;
                else
                    *byte = (uint8_t)(*byte | (c << 4));
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Symmetric integer quantization with a per-block fp16 scale and an         */
/* MSE-chosen clip ratio [S1 sections 1 and 2; S3 "Quantization"].           */
/* ------------------------------------------------------------------------ */

/* Reading of the elided clip grid: seven ratios in steps of 0.05 from 1.0 down
   to 0.7, tried in that order; a later ratio replaces the kept one only when
   its block error is strictly smaller. */
static const float kClipsInt4[7] = {1.0f, 0.95f, 0.9f, 0.85f, 0.8f, 0.75f, 0.7f};
static const float kClipsNone[1] = {1.0f};

/* One block of 32: q holds the signed integers, returns the fp16 scale bits.
   Arithmetic in fp32, one rounding per operation:
     s  = fp16(fp32(fp32(c * amax) / qmax))   (scale stored as fp16, used rounded)
     q  = clamp(rint(w / s), -qmax, qmax)      (rint: nearest, ties to even)
     err = sum over k ascending of fmaf(d, d, err), d = w - s*q                 */
static uint16_t quant_block_sym(const float *w, int qmax, const float *clips, int nclips, int *q)
{
    float amax = 0.0f;
    for (int k = 0; k < 32; k++)
        if (fabsf(w[k]) > amax)
            amax = fabsf(w[k]);
    float best = INFINITY;
    uint16_t best_s16 = 0;
    for (int ci = 0; ci < nclips; ci++) {
        float t = clips[ci] * amax;
        float s32 = t / (float)qmax;
        uint16_t s16 = orc_f64_to_f16((double)s32);
        float s = (float)orc_f16_to_f64(s16);
        int qc[32];
        float err = 0.0f;
        for (int k = 0; k < 32; k++) {
            if (s == 0.0f) {
                qc[k] = 0;
            } else {
                float r = rintf(w[k] / s);
                if (r > (float)qmax) r = (float)qmax;
                if (r < (float)-qmax) r = (float)-qmax;
                qc[k] = (int)r;
            }
            float d = w[k] - s * (float)qc[k];
            err = fmaf(d, d, err);
        }
        if (err < best) {
            best = err;
            best_s16 = s16;
            memcpy(q, qc, sizeof(qc));
        }
    }
    return best_s16;
}

/* int4: codes N x K/2 bytes of u = q + 8 (element 2j in the low nibble);
   scale N x K/32 fp16 bits. nclips = 7 uses the clip grid, 1 plain absmax. */
void orc_pack_int4(const float *W, int64_t N, int64_t K, int nclips, uint8_t *codes, uint16_t *scale)
{
    const float *clips = (nclips == 1) ? kClipsNone : kClipsInt4;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        for (int64_t b = 0; b < K / 32; b++) {
            int q[32];
            scale[n * (K / 32) + b] = quant_block_sym(W + n * K + b * 32, 7, clips, nclips, q);
            for (int j = 0; j < 16; j++)
                codes[n * (K / 2) + b * 16 + j] = (uint8_t)((q[2 * j] + 8) | ((q[2 * j + 1] + 8) << 4));
        }
    }
}

/* int8 (per-block-32, symmetric, no clipping [S5]): codes N x K int8 in
   [-127, 127]; scale N x K/32 fp16 bits. */
void orc_pack_int8(const float *W, int64_t N, int64_t K, int8_t *codes, uint16_t *scale)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        for (int64_t b = 0; b < K / 32; b++) {
            int q[32];
            scale[n * (K / 32) + b] = quant_block_sym(W + n * K + b * 32, 127, kClipsNone, 1, q);
            for (int k = 0; k < 32; k++)
                codes[n * K + b * 32 + k] = (int8_t)q[k];
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Affine int4 per block of 32 [S1 section 1: the production MoE gather      */
/* formats include affine int4 with a scale and a bias per 32-block; S2      */
/* section 8: fp4 is that affine structure without the bias].               */
/* ------------------------------------------------------------------------ */

/* Reading: min-max affine, every step one fp32 operation:
     b = fp16(min), s = fp16((max - min) / 15),
     u = clamp(rint((w - b) / s), 0, 15)   (s == 0: u = 0),
   dequant w' = s * u + b. Plane: one 32-bit word per block with the fp16
   scale in the low half and the fp16 bias in the high half. Codes as int4:
   element 2j in the low nibble of byte j. */
void orc_pack_int4aff(const float *W, int64_t N, int64_t K, uint8_t *codes, uint32_t *plane)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        for (int64_t blk = 0; blk < K / 32; blk++) {
            const float *w = W + n * K + blk * 32;
            float mn = w[0], mx = w[0];
            for (int k = 1; k < 32; k++) {
                if (w[k] < mn) mn = w[k];
                if (w[k] > mx) mx = w[k];
            }
            uint16_t s16 = orc_f64_to_f16((double)((mx - mn) / 15.0f));
            uint16_t b16 = orc_f64_to_f16((double)mn);
            float s = (float)orc_f16_to_f64(s16), b = (float)orc_f16_to_f64(b16);
            plane[n * (K / 32) + blk] = (uint32_t)s16 | ((uint32_t)b16 << 16);
            int u[32];
            for (int k = 0; k < 32; k++) {
                float r = 0.0f;
                if (s != 0.0f) {
                    r = rintf((w[k] - b) / s);
                    if (r < 0.0f) r = 0.0f;
                    if (r > 15.0f) r = 15.0f;
                }
                u[k] = (int)r;
            }
            for (int j = 0; j < 16; j++)
                codes[n * (K / 2) + blk * 16 + j] = (uint8_t)(u[2 * j] | (u[2 * j + 1] << 4));
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Embedding table: int8 with one fp16 scale per row, and its dequant-gather */
/* [S3 "The LM head + embeddings": the front-end table gather is a plain     */
/* int8 per-row dequant-gather, q[ids] as fp16 times scale[ids]].            */
/* ------------------------------------------------------------------------ */

/* Reading: the per-row scale follows the block recipe with the block being
   the whole row and no clipping: s = fp16(fp32(amax) / 127), q = clamp(rint(
   w / s), -127, 127) in fp32; an all-zero row has s = +0 and q = 0. */
void orc_pack_int8_rows(const float *W, int64_t V, int64_t H, int8_t *codes, uint16_t *scale)
{
#pragma omp parallel for schedule(static)
    for (int64_t v = 0; v < V; v++) {
        const float *w = W + v * H;
        float amax = 0.0f;
        for (int64_t h = 0; h < H; h++)
            if (fabsf(w[h]) > amax)
                amax = fabsf(w[h]);
        uint16_t s16 = orc_f64_to_f16((double)(amax / 127.0f));
        float s = (float)orc_f16_to_f64(s16);
        scale[v] = s16;
        for (int64_t h = 0; h < H; h++) {
            float r = 0.0f;
            if (s != 0.0f) {
                r = rintf(w[h] / s);
                if (r > 127.0f) r = 127.0f;
                if (r < -127.0f) r = -127.0f;
            }
            codes[v * H + h] = (int8_t)r;
        }
    }
}

/* out[t][h] = fp16(q[ids[t]][h] * scale[ids[t]]): the product of an int8 and
   an fp16 number is exact in fp64, so this is one rounding to fp16. Reading
   (the pages do not cover it): an id outside [0, V) names no row and gives a
   zero row. */
void orc_embed_gather_int8(const int8_t *codes, const uint16_t *scale, int64_t V, int64_t H, const int32_t *ids,
                           int64_t T, uint16_t *out)
{
    for (int64_t t = 0; t < T; t++) {
        const int64_t v = ids[t];
        if (v < 0 || v >= V) {
            for (int64_t h = 0; h < H; h++)
                out[t * H + h] = 0;
            continue;
        }
        const double s = orc_f16_to_f64(scale[v]);
        for (int64_t h = 0; h < H; h++)
            out[t * H + h] = orc_f64_to_f16((double)codes[v * H + h] * s);
    }
}

/* ------------------------------------------------------------------------ */
/* 4-bit k-means palettization, one 16-entry fp16 table per output row       */
/* [S2 sections 1, 8, 8b; S3 "Palettization"].                               */
/*                                                                          */
/* Reading: all arithmetic is exact integer arithmetic on values scaled by    */
/* 2^24 (every fp16 number is an integer multiple of 2^-24), centroids are    */
/* always fp16 numbers, so the table is the centroid set itself.             */
/*   1. few distinct values: if the row holds at most 16 distinct numbers,    */
/*      they are the table (ascending, padded with the largest);             */
/*   2. otherwise start from the order statistics at ranks (2j+1)K/32;       */
/*   3. Lloyd steps, at most max_iter: assign each weight to the nearest      */
/*      centroid (a tie goes to the lower index), move every non-empty        */
/*      centroid to its members' mean rounded to the nearest fp16 number      */
/*      (ties to even), leave empty ones; stop when no centroid moves;        */
/*   4. assign once more with the final centroids.                            */
/* ------------------------------------------------------------------------ */

static int64_t f16_to_units(uint16_t h)
{
    int e = (h >> 10) & 0x1f;
    int64_t f = h & 0x3ff;
    int64_t mag = (e == 0) ? f : (1024 + f) << (e - 1);
    return (h & 0x8000) ? -mag : mag;
}

static uint16_t units_to_f16(int64_t v)
{
    return f16_encode_exact(ldexp((double)v, -24));
}

/* Nearest fp16 number to the rational a/n (units of 2^-24), ties to even. */
static int64_t round_mean_to_f16_units(int64_t a, int64_t n)
{
    int neg = a < 0;
    int64_t A = neg ? -a : a;
    int64_t q = 1;                       /* grid spacing at A/n */
    while (A >= 2048 * q * n)
        q *= 2;
    int64_t m = A / (q * n);
    int64_t r = A - m * q * n;
    if (2 * r > q * n || (2 * r == q * n && (m & 1)))
        m++;
    return neg ? -(m * q) : m * q;
}

static int cmp_i64(const void *a, const void *b)
{
    int64_t x = *(const int64_t *)a, y = *(const int64_t *)b;
    return (x > y) - (x < y);
}

static int nearest_centroid(const int64_t *C, int64_t x)
{
    int a = 0;
    for (int i = 0; i < 15; i++)
        if (C[i] + C[i + 1] < 2 * x)  /* midpoint strictly below x */
            a++;
    return a;
}

/* Returns the number of Lloyd updates taken (for tests). */
static int km4_row(const uint16_t *w, int64_t K, int max_iter, uint8_t *codes, uint16_t *lut)
{
    int64_t *X = malloc(sizeof(int64_t) * K);
    int64_t *S = malloc(sizeof(int64_t) * K);
    int *a = malloc(sizeof(int) * K);
    for (int64_t k = 0; k < K; k++)
        X[k] = S[k] = f16_to_units(w[k]);
    qsort(S, K, sizeof(int64_t), cmp_i64);

    int64_t C[16];
    int64_t D = 1;
    for (int64_t k = 1; k < K; k++)
        if (S[k] != S[k - 1])
            D++;
    int iters = 0;
    if (D <= 16) {
        int j = 0;
        for (int64_t k = 0; k < K; k++)
            if (k == 0 || S[k] != S[k - 1])
                C[j++] = S[k];
        for (; j < 16; j++)
            C[j] = S[K - 1];
    } else {
        for (int j = 0; j < 16; j++)
            C[j] = S[(2 * j + 1) * K / 32];
        for (int it = 0; it < max_iter; it++) {
            int64_t sum[16] = {0}, cnt[16] = {0}, Cn[16];
            for (int64_t k = 0; k < K; k++) {
                int j = nearest_centroid(C, X[k]);
                sum[j] += X[k];
                cnt[j] += 1;
            }
            int moved = 0;
            for (int j = 0; j < 16; j++) {
                Cn[j] = cnt[j] ? round_mean_to_f16_units(sum[j], cnt[j]) : C[j];
                if (Cn[j] != C[j])
                    moved = 1;
            }
            iters++;
            if (!moved)
                break;
            memcpy(C, Cn, sizeof(C));
        }
    }
    for (int64_t k = 0; k < K; k++)
        a[k] = nearest_centroid(C, X[k]);
    for (int j = 0; j < 16; j++)
        lut[j] = units_to_f16(C[j]);
    for (int64_t j = 0; j < K / 2; j++)
        codes[j] = (uint8_t)(a[2 * j] | (a[2 * j + 1] << 4));
    free(X);
    free(S);
    free(a);
    return iters;
}

/* W_f16: N x K fp16 bits; codes N x K/2; lut N x 16 fp16 bits; iters (may be
   NULL) receives the Lloyd update count per row. */
void orc_pack_km4(const uint16_t *W_f16, int64_t N, int64_t K, int max_iter,
                  uint8_t *codes, uint16_t *lut, int32_t *iters)
{
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n = 0; n < N; n++) {
        int it = km4_row(W_f16 + n * K, K, max_iter, codes + n * (K / 2), lut + n * 16);
        if (iters)
            iters[n] = it;
    }
}

/* ------------------------------------------------------------------------ */
/* 4-bit k-means rows plus int8 outliers [S4 "NEXT per lever", Stream D:     */
/* a mixed int4 + int8-outlier matvec built on the int4 k-means linear, to   */
/* bridge the int4 quality cliff at about int4 bandwidth].                   */
/*                                                                          */
/* Reading (the page names the idea only): per row, the P entries of largest */
/* magnitude (ties to the lower column) are outliers, listed by increasing   */
/* column. They are stored as int8 with one fp16 scale per row, the int8    */
/* per-row recipe: s = fp16(fp32(max |w|) / 127), q = clamp(rint(w / s),     */
/* -127, 127) in fp32 (s = 0 gives q = 0). The row with its outliers set to  */
/* +0 is palettized by the 4-bit k-means above. The weight is the sum of the */
/* two parts: W_hat[n][k] = lut[n][code] + (k an outlier ? s * q : 0).       */
/* ------------------------------------------------------------------------ */

/* W_f16: N x K fp16 bits; codes N x K/2; lut N x 16; ocol N x P (uint16);
   oval N x P (int8); oscale N (fp16 bits). 0 <= P <= K. */
void orc_pack_km4o(const uint16_t *W_f16, int64_t N, int64_t K, int P, int max_iter,
                   uint8_t *codes, uint16_t *lut, uint16_t *ocol, int8_t *oval, uint16_t *oscale)
{
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n = 0; n < N; n++) {
        const uint16_t *w = W_f16 + n * K;
        uint16_t *res = malloc(sizeof(uint16_t) * K);
        char *taken = calloc(K, 1);
        memcpy(res, w, sizeof(uint16_t) * K);
        /* the P largest magnitudes, ties to the lower column */
        for (int o = 0; o < P; o++) {
            int64_t best = -1;
            for (int64_t k = 0; k < K; k++)
                if (!taken[k] && (best < 0 || fabs(orc_f16_to_f64(w[k])) > fabs(orc_f16_to_f64(w[best]))))
                    best = k;
            taken[best] = 1;
        }
        float amax = 0.0f;
        for (int64_t k = 0; k < K; k++)
            if (taken[k] && fabsf((float)orc_f16_to_f64(w[k])) > amax)
                amax = fabsf((float)orc_f16_to_f64(w[k]));
        uint16_t s16 = orc_f64_to_f16((double)(amax / 127.0f));
        float s = (float)orc_f16_to_f64(s16);
        oscale[n] = s16;
        int o = 0;
        for (int64_t k = 0; k < K; k++) {
            if (!taken[k])
                continue;
            float q = 0.0f;
            if (s != 0.0f) {
                q = rintf((float)orc_f16_to_f64(w[k]) / s);
                if (q > 127.0f) q = 127.0f;
                if (q < -127.0f) q = -127.0f;
            }
            ocol[n * P + o] = (uint16_t)k;
            oval[n * P + o] = (int8_t)q;
            o++;
            res[k] = 0x0000;
        }
        km4_row(res, K, max_iter, codes + n * (K / 2), lut + n * 16);
        free(res);
        free(taken);
    }
}

/* y[b][n] = sum over k ascending of W_hat[n][k] * x[b][k] in fp64, W_hat as
   above (the dense part and the outlier part of a weight summed first). */
void orc_matvec_km4o(const uint8_t *codes, const uint16_t *lut, const uint16_t *ocol, const int8_t *oval,
                     const uint16_t *oscale, int64_t N, int64_t K, int P, const double *x, int B, double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        double *wh = malloc(sizeof(double) * K);
        for (int64_t k = 0; k < K; k++) {
            uint8_t byte = codes[n * (K / 2) + k / 2];
            int c = (k % 2 == 0) ? (byte & 0xf) : (byte >> 4);
            wh[k] = orc_f16_to_f64(lut[n * 16 + c]);
        }
        for (int o = 0; o < P; o++)
            wh[ocol[n * P + o]] += orc_f16_to_f64(oscale[n]) * (double)oval[n * P + o];
        for (int b = 0; b < B; b++) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; k++)
                acc += wh[k] * x[b * K + k];
            y[b * N + n] = acc;
        }
        free(wh);
    }
}

/* ------------------------------------------------------------------------ */
/* 8-bit k-means palettization, one 256-entry fp16 table per group of 32     */
/* consecutive output rows [S3 "Palettization": 2^n_bits centroids, 1-D     */
/* k-means, per-grouped-channel granularity; S3 "The LM head + embeddings"  */
/* and S5 "int8 k-means > whole-model int4": int8 k-means with group 32].    */
/*                                                                          */
/* Reading: the same procedure as the 4-bit tables above, over the 32*K      */
/* values of a group taken together (row-major), with 256 centroids:        */
/*   1. at most 256 distinct numbers: they are the table (ascending, padded  */
/*      with the largest);                                                   */
/*   2. otherwise start from the order statistics at ranks (2j+1)M/512 of    */
/*      the M = 32K sorted values;                                           */
/*   3. Lloyd steps, at most max_iter: a value v goes to the index equal to  */
/*      the number of adjacent centroid pairs (C[i], C[i+1]) whose midpoint  */
/*      lies strictly below v (the nearest centroid, a tie to the lower      */
/*      index; the centroids stay in ascending order); every non-empty       */
/*      centroid moves to its members' mean rounded to the nearest fp16      */
/*      number (ties to even), empty ones stay; stop when none moves;        */
/*   4. assign once more with the final centroids.                           */
/* A row count that is not a multiple of 32 is not a group layout.           */
/* ------------------------------------------------------------------------ */

#define KM8_L 256

static int nearest_centroid_l(const int64_t *C, int L, int64_t x)
{
    int a = 0;
    for (int i = 0; i + 1 < L; i++)
        if (C[i] + C[i + 1] < 2 * x)
            a++;
    return a;
}

/* w: M fp16 values of one group; idx: M indices; lut: 256 fp16 entries.
   Returns the number of Lloyd updates taken. max_iter 0 keeps the starting
   centroids (used by tests). */
static int km8_group(const uint16_t *w, int64_t M, int max_iter, uint8_t *idx, uint16_t *lut)
{
    int64_t *X = malloc(sizeof(int64_t) * M);
    int64_t *S = malloc(sizeof(int64_t) * M);
    for (int64_t k = 0; k < M; k++)
        X[k] = S[k] = f16_to_units(w[k]);
    qsort(S, M, sizeof(int64_t), cmp_i64);

    int64_t C[KM8_L];
    int64_t D = 1;
    for (int64_t k = 1; k < M; k++)
        if (S[k] != S[k - 1])
            D++;
    int iters = 0;
    if (D <= KM8_L) {
        int j = 0;
        for (int64_t k = 0; k < M; k++)
            if (k == 0 || S[k] != S[k - 1])
                C[j++] = S[k];
        for (; j < KM8_L; j++)
            C[j] = S[M - 1];
    } else {
        for (int j = 0; j < KM8_L; j++)
            C[j] = S[(2 * (int64_t)j + 1) * M / (2 * KM8_L)];
        for (int it = 0; it < max_iter; it++) {
            int64_t sum[KM8_L] = {0}, cnt[KM8_L] = {0}, Cn[KM8_L];
            for (int64_t k = 0; k < M; k++) {
                int j = nearest_centroid_l(C, KM8_L, X[k]);
                sum[j] += X[k];
                cnt[j] += 1;
            }
            int moved = 0;
            for (int j = 0; j < KM8_L; j++) {
                Cn[j] = cnt[j] ? round_mean_to_f16_units(sum[j], cnt[j]) : C[j];
                if (Cn[j] != C[j])
                    moved = 1;
            }
            iters++;
            if (!moved)
                break;
            memcpy(C, Cn, sizeof(C));
        }
    }
    for (int64_t k = 0; k < M; k++)
        idx[k] = (uint8_t)nearest_centroid_l(C, KM8_L, X[k]);
    for (int j = 0; j < KM8_L; j++)
        lut[j] = units_to_f16(C[j]);
    free(X);
    free(S);
    return iters;
}

/* W_f16: N x K fp16 bits, N % 32 == 0; codes N x K (indices); lut
   (N/32) x 256 fp16 bits; iters (may be NULL): Lloyd updates per group. */
void orc_pack_int8km(const uint16_t *W_f16, int64_t N, int64_t K, int max_iter,
                     uint8_t *codes, uint16_t *lut, int32_t *iters)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t g = 0; g < N / 32; g++) {
        int it = km8_group(W_f16 + g * 32 * K, 32 * K, max_iter, codes + g * 32 * K, lut + g * KM8_L);
        if (iters)
            iters[g] = it;
    }
}

/* ------------------------------------------------------------------------ */
/* Dequantization: every reconstructed weight is exact in fp64 (and fp32).   */
/* fmt: 0 int4, 1 fp4, 2 int8, 3 km4, 4 int4aff, 5 int8km.                  */
/* ------------------------------------------------------------------------ */

static double dequant_one(int fmt, const void *codes, const void *plane, int64_t K, int64_t n, int64_t k)
{
    if (fmt == 5) {   /* int8km: the group's table at the byte's index */
        const uint8_t *c = (const uint8_t *)codes;
        const uint16_t *lut = (const uint16_t *)plane;
        return orc_f16_to_f64(lut[(n / 32) * KM8_L + c[n * K + k]]);
    }
    if (fmt == 2) {
        const int8_t *c = (const int8_t *)codes;
        const uint16_t *s = (const uint16_t *)plane;
        return orc_f16_to_f64(s[n * (K / 32) + k / 32]) * (double)c[n * K + k];
    }
    const uint8_t *c8 = (const uint8_t *)codes;
    uint8_t byte = c8[n * (K / 2) + k / 2];
    int c = (k % 2 == 0) ? (byte & 0xf) : (byte >> 4);
    if (fmt == 0) {
        const uint16_t *s = (const uint16_t *)plane;
        return orc_f16_to_f64(s[n * (K / 32) + k / 32]) * (double)(c - 8);
    }
    if (fmt == 1) {
        const uint8_t *e = (const uint8_t *)plane;
        double mag = kE2M1[c & 7];
        double v = ldexp(mag, (int)e[n * (K / 32) + k / 32] - 127);
        return (c & 8) ? -v : v;
    }
    if (fmt == 4) {
        const uint32_t word = ((const uint32_t *)plane)[n * (K / 32) + k / 32];
        return orc_f16_to_f64((uint16_t)(word & 0xFFFF)) * (double)c + orc_f16_to_f64((uint16_t)(word >> 16));
    }
    /* km4 */
    const uint16_t *lut = (const uint16_t *)plane;
    return orc_f16_to_f64(lut[n * 16 + c]);
}

void orc_dequant(int fmt, const void *codes, const void *plane, int64_t N, int64_t K, double *W_hat)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++)
            W_hat[n * K + k] = dequant_one(fmt, codes, plane, K, n, k);
}

/* y[b][n] = sum over k ascending of dequant(W)[n][k] * x[b][k], in fp64.
   x is B x K (fp16 or fp32 inputs given as fp64). Only rows listed in `rows`
   (nrows of them) are computed when rows != NULL; y is then B x nrows. */
void orc_matvec(int fmt, const void *codes, const void *plane, int64_t N, int64_t K,
                const double *x, int B, const int64_t *rows, int64_t nrows, double *y)
{
    int64_t M = rows ? nrows : N;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; i++) {
        int64_t n = rows ? rows[i] : i;
        for (int b = 0; b < B; b++) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; k++)
                acc += dequant_one(fmt, codes, plane, K, n, k) * x[b * K + k];
            y[b * M + i] = acc;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Mixture-of-experts decode: top-k routing, per-expert SwiGLU FFN with int4 */
/* weights, weighted combine [S1 sections 1 and 4: routed-expert gather over */
/* expert slabs blocked along K; S2 section 1: only routed experts are read]. */
/* ------------------------------------------------------------------------ */

/* logits T x E (fp32). ids T x topk: the topk largest logits, largest first,
   equal logits in increasing expert order. weights T x topk: softmax over the
   selected logits, in fp64. */
void orc_moe_route(const float *logits, int T, int E, int topk, int32_t *ids, double *weights)
{
    for (int t = 0; t < T; t++) {
        const float *l = logits + (int64_t)t * E;
        char *taken = calloc(E, 1);
        for (int j = 0; j < topk; j++) {
            int best = -1;
            for (int e = 0; e < E; e++)
                if (!taken[e] && (best < 0 || l[e] > l[best]))
                    best = e;
            taken[best] = 1;
            ids[t * topk + j] = best;
        }
        free(taken);
        double mx = l[ids[t * topk]];
        double z = 0.0;
        for (int j = 0; j < topk; j++)
            z += exp((double)l[ids[t * topk + j]] - mx);
        for (int j = 0; j < topk; j++)
            weights[t * topk + j] = exp((double)l[ids[t * topk + j]] - mx) / z;
    }
}

/* Bytes of one row of codes, and of one row of the scale / table plane,
   for a K-long row in format fmt (0 int4, 1 fp4, 2 int8, 3 km4, 4 int4aff,
   5 int8km; int8km rows come in groups of 32, so 16 bytes of table per row). */
static int64_t code_row_bytes(int fmt, int64_t K) { return (fmt == 2 || fmt == 5) ? K : K / 2; }
static int64_t plane_row_bytes(int fmt, int64_t K)
{
    if (fmt == 5) return 16;          /* a 512-byte table per 32 rows */
    if (fmt == 1) return K / 32;      /* one e8m0 byte per block */
    if (fmt == 3) return 32;          /* sixteen fp16 table entries */
    if (fmt == 4) return 4 * (K / 32);   /* fp16 scale + fp16 bias per block */
    return 2 * (K / 32);              /* one fp16 scale per block */
}

/* One token's expert FFN for every selected slot, then the weighted sum.
   gu_codes/gu_plane: E experts of [2I][H] in format fmt (rows 0..I-1 gate,
   I..2I-1 up); dn_codes/dn_plane: E experts of [H][I].
   x: T x H (fp64 of fp16 inputs). h_out (may be NULL): T x topk x I, the fp16
   activations silu(g)*u rounded to fp16, as fp64. y: T x H in fp64. */
void orc_moe_ffn(int fmt, const void *gu_codes, const void *gu_plane,
                 const void *dn_codes, const void *dn_plane,
                 int E, int64_t H, int64_t I,
                 const double *x, int T, int topk, const int32_t *ids, const double *weights,
                 double *h_out, double *y)
{
    (void)E;
    double *h = malloc(sizeof(double) * I);
    double *g = malloc(sizeof(double) * 2 * I);
    double *part = malloc(sizeof(double) * H);
    const uint8_t *gu_c = gu_codes, *gu_p = gu_plane, *dn_c = dn_codes, *dn_p = dn_plane;
    for (int t = 0; t < T; t++) {
        for (int64_t n = 0; n < H; n++)
            y[t * H + n] = 0.0;
        for (int j = 0; j < topk; j++) {
            int64_t e = ids[t * topk + j];
            orc_matvec(fmt, gu_c + e * 2 * I * code_row_bytes(fmt, H), gu_p + e * 2 * I * plane_row_bytes(fmt, H),
                       2 * I, H, x + t * H, 1, NULL, 0, g);
            for (int64_t i = 0; i < I; i++) {
                double gate = g[i], up = g[I + i];
                double silu = gate / (1.0 + exp(-gate));
                h[i] = orc_f16_to_f64(orc_f64_to_f16(silu * up));
                if (h_out)
                    h_out[((int64_t)t * topk + j) * I + i] = h[i];
            }
            orc_matvec(fmt, dn_c + e * H * code_row_bytes(fmt, I), dn_p + e * H * plane_row_bytes(fmt, I),
                       H, I, h, 1, NULL, 0, part);
            for (int64_t n = 0; n < H; n++)
                y[t * H + n] += weights[t * topk + j] * part[n];
        }
    }
    free(h);
    free(g);
    free(part);
}

/* Threads the OpenMP loops above use (for reporting the CPU baseline). */
int orc_num_threads(void)
{
    return omp_get_max_threads();
}

/* Set the thread count of the OpenMP loops (the CPU baseline is timed on all
 * cores and on one). Results do not depend on it: every parallel loop writes
 * disjoint outputs and sums in a fixed order. */
void orc_set_num_threads(int n)
{
    omp_set_num_threads(n > 0 ? n : 1);
}
