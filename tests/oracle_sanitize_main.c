/*
 * Driver for a sanitizer build of the CPU oracle (test infrastructure only):
 * gcc -fsanitize=address,undefined oracle/oracle.c tests/oracle_sanitize_main.c
 * runs every oracle entry point on small and edge-case shapes with output
 * buffers of exactly the documented sizes, so that any read or write past a
 * buffer, any use after free, leak or undefined arithmetic is reported and the
 * process fails. Exit status 0 means a clean run.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double orc_f16_to_f64(uint16_t h);
uint16_t orc_f64_to_f16(double v);
void orc_pack_fp4(const float *W, int64_t N, int64_t K, uint8_t *codes, uint8_t *scale);
void orc_pack_int4(const float *W, int64_t N, int64_t K, int nclips, uint8_t *codes, uint16_t *scale);
void orc_pack_int8(const float *W, int64_t N, int64_t K, int8_t *codes, uint16_t *scale);
void orc_pack_int4aff(const float *W, int64_t N, int64_t K, uint8_t *codes, uint32_t *plane);
void orc_pack_int8_rows(const float *W, int64_t V, int64_t H, int8_t *codes, uint16_t *scale);
void orc_embed_gather_int8(const int8_t *codes, const uint16_t *scale, int64_t V, int64_t H, const int32_t *ids,
                           int64_t T, uint16_t *out);
void orc_pack_km4(const uint16_t *W_f16, int64_t N, int64_t K, int max_iter, uint8_t *codes, uint16_t *lut,
                  int32_t *iters);
void orc_pack_km4o(const uint16_t *W_f16, int64_t N, int64_t K, int P, int max_iter, uint8_t *codes, uint16_t *lut,
                   uint16_t *ocol, int8_t *oval, uint16_t *oscale);
void orc_matvec_km4o(const uint8_t *codes, const uint16_t *lut, const uint16_t *ocol, const int8_t *oval,
                     const uint16_t *oscale, int64_t N, int64_t K, int P, const double *x, int B, double *y);
void orc_pack_int8km(const uint16_t *W_f16, int64_t N, int64_t K, int max_iter, uint8_t *codes, uint16_t *lut,
                     int32_t *iters);
void orc_dequant(int fmt, const void *codes, const void *plane, int64_t N, int64_t K, double *W_hat);
void orc_matvec(int fmt, const void *codes, const void *plane, int64_t N, int64_t K, const double *x, int B,
                const int64_t *rows, int64_t nrows, double *y);
void orc_moe_route(const float *logits, int T, int E, int topk, int32_t *ids, double *weights);
void orc_moe_ffn(int fmt, const void *gu_codes, const void *gu_plane, const void *dn_codes, const void *dn_plane,
                 int E, int64_t H, int64_t I, const double *x, int T, int topk, const int32_t *ids,
                 const double *weights, double *h_out, double *y);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static double uniform(void) /* xorshift64*, in [-1, 1) */
{
    state ^= state >> 12;
    state ^= state << 25;
    state ^= state >> 27;
    return (double)((state * 0x2545F4914F6CDD1Dull) >> 11) / 4503599627370496.0 - 1.0;
}

static void *must(size_t n)
{
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

/* weights: small random values, an all-zero row, a row of one repeated value,
   a row with one large outlier */
static void fill(float *W, uint16_t *W16, int64_t N, int64_t K)
{
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++) {
            double v = 0.02 * uniform();
            if (n % 5 == 1) v = 0.0;
            if (n % 5 == 2) v = 0.25;
            if (n % 5 == 3 && k == K / 2) v = 3.0;
            W16[n * K + k] = orc_f64_to_f16(v);
            W[n * K + k] = (float)orc_f16_to_f64(W16[n * K + k]);
        }
}

static size_t plane_bytes(int fmt, int64_t N, int64_t K)
{
    switch (fmt) {
    case 1: return (size_t)(N * (K / 32));
    case 3: return (size_t)(N * 32);
    case 4: return (size_t)(N * (K / 32) * 4);
    case 5: return (size_t)((N / 32) * 512);
    default: return (size_t)(N * (K / 32) * 2);
    }
}

static void dense(int64_t N, int64_t K)
{
    float *W = must(sizeof(float) * N * K);
    uint16_t *W16 = must(sizeof(uint16_t) * N * K);
    fill(W, W16, N, K);
    const int B = 3;
    double *x = must(sizeof(double) * B * K);
    for (int64_t i = 0; i < B * K; i++)
        x[i] = orc_f16_to_f64(orc_f64_to_f16(uniform()));
    for (int fmt = 0; fmt <= 5; fmt++) {
        if (fmt == 5 && N % 32 != 0)
            continue;
        size_t cb = (size_t)((fmt == 2 || fmt == 5) ? N * K : N * K / 2);
        uint8_t *codes = must(cb);
        void *plane = must(plane_bytes(fmt, N, K));
        int32_t *iters = must(sizeof(int32_t) * (N > 32 ? N : 32));
        switch (fmt) {
        case 0:
            orc_pack_int4(W, N, K, 1, codes, plane);
            orc_pack_int4(W, N, K, 7, codes, plane);
            break;
        case 1: orc_pack_fp4(W, N, K, codes, plane); break;
        case 2: orc_pack_int8(W, N, K, (int8_t *)codes, plane); break;
        case 3:
            orc_pack_km4(W16, N, K, 0, codes, plane, iters);
            orc_pack_km4(W16, N, K, 20, codes, plane, iters);
            break;
        case 4: orc_pack_int4aff(W, N, K, codes, plane); break;
        default: orc_pack_int8km(W16, N, K, 3, codes, plane, iters); break;
        }
        double *D = must(sizeof(double) * N * K);
        orc_dequant(fmt, codes, plane, N, K, D);
        double *y = must(sizeof(double) * B * N);
        orc_matvec(fmt, codes, plane, N, K, x, B, NULL, 0, y);
        free(y);
        int64_t rows[2] = {N - 1, 0};
        double *yr = must(sizeof(double) * B * 2);   /* B x nrows */
        orc_matvec(fmt, codes, plane, N, K, x, B, rows, 2, yr);
        free(yr);
        free(D);
        free(iters);
        free(plane);
        free(codes);
    }
    /* k-means rows plus int8 outliers */
    const int Ps[3] = {0, 3, K < 256 ? (int)K : 256};
    for (int i = 0; i < 3; i++) {
        int P = Ps[i];
        uint8_t *codes = must((size_t)(N * K / 2));
        uint16_t *lut = must(sizeof(uint16_t) * N * 16);
        uint16_t *ocol = must(sizeof(uint16_t) * N * P);
        int8_t *oval = must((size_t)(N * P));
        uint16_t *oscale = must(sizeof(uint16_t) * N);
        orc_pack_km4o(W16, N, K, P, 5, codes, lut, ocol, oval, oscale);
        double *y = must(sizeof(double) * B * N);
        orc_matvec_km4o(codes, lut, ocol, oval, oscale, N, K, P, x, B, y);
        free(y);
        free(oscale);
        free(oval);
        free(ocol);
        free(lut);
        free(codes);
    }
    /* int8 embedding rows and the gather, ids out of range included */
    int8_t *q = must((size_t)(N * K));
    uint16_t *s = must(sizeof(uint16_t) * N);
    orc_pack_int8_rows(W, N, K, q, s);
    int32_t ids[4] = {0, (int32_t)(N - 1), -1, (int32_t)N};
    uint16_t *out = must(sizeof(uint16_t) * 4 * K);
    orc_embed_gather_int8(q, s, N, K, ids, 4, out);
    free(out);
    free(s);
    free(q);
    free(x);
    free(W16);
    free(W);
}

static void moe(void)
{
    const int E = 4, T = 2, topk = 3;
    const int64_t H = 64, I = 32;
    float *logits = must(sizeof(float) * T * E);
    for (int i = 0; i < T * E; i++)
        logits[i] = (float)uniform();
    logits[1] = logits[2]; /* a tie */
    int32_t *ids = must(sizeof(int32_t) * T * topk);
    double *w = must(sizeof(double) * T * topk);
    orc_moe_route(logits, T, E, topk, ids, w);
    float *Wg = must(sizeof(float) * E * 2 * I * H);
    uint16_t *Wg16 = must(sizeof(uint16_t) * E * 2 * I * H);
    float *Wd = must(sizeof(float) * E * H * I);
    uint16_t *Wd16 = must(sizeof(uint16_t) * E * H * I);
    fill(Wg, Wg16, E * 2 * I, H);
    fill(Wd, Wd16, E * H, I);
    uint8_t *gc = must((size_t)(E * 2 * I * H / 2));
    uint16_t *gs = must(sizeof(uint16_t) * E * 2 * I * (H / 32));
    uint8_t *dc = must((size_t)(E * H * I / 2));
    uint16_t *ds = must(sizeof(uint16_t) * E * H * (I / 32));
    orc_pack_int4(Wg, E * 2 * I, H, 7, gc, gs);
    orc_pack_int4(Wd, E * H, I, 7, dc, ds);
    double *x = must(sizeof(double) * T * H);
    for (int64_t i = 0; i < T * H; i++)
        x[i] = orc_f16_to_f64(orc_f64_to_f16(uniform()));
    double *h = must(sizeof(double) * T * topk * I);
    double *y = must(sizeof(double) * T * H);
    orc_moe_ffn(0, gc, gs, dc, ds, E, H, I, x, T, topk, ids, w, h, y);
    orc_moe_ffn(0, gc, gs, dc, ds, E, H, I, x, T, topk, ids, w, NULL, y);
    free(y);
    free(h);
    free(x);
    free(ds);
    free(dc);
    free(gs);
    free(gc);
    free(Wd16);
    free(Wd);
    free(Wg16);
    free(Wg);
    free(w);
    free(ids);
    free(logits);
}

int main(void)
{
    const int64_t shapes[][2] = {{1, 32}, {3, 64}, {32, 96}, {37, 256}, {64, 32}};
    for (size_t i = 0; i < sizeof(shapes) / sizeof(shapes[0]); i++)
        dense(shapes[i][0], shapes[i][1]);
    moe();
    printf("oracle sanitizer run: clean\n");
    return 0;
}
