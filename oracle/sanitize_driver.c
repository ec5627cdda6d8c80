/*
 * sanitize_driver.c -- TEST INFRASTRUCTURE: runs every entry point of
 * qmv_oracle.c on small seeded inputs, every buffer allocated to its exact
 * size, so that a build with -fsanitize=address,undefined reports any
 * out-of-bounds access, use of freed memory or undefined behaviour in the
 * oracle (tests/test_oracle_sanitizers.py builds and runs it).  It checks
 * nothing numerically; the oracle's pins do that.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_block_weights(int type);
int oracle_block_bytes(int type);
float oracle_half_to_float(uint16_t h);
uint16_t oracle_float_to_half(float f);
int oracle_dequant(int type, const uint8_t *blocks, int64_t M, int64_t K, float *w_out);
int oracle_quantize(int type, const float *w, int64_t M, int64_t K, uint8_t *blocks_out);
int oracle_qmv_rows(int type, const uint8_t *blocks, int64_t M, int64_t K, const float *x,
                    int64_t nrows, const int64_t *rows, double *y, double *a);
int oracle_qmv(int type, const uint8_t *blocks, int64_t M, int64_t K, const float *x, double *y,
               double *a);
int oracle_gate_up_silu(int type, const uint8_t *blocks, int64_t I, int64_t K, const float *x,
                        double *h, double *g, double *u, double *a_g, double *a_u);
int oracle_short_conv(int in_type, const uint8_t *in_proj, int64_t D, int64_t H, const float *h,
                      const float *w_conv, const float *state_in, int out_type,
                      const uint8_t *out_proj, double *state_out, double *y, double *bx_out,
                      double *out, double *a_out, double *A);
int oracle_argmax(int type, const uint8_t *blocks, int64_t M, int64_t K, const float *x,
                  int64_t *idx, double *vmax, double *a_at);
int oracle_gemm_n(int type, const uint8_t *blocks, int64_t M, int64_t K, int32_t n,
                  const float *X, double *Y, double *A);
int oracle_moe(const float *x, int64_t H, const float *router, const float *bias, int32_t E,
               int32_t k, int gu_type, const uint8_t *gate_up, int dn_type, const uint8_t *down,
               int64_t I, double *y, int32_t *sel, double *wsel, double *logits, double *scores,
               double *g_out, double *u_out, double *h_out, double *a_y);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;

/* uniform in [-1, 1) from a 64-bit linear congruential step */
static float uniform(void)
{
    g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
    return (float)((g_state >> 40) & 0xFFFFFF) / 8388608.0f - 1.0f;
}

static void *xalloc(size_t n)
{
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static float *random_f32(size_t n, float scale)
{
    float *v = (float *)xalloc(n * sizeof(float));
    for (size_t i = 0; i < n; i++) v[i] = uniform() * scale;
    return v;
}

static uint8_t *quantized(int t, int64_t M, int64_t K)
{
    float *w = random_f32((size_t)(M * K), 0.02f);
    size_t nb = (size_t)(M * (K / oracle_block_weights(t)) * oracle_block_bytes(t));
    uint8_t *b = (uint8_t *)xalloc(nb);
    if (oracle_quantize(t, w, M, K, b) != 0) {
        fprintf(stderr, "quantize failed for type %d\n", t);
        exit(1);
    }
    free(w);
    return b;
}

#define CHECK(call)                                                  \
    do {                                                             \
        if ((call) != 0) {                                           \
            fprintf(stderr, "%s failed (type %d)\n", #call, t);      \
            return 1;                                                \
        }                                                            \
    } while (0)

static int run_format(int t)
{
    const int64_t M = 5, K = 512, n = 3, I = 2;
    uint8_t *b = quantized(t, M, K);
    float *w = (float *)xalloc((size_t)(M * K) * sizeof(float));
    CHECK(oracle_dequant(t, b, M, K, w));
    float *x = random_f32((size_t)K, 1.0f);
    double *y = (double *)xalloc((size_t)M * sizeof(double));
    double *a = (double *)xalloc((size_t)M * sizeof(double));
    CHECK(oracle_qmv(t, b, M, K, x, y, a));
    const int64_t rows[2] = {0, M - 1};
    CHECK(oracle_qmv_rows(t, b, M, K, x, 2, rows, y, a));
    int64_t idx = -1;
    double vmax = 0, a_at = 0;
    CHECK(oracle_argmax(t, b, M, K, x, &idx, &vmax, &a_at));
    float *X = random_f32((size_t)(n * K), 1.0f);
    double *Y = (double *)xalloc((size_t)(n * M) * sizeof(double));
    double *A = (double *)xalloc((size_t)(n * M) * sizeof(double));
    CHECK(oracle_gemm_n(t, b, M, K, (int32_t)n, X, Y, A));
    /* the first 2I rows as a gate+up stack */
    double *h = (double *)xalloc((size_t)I * sizeof(double));
    double *g = (double *)xalloc((size_t)I * sizeof(double));
    double *u = (double *)xalloc((size_t)I * sizeof(double));
    double *ag = (double *)xalloc((size_t)I * sizeof(double));
    double *au = (double *)xalloc((size_t)I * sizeof(double));
    CHECK(oracle_gate_up_silu(t, b, I, K, x, h, g, u, ag, au));
    free(b); free(w); free(x); free(y); free(a); free(X); free(Y); free(A);
    free(h); free(g); free(u); free(ag); free(au);

    /* gated short convolution: in_proj 3D x H in t, out_proj H x D in Q8_0 */
    {
        const int64_t D = 256, H = 256;
        uint8_t *in = quantized(t, 3 * D, H);
        uint8_t *out_proj = quantized(8, H, D);
        float *hh = random_f32((size_t)H, 1.0f);
        float *wc = random_f32((size_t)(3 * D), 0.5f);
        float *st = random_f32((size_t)(2 * D), 1.0f);
        double *st_out = (double *)xalloc((size_t)(2 * D) * sizeof(double));
        double *yy = (double *)xalloc((size_t)D * sizeof(double));
        double *bx = (double *)xalloc((size_t)D * sizeof(double));
        double *out = (double *)xalloc((size_t)H * sizeof(double));
        double *a_out = (double *)xalloc((size_t)H * sizeof(double));
        double *AA = (double *)xalloc((size_t)(3 * D) * sizeof(double));
        CHECK(oracle_short_conv(t, in, D, H, hh, wc, st, 8, out_proj, st_out, yy, bx, out, a_out,
                                AA));
        free(in); free(out_proj); free(hh); free(wc); free(st); free(st_out); free(yy); free(bx);
        free(out); free(a_out); free(AA);
    }

    /* MoE: E = 4 experts, top-2, gate/up in t, down in Q6_K */
    {
        const int32_t E = 4, k = 2;
        const int64_t H = 256, In = 256;
        uint8_t *gu = quantized(t, E * 2 * In, H);
        uint8_t *dn = quantized(14, E * H, In);
        float *xx = random_f32((size_t)H, 1.0f);
        float *R = random_f32((size_t)(E * H), 0.05f);
        float *bias = random_f32((size_t)E, 0.1f);
        double *yy = (double *)xalloc((size_t)H * sizeof(double));
        int32_t sel[2];
        double wsel[2];
        double *logits = (double *)xalloc((size_t)E * sizeof(double));
        double *scores = (double *)xalloc((size_t)E * sizeof(double));
        double *go = (double *)xalloc((size_t)(k * In) * sizeof(double));
        double *uo = (double *)xalloc((size_t)(k * In) * sizeof(double));
        double *ho = (double *)xalloc((size_t)(k * In) * sizeof(double));
        double *ay = (double *)xalloc((size_t)H * sizeof(double));
        CHECK(oracle_moe(xx, H, R, bias, E, k, t, gu, 14, dn, In, yy, sel, wsel, logits, scores, go,
                         uo, ho, ay));
        free(gu); free(dn); free(xx); free(R); free(bias); free(yy); free(logits); free(scores);
        free(go); free(uo); free(ho); free(ay);
    }
    return 0;
}

int main(void)
{
    static const int types[] = {2, 3, 6, 7, 8, 9, 10, 11, 12, 13, 14};
    for (unsigned h = 0; h < 65536; h++) {
        const float f = oracle_half_to_float((uint16_t)h);
        (void)oracle_float_to_half(f);
    }
    for (size_t i = 0; i < sizeof(types) / sizeof(types[0]); i++)
        if (run_format(types[i]) != 0) return 1;
    /* argument checks: bad shapes and null pointers return -1 */
    float one = 1.0f;
    double d = 0;
    if (oracle_qmv(12, NULL, 1, 256, &one, &d, NULL) != -1) return 1;
    if (oracle_qmv(12, (const uint8_t *)&one, 1, 100, &one, &d, NULL) != -1) return 1;
    printf("sanitized oracle run: ok\n");
    return 0;
}
