/*
 * Driver for the sanitizer build of the CPU oracle (test infrastructure).
 *
 * Built with gcc -fsanitize=address,undefined -fno-sanitize-recover=all next
 * to oracle/oracle.c and run by tests/test_sanitize.py. It calls every oracle
 * entry point on small ragged inputs held in heap buffers of exactly the size
 * each call may touch, so a read or write past an end, an integer overflow or
 * a misaligned access stops the run, and it takes each rejection path once.
 * The inputs come from a fixed 64-bit LCG; no expected value is checked here
 * (the pins do that), only the return codes.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/oracle.h"

static uint64_t g_state = 0x9E3779B97F4A7C15ull;

static double uniform(void) {
    g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(g_state >> 11) * (1.0 / 9007199254740992.0);
}

static double normal(void) { /* Box-Muller */
    double a = uniform(), b = uniform();
    if (a < 1e-300) a = 1e-300;
    return sqrt(-2.0 * log(a)) * cos(6.283185307179586 * b);
}

static void* xmalloc(size_t bytes) {
    void* p = malloc(bytes ? bytes : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(3);
    }
    return p;
}

static int g_fail = 0;

static void expect(const char* what, int rc, int want_ok) {
    if ((rc == 0) != want_ok) {
        fprintf(stderr, "%s: rc %d (expected %s)\n", what, rc, want_ok ? "0" : "a rejection");
        g_fail = 1;
    }
}

static float* randn_f32(int64_t n, double sigma) {
    float* p = xmalloc((size_t)n * sizeof(float));
    for (int64_t i = 0; i < n; ++i) p[i] = (float)(sigma * normal());
    return p;
}

static uint16_t* randn_bf16(int64_t n, double sigma) {
    uint16_t* p = xmalloc((size_t)n * sizeof(uint16_t));
    for (int64_t i = 0; i < n; ++i) p[i] = oracle_f32_to_bf16((float)(sigma * normal()));
    return p;
}

static void codebook_and_codes(void) {
    double l64[16];
    float lv[16], th[15];
    oracle_nf4_levels_f64(l64);
    oracle_nf4_codebook(lv, th);
    (void)oracle_norm_ppf(0.3);
    (void)oracle_norm_cdf(-1.0);
    for (int i = 0; i < 16; ++i) (void)oracle_nf4_code(lv[i]);
    float* x = randn_f32(7, 0.5);
    uint8_t* c = xmalloc(7);
    expect("codes_batch n=7", oracle_nf4_codes_batch(x, 7, c), 1);
    expect("codes_batch n=0", oracle_nf4_codes_batch(x, 0, c), 1);
    expect("codes_batch NULL", oracle_nf4_codes_batch(NULL, 7, c), 0);
    free(x);
    free(c);
    for (int b = 0; b < 256; ++b) {
        const float v = oracle_e4m3_to_f32((uint8_t)b);
        if (isfinite(v) && v >= 0.0f) (void)oracle_f32_to_e4m3(v);
        for (int f = 0; f < 3; ++f) (void)oracle_q8_value((uint8_t)b, f);
    }
    (void)oracle_f32_to_e4m3(1e9f);
    (void)oracle_f32_to_e4m3(1e-9f);
}

/* Both levels and the dequantization for n weights in format fmt. */
static void quantize_roundtrip(int64_t n, int fmt) {
    const int64_t nb = n / 64, ng = (nb + 255) / 256;
    float* w32 = randn_f32(n, 0.02);
    uint16_t* w16 = randn_bf16(n, 0.02);
    uint8_t* codes = xmalloc((size_t)n / 2);
    uint8_t* q8 = xmalloc((size_t)nb);
    float* s2 = xmalloc((size_t)ng * sizeof(float));
    float* c1 = xmalloc((size_t)nb * sizeof(float));
    float* o32 = xmalloc((size_t)n * sizeof(float));
    uint16_t* o16 = xmalloc((size_t)n * sizeof(uint16_t));

    expect("quantize f32", oracle_quantize_nf4_f32(w32, n, codes, c1), 1);
    expect("dequant nodq", oracle_dequant_nodq(codes, c1, n, o32, o16), 1);
    expect("double_quant_fmt", oracle_double_quant_fmt(c1, nb, fmt, q8, s2), 1);
    expect("quantize_dq_fmt f32", oracle_quantize_nf4_dq_fmt(w32, 0, n, fmt, codes, q8, s2), 1);
    expect("dequant_dq_fmt", oracle_dequant_dq_fmt(codes, q8, s2, n, fmt, o32, o16), 1);
    expect("dequant_dq_fmt w32 only", oracle_dequant_dq_fmt(codes, q8, s2, n, fmt, o32, NULL), 1);
    expect("quantize_dq_fmt bf16", oracle_quantize_nf4_dq_fmt(w16, 1, n, fmt, codes, q8, s2), 1);
    expect("dequant_dq_fmt bf16 only", oracle_dequant_dq_fmt(codes, q8, s2, n, fmt, NULL, o16), 1);
    if (fmt == ORACLE_DQ_INT8) {
        expect("double_quant", oracle_double_quant(c1, nb, (int8_t*)q8, s2), 1);
        expect("quantize_dq_f32", oracle_quantize_nf4_dq_f32(w32, n, codes, (int8_t*)q8, s2), 1);
        expect("quantize_dq_bf16", oracle_quantize_nf4_dq_bf16(w16, n, codes, (int8_t*)q8, s2), 1);
        expect("dequant_dq", oracle_dequant_dq(codes, (const int8_t*)q8, s2, n, o32, o16), 1);
    }
    free(w32);
    free(w16);
    free(codes);
    free(q8);
    free(s2);
    free(c1);
    free(o32);
    free(o16);
}

static void quantize_rejections(void) {
    float w[64] = {0};
    uint8_t codes[32], q8[1];
    float s2[1], c1[1];
    w[3] = NAN;
    expect("quantize n=63", oracle_quantize_nf4_f32(w, 63, codes, c1), 0);
    expect("quantize NaN", oracle_quantize_nf4_f32(w, 64, codes, c1), 0);
    w[3] = 0.0f;
    expect("quantize zero block", oracle_quantize_nf4_f32(w, 64, codes, c1), 1);
    expect("quantize n=0", oracle_quantize_nf4_dq_fmt(w, 0, 0, 0, codes, q8, s2), 1);
    expect("quantize bad fmt", oracle_quantize_nf4_dq_fmt(w, 0, 64, 7, codes, q8, s2), 0);
    expect("dequant n=-64", oracle_dequant_dq_fmt(codes, q8, s2, -64, 0, NULL, NULL), 0);
    expect("double_quant bad fmt", oracle_double_quant_fmt(c1, 1, -1, q8, s2), 0);
}

static void int4_example(void) {
    float* w = randn_f32(200, 1.0);
    int8_t* q = xmalloc(200);
    float* sc = xmalloc(25 * sizeof(float));
    float* wh = xmalloc(200 * sizeof(float));
    expect("int4 block 8", oracle_int4_absmax(w, 200, 8, q, sc, wh), 1);
    expect("int4 no what", oracle_int4_absmax(w, 200, 8, q, sc, NULL), 1);
    expect("int4 ragged", oracle_int4_absmax(w, 200, 64, q, sc, wh), 0);
    free(w);
    free(q);
    free(sc);
    free(wh);
}

static void layer(int64_t M, int64_t N, int64_t K, int r) {
    uint16_t* x = randn_bf16(M * K, 1.0);
    uint16_t* dY = randn_bf16(M * N, 1.0);
    uint16_t* W = randn_bf16(N * K, 0.02);
    uint16_t* A = randn_bf16(K * r, 1.0 / sqrt((double)K));
    uint16_t* B = randn_bf16((int64_t)r * N, 0.01);
    double* u = xmalloc((size_t)(M * r) * sizeof(double));
    double* v = xmalloc((size_t)(M * r) * sizeof(double));
    double* y = xmalloc((size_t)(M * N) * sizeof(double));
    double* dX = xmalloc((size_t)(M * K) * sizeof(double));
    double* dA = xmalloc((size_t)(K * r) * sizeof(double));
    double* dB = xmalloc((size_t)((int64_t)r * N) * sizeof(double));
    expect("lora_down_xa", oracle_lora_down_xa(x, M, K, A, r, u), 1);
    expect("lora_down_dybt", oracle_lora_down_dybt(dY, M, N, B, r, v), 1);
    expect("linear_fwd", oracle_linear_fwd(x, M, K, W, N, A, B, r, 16.0, y, u), 1);
    expect("linear_fwd no u", oracle_linear_fwd(x, M, K, W, N, A, B, r, 16.0, y, NULL), 1);
    expect("linear_bwd", oracle_linear_bwd(x, dY, M, K, W, N, A, B, r, 16.0, dX, dA, dB), 1);
    expect("linear_bwd dX only", oracle_linear_bwd(NULL, dY, M, K, W, N, A, B, r, 16.0, dX, NULL, NULL), 1);
    expect("linear_bwd dA without x", oracle_linear_bwd(NULL, dY, M, K, W, N, A, B, r, 16.0, NULL, dA, NULL), 0);
    expect("linear_fwd r=0", oracle_linear_fwd(x, M, K, W, N, A, B, 0, 16.0, y, u), 0);
    free(x);
    free(dY);
    free(W);
    free(A);
    free(B);
    free(u);
    free(v);
    free(y);
    free(dX);
    free(dA);
    free(dB);
}

static void merge(int64_t N, int64_t K, int r, int fmt) {
    const int64_t n = N * K, nb = n / 64, ng = (nb + 255) / 256;
    float* w32 = randn_f32(n, 0.02);
    uint16_t* w16 = randn_bf16(n, 0.02);
    uint8_t* codes = xmalloc((size_t)n / 2);
    uint8_t* q8 = xmalloc((size_t)nb);
    float* s2 = xmalloc((size_t)ng * sizeof(float));
    uint16_t* A = randn_bf16(K * r, 0.05);
    uint16_t* B = randn_bf16((int64_t)r * N, 0.05);
    float* out = xmalloc((size_t)n * sizeof(float));
    expect("merge quantize", oracle_quantize_nf4_dq_fmt(w32, 0, n, fmt, codes, q8, s2), 1);
    expect("merge 4-bit base",
           oracle_merge_lora(codes, (const int8_t*)q8, s2, fmt, NULL, N, K, A, B, r, 32.0f, out), 1);
    expect("merge bf16 base", oracle_merge_lora(NULL, NULL, NULL, fmt, w16, N, K, A, B, r, 32.0f, out), 1);
    expect("merge K=65", oracle_merge_lora(NULL, NULL, NULL, fmt, w16, 1, 65, A, B, r, 1.0f, out), 0);
    free(w32);
    free(w16);
    free(codes);
    free(q8);
    free(s2);
    free(A);
    free(B);
    free(out);
}

static void adamw(int64_t n) {
    float* p = randn_f32(n, 0.02);
    float* m = randn_f32(n, 1e-3);
    float* v = randn_f32(n, 1e-3);
    for (int64_t i = 0; i < n; ++i) v[i] = v[i] * v[i];
    float* g32 = randn_f32(n, 1e-2);
    uint16_t* g16 = randn_bf16(n, 1e-2);
    uint16_t* pb = xmalloc((size_t)n * sizeof(uint16_t));
    for (int64_t t = 1; t <= 3; ++t) {
        expect("adamw bf16 grad", oracle_adamw_step(p, g16, 1, m, v, n, 1e-3, 0.9, 0.999, 1e-8, 0.01, t, pb), 1);
        expect("adamw fp32 grad", oracle_adamw_step(p, g32, 0, m, v, n, 1e-3, 0.9, 0.999, 1e-8, 0.01, t, NULL), 1);
    }
    expect("adamw t=0", oracle_adamw_step(p, g16, 1, m, v, n, 1e-3, 0.9, 0.999, 1e-8, 0.01, 0, pb), 0);
    expect("adamw beta1=1", oracle_adamw_step(p, g16, 1, m, v, n, 1e-3, 1.0, 0.999, 1e-8, 0.01, 1, pb), 0);
    expect("adamw n=0", oracle_adamw_step(NULL, NULL, 1, NULL, NULL, 0, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1, NULL), 1);
    free(p);
    free(m);
    free(v);
    free(g32);
    free(g16);
    free(pb);
}

int main(void) {
    codebook_and_codes();
    for (int fmt = 0; fmt < 3; ++fmt) {
        quantize_roundtrip(64, fmt);
        quantize_roundtrip(64 * 300, fmt); /* a full group and a ragged one */
    }
    quantize_rejections();
    int4_example();
    layer(3, 72, 128, 16);
    layer(1, 1, 64, 32);
    layer(0, 40, 64, 16);
    merge(5, 192, 16, 0);
    merge(3, 64, 48, 2);
    adamw(1003);
    adamw(1);
    if (g_fail) return 1;
    printf("oracle sanitize driver: all calls returned as expected\n");
    return 0;
}
