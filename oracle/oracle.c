/*
 * CPU oracle for the QLoRA frozen-base path. TEST INFRASTRUCTURE ONLY: only
 * the test suite, the smoke check and the benchmark's CPU-baseline leg use it;
 * the GPU library never links or calls it. See oracle.h for the format.
 *
 * Plain single-threaded C11; build with -O2 -ffp-contract=off, no fast-math,
 * so that every float operation below is one IEEE binary32 operation rounded
 * to nearest-even, exactly as written.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* bf16 helpers                                                             */
/* ------------------------------------------------------------------------ */

float oracle_bf16_to_f32(uint16_t b) {
    /* bf16 is the top half of an fp32 bit pattern: widening is exact. */
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

uint16_t oracle_f32_to_bf16(float f) {
    /* Round-to-nearest-even on the fp32 bit pattern (finite inputs; an
     * overflow past the largest bf16 correctly becomes infinity). */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------------ */
/* NF4 codebook                                                             */
/* [P1] bullets "NF4 instead of a uniform grid": 16 levels at quantiles of a */
/* normal distribution, dense near zero; [P2] s1 "Key Innovation: NF4":     */
/* levels at the quantiles of a normal distribution. The pages print no     */
/* values; the reading used here (equal probability steps on each side,     */
/* 8 positive and 7 negative levels, an exact zero, levels normalised so    */
/* the outermost ones are exactly -1 and +1) is recorded with the build's   */
/* other readings.                                                          */
/* ------------------------------------------------------------------------ */

double oracle_norm_cdf(double t) { return 0.5 * erfc(-t / sqrt(2.0)); }

double oracle_norm_ppf(double p) {
    /* Bisection on the monotone CDF until the bracket cannot shrink. */
    double lo = -40.0, hi = 40.0;
    for (int it = 0; it < 2000; ++it) {
        double mid = 0.5 * (lo + hi);
        if (mid == lo || mid == hi) break;
        if (oracle_norm_cdf(mid) < p)
            lo = mid;
        else
            hi = mid;
    }
    return 0.5 * (lo + hi);
}

void oracle_nf4_levels_f64(double levels[16]) {
    /* The outermost level sits at the centre of the outermost
     * equal-probability bin: 1 - 1/32 for the 16-bin (8-level) side and
     * 1 - 1/30 for the 15-bin (7-level) side; one shared delta (their mean)
     * makes both ends land exactly on +-1 after normalisation. */
    const double delta = 1.0 - (1.0 / 32.0 + 1.0 / 30.0) / 2.0;
    const double zstar = oracle_norm_ppf(delta);
    for (int i = 0; i < 7; ++i) {
        double p = 0.5 + (double)(7 - i) * (delta - 0.5) / 7.0;
        levels[i] = -oracle_norm_ppf(p) / zstar;
    }
    levels[7] = 0.0;
    for (int j = 0; j < 8; ++j) {
        double p = 0.5 + (double)(j + 1) * (delta - 0.5) / 8.0;
        levels[8 + j] = oracle_norm_ppf(p) / zstar;
    }
    levels[0] = -1.0;
    levels[15] = 1.0;
}

void oracle_nf4_codebook(float levels[16], float thresholds[15]) {
    double l64[16];
    oracle_nf4_levels_f64(l64);
    for (int i = 0; i < 16; ++i) levels[i] = (float)l64[i]; /* RN to fp32 */
    for (int i = 0; i < 15; ++i) {
        /* Midpoint of two fp32 levels: the double sum is exact, the halving
         * is exact. Round it DOWN to fp32, so that for any fp32 x,
         * "x > T" holds exactly when x lies strictly above the true
         * midpoint: ties then go to the lower code. */
        double m = ((double)levels[i] + (double)levels[i + 1]) / 2.0;
        float t = (float)m;
        if ((double)t > m) t = nextafterf(t, -INFINITY);
        thresholds[i] = t;
    }
}

int oracle_nf4_code(float x) {
    float lv[16], th[15];
    oracle_nf4_codebook(lv, th);
    int c = 0;
    for (int i = 0; i < 15; ++i) c += (x > th[i]);
    return c;
}

/* ------------------------------------------------------------------------ */
/* Quantization                                                             */
/* [P1] "Quantization here is just controlled rounding": take a block, find */
/* its absmax, divide it into a grid, store each weight as the index of its */
/* nearest grid point plus one scale per block. [P1] bullets: blocks of 64. */
/* ------------------------------------------------------------------------ */

/* First level for nb blocks with a given threshold table. */
static int quantize_blocks(const float* w, int64_t nb, uint8_t* codes, float* c1,
                           const float th[15]) {
    for (int64_t b = 0; b < nb; ++b) {
        const float* wb = w + b * ORACLE_BLOCK;
        float amax = 0.0f;
        for (int i = 0; i < ORACLE_BLOCK; ++i) {
            if (!isfinite(wb[i])) return 2; /* finite input is a precondition */
            float a = fabsf(wb[i]);
            if (a > amax) amax = a;
        }
        c1[b] = amax;
        for (int i = 0; i < ORACLE_BLOCK; i += 2) {
            int code[2];
            for (int h = 0; h < 2; ++h) {
                if (amax == 0.0f) {
                    code[h] = 7; /* an all-zero block maps to the exact-zero level */
                } else {
                    float x = wb[i + h] / amax; /* one correctly rounded fp32 division */
                    int c = 0;
                    for (int t = 0; t < 15; ++t) c += (x > th[t]);
                    code[h] = c;
                }
            }
            codes[(b * ORACLE_BLOCK + i) / 2] = (uint8_t)(code[0] | (code[1] << 4));
        }
    }
    return 0;
}

int oracle_quantize_nf4_f32(const float* w, int64_t n, uint8_t* codes, float* c1) {
    if (!w || !codes || !c1 || n < 0 || n % ORACLE_BLOCK) return 1;
    float lv[16], th[15];
    oracle_nf4_codebook(lv, th);
    return quantize_blocks(w, n / ORACLE_BLOCK, codes, c1, th);
}

int oracle_nf4_codes_batch(const float* x, int64_t n, uint8_t* out) {
    if (!x || !out || n < 0) return 1;
    float lv[16], th[15];
    oracle_nf4_codebook(lv, th);
    for (int64_t e = 0; e < n; ++e) {
        int c = 0;
        for (int t = 0; t < 15; ++t) c += (x[e] > th[t]);
        out[e] = (uint8_t)c;
    }
    return 0;
}

/* OCP FP8 E4M3 (E4M3FN): sign, 4 exponent bits with bias 7, 3 mantissa bits;
 * no infinities; S.1111.111 is NaN; largest finite value 448; exponent field
 * 0 holds the subnormals m * 2^-9. */
float oracle_e4m3_to_f32(uint8_t b) {
    const int sgn = b >> 7, e = (b >> 3) & 15, m = b & 7;
    if (e == 15 && m == 7) return NAN;
    const double v = e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return (float)(sgn ? -v : v);
}

/* Nearest E4M3 value to a non-negative x, ties to the even code (the even
 * mantissa); x >= 448 (or +inf) gives 448. Non-negative codes 0x00..0x7E
 * increase with their value, so the code is found by walking up to the
 * interval [v_k, v_k+1) that holds x and comparing x with its midpoint,
 * which is exact in double. */
uint8_t oracle_f32_to_e4m3(float x) {
    if (!(x < 448.0f)) return 0x7E;
    int k = 0;
    while (k < 0x7E && (double)x >= (double)oracle_e4m3_to_f32((uint8_t)(k + 1))) ++k;
    if (k == 0x7E) return 0x7E;
    const double lo = oracle_e4m3_to_f32((uint8_t)k), hi = oracle_e4m3_to_f32((uint8_t)(k + 1));
    const double mid = (lo + hi) / 2.0;
    if ((double)x > mid) return (uint8_t)(k + 1);
    if ((double)x < mid) return (uint8_t)k;
    return (uint8_t)((k & 1) ? k + 1 : k);
}

/* The value of a stored 8-bit absmax code in each second-level format. */
float oracle_q8_value(uint8_t b, int fmt) {
    if (fmt == ORACLE_DQ_INT8) return (float)(int8_t)b;
    if (fmt == ORACLE_DQ_UINT8) return (float)b;
    return oracle_e4m3_to_f32(b);
}

/* [P1] bullets "double quantization quantizes the scales themselves to
 * 8-bit"; [P2] s1 "Double Quantization" (the scales are quantized to FP8);
 * [P5] "Double Quantization". Over groups of 256 blocks, with c2 the largest
 * block constant of the group and every operation in binary32:
 *   ORACLE_DQ_INT8:  the pages' one quantizer formula ([P1] controlled-
 *                    rounding equation) on an 8-bit symmetric grid:
 *                    s2 = c2/127, q8 = round(c1/s2), ties to the lower, 0..127;
 *   ORACLE_DQ_UINT8: the same on the unsigned byte: s2 = c2/255, 0..255;
 *   ORACLE_DQ_E4M3:  s2 = c2/448, q8 = the nearest E4M3 value of c1/s2
 *                    (ties to even, saturating at 448).
 * A zero constant always gets the code 0. */
int oracle_double_quant_fmt(const float* c1, int64_t nblocks, int fmt, uint8_t* q8, float* s2) {
    if (!c1 || !q8 || !s2 || nblocks < 0) return 1;
    if (fmt != ORACLE_DQ_INT8 && fmt != ORACLE_DQ_UINT8 && fmt != ORACLE_DQ_E4M3) return 1;
    const float top = fmt == ORACLE_DQ_INT8 ? 127.0f : fmt == ORACLE_DQ_UINT8 ? 255.0f : 448.0f;
    int64_t ng = (nblocks + ORACLE_GROUP - 1) / ORACLE_GROUP;
    for (int64_t g = 0; g < ng; ++g) {
        int64_t b0 = g * ORACLE_GROUP;
        int64_t b1 = b0 + ORACLE_GROUP;
        if (b1 > nblocks) b1 = nblocks;
        float c2 = 0.0f;
        for (int64_t b = b0; b < b1; ++b)
            if (c1[b] > c2) c2 = c1[b];
        float scale = c2 / top;
        s2[g] = scale;
        for (int64_t b = b0; b < b1; ++b) {
            if (c1[b] == 0.0f) {
                q8[b] = 0;
                continue;
            }
            float v = c1[b] / scale; /* +inf if scale underflowed to 0 */
            if (fmt == ORACLE_DQ_E4M3) {
                q8[b] = oracle_f32_to_e4m3(v);
            } else {
                double r = ceil((double)v - 0.5); /* nearest, ties to the lower */
                if (r < 0.0) r = 0.0;
                if (r > (double)top) r = (double)top;
                q8[b] = (uint8_t)(int)r;
            }
        }
    }
    return 0;
}

int oracle_double_quant(const float* c1, int64_t nblocks, int8_t* q8, float* s2) {
    return oracle_double_quant_fmt(c1, nblocks, ORACLE_DQ_INT8, (uint8_t*)q8, s2);
}

/* Both levels for fp32 (is_bf16 == 0) or bf16 input (raw 16-bit patterns,
 * widened exactly) in the second-level format fmt. */
int oracle_quantize_nf4_dq_fmt(const void* w, int is_bf16, int64_t n, int fmt, uint8_t* codes,
                               uint8_t* q8, float* s2) {
    if (!w || !codes || !q8 || !s2 || n < 0 || n % ORACLE_BLOCK) return 1;
    float lv[16], th[15];
    oracle_nf4_codebook(lv, th);
    float buf[ORACLE_BLOCK];
    int64_t nb = n / ORACLE_BLOCK;
    float* c1 = (float*)malloc((size_t)(nb > 0 ? nb : 1) * sizeof(float));
    if (!c1) return 3;
    for (int64_t b = 0; b < nb; ++b) {
        for (int i = 0; i < ORACLE_BLOCK; ++i)
            buf[i] = is_bf16 ? oracle_bf16_to_f32(((const uint16_t*)w)[b * ORACLE_BLOCK + i])
                             : ((const float*)w)[b * ORACLE_BLOCK + i];
        int rc = quantize_blocks(buf, 1, codes + b * (ORACLE_BLOCK / 2), c1 + b, th);
        if (rc) {
            free(c1);
            return rc;
        }
    }
    int rc = oracle_double_quant_fmt(c1, nb, fmt, q8, s2);
    free(c1);
    return rc;
}

int oracle_quantize_nf4_dq_f32(const float* w, int64_t n, uint8_t* codes, int8_t* q8, float* s2) {
    return oracle_quantize_nf4_dq_fmt(w, 0, n, ORACLE_DQ_INT8, codes, (uint8_t*)q8, s2);
}

int oracle_quantize_nf4_dq_bf16(const uint16_t* w, int64_t n, uint8_t* codes, int8_t* q8,
                                float* s2) {
    return oracle_quantize_nf4_dq_fmt(w, 1, n, ORACLE_DQ_INT8, codes, (uint8_t*)q8, s2);
}

/* ------------------------------------------------------------------------ */
/* Dequantization                                                           */
/* [P1] controlled-rounding equation: w_hat = q * scale; [P1] bullets       */
/* "Compute never happens in 4-bit": weights are dequantized to bf16 just   */
/* in time; [P2] s3 "The Backward Pass Through Quantization" step 1.        */
/* ------------------------------------------------------------------------ */

int oracle_dequant_dq_fmt(const uint8_t* codes, const uint8_t* q8, const float* s2, int64_t n,
                          int fmt, float* w32, uint16_t* wbf16) {
    if (!codes || !q8 || !s2 || n < 0 || n % ORACLE_BLOCK) return 1;
    if (fmt != ORACLE_DQ_INT8 && fmt != ORACLE_DQ_UINT8 && fmt != ORACLE_DQ_E4M3) return 1;
    float lv[16], th[15];
    oracle_nf4_codebook(lv, th);
    for (int64_t e = 0; e < n; ++e) {
        int64_t b = e / ORACLE_BLOCK;
        float c1hat = oracle_q8_value(q8[b], fmt) * s2[b / ORACLE_GROUP];
        int code = (e & 1) ? (codes[e / 2] >> 4) : (codes[e / 2] & 15);
        float v = lv[code] * c1hat;
        if (w32) w32[e] = v;
        if (wbf16) wbf16[e] = oracle_f32_to_bf16(v);
    }
    return 0;
}

int oracle_dequant_dq(const uint8_t* codes, const int8_t* q8, const float* s2, int64_t n,
                      float* w32, uint16_t* wbf16) {
    return oracle_dequant_dq_fmt(codes, (const uint8_t*)q8, s2, n, ORACLE_DQ_INT8, w32, wbf16);
}

int oracle_dequant_nodq(const uint8_t* codes, const float* c1, int64_t n, float* w32,
                        uint16_t* wbf16) {
    if (!codes || !c1 || n < 0 || n % ORACLE_BLOCK) return 1;
    float lv[16], th[15];
    oracle_nf4_codebook(lv, th);
    for (int64_t e = 0; e < n; ++e) {
        int code = (e & 1) ? (codes[e / 2] >> 4) : (codes[e / 2] & 15);
        float v = lv[code] * c1[e / ORACLE_BLOCK];
        if (w32) w32[e] = v;
        if (wbf16) wbf16[e] = oracle_f32_to_bf16(v);
    }
    return 0;
}

/* [P1] controlled-rounding equation and its worked 8-weight example:
 * scale = absmax/7, q = round(w/scale) clamped to [-8, 7], w_hat = q*scale,
 * round() being round-half-to-even. An all-zero block gives q = 0. */
int oracle_int4_absmax(const float* w, int64_t n, int64_t block, int8_t* q, float* scale,
                       float* what) {
    if (!w || !q || !scale || block <= 0 || n < 0 || n % block) return 1;
    for (int64_t b = 0; b < n / block; ++b) {
        float amax = 0.0f;
        for (int64_t i = 0; i < block; ++i) {
            float a = fabsf(w[b * block + i]);
            if (a > amax) amax = a;
        }
        float sc = amax / 7.0f;
        scale[b] = sc;
        for (int64_t i = 0; i < block; ++i) {
            int64_t e = b * block + i;
            float qq = 0.0f;
            if (sc != 0.0f) {
                qq = rintf(w[e] / sc); /* default rounding mode: half to even */
                if (qq < -8.0f) qq = -8.0f;
                if (qq > 7.0f) qq = 7.0f;
            }
            q[e] = (int8_t)qq;
            if (what) what[e] = qq * sc;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* QLoRA linear layer, double precision                                     */
/* [P1] forward equation: h = W_hat x + (alpha/r) B (A x), written here in  */
/* row-major form y = x W_hat^T + s (x A) B with A [K,r], B [r,N].          */
/* [P2] s3 "The Backward Pass Through Quantization": gradients flow through */
/* the dequantized frozen base; only the adapters receive gradients.        */
/* ------------------------------------------------------------------------ */

static double bfd(uint16_t b) { return (double)oracle_bf16_to_f32(b); }

int oracle_lora_down_xa(const uint16_t* x, int64_t M, int64_t K, const uint16_t* A, int r,
                        double* u) {
    if (!x || !A || !u || M < 0 || K < 0 || r <= 0) return 1;
    for (int64_t m = 0; m < M; ++m)
        for (int j = 0; j < r; ++j) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += bfd(x[m * K + k]) * bfd(A[k * r + j]);
            u[m * r + j] = acc;
        }
    return 0;
}

int oracle_lora_down_dybt(const uint16_t* dY, int64_t M, int64_t N, const uint16_t* B, int r,
                          double* v) {
    if (!dY || !B || !v || M < 0 || N < 0 || r <= 0) return 1;
    for (int64_t m = 0; m < M; ++m)
        for (int j = 0; j < r; ++j) {
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) acc += bfd(dY[m * N + n]) * bfd(B[(int64_t)j * N + n]);
            v[m * r + j] = acc;
        }
    return 0;
}

int oracle_linear_fwd(const uint16_t* x, int64_t M, int64_t K, const uint16_t* What, int64_t N,
                      const uint16_t* A, const uint16_t* B, int r, double alpha, double* y,
                      double* u) {
    if (!x || !What || !A || !B || M < 0 || K < 0 || N < 0 || r <= 0) return 1;
    const double s = alpha / (double)r;
    double* ub = (double*)malloc((size_t)(M * r > 0 ? M * r : 1) * sizeof(double));
    double* xr = (double*)malloc((size_t)(M * K > 0 ? M * K : 1) * sizeof(double));
    double* wr = (double*)malloc((size_t)(K > 0 ? K : 1) * sizeof(double));
    if (!ub || !xr || !wr) {
        free(ub);
        free(xr);
        free(wr);
        return 3;
    }
    oracle_lora_down_xa(x, M, K, A, r, ub);
    if (u) memcpy(u, ub, (size_t)(M * r) * sizeof(double));
    if (y) {
        for (int64_t i = 0; i < M * K; ++i) xr[i] = bfd(x[i]);
        /* base term: y[m,n] = sum_k x[m,k] * What[n,k], k ascending */
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t k = 0; k < K; ++k) wr[k] = bfd(What[n * K + k]);
            for (int64_t m = 0; m < M; ++m) {
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k) acc += xr[m * K + k] * wr[k];
                y[m * N + n] = acc;
            }
        }
        /* adapter term: + s * sum_j u[m,j] * B[j,n] */
        for (int64_t m = 0; m < M; ++m)
            for (int64_t n = 0; n < N; ++n) {
                double acc = 0.0;
                for (int j = 0; j < r; ++j) acc += ub[m * r + j] * bfd(B[(int64_t)j * N + n]);
                y[m * N + n] += s * acc;
            }
    }
    free(ub);
    free(xr);
    free(wr);
    return 0;
}

int oracle_linear_bwd(const uint16_t* x, const uint16_t* dY, int64_t M, int64_t K,
                      const uint16_t* What, int64_t N, const uint16_t* A, const uint16_t* B,
                      int r, double alpha, double* dX, double* dA, double* dB) {
    if (!dY || !What || !A || !B || M < 0 || K < 0 || N < 0 || r <= 0) return 1;
    if ((dA || dB) && !x) return 1;
    const double s = alpha / (double)r;
    double* v = (double*)malloc((size_t)(M * r > 0 ? M * r : 1) * sizeof(double));
    double* wr = (double*)malloc((size_t)(K > 0 ? K : 1) * sizeof(double));
    if (!v || !wr) {
        free(v);
        free(wr);
        return 3;
    }
    oracle_lora_down_dybt(dY, M, N, B, r, v); /* v = dY B^T */
    if (dX) {
        /* base term: dX[m,k] = sum_n dY[m,n] * What[n,k], n ascending */
        for (int64_t i = 0; i < M * K; ++i) dX[i] = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t k = 0; k < K; ++k) wr[k] = bfd(What[n * K + k]);
            for (int64_t m = 0; m < M; ++m) {
                double d = bfd(dY[m * N + n]);
                double* row = dX + m * K;
                for (int64_t k = 0; k < K; ++k) row[k] += d * wr[k];
            }
        }
        /* adapter term: + s * sum_j v[m,j] * A[k,j] */
        for (int64_t m = 0; m < M; ++m)
            for (int64_t k = 0; k < K; ++k) {
                double acc = 0.0;
                for (int j = 0; j < r; ++j) acc += v[m * r + j] * bfd(A[k * r + j]);
                dX[m * K + k] += s * acc;
            }
    }
    if (dA) {
        /* dA[k,j] = s * sum_m x[m,k] * v[m,j] */
        for (int64_t i = 0; i < K * r; ++i) dA[i] = 0.0;
        for (int64_t m = 0; m < M; ++m)
            for (int64_t k = 0; k < K; ++k) {
                double xv = bfd(x[m * K + k]);
                for (int j = 0; j < r; ++j) dA[k * r + j] += xv * v[m * r + j];
            }
        for (int64_t i = 0; i < K * r; ++i) dA[i] *= s;
    }
    if (dB) {
        /* dB[j,n] = s * sum_m u[m,j] * dY[m,n], u = x A */
        double* u = (double*)malloc((size_t)(M * r > 0 ? M * r : 1) * sizeof(double));
        if (!u) {
            free(v);
            free(wr);
            return 3;
        }
        oracle_lora_down_xa(x, M, K, A, r, u);
        for (int64_t i = 0; i < (int64_t)r * N; ++i) dB[i] = 0.0;
        for (int64_t m = 0; m < M; ++m)
            for (int j = 0; j < r; ++j) {
                double uv = u[m * r + j];
                double* row = dB + (int64_t)j * N;
                for (int64_t n = 0; n < N; ++n) row[n] += uv * bfd(dY[m * N + n]);
            }
        for (int64_t i = 0; i < (int64_t)r * N; ++i) dB[i] *= s;
        free(u);
    }
    free(v);
    free(wr);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Merge of the adapter into the base                                       */
/* [P1] bullets ("Merging the adapter is no longer clean": folding BA into  */
/* a 4-bit W forces a re-quantization); [P4] "What it costs", "Merge        */
/* friction" (the clean path merges into the 16-bit weights and quantizes   */
/* afterwards).                                                             */
/*   out[n][k] = base[n][k] + s * d[n][k],  d[n][k] = sum_j A[k][j] B[j][n] */
/* evaluated in binary32 as written: d starts at +0 and takes the terms     */
/* j = 0, 1, ... r-1 in order; each product A*B rounds to binary32 (exact   */
/* unless it falls below the normal range) and each addition rounds, then  */
/* t = s*d rounds, then base + t rounds. No operation is fused. s = alpha/r */
/* in binary32. base is the dequantized NF4 weight (w_hat as bf16,          */
/* widened) when wbf16 is NULL, else the bf16 weight.                       */
/* ------------------------------------------------------------------------ */
int oracle_merge_lora(const uint8_t* codes, const int8_t* q8, const float* s2, int fmt,
                      const uint16_t* wbf16, int64_t N, int64_t K, const uint16_t* A,
                      const uint16_t* B, int r, float alpha, float* out) {
    if (N < 1 || K < 1 || K % ORACLE_BLOCK || r < 1 || !A || !B || !out) return 1;
    if (!wbf16 && (!codes || !q8 || !s2)) return 1;
    const float s = alpha / (float)r;
    uint16_t* base = NULL;
    if (!wbf16) {
        base = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(N * K));
        if (!base) return 2;
        if (oracle_dequant_dq_fmt(codes, (const uint8_t*)q8, s2, N * K, fmt, NULL, base)) {
            free(base);
            return 1;
        }
    }
    const uint16_t* w = wbf16 ? wbf16 : base;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            float d = 0.0f;
            for (int j = 0; j < r; ++j) {
                const float p = oracle_bf16_to_f32(A[k * r + j]) * oracle_bf16_to_f32(B[(int64_t)j * N + n]);
                d = d + p;
            }
            const float t = s * d;
            out[n * K + k] = oracle_bf16_to_f32(w[n * K + k]) + t;
        }
    }
    free(base);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* AdamW step on the adapter parameters                                     */
/* [P2] precision table (the Adam state of an adapter parameter is fp32,    */
/* 12 bytes); [P4] "The memory term LoRA does not remove" (what a trained   */
/* parameter carries: optimizer moments and a master copy). The 12 bytes   */
/* are read as the fp32 master value p and the two fp32 moments m and v;    */
/* the bf16 adapter the layer reads is the master value rounded to bf16.    */
/* [P1] paragraph on paged optimizers, [P3] "How it works": the state may   */
/* sit in host memory; that changes where it lives, not what is computed.  */
/*                                                                          */
/* Decoupled weight decay (AdamW). Step t >= 1. The hyper-parameters are    */
/* given in double; every scalar below is computed in double from them and  */
/* rounded once to binary32:                                                */
/*   b1 = beta1, b2 = beta2, e = eps, decay = 1 - lr*wd, c1 = 1 - beta1,    */
/*   c2 = 1 - beta2, step_size = lr / (1 - beta1^t),                        */
/*   bc2_sqrt = sqrt(1 - beta2^t).                                          */
/* Per element in binary32, every operation rounded, no fused operations:   */
/*   p <- p*decay                                                           */
/*   m <- b1*m + c1*g                                                       */
/*   v <- b2*v + c2*(g*g)                                                   */
/*   p <- p - step_size * (m / (sqrt(v)/bc2_sqrt + e))                      */
/* g is the gradient (bf16 widened, or fp32).                               */
/* ------------------------------------------------------------------------ */
static void adamw_scalars(double lr, double beta1, double beta2, double eps, double wd,
                          int64_t t, float sc[8]) {
    const double b1t = pow(beta1, (double)t), b2t = pow(beta2, (double)t);
    sc[0] = (float)beta1;
    sc[1] = (float)beta2;
    sc[2] = (float)eps;
    sc[3] = (float)(1.0 - lr * wd);
    sc[4] = (float)(1.0 - beta1);
    sc[5] = (float)(1.0 - beta2);
    sc[6] = (float)(lr / (1.0 - b1t));
    sc[7] = (float)sqrt(1.0 - b2t);
}

int oracle_adamw_step(float* p, const void* g, int g_is_bf16, float* m, float* v, int64_t n,
                      double lr, double beta1, double beta2, double eps, double wd, int64_t t,
                      uint16_t* p_bf16) {
    if (n < 0 || t < 1 || (n > 0 && (!p || !g || !m || !v))) return 1;
    if (!(beta1 >= 0.0 && beta1 < 1.0 && beta2 >= 0.0 && beta2 < 1.0)) return 1;
    float sc[8];
    adamw_scalars(lr, beta1, beta2, eps, wd, t, sc);
    const float b1 = sc[0], b2 = sc[1], e = sc[2], decay = sc[3], c1 = sc[4], c2 = sc[5];
    const float step_size = sc[6], bc2_sqrt = sc[7];
    for (int64_t i = 0; i < n; ++i) {
        const float gi = g_is_bf16 ? oracle_bf16_to_f32(((const uint16_t*)g)[i])
                                   : ((const float*)g)[i];
        const float pd = p[i] * decay;
        const float mb = b1 * m[i];
        const float mg = c1 * gi;
        const float mi = mb + mg;
        const float vb = b2 * v[i];
        const float gg = gi * gi;
        const float vg = c2 * gg;
        const float vi = vb + vg;
        const float sq = sqrtf(vi);
        const float dn = sq / bc2_sqrt;
        const float de = dn + e;
        const float q = mi / de;
        const float up = step_size * q;
        p[i] = pd - up;
        m[i] = mi;
        v[i] = vi;
        if (p_bf16) p_bf16[i] = oracle_f32_to_bf16(p[i]);
    }
    return 0;
}
