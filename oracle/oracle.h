/*
 * CPU oracle for the QLoRA frozen-base path: blockwise NF4 quantization with
 * double quantization of the block constants, dequantization to bf16, the
 * QLoRA linear layer (forward and backward) in double precision, the merge of
 * the adapter into the base and the AdamW step on the adapter (binary32).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or call
 * this code: only the test suite, the smoke check and the benchmark's CPU
 * baseline leg use it. It shares no code, header, table or constant generator
 * with the GPU library.
 *
 * Plain single-threaded C11, no SIMD intrinsics, no BLAS, no fast-math, no FP
 * contraction. Every function names the passage of the pages it follows:
 *   [P1] "QLoRA", learning-llms.pages.dev/topics/qlora
 *   [P2] "QLoRA", infra.bea.ai/guide/training/fine-tuning-adapters/qlora
 *   [P3] "QLoRA", scalata.ai/resources/model-training/qlora
 *   [P4] "What does QLoRA change about a LoRA run...", katajob.com
 *   [P5] "QLoRA viz", engineersofai.com/playground/qlora-viz
 *
 * Storage format (shared by contract with the GPU library, not by code):
 *   W is [N,K] row-major, flat index e = n*K + k.
 *   block b = e / 64 (64 consecutive weights), group g = b / 256.
 *   codes[e/2]: even e in the low nibble, odd e in the high nibble.
 *   q8[b]: 8-bit code of the block's absmax (0..127).
 *   s2[g]: fp32 second-level scale of group g.
 *
 * All functions return 0 on success, nonzero on a rejected input.
 */
#ifndef QLORA_ORACLE_H
#define QLORA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_BLOCK 64
#define ORACLE_GROUP 256

/* Second-level (double quantization) formats of the 8-bit absmax code. */
#define ORACLE_DQ_INT8 0  /* s2 = c2/127, q8 in 0..127 (the default) */
#define ORACLE_DQ_UINT8 1 /* s2 = c2/255, q8 in 0..255 */
#define ORACLE_DQ_E4M3 2  /* s2 = c2/448, q8 an FP8 E4M3 value */

/* Standard normal CDF and its inverse (bisection on the CDF). */
double oracle_norm_cdf(double t);
double oracle_norm_ppf(double p);

/* NF4 levels in double (exact definition) and rounded to fp32, plus the 15
 * fp32 decision thresholds T[i] = round-down((L[i] + L[i+1]) / 2). */
void oracle_nf4_levels_f64(double levels[16]);
void oracle_nf4_codebook(float levels[16], float thresholds[15]);

/* Nearest-level code of a normalised value x by the threshold rule. */
int oracle_nf4_code(float x);
int oracle_nf4_codes_batch(const float* x, int64_t n, uint8_t* out);

/* First level: per-64 absmax and packed NF4 codes. n % 64 == 0. */
int oracle_quantize_nf4_f32(const float* w, int64_t n, uint8_t* codes, float* c1);

/* FP8 E4M3 (OCP E4M3FN) decoding, and encoding of x >= 0 to the nearest
 * value with ties to even, saturating at 448. */
float oracle_e4m3_to_f32(uint8_t b);
uint8_t oracle_f32_to_e4m3(float x);

/* The value of a stored 8-bit absmax code in format fmt. */
float oracle_q8_value(uint8_t b, int fmt);

/* Second level: q8/s2 from the fp32 block constants (default format, and
 * any format). */
int oracle_double_quant(const float* c1, int64_t nblocks, int8_t* q8, float* s2);
int oracle_double_quant_fmt(const float* c1, int64_t nblocks, int fmt, uint8_t* q8, float* s2);

/* Both levels, fp32 input and bf16 input (bf16 given as raw 16-bit patterns). */
int oracle_quantize_nf4_dq_f32(const float* w, int64_t n, uint8_t* codes, int8_t* q8, float* s2);
int oracle_quantize_nf4_dq_bf16(const uint16_t* w, int64_t n, uint8_t* codes, int8_t* q8, float* s2);
int oracle_quantize_nf4_dq_fmt(const void* w, int is_bf16, int64_t n, int fmt, uint8_t* codes,
                               uint8_t* q8, float* s2);

/* Dequantization with double-quantized constants: writes fp32 product and its
 * bf16 rounding (either output may be NULL). */
int oracle_dequant_dq(const uint8_t* codes, const int8_t* q8, const float* s2, int64_t n,
                      float* w32, uint16_t* wbf16);
int oracle_dequant_dq_fmt(const uint8_t* codes, const uint8_t* q8, const float* s2, int64_t n,
                          int fmt, float* w32, uint16_t* wbf16);

/* Dequantization with the exact fp32 block constants (no second level). */
int oracle_dequant_nodq(const uint8_t* codes, const float* c1, int64_t n, float* w32,
                        uint16_t* wbf16);

/* The symmetric absmax int4 quantizer of the pages' worked example, per block
 * of `block` elements: scale = absmax/7, q = clamp(round(w/scale), -8, 7). */
int oracle_int4_absmax(const float* w, int64_t n, int64_t block, int8_t* q, float* scale,
                       float* what);

/* bf16 <-> fp32 helpers (exact widening; round-to-nearest-even narrowing). */
float oracle_bf16_to_f32(uint16_t b);
uint16_t oracle_f32_to_bf16(float f);

/* QLoRA linear layer in double. All matrices row-major; bf16 inputs as raw bits.
 *   x [M,K], What [N,K] (the dequantized weight), A [K,r], B [r,N], dY [M,N]
 *   s = alpha / r
 * Forward:  u = x A ;  y = x What^T + s u B
 * Backward: v = dY B^T ; dX = dY What + s v A^T ; dA = s x^T v ; dB = s u^T dY
 * Any output pointer may be NULL to skip it. */
int oracle_lora_down_xa(const uint16_t* x, int64_t M, int64_t K, const uint16_t* A, int r,
                        double* u);
int oracle_lora_down_dybt(const uint16_t* dY, int64_t M, int64_t N, const uint16_t* B, int r,
                          double* v);
int oracle_linear_fwd(const uint16_t* x, int64_t M, int64_t K, const uint16_t* What, int64_t N,
                      const uint16_t* A, const uint16_t* B, int r, double alpha, double* y,
                      double* u);
int oracle_linear_bwd(const uint16_t* x, const uint16_t* dY, int64_t M, int64_t K,
                      const uint16_t* What, int64_t N, const uint16_t* A, const uint16_t* B,
                      int r, double alpha, double* dX, double* dA, double* dB);

/* Merge of the adapter into the base in binary32 (see oracle.c):
 * out = base + s * (A B)^T with the adapter sum taken in order j = 0..r-1,
 * each product rounded to binary32 and then added (nothing fused).
 * base = the dequantized NF4 weight (wbf16 == NULL) or the bf16 weight. */
int oracle_merge_lora(const uint8_t* codes, const int8_t* q8, const float* s2, int fmt,
                      const uint16_t* wbf16, int64_t N, int64_t K, const uint16_t* A,
                      const uint16_t* B, int r, float alpha, float* out);

/* AdamW step in binary32 on n adapter parameters (see oracle.c): fp32
 * master values p, fp32 moments m and v updated in place; g is bf16
 * (g_is_bf16 != 0) or fp32; t >= 1 is the step number; p_bf16 (may be NULL)
 * receives the master values rounded to bf16. The hyper-parameters are
 * double; the per-element arithmetic is binary32. */
int oracle_adamw_step(float* p, const void* g, int g_is_bf16, float* m, float* v, int64_t n,
                      double lr, double beta1, double beta2, double eps, double wd, int64_t t,
                      uint16_t* p_bf16);

#ifdef __cplusplus
}
#endif
#endif
