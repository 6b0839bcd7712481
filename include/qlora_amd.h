/*
 * qlora_amd.h - C ABI of the MI355X (gfx950) QLoRA frozen-base library.
 *
 * The library implements the frozen-base hot path of QLoRA as the pages on
 * the method describe it:
 *   [P1] "QLoRA", learning-llms.pages.dev/topics/qlora
 *   [P2] "QLoRA", infra.bea.ai/guide/training/fine-tuning-adapters/qlora
 *   [P3] "QLoRA", scalata.ai/resources/model-training/qlora
 *   [P4] "What does QLoRA change about a LoRA run, and why does it fit on one
 *        GPU?", katajob.com/questions/found-fine-tuning-peft-qlora-memory
 *   [P5] "QLoRA viz", engineersofai.com/playground/qlora-viz
 *
 * STORAGE FORMAT (one format for every entry point)
 *   A weight W is [N, K] row-major (N out-features, K in-features), flat
 *   index e = n*K + k. K must be a multiple of 64 so that blocks never
 *   straddle rows.
 *   - block b = e / 64: 64 consecutive weights sharing one absmax ([P1]
 *     bullets: small blocks of 64 weights, one scale per block);
 *   - codes   uint8[N*K/2]: NF4 code of weight e in the low nibble of byte
 *     e/2 when e is even, in the high nibble when e is odd;
 *   - absmax_q int8[N*K/64]: one byte per block, the block absmax quantized
 *     to 8 bits - the double quantization of [P1] bullets ("8-bit"), [P2] s1
 *     "Double Quantization" ("FP8"), [P5] "Double Quantization". The byte's
 *     meaning is the second-level format (dq_format) the weight was
 *     quantized with, and every call on the weight must pass the same one:
 *       QLORA_DQ_INT8   signed byte 0..127, s2 = c2/127 (the default);
 *       QLORA_DQ_UINT8  unsigned byte 0..255, s2 = c2/255;
 *       QLORA_DQ_E4M3   an FP8 E4M3 value (OCP E4M3FN: exponent bias 7,
 *                       subnormals m*2^-9, largest 448), s2 = c2/448; the
 *                       NaN codes 0x7F and 0xFF never occur.
 *   - absmax_scale float[ceil(N*K/16384)]: one fp32 second-level scale per
 *     group of 256 consecutive blocks.
 *   Total 4 + 8/64 + 32/16384 = 4.126953125 bits per weight in every format.
 *
 *   Dequantization ([P1] bullets: compute never happens in 4-bit; weights are
 *   dequantized to bf16 just in time): with L the 16 NF4 levels and value()
 *   the format's reading of the byte (exact in fp32),
 *     c1_hat = fp32(value(absmax_q[b]) * absmax_scale[b/256])
 *     w_hat  = bf16_rne(fp32(L[code] * c1_hat)).
 *
 * CONVENTIONS
 *   - A quantized weight travels as a qlora_nf4 descriptor (below): its
 *     buffers plus the format version and quantization setup it was made
 *     with. dq_format is one of the QLORA_DQ_* formats.
 *   - Every pointer argument of a compute entry point is a DEVICE pointer
 *     owned by the caller; the library allocates nothing and keeps no state
 *     besides a constant codebook built on first use.
 *   - bf16 tensors are passed as uint16_t bit patterns.
 *   - `stream` is a hipStream_t (NULL = the default stream). Every compute
 *     entry point only enqueues work on it and returns without synchronizing.
 *   - Device pointers must be 16-byte aligned. Outputs must not alias inputs.
 *   - Return value: QLORA_OK (0) or a status below. Argument errors are
 *     detected on the host before anything is enqueued. No C++ exception
 *     crosses the ABI.
 *   - Concurrent calls on different streams are safe; calls sharing a
 *     workspace buffer must be ordered by the caller.
 */
#ifndef QLORA_AMD_H
#define QLORA_AMD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define QLORA_OK 0
#define QLORA_ERR_INVALID_ARG 1 /* NULL pointer, negative size, bad enum */
#define QLORA_ERR_SHAPE 2       /* K % 64 != 0, N or K < 1, or two of M, N, K
                                   whose product passes 2^40 elements */
#define QLORA_ERR_ALIGN 3       /* a device pointer is not 16-byte aligned */
#define QLORA_ERR_DTYPE 4       /* unsupported dtype enum */
#define QLORA_ERR_RANK 5        /* r not a positive multiple of 16, or r > 256 */
#define QLORA_ERR_WORKSPACE 6   /* workspace smaller than qlora_workspace_bytes() */
#define QLORA_ERR_LAUNCH 7      /* the HIP runtime reported an error on launch */
#define QLORA_ERR_INTERNAL 8    /* codebook construction failed its self-check */
#define QLORA_ERR_SETUP 9       /* weight descriptor from another format version or
                                   quantization setup than this library's */
#define QLORA_ERR_TOO_LARGE 10  /* the call needs more workspace than the
                                   allocation-free entry point holds */

/* Element types. */
#define QLORA_DTYPE_F32 0
#define QLORA_DTYPE_BF16 1

/* Second-level formats of absmax_q (see STORAGE FORMAT). */
#define QLORA_DQ_INT8 0
#define QLORA_DQ_UINT8 1
#define QLORA_DQ_E4M3 2

/* Layouts of a dequantized bf16 weight (and of the dense stage's b operand):
 *   QLORA_LAYOUT_ROWS     [N, K] row-major;
 *   QLORA_LAYOUT_KSLAB32  [K/32][N][32]: the 32 consecutive k of slab s of row
 *                         n are the 64 bytes at ((s*N + n)*32) elements, so
 *                         the slab's rows are contiguous. The large-batch
 *                         path keeps its dequantized weight in this layout:
 *                         a load of 16 rows of one slab is 1 KB of consecutive
 *                         bytes, whole cache lines. */
#define QLORA_LAYOUT_ROWS 0
#define QLORA_LAYOUT_KSLAB32 1

/* Operations for qlora_workspace_bytes. */
#define QLORA_OP_FWD 0
#define QLORA_OP_BWD 1
#define QLORA_OP_MERGE 2
#define QLORA_OP_FWD_LEAN 3 /* the forward without a bf16 copy of the weight */
#define QLORA_OP_BWD_LEAN 4 /* the backward without a bf16 copy of the weight */

/* Format version of the storage layout above. */
#define QLORA_FORMAT_VERSION 1u

/* Descriptor of one quantized weight: its shape, its three device buffers
 * and the metadata that says how it was quantized. [P4] "Operational
 * coupling": the quantization setup belongs in the adapter's recorded
 * metadata, because an adapter trained against one quantized base is tied
 * to exactly that base. qlora_quantize_nf4_dq writes every field except the
 * three buffer pointers, which the caller sets; a caller that stores a
 * quantized weight stores the metadata fields with it and restores them.
 * Every entry point that reads the weight first checks the descriptor with
 * qlora_nf4_check and fails with its status (QLORA_ERR_SETUP when
 * format_version or setup_id do not match this library), so a weight is
 * never decoded with another codebook or second-level format than the one
 * it was quantized with. */
typedef struct qlora_nf4 {
  int64_t N, K;           /* W is [N, K] row-major, K % 64 == 0 */
  uint8_t* codes;         /* device, N*K/2 bytes (see STORAGE FORMAT) */
  int8_t* absmax_q;       /* device, N*K/64 bytes */
  float* absmax_scale;    /* device, ceil(N*K/16384) floats */
  int32_t dq_format;      /* QLORA_DQ_* second-level format of absmax_q */
  uint32_t format_version; /* QLORA_FORMAT_VERSION of the storage layout */
  uint32_t setup_id;      /* qlora_setup_id(dq_format) of the quantizing library */
  uint32_t reserved;      /* 0 */
} qlora_nf4;

/* Human-readable text of a status code (static storage, never NULL). */
const char* qlora_strerror(int status);

/* Byte sizes of the three quantized buffers of an [N,K] weight. Host only.
 * Returns QLORA_ERR_SHAPE unless N >= 1, K >= 64, K % 64 == 0 and
 * N*K <= 2^40. */
int qlora_nf4_sizes(int64_t N, int64_t K, size_t* codes_bytes, size_t* absmax_q_bytes,
                    size_t* absmax_scale_bytes);

/* The library's NF4 codebook: 16 fp32 levels and the 15 fp32 decision
 * thresholds used by the quantizer. Host only.
 * Levels: quantiles of a standard normal distribution ([P1] bullets "NF4
 * instead of a uniform grid"; [P2] s1 "Key Innovation: NF4") with equal
 * probability steps, 8 positive and 7 negative levels, an exact 0, scaled so
 * that the outermost levels are exactly -1 and +1. Threshold i is the
 * midpoint of levels i and i+1 rounded toward -infinity to fp32, so that a
 * normalised value x gets code #{i : x > threshold[i]}: the nearest level,
 * ties to the lower code. */
int qlora_codebook(float levels[16], float thresholds[15]);

/* The same decisions for bf16 weights, stated on the weight and the block
 * absmax directly (the quantizer's bf16 path uses these): thresholds_q[i] is
 * thresholds[i] or its fp32 successor, such that for bf16 values w and c1
 * with c1 in [2^-60, 2^60] and |w| <= c1 the exact comparison
 * w > thresholds_q[i] * c1 holds exactly when RN(w / c1) > thresholds[i]
 * (RN: fp32 division, round to nearest even). Host only; QLORA_ERR_INVALID_ARG
 * for a NULL array. */
int qlora_codebook_quotient_thresholds(float thresholds_q[15]);

/* Identifier of the quantization setup (FNV-1a over the 16 level bit
 * patterns, the block and group sizes, the nibble order and the form of the
 * second level). [P4] "Operational coupling": the quantization setup belongs
 * in the adapter's recorded metadata. Host only; 0 if the codebook failed. */
uint32_t qlora_codebook_id(void);

/* Identifier of the quantization setup with second-level format dq_format:
 * the codebook id's hash with that format's top code value (127, 255, 448)
 * in place of 127, so qlora_setup_id(QLORA_DQ_INT8) == qlora_codebook_id().
 * Host only; 0 for an unknown format or if the codebook failed. */
uint32_t qlora_setup_id(int dq_format);

/* Checks a weight descriptor on the host: QLORA_ERR_INVALID_ARG for a NULL
 * descriptor or buffer, an unknown dq_format or reserved != 0;
 * QLORA_ERR_SHAPE unless N >= 1, K >= 64, K % 64 == 0 and N*K <= 2^40;
 * QLORA_ERR_ALIGN for a buffer that is not 16-byte aligned; QLORA_ERR_SETUP when
 * format_version != QLORA_FORMAT_VERSION or setup_id !=
 * qlora_setup_id(dq_format). QLORA_OK otherwise. */
int qlora_nf4_check(const qlora_nf4* w);

/* Device workspace, in bytes, that qlora_linear_fwd (op = QLORA_OP_FWD),
 * qlora_linear_bwd (op = QLORA_OP_BWD) or qlora_merge_lora (op =
 * QLORA_OP_MERGE, M ignored) needs for these sizes, assuming no saved u.
 * From M = 512 rows on, QLORA_OP_FWD and QLORA_OP_BWD include N*K*2 bytes for
 * one dequantized bf16 copy of the weight (the pages' one layer's worth of
 * 16-bit weights, [P3] "How it works"): the fast route. QLORA_OP_FWD_LEAN is
 * the forward's workspace without that copy: with less than the QLORA_OP_FWD
 * size but at least this one, qlora_linear_fwd runs its fused kernels, which
 * dequantize each weight tile in registers right before the matrix cores
 * use it and never hold a bf16 copy ([P4] "The mechanism"). For some shapes
 * below 512 rows this size includes fp32 partial sums that split the
 * reduction over K across workgroups; a workspace too small for them but
 * large enough for the rest runs the same kernel unsplit (the same result
 * within rounding, not bit for bit). Likewise
 * QLORA_OP_BWD_LEAN for the backward: with less than the QLORA_OP_BWD size
 * but at least this one, dX runs through the kernel that dequantizes the
 * transposed operand in registers ([P2] s3). Host only; 0 on invalid
 * sizes. */
size_t qlora_workspace_bytes(int op, int64_t M, int64_t N, int64_t K, int r);

/* Quantize once, at load time ([P4] "The mechanism": the pretrained weights
 * are quantized once, at load time, and never updated; [P1] "controlled
 * rounding" and its bullets; [P2] s1; [P3] "How it works").
 *   W        [N,K] row-major, fp32 (w_dtype = QLORA_DTYPE_F32) or bf16
 *            (QLORA_DTYPE_BF16). Values must be finite; a non-finite input
 *            gives unspecified codes (no fault).
 *   out      descriptor whose codes, absmax_q and absmax_scale the caller
 *            has pointed at device buffers of the sizes qlora_nf4_sizes
 *            gives; the call writes its N, K, dq_format, format_version,
 *            setup_id and reserved fields (host side, before the launch) and
 *            the three buffers (on the stream).
 * Per block: c1 = max|w|; x = w / c1 (correctly rounded fp32 division);
 * code = #{i : x > threshold[i]}; an all-zero block gets code 7 (level 0).
 * Per group of 256 blocks: c2 = max c1; s2 = c2 / top (fp32 division; top =
 * 127, 255 or 448 by dq_format); absmax_q = the nearest integer to c1 / s2
 * (ties to the lower) clamped to [0, top] for the integer formats, or the
 * nearest E4M3 value (ties to even, saturating at 448); 0 for c1 == 0. The
 * NF4 codes use the exact fp32 c1. QLORA_ERR_INVALID_ARG for an unknown
 * dq_format or a NULL buffer; the descriptor is left untouched on any
 * error. */
int qlora_quantize_nf4_dq(const void* W, int w_dtype, int64_t N, int64_t K, int dq_format,
                          qlora_nf4* out, void* stream);

/* Dequantize to bf16 ([P1] bullets "Compute never happens in 4-bit"; [P3]
 * "How it works": each layer's 4-bit weights are unpacked into 16-bit).
 *   w       weight descriptor (qlora_nf4_check must pass).
 *   W_out   N*K bf16, w_hat as in the format section, in `layout`
 *           (QLORA_LAYOUT_ROWS or QLORA_LAYOUT_KSLAB32; the K-slab layout
 *           needs N*K/64 < 2^32, else QLORA_ERR_SHAPE).
 * QLORA_ERR_INVALID_ARG for another layout. */
int qlora_dequant_bf16(const qlora_nf4* w, uint16_t* W_out, int layout, void* stream);

/* QLoRA linear forward ([P1] forward equation h = W_hat x + (alpha/r) B(Ax),
 * here in row-major form):
 *   u = x A                     (fp32 [M,r])
 *   y = x W_hat^T + (alpha/r) u B
 *   w  weight descriptor, W_hat [N,K] (qlora_nf4_check must pass);
 *   x  [M,K] bf16;  A [K,r] bf16;  B [r,N] bf16;  y [M,N] fp32 or bf16
 *      (y_dtype; the bf16 output is the round-to-nearest-even of the fp32
 *      result of the same computation).
 *   u_out      fp32 [M,r] or NULL; when given it receives u (for the backward).
 *   workspace  device buffer of at least qlora_workspace_bytes(FWD_LEAN,
 *              M,N,K,r); from M = 512 on, a workspace of the FWD size selects
 *              the faster route through one bf16 copy of the weight.
 * The weight is read through its dequantized bf16 values, products are exact
 * and accumulate in fp32. M == 0 is a successful no-op. r % 16 == 0.
 * QLORA_ERR_SHAPE when M*N or M*K passes 2^40. */
int qlora_linear_fwd(const qlora_nf4* w, const uint16_t* x, int64_t M,
                     const uint16_t* A, const uint16_t* B, int r, float alpha, void* y,
                     int y_dtype, float* u_out, void* workspace, size_t workspace_bytes,
                     void* stream);

/* QLoRA linear backward ([P2] s3 "The Backward Pass Through Quantization":
 * gradients flow through the dequantized frozen base, only the adapters get
 * gradients; [P4] "The mechanism"):
 *   v  = dY B^T                      (fp32 [M,r])
 *   dX = dY W_hat + (alpha/r) v A^T  ([M,K], dx_dtype fp32 or bf16)
 *   dA = (alpha/r) x^T v             ([K,r], grad_dtype fp32 or bf16)
 *   dB = (alpha/r) u^T dY            ([r,N], grad_dtype), u = x A
 *   dY [M,N] bf16; x, A, B as in the forward.
 *   u_saved  fp32 [M,r] from qlora_linear_fwd's u_out, or NULL to recompute.
 *   dX, dA, dB may each be NULL to skip that output (x may then be NULL if
 *   both dA and dB are NULL).
 *   workspace  device buffer of at least qlora_workspace_bytes(BWD_LEAN,
 *              M,N,K,r); from M = 512 on, a workspace of the BWD size selects
 *              the faster route through one transposed bf16 copy of the
 *              weight.
 * The frozen base is never written. M == 0 writes zero dA and dB.
 * QLORA_ERR_SHAPE when M*N or M*K passes 2^40. */
int qlora_linear_bwd(const qlora_nf4* w, const uint16_t* x, const uint16_t* dY,
                     int64_t M, const uint16_t* A, const uint16_t* B, int r, float alpha,
                     const float* u_saved, void* dX, int dx_dtype, void* dA, void* dB,
                     int grad_dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Merge the trained adapter into the base, in binary32 ([P1] bullets:
 * folding BA into a 4-bit W forces a re-quantization, a second rounding;
 * [P4] "What it costs", "Merge friction": the clean path merges into the
 * 16-bit weights and quantizes once afterwards):
 *   merged[n][k] = base[n][k] + s * d[n][k],  s = alpha / r (binary32),
 *   d[n][k] = sum_j A[k][j] B[j][n], starting from +0 and taking the terms
 *   j = 0..r-1 in order, each product rounded to binary32 and then each
 *   addition rounded (nothing fused); then s*d rounds, then the final sum
 *   rounds (nearest-even).
 *   base = w_hat (the dequantized NF4 weight of descriptor w, whose N and K
 *          must equal N and K) when W is NULL, else the bf16 weight W [N,K]
 *          (w is then ignored and may be NULL).
 *   A [K,r] bf16; B [r,N] bf16; merged fp32 [N,K] (caller-owned output).
 *   workspace  at least qlora_workspace_bytes(QLORA_OP_MERGE, 0, N, K, r).
 * Requantizing the merged weight is qlora_quantize_nf4_dq with
 * QLORA_DTYPE_F32 input. Same shape and rank rules as the linear entry
 * points; QLORA_ERR_INVALID_ARG when neither base is given, QLORA_ERR_SHAPE
 * when w's shape is not [N,K]. */
int qlora_merge_lora(const qlora_nf4* w, const uint16_t* W, int64_t N, int64_t K, const uint16_t* A,
                     const uint16_t* B, int r, float alpha, float* merged, void* workspace,
                     size_t workspace_bytes, void* stream);

/* AdamW step on the adapter parameters, in place ([P2] precision table: the
 * Adam state of an adapter parameter is fp32, 12 bytes - read as the fp32
 * master value and two fp32 moments; [P4] "The memory term LoRA does not
 * remove": master copies and optimizer moments are the trained parameters'
 * state). n parameters as flat arrays, typically every adapter of a model
 * laid out in one buffer so that one call steps them all:
 *   param       fp32[n]  master values, updated in place;
 *   grad        [n]      QLORA_DTYPE_BF16 (the pages' adapter gradients) or
 *                        QLORA_DTYPE_F32, read only;
 *   exp_avg     fp32[n]  first moment m, updated in place;
 *   exp_avg_sq  fp32[n]  second moment v, updated in place;
 *   param_bf16  bf16[n]  receives RNbf16 of the new master values (the
 *                        adapter the linear layer reads), or NULL.
 *   step        the 1-based step number t.
 * Scalars, each computed on the host in double and rounded once to fp32:
 *   decay = 1 - lr*weight_decay, c1 = 1 - beta1, c2 = 1 - beta2,
 *   step_size = lr / (1 - beta1^t), bc2_sqrt = sqrt(1 - beta2^t), and
 *   beta1, beta2, eps themselves. Per element in fp32, every operation
 *   rounded to nearest-even and none fused:
 *   p = p*decay;  m = beta1*m + c1*g;  v = beta2*v + c2*(g*g);
 *   p = p - step_size * (m / (sqrt(v)/bc2_sqrt + eps)).
 * Paged state ([P1] paragraph on paged optimizers; [P3] "How it works": the
 * optimizer state moves to CPU memory instead of the run failing): every
 * array may live in device memory or in pinned, mapped host memory
 * (hipHostMalloc); the kernel then streams that array across the host link.
 * Pageable host memory is rejected with QLORA_ERR_INVALID_ARG. The arrays
 * must not overlap. n == 0 is a no-op. QLORA_ERR_INVALID_ARG for n < 0,
 * step < 1, beta outside [0, 1), non-finite lr, eps or weight_decay, or a
 * NULL array (param_bf16 aside); QLORA_ERR_DTYPE for another grad_dtype;
 * QLORA_ERR_ALIGN for an array not 16-byte aligned. */
int qlora_adamw_step(float* param, const void* grad, int grad_dtype, float* exp_avg,
                     float* exp_avg_sq, uint16_t* param_bf16, int64_t n, double lr, double beta1,
                     double beta2, double eps, double weight_decay, int64_t step, void* stream);

/* Dense stage of the large-batch path: the product with a weight that is
 * already dequantized ([P1] bullets: the 4-bit weight is expanded to bf16
 * just in time, then multiplied in bf16 with fp32 accumulation; [P3] "How it
 * works"), plus a rank extension:
 *   y = a b^T + e [f | f]^T
 *   a  [M,K] bf16, row stride lda elements;  b [N,K] bf16 in b_layout:
 *      QLORA_LAYOUT_ROWS with row stride ldb, or QLORA_LAYOUT_KSLAB32 (ldb
 *      ignored; for instance W_out of qlora_dequant_bf16);  e [M,2r] bf16;
 *   f  [N,r] bf16;  y [M,N] fp32 or bf16 (y_dtype; bf16 is the
 *      round-to-nearest-even of the fp32 result).
 * From M = 512 rows on, qlora_linear_bwd dequantizes the transposed weight
 * once into its workspace (K-slab layout) and runs this stage for dX with
 * a = dY, b = w_hat^T, f = A and e the two-term split [hi | lo] of
 * (alpha/r) v (hi = bf16(v), lo = bf16(v - hi)), so that e [f|f]^T adds
 * (hi + lo) A^T. With qlora_dequant_bf16 it also forms the unfused
 * counterpart of the forward, whose large-batch kernel dequantizes in
 * registers instead. Requires K >= 32 and K % 32 ==
 * 0, lda a multiple of 8 with 512*lda + 2*K < 2^31 and lda >= K; for
 * QLORA_LAYOUT_ROWS ldb likewise, for QLORA_LAYOUT_KSLAB32 2*N*K < 2^31; r as
 * for the linear entry points (QLORA_ERR_SHAPE / QLORA_ERR_RANK otherwise;
 * QLORA_ERR_INVALID_ARG for another b_layout). M == 0 is a successful
 * no-op. */
int qlora_gemm_bf16_nt(const uint16_t* a, int64_t lda, const uint16_t* b, int64_t ldb,
                       int b_layout, const uint16_t* e, const uint16_t* f, int64_t M, int64_t N,
                       int64_t K, int r, void* y, int y_dtype, void* stream);

/* Bytes of the device array that qlora_linear_fwd_noalloc uses as its
 * workspace (one array per GPU, held until the process ends). */
#define QLORA_NOALLOC_SCRATCH_BYTES (32u << 20)

/* qlora_linear_fwd for callers that cannot allocate device memory: code
 * being captured into a HIP graph, tight serving loops, harnesses that forbid
 * allocation. Same arguments and results as qlora_linear_fwd without the
 * workspace: the call takes its workspace from a file-scope device array of
 * QLORA_NOALLOC_SCRATCH_BYTES on the current device and allocates nothing
 * (no hipMalloc, no host allocation). It runs the launches that
 * qlora_linear_fwd runs with a workspace of exactly
 * qlora_workspace_bytes(QLORA_OP_FWD_LEAN, M, N, K, r) bytes (from 512 rows
 * on, the fused route that holds no bf16 copy of the weight), so its
 * results equal that call's bit for bit. QLORA_ERR_TOO_LARGE when that size
 * exceeds QLORA_NOALLOC_SCRATCH_BYTES, before anything is enqueued; the
 * other errors as qlora_linear_fwd. All calls on one GPU share its array:
 * calls that overlap on one GPU (other streams, other threads) race, and the
 * caller must order them. */
int qlora_linear_fwd_noalloc(const qlora_nf4* w, const uint16_t* x, int64_t M,
                             const uint16_t* A, const uint16_t* B, int r, float alpha, void* y,
                             int y_dtype, float* u_out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* QLORA_AMD_H */
