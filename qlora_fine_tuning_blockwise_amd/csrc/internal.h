// Internal declarations shared by the host API and the kernels of the library.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace qlora {

constexpr int kBlock = 64;   // weights per first-level block
constexpr int kGroup = 256;  // blocks per second-level group

// Second-level formats of the 8-bit absmax code (one byte per block).
constexpr int kDqInt8 = 0;   // s2 = c2/127, signed byte 0..127
constexpr int kDqUint8 = 1;  // s2 = c2/255, unsigned byte 0..255
constexpr int kDqE4m3 = 2;   // s2 = c2/448, FP8 E4M3 value

// NF4 codebook and the call's second-level format, as the kernels receive
// them (by value, in kernel arguments).
struct Codebook {
  float level[16];
  float thr[15];
  // thr_q[i] is thr[i] or its fp32 successor, chosen so that for bf16 w and
  // c1 (c1 in [2^-60, 2^60], |w| <= c1) the exact comparison w > thr_q[i]*c1
  // agrees with RN(w/c1) > thr[i].
  float thr_q[15];
  int dq_format;
};

// Builds the codebook once (thread safe). Returns QLORA_OK or
// QLORA_ERR_INTERNAL; `cb` and `id` are valid only on QLORA_OK.
int get_codebook(const Codebook** cb, uint32_t* id);

// Identifier of the quantization setup with second-level format dq_format
// (0 for an unknown format); setup_id(kDqInt8) is the codebook id.
uint32_t setup_id(int dq_format);

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error. Sizes are pre-validated.
hipError_t launch_quantize(const void* W, bool f32_in, int64_t n, uint8_t* codes, int8_t* q8,
                           float* s2, const Codebook& cb, hipStream_t st);
// w_hat as bf16, row-major [N,K] (rows = 0), or in the K-slab layout
// [K/32][N][32] of rows = N weight rows of length K = n / N.
hipError_t launch_dequant(const uint8_t* codes, const int8_t* q8, const float* s2, int64_t n,
                          uint16_t* out, int64_t rows, const Codebook& cb, hipStream_t st);

// out[c][r'] = in[r'][c] for a bf16 [rows, cols] matrix; the second form
// transposes two matrices in one launch (in1 may be NULL).
hipError_t launch_transpose_bf16(const uint16_t* in, int64_t rows, int64_t cols, uint16_t* out,
                                 hipStream_t st);
hipError_t launch_transpose2_bf16(const uint16_t* in0, int64_t rows0, int64_t cols0,
                                  uint16_t* out0, const uint16_t* in1, int64_t rows1,
                                  int64_t cols1, uint16_t* out1, hipStream_t st);

// Rank-r down projection out[m][j] = sum_t X[m][t] * P[j][t] (X [M,T] bf16,
// P [r,T] bf16, fp32 result) in t-slices: launch_lora_down_parts writes
// part[slice][m][j]; launch_lora_down_finalize sums the slices into out (if
// out != NULL) and writes a two-term bf16 split of s*out: if lr != NULL as
// lr[m][0..r) = bf16(s*out), lr[m][r..2r) = bf16(s*out - hi); if lrT != NULL
// transposed as lrT[j][m] (hi) and lrT[r+j][m] (lo), row stride
// Mp = round_up(M, 8), zero for m >= M.
int lora_down_slices(int64_t M, int64_t T, int r);
hipError_t launch_lora_down_parts(const uint16_t* X, const uint16_t* P, int64_t M, int64_t T,
                                  int r, float* part, hipStream_t st);
// lora_down and lora_down_finalize in one pass, for large M (see
// lora_down_full_ok): out, lr, lrT as lora_down_finalize writes them; with
// u2T != NULL also the transposed split of s*u2 (u2 fp32 [M, r]), as a
// one-slice lora_down_finalize of u2 writes it.
bool lora_down_full_ok(int64_t M, int64_t T, int r);
hipError_t launch_lora_down_full(const uint16_t* X, const uint16_t* P, int64_t M, int64_t T,
                                 int r, float s, float* out, uint16_t* lr, uint16_t* lrT,
                                 const float* u2, uint16_t* u2T, hipStream_t st);
hipError_t launch_lora_down_finalize(const float* part, int slices, int64_t M, int r, float s,
                                     float* out, uint16_t* lr, uint16_t* lrT, hipStream_t st);
// Two independent finalizes of the same M and r in one launch.
hipError_t launch_lora_down_finalize2(const float* part0, int slices0, float* out0, uint16_t* lr0,
                                      uint16_t* lrT0, const float* part1, int slices1,
                                      float* out1, uint16_t* lr1, uint16_t* lrT1, int64_t M, int r,
                                      float s, hipStream_t st);

// y = x W_hat^T + [ulr-extended term], M > 16 path (MFMA tiles).
// With a buffer `part` of gemm_fwd_splits(M, N, K) * M * N floats (when that
// count is above 1) the reduction over K is split across workgroups and the
// splits are added in order; part = NULL: no split.
int gemm_fwd_splits(int64_t M, int64_t N, int64_t K);
// The lean forward's workspace without the tile kernel's split sums (the
// smallest workspace qlora_linear_fwd accepts; 0 for invalid sizes).
size_t fwd_workspace_nosplit(int64_t M, int64_t N, int64_t K, int r);
hipError_t launch_gemm_fwd(const uint16_t* x, const uint8_t* codes, const int8_t* q8,
                           const float* s2, const uint16_t* ulr, const uint16_t* Bt, int64_t M,
                           int64_t N, int64_t K, int r, void* y, bool y_bf16, const Codebook& cb,
                           hipStream_t st, float* part = nullptr);

// Decode path (M <= 16), two launches: part[slice][m][j] = sum over one of
// decode_down_slices(K) slices of K of x[m,k] A[k,j] (A [K,r] as given), then the GEMV with
// y = x W_hat^T + s * (sum_slice part) B in its epilogue; u_out (if not NULL)
// receives u = sum_slice part.
int decode_down_slices(int64_t K);
hipError_t launch_lora_down_decode(const uint16_t* x, const uint16_t* A, int64_t M, int64_t K,
                                   int r, float* part, hipStream_t st);
hipError_t launch_gemv(const uint16_t* x, const uint8_t* codes, const int8_t* q8,
                       const float* s2, const float* upart, int slices, const uint16_t* B,
                       int64_t M, int64_t N, int64_t K, int r, float s, float* u_out, void* y,
                       bool y_bf16, const Codebook& cb, hipStream_t st);

// The decode GEMV with one memory round trip per wave (decode_tiles_ok:
// M <= 4, K <= 4096, K % 256 == 0, r <= 32): one workgroup per 16-row tile;
// same arguments and results as launch_gemv.
bool decode_tiles_ok(int64_t M, int64_t N, int64_t K, int r);
hipError_t launch_gemv_tiles(const uint16_t* x, const uint8_t* codes, const int8_t* q8,
                             const float* s2, const float* upart, int slices, const uint16_t* B,
                             int64_t M, int64_t N, int64_t K, int r, float s, float* u_out,
                             void* y, bool y_bf16, const Codebook& cb, hipStream_t st);

// dX = dY W_hat + [svlr-extended term with A].
// With a buffer `part` of gemm_bwd_splits(M, N, K) * M * K floats (when that
// count is above 1) the reduction over N is split across workgroups and the
// splits are added in order; part = NULL: no split.
int gemm_bwd_splits(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_bwd(const uint16_t* dY, const uint8_t* codes, const int8_t* q8,
                           const float* s2, const uint16_t* svlr, const uint16_t* A, int64_t M,
                           int64_t N, int64_t K, int r, void* dX, bool dx_bf16,
                           const Codebook& cb, hipStream_t st, float* part = nullptr);
// y[i] = sum over s of part[s][i] for i < n, in split order (fp32, or bf16 by
// round to nearest even of the fp32 sum).
hipError_t launch_split_reduce(const float* part, int splits, int64_t n, void* y, bool y_bf16,
                               hipStream_t st);

// Large-M path: plain bf16 GEMM y[M,N] = a[M,Kr] b[N,Kr]^T + e[M,2r] [f|f][N,2r]^T
// (a row-major with row stride lda; b row-major with row stride ldb, or in
// the K-slab layout [Kr/32][N][32] when b_kslab; e the two-term split written
// by launch_lora_down_finalize; f [N,r]). gemm_nt_supported says whether the
// shape fits the kernel (Kr a multiple of 32, 16-byte aligned rows, 32-bit
// buffer offsets).
// With few output tiles the reduction is split (gemm_nt_splits > 1): each
// split writes fp32 sums to part [splits][M][N] and a reduce launch adds
// them in split order into y.
bool gemm_nt_supported(int64_t Kr, int64_t lda, int64_t ldb, int64_t N, bool b_kslab);
int gemm_nt_splits(int64_t M, int64_t N, int64_t Kr);
hipError_t launch_gemm_nt(const uint16_t* a, int64_t lda, const uint16_t* b, int64_t ldb,
                          const uint16_t* e, const uint16_t* f, int64_t M, int64_t N, int64_t Kr,
                          int r, void* y, bool y_bf16, bool b_kslab, hipStream_t st,
                          int ksplit = 1, float* part = nullptr);
// Fused large-M forward: y = x W_hat^T + e [f|f]^T with the NF4 weight
// dequantized in registers right before the MFMAs (no bf16 copy of the
// weight). e is the two-term split of s*u (launch_lora_down_*), f = B^T.
bool gemm_nf4_supported(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_nf4_fwd(const uint16_t* x, const uint8_t* codes, const int8_t* q8,
                               const float* s2, const uint16_t* e, const uint16_t* f, int64_t M,
                               int64_t N, int64_t K, int r, void* y, bool y_bf16,
                               const Codebook& cb, hipStream_t st);

// w_hat^T as bf16 in the K-slab layout [N/32][K][32]: out[s][k][j] =
// w_hat[32 s + j][k] (N % 32 == 0, K % 64 == 0, else hipErrorInvalidValue).
hipError_t launch_dequant_t(const uint8_t* codes, const int8_t* q8, const float* s2, int64_t N,
                            int64_t K, uint16_t* out, const Codebook& cb, hipStream_t st);

// merged = base + s (A B)^T in binary32 (adapter sum in order j = 0..r-1);
// base = the dequantized NF4 weight (W == NULL) or the bf16 weight W.
// At = A^T [r,K], Bt = B^T [N,r].
hipError_t launch_merge(const uint8_t* codes, const int8_t* q8, const float* s2,
                        const uint16_t* W, int64_t N, int64_t K, const uint16_t* At,
                        const uint16_t* Bt, int r, float s, float* out, const Codebook& cb,
                        hipStream_t st);

// AdamW step scalars, each computed on the host in double from the
// hyper-parameters and rounded once to binary32.
struct AdamScalars {
  float b1, b2, eps;  // beta1, beta2, eps
  float decay;        // 1 - lr*wd
  float c1, c2;       // 1 - beta1, 1 - beta2
  float step_size;    // lr / (1 - beta1^t)
  float bc2_sqrt;     // sqrt(1 - beta2^t)
};

// AdamW on n parameters in place (p, m, v fp32; g bf16 or fp32; pb the bf16
// copy of p, may be NULL). Pointers may be device or mapped host memory.
hipError_t launch_adamw(float* p, const void* g, bool g_bf16, float* m, float* v, uint16_t* pb,
                        int64_t n, const AdamScalars& s, hipStream_t st);

// Adapter gradients: part[split][c][j] = sum_{m in split} X[m][c] * P[m][j]
// (X [M,C] bf16; P given as the transposed two-term bf16 split PT [2r, Mp]
// written by launch_lora_down_finalize), then out = s * sum_split part,
// written as [C,r] (transpose_out = false) or [r,C] (true), fp32 or bf16.
int colred_splits(int64_t M);
hipError_t launch_colred(const uint16_t* X, const uint16_t* PT, int64_t M, int64_t C, int r,
                         float* part, hipStream_t st);
hipError_t launch_colred_finalize(const float* part, int splits, int64_t C, int r, float s,
                                  bool transpose_out, void* out, bool out_bf16, hipStream_t st);
// The same for two reductions over the same M rows in one launch each (the
// second job is skipped when X1 / part1 is NULL).
hipError_t launch_colred2(const uint16_t* X0, const uint16_t* PT0, int64_t C0, float* part0,
                          const uint16_t* X1, const uint16_t* PT1, int64_t C1, float* part1,
                          int64_t M, int r, hipStream_t st);
// Both reductions in one launch written straight to their outputs (no
// partial sums, no finalize): out = sum_m X[m][c] (PT[j][m] + PT[r+j][m]) as
// [C, r] or transposed [r, C]. colred_direct_cg(M, K, N, r) decides from the
// layer's shape alone whether it applies (0: no) and with how many 32-column
// groups a workgroup (2 or 4; the bits do not depend on it); X1 = NULL: one
// job.
int colred_direct_cg(int64_t M, int64_t K, int64_t N, int r);
hipError_t launch_colred_direct2(const uint16_t* X0, const uint16_t* PT0, int64_t C0,
                                 void* out0, bool transpose0, const uint16_t* X1,
                                 const uint16_t* PT1, int64_t C1, void* out1, bool transpose1,
                                 int64_t M, int r, int cg, bool out_bf16, hipStream_t st);
hipError_t launch_colred_finalize2(const float* part0, int64_t C0, bool transpose_out0,
                                   void* out0, const float* part1, int64_t C1,
                                   bool transpose_out1, void* out1, int splits, int r, float s,
                                   bool out_bf16, hipStream_t st);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t st);

}  // namespace qlora
