// Dequantize-into-MFMA kernels of the QLoRA linear layer on gfx950.
//
// [P1] "QLoRA" forward equation h = W_hat x + (alpha/r) B(Ax) and bullets
// ("Compute never happens in 4-bit": the weight is dequantized to bf16 just in
// time for the matmul); [P2] s3 "The Backward Pass Through Quantization"
// (dequantize on the fly, compute in bf16, only adapter gradients).
//
// Structure shared by the forward and backward tile kernels:
//  - a workgroup of 4 waves owns a 256 (M) x 256 (output columns) tile; each
//    wave owns all 256 rows of its 64 columns, so every weight element of the
//    tile is dequantized exactly once per workgroup, in registers, straight
//    into the MFMA B operand - no bf16 copy of the weight goes through LDS;
//  - the activation tile (x or dY, 256 x 64 bf16) is staged through LDS,
//    double buffered, padded rows, and read as MFMA A operands;
//  - per 64-wide reduction step each thread builds one 16-entry bf16 table
//    (bf16(L[i] * c1_hat)) for one (weight row, block) into LDS; a code is
//    dequantized by one LDS lookup, exactly as the standalone dequant kernel;
//  - v_mfma_f32_16x16x32_bf16 with fp32 accumulators (256 per lane);
//  - the LoRA term rides the same accumulators as extra reduction steps:
//    [s*u_hi | s*u_lo] (bf16 split of the fp32 adapter product) times the
//    matching adapter columns.
#include "device.h"

namespace qlora {
namespace {

constexpr int kBM = 256;       // rows of M per workgroup
constexpr int kBN = 256;       // output columns per workgroup (64 per wave)
constexpr int kXS = 64 + 8;    // LDS row stride (bf16) of the activation tile

// Stage the 256 x 64 bf16 activation tile rows [m0, m0+256) x cols [c0, c0+64)
// of a row-major [rows, ld] matrix into registers. Thread t takes rows
// t/8 + 32i (i = 0..7), 8 columns at (t%8)*8. Out-of-range rows or columns
// read as zero. `vec_ok` says every row start is 16-byte aligned.
__device__ __forceinline__ void load_act_tile(const uint16_t* __restrict__ a, int64_t rows,
                                              int64_t ld, int64_t m0, int64_t c0, bool vec_ok,
                                              int tid, u32x4_t (&reg)[8]) {
  const int cc = (tid & 7) * 8;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t m = m0 + (tid >> 3) + 32 * i;
    const int64_t c = c0 + cc;
    if (m < rows && vec_ok && c + 8 <= ld) {
      reg[i] = *reinterpret_cast<const u32x4_t*>(a + m * ld + c);
    } else {
      uint16_t h[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) h[j] = (m < rows && c + j < ld) ? a[m * ld + c + j] : (uint16_t)0;
      reg[i] = u32x4_t{h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16),
                       h[4] | ((uint32_t)h[5] << 16), h[6] | ((uint32_t)h[7] << 16)};
    }
  }
}

__device__ __forceinline__ void store_act_tile(uint16_t* lds, int tid, const u32x4_t (&reg)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<u32x4_t*>(lds + ((tid >> 3) + 32 * i) * kXS + (tid & 7) * 8) = reg[i];
}

// Write 4 consecutive fp32 (or bf16) outputs of row m starting at column c.
template <bool kBf16>
__device__ __forceinline__ void store4(void* out, int64_t ld, int64_t m, int64_t c, int64_t cols,
                                       float v0, float v1, float v2, float v3) {
  if (kBf16) {
    uint16_t* o = static_cast<uint16_t*>(out) + m * ld + c;
    if (c + 4 <= cols && (ld & 3) == 0) {
      *reinterpret_cast<u32x2_t*>(o) = u32x2_t{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
    } else {
      const float v[4] = {v0, v1, v2, v3};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (c + j < cols) o[j] = (uint16_t)(pack_bf16x2(v[j], 0.0f) & 0xFFFFu);
    }
  } else {
    float* o = static_cast<float*>(out) + m * ld + c;
    if (c + 4 <= cols && (ld & 3) == 0) {
      *reinterpret_cast<f32x4_t*>(o) = f32x4_t{v0, v1, v2, v3};
    } else {
      const float v[4] = {v0, v1, v2, v3};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (c + j < cols) o[j] = v[j];
    }
  }
}

// ----------------------------------------------------------------- forward
// y[m,n] = sum_k x[m,k] w_hat[n,k] + sum_j ulr[m,j] Bt[n, j mod r]
// Wave w owns output columns n0 + 64w + 4c + t (c = lane%16, t = 0..3): MFMA
// t of a row tile holds column 4c + t at lane column c, so each lane ends
// with 4 adjacent columns and stores them with one vector store.
// Reduction chunk for lane group g = lane/16 at half kf of a 64-step:
// k = k0 + 16g + 8kf + (0..7), for both operands.
template <bool kOutBf16>
__global__ __launch_bounds__(256, 1) void gemm_fwd_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ codes,
    const int8_t* __restrict__ q8, const float* __restrict__ s2, const uint16_t* __restrict__ ulr,
    const uint16_t* __restrict__ Bt, int64_t M, int64_t N, int64_t K, int r,
    void* __restrict__ y, Codebook cb) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][kBM * kXS];
  __shared__ __attribute__((aligned(16))) uint16_t tabs[2][kBN * 16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 15, g = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.y * kBM, n0 = (int64_t)blockIdx.x * kBN;
  const int64_t KB = K / 64;

  u32x4_t xr[8];
  int qv = 0;
  float sv = 0.0f;
  u32x2_t cr[4];

  auto load = [&](int64_t kb) {
    const int64_t k0 = kb * 64;
    load_act_tile(x, M, K, m0, k0, true, tid, xr);
    const int64_t nt_row = n0 + tid;
    if (nt_row < N) {
      const int64_t bi = nt_row * KB + kb;
      qv = q8[bi];
      sv = s2[bi >> 8];
    } else {
      qv = 0;
      sv = 0.0f;
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int64_t n = n0 + 64 * w + 4 * c + t;
      cr[t] = n < N ? *reinterpret_cast<const u32x2_t*>(codes + ((n * K + k0) >> 1) + 8 * g)
                    : u32x2_t{0u, 0u};
    }
  };

  f32x4_t acc[16][4];
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[i][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  load(0);
  for (int64_t kb = 0; kb < KB; ++kb) {
    const int buf = (int)(kb & 1);
    u32x2_t cc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) cc[t] = cr[t];
    store_act_tile(xs[buf], tid, xr);
    build_table(cb, qv, sv, &tabs[buf][tid * 16]);
    __syncthreads();
    if (kb + 1 < KB) load(kb + 1);
    const uint16_t* xb = xs[buf];
    const uint16_t* tb = tabs[buf];
#pragma unroll
    for (int kf = 0; kf < 2; ++kf) {
      u32x4_t bfr[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        bfr[t] = lut8(kf ? cc[t].y : cc[t].x, tb + (64 * w + 4 * c + t) * 16);
#pragma unroll
      for (int mt = 0; mt < 16; ++mt) {
        const u32x4_t a =
            *reinterpret_cast<const u32x4_t*>(xb + (16 * mt + c) * kXS + 16 * g + 8 * kf);
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[mt][t] = mfma_16x16x32(a, bfr[t], acc[mt][t]);
      }
    }
  }

  // Adapter term as 2r extra reduction elements.
  const int r2 = 2 * r;
  for (int q = 0; q < r2 / 32; ++q) {
    const int jj = 32 * q + 8 * g;
    const int jb = jj % r;
    u32x4_t bfr[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int64_t n = n0 + 64 * w + 4 * c + t;
      bfr[t] = n < N ? *reinterpret_cast<const u32x4_t*>(Bt + n * r + jb) : zero4();
    }
#pragma unroll
    for (int mt = 0; mt < 16; ++mt) {
      const int64_t m = m0 + 16 * mt + c;
      const u32x4_t a = m < M ? *reinterpret_cast<const u32x4_t*>(ulr + m * r2 + jj) : zero4();
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[mt][t] = mfma_16x16x32(a, bfr[t], acc[mt][t]);
    }
  }

  const int64_t ncol = n0 + 64 * w + 4 * c;
  if (ncol < N) {
#pragma unroll
    for (int mt = 0; mt < 16; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t m = m0 + 16 * mt + 4 * g + v;
        if (m < M)
          store4<kOutBf16>(y, N, m, ncol, N, acc[mt][0][v], acc[mt][1][v], acc[mt][2][v],
                           acc[mt][3][v]);
      }
  }
}

// ----------------------------------------------------------------- backward dX
// dX[m,k] = sum_n dY[m,n] w_hat[n,k] + sum_j svlr[m,j] A[k, j mod r]
// The reduction runs over weight rows n, so the B operand needs 8 consecutive
// rows of one weight column per lane. Lane (c, g) reads 2 code bytes (4
// adjacent columns 4c..4c+3) from each of its 8 rows and so feeds 4 MFMAs:
// MFMA t takes column 4c + t. Every wave's 64 columns are one block of each
// weight row, so the 8 rows use 8 tables of the same block column.
template <bool kOutBf16>
__global__ __launch_bounds__(256, 1) void gemm_bwd_kernel(
    const uint16_t* __restrict__ dY, const uint8_t* __restrict__ codes,
    const int8_t* __restrict__ q8, const float* __restrict__ s2,
    const uint16_t* __restrict__ svlr, const uint16_t* __restrict__ A, int64_t M, int64_t N,
    int64_t K, int r, void* __restrict__ dX, Codebook cb) {
  __shared__ __attribute__((aligned(16))) uint16_t ys[2][kBM * kXS];
  __shared__ __attribute__((aligned(16))) uint16_t tabs[2][4 * 64 * 16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 15, g = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.y * kBM;
  const int64_t kt0 = (int64_t)blockIdx.x * kBN;
  const int64_t kbase = kt0 + 64 * w;  // this wave's first column (a block boundary)
  const bool wave_live = kbase < K;
  const int64_t KB = K / 64;
  const int64_t NS = (N + 63) / 64;
  const bool vec_ok = (N & 7) == 0;

  u32x4_t yr[8];
  int qv = 0;
  float sv = 0.0f;
  uint32_t cr[2][8];

  auto load = [&](int64_t ns) {
    const int64_t nb0 = ns * 64;
    load_act_tile(dY, M, N, m0, nb0, vec_ok, tid, yr);
    {
      const int64_t nn = nb0 + (tid & 63);
      const int64_t kb = kt0 / 64 + (tid >> 6);
      if (nn < N && kb < KB) {
        const int64_t bi = nn * KB + kb;
        qv = q8[bi];
        sv = s2[bi >> 8];
      } else {
        qv = 0;
        sv = 0.0f;
      }
    }
#pragma unroll
    for (int kf = 0; kf < 2; ++kf)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t nn = nb0 + 16 * g + 8 * kf + i;
        cr[kf][i] = (nn < N && wave_live)
                        ? (uint32_t)*reinterpret_cast<const uint16_t*>(
                              codes + ((nn * K + kbase + 4 * c) >> 1))
                        : 0u;
      }
  };

  f32x4_t acc[16][4];
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[i][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  load(0);
  for (int64_t ns = 0; ns < NS; ++ns) {
    const int buf = (int)(ns & 1);
    uint32_t cc[2][8];
#pragma unroll
    for (int kf = 0; kf < 2; ++kf)
#pragma unroll
      for (int i = 0; i < 8; ++i) cc[kf][i] = cr[kf][i];
    store_act_tile(ys[buf], tid, yr);
    build_table(cb, qv, sv, &tabs[buf][((tid >> 6) * 64 + (tid & 63)) * 16]);
    __syncthreads();
    if (ns + 1 < NS) load(ns + 1);
    const uint16_t* yb = ys[buf];
    const uint16_t* tb = tabs[buf] + w * 64 * 16;
#pragma unroll
    for (int kf = 0; kf < 2; ++kf) {
      u32x4_t bfr[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        uint32_t h[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          h[i] = tb[(16 * g + 8 * kf + i) * 16 + ((cc[kf][i] >> (4 * t)) & 15u)];
        bfr[t] = u32x4_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                         h[6] | (h[7] << 16)};
      }
#pragma unroll
      for (int mt = 0; mt < 16; ++mt) {
        const u32x4_t a =
            *reinterpret_cast<const u32x4_t*>(yb + (16 * mt + c) * kXS + 16 * g + 8 * kf);
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[mt][t] = mfma_16x16x32(a, bfr[t], acc[mt][t]);
      }
    }
  }

  const int r2 = 2 * r;
  for (int q = 0; q < r2 / 32; ++q) {
    const int jj = 32 * q + 8 * g;
    const int jb = jj % r;
    u32x4_t bfr[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int64_t kc = kbase + 4 * c + t;
      bfr[t] = kc < K ? *reinterpret_cast<const u32x4_t*>(A + kc * r + jb) : zero4();
    }
#pragma unroll
    for (int mt = 0; mt < 16; ++mt) {
      const int64_t m = m0 + 16 * mt + c;
      const u32x4_t a = m < M ? *reinterpret_cast<const u32x4_t*>(svlr + m * r2 + jj) : zero4();
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[mt][t] = mfma_16x16x32(a, bfr[t], acc[mt][t]);
    }
  }

  const int64_t kcol = kbase + 4 * c;
  if (wave_live) {
#pragma unroll
    for (int mt = 0; mt < 16; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t m = m0 + 16 * mt + 4 * g + v;
        if (m < M)
          store4<kOutBf16>(dX, K, m, kcol, K, acc[mt][0][v], acc[mt][1][v], acc[mt][2][v],
                           acc[mt][3][v]);
      }
  }
}

// ----------------------------------------------------------------- decode GEMV
// M <= 16. A workgroup covers 64 weight rows and a 512-wide slice of K; wave w
// owns rows n0 + 16w + c. The x slice [16 x 512] and the slice's 512 block
// tables live in LDS; the codes stream from HBM with 16-byte loads, all
// issued before any compute. MFMA rows are the (zero-padded) tokens.
constexpr int kGemvKC = 512;
constexpr int kGemvXS = kGemvKC + 8;

__global__ __launch_bounds__(256) void gemv_fwd_kernel(const uint16_t* __restrict__ x,
                                                       const uint8_t* __restrict__ codes,
                                                       const int8_t* __restrict__ q8,
                                                       const float* __restrict__ s2, int64_t M,
                                                       int64_t N, int64_t K,
                                                       float* __restrict__ partial, Codebook cb) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[16 * kGemvXS];
  __shared__ __attribute__((aligned(16))) uint16_t tabs[64 * (kGemvKC / 64) * 16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 15, g = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 64;
  const int split = blockIdx.y;
  const int64_t ks0 = (int64_t)split * kGemvKC;
  const int kc = (int)min((int64_t)kGemvKC, K - ks0);  // multiple of 64
  const int nblk = kc / 64;
  const int64_t KB = K / 64;
  const int64_t n = n0 + 16 * w + c;

  // Codes of this lane: row n, 4 x 32 nibbles at k = ks0 + 128*it + 32g.
  u32x4_t cw[kGemvKC / 128];
#pragma unroll
  for (int it = 0; it < kGemvKC / 128; ++it) {
    const int kk = 128 * it + 32 * g;
    cw[it] = (n < N && kk < kc)
                 ? *reinterpret_cast<const u32x4_t*>(codes + ((n * K + ks0 + kk) >> 1))
                 : zero4();
  }
  // x slice into LDS: 16 rows x kc columns; rows >= M are zero.
  for (int i = tid; i < 16 * (kGemvKC / 8); i += 256) {
    const int row = i / (kGemvKC / 8), col = (i % (kGemvKC / 8)) * 8;
    u32x4_t v = zero4();
    if (row < M && col < kc) v = *reinterpret_cast<const u32x4_t*>(x + row * K + ks0 + col);
    *reinterpret_cast<u32x4_t*>(&xs[row * kGemvXS + col]) = v;
  }
  // Tables: 64 rows x nblk blocks.
  for (int i = tid; i < 64 * (kGemvKC / 64); i += 256) {
    const int row = i & 63, blk = i >> 6;
    const int64_t nn = n0 + row;
    int qv = 0;
    float sv = 0.0f;
    if (nn < N && blk < nblk) {
      const int64_t bi = nn * KB + ks0 / 64 + blk;
      qv = q8[bi];
      sv = s2[bi >> 8];
    }
    build_table(cb, qv, sv, &tabs[(row * (kGemvKC / 64) + blk) * 16]);
  }
  __syncthreads();

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  const uint16_t* trow = &tabs[(16 * w + c) * (kGemvKC / 64) * 16];
#pragma unroll
  for (int it = 0; it < kGemvKC / 128; ++it) {
    const int kk = 128 * it + 32 * g;  // this lane's 32 k, all in one block
    if (128 * it < kc) {
      const uint16_t* tb = trow + (kk / 64) * 16;
      const uint32_t wd[4] = {cw[it].x, cw[it].y, cw[it].z, cw[it].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4_t b = lut8(wd[q], tb);
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(&xs[c * kGemvXS + kk + 8 * q]);
        acc = mfma_16x16x32(a, b, acc);
      }
    }
  }
  if (n < N) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * g + v;
      if (m < M) partial[((int64_t)split * M + m) * N + n] = acc[v];
    }
  }
}

// y[m,n] = sum_split partial + s * sum_j u[m,j] B[j,n]
template <bool kOutBf16>
__global__ __launch_bounds__(256) void gemv_finalize_kernel(const float* __restrict__ partial,
                                                            int splits,
                                                            const float* __restrict__ u,
                                                            const uint16_t* __restrict__ B,
                                                            int64_t M, int64_t N, int r, float s,
                                                            void* __restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= M * N) return;
  const int64_t m = i / N, n = i % N;
  float acc = 0.0f;
  for (int sp = 0; sp < splits; ++sp) acc += partial[((int64_t)sp * M + m) * N + n];
  float lo = 0.0f;
  for (int j = 0; j < r; ++j) lo = __builtin_fmaf(u[m * r + j], bf16_lo(B[(int64_t)j * N + n]), lo);
  const float v = __builtin_fmaf(s, lo, acc);
  if (kOutBf16)
    static_cast<uint16_t*>(y)[i] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
  else
    static_cast<float*>(y)[i] = v;
}

}  // namespace

hipError_t launch_gemm_fwd(const uint16_t* x, const uint8_t* codes, const int8_t* q8,
                           const float* s2, const uint16_t* ulr, const uint16_t* Bt, int64_t M,
                           int64_t N, int64_t K, int r, void* y, bool y_bf16, const Codebook& cb,
                           hipStream_t st) {
  const dim3 grid((unsigned)((N + kBN - 1) / kBN), (unsigned)((M + kBM - 1) / kBM));
  if (y_bf16)
    hipLaunchKernelGGL(gemm_fwd_kernel<true>, grid, dim3(256), 0, st, x, codes, q8, s2, ulr, Bt,
                       M, N, K, r, y, cb);
  else
    hipLaunchKernelGGL(gemm_fwd_kernel<false>, grid, dim3(256), 0, st, x, codes, q8, s2, ulr, Bt,
                       M, N, K, r, y, cb);
  return hipGetLastError();
}

hipError_t launch_gemm_bwd(const uint16_t* dY, const uint8_t* codes, const int8_t* q8,
                           const float* s2, const uint16_t* svlr, const uint16_t* A, int64_t M,
                           int64_t N, int64_t K, int r, void* dX, bool dx_bf16,
                           const Codebook& cb, hipStream_t st) {
  const dim3 grid((unsigned)((K + kBN - 1) / kBN), (unsigned)((M + kBM - 1) / kBM));
  if (dx_bf16)
    hipLaunchKernelGGL(gemm_bwd_kernel<true>, grid, dim3(256), 0, st, dY, codes, q8, s2, svlr, A,
                       M, N, K, r, dX, cb);
  else
    hipLaunchKernelGGL(gemm_bwd_kernel<false>, grid, dim3(256), 0, st, dY, codes, q8, s2, svlr, A,
                       M, N, K, r, dX, cb);
  return hipGetLastError();
}

int gemv_splits(int64_t K) { return (int)((K + kGemvKC - 1) / kGemvKC); }

hipError_t launch_gemv_fwd(const uint16_t* x, const uint8_t* codes, const int8_t* q8,
                           const float* s2, int64_t M, int64_t N, int64_t K, float* partial,
                           const Codebook& cb, hipStream_t st) {
  const dim3 grid((unsigned)((N + 63) / 64), (unsigned)gemv_splits(K));
  hipLaunchKernelGGL(gemv_fwd_kernel, grid, dim3(256), 0, st, x, codes, q8, s2, M, N, K, partial,
                     cb);
  return hipGetLastError();
}

hipError_t launch_gemv_finalize(const float* partial, int splits, const float* u,
                                const uint16_t* B, int64_t M, int64_t N, int r, float s, void* y,
                                bool y_bf16, hipStream_t st) {
  const int64_t total = M * N;
  const dim3 grid((unsigned)((total + 255) / 256));
  if (y_bf16)
    hipLaunchKernelGGL(gemv_finalize_kernel<true>, grid, dim3(256), 0, st, partial, splits, u, B,
                       M, N, r, s, y);
  else
    hipLaunchKernelGGL(gemv_finalize_kernel<false>, grid, dim3(256), 0, st, partial, splits, u, B,
                       M, N, r, s, y);
  return hipGetLastError();
}

}  // namespace qlora
