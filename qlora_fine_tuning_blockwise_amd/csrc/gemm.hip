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
//
// Workgroup tile 256 (M) x 256 (N), 4 waves; wave w owns output columns
// n0 + 64w + 4c + t (c = lane%16, t = 0..3): MFMA t of a row tile holds column
// 4c + t at lane column c, so each lane ends with 4 adjacent columns.
// Reduction chunk for lane group g = lane/16 in half kf of a 64-wide step:
// k = k0 + 16g + 8kf + (0..7), for both operands.
//
// The x tile (256 x 64 bf16 = 32 KB) arrives by direct-to-LDS DMA
// (global_load_lds_dwordx4: lane l of an instruction writes LDS bytes
// [16l, 16l+16) of that instruction's 1 KB window), two buffers. Rows are 128 B;
// 16-byte chunk c of row r sits at chunk slot c ^ (r & 7), so the 16 rows one
// A-fragment read touches spread over all 32 banks. Rows past M are clamped to
// row M-1 (their results are never stored).
constexpr int kTileBytes = 256 * 128;

struct FwdArgs {
  const uint16_t* x;
  const uint8_t* codes;
  const int8_t* q8;
  const float* s2;
  const uint16_t* ulr;
  const uint16_t* Bt;
  void* y;
  int64_t M, N, K;
  int r;
};

template <bool kOutBf16>
__global__ __launch_bounds__(256, 1) void gemm_fwd_kernel(FwdArgs p, Codebook cb) {
  __shared__ __attribute__((aligned(1024))) uint16_t xs0[kTileBytes / 2];
  __shared__ __attribute__((aligned(1024))) uint16_t xs1[kTileBytes / 2];
  __shared__ __attribute__((aligned(16))) uint16_t tab0[256 * 16];
  __shared__ __attribute__((aligned(16))) uint16_t tab1[256 * 16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 15, g = lane >> 4;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t m0 = (int64_t)blockIdx.y * kBM, n0 = (int64_t)blockIdx.x * kBN;
  const int64_t KB = K / 64;

  // DMA source offsets (elements, from the tile's first row) of the 8
  // instructions of this lane: slot (w*8+j)*64 + lane -> row (w*8+j)*8 + lane/8,
  // stored chunk lane%8, holding global chunk (lane%8) ^ ((lane/8)%8).
  const uint16_t* xrow0 = p.x + m0 * K;
  uint32_t xoff[8];
  {
    const int chunk = (lane & 7) ^ ((lane >> 3) & 7);
    const int64_t last = M - 1 - m0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int64_t row = (w * 8 + j) * 8 + (lane >> 3);
      row = row < last ? row : last;
      xoff[j] = (uint32_t)(row * K + chunk * 8);
    }
  }
  // Codes of the 4 weight rows of this lane (clamped into the matrix; rows
  // past N get an all-zero table below).
  const uint8_t* crow0 = p.codes + ((n0 * K) >> 1);
  uint32_t coff[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    int64_t row = 64 * w + 4 * c + t;
    row = n0 + row < N ? row : N - 1 - n0;
    coff[t] = (uint32_t)((row * K) >> 1) + 8 * g;
  }
  // Table row of this thread.
  const int64_t trow = n0 + tid;
  const bool trow_ok = trow < N;
  const int64_t tbase = (trow_ok ? trow : N - 1) * KB;

  auto issue_x = [&](int64_t kb, uint16_t* dst) {
    const uint16_t* src = xrow0 + kb * 64;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      __builtin_amdgcn_global_load_lds(src + xoff[j], dst + (w * 8 + j) * 512, 16, 0, 0);
  };
  auto load_codes = [&](int64_t kb, u32x2_t (&cr)[4]) {
    const uint8_t* src = crow0 + kb * 32;
#pragma unroll
    for (int t = 0; t < 4; ++t) cr[t] = *reinterpret_cast<const u32x2_t*>(src + coff[t]);
  };
  auto load_scale = [&](int64_t kb, int& qv, float& sv) {
    const int64_t bi = tbase + kb;
    qv = trow_ok ? (int)p.q8[bi] : 0;
    sv = p.s2[bi >> 8];
  };

  f32x4_t acc[16][4];
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[i][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Lane-constant LDS offsets (elements).
  const int a_off0 = c * 64 + (((2 * g) ^ (c & 7)) << 3);
  const int a_off1 = c * 64 + (((2 * g + 1) ^ (c & 7)) << 3);
  const int t_off = (64 * w + 4 * c) * 16;

  auto compute = [&](const uint16_t* xb, const uint16_t* tb, const u32x2_t (&cc)[4]) {
#pragma unroll
    for (int kf = 0; kf < 2; ++kf) {
      u32x4_t bfr[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) bfr[t] = lut8(kf ? cc[t].y : cc[t].x, tb + t_off + t * 16);
      const uint16_t* xa = xb + (kf ? a_off1 : a_off0);
#pragma unroll
      for (int mt = 0; mt < 16; ++mt) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(xa + mt * 1024);
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[mt][t] = mfma_16x16x32(a, bfr[t], acc[mt][t]);
      }
    }
  };

  // Prologue: tile 0 in flight, table 0 built, codes 0 and scales 1 loaded.
  u32x2_t cc[4], cn[4];
  int qv, qn;
  float sv, sn;
  issue_x(0, xs0);
  load_codes(0, cc);
  load_scale(0, qv, sv);
  build_table(cb, qv, sv, tab0 + tid * 16);
  if (KB > 1) load_scale(1, qn, sn);
  __syncthreads();

  // Steady state, two steps per trip so every LDS address is static.
  // Step kb computes from buffer kb&1 while the DMA for kb+1 fills the other
  // buffer and the loads for kb+1 / kb+2 land; one barrier per step.
  auto step = [&](int64_t kb, uint16_t* xcur, uint16_t* tcur, uint16_t* xnext, uint16_t* tnext) {
    const bool more = kb + 1 < KB;
    if (more) {
      issue_x(kb + 1, xnext);
      load_codes(kb + 1, cn);
    }
    int q2 = 0;
    float s2v = 0.0f;
    if (kb + 2 < KB) load_scale(kb + 2, q2, s2v);
    compute(xcur, tcur, cc);
    if (more) build_table(cb, qn, sn, tnext + tid * 16);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 4; ++t) cc[t] = cn[t];
    qn = q2;
    sn = s2v;
  };
  for (int64_t kb = 0; kb < KB; kb += 2) {
    step(kb, xs0, tab0, xs1, tab1);
    if (kb + 1 < KB) step(kb + 1, xs1, tab1, xs0, tab0);
  }

  // Adapter term as 2r extra reduction elements.
  const int r = p.r, r2 = 2 * r;
  for (int q = 0; q < r2 / 32; ++q) {
    const int jj = 32 * q + 8 * g;
    const int jb = jj % r;
    u32x4_t bfr[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int64_t n = n0 + 64 * w + 4 * c + t;
      bfr[t] = n < N ? *reinterpret_cast<const u32x4_t*>(p.Bt + n * r + jb) : zero4();
    }
#pragma unroll
    for (int mt = 0; mt < 16; ++mt) {
      const int64_t m = m0 + 16 * mt + c;
      const u32x4_t a = m < M ? *reinterpret_cast<const u32x4_t*>(p.ulr + m * r2 + jj) : zero4();
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
          store4<kOutBf16>(p.y, N, m, ncol, N, acc[mt][0][v], acc[mt][1][v], acc[mt][2][v],
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
__global__ __launch_bounds__(256, 1) void gemm_bwd_general_kernel(
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

// Fast backward path (N % 8 == 0). The dY tile (256 x 64 bf16) and the code
// tile (64 weight rows x the workgroup's 256 columns = 64 x 128 bytes) both
// arrive by direct-to-LDS DMA, double buffered. dY uses the same swizzled
// 128-byte rows as the forward x tile; rows past M are clamped to M-1 and
// chunks past N to the last in-range chunk (their weight rows get all-zero
// tables, so they add exact zeros). Lane (c, g) reads, for each of its 8 rows,
// the 2 code bytes of columns 4c..4c+3 of its wave's block from LDS.
struct BwdArgs {
  const uint16_t* dY;
  const uint8_t* codes;
  const int8_t* q8;
  const float* s2;
  const uint16_t* svlr;
  const uint16_t* A;
  void* dX;
  int64_t M, N, K;
  int r;
};

template <bool kOutBf16>
__global__ __launch_bounds__(256, 1) void gemm_bwd_kernel(BwdArgs p, Codebook cb) {
  __shared__ __attribute__((aligned(1024))) uint16_t ys0[kTileBytes / 2];
  __shared__ __attribute__((aligned(1024))) uint16_t ys1[kTileBytes / 2];
  __shared__ __attribute__((aligned(1024))) uint8_t cs0[64 * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t cs1[64 * 128];
  __shared__ __attribute__((aligned(16))) uint16_t tab0[256 * 16];
  __shared__ __attribute__((aligned(16))) uint16_t tab1[256 * 16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 15, g = lane >> 4;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t m0 = (int64_t)blockIdx.y * kBM;
  const int64_t kt0 = (int64_t)blockIdx.x * kBN;
  const int64_t KB = K / 64;
  const int64_t NS = (N + 63) / 64;
  const int64_t kbase = kt0 + 64 * w;
  const bool wave_live = kbase < K;

  // dY DMA: slot (w*8+j)*64 + lane -> row (w*8+j)*8 + lane/8, chunk slot lane%8
  // holding global chunk (lane%8) ^ ((lane/8)%8) of that row.
  const uint16_t* yrow0 = p.dY + m0 * N;
  uint32_t yoff[8];
  const int ychunk = (lane & 7) ^ ((lane >> 3) & 7);
  {
    const int64_t last = M - 1 - m0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int64_t row = (w * 8 + j) * 8 + (lane >> 3);
      row = row < last ? row : last;
      yoff[j] = (uint32_t)(row * N);
    }
  }
  // Code DMA: 512 chunks of 16 B per step; wave w moves chunks [128w, 128w+128):
  // instruction j, lane l -> chunk 128w + 64j + l -> row (128w+64j+l)/8, byte
  // column 16*((128w+64j+l)%8) of the workgroup's 128-byte span. Columns past
  // K are clamped to the last in-range chunk of the row (never used).
  uint32_t ccol[2];
  int crow[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int ch = 128 * w + 64 * j + lane;
    crow[j] = ch >> 3;
    int64_t col = kt0 / 2 + 16 * (ch & 7);
    if (col + 16 > K / 2) col = K / 2 - 16;
    ccol[j] = (uint32_t)col;
  }
  // Table of this thread: weight row nb0 + (tid & 63), block kt0/64 + (tid >> 6).
  const int64_t tblk = kt0 / 64 + (tid >> 6);
  const bool tblk_ok = tblk < KB;

  auto issue = [&](int64_t ns, uint16_t* ydst, uint8_t* cdst) {
    const int64_t nb0 = ns * 64;
    int64_t ccl = nb0 + ychunk * 8;
    if (ccl + 8 > N) ccl = N - 8;
    const uint16_t* ysrc = yrow0 + ccl;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      __builtin_amdgcn_global_load_lds(ysrc + yoff[j], ydst + (w * 8 + j) * 512, 16, 0, 0);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      int64_t row = nb0 + crow[j];
      row = row < N ? row : N - 1;
      __builtin_amdgcn_global_load_lds(p.codes + row * (K / 2) + ccol[j],
                                       cdst + (128 * w + 64 * j) * 16, 16, 0, 0);
    }
  };
  auto load_scale = [&](int64_t ns, int& qv, float& sv) {
    const int64_t nn = ns * 64 + (tid & 63);
    const bool ok = nn < N && tblk_ok;
    const int64_t bi = (nn < N ? nn : N - 1) * KB + (tblk_ok ? tblk : KB - 1);
    qv = ok ? (int)p.q8[bi] : 0;
    sv = p.s2[bi >> 8];
  };

  f32x4_t acc[16][4];
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[i][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int a_off0 = c * 64 + (((2 * g) ^ (c & 7)) << 3);
  const int a_off1 = c * 64 + (((2 * g + 1) ^ (c & 7)) << 3);
  const int tb_off = (w * 64 + 16 * g) * 16;       // table of this lane's first row
  const int cb_off = (16 * g) * 128 + w * 32 + 2 * c;  // code bytes of this lane's first row

  auto compute = [&](const uint16_t* yb, const uint8_t* cbuf, const uint16_t* tb) {
#pragma unroll
    for (int kf = 0; kf < 2; ++kf) {
      uint32_t cw[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        cw[i] = *reinterpret_cast<const uint16_t*>(cbuf + cb_off + (8 * kf + i) * 128);
      u32x4_t bfr[4];
      const uint16_t* trow = tb + tb_off + kf * 8 * 16;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        uint32_t h[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) h[i] = trow[i * 16 + ((cw[i] >> (4 * t)) & 15u)];
        bfr[t] = u32x4_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                         h[6] | (h[7] << 16)};
      }
      const uint16_t* ya = yb + (kf ? a_off1 : a_off0);
#pragma unroll
      for (int mt = 0; mt < 16; ++mt) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(ya + mt * 1024);
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[mt][t] = mfma_16x16x32(a, bfr[t], acc[mt][t]);
      }
    }
  };

  int qv, qn;
  float sv, sn;
  issue(0, ys0, cs0);
  load_scale(0, qv, sv);
  build_table(cb, qv, sv, tab0 + tid * 16);
  if (NS > 1) load_scale(1, qn, sn);
  __syncthreads();

  auto step = [&](int64_t ns, uint16_t* ycur, uint8_t* ccur, uint16_t* tcur, uint16_t* ynext,
                  uint8_t* cnext, uint16_t* tnext) {
    const bool more = ns + 1 < NS;
    if (more) issue(ns + 1, ynext, cnext);
    int q2 = 0;
    float s2v = 0.0f;
    if (ns + 2 < NS) load_scale(ns + 2, q2, s2v);
    compute(ycur, ccur, tcur);
    if (more) build_table(cb, qn, sn, tnext + tid * 16);
    __syncthreads();
    qn = q2;
    sn = s2v;
  };
  for (int64_t ns = 0; ns < NS; ns += 2) {
    step(ns, ys0, cs0, tab0, ys1, cs1, tab1);
    if (ns + 1 < NS) step(ns + 1, ys1, cs1, tab1, ys0, cs0, tab0);
  }

  const int r = p.r, r2 = 2 * r;
  for (int q = 0; q < r2 / 32; ++q) {
    const int jj = 32 * q + 8 * g;
    const int jb = jj % r;
    u32x4_t bfr[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int64_t kc = kbase + 4 * c + t;
      bfr[t] = kc < K ? *reinterpret_cast<const u32x4_t*>(p.A + kc * r + jb) : zero4();
    }
#pragma unroll
    for (int mt = 0; mt < 16; ++mt) {
      const int64_t m = m0 + 16 * mt + c;
      const u32x4_t a = m < M ? *reinterpret_cast<const u32x4_t*>(p.svlr + m * r2 + jj) : zero4();
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
          store4<kOutBf16>(p.dX, K, m, kcol, K, acc[mt][0][v], acc[mt][1][v], acc[mt][2][v],
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
  const FwdArgs a{x, codes, q8, s2, ulr, Bt, y, M, N, K, r};
  if (y_bf16)
    hipLaunchKernelGGL(gemm_fwd_kernel<true>, grid, dim3(256), 0, st, a, cb);
  else
    hipLaunchKernelGGL(gemm_fwd_kernel<false>, grid, dim3(256), 0, st, a, cb);
  return hipGetLastError();
}

hipError_t launch_gemm_bwd(const uint16_t* dY, const uint8_t* codes, const int8_t* q8,
                           const float* s2, const uint16_t* svlr, const uint16_t* A, int64_t M,
                           int64_t N, int64_t K, int r, void* dX, bool dx_bf16,
                           const Codebook& cb, hipStream_t st) {
  const dim3 grid((unsigned)((K + kBN - 1) / kBN), (unsigned)((M + kBM - 1) / kBM));
  if (N % 8 == 0) {
    const BwdArgs a{dY, codes, q8, s2, svlr, A, dX, M, N, K, r};
    if (dx_bf16)
      hipLaunchKernelGGL(gemm_bwd_kernel<true>, grid, dim3(256), 0, st, a, cb);
    else
      hipLaunchKernelGGL(gemm_bwd_kernel<false>, grid, dim3(256), 0, st, a, cb);
  } else if (dx_bf16) {
    hipLaunchKernelGGL(gemm_bwd_general_kernel<true>, grid, dim3(256), 0, st, dY, codes, q8, s2,
                       svlr, A, M, N, K, r, dX, cb);
  } else {
    hipLaunchKernelGGL(gemm_bwd_general_kernel<false>, grid, dim3(256), 0, st, dY, codes, q8, s2,
                       svlr, A, M, N, K, r, dX, cb);
  }
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
