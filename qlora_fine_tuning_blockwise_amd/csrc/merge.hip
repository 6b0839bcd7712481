// Merge of the trained adapter into the frozen base on gfx950.
//
// [P1] "QLoRA" bullets (merging is no longer clean: folding BA into a 4-bit W
// forces a re-quantization, a second rounding on top of training); [P4]
// "What it costs", "Merge friction" (the clean path merges into the 16-bit
// weights and quantizes once afterwards).
//
// out[n][k] = base[n][k] + s * d[n][k],  d[n][k] = sum_j A[k][j] B[j][n],
// in binary32 as written: d starts at +0 and takes the terms j = 0..r-1 in
// order, each product rounded, then each addition rounded (nothing fused:
// the build's -ffp-contract=off keeps the multiply and the add apart), then
// s*d rounds, then the sum with the base rounds. base is the dequantized NF4 weight
// (bf16(L[code] * c1_hat), widened) or the bf16 weight. Requantizing the
// result is the fp32 path of the quantizer.
//
// A thread takes the same 8 consecutive columns of four adjacent rows
// (K % 64 == 0, so they never straddle rows): every A value it unpacks feeds
// four FMAs, and A^T is read once per four rows. The adapter operands arrive transposed (A^T [r,K], B^T [N,r]) so
// that every load is a contiguous 16-byte vector: per 8 terms one load of
// B^T[n][j..j+7] per row and eight loads of A^T[j][k..k+7].
#include "device.h"

namespace qlora {
namespace {

constexpr int kRows = 4;  // rows per thread: each unpacked A value feeds kRows FMAs

template <bool kNf4Base>
__global__ __launch_bounds__(256) void merge_kernel(const uint8_t* __restrict__ codes,
                                                    const int8_t* __restrict__ q8,
                                                    const float* __restrict__ s2,
                                                    const uint16_t* __restrict__ wb, int64_t N,
                                                    int64_t K, const uint16_t* __restrict__ At,
                                                    const uint16_t* __restrict__ Bt, int r, float s,
                                                    float* __restrict__ out, Codebook cb) {
  __shared__ float lv[16];
  if (threadIdx.x < 16) lv[threadIdx.x] = cb.level[threadIdx.x];
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t kg = K / 8;
  if (t >= (N + kRows - 1) / kRows * kg) return;
  const int64_t n0 = kRows * (t / kg), k0 = 8 * (t % kg);
  int64_t nr[kRows];  // rows past N repeat the last row (computed, not stored)
#pragma unroll
  for (int rr = 0; rr < kRows; ++rr) nr[rr] = n0 + rr < N ? n0 + rr : N - 1;

  // The base's raw words are loaded now and decoded after the adapter sum,
  // so only they (not 8 floats per row) stay live across the sum.
  uint32_t braw[kRows][4];
  float bch[kRows];
#pragma unroll
  for (int rr = 0; rr < kRows; ++rr) {
    const int64_t e0 = nr[rr] * K + k0;
    if (kNf4Base) {
      braw[rr][0] = *reinterpret_cast<const uint32_t*>(codes + e0 / 2);
      const int64_t b = e0 / 64;
      bch[rr] = q8_value(q8[b], cb.dq_format) * s2[b >> 8];
    } else {
      const u32x4_t w = *reinterpret_cast<const u32x4_t*>(wb + e0);
      braw[rr][0] = w.x;
      braw[rr][1] = w.y;
      braw[rr][2] = w.z;
      braw[rr][3] = w.w;
      bch[rr] = 0.0f;
    }
  }

  float d[kRows][8];
#pragma unroll
  for (int rr = 0; rr < kRows; ++rr)
#pragma unroll
    for (int i = 0; i < 8; ++i) d[rr][i] = 0.0f;
  for (int j0 = 0; j0 < r; j0 += 8) {
    uint32_t bw[kRows][4];
#pragma unroll
    for (int rr = 0; rr < kRows; ++rr) {
      const u32x4_t bq = *reinterpret_cast<const u32x4_t*>(Bt + nr[rr] * r + j0);
      bw[rr][0] = bq.x;
      bw[rr][1] = bq.y;
      bw[rr][2] = bq.z;
      bw[rr][3] = bq.w;
    }
    u32x4_t a[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
      a[jj] = *reinterpret_cast<const u32x4_t*>(At + (int64_t)(j0 + jj) * K + k0);
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      float bj[kRows];
#pragma unroll
      for (int rr = 0; rr < kRows; ++rr)
        bj[rr] = (jj & 1) ? bf16_hi(bw[rr][jj >> 1]) : bf16_lo(bw[rr][jj >> 1]);
      const uint32_t av[4] = {a[jj].x, a[jj].y, a[jj].z, a[jj].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float ai = (i & 1) ? bf16_hi(av[i >> 1]) : bf16_lo(av[i >> 1]);
#pragma unroll
        for (int rr = 0; rr < kRows; ++rr) {
          const float prod = ai * bj[rr];
          d[rr][i] = d[rr][i] + prod;
        }
      }
    }
  }
#pragma unroll
  for (int rr = 0; rr < kRows; ++rr) {
    if (n0 + rr >= N) break;
    float base[8];
    if (kNf4Base) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        base[i] = bf16_lo(pack_bf16x2(lv[(braw[rr][0] >> (4 * i)) & 15u] * bch[rr], 0.0f));
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        base[2 * i] = bf16_lo(braw[rr][i]);
        base[2 * i + 1] = bf16_hi(braw[rr][i]);
      }
    }
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float tv = s * d[rr][i];
      o[i] = base[i] + tv;
    }
    float* dst = out + (n0 + rr) * K + k0;
    *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{o[0], o[1], o[2], o[3]};
    *reinterpret_cast<f32x4_t*>(dst + 4) = f32x4_t{o[4], o[5], o[6], o[7]};
  }
}

}  // namespace

hipError_t launch_merge(const uint8_t* codes, const int8_t* q8, const float* s2,
                        const uint16_t* W, int64_t N, int64_t K, const uint16_t* At,
                        const uint16_t* Bt, int r, float s, float* out, const Codebook& cb,
                        hipStream_t st) {
  const int64_t threads = (N + kRows - 1) / kRows * (K / 8);
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (W)
    hipLaunchKernelGGL(merge_kernel<false>, grid, dim3(256), 0, st, codes, q8, s2, W, N, K, At,
                       Bt, r, s, out, cb);
  else
    hipLaunchKernelGGL(merge_kernel<true>, grid, dim3(256), 0, st, codes, q8, s2, W, N, K, At,
                       Bt, r, s, out, cb);
  return hipGetLastError();
}

}  // namespace qlora
