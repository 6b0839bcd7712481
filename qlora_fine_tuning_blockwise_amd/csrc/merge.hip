// Merge of the trained adapter into the frozen base on gfx950.
//
// [P1] "QLoRA" bullets (merging is no longer clean: folding BA into a 4-bit W
// forces a re-quantization, a second rounding on top of training); [P4]
// "What it costs", "Merge friction" (the clean path merges into the 16-bit
// weights and quantizes once afterwards).
//
// out[n][k] = base[n][k] + s * d[n][k],  d[n][k] = sum_j A[k][j] B[j][n],
// in binary32: d starts at +0 and takes the terms j = 0..r-1 in order, each
// as one fused multiply-add (one rounding per step), then s*d rounds, then
// the sum with the base rounds. base is the dequantized NF4 weight
// (bf16(L[code] * c1_hat), widened) or the bf16 weight. Requantizing the
// result is the fp32 path of the quantizer.
//
// A thread takes the same 8 consecutive columns of two adjacent rows
// (K % 64 == 0, so they never straddle rows): every A value it unpacks feeds
// two FMAs. The adapter operands arrive transposed (A^T [r,K], B^T [N,r]) so
// that every load is a contiguous 16-byte vector: per 8 terms one load of
// B^T[n][j..j+7] per row and eight loads of A^T[j][k..k+7].
#include "device.h"

namespace qlora {
namespace {

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
  if (t >= (N + 1) / 2 * kg) return;
  const int64_t n0 = 2 * (t / kg), k0 = 8 * (t % kg);
  const bool two = n0 + 1 < N;  // the second row exists
  const int64_t n1 = two ? n0 + 1 : n0;

  float base[2][8];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int64_t e0 = (rr ? n1 : n0) * K + k0;
    if (kNf4Base) {
      const uint32_t cw = *reinterpret_cast<const uint32_t*>(codes + e0 / 2);
      const int64_t b = e0 / 64;
      const float ch = q8_value(q8[b], cb.dq_format) * s2[b >> 8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        base[rr][i] = bf16_lo(pack_bf16x2(lv[(cw >> (4 * i)) & 15u] * ch, 0.0f));
    } else {
      const u32x4_t w = *reinterpret_cast<const u32x4_t*>(wb + e0);
      const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        base[rr][2 * i] = bf16_lo(wv[i]);
        base[rr][2 * i + 1] = bf16_hi(wv[i]);
      }
    }
  }

  float d[2][8];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr)
#pragma unroll
    for (int i = 0; i < 8; ++i) d[rr][i] = 0.0f;
  for (int j0 = 0; j0 < r; j0 += 8) {
    const u32x4_t bq0 = *reinterpret_cast<const u32x4_t*>(Bt + n0 * r + j0);
    const u32x4_t bq1 = *reinterpret_cast<const u32x4_t*>(Bt + n1 * r + j0);
    const uint32_t bw[2][4] = {{bq0.x, bq0.y, bq0.z, bq0.w}, {bq1.x, bq1.y, bq1.z, bq1.w}};
    u32x4_t a[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
      a[jj] = *reinterpret_cast<const u32x4_t*>(At + (int64_t)(j0 + jj) * K + k0);
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const float b0 = (jj & 1) ? bf16_hi(bw[0][jj >> 1]) : bf16_lo(bw[0][jj >> 1]);
      const float b1 = (jj & 1) ? bf16_hi(bw[1][jj >> 1]) : bf16_lo(bw[1][jj >> 1]);
      const uint32_t av[4] = {a[jj].x, a[jj].y, a[jj].z, a[jj].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float ai = (i & 1) ? bf16_hi(av[i >> 1]) : bf16_lo(av[i >> 1]);
        d[0][i] = __builtin_fmaf(ai, b0, d[0][i]);
        d[1][i] = __builtin_fmaf(ai, b1, d[1][i]);
      }
    }
  }
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    if (rr == 1 && !two) break;
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float tv = s * d[rr][i];
      o[i] = base[rr][i] + tv;
    }
    float* dst = out + (rr ? n1 : n0) * K + k0;
    *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{o[0], o[1], o[2], o[3]};
    *reinterpret_cast<f32x4_t*>(dst + 4) = f32x4_t{o[4], o[5], o[6], o[7]};
  }
}

}  // namespace

hipError_t launch_merge(const uint8_t* codes, const int8_t* q8, const float* s2,
                        const uint16_t* W, int64_t N, int64_t K, const uint16_t* At,
                        const uint16_t* Bt, int r, float s, float* out, const Codebook& cb,
                        hipStream_t st) {
  const int64_t threads = (N + 1) / 2 * (K / 8);
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
