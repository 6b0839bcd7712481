// Adapter-side kernels of the QLoRA layer on gfx950.
//
// [P1] "QLoRA" forward equation: the adapter path (alpha/r) B(Ax) beside the
// frozen base; [P2] s1 precision table (adapters and their gradients in bf16)
// and s3 "The Backward Pass Through Quantization" (only adapter gradients).
//
//  - transpose: bf16 matrix transpose (A -> A^T, B -> B^T) through LDS.
//  - lora_down: out[m,j] = sum_t X[m,t] P[j,t] with both operands contiguous
//    in t (u = x A with P = A^T; v = dY B^T with P = B), on MFMA. Work is
//    split over t across the 4 waves of a workgroup and across workgroups;
//    a finalize kernel sums the slices in a fixed order and also emits the
//    two-term bf16 split of s*out used by the tile kernels.
//  - colred: the adapter gradients dA = s x^T v and dB = s u^T dY reduce over
//    the token dimension M; each thread owns one column of X and accumulates
//    r fp32 products per element against rows of P staged in LDS. Slices of M
//    go to separate partial buffers, summed in a fixed order by a finalize.
#include "device.h"

namespace qlora {
namespace {

// ----------------------------------------------------------------- transpose
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t* __restrict__ in,
                                                        int64_t rows, int64_t cols,
                                                        uint16_t* __restrict__ out) {
  __shared__ uint16_t tile[32][33];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  const int64_t r0 = (int64_t)blockIdx.y * 32, c0 = (int64_t)blockIdx.x * 32;
#pragma unroll
  for (int i = 0; i < 32; i += 8) {
    const int64_t rr = r0 + ty + i, cc = c0 + tx;
    tile[ty + i][tx] = (rr < rows && cc < cols) ? in[rr * cols + cc] : (uint16_t)0;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 32; i += 8) {
    const int64_t cc = c0 + ty + i, rr = r0 + tx;
    if (cc < cols && rr < rows) out[cc * rows + rr] = tile[tx][ty + i];
  }
}

// ----------------------------------------------------------------- lora_down
constexpr int kDownTC = 1024;  // t per workgroup slice (256 per wave)

// 8 consecutive bf16 of row `row` at column t of a [rows, ld] matrix; zero
// outside. `vec_ok`: rows start 16-byte aligned.
__device__ __forceinline__ u32x4_t load8(const uint16_t* __restrict__ a, int64_t rows, int64_t ld,
                                         int64_t row, int64_t t, bool vec_ok) {
  if (row < rows && vec_ok && t + 8 <= ld)
    return *reinterpret_cast<const u32x4_t*>(a + row * ld + t);
  uint16_t h[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) h[j] = (row < rows && t + j < ld) ? a[row * ld + t + j] : (uint16_t)0;
  return u32x4_t{h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16),
                 h[4] | ((uint32_t)h[5] << 16), h[6] | ((uint32_t)h[7] << 16)};
}

// grid: (ceil(M/16), ceil(r/64), slices). part[slice][m][j].
__global__ __launch_bounds__(256) void lora_down_kernel(const uint16_t* __restrict__ X,
                                                        const uint16_t* __restrict__ P, int64_t M,
                                                        int64_t T, int r,
                                                        float* __restrict__ part) {
  __shared__ float red[4][16][65];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 15, g = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * 16;
  const int j0 = blockIdx.y * 64;
  const int ntile = min(4, (r - j0) / 16);
  const int slice = blockIdx.z;
  const int64_t tw0 = (int64_t)slice * kDownTC + (int64_t)w * (kDownTC / 4);
  const int64_t tw1 = min(T, tw0 + kDownTC / 4);
  const bool vec_ok = (T & 7) == 0;

  f32x4_t acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int64_t t = tw0; t < tw1; t += 32) {
    const u32x4_t a = load8(X, M, T, m0 + c, t + 8 * g, vec_ok);
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      if (jt < ntile) {
        const u32x4_t b = load8(P, r, T, j0 + 16 * jt + c, t + 8 * g, vec_ok);
        acc[jt] = mfma_16x16x32(a, b, acc[jt]);
      }
    }
  }
#pragma unroll
  for (int jt = 0; jt < 4; ++jt)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[w][4 * g + v][16 * jt + c] = acc[jt][v];
  __syncthreads();
  const int mm = tid >> 4, jq = tid & 15;
  const int64_t m = m0 + mm;
  if (m < M) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = 4 * jq + i;
      if (j < 16 * ntile) {
        const float s = red[0][mm][j] + red[1][mm][j] + red[2][mm][j] + red[3][mm][j];
        part[((int64_t)slice * M + m) * r + j0 + j] = s;
      }
    }
  }
}

// out[m][j] = sum over slices; lr[m][j] = bf16(s*out), lr[m][r+j] = bf16(s*out - hi).
__global__ __launch_bounds__(256) void lora_down_finalize_kernel(const float* __restrict__ part,
                                                                 int slices, int64_t M, int r,
                                                                 float s, float* __restrict__ out,
                                                                 uint16_t* __restrict__ lr) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= M * r) return;
  float v = 0.0f;
  for (int sl = 0; sl < slices; ++sl) v += part[(int64_t)sl * M * r + i];
  out[i] = v;
  if (lr) {
    const int64_t m = i / r;
    const int j = (int)(i % r);
    const float sv = s * v;
    const uint32_t hi = pack_bf16x2(sv, 0.0f) & 0xFFFFu;
    const float rem = sv - __uint_as_float(hi << 16);
    const uint32_t lo = pack_bf16x2(rem, 0.0f) & 0xFFFFu;
    lr[m * 2 * r + j] = (uint16_t)hi;
    lr[m * 2 * r + r + j] = (uint16_t)lo;
  }
}

// ----------------------------------------------------------------- colred
constexpr int kColMS = 256;  // rows of M per slice
constexpr int kColStage = 64;  // rows of P staged in LDS at a time

// part[slice][c][j0 + j] = sum_{m in slice} X[m][c] * P[m][j0 + j], j < RW.
// grid: (ceil(C/256), slices, r/RW).
template <int RW>
__global__ __launch_bounds__(256) void colred_kernel(const uint16_t* __restrict__ X,
                                                     const float* __restrict__ P, int64_t M,
                                                     int64_t C, int r, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) float ps[kColStage][RW];
  const int tid = threadIdx.x;
  const int64_t col = (int64_t)blockIdx.x * 256 + tid;
  const int slice = blockIdx.y;
  const int j0 = blockIdx.z * RW;
  const int64_t ms0 = (int64_t)slice * kColMS;
  const int64_t ms1 = min(M, ms0 + kColMS);
  float acc[RW];
#pragma unroll
  for (int j = 0; j < RW; ++j) acc[j] = 0.0f;
  for (int64_t mb = ms0; mb < ms1; mb += kColStage) {
    const int rows = (int)min((int64_t)kColStage, ms1 - mb);
    __syncthreads();
    for (int i = tid; i < kColStage * RW; i += 256) {
      const int rr = i / RW, jj = i % RW;
      ps[rr][jj] = rr < rows ? P[(mb + rr) * r + j0 + jj] : 0.0f;
    }
    __syncthreads();
    if (col < C) {
      for (int rr = 0; rr < rows; ++rr) {
        const float xv = bf16_lo(X[(mb + rr) * C + col]);
#pragma unroll
        for (int j = 0; j < RW; j += 4) {
          const f32x4_t p = *reinterpret_cast<const f32x4_t*>(&ps[rr][j]);
          acc[j] = __builtin_fmaf(xv, p.x, acc[j]);
          acc[j + 1] = __builtin_fmaf(xv, p.y, acc[j + 1]);
          acc[j + 2] = __builtin_fmaf(xv, p.z, acc[j + 2]);
          acc[j + 3] = __builtin_fmaf(xv, p.w, acc[j + 3]);
        }
      }
    }
  }
  if (col < C) {
    float* o = part + ((int64_t)slice * C + col) * r + j0;
#pragma unroll
    for (int j = 0; j < RW; j += 4)
      *reinterpret_cast<f32x4_t*>(o + j) = f32x4_t{acc[j], acc[j + 1], acc[j + 2], acc[j + 3]};
  }
}

// out = s * sum_slice part[slice][c][j], as [C, r] or transposed [r, C].
template <bool kBf16>
__global__ __launch_bounds__(256) void colred_finalize_kernel(const float* __restrict__ part,
                                                              int slices, int64_t C, int r,
                                                              float s, bool transpose_out,
                                                              void* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // index in [C, r] order
  if (i >= C * r) return;
  float v = 0.0f;
  for (int sl = 0; sl < slices; ++sl) v += part[(int64_t)sl * C * r + i];
  v *= s;
  const int64_t c = i / r;
  const int j = (int)(i % r);
  const int64_t o = transpose_out ? (int64_t)j * C + c : i;
  if (kBf16)
    static_cast<uint16_t*>(out)[o] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
  else
    static_cast<float*>(out)[o] = v;
}

__global__ __launch_bounds__(256) void zero_kernel(uint32_t* __restrict__ p, int64_t words) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < words) p[i] = 0u;
}

}  // namespace

hipError_t launch_transpose_bf16(const uint16_t* in, int64_t rows, int64_t cols, uint16_t* out,
                                 hipStream_t st) {
  const dim3 grid((unsigned)((cols + 31) / 32), (unsigned)((rows + 31) / 32));
  hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, st, in, rows, cols, out);
  return hipGetLastError();
}

int lora_down_slices(int64_t T) { return (int)((T + kDownTC - 1) / kDownTC); }

hipError_t launch_lora_down_parts(const uint16_t* X, const uint16_t* P, int64_t M, int64_t T,
                                  int r, float* part, hipStream_t st) {
  const dim3 grid((unsigned)((M + 15) / 16), (unsigned)((r + 63) / 64),
                  (unsigned)lora_down_slices(T));
  hipLaunchKernelGGL(lora_down_kernel, grid, dim3(256), 0, st, X, P, M, T, r, part);
  return hipGetLastError();
}

hipError_t launch_lora_down_finalize(const float* part, int slices, int64_t M, int r, float s,
                                     float* out, uint16_t* lr, hipStream_t st) {
  const dim3 grid((unsigned)((M * r + 255) / 256));
  hipLaunchKernelGGL(lora_down_finalize_kernel, grid, dim3(256), 0, st, part, slices, M, r, s, out,
                     lr);
  return hipGetLastError();
}

int colred_splits(int64_t M) { return (int)((M + kColMS - 1) / kColMS); }

hipError_t launch_colred(const uint16_t* X, const float* P, int64_t M, int64_t C, int r,
                         float* part, hipStream_t st) {
  const int slices = colred_splits(M);
  if (r % 64 == 0) {
    const dim3 grid((unsigned)((C + 255) / 256), (unsigned)slices, (unsigned)(r / 64));
    hipLaunchKernelGGL(colred_kernel<64>, grid, dim3(256), 0, st, X, P, M, C, r, part);
  } else {
    const dim3 grid((unsigned)((C + 255) / 256), (unsigned)slices, (unsigned)(r / 16));
    hipLaunchKernelGGL(colred_kernel<16>, grid, dim3(256), 0, st, X, P, M, C, r, part);
  }
  return hipGetLastError();
}

hipError_t launch_colred_finalize(const float* part, int splits, int64_t C, int r, float s,
                                  bool transpose_out, void* out, bool out_bf16, hipStream_t st) {
  const dim3 grid((unsigned)((C * r + 255) / 256));
  if (out_bf16)
    hipLaunchKernelGGL(colred_finalize_kernel<true>, grid, dim3(256), 0, st, part, splits, C, r, s,
                       transpose_out, out);
  else
    hipLaunchKernelGGL(colred_finalize_kernel<false>, grid, dim3(256), 0, st, part, splits, C, r,
                       s, transpose_out, out);
  return hipGetLastError();
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t st) {
  const int64_t words = (int64_t)(bytes / 4);
  if (words == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, st,
                     static_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

}  // namespace qlora
