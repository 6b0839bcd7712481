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
//    the token dimension M, on MFMA with a transposed read of x from LDS and
//    the fp32 rank-side operand split into two bf16 terms. Slices of M go to
//    separate partial buffers, summed in a fixed order by a finalize.
#include "device.h"

namespace qlora {
namespace {

// ----------------------------------------------------------------- transpose
// out[c][r'] = in[r'][c] for up to two bf16 matrices in one launch: the 1-D
// grid holds the 32 x 32 tiles of the first matrix, then those of the second.
struct TransposeJob {
  const uint16_t* in;
  uint16_t* out;
  int64_t rows, cols;
  unsigned tiles_c, tiles;  // tiles per tile row, tiles in all
};

__global__ __launch_bounds__(256) void transpose_kernel(TransposeJob j0, TransposeJob j1) {
  __shared__ uint16_t tile[32][33];
  const unsigned b = blockIdx.x;
  const bool second = b >= j0.tiles;
  const TransposeJob& j = second ? j1 : j0;
  const unsigned t = second ? b - j0.tiles : b;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  const int64_t r0 = (int64_t)(t / j.tiles_c) * 32, c0 = (int64_t)(t % j.tiles_c) * 32;
  const int64_t rows = j.rows, cols = j.cols;
#pragma unroll
  for (int i = 0; i < 32; i += 8) {
    const int64_t rr = r0 + ty + i, cc = c0 + tx;
    tile[ty + i][tx] = (rr < rows && cc < cols) ? j.in[rr * cols + cc] : (uint16_t)0;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 32; i += 8) {
    const int64_t cc = c0 + ty + i, rr = r0 + tx;
    if (cc < cols && rr < rows) j.out[cc * rows + rr] = tile[tx][ty + i];
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
// X is the large operand (read once from HBM): on the fast path each wave
// loads its 16 rows x 256 t with every instruction covering 2 rows x 512
// bytes (whole cache lines), stages them in LDS with a 528-byte row stride
// (the 16 lanes of each phase of a fragment read then hit 16 distinct bank
// groups) and reads the MFMA fragments back from there. P is small and
// stays in L2; its fragments load directly.
constexpr int kDownLd = 264;  // staged X row stride in bf16 (528 bytes)

__global__ __launch_bounds__(256) void lora_down_kernel(const uint16_t* __restrict__ X,
                                                        const uint16_t* __restrict__ P, int64_t M,
                                                        int64_t T, int r,
                                                        float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[4][16 * kDownLd];
  float(*red)[16][65] = reinterpret_cast<float(*)[16][65]>(&xs[0][0]);  // reused after the MFMAs
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
  if (vec_ok && (T & 31) == 0) {
    // Fixed trip count with every load issued first: indices are clamped into
    // the matrix and the steps past this wave's range (or rows past M) are
    // zeroed, which adds +0 to the same accumulation order.
    constexpr int kSteps = kDownTC / 4 / 32;
    {
      // Staging: instruction q loads rows 2q, 2q+1 of the wave's tile; lane
      // L takes 8 t at tw0 + 8*(L%32) of row 2q + L/32. Past T: zero.
      const int half = lane >> 5, ch = lane & 31;
      const int64_t t = tw0 + 8 * ch;
      const bool tok = t < tw1;
      const int64_t tc = tok ? t : T - 8;
      u32x4_t xv[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int64_t row = min(m0 + 2 * q + half, M - 1);
        xv[q] = *reinterpret_cast<const u32x4_t*>(X + row * T + tc);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q)
        *reinterpret_cast<u32x4_t*>(&xs[w][(2 * q + half) * kDownLd + 8 * ch]) =
            tok ? xv[q] : zero4();
    }
    // the wave reads back only what it wrote: no barrier, LDS keeps its order
    u32x4_t av[kSteps];
#pragma unroll
    for (int it = 0; it < kSteps; ++it)
      av[it] = *reinterpret_cast<const u32x4_t*>(&xs[w][c * kDownLd + 32 * it + 8 * g]);
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      if (jt < ntile) {
        u32x4_t bv[kSteps];
#pragma unroll
        for (int it = 0; it < kSteps; ++it) {
          const int64_t t = tw0 + 32 * it;
          const int64_t tc = t + 32 <= T ? t : T - 32;
          const u32x4_t v =
              *reinterpret_cast<const u32x4_t*>(P + (int64_t)(j0 + 16 * jt + c) * T + tc + 8 * g);
          bv[it] = t < tw1 ? v : zero4();
        }
#pragma unroll
        for (int it = 0; it < kSteps; ++it) acc[jt] = mfma_16x16x32(av[it], bv[it], acc[jt]);
      }
    }
  } else {
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
  }
  __syncthreads();  // every wave is done with its staged X before red reuses it
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

// Single-pass form for large M (enough 16-row tiles to fill the GPU) and
// r = 16 kTiles <= 32: one 8-wave workgroup per 16 rows walks the whole of T,
// wave w taking the 256-wide chunks w, w+8, .... Each iteration but the
// wave's last first issues the next chunk's loads, its P fragments (clamped
// into P: past T the staged X is zero, so they multiply zeros) and its X (two
// rows x 512 bytes per instruction), then stages the current X through LDS
// and runs the MFMAs on the current P fragments; both of the next chunk's
// operands stay in flight meanwhile. The eight waves' sums are added in a fixed order in LDS and the
// workgroup writes the outputs of lora_down_finalize (out, the row-major and
// transposed two-term splits of s*out, zero rows of lrT for M <= m < Mp)
// itself. Requires T % 32 == 0.
template <int kTiles>
__global__ __launch_bounds__(512) void lora_down_full_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ P, int64_t M, int64_t Mp,
    int64_t T, int r, float s, float* __restrict__ out, uint16_t* __restrict__ lr,
    uint16_t* __restrict__ lrT) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[8][16 * kDownLd];
  float(*red)[16][33] = reinterpret_cast<float(*)[16][33]>(&xs[0][0]);  // reused after the MFMAs
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 15, g = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * 16;
  constexpr int j0 = 0, ntile = kTiles;
  const int nchunks = (int)((T + 255) / 256);
  const int half = lane >> 5, ch = lane & 31;
  constexpr int kSteps = 8;

  auto load_chunk = [&](int ck, u32x4_t (&xv)[8]) {  // clamped: always in bounds
    const int64_t t = (int64_t)min(ck, nchunks - 1) * 256 + 8 * ch;
    const int64_t tc = t < T ? t : T - 8;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int64_t row = min(m0 + 2 * q + half, M - 1);
      xv[q] = *reinterpret_cast<const u32x4_t*>(X + row * T + tc);
    }
  };
  auto load_p = [&](int ck, u32x4_t (&bv)[kTiles][kSteps]) {  // clamped: always in bounds
    const int64_t tw0 = (int64_t)min(ck, nchunks - 1) * 256;
#pragma unroll
    for (int jt = 0; jt < kTiles; ++jt) {
      const int64_t prow = 16 * jt + c;
#pragma unroll
      for (int it = 0; it < kSteps; ++it) {
        const int64_t t = tw0 + 32 * it;
        const int64_t tc = t + 32 <= T ? t : T - 32;
        bv[jt][it] = *reinterpret_cast<const u32x4_t*>(P + prow * T + tc + 8 * g);
      }
    }
  };
  f32x4_t acc[kTiles];
#pragma unroll
  for (int i = 0; i < kTiles; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  u32x4_t xv[8], bv[kTiles][kSteps];
  // One chunk: stage the current X through LDS and run its MFMAs.
  auto compute = [&](int ck) {
    const int64_t tw0 = (int64_t)ck * 256, tw1 = min(T, tw0 + 256);
    const bool tok = tw0 + 8 * ch < tw1;
#pragma unroll
    for (int q = 0; q < 8; ++q)
      *reinterpret_cast<u32x4_t*>(&xs[w][(2 * q + half) * kDownLd + 8 * ch]) =
          tok ? xv[q] : zero4();
    u32x4_t av[kSteps];
#pragma unroll
    for (int it = 0; it < kSteps; ++it)
      av[it] = *reinterpret_cast<const u32x4_t*>(&xs[w][c * kDownLd + 32 * it + 8 * g]);
#pragma unroll
    for (int jt = 0; jt < kTiles; ++jt)
#pragma unroll
      for (int it = 0; it < kSteps; ++it) acc[jt] = mfma_16x16x32(av[it], bv[jt][it], acc[jt]);
  };
  if (w < nchunks) {
    load_p(w, bv);
    load_chunk(w, xv);
    int ck = w;
    // Every chunk but the wave's last: the next chunk's loads fly while this
    // one is used. The last chunk issues no loads, so nothing is left in
    // flight for the epilogue's barrier to wait on.
    for (; ck + 8 < nchunks; ck += 8) {
      u32x4_t bn[kTiles][kSteps], xn[8];
      load_p(ck + 8, bn);
      load_chunk(ck + 8, xn);
      compute(ck);
#pragma unroll
      for (int q = 0; q < 8; ++q) xv[q] = xn[q];
#pragma unroll
      for (int jt = 0; jt < kTiles; ++jt)
#pragma unroll
        for (int it = 0; it < kSteps; ++it) bv[jt][it] = bn[jt][it];
    }
    compute(ck);
  }
  __syncthreads();  // every wave is done with its staged X before red reuses it
#pragma unroll
  for (int jt = 0; jt < kTiles; ++jt)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[w][4 * g + v][16 * jt + c] = acc[jt][v];
  __syncthreads();
  const int mm = tid >> 5, j = tid & 31;
  const int64_t m = m0 + mm;
  if (j >= 16 * ntile) return;
  const int jg = j0 + j;
  if (m >= M) {
    if (lrT && m < Mp) {
      lrT[(int64_t)jg * Mp + m] = 0;
      lrT[(int64_t)(r + jg) * Mp + m] = 0;
    }
    return;
  }
  float v = red[0][mm][j];
#pragma unroll
  for (int ww = 1; ww < 8; ++ww) v += red[ww][mm][j];
  if (out) out[m * r + jg] = v;
  const float sv = s * v;
  const uint32_t hi = pack_bf16x2(sv, 0.0f) & 0xFFFFu;
  const float rem = sv - __uint_as_float(hi << 16);
  const uint32_t lo = pack_bf16x2(rem, 0.0f) & 0xFFFFu;
  if (lr) {
    lr[m * 2 * r + jg] = (uint16_t)hi;
    lr[m * 2 * r + r + jg] = (uint16_t)lo;
  }
  if (lrT) {
    lrT[(int64_t)jg * Mp + m] = (uint16_t)hi;
    lrT[(int64_t)(r + jg) * Mp + m] = (uint16_t)lo;
  }
}

// out[m][j] = sum over slices (skipped if out == NULL); with sv = s*out:
// lr[m][j] = bf16(sv), lr[m][r+j] = bf16(sv - hi) (row-major two-term split),
// lrT[j][m] = bf16(sv), lrT[r+j][m] = bf16(sv - hi) (transposed, row stride
// Mp, zero for M <= m < Mp). Either split output may be NULL. The grid
// covers Mp * r elements.
__global__ __launch_bounds__(256) void lora_down_finalize_kernel(
    const float* __restrict__ part, int slices, int64_t M, int64_t Mp, int r, float s,
    float* __restrict__ out, uint16_t* __restrict__ lr, uint16_t* __restrict__ lrT) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= Mp * r) return;
  const int64_t m = i / r;
  const int j = (int)(i % r);
  if (m >= M) {
    if (lrT) {
      lrT[(int64_t)j * Mp + m] = 0;
      lrT[(int64_t)(r + j) * Mp + m] = 0;
    }
    return;
  }
  const float v = sum_strided<8>(part + i, M * r, slices);
  if (out) out[i] = v;
  const float sv = s * v;
  const uint32_t hi = pack_bf16x2(sv, 0.0f) & 0xFFFFu;
  const float rem = sv - __uint_as_float(hi << 16);
  const uint32_t lo = pack_bf16x2(rem, 0.0f) & 0xFFFFu;
  if (lr) {
    lr[m * 2 * r + j] = (uint16_t)hi;
    lr[m * 2 * r + r + j] = (uint16_t)lo;
  }
  if (lrT) {
    lrT[(int64_t)j * Mp + m] = (uint16_t)hi;
    lrT[(int64_t)(r + j) * Mp + m] = (uint16_t)lo;
  }
}

// ----------------------------------------------------------------- colred
constexpr int kColMS = 512;   // rows of M per workgroup slice
constexpr int kColStep = 64;  // rows of M staged in LDS per step
constexpr int kColLdX = 66;   // x tile row stride in bf16 (132 B)
constexpr int kColLdP = 72;   // P tile row stride in bf16 (144 B)

// part[slice][c][j] = sum_{m in slice} X[m][c] * (PT[j][m] + PT[r + j][m]).
// X [M, C] bf16; PT [2r, Mp] bf16 holds a two-term split of the rank-side
// operand, transposed, zero for m >= M (Mp = M rounded up to 8).
// MFMA 16x16x32 with the reduction over m: the x operand needs 8 consecutive
// rows of one column per lane, read from an LDS tile with one 16-bit read per
// element (row stride 132 B puts the four 8-row groups of a read in distinct
// banks); the P operand is one 16-byte LDS read per lane.
// grid: (ceil(C/64), slices, ceil(r/64)); wave w owns columns 16w..16w+15.
// Two reductions over the same rows share a launch: workgroup columns
// 0 .. j0.tiles-1 take job j0, the rest job j1 (tiles = 0: no second job).
struct ColJob {
  const uint16_t* X;
  const uint16_t* PT;
  int64_t C;
  float* part;
  unsigned tiles;  // 64-column tiles
};

template <bool kVec>
__global__ __launch_bounds__(256) void colred_kernel(ColJob j0, ColJob j1, int64_t M, int64_t Mp,
                                                     int r) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[kColStep][kColLdX];
  __shared__ __attribute__((aligned(16))) uint16_t ps[2][64][kColLdP];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, i = lane & 15, g = lane >> 4;
  const bool second = blockIdx.x >= j0.tiles;
  const uint16_t* __restrict__ X = second ? j1.X : j0.X;
  const uint16_t* __restrict__ PT = second ? j1.PT : j0.PT;
  const int64_t C = second ? j1.C : j0.C;
  float* __restrict__ part = second ? j1.part : j0.part;
  const int64_t c0 = (int64_t)(second ? blockIdx.x - j0.tiles : blockIdx.x) * 64;
  const int slice = blockIdx.y;
  const int jt0 = blockIdx.z * 4;
  const int ntile = min(4, r / 16 - jt0);
  const int64_t ms0 = (int64_t)slice * kColMS;
  const int64_t ms1 = min(M, ms0 + kColMS);
  const int nsteps = (int)((ms1 - ms0 + kColStep - 1) / kColStep);

  // Staging roles: x rows (tid >> 3) and (tid >> 3) + 32, columns 8*(tid & 7);
  // P chunk q = tid + 256*t (t < ntile): tile row jr = q >> 3 of 16*ntile
  // hi rows then 16*ntile lo rows, m chunk 8*(q & 7).
  const int xr = tid >> 3, xq = tid & 7;
  const int64_t xc = c0 + 8 * xq;
  u32x4_t xv[2], pv[4];

  auto load_step = [&](int st) {
    const int64_t mb = ms0 + (int64_t)st * kColStep;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t m = mb + xr + 32 * h;
      if (kVec) {
        xv[h] = (m < ms1 && xc < C) ? *reinterpret_cast<const u32x4_t*>(X + m * C + xc) : zero4();
      } else {
        uint16_t e[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
          e[k] = (m < ms1 && xc + k < C) ? X[m * C + xc + k] : (uint16_t)0;
        xv[h] = u32x4_t{e[0] | ((uint32_t)e[1] << 16), e[2] | ((uint32_t)e[3] << 16),
                        e[4] | ((uint32_t)e[5] << 16), e[6] | ((uint32_t)e[7] << 16)};
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t < ntile) {
        const int q = tid + 256 * t;
        const int jr = q >> 3;  // 0 .. 32*ntile-1
        const int hl = jr >= 16 * ntile;
        const int j = 16 * jt0 + jr - hl * 16 * ntile;
        const int64_t m = mb + 8 * (q & 7);
        pv[t] = m < Mp ? *reinterpret_cast<const u32x4_t*>(PT + ((int64_t)hl * r + j) * Mp + m)
                       : zero4();
      }
    }
  };
  auto store_step = [&]() {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t* d = reinterpret_cast<uint32_t*>(&xs[xr + 32 * h][8 * xq]);
      d[0] = xv[h].x;
      d[1] = xv[h].y;
      d[2] = xv[h].z;
      d[3] = xv[h].w;
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t < ntile) {
        const int q = tid + 256 * t;
        const int jr = q >> 3;
        const int hl = jr >= 16 * ntile;
        *reinterpret_cast<u32x4_t*>(&ps[hl][jr - hl * 16 * ntile][8 * (q & 7)]) = pv[t];
      }
    }
  };

  f32x4_t acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (nsteps > 0) load_step(0);
  for (int st = 0; st < nsteps; ++st) {
    __syncthreads();  // previous step's reads are done
    store_step();
    if (st + 1 < nsteps) load_step(st + 1);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint16_t* xb = &xs[32 * ks + 8 * g][16 * w + i];
      u32x4_t a;
      a.x = (uint32_t)xb[0 * kColLdX] | ((uint32_t)xb[1 * kColLdX] << 16);
      a.y = (uint32_t)xb[2 * kColLdX] | ((uint32_t)xb[3 * kColLdX] << 16);
      a.z = (uint32_t)xb[4 * kColLdX] | ((uint32_t)xb[5 * kColLdX] << 16);
      a.w = (uint32_t)xb[6 * kColLdX] | ((uint32_t)xb[7 * kColLdX] << 16);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (t < ntile) {
          const u32x4_t bh = *reinterpret_cast<const u32x4_t*>(&ps[0][16 * t + i][32 * ks + 8 * g]);
          const u32x4_t bl = *reinterpret_cast<const u32x4_t*>(&ps[1][16 * t + i][32 * ks + 8 * g]);
          acc[t] = mfma_16x16x32(a, bh, acc[t]);
          acc[t] = mfma_16x16x32(a, bl, acc[t]);
        }
      }
    }
  }
  // acc[t][v] = sum for column c0 + 16w + 4g + v and rank index 16(jt0 + t) + i.
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t c = c0 + 16 * w + 4 * g + v;
    if (c < C) {
      float* o = part + ((int64_t)slice * C + c) * r + 16 * jt0 + i;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (t < ntile) o[16 * t] = acc[t][v];
    }
  }
}

// out = s * sum_slice part[slice][c][j], as [C, r] or transposed [r, C];
// workgroups 0 .. j0.blocks-1 take job j0, the rest job j1.
struct FinJob {
  const float* part;
  int64_t C;
  void* out;
  bool transpose_out;
  unsigned blocks;  // 256-element blocks
};

template <bool kBf16>
__global__ __launch_bounds__(256) void colred_finalize_kernel(FinJob j0, FinJob j1, int slices,
                                                              int r, float s) {
  const bool second = blockIdx.x >= j0.blocks;
  const float* __restrict__ part = second ? j1.part : j0.part;
  const int64_t C = second ? j1.C : j0.C;
  void* __restrict__ out = second ? j1.out : j0.out;
  const bool transpose_out = second ? j1.transpose_out : j0.transpose_out;
  const int64_t i = (int64_t)(second ? blockIdx.x - j0.blocks : blockIdx.x) * 256 +
                    threadIdx.x;  // index in [C, r] order
  if (i >= C * r) return;
  const float v = s * sum_strided<8>(part + i, C * r, slices);
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

namespace {
TransposeJob transpose_job(const uint16_t* in, int64_t rows, int64_t cols, uint16_t* out) {
  const unsigned tc = (unsigned)((cols + 31) / 32), tr = (unsigned)((rows + 31) / 32);
  return TransposeJob{in, out, rows, cols, tc, in ? tc * tr : 0u};
}
}  // namespace

hipError_t launch_transpose_bf16(const uint16_t* in, int64_t rows, int64_t cols, uint16_t* out,
                                 hipStream_t st) {
  return launch_transpose2_bf16(in, rows, cols, out, nullptr, 0, 0, nullptr, st);
}

hipError_t launch_transpose2_bf16(const uint16_t* in0, int64_t rows0, int64_t cols0,
                                  uint16_t* out0, const uint16_t* in1, int64_t rows1,
                                  int64_t cols1, uint16_t* out1, hipStream_t st) {
  const TransposeJob j0 = transpose_job(in0, rows0, cols0, out0);
  const TransposeJob j1 = transpose_job(in1, rows1, cols1, out1);
  const unsigned tiles = j0.tiles + j1.tiles;
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_kernel, dim3(tiles), dim3(256), 0, st, j0, j1);
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
                                     float* out, uint16_t* lr, uint16_t* lrT, hipStream_t st) {
  const int64_t Mp = (M + 7) & ~(int64_t)7;
  const dim3 grid((unsigned)((Mp * r + 255) / 256));
  hipLaunchKernelGGL(lora_down_finalize_kernel, grid, dim3(256), 0, st, part, slices, M, Mp, r, s,
                     out, lr, lrT);
  return hipGetLastError();
}

bool lora_down_full_ok(int64_t M, int64_t T, int r) {
  return M >= 2048 && T % 32 == 0 && (r == 16 || r == 32);
}

hipError_t launch_lora_down_full(const uint16_t* X, const uint16_t* P, int64_t M, int64_t T,
                                 int r, float s, float* out, uint16_t* lr, uint16_t* lrT,
                                 hipStream_t st) {
  const int64_t Mp = (M + 7) & ~(int64_t)7;
  const dim3 grid((unsigned)((M + 15) / 16));
  if (r == 16)
    hipLaunchKernelGGL(lora_down_full_kernel<1>, grid, dim3(512), 0, st, X, P, M, Mp, T, r, s, out,
                       lr, lrT);
  else if (r == 32)
    hipLaunchKernelGGL(lora_down_full_kernel<2>, grid, dim3(512), 0, st, X, P, M, Mp, T, r, s, out,
                       lr, lrT);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

int colred_splits(int64_t M) { return (int)((M + kColMS - 1) / kColMS); }

hipError_t launch_colred(const uint16_t* X, const uint16_t* PT, int64_t M, int64_t C, int r,
                         float* part, hipStream_t st) {
  return launch_colred2(X, PT, C, part, nullptr, nullptr, 0, nullptr, M, r, st);
}

hipError_t launch_colred2(const uint16_t* X0, const uint16_t* PT0, int64_t C0, float* part0,
                          const uint16_t* X1, const uint16_t* PT1, int64_t C1, float* part1,
                          int64_t M, int r, hipStream_t st) {
  const int64_t Mp = (M + 7) & ~(int64_t)7;
  const ColJob j0{X0, PT0, C0, part0, (unsigned)((C0 + 63) / 64)};
  const ColJob j1{X1, PT1, C1, part1, X1 ? (unsigned)((C1 + 63) / 64) : 0u};
  const dim3 grid(j0.tiles + j1.tiles, (unsigned)colred_splits(M), (unsigned)((r / 16 + 3) / 4));
  if (C0 % 8 == 0 && (!X1 || C1 % 8 == 0))
    hipLaunchKernelGGL(colred_kernel<true>, grid, dim3(256), 0, st, j0, j1, M, Mp, r);
  else
    hipLaunchKernelGGL(colred_kernel<false>, grid, dim3(256), 0, st, j0, j1, M, Mp, r);
  return hipGetLastError();
}

hipError_t launch_colred_finalize(const float* part, int splits, int64_t C, int r, float s,
                                  bool transpose_out, void* out, bool out_bf16, hipStream_t st) {
  return launch_colred_finalize2(part, C, transpose_out, out, nullptr, 0, false, nullptr, splits,
                                 r, s, out_bf16, st);
}

hipError_t launch_colred_finalize2(const float* part0, int64_t C0, bool transpose_out0,
                                   void* out0, const float* part1, int64_t C1,
                                   bool transpose_out1, void* out1, int splits, int r, float s,
                                   bool out_bf16, hipStream_t st) {
  const FinJob j0{part0, C0, out0, transpose_out0, (unsigned)((C0 * r + 255) / 256)};
  const FinJob j1{part1, C1, out1, transpose_out1, part1 ? (unsigned)((C1 * r + 255) / 256) : 0u};
  const dim3 grid(j0.blocks + j1.blocks);
  if (out_bf16)
    hipLaunchKernelGGL(colred_finalize_kernel<true>, grid, dim3(256), 0, st, j0, j1, splits, r, s);
  else
    hipLaunchKernelGGL(colred_finalize_kernel<false>, grid, dim3(256), 0, st, j0, j1, splits, r,
                       s);
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
