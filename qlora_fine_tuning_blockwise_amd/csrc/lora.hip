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
// r = 16, 32 or 64: one 8-wave workgroup per 16 rows and 16 kTiles rank
// columns (blockIdx.y: the 32-wide rank block at r = 64) walks the whole of T,
// wave w taking the 256-wide chunks w, w+8, .... Each iteration but the
// wave's last first issues the next chunk's loads, its P fragments (clamped
// into P: past T the staged X is zero, so they multiply zeros) and its X (two
// rows x 512 bytes per instruction), then stages the current X through LDS
// and runs the MFMAs on the current P fragments; both of the next chunk's
// operands stay in flight meanwhile. The eight waves' sums are added in a fixed order in LDS and the
// workgroup writes the outputs of lora_down_finalize (out, the row-major and
// transposed two-term splits of s*out, zero rows of lrT for M <= m < Mp)
// itself. With u2T != NULL the same epilogue also writes the transposed
// two-term split of s*u2 (an fp32 [M, r] matrix the caller already holds,
// as lora_down_finalize with one slice would) for its rows and rank
// columns. Requires T % 32 == 0. At r = 64 the two rank blocks of a row
// block read the same X rows at about the same time, from the same XCD
// (their workgroup ids differ by a multiple of 8), so the second read is
// served by that XCD's L2.
template <int kTiles>
__global__ __launch_bounds__(512) void lora_down_full_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ P, int64_t M, int64_t Mp,
    int64_t T, int r, float s, float* __restrict__ out, uint16_t* __restrict__ lr,
    uint16_t* __restrict__ lrT, const float* __restrict__ u2, uint16_t* __restrict__ u2T) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[8][16 * kDownLd];
  float(*red)[16][33] = reinterpret_cast<float(*)[16][33]>(&xs[0][0]);  // reused after the MFMAs
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 15, g = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * 16;
  const int j0 = 16 * kTiles * (int)blockIdx.y;
  constexpr int ntile = kTiles;
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
      const int64_t prow = j0 + 16 * jt + c;
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
    if (u2T && m < Mp) {
      u2T[(int64_t)jg * Mp + m] = 0;
      u2T[(int64_t)(r + jg) * Mp + m] = 0;
    }
    return;
  }
  if (u2T) {
    const float su = s * u2[m * r + jg];
    const uint32_t uh = pack_bf16x2(su, 0.0f) & 0xFFFFu;
    const uint32_t ul = pack_bf16x2(su - __uint_as_float(uh << 16), 0.0f) & 0xFFFFu;
    u2T[(int64_t)jg * Mp + m] = (uint16_t)uh;
    u2T[(int64_t)(r + jg) * Mp + m] = (uint16_t)ul;
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

// Tiled form for large M and ranks that are multiples of 32 (from 64 on),
// where the 16-row kernel above re-reads the whole rank-side operand from L2
// for every 16 rows (at r = 64 four times the activation bytes): a
// 256-thread workgroup owns 128 rows x 64 rank columns of one 512-wide slice
// of T. Its slice of P [64 rows x 512 t] is staged once in LDS and read by
// all four waves (row stride 520 elements: consecutive rows start 4 banks
// apart); wave w owns rows 32w .. 32w+31 and loads its activation fragments
// straight from X (row i, 8 consecutive t per lane: two lanes per row cover
// 32 bytes per instruction, and the four instructions of each 64-t group
// cover whole 128-byte lines). All of a workgroup's loads are issued before
// it waits (one round trip to memory). v_mfma_f32_32x32x16_bf16, two
// 32-column tiles; the slice's partial sums go to part[slice][m][j] for the
// finalize, which adds the slices in order. Requires T % 8 == 0; reads past
// T read zeros.
constexpr int kTileT = 512;   // t per slice
constexpr int kTileLd = 520;  // staged P row stride (bf16)

__global__ __launch_bounds__(256) void lora_down_tile_kernel(const uint16_t* __restrict__ X,
                                                             const uint16_t* __restrict__ P,
                                                             int64_t M, int64_t T, int r,
                                                             float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint16_t ps[64 * kTileLd];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, i = lane & 31, h = lane >> 5;
  const int64_t m0 = (int64_t)blockIdx.x * 128 + 32 * w;
  const int j0 = blockIdx.y * 64;
  const int ncol = min(2, (r - j0) / 32);  // 32-column tiles of this workgroup
  const int slice = blockIdx.z;
  const int64_t t0 = (int64_t)slice * kTileT;
  const int64_t tend = min(T, t0 + kTileT);

  // Every load is issued first, so the workgroup waits for memory once:
  // the P slice (rows j0 .. j0+63; rows past r read row r-1, multiplied by
  // nothing that is stored; t past T read zero), then the wave's 32
  // activation fragments (row m0 + i clamped to M-1, t = t0 + 16 st + 8h).
  u32x4_t pv[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int e = q * 256 + tid;  // 16-byte chunk: row e/64, t 8*(e%64)
    const int64_t prow = min(j0 + (e >> 6), r - 1);
    const int64_t t = t0 + 8 * (e & 63);
    pv[q] = t < tend ? *reinterpret_cast<const u32x4_t*>(P + prow * T + t) : zero4();
  }
  const int64_t arow = min(m0 + i, M - 1);
  const uint16_t* xr = X + arow * T;
  u32x4_t xv[32];
#pragma unroll
  for (int st = 0; st < 32; ++st) {
    const int64_t t = t0 + 16 * st + 8 * h;
    xv[st] = t < tend ? *reinterpret_cast<const u32x4_t*>(xr + t) : zero4();
  }
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int e = q * 256 + tid;
    *reinterpret_cast<u32x4_t*>(&ps[(e >> 6) * kTileLd + 8 * (e & 63)]) = pv[q];
  }
  f32x16_t acc[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[ct][e] = 0.0f;
  __syncthreads();  // P staged
#pragma unroll
  for (int st = 0; st < 32; ++st) {
    const int tt = 16 * st + 8 * h;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      if (ct < ncol) {
        const u32x4_t b = *reinterpret_cast<const u32x4_t*>(&ps[(32 * ct + i) * kTileLd + tt]);
        acc[ct] = mfma_32x32x16(xv[st], b, acc[ct]);
      }
    }
  }
  // element e of tile ct: row 8(e/4) + 4h + e%4 of the wave's 32, column
  // 32ct + i of the workgroup's 64
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    if (ct < ncol) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t m = m0 + 8 * (e >> 2) + 4 * h + (e & 3);
        if (m < M) part[((int64_t)slice * M + m) * r + j0 + 32 * ct + i] = acc[ct][e];
      }
    }
  }
}

// Streaming form for large M and ranks that are multiples of 32: a 256-thread
// workgroup owns 128 rows x 64 rank columns of one slice of T and walks the
// slice in 64-wide chunks. Each chunk of X (128 rows) and of P (64 rows) is
// loaded as whole 128-byte lines (eight lanes a row, one 16-byte piece
// each), staged in LDS (row stride 144 bytes: the 16 lanes of each phase of
// a fragment read hit 16 distinct bank groups) and consumed by
// v_mfma_f32_32x32x16_bf16, wave w taking rows 32w .. 32w+31 and both
// 32-column tiles. Two LDS buffers alternate, and the loads of the next two
// chunks are in flight while one chunk is computed, so the workgroup keeps
// about 48 KB of reads outstanding. Every load is clamped into the matrices
// and every stage is unconditional: positions past the slice are stored as
// zeros (a chunk past the end adds +0), so no branch separates a load from
// its wait. part[slice][m][j] as above. Requires T % 8 == 0 and r % 32 == 0.
constexpr int kStrT = 64;   // t per chunk
constexpr int kStrLd = 72;  // staged row stride (bf16)

__global__ __launch_bounds__(256) void lora_down_stream_kernel(const uint16_t* __restrict__ X,
                                                               const uint16_t* __restrict__ P,
                                                               int64_t M, int64_t T, int r,
                                                               int64_t tslice,
                                                               float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][128 * kStrLd];
  __shared__ __attribute__((aligned(16))) uint16_t ps[2][64 * kStrLd];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, i = lane & 31, h = lane >> 5;
  const int64_t m0 = (int64_t)blockIdx.x * 128;
  const int j0 = blockIdx.y * 64;
  const int ncol = min(2, (r - j0) / 32);  // 32-column tiles of this workgroup
  const int slice = blockIdx.z;
  const int64_t t0 = (int64_t)slice * tslice;
  const int64_t t1 = min(T, t0 + tslice);
  const int npairs = (int)((t1 - t0 + 2 * kStrT - 1) / (2 * kStrT));
  // Staging roles: rows srow + 32q (X: q < 4, P: q < 2), 8 t at 8*sc.
  const int srow = tid >> 3, sc = tid & 7;
  int64_t xoff[4], poff[2];
#pragma unroll
  for (int q = 0; q < 4; ++q) xoff[q] = min(m0 + srow + 32 * q, M - 1) * T;
#pragma unroll
  for (int q = 0; q < 2; ++q) poff[q] = (int64_t)min(j0 + srow + 32 * q, r - 1) * T;

  auto load = [&](int c, u32x4_t (&xv)[4], u32x4_t (&pv)[2]) {
    const int64_t t = t0 + (int64_t)c * kStrT + 8 * sc;
    const int64_t tc = t < t1 ? t : t1 - 8;  // t1 - t0 >= 8: T % 8 == 0
#pragma unroll
    for (int q = 0; q < 4; ++q) xv[q] = *reinterpret_cast<const u32x4_t*>(X + xoff[q] + tc);
#pragma unroll
    for (int q = 0; q < 2; ++q) pv[q] = *reinterpret_cast<const u32x4_t*>(P + poff[q] + tc);
  };
  auto stage = [&](int c, uint16_t* xb, uint16_t* pb, const u32x4_t (&xv)[4],
                   const u32x4_t (&pv)[2]) {
    const bool ok = t0 + (int64_t)c * kStrT + 8 * sc < t1;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<u32x4_t*>(&xb[(srow + 32 * q) * kStrLd + 8 * sc]) = ok ? xv[q] : zero4();
#pragma unroll
    for (int q = 0; q < 2; ++q)
      *reinterpret_cast<u32x4_t*>(&pb[(srow + 32 * q) * kStrLd + 8 * sc]) = ok ? pv[q] : zero4();
  };
  f32x16_t acc[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[ct][e] = 0.0f;
  auto compute = [&](const uint16_t* xb, const uint16_t* pb) {
#pragma unroll
    for (int st = 0; st < kStrT / 16; ++st) {
      const int tt = 16 * st + 8 * h;
      const u32x4_t a = *reinterpret_cast<const u32x4_t*>(&xb[(32 * w + i) * kStrLd + tt]);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {  // a second tile past r holds row r-1 of P, not stored
        const u32x4_t b = *reinterpret_cast<const u32x4_t*>(&pb[(32 * ct + i) * kStrLd + tt]);
        acc[ct] = mfma_32x32x16(a, b, acc[ct]);
      }
    }
  };

  u32x4_t xa[4], pa[2], xn[4], pn[2];
  load(0, xa, pa);
  load(1, xn, pn);
  stage(0, xs[0], ps[0], xa, pa);
  __syncthreads();
  // The scheduling barriers keep each chunk's loads ahead of the previous
  // chunk's compute (left alone, the compiler reuses the fragment registers
  // for them and waits for every load before the next one issues).
  for (int p = 0; p < npairs; ++p) {
    const int c = 2 * p;
    // buffer 0 holds chunk c; chunk c+1 is in flight (xn, pn)
    load(c + 2, xa, pa);
    __builtin_amdgcn_sched_barrier(0);
    compute(xs[0], ps[0]);
    stage(c + 1, xs[1], ps[1], xn, pn);
    __syncthreads();
    load(c + 3, xn, pn);
    __builtin_amdgcn_sched_barrier(0);
    compute(xs[1], ps[1]);
    stage(c + 2, xs[0], ps[0], xa, pa);
    __syncthreads();
  }
  // the last loads (chunk 2 npairs + 1) land before the workgroup ends
  stage(2 * npairs + 1, xs[1], ps[1], xn, pn);

  // element e of tile ct: row 8(e/4) + 4h + e%4 of the wave's 32, column
  // 32ct + i of the workgroup's 64
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    if (ct < ncol) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t m = m0 + 32 * w + 8 * (e >> 2) + 4 * h + (e & 3);
        if (m < M) part[((int64_t)slice * M + m) * r + j0 + 32 * ct + i] = acc[ct][e];
      }
    }
  }
}

// out[m][j] = sum over slices (skipped if out == NULL); with sv = s*out:
// lr[m][j] = bf16(sv), lr[m][r+j] = bf16(sv - hi) (row-major two-term split),
// lrT[j][m] = bf16(sv), lrT[r+j][m] = bf16(sv - hi) (transposed, row stride
// Mp, zero for M <= m < Mp). Either split output may be NULL. Two
// independent jobs of the same M and r share a launch: workgroups 0 ..
// j0.blocks-1 take job j0 (each job's blocks cover Mp * r elements).
struct FinJobD {
  const float* part;
  int slices;
  float* out;
  uint16_t* lr;
  uint16_t* lrT;
  unsigned blocks;
};

__global__ __launch_bounds__(256) void lora_down_finalize_kernel(FinJobD j0, FinJobD j1, int64_t M,
                                                                 int64_t Mp, int r, float s) {
  const bool second = blockIdx.x >= j0.blocks;
  const FinJobD& J = second ? j1 : j0;
  const int64_t i = (int64_t)(second ? blockIdx.x - j0.blocks : blockIdx.x) * 256 + threadIdx.x;
  if (i >= Mp * r) return;
  const int64_t m = i / r;
  const int j = (int)(i % r);
  uint16_t* __restrict__ lr = J.lr;
  uint16_t* __restrict__ lrT = J.lrT;
  if (m >= M) {
    if (lrT) {
      lrT[(int64_t)j * Mp + m] = 0;
      lrT[(int64_t)(r + j) * Mp + m] = 0;
    }
    return;
  }
  const float v = sum_strided<8>(J.part + i, M * r, J.slices);
  if (J.out) J.out[i] = v;
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

// Direct form for M >= 256 and column counts that are multiples of 8: a
// workgroup owns 32*kCG columns c of one job and 64 rank columns j, walks the
// whole of M in 64-row chunks and writes the result itself (no slices, no
// finalize): out[c][j] = sum_m X[m][c] (PT[j][m] + PT[r+j][m]), stored as
// [C, r] or transposed [r, C], fp32 or bf16. Chunks of X (64 rows x 32*kCG
// columns, whole 128-byte lines) and of the split (128 rows: 64 hi, 64 lo,
// x 64 m) are staged in double-buffered LDS. Wave w takes the 32
// columns of group w % kCG and, for kCG = 4, both 32-wide rank tiles (for
// kCG = 2, rank tile w / 2); v_mfma_f32_32x32x16_bf16 with the reduction
// over m: the x operand reads 8 rows of one column (16-bit LDS reads; the
// row stride puts the two 8-row halves of a read in distinct banks), the
// split operand one 16-byte read per lane. The loads run three chunks ahead
// (the grids are small: about one workgroup per CU for the 70B-shaped
// projections). Rows past M and past the split's
// padded length are staged as zeros; rank rows past r are clamped and not
// stored.
struct ColOut {
  const uint16_t* X;
  const uint16_t* PT;
  int64_t C;
  void* out;
  int transpose_out;
  unsigned tiles;  // column tiles of 32*kCG
};

template <int kCG, bool kBf16>
__global__ __launch_bounds__(256) void colred_direct_kernel(ColOut j0, ColOut j1, int64_t M,
                                                            int64_t Mp, int r) {
  constexpr int kCT = 32 * kCG;          // columns per workgroup
  constexpr int kLdX = kCT + 8;          // staged x row stride (bf16)
  constexpr int kXP = 64 * kCT / 8 / 256;  // 16-byte x pieces per thread and chunk
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][64 * kLdX];
  __shared__ __attribute__((aligned(16))) uint16_t ps[2][128 * kStrLd];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, i = lane & 31, h = lane >> 5;
  const bool second = blockIdx.x >= j0.tiles;
  const ColOut& J = second ? j1 : j0;
  const uint16_t* __restrict__ X = J.X;
  const uint16_t* __restrict__ PT = J.PT;
  const int64_t C = J.C;
  const int64_t c0 = (int64_t)(second ? blockIdx.x - j0.tiles : blockIdx.x) * kCT;
  const int jb = blockIdx.y * 64;
  const int nquads = (int)((M + 255) / 256);  // four 64-row chunks each

  // Staging roles. x piece e = tid + 256q: row e / (kCT/8), columns
  // 8 (e % (kCT/8)) (clamped into the matrix). Split piece e = tid + 256q:
  // tile row e >> 3 (hi rows 0..63, lo rows 64..127), m 8 (e & 7).
  int64_t xoff[kXP];
  int xrow[kXP], xcol[kXP];
#pragma unroll
  for (int q = 0; q < kXP; ++q) {
    const int e = tid + 256 * q;
    xrow[q] = e / (kCT / 8);
    xcol[q] = 8 * (e % (kCT / 8));
    xoff[q] = min(c0 + xcol[q], C - 8);
  }
  int64_t poff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int pr = (tid >> 3) + 32 * q;
    const int j = min(jb + (pr & 63), r - 1);
    poff[q] = (int64_t)(pr < 64 ? j : r + j) * Mp;
  }
  const int pm = 8 * (tid & 7);

  auto load = [&](int c, u32x4_t (&xv)[kXP], u32x4_t (&pv)[4]) {
    const int64_t m = (int64_t)c * 64;
#pragma unroll
    for (int q = 0; q < kXP; ++q) {
      const int64_t row = min(m + xrow[q], M - 1);
      xv[q] = *reinterpret_cast<const u32x4_t*>(X + row * C + xoff[q]);
    }
    const int64_t mm = min(m + pm, Mp - 8);
#pragma unroll
    for (int q = 0; q < 4; ++q) pv[q] = *reinterpret_cast<const u32x4_t*>(PT + poff[q] + mm);
  };
  auto stage = [&](int c, uint16_t* xb, uint16_t* pb, const u32x4_t (&xv)[kXP],
                   const u32x4_t (&pv)[4]) {
    const int64_t m = (int64_t)c * 64;
#pragma unroll
    for (int q = 0; q < kXP; ++q)
      *reinterpret_cast<u32x4_t*>(&xb[xrow[q] * kLdX + xcol[q]]) =
          m + xrow[q] < M ? xv[q] : zero4();
    const bool pok = m + pm < Mp;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<u32x4_t*>(&pb[((tid >> 3) + 32 * q) * kStrLd + pm]) =
          pok ? pv[q] : zero4();
  };
  constexpr int kJT = kCG == 4 ? 2 : 1;  // rank tiles per wave
  const int cb = 32 * (w % kCG);
  const int jt0 = kCG == 4 ? 0 : w / 2;
  f32x16_t acc[kJT];
#pragma unroll
  for (int t = 0; t < kJT; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.0f;
  auto compute = [&](const uint16_t* xb, const uint16_t* pb) {
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const uint16_t* xa = &xb[(16 * st + 8 * h) * kLdX + cb + i];
      u32x4_t a;
      a.x = (uint32_t)xa[0 * kLdX] | ((uint32_t)xa[1 * kLdX] << 16);
      a.y = (uint32_t)xa[2 * kLdX] | ((uint32_t)xa[3 * kLdX] << 16);
      a.z = (uint32_t)xa[4 * kLdX] | ((uint32_t)xa[5 * kLdX] << 16);
      a.w = (uint32_t)xa[6 * kLdX] | ((uint32_t)xa[7 * kLdX] << 16);
#pragma unroll
      for (int t = 0; t < kJT; ++t) {
        const int tr = 32 * (jt0 + t) + i;
        const u32x4_t bh = *reinterpret_cast<const u32x4_t*>(&pb[tr * kStrLd + 16 * st + 8 * h]);
        const u32x4_t bl =
            *reinterpret_cast<const u32x4_t*>(&pb[(64 + tr) * kStrLd + 16 * st + 8 * h]);
        acc[t] = mfma_32x32x16(a, bh, acc[t]);
        acc[t] = mfma_32x32x16(a, bl, acc[t]);
      }
    }
  };

  // Four register slots: while one chunk is computed from LDS, the loads of
  // the next three are in flight (about 96 KB a workgroup).
  u32x4_t x0[kXP], p0[4], x1[kXP], p1[4], x2[kXP], p2[4], x3[kXP], p3[4];
  load(0, x0, p0);
  load(1, x1, p1);
  load(2, x2, p2);
  stage(0, xs[0], ps[0], x0, p0);
  __syncthreads();
  for (int qd = 0; qd < nquads; ++qd) {
    const int c = 4 * qd;
    load(c + 3, x3, p3);
    __builtin_amdgcn_sched_barrier(0);
    compute(xs[0], ps[0]);
    stage(c + 1, xs[1], ps[1], x1, p1);
    __syncthreads();
    load(c + 4, x0, p0);
    __builtin_amdgcn_sched_barrier(0);
    compute(xs[1], ps[1]);
    stage(c + 2, xs[0], ps[0], x2, p2);
    __syncthreads();
    load(c + 5, x1, p1);
    __builtin_amdgcn_sched_barrier(0);
    compute(xs[0], ps[0]);
    stage(c + 3, xs[1], ps[1], x3, p3);
    __syncthreads();
    load(c + 6, x2, p2);
    __builtin_amdgcn_sched_barrier(0);
    compute(xs[1], ps[1]);
    stage(c + 4, xs[0], ps[0], x0, p0);
    __syncthreads();
  }
  // the last loads land before the workgroup ends
  stage(4 * nquads + 1, xs[1], ps[1], x1, p1);
  stage(4 * nquads + 2, xs[1], ps[1], x2, p2);

  // Element e of tile t: column c0 + cb + 8(e/4) + 4h + e%4, rank
  // jb + 32(jt0 + t) + i.
#pragma unroll
  for (int t = 0; t < kJT; ++t) {
    const int j = jb + 32 * (jt0 + t) + i;
    if (j >= r) continue;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int64_t c = c0 + cb + 8 * g + 4 * h;  // four consecutive columns
      if (c >= C) continue;                       // C % 8 == 0: all four or none
      const float v0 = acc[t][4 * g], v1 = acc[t][4 * g + 1], v2 = acc[t][4 * g + 2],
                  v3 = acc[t][4 * g + 3];
      if (J.transpose_out) {
        const int64_t o = (int64_t)j * C + c;
        if (kBf16)
          *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(J.out) + o) =
              u32x2_t{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
        else
          *reinterpret_cast<f32x4_t*>(static_cast<float*>(J.out) + o) = f32x4_t{v0, v1, v2, v3};
      } else {
        const float vv[4] = {v0, v1, v2, v3};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int64_t o = (c + k) * r + j;
          if (kBf16)
            static_cast<uint16_t*>(J.out)[o] = (uint16_t)(pack_bf16x2(vv[k], 0.0f) & 0xFFFFu);
          else
            static_cast<float*>(J.out)[o] = vv[k];
        }
      }
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

// The tiled down projection serves large M with ranks that are multiples of
// 32 from 64 on (r = 16 and 32 take the single-pass kernel from M = 2048).
static bool lora_down_tiled(int64_t M, int64_t T, int r) {
  const int64_t wgs = ((M + 127) / 128) * ((r + 63) / 64) * ((T + kTileT - 1) / kTileT);
  // measured: 21 vs 23 us at T = 8192, but slower than the 16-row kernel at
  // T = 28672 (82 vs 75 us) and with few workgroups (T = 1024)
  return M >= 1024 && r >= 64 && r % 32 == 0 && T % 8 == 0 && wgs >= 128 && T <= 16384;
}

// The streaming form: large M, ranks that are multiples of 32, long T.
static bool lora_down_streamed(int64_t M, int64_t T, int r) {
  return M >= 512 && r % 32 == 0 && T % 8 == 0 && T >= 4096;
}

// t per slice of the streaming form: about 512 workgroups (two per CU), at
// least 8 chunks a slice.
static int64_t lora_down_tslice(int64_t M, int64_t T, int r) {
  const int64_t base = ((M + 127) / 128) * ((r + 63) / 64);
  const int64_t chunks = (T + kStrT - 1) / kStrT;
  int64_t S = (512 + base - 1) / base;
  if (S > chunks / 8) S = chunks / 8;
  if (S < 1) S = 1;
  return (chunks + S - 1) / S * kStrT;
}

int lora_down_slices(int64_t M, int64_t T, int r) {
  if (lora_down_streamed(M, T, r)) {
    const int64_t ts = lora_down_tslice(M, T, r);
    return (int)((T + ts - 1) / ts);
  }
  return lora_down_tiled(M, T, r) ? (int)((T + kTileT - 1) / kTileT)
                                  : (int)((T + kDownTC - 1) / kDownTC);
}

hipError_t launch_lora_down_parts(const uint16_t* X, const uint16_t* P, int64_t M, int64_t T,
                                  int r, float* part, hipStream_t st) {
  if (lora_down_streamed(M, T, r)) {
    const int64_t ts = lora_down_tslice(M, T, r);
    const dim3 grid((unsigned)((M + 127) / 128), (unsigned)((r + 63) / 64),
                    (unsigned)((T + ts - 1) / ts));
    hipLaunchKernelGGL(lora_down_stream_kernel, grid, dim3(256), 0, st, X, P, M, T, r, ts, part);
    return hipGetLastError();
  }
  if (lora_down_tiled(M, T, r)) {
    const dim3 grid((unsigned)((M + 127) / 128), (unsigned)((r + 63) / 64),
                    (unsigned)lora_down_slices(M, T, r));
    hipLaunchKernelGGL(lora_down_tile_kernel, grid, dim3(256), 0, st, X, P, M, T, r, part);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((M + 15) / 16), (unsigned)((r + 63) / 64),
                  (unsigned)lora_down_slices(M, T, r));
  hipLaunchKernelGGL(lora_down_kernel, grid, dim3(256), 0, st, X, P, M, T, r, part);
  return hipGetLastError();
}

hipError_t launch_lora_down_finalize(const float* part, int slices, int64_t M, int r, float s,
                                     float* out, uint16_t* lr, uint16_t* lrT, hipStream_t st) {
  return launch_lora_down_finalize2(part, slices, out, lr, lrT, nullptr, 0, nullptr, nullptr,
                                    nullptr, M, r, s, st);
}

hipError_t launch_lora_down_finalize2(const float* part0, int slices0, float* out0, uint16_t* lr0,
                                      uint16_t* lrT0, const float* part1, int slices1,
                                      float* out1, uint16_t* lr1, uint16_t* lrT1, int64_t M, int r,
                                      float s, hipStream_t st) {
  const int64_t Mp = (M + 7) & ~(int64_t)7;
  const unsigned blocks = (unsigned)((Mp * r + 255) / 256);
  const FinJobD j0{part0, slices0, out0, lr0, lrT0, blocks};
  const FinJobD j1{part1, slices1, out1, lr1, lrT1, part1 ? blocks : 0u};
  hipLaunchKernelGGL(lora_down_finalize_kernel, dim3(j0.blocks + j1.blocks), dim3(256), 0, st, j0,
                     j1, M, Mp, r, s);
  return hipGetLastError();
}

bool lora_down_full_ok(int64_t M, int64_t T, int r) {
  // r = 64 re-reads 64 x T of the rank-side operand per 16 rows: measured at
  // M = 2048 it beats the sliced kernels with their finalize at T = 1024
  // (the 70B k and v backward, 85 -> 77 us per call) but loses to the
  // streaming form from T = 8192 on (4-40 us per call)
  return M >= 2048 && T % 32 == 0 && (r == 16 || r == 32 || (r == 64 && T < 4096));
}

hipError_t launch_lora_down_full(const uint16_t* X, const uint16_t* P, int64_t M, int64_t T,
                                 int r, float s, float* out, uint16_t* lr, uint16_t* lrT,
                                 const float* u2, uint16_t* u2T, hipStream_t st) {
  const int64_t Mp = (M + 7) & ~(int64_t)7;
  if (u2T && !u2) return hipErrorInvalidValue;
  if (r == 16) {
    hipLaunchKernelGGL(lora_down_full_kernel<1>, dim3((unsigned)((M + 15) / 16)), dim3(512), 0,
                       st, X, P, M, Mp, T, r, s, out, lr, lrT, u2, u2T);
  } else if (r == 32 || r == 64) {
    hipLaunchKernelGGL(lora_down_full_kernel<2>, dim3((unsigned)((M + 15) / 16), r / 32),
                       dim3(512), 0, st, X, P, M, Mp, T, r, s, out, lr, lrT, u2, u2T);
  } else {
    return hipErrorInvalidValue;
  }
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

int colred_direct_cg(int64_t M, int64_t K, int64_t N, int r) {
  if (M < 256 || K % 8 || N % 8) return 0;
  // measured on the 70B-shaped layer (M = 2048, r = 64): dA and dB of up
  // and down 75 -> 59 us, of q 36 -> 28 us; with fewer workgroups than CUs
  // (k and v: 144) the sliced form with its finalize is as fast
  const int64_t rb = (r + 63) / 64;
  if (((K + 63) / 64 + (N + 63) / 64) * rb < 256) return 0;
  return ((K + 127) / 128 + (N + 127) / 128) * rb >= 256 ? 4 : 2;
}

hipError_t launch_colred_direct2(const uint16_t* X0, const uint16_t* PT0, int64_t C0,
                                 void* out0, bool transpose0, const uint16_t* X1,
                                 const uint16_t* PT1, int64_t C1, void* out1, bool transpose1,
                                 int64_t M, int r, int cg, bool out_bf16, hipStream_t st) {
  if ((cg != 2 && cg != 4) || M < 256 || C0 % 8 || (X1 && C1 % 8)) return hipErrorInvalidValue;
  const int64_t Mp = (M + 7) & ~(int64_t)7;
  const int64_t ct = 32 * cg;
  const ColOut a{X0, PT0, C0, out0, transpose0 ? 1 : 0, (unsigned)((C0 + ct - 1) / ct)};
  const ColOut b{X1, PT1, C1, out1, transpose1 ? 1 : 0, X1 ? (unsigned)((C1 + ct - 1) / ct) : 0u};
  const dim3 grid(a.tiles + b.tiles, (unsigned)((r + 63) / 64));
  if (cg == 4) {
    if (out_bf16)
      hipLaunchKernelGGL((colred_direct_kernel<4, true>), grid, dim3(256), 0, st, a, b, M, Mp, r);
    else
      hipLaunchKernelGGL((colred_direct_kernel<4, false>), grid, dim3(256), 0, st, a, b, M, Mp, r);
  } else {
    if (out_bf16)
      hipLaunchKernelGGL((colred_direct_kernel<2, true>), grid, dim3(256), 0, st, a, b, M, Mp, r);
    else
      hipLaunchKernelGGL((colred_direct_kernel<2, false>), grid, dim3(256), 0, st, a, b, M, Mp, r);
  }
  return hipGetLastError();
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
