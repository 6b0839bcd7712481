// Large-M path of the QLoRA linear layer on gfx950: the NF4 weight is
// dequantized once per call into a bf16 workspace, then a plain bf16 GEMM with
// the rank-r adapter term runs on the matrix cores.
//
// [P1] "QLoRA" forward equation h = W_hat x + (alpha/r) B(Ax) and bullets
// (the 4-bit weight is expanded to the 16-bit compute type right before the
// matmul); [P2] s3 "The Backward Pass Through Quantization" (the input
// gradient goes through the dequantized weight, in the compute type).
//
//  - The weight operand comes from quantize.hip: the row-major
//    dequantization for the forward, the transposed one (w_hat^T, [K, N]) for
//    the input gradient, so that dX = dY w_hat reduces over contiguous rows
//    like the forward.
//  - gemm_nt_kernel: y[M,N] = a[M,Kr] b[N,Kr]^T + e[M,2r] f'[N,2r]^T where
//    f' repeats the r columns of f twice (e holds the two-term bf16 split of
//    the scaled adapter product, so the extension adds s*u B exactly as the
//    split represents it). 256 x 256 output tiles, four waves of 128 x 128
//    on v_mfma_f32_32x32x16_bf16; both operand tiles arrive by direct-to-LDS
//    loads (buffer_load_dwordx4 ... lds): a in a three-slot ring of 64-wide
//    pairs of K steps (whole 128-byte lines of a row-major a per load), b in
//    a four-deep ring of 32-wide steps; the fragments of the next substep are
//    read while the MFMAs of the current one run, so the one barrier per
//    step never waits on LDS.
//    Workgroups are mapped to tiles so that each XCD works on a compact block
//    of tiles (shared operand panels stay in that XCD's L2).
#include "device.h"

namespace qlora {
namespace {

constexpr int kNtBM = 256;              // output rows per tile
constexpr int kNtBN = 256;              // output columns per tile
constexpr int kNtBK = 32;               // reduction elements per step
constexpr int kNtOp = kNtBM * kNtBK;    // bf16 elements of one operand tile (16 KB)
constexpr int kNtGroup = 4;             // tile rows per group in the tile order

struct NtArgs {
  const uint16_t* a;  // [M, Kr], row stride lda elements
  const uint16_t* b;  // [N, Kr], row stride ldb elements, or K-slab layout (b_kslab)
  const uint16_t* e;  // [M, 2r]
  const uint16_t* f;  // [N, r]
  void* y;            // [M, N]
  int64_t M, N, Kr, lda, ldb;
  int r;
  int tiles_m, tiles_n;
  // K split: workgroup wg takes tile wg / ksplit and the split wg % ksplit
  // of the reduction steps; with ksplit > 1 every split stores its fp32 sums
  // to part + split * M * N (the rank extension rides in split 0) and a
  // reduce kernel adds the splits in order into y.
  int ksplit;
  float* part;
  // b in the K-slab layout [Kr/32][N][32]: the 32 reduction elements of one
  // step of every row are one contiguous 64-byte piece, and a step's rows
  // follow each other, so a direct-to-LDS load of 16 rows reads 1 KB of
  // consecutive bytes (whole cache lines) instead of 16 half lines.
  int b_kslab;
};

// Tile of workgroup `wg`. Workgroups are dealt to the eight XCDs round robin
// (wg % 8); each XCD gets a contiguous range of the tile order, and the order
// walks groups of kNtGroup tile rows column by column, so the tiles that run
// together on one XCD share a few row panels of a and column panels of b.
__device__ __forceinline__ void nt_tile(int wg, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int T = tiles_m * tiles_n;
  const int xcd = wg & 7, idx = wg >> 3;
  const int per = T >> 3, extra = T & 7;
  const int t = xcd * per + (xcd < extra ? xcd : extra) + idx;
  const int group = t / (kNtGroup * tiles_n);
  const int first = group * kNtGroup;
  const int rows = tiles_m - first < kNtGroup ? tiles_m - first : kNtGroup;
  const int in = t - group * kNtGroup * tiles_n;
  tm = first + in % rows;
  tn = in / rows;
}

// s_waitcnt: at most n vector-memory operations in flight, no LDS operation.
template <int n>
__device__ __forceinline__ void wait_vmem_lgkm0() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4));
  __builtin_amdgcn_sched_barrier(0);
}

// A pointer the compiler must keep in scalar registers (its value is the
// same in every lane).
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
}

template <int S, int N, typename T>
__device__ __forceinline__ T* pick(T* const (&arr)[N]) {
  static_assert(S >= 0 && S < N, "stage index");
  return arr[S];
}

// LDS rings (160 KB in all):
//  - a: three slots of a 256 x 64 tile (two 32-wide K steps, a "pair"), rows
//    of 128 bytes; 16-byte chunk c (0..7: step half c/4, then 8 k each) of
//    row r sits at position c ^ ((r >> 1) & 7). A direct-to-LDS load of 8
//    rows x 128 bytes fills 1 KB with whole cache lines of a row-major a; a
//    fragment read (16 rows per LDS phase, one chunk each) touches 16
//    distinct 16-byte bank groups. Pair p lives in slot p % 3 and is loaded
//    during steps 2p-4 and 2p-3 (four loads per wave in each).
//  - b: four stages of a 256 x 32 tile, rows of 64 bytes, chunk c (0..3) of
//    row r at c ^ ((r >> 2) & 3); step kb lives in stage kb % 4 and is
//    loaded during step kb-3. A load covers 16 rows x 64 bytes: 1 KB of
//    consecutive bytes in the K-slab layout, 16 half lines in row-major.
// Every load of a step lands by the end of the next step (wait for all but
// the step's own eight), and the barrier then publishes it; what a load
// overwrites was last read before the previous barrier.
constexpr int kNtPair = kNtBM * 2 * kNtBK;  // bf16 elements of one a pair slot (32 KB)

template <bool kOutBf16, bool kSplit>
__global__ __launch_bounds__(256, 1) void gemm_nt_kernel(NtArgs p) {
  __shared__ __attribute__((aligned(1024))) uint16_t sa0[kNtPair];
  __shared__ __attribute__((aligned(1024))) uint16_t sa1[kNtPair];
  __shared__ __attribute__((aligned(1024))) uint16_t sa2[kNtPair];
  __shared__ __attribute__((aligned(1024))) uint16_t sb0[kNtOp];
  __shared__ __attribute__((aligned(1024))) uint16_t sb1[kNtOp];
  __shared__ __attribute__((aligned(1024))) uint16_t sb2[kNtOp];
  __shared__ __attribute__((aligned(1024))) uint16_t sb3[kNtOp];
  uint16_t* const sa[3] = {sa0, sa1, sa2};
  uint16_t* const sb[4] = {sb0, sb1, sb2, sb3};
  const int tid = threadIdx.x, lane = tid & 63, i = lane & 31, h = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = w >> 1, wn = w & 1;
  int tm, tn;
  const int split = kSplit ? (int)blockIdx.x % p.ksplit : 0;
  nt_tile(kSplit ? (int)blockIdx.x / p.ksplit : (int)blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
  const int64_t M = p.M, N = p.N;
  const int64_t m0 = (int64_t)tm * kNtBM, n0 = (int64_t)tn * kNtBN;
  // this split's reduction steps [ks0, ks0 + nsteps)
  const int steps_all = (int)(p.Kr / kNtBK);
  const int per_split = kSplit ? (steps_all + p.ksplit - 1) / p.ksplit : steps_all;
  const int ks0 = split * per_split;
  const int nsteps = kSplit ? min(per_split, steps_all - ks0) : steps_all;
  const int npairs = (nsteps + 1) / 2;
  const int64_t k0 = (int64_t)ks0 * kNtBK;  // first reduction element

  // Direct-to-LDS roles. a: wave w loads rows 64w + 8q + L/8 (q = 0..7) of
  // each pair, lane L at LDS position L%8 (global chunk (L%8) ^ ((row>>1)&7));
  // the pair's scalar offset is 128 bytes per pair. The a resource ends at
  // the last element of the matrix, so the missing half of a final odd pair
  // reads zeros. b: wave w loads windows 4w .. 4w+3 (16 rows each) of each
  // step, as before. Rows past the matrix read its last row (their results
  // are never stored).
  uint32_t aoff[8], boff[4];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int row = 64 * w + 8 * q + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    const int64_t ar = m0 + row < M ? row : M - 1 - m0;
    aoff[q] = (uint32_t)(ar * p.lda * 2 + 16 * c);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 16 * (4 * w + j) + (lane >> 2);
    const int c = (lane & 3) ^ ((row >> 2) & 3);
    const int64_t br = n0 + row < N ? row : N - 1 - n0;
    boff[j] = (uint32_t)(br * (p.b_kslab ? 64 : p.ldb * 2) + 16 * c);
  }
  // Bytes from the tile's first row to the matrix's last element; a tile's
  // own offsets stay below 2^31 (gemm_nt_supported), so clamping a longer
  // range only matters for tiles that are not the last and read in bounds.
  const int64_t a_bytes = min(((M - 1 - m0) * p.lda + p.Kr - k0) * 2, (int64_t)0x7FFFFFFF);
  const __amdgpu_buffer_rsrc_t ares = __builtin_amdgcn_make_buffer_rsrc(
      (void*)uniform_ptr(p.a + m0 * p.lda + k0), (short)0, (int)a_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t bres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)uniform_ptr(p.b + (p.b_kslab ? n0 * 32 + k0 * N : n0 * p.ldb + k0)), (short)0,
      (int)0x7FFFFFFF, 0x00020000);
  const int bstep = p.b_kslab ? (int)(64 * N) : 64;  // bytes from one step to the next
  typedef __attribute__((address_space(3))) void lds_void;
  auto dma_a = [&](int q, int pair, uint16_t* slot) {
    const int ps = pair < npairs ? pair : npairs - 1;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ares, (lds_void*)(slot + (64 * w + 8 * q) * 64), 16,
                                             aoff[q], 128 * ps, 0, 0);
  };
  auto dma_b = [&](int j, int kb, uint16_t* stage) {
    const int ks = kb < nsteps ? kb : nsteps - 1;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(bres, (lds_void*)(stage + 512 * (4 * w + j)), 16,
                                             boff[j], bstep * ks, 0, 0);
  };

  // Fragment reads: A fragment (mt, step half par, substep s): tile row
  // 128wm + 32mt + i, chunk 4par + 2s + h, at position chunk ^ ((i >> 1) & 7)
  // (bits 1..3 of the row are those of i). B fragment (nt, s): tile row
  // 128wn + 32nt + i, chunk 2s + h at (2s + h) ^ ((i >> 2) & 3).
  const int swa = (i >> 1) & 7, swb = (i >> 2) & 3;
  int fa[2][2];
#pragma unroll
  for (int par = 0; par < 2; ++par)
#pragma unroll
    for (int ss = 0; ss < 2; ++ss)
      fa[par][ss] = (128 * wm + i) * 64 + 8 * ((4 * par + 2 * ss + h) ^ swa);
  const int fb0 = (128 * wn + i) * 32 + 8 * (h ^ swb);
  const int fb1 = (128 * wn + i) * 32 + 8 * ((2 + h) ^ swb);

  f32x16_t acc[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mt][nt][e] = 0.0f;

  // Adapter operands: lane group h supplies extension elements 16q + 8h +
  // (0..7); column jj of e pairs with column jj mod r of f. The first two
  // groups are loaded now (they land with the prologue's loads), the rest
  // after the main loop.
  const int r = p.r, r2 = 2 * r;
  auto ext_load = [&](int q, u32x4_t (&ev)[4], u32x4_t (&fv)[4]) {
    const int jj = 16 * q + 8 * h;
    const int jb = jj % r;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int64_t n = n0 + 128 * wn + 32 * nt + i;
      fv[nt] = n < N ? *reinterpret_cast<const u32x4_t*>(p.f + n * r + jb) : zero4();
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int64_t m = m0 + 128 * wm + 32 * mt + i;
      ev[mt] = m < M ? *reinterpret_cast<const u32x4_t*>(p.e + m * r2 + jj) : zero4();
    }
  };
  auto ext_mfma = [&](const u32x4_t (&ev)[4], const u32x4_t (&fv)[4]) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mfma_32x32x16(ev[mt], fv[nt], acc[mt][nt]);
  };
  u32x4_t e0[4], f0[4], e1[4], f1[4];
  ext_load(0, e0, f0);
  ext_load(1, e1, f1);  // r2 >= 32: groups 0 and 1 always exist

  // Prologue: pair 0, steps 0 and 1 of b, pair 1, step 2 of b; wait for the
  // first three (all that steps 0 and 1 read before the first barrier of the
  // loop); fragments of step 0, substep 0.
#pragma unroll
  for (int q = 0; q < 8; ++q) dma_a(q, 0, sa0);
#pragma unroll
  for (int j = 0; j < 4; ++j) dma_b(j, 0, sb0);
#pragma unroll
  for (int j = 0; j < 4; ++j) dma_b(j, 1, sb1);
#pragma unroll
  for (int q = 0; q < 8; ++q) dma_a(q, 1, sa1);
#pragma unroll
  for (int j = 0; j < 4; ++j) dma_b(j, 2, sb2);
  wait_vmem_lgkm0<12>();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  u32x4_t a0[4], b0[4], a1[4], b1[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    a0[t] = *reinterpret_cast<const u32x4_t*>(&sa0[fa[0][0] + 2048 * t]);
    b0[t] = *reinterpret_cast<const u32x4_t*>(&sb0[fb0 + 1024 * t]);
  }

  // One step kb (B stage kb % 4 = SB, A slot (kb / 2) % 3 = SA, half PAR):
  // substep 0 computes on (a0, b0) while (kb, 1) is read into (a1, b1);
  // substep 1 computes on (a1, b1) while (kb+1, 0) is read into (a0, b0)
  // (complete since the previous barrier). One load after every fourth
  // MFMA: b of step kb+3 in substep 0, four a loads of pair kb/2 + 2 in
  // substep 1.
  auto step = [&](int kb, auto sbc, auto sac, auto parc) {
    constexpr int SB = decltype(sbc)::value, SA = decltype(sac)::value;
    constexpr int PAR = decltype(parc)::value;
    constexpr int SA1 = PAR ? (SA + 1) % 3 : SA;  // slot of step kb+1
    constexpr int PAR1 = PAR ^ 1;
    uint16_t* const acur = pick<SA>(sa);
    uint16_t* const anxt = pick<SA1>(sa);
    uint16_t* const ald = pick<(SA + 2) % 3>(sa);
    uint16_t* const bcur = pick<SB>(sb);
    uint16_t* const bnxt = pick<(SB + 1) % 4>(sb);
    uint16_t* const bld = pick<(SB + 3) % 4>(sb);
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      const int mt = g >> 2, nt = g & 3;
      acc[mt][nt] = mfma_32x32x16(a0[mt], b0[nt], acc[mt][nt]);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (g < 8) {
        const int t = g >> 1;
        if (g & 1)
          b1[t] = *reinterpret_cast<const u32x4_t*>(&bcur[fb1 + 1024 * t]);
        else
          a1[t] = *reinterpret_cast<const u32x4_t*>(&acur[fa[PAR][1] + 2048 * t]);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      if ((g & 3) == 3) {
        dma_b(g >> 2, kb + 3, bld);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      const int mt = g >> 2, nt = g & 3;
      acc[mt][nt] = mfma_32x32x16(a1[mt], b1[nt], acc[mt][nt]);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (g < 8) {
        const int t = g >> 1;
        if (g & 1)
          b0[t] = *reinterpret_cast<const u32x4_t*>(&bnxt[fb0 + 1024 * t]);
        else
          a0[t] = *reinterpret_cast<const u32x4_t*>(&anxt[fa[PAR1][0] + 2048 * t]);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      if ((g & 3) == 3) {
        dma_a(4 * PAR + (g >> 2), kb / 2 + 2, ald);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // This step's eight loads may still fly; everything earlier has landed,
    // this wave's LDS reads are done; then every wave's loads are visible
    // and the stage and slot read last before this barrier are free.
    wait_vmem_lgkm0<8>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  // Twelve steps bring both rings back to their first stage and slot.
  int kb = 0;
  for (; kb + 12 <= nsteps; kb += 12) {
    step(kb + 0, I0(), I0(), I0());
    step(kb + 1, I1(), I0(), I1());
    step(kb + 2, I2(), I1(), I0());
    step(kb + 3, I3(), I1(), I1());
    step(kb + 4, I0(), I2(), I0());
    step(kb + 5, I1(), I2(), I1());
    step(kb + 6, I2(), I0(), I0());
    step(kb + 7, I3(), I0(), I1());
    step(kb + 8, I0(), I1(), I0());
    step(kb + 9, I1(), I1(), I1());
    step(kb + 10, I2(), I2(), I0());
    step(kb + 11, I3(), I2(), I1());
  }
  if (kb + 0 < nsteps) step(kb + 0, I0(), I0(), I0());
  if (kb + 1 < nsteps) step(kb + 1, I1(), I0(), I1());
  if (kb + 2 < nsteps) step(kb + 2, I2(), I1(), I0());
  if (kb + 3 < nsteps) step(kb + 3, I3(), I1(), I1());
  if (kb + 4 < nsteps) step(kb + 4, I0(), I2(), I0());
  if (kb + 5 < nsteps) step(kb + 5, I1(), I2(), I1());
  if (kb + 6 < nsteps) step(kb + 6, I2(), I0(), I0());
  if (kb + 7 < nsteps) step(kb + 7, I3(), I0(), I1());
  if (kb + 8 < nsteps) step(kb + 8, I0(), I1(), I0());
  if (kb + 9 < nsteps) step(kb + 9, I1(), I1(), I1());
  if (kb + 10 < nsteps) step(kb + 10, I2(), I2(), I0());
  // Direct-to-LDS loads still in flight must land before the workgroup ends.
  wait_vmem_lgkm0<0>();

  // Adapter term as 2r extra reduction elements, 16 per MFMA (split 0 only).
  if (!kSplit || split == 0) {
    ext_mfma(e0, f0);
    ext_mfma(e1, f1);
    for (int q = 2; q < r2 / 16; ++q) {
      ext_load(q, e0, f0);
      ext_mfma(e0, f0);
    }
  }
  if (kSplit) {  // fp32 partial sums of this split
    float* dst = p.part + (int64_t)split * M * N;
    const int64_t mw = m0 + 128 * wm + 4 * h, nw = n0 + 128 * wn + i;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int64_t n = nw + 32 * nt;
      if (n < N) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int64_t m = mw + 32 * mt + 8 * (e >> 2) + (e & 3);
            if (m < M) dst[m * N + n] = acc[mt][nt][e];
          }
      }
    }
    return;
  }

  // Output. Accumulator element e of (mt, nt) is row 32mt + 8(e/4) + 4h +
  // e%4, column 32nt + i of this wave's 128 x 128 block. Whole tiles take one
  // row address per row and four stores with constant column offsets.
  const int64_t mw = m0 + 128 * wm + 4 * h, nw = n0 + 128 * wn + i;
  if (m0 + kNtBM <= M && n0 + kNtBN <= N) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = mw + 32 * mt + 8 * (e >> 2) + (e & 3);
        if (kOutBf16) {
          uint16_t* yr = static_cast<uint16_t*>(p.y) + row * N + nw;
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
            yr[32 * nt] = (uint16_t)(pack_bf16x2(acc[mt][nt][e], 0.0f) & 0xFFFFu);
        } else {
          float* yr = static_cast<float*>(p.y) + row * N + nw;
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) yr[32 * nt] = acc[mt][nt][e];
        }
      }
  } else {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int64_t n = nw + 32 * nt;
      if (n < N) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int64_t m = mw + 32 * mt + 8 * (e >> 2) + (e & 3);
            if (m < M) {
              if (kOutBf16)
                static_cast<uint16_t*>(p.y)[m * N + n] =
                    (uint16_t)(pack_bf16x2(acc[mt][nt][e], 0.0f) & 0xFFFFu);
              else
                static_cast<float*>(p.y)[m * N + n] = acc[mt][nt][e];
            }
          }
      }
    }
  }
}

// y[i] = sum over splits s = 0, 1, ... of part[s][i], in that order (fp32,
// or bf16 by round to nearest even of the fp32 sum); four elements a thread.
template <bool kOutBf16>
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ part,
                                                           int splits, int64_t n, void* y) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  if (i + 4 <= n && (n & 3) == 0) {
    f32x4_t v = *reinterpret_cast<const f32x4_t*>(part + i);
    for (int s = 1; s < splits; ++s) {
      const f32x4_t t = *reinterpret_cast<const f32x4_t*>(part + (int64_t)s * n + i);
      v = f32x4_t{v[0] + t[0], v[1] + t[1], v[2] + t[2], v[3] + t[3]};
    }
    if (kOutBf16)
      *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(y) + i) =
          u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    else
      *reinterpret_cast<f32x4_t*>(static_cast<float*>(y) + i) = v;
    return;
  }
  for (int64_t j = i; j < i + 4 && j < n; ++j) {
    float v = part[j];
    for (int s = 1; s < splits; ++s) v += part[(int64_t)s * n + j];
    if (kOutBf16)
      static_cast<uint16_t*>(y)[j] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
    else
      static_cast<float*>(y)[j] = v;
  }
}

}  // namespace

int gemm_nt_splits(int64_t M, int64_t N, int64_t Kr) {
  // Few output tiles (under a quarter of the 256 CUs) and a long reduction:
  // split the reduction so that the launch fills the GPU, at least 16 steps
  // of 32 per split.
  const int64_t tiles = ((M + kNtBM - 1) / kNtBM) * ((N + kNtBN - 1) / kNtBN);
  if (tiles >= 64) return 1;
  int s = (int)(256 / tiles);
  if (s > 8) s = 8;
  while (s > 1 && Kr / kNtBK / s < 16) --s;
  return s < 1 ? 1 : s;
}

bool gemm_nt_supported(int64_t Kr, int64_t lda, int64_t ldb, int64_t N, bool b_kslab) {
  // Buffer offsets (tile row offset + step offset) stay below 2^31.
  const int64_t lim = (int64_t)1 << 31;
  const bool b_ok = b_kslab ? 2 * N * Kr < lim : ldb % 8 == 0 && 2 * kNtBN * ldb + 2 * Kr < lim;
  return Kr >= kNtBK && Kr % kNtBK == 0 && lda % 8 == 0 && 2 * kNtBM * lda + 2 * Kr < lim && b_ok;
}

hipError_t launch_split_reduce(const float* part, int splits, int64_t n, void* y, bool y_bf16,
                               hipStream_t st) {
  const dim3 rg((unsigned)((n + 1023) / 1024));
  if (y_bf16)
    hipLaunchKernelGGL(split_reduce_kernel<true>, rg, dim3(256), 0, st, part, splits, n, y);
  else
    hipLaunchKernelGGL(split_reduce_kernel<false>, rg, dim3(256), 0, st, part, splits, n, y);
  return hipGetLastError();
}

hipError_t launch_gemm_nt(const uint16_t* a, int64_t lda, const uint16_t* b, int64_t ldb,
                          const uint16_t* e, const uint16_t* f, int64_t M, int64_t N, int64_t Kr,
                          int r, void* y, bool y_bf16, bool b_kslab, hipStream_t st,
                          int ksplit, float* part) {
  if (ksplit < 1 || !part) ksplit = 1;
  // every split must hold at least one step
  const int64_t steps = Kr / kNtBK;
  while (ksplit > 1 && (ksplit - 1) * ((steps + ksplit - 1) / ksplit) >= steps) --ksplit;
  const int tiles_m = (int)((M + kNtBM - 1) / kNtBM), tiles_n = (int)((N + kNtBN - 1) / kNtBN);
  const NtArgs args{a,       b,       e, f, y, M, N, Kr, lda, ldb, r, tiles_m, tiles_n, ksplit,
                    part, b_kslab ? 1 : 0};
  const dim3 grid((unsigned)(tiles_m * tiles_n * ksplit));
  if (ksplit > 1)
    hipLaunchKernelGGL((gemm_nt_kernel<false, true>), grid, dim3(256), 0, st, args);
  else if (y_bf16)
    hipLaunchKernelGGL((gemm_nt_kernel<true, false>), grid, dim3(256), 0, st, args);
  else
    hipLaunchKernelGGL((gemm_nt_kernel<false, false>), grid, dim3(256), 0, st, args);
  if (ksplit > 1) {
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_split_reduce(part, ksplit, M * N, y, y_bf16, st);
  }
  return hipGetLastError();
}


}  // namespace qlora
