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
//    loads (global_load_lds_dwordx4) in a four-deep ring of 32-wide K steps;
//    the fragments of the next substep are read while the MFMAs of the
//    current one run, so the one barrier per step never waits on LDS.
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

template <int S>
__device__ __forceinline__ uint16_t* pick4(uint16_t* s0, uint16_t* s1, uint16_t* s2, uint16_t* s3) {
  if constexpr (S == 0) return s0;
  else if constexpr (S == 1) return s1;
  else if constexpr (S == 2) return s2;
  else return s3;
}

// Operand tile layout in LDS (per stage: the a tile, then the b tile): tile
// row r (0..255) holds 32 bf16 = 64 bytes; its 16-byte chunk c sits at slot
// c ^ ((r >> 2) & 3). A fragment read (32 rows, one chunk each, 16 lanes per
// LDS cycle) then touches 16 distinct 16-byte bank groups.
// Direct-to-LDS load q (0..15) of an operand tile covers tile rows
// 16q .. 16q+15: lane L writes LDS bytes [16L, 16L+16) of that 1 KB window,
// i.e. row 16q + L/4, slot L%4, so it reads global chunk (L%4) ^ ((row>>2)&3).
template <bool kOutBf16>
__global__ __launch_bounds__(256, 1) void gemm_nt_kernel(NtArgs p) {
  __shared__ __attribute__((aligned(1024))) uint16_t st0[2 * kNtOp];
  __shared__ __attribute__((aligned(1024))) uint16_t st1[2 * kNtOp];
  __shared__ __attribute__((aligned(1024))) uint16_t st2[2 * kNtOp];
  __shared__ __attribute__((aligned(1024))) uint16_t st3[2 * kNtOp];
  const int tid = threadIdx.x, lane = tid & 63, i = lane & 31, h = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = w >> 1, wn = w & 1;
  int tm, tn;
  nt_tile((int)blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
  const int64_t M = p.M, N = p.N;
  const int64_t m0 = (int64_t)tm * kNtBM, n0 = (int64_t)tn * kNtBN;
  const int nsteps = (int)(p.Kr / kNtBK);

  // Direct-to-LDS role: wave w loads windows 4w .. 4w+3 of both tiles through
  // buffer resources based at the tile's first row: the per-lane byte offset
  // is fixed, the step's offset (64 bytes per step) is a scalar. Rows past
  // the matrix read its last row (their results are never stored).
  uint32_t aoff[4], boff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 16 * (4 * w + j) + (lane >> 2);
    const int c = (lane & 3) ^ ((row >> 2) & 3);
    const int64_t ar = m0 + row < M ? row : M - 1 - m0;
    const int64_t br = n0 + row < N ? row : N - 1 - n0;
    aoff[j] = (uint32_t)(ar * p.lda * 2 + 16 * c);
    boff[j] = (uint32_t)(br * (p.b_kslab ? 64 : p.ldb * 2) + 16 * c);
  }
  const __amdgpu_buffer_rsrc_t ares = __builtin_amdgcn_make_buffer_rsrc(
      (void*)uniform_ptr(p.a + m0 * p.lda), (short)0, (int)0x7FFFFFFF, 0x00020000);
  const __amdgpu_buffer_rsrc_t bres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)uniform_ptr(p.b + n0 * (p.b_kslab ? 32 : p.ldb)), (short)0, (int)0x7FFFFFFF,
      0x00020000);
  const int bstep = p.b_kslab ? (int)(64 * N) : 64;  // bytes from one step to the next
  const int win = 4 * w * 512;  // element offset of this wave's first window
  typedef __attribute__((address_space(3))) void lds_void;
  auto dma = [&](int j, int kb, uint16_t* stage) {
    const int ks = kb < nsteps ? kb : nsteps - 1;
    if (j < 4)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ares, (lds_void*)(stage + win + 512 * j), 16, aoff[j],
                                               64 * ks, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(bres, (lds_void*)(stage + kNtOp + win + 512 * (j - 4)),
                                               16, boff[j - 4], bstep * ks, 0, 0);
  };
  auto issue = [&](int kb, uint16_t* stage) {
#pragma unroll
    for (int j = 0; j < 8; ++j) dma(j, kb, stage);
  };

  // Fragment reads: A fragment (mt, substep s): tile row 128wm + 32mt + i,
  // chunk 2s + h; B fragment (nt, s): tile row 128wn + 32nt + i. Bits 2..3 of
  // the row are those of i, so the slot is (2s + h) ^ ((i >> 2) & 3).
  const int sw = (i >> 2) & 3;
  const int fa0 = (128 * wm + i) * 32 + 8 * (h ^ sw);
  const int fa1 = (128 * wm + i) * 32 + 8 * ((2 + h) ^ sw);
  const int fb0 = kNtOp + (128 * wn + i) * 32 + 8 * (h ^ sw);
  const int fb1 = kNtOp + (128 * wn + i) * 32 + 8 * ((2 + h) ^ sw);

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

  // Prologue: steps 0, 1, 2 in flight; wait for 0 and 1; fragments (0, 0).
  issue(0, st0);
  issue(1, st1);
  issue(2, st2);
  wait_vmem_lgkm0<8>();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  u32x4_t a0[4], b0[4], a1[4], b1[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    a0[t] = *reinterpret_cast<const u32x4_t*>(&st0[fa0 + 1024 * t]);
    b0[t] = *reinterpret_cast<const u32x4_t*>(&st0[fb0 + 1024 * t]);
  }

  // One step on stage S: loads for step kb+3 go to stage S+3 (read last in
  // the previous step, before its barrier), one after every fourth MFMA.
  // Substep 0 computes on (a0, b0) while (kb, 1) is read into (a1, b1);
  // substep 1 computes on (a1, b1) while (kb+1, 0) is read from stage S+1
  // (complete since the previous barrier).
  auto step = [&](int kb, auto sc) {
    constexpr int S = decltype(sc)::value;
    uint16_t* const cur = pick4<S>(st0, st1, st2, st3);
    uint16_t* const nxt = pick4<(S + 1) & 3>(st0, st1, st2, st3);
    uint16_t* const ld = pick4<(S + 3) & 3>(st0, st1, st2, st3);
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      const int mt = g >> 2, nt = g & 3;
      acc[mt][nt] = mfma_32x32x16(a0[mt], b0[nt], acc[mt][nt]);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (g < 8) {
        const int t = g >> 1;
        if (g & 1)
          b1[t] = *reinterpret_cast<const u32x4_t*>(&cur[fb1 + 1024 * t]);
        else
          a1[t] = *reinterpret_cast<const u32x4_t*>(&cur[fa1 + 1024 * t]);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      if ((g & 3) == 3) {
        dma(g >> 2, kb + 3, ld);
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
          b0[t] = *reinterpret_cast<const u32x4_t*>(&nxt[fb0 + 1024 * t]);
        else
          a0[t] = *reinterpret_cast<const u32x4_t*>(&nxt[fa0 + 1024 * t]);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      if ((g & 3) == 3) {
        dma(4 + (g >> 2), kb + 3, ld);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // Loads of step kb+2 complete (kb+3 may still fly), this wave's LDS reads
    // done; then every wave's stage kb+2 is visible and stage S is free.
    wait_vmem_lgkm0<8>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  int kb = 0;
  for (; kb + 4 <= nsteps; kb += 4) {
    step(kb, std::integral_constant<int, 0>());
    step(kb + 1, std::integral_constant<int, 1>());
    step(kb + 2, std::integral_constant<int, 2>());
    step(kb + 3, std::integral_constant<int, 3>());
  }
  if (kb < nsteps) step(kb, std::integral_constant<int, 0>());
  if (kb + 1 < nsteps) step(kb + 1, std::integral_constant<int, 1>());
  if (kb + 2 < nsteps) step(kb + 2, std::integral_constant<int, 2>());
  // Direct-to-LDS loads still in flight must land before the workgroup ends.
  wait_vmem_lgkm0<0>();

  // Adapter term as 2r extra reduction elements, 16 per MFMA.
  ext_mfma(e0, f0);
  ext_mfma(e1, f1);
  for (int q = 2; q < r2 / 16; ++q) {
    ext_load(q, e0, f0);
    ext_mfma(e0, f0);
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

}  // namespace

bool gemm_nt_supported(int64_t Kr, int64_t lda, int64_t ldb, int64_t N, bool b_kslab) {
  // Buffer offsets (tile row offset + step offset) stay below 2^31.
  const int64_t lim = (int64_t)1 << 31;
  const bool b_ok = b_kslab ? 2 * N * Kr < lim : ldb % 8 == 0 && 2 * kNtBN * ldb + 2 * Kr < lim;
  return Kr >= kNtBK && Kr % kNtBK == 0 && lda % 8 == 0 && 2 * kNtBM * lda + 2 * Kr < lim && b_ok;
}

hipError_t launch_gemm_nt(const uint16_t* a, int64_t lda, const uint16_t* b, int64_t ldb,
                          const uint16_t* e, const uint16_t* f, int64_t M, int64_t N, int64_t Kr,
                          int r, void* y, bool y_bf16, bool b_kslab, hipStream_t st) {
  const int tiles_m = (int)((M + kNtBM - 1) / kNtBM), tiles_n = (int)((N + kNtBN - 1) / kNtBN);
  const NtArgs args{a, b, e, f, y, M, N, Kr, lda, ldb, r, tiles_m, tiles_n, b_kslab ? 1 : 0};
  const dim3 grid((unsigned)(tiles_m * tiles_n));
  if (y_bf16)
    hipLaunchKernelGGL(gemm_nt_kernel<true>, grid, dim3(256), 0, st, args);
  else
    hipLaunchKernelGGL(gemm_nt_kernel<false>, grid, dim3(256), 0, st, args);
  return hipGetLastError();
}


}  // namespace qlora
