// Fused NF4 dequantize-GEMM of the QLoRA linear layer for training batch
// sizes on gfx950: the 4-bit weight is expanded to bf16 tile by tile in
// registers, right before the matrix cores consume it, and never exists as a
// whole bf16 copy.
//
// [P1] "QLoRA" forward equation h = W_hat x + (alpha/r) B(Ax) and bullets
// (compute never happens in 4-bit: each block is expanded to bf16 right
// before its matmul); [P4] "The mechanism" (a block is dequantized
// immediately before its multiplication and discarded afterwards, so the
// high-precision copy only exists transiently for the block in use).
//
// y[M,N] = x[M,K] w_hat[N,K]^T + e[M,2r] [f|f][N,2r]^T, where e is the
// two-term bf16 split of (alpha/r) u and f = B^T (the same extension the
// dense stage uses). 256 x 256 output tiles, four waves; wave w owns all 256
// rows of output columns 64w .. 64w+63 of the tile (8 x 2 accumulators of
// v_mfma_f32_32x32x16_bf16), so each weight element is dequantized exactly
// once per workgroup, straight into the lane that feeds it to the MFMA:
//
//  - x arrives by direct-to-LDS loads (buffer_load_dwordx4 ... lds) in a
//    four-slot ring of 64-wide K "pairs" (one 64-weight block, two 32-wide
//    steps), 256 rows x 128 bytes per slot, 16-byte chunk c of row r at
//    position c ^ ((r >> 1) & 7): every load covers whole cache lines and
//    every fragment read touches all 64 banks once.
//  - The weight arrives as packed codes in registers. Within a pair the MFMA
//    reduction order is permuted so that lane half h of a 32x32x16 operand
//    always takes the 32 consecutive weights 32h .. 32h+31 of the block: one
//    16-byte code load per (row, block) and lane, one table per (row, block)
//    and lane pair. The A fragments read the matching chunks of x.
//  - Per (row, block) the 16 dequantized values bf16(fp32(L[i] * c1_hat))
//    are formed once (16 multiplies, 8 conversions) and held as two 16-byte
//    planes (low bytes, high bytes). A dword of 8 codes becomes the 8 bf16
//    values of one MFMA operand with 27 byte-permutes and masks (v_perm_b32
//    selects 4 bytes out of 8: the code's low 3 bits pick among 8 entries,
//    bit 3 picks the half of the table), so the expansion costs no LDS
//    traffic and overlaps the matrix cores of the previous pair's MFMAs.
//  - Workgroups map to tiles so that each XCD works on a compact group of
//    tiles (their x panels and code panels stay in that XCD's L2).
#include <type_traits>

#include "device.h"

namespace qlora {
namespace {

constexpr int kFBM = 256;   // output rows per tile (x rows)
constexpr int kFBN = 256;   // output columns per tile (weight rows)
constexpr int kFGroup = 4;  // tile rows per group in the tile order
constexpr int kSlot = 256 * 64;  // bf16 elements of one x pair slot (32 KB)

struct Nf4Args {
  const uint16_t* x;      // [M, K] row-major
  const uint8_t* codes;   // [N*K/2]
  const int8_t* q8;       // [N*K/64]
  const float* s2;        // [ceil(N*K/16384)]
  const uint16_t* e;      // [M, 2r]
  const uint16_t* f;      // [N, r]
  void* y;                // [M, N]
  int64_t M, N, K;
  int r;
  int tiles_m, tiles_n;
};

__device__ __forceinline__ uint32_t perm(uint32_t s0, uint32_t s1, uint32_t sel) {
  return __builtin_amdgcn_perm(s0, s1, sel);
}

// The 16 values bf16(fp32(L[i] * ch)) of one block as byte planes: pl[g]
// holds the low bytes of entries 4g .. 4g+3, ph[g] their high bytes.
__device__ __forceinline__ void nf4_planes(const Codebook& cb, float ch, uint32_t (&pl)[4],
                                           uint32_t (&ph)[4]) {
  uint32_t t[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) t[j] = pack_bf16x2(cb.level[2 * j] * ch, cb.level[2 * j + 1] * ch);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    pl[g] = perm(t[2 * g + 1], t[2 * g], 0x06040200u);
    ph[g] = perm(t[2 * g + 1], t[2 * g], 0x07050301u);
  }
}

// The 8 codes of dword d (nibble j = weight j) to the 8 bf16 values of one
// MFMA operand (weight j in bf16 slot j), through the planes of their block.
// Even and odd nibbles are looked up separately: the low 3 bits of a code
// select a byte among entries 0..7 and among 8..15, bit 3 picks one of the
// two, then the low and high bytes are interleaved into bf16 pairs.
__device__ __forceinline__ u32x4_t nf4_lut(uint32_t d, const uint32_t (&pl)[4],
                                           const uint32_t (&ph)[4]) {
  const uint32_t se = d & 0x07070707u;
  const uint32_t d4 = d >> 4;
  const uint32_t so = d4 & 0x07070707u;
  const uint32_t ke = ((d >> 1) & 0x04040404u) | 0x03020100u;
  const uint32_t ko = ((d4 >> 1) & 0x04040404u) | 0x03020100u;
  const uint32_t le = perm(perm(pl[3], pl[2], se), perm(pl[1], pl[0], se), ke);
  const uint32_t he = perm(perm(ph[3], ph[2], se), perm(ph[1], ph[0], se), ke);
  const uint32_t lo = perm(perm(pl[3], pl[2], so), perm(pl[1], pl[0], so), ko);
  const uint32_t ho = perm(perm(ph[3], ph[2], so), perm(ph[1], ph[0], so), ko);
  const uint32_t e01 = perm(he, le, 0x05010400u), e23 = perm(he, le, 0x07030602u);
  const uint32_t o01 = perm(ho, lo, 0x05010400u), o23 = perm(ho, lo, 0x07030602u);
  return u32x4_t{perm(o01, e01, 0x05040100u), perm(o01, e01, 0x07060302u),
                 perm(o23, e23, 0x05040100u), perm(o23, e23, 0x07060302u)};
}

// Tile of workgroup `wg`: workgroups are dealt to the eight XCDs round robin
// (wg % 8); each XCD gets a contiguous range of the tile order, which walks
// groups of kFGroup tile rows column by column.
__device__ __forceinline__ void nf4_tile(int wg, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int T = tiles_m * tiles_n;
  const int xcd = wg & 7, idx = wg >> 3;
  const int per = T >> 3, extra = T & 7;
  const int t = xcd * per + (xcd < extra ? xcd : extra) + idx;
  const int group = t / (kFGroup * tiles_n);
  const int first = group * kFGroup;
  const int rows = tiles_m - first < kFGroup ? tiles_m - first : kFGroup;
  const int in = t - group * kFGroup * tiles_n;
  tm = first + in % rows;
  tn = in / rows;
}

// s_waitcnt: at most n vector-memory operations in flight, no LDS operation.
template <int n>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4));
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = (int)(bytes < (int64_t)0x7FFFFFFF ? (bytes > 0 ? bytes : 0) : 0x7FFFFFFF);
  return __builtin_amdgcn_make_buffer_rsrc((void*)uniform_ptr(base), (short)0, n, 0x00020000);
}

template <int S, int N, typename T>
__device__ __forceinline__ T* pick(T* const (&arr)[N]) {
  static_assert(S >= 0 && S < N, "slot index");
  return arr[S];
}

// Codes and block constants of one pair (block) for the lane's two rows.
struct PairCodes {
  u32x4_t c[2];  // 16 bytes of codes per row: weights 32h .. 32h+31 of the block
  int q[2];      // absmax code byte
  float s[2];    // second-level scale of the block's group
};

template <int kFmt, bool kOutBf16>
__global__ __launch_bounds__(256, 1) void gemm_nf4_fwd_kernel(Nf4Args p, Codebook cb) {
  __shared__ __attribute__((aligned(1024))) uint16_t sa0[kSlot];
  __shared__ __attribute__((aligned(1024))) uint16_t sa1[kSlot];
  __shared__ __attribute__((aligned(1024))) uint16_t sa2[kSlot];
  __shared__ __attribute__((aligned(1024))) uint16_t sa3[kSlot];
  uint16_t* const sa[4] = {sa0, sa1, sa2, sa3};
  const int tid = threadIdx.x, lane = tid & 63, i = lane & 31, h = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int tm, tn;
  nf4_tile((int)blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t m0 = (int64_t)tm * kFBM, n0 = (int64_t)tn * kFBN;
  const int npairs = (int)(K / 64);
  const int64_t KB = K / 64;

  // x by direct-to-LDS loads: wave w loads rows 64w + 8q + L/8 (q = 0..7) of
  // each pair, lane L into position L%8 (global chunk (L%8) ^ ((row>>1)&7)),
  // 128 bytes per pair of scalar offset. Rows past M read row M-1 (never
  // stored).
  uint32_t aoff[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int row = 64 * w + 8 * q + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    const int64_t ar = m0 + row < M ? row : M - 1 - m0;
    aoff[q] = (uint32_t)(ar * K * 2 + 16 * c);
  }
  const __amdgpu_buffer_rsrc_t xres = make_rsrc(p.x + m0 * K, ((M - 1 - m0) * K + K) * 2);
  typedef __attribute__((address_space(3))) void lds_void;
  auto dma_x = [&](int q, int pair, uint16_t* slot) {
    const int ps = pair < npairs ? pair : npairs - 1;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(xres, (lds_void*)(slot + (64 * w + 8 * q) * 64), 16,
                                             aoff[q], 128 * ps, 0, 0);
  };

  // The weight: lane (i, h) of wave w feeds rows n0 + 64w + 32nt + i (nt =
  // 0, 1). Code and constant loads go through buffer resources that end at
  // the weight's last row, so rows past N read zeros (never stored).
  const __amdgpu_buffer_rsrc_t cres = make_rsrc(p.codes + n0 * (K / 2), (N - n0) * (K / 2));
  const __amdgpu_buffer_rsrc_t qres = make_rsrc(p.q8 + n0 * KB, (N - n0) * KB);
  const __amdgpu_buffer_rsrc_t sres = make_rsrc(p.s2, ((N * KB + 255) / 256) * 4);
  uint32_t coff[2], qoff[2];
  int64_t bfirst[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int row = 64 * w + 32 * nt + i;
    coff[nt] = (uint32_t)(row * (K / 2) + 16 * h);
    qoff[nt] = (uint32_t)(row * KB);
    bfirst[nt] = (n0 + row) * KB;  // global block index of the row's first block
  }
  auto load_pair = [&](int pair, PairCodes& pc) {
    const int ps = pair < npairs ? pair : npairs - 1;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      pc.c[nt] = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(cres, coff[nt], 32 * ps, 0));
      pc.q[nt] = (int)(int8_t)__builtin_amdgcn_raw_buffer_load_b8(qres, qoff[nt], ps, 0);
      const int64_t b = bfirst[nt] + ps;
      pc.s[nt] = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(sres, (uint32_t)((b >> 8) * 4), 0, 0));
    }
  };
  // Dequantize one pair: B operand (nt, t, s) of the pair, t = step, s =
  // substep, is dword 2t+s of the row's 16 code bytes.
  auto dequant_pair = [&](const PairCodes& pc, u32x4_t (&bo)[2][4]) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      uint32_t pl[4], ph[4];
      nf4_planes(cb, q8_value(pc.q[nt], kFmt) * pc.s[nt], pl, ph);
      bo[nt][0] = nf4_lut(pc.c[nt].x, pl, ph);
      bo[nt][1] = nf4_lut(pc.c[nt].y, pl, ph);
      bo[nt][2] = nf4_lut(pc.c[nt].z, pl, ph);
      bo[nt][3] = nf4_lut(pc.c[nt].w, pl, ph);
    }
  };

  // A fragment of (mt, t, s): tile row 32mt + i, chunk 4h + 2t + s of the
  // pair, at position chunk ^ ((i >> 1) & 7).
  const int swa = (i >> 1) & 7;
  int fa[4];
#pragma unroll
  for (int ts = 0; ts < 4; ++ts) fa[ts] = i * 64 + 8 * ((4 * h + ts) ^ swa);

  f32x16_t acc[8][2];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mt][nt][e] = 0.0f;

  // Prologue: x pairs 0 and 1, codes of pairs 0 and 1; pair 0's operands.
  PairCodes cA, cB;
#pragma unroll
  for (int q = 0; q < 8; ++q) dma_x(q, 0, sa0);
  load_pair(0, cA);
#pragma unroll
  for (int q = 0; q < 8; ++q) dma_x(q, 1, sa1);
  load_pair(1, cB);
  u32x4_t bA[2][4], bB[2][4];
  dequant_pair(cA, bA);  // the compiler waits for pair 0's codes
  wait_vm_lgkm0<14>();   // pair 0's x has landed (pair 1 and its codes may fly)
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  u32x4_t a0[8], a1[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
    a0[mt] = *reinterpret_cast<const u32x4_t*>(&sa0[fa[0] + 2048 * mt]);

  // One pair (a 64-weight block): four substeps q = 2t + s. Substep q runs
  // 16 MFMAs on (a_cur, bc[.][q]) while the fragments of substep q+1 (or of
  // the next pair's first substep, from the next slot) are read and a
  // quarter of the next pair's operands is dequantized: in step t the
  // operands of row nt = t, its table in substep 0, dwords 0-1 in substep 0
  // and 2-3 in substep 1. Step t issues four x loads of pair + 2; step 0
  // also issues the code loads of pair + 2. Each step ends with a wait for
  // all but its own loads and one barrier. The last pair dequantizes a
  // repeat of itself (codes of pair + 1 are clamped): one basic block per
  // pair keeps the VALU work interleaved with the MFMAs.
  auto pair_fn = [&](int pr, auto slotc, u32x4_t (&bc)[2][4], u32x4_t (&bn)[2][4],
                     PairCodes& cuse, PairCodes& cload) {
    constexpr int SL = decltype(slotc)::value;
    uint16_t* const acur = pick<SL>(sa);
    uint16_t* const anxt = pick<(SL + 1) & 3>(sa);
    uint16_t* const ald = pick<(SL + 2) & 3>(sa);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      uint32_t pl[4], ph[4];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int qs = 2 * t + s;
        u32x4_t(&acu)[8] = (qs & 1) ? a1 : a0;
        u32x4_t(&anx)[8] = (qs & 1) ? a0 : a1;
        uint16_t* const src = qs == 3 ? anxt : acur;
        const int fnext = fa[(qs + 1) & 3];
        if (qs == 0) load_pair(pr + 2, cload);
        if (s == 0) nf4_planes(cb, q8_value(cuse.q[t], kFmt) * cuse.s[t], pl, ph);
        const uint32_t d0 = s ? cuse.c[t].z : cuse.c[t].x;
        const uint32_t d1 = s ? cuse.c[t].w : cuse.c[t].y;
        bn[t][2 * s] = nf4_lut(d0, pl, ph);
        bn[t][2 * s + 1] = nf4_lut(d1, pl, ph);
#pragma unroll
        for (int g = 0; g < 16; ++g) {
          const int mt = g >> 1, nt = g & 1;
          acc[mt][nt] = mfma_32x32x16(acu[mt], bc[nt][qs], acc[mt][nt]);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
          if (g & 1) {
            anx[g >> 1] = *reinterpret_cast<const u32x4_t*>(&src[fnext + 2048 * (g >> 1)]);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          if (qs == 0 && g == 2) __builtin_amdgcn_sched_group_barrier(0x020, 6, 0);
          if ((g & 7) == 7) {
            dma_x(4 * t + 2 * s + (g >> 3), pr + 2, ald);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (t == 0)
        wait_vm_lgkm0<10>();  // all but this step's 4 x loads and 6 code loads
      else
        wait_vm_lgkm0<4>();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  int pr = 0;
  for (; pr + 4 <= npairs; pr += 4) {
    pair_fn(pr + 0, S0(), bA, bB, cB, cA);
    pair_fn(pr + 1, S1(), bB, bA, cA, cB);
    pair_fn(pr + 2, S2(), bA, bB, cB, cA);
    pair_fn(pr + 3, S3(), bB, bA, cA, cB);
  }
  if (pr + 0 < npairs) pair_fn(pr + 0, S0(), bA, bB, cB, cA);
  if (pr + 1 < npairs) pair_fn(pr + 1, S1(), bB, bA, cA, cB);
  if (pr + 2 < npairs) pair_fn(pr + 2, S2(), bA, bB, cB, cA);
  wait_vm_lgkm0<0>();  // direct-to-LDS loads must land before the workgroup ends

  // Adapter term: 2r extra reduction elements, 16 per MFMA; lane half h
  // supplies extension elements 16q + 8h .. +7; column jj of e pairs with
  // column jj mod r of f.
  const int r = p.r, r2 = 2 * r;
  for (int q = 0; q < r2 / 16; ++q) {
    const int jj = 16 * q + 8 * h, jb = jj % r;
    u32x4_t ev[8], fv[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int64_t n = n0 + 64 * w + 32 * nt + i;
      fv[nt] = n < N ? *reinterpret_cast<const u32x4_t*>(p.f + n * r + jb) : zero4();
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const int64_t m = m0 + 32 * mt + i;
      ev[mt] = m < M ? *reinterpret_cast<const u32x4_t*>(p.e + m * r2 + jj) : zero4();
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = mfma_32x32x16(ev[mt], fv[nt], acc[mt][nt]);
  }

  // Output: accumulator element e of (mt, nt) is row 32mt + 8(e/4) + 4h +
  // e%4, column 64w + 32nt + i of the tile.
  const int64_t mw = m0 + 4 * h, nw = n0 + 64 * w + i;
  if (m0 + kFBM <= M && n0 + kFBN <= N) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = mw + 32 * mt + 8 * (e >> 2) + (e & 3);
        if (kOutBf16) {
          uint16_t* yr = static_cast<uint16_t*>(p.y) + row * N + nw;
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
            yr[32 * nt] = (uint16_t)(pack_bf16x2(acc[mt][nt][e], 0.0f) & 0xFFFFu);
        } else {
          float* yr = static_cast<float*>(p.y) + row * N + nw;
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) yr[32 * nt] = acc[mt][nt][e];
        }
      }
  } else {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int64_t n = nw + 32 * nt;
      if (n < N) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
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

template <int kFmt>
hipError_t launch_fwd_fmt(const Nf4Args& a, bool y_bf16, const Codebook& cb, hipStream_t st) {
  const dim3 grid((unsigned)(a.tiles_m * a.tiles_n));
  if (y_bf16)
    hipLaunchKernelGGL((gemm_nf4_fwd_kernel<kFmt, true>), grid, dim3(256), 0, st, a, cb);
  else
    hipLaunchKernelGGL((gemm_nf4_fwd_kernel<kFmt, false>), grid, dim3(256), 0, st, a, cb);
  return hipGetLastError();
}

}  // namespace

bool gemm_nf4_supported(int64_t M, int64_t N, int64_t K) {
  // 32-bit buffer offsets: one tile's x rows and code rows, and block indices.
  const int64_t lim = (int64_t)1 << 31;
  return M >= 1 && N >= 1 && K >= 64 && K % 64 == 0 && 2 * kFBM * K < lim &&
         kFBN * (K / 2) + K < lim && N * (K / 64) < lim;
}

hipError_t launch_gemm_nf4_fwd(const uint16_t* x, const uint8_t* codes, const int8_t* q8,
                               const float* s2, const uint16_t* e, const uint16_t* f, int64_t M,
                               int64_t N, int64_t K, int r, void* y, bool y_bf16,
                               const Codebook& cb, hipStream_t st) {
  Nf4Args a{x, codes, q8, s2, e, f, y, M, N, K, r,
            (int)((M + kFBM - 1) / kFBM), (int)((N + kFBN - 1) / kFBN)};
  switch (cb.dq_format) {
    case kDqUint8: return launch_fwd_fmt<kDqUint8>(a, y_bf16, cb, st);
    case kDqE4m3: return launch_fwd_fmt<kDqE4m3>(a, y_bf16, cb, st);
    default: return launch_fwd_fmt<kDqInt8>(a, y_bf16, cb, st);
  }
}

}  // namespace qlora
