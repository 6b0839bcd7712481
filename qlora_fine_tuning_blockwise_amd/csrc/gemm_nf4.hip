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
// The two selector constants in VGPRs (kb4 = 0x04040404, kid = 0x03020100):
// a VOP3 operation on gfx950 reads at most one scalar, so with both in
// scalars (x & kb4) | kid would take two instructions instead of one
// v_and_or_b32.
__device__ __forceinline__ u32x4_t nf4_lut(uint32_t d, const uint32_t (&pl)[4],
                                           const uint32_t (&ph)[4], uint32_t kb4, uint32_t kid) {
  const uint32_t se = d & 0x07070707u;
  const uint32_t d4 = d >> 4;
  const uint32_t so = d4 & 0x07070707u;
  const uint32_t ke = ((d >> 1) & kb4) | kid;
  const uint32_t ko = ((d4 >> 1) & kb4) | kid;
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

// Value of an absmax code byte b (0..255, loaded zero-extended) in format
// kFmt, exact in fp32. The signed byte is read as (b ^ 0x80) - 128, so that
// the compiler never turns the byte load into a sign-extending load issued
// again next to this use.
template <int kFmt>
__device__ __forceinline__ float absmax_value(int b) {
  if constexpr (kFmt == kDqInt8) {
    return (float)(b ^ 0x80) - 128.0f;
  } else {
    return q8_value(b, kFmt);
  }
}

// Codes of one pair (block) for the lane's two rows, and the block constants
// of the row whose table this lane builds (row h; the lane pair (i, 0),
// (i, 1) builds one table each and they swap).
struct PairCodes {
  u32x4_t c[2];  // 16 bytes of codes per row: weights 32h .. 32h+31 of the block
  int q;         // absmax code byte of row h, zero-extended
  float s;       // second-level scale of row h's block group
  float ch;      // c1_hat of row h: value(q) * s, formed once the loads have landed
};

// Dequantization tables of one pair for the lane's two rows (byte planes).
struct Planes {
  uint32_t lo[2][4], hi[2][4];
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
  uint32_t coff[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) coff[nt] = (uint32_t)((64 * w + 32 * nt + i) * (K / 2) + 16 * h);
  const int trow = 64 * w + 32 * h + i;  // the row whose table this lane builds
  const uint32_t qoff = (uint32_t)(trow * KB);
  const uint32_t bfirst = (uint32_t)((n0 + trow) * KB);  // N * K/64 < 2^31 (gemm_nf4_supported)
  auto load_pair = [&](int pair, PairCodes& pc) {
    const int ps = pair < npairs ? pair : npairs - 1;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
      pc.c[nt] = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(cres, coff[nt], 32 * ps, 0));
    pc.q = (int)__builtin_amdgcn_raw_buffer_load_b8(qres, qoff, ps, 0);
    pc.s = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(sres, ((bfirst + (uint32_t)ps) >> 8) * 4, 0, 0));
  };
  // mbcnt_lo(0, c) is c in every lane, but the compiler treats it as
  // lane-varying and keeps it in a VGPR.
  const uint32_t kb4 = __builtin_amdgcn_mbcnt_lo(0u, 0x04040404u);
  const uint32_t kid = __builtin_amdgcn_mbcnt_lo(0u, 0x03020100u);
  // Planes of row nt of a pair, and the operand of substep d (dword d of the
  // row's 16 code bytes) for both rows.
  // The planes of both rows: this lane builds row h's, then lanes l and
  // l + 32 swap halves (v_permlane32_swap: the upper 32 lanes of the first
  // operand trade places with the lower 32 lanes of the second), which
  // leaves row 0's planes in the first result and row 1's in the second.
  auto planes = [&](const PairCodes& pc, Planes& pl) {
    uint32_t lo[4], hi[4];
    nf4_planes(cb, pc.ch, lo, hi);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const auto xl = __builtin_amdgcn_permlane32_swap(lo[g], lo[g], false, false);
      const auto xh = __builtin_amdgcn_permlane32_swap(hi[g], hi[g], false, false);
      pl.lo[0][g] = xl[0];
      pl.lo[1][g] = xl[1];
      pl.hi[0][g] = xh[0];
      pl.hi[1][g] = xh[1];
    }
  };
  auto operands = [&](const PairCodes& pc, const Planes& pl, int d, u32x4_t (&bo)[2]) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const uint32_t c = d == 0 ? pc.c[nt].x : d == 1 ? pc.c[nt].y : d == 2 ? pc.c[nt].z
                                                                           : pc.c[nt].w;
      bo[nt] = nf4_lut(c, pl.lo[nt], pl.hi[nt], kb4, kid);
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

  // Prologue: x pairs 0 and 1, codes of pairs 0 and 1; pair 0's planes and
  // the operands of its first substep.
  PairCodes c0, c1, c2;
  Planes pA, pB;
#pragma unroll
  for (int q = 0; q < 8; ++q) dma_x(q, 0, sa0);
  load_pair(0, c0);
  load_pair(1, c1);
#pragma unroll
  for (int q = 0; q < 8; ++q) dma_x(q, 1, sa1);
  u32x4_t b0[2], b1[2];
  c0.ch = absmax_value<kFmt>(c0.q) * c0.s;  // the compiler waits for pair 0's codes
  planes(c0, pA);
  operands(c0, pA, 0, b0);
  wait_vm_lgkm0<8>();  // pair 0's x and pair 1's codes have landed (pair 1's x may fly)
  c1.ch = absmax_value<kFmt>(c1.q) * c1.s;
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  u32x4_t a0[8], a1[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
    a0[mt] = *reinterpret_cast<const u32x4_t*>(&sa0[fa[0] + 2048 * mt]);

  // One pair (a 64-weight block): four substeps q = 2t + s. Substep q runs
  // 16 MFMAs on (a_cur, b_cur) while the x fragments of substep q+1 (of the
  // next pair's first substep, from the next slot, when q = 3) are read and
  // the weight operands of substep q+1 are dequantized: dwords 1..3 of this
  // pair's codes through its planes, then dword 0 of the next pair's. The
  // next pair's planes are built in substeps 1 (row 0) and 2 (row 1). Step t
  // issues four x loads of pair + 2; substep 0 also issues the code loads of
  // pair + 2. Each step ends with a wait for all but its own loads and one
  // barrier. The last pair prepares a repeat of itself (the loads clamp to
  // the last pair), so each pair stays one basic block.
  auto pair_fn = [&](int pr, auto slotc, const PairCodes& cc, const PairCodes& cn,
                     PairCodes& cl, const Planes& pc, Planes& pn) {
    constexpr int SL = decltype(slotc)::value;
    uint16_t* const acur = pick<SL>(sa);
    uint16_t* const anxt = pick<(SL + 1) & 3>(sa);
    uint16_t* const ald = pick<(SL + 2) & 3>(sa);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int qs = 2 * t + s;
        u32x4_t(&acu)[8] = (qs & 1) ? a1 : a0;
        u32x4_t(&anx)[8] = (qs & 1) ? a0 : a1;
        u32x4_t(&bcu)[2] = (qs & 1) ? b1 : b0;
        u32x4_t(&bnx)[2] = (qs & 1) ? b0 : b1;
        uint16_t* const src = qs == 3 ? anxt : acur;
        const int fnext = fa[(qs + 1) & 3];
        if (qs == 0) load_pair(pr + 2, cl);
        if (qs == 1) planes(cn, pn);
        if (qs < 3)
          operands(cc, pc, qs + 1, bnx);
        else
          operands(cn, pn, 0, bnx);
#pragma unroll
        for (int g = 0; g < 16; ++g) {
          const int mt = g >> 1, nt = g & 1;
          acc[mt][nt] = mfma_32x32x16(acu[mt], bcu[nt], acc[mt][nt]);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
          if (g & 1) {
            anx[g >> 1] = *reinterpret_cast<const u32x4_t*>(&src[fnext + 2048 * (g >> 1)]);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          if (qs == 0 && g == 2) __builtin_amdgcn_sched_group_barrier(0x020, 4, 0);
          if ((g & 7) == 7) {
            dma_x(4 * t + 2 * s + (g >> 3), pr + 2, ald);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (t == 0)
        wait_vm_lgkm0<8>();  // all but this step's 4 x loads and 4 code loads
      else
        wait_vm_lgkm0<4>();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
    // pair + 2's constants have landed: form its c1_hat now, so that no
    // load result crosses the loop's back edge still pending
    cl.ch = absmax_value<kFmt>(cl.q) * cl.s;
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  // Pair p: codes p, p+1 in use, p+2 loading (three sets, rotating); planes
  // of p in use, p+1 being built (two sets); x slot p % 4.
  int pr = 0;
  for (; pr + 4 <= npairs; pr += 4) {
    pair_fn(pr + 0, S0(), c0, c1, c2, pA, pB);
    pair_fn(pr + 1, S1(), c1, c2, c0, pB, pA);
    pair_fn(pr + 2, S2(), c2, c0, c1, pA, pB);
    pair_fn(pr + 3, S3(), c0, c1, c2, pB, pA);
    // four pairs move the code sets on by one: rename for the next round
    const PairCodes t0 = c0;
    c0 = c1;
    c1 = c2;
    c2 = t0;
  }
  if (pr + 0 < npairs) pair_fn(pr + 0, S0(), c0, c1, c2, pA, pB);
  if (pr + 1 < npairs) pair_fn(pr + 1, S1(), c1, c2, c0, pB, pA);
  if (pr + 2 < npairs) pair_fn(pr + 2, S2(), c2, c0, c1, pA, pB);
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
