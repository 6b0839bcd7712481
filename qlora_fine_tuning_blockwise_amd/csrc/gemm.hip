// Dequantize-into-MFMA kernels of the QLoRA linear layer on gfx950, used for
// 16 < M < 512 rows (from 512 rows on the weight is dequantized once and the
// plain GEMM of gemm_nt.hip runs instead).
//
// [P1] "QLoRA" forward equation h = W_hat x + (alpha/r) B(Ax) and bullets
// ("Compute never happens in 4-bit": the weight is dequantized to bf16 just in
// time for the matmul); [P2] s3 "The Backward Pass Through Quantization"
// (dequantize on the fly, compute in bf16, only adapter gradients).
//
//  - Forward (gemm_fwd_kernel): 512 x 128 output tiles; the NF4 weight tile
//    is dequantized once per workgroup into a bf16 LDS tile shared by the four
//    waves; x is staged through LDS with coalesced loads.
//  - Backward dX (gemm_bwd_kernel): 256 x 256 output tiles; each wave owns
//    all 256 rows of its 64 output columns and dequantizes its weight
//    fragments in registers, straight into the MFMA B operand; the dY tile
//    arrives by direct-to-LDS loads. gemm_bwd_general_kernel covers N not a
//    multiple of 8.
//  - All use v_mfma_f32_32x32x16_bf16 (16x16x32 in the general kernel) with
//    fp32 accumulators. A code is dequantized by one LDS lookup in a 16-entry
//    bf16 table (bf16(L[i] * c1_hat)) of its (row, block), exactly as the
//    standalone dequant kernel.
//  - The LoRA term rides the same accumulators as extra reduction steps:
//    [s*u_hi | s*u_lo] (bf16 split of the fp32 adapter product) times the
//    matching adapter columns.
#include <type_traits>

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

// Bytes of a 256 x 64 bf16 activation tile staged by direct-to-LDS loads
// (global_load_lds_dwordx4: lane l of an instruction writes LDS bytes
// [16l, 16l+16) of that instruction's 1 KB window). Rows are 128 B; 16-byte
// chunk c of row r sits at chunk slot c ^ (r & 7), so the 16 rows one
// A-fragment read touches spread over all banks. Rows past M are clamped to
// row M-1 (their results are never stored).
constexpr int kTileBytes = 256 * 128;

// Static choice among three LDS buffers, so that every access names its
// __shared__ array directly (keeps the buffers distinguishable to the
// compiler's alias analysis, which decides where direct-to-LDS loads must be
// waited for).
template <int S, typename T>
__device__ __forceinline__ T* pick3(T* a, T* b, T* c) {
  if constexpr (S == 0)
    return a;
  else if constexpr (S == 1)
    return b;
  else
    return c;
}

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
  // Reduction split (nsplit > 1): workgroup z takes the z-th range of whole
  // 64-weight blocks of K and stores fp32 sums for rows m < M to
  // part + z*M*N (the adapter term rides in split 0); a reduce launch adds
  // the splits in order into y.
  int nsplit;
  float* part;
};

// Write 2 adjacent fp32 (or bf16) outputs of row m starting at column c.
template <bool kBf16>
__device__ __forceinline__ void store2(void* out, int64_t ld, int64_t m, int64_t c, int64_t cols,
                                       float v0, float v1) {
  if (kBf16) {
    uint16_t* o = static_cast<uint16_t*>(out) + m * ld + c;
    if (c + 2 <= cols && (ld & 1) == 0) {
      *reinterpret_cast<uint32_t*>(o) = pack_bf16x2(v0, v1);
    } else {
      if (c < cols) o[0] = (uint16_t)(pack_bf16x2(v0, 0.0f) & 0xFFFFu);
      if (c + 1 < cols) o[1] = (uint16_t)(pack_bf16x2(v1, 0.0f) & 0xFFFFu);
    }
  } else {
    float* o = static_cast<float*>(out) + m * ld + c;
    if (c + 2 <= cols && (ld & 1) == 0) {
      *reinterpret_cast<f32x2_t*>(o) = f32x2_t{v0, v1};
    } else {
      if (c < cols) o[0] = v0;
      if (c + 1 < cols) o[1] = v1;
    }
  }
}

// ----------------------------------------------------------------- forward
// y[m,n] = sum_k x[m,k] w_hat[n,k] + sum_j ulr[m,j] Bt[n, j mod r]
//
// Workgroup tile 512 (M) x 128 (N), reduction steps of 32; wave w owns rows
// m0 + 128w .. +127 and all 128 columns (4 x 4 v_mfma_f32_32x32x16_bf16
// tiles). Every weight element of the tile is dequantized once per
// workgroup into a bf16 tile in LDS that all four waves read, so each
// dequantized element feeds 512 rows of x.
//
// x tile (512 x 32 bf16 = 32 KB per step): coalesced 16-byte loads (four
// lanes cover a row's 64 bytes) into registers one step ahead, stored to a
// three-buffer LDS ring the step after; 16-byte chunk c of row r sits at
// chunk slot c ^ ((r / 4) % 4), so the 16 rows of one fragment read fall in
// distinct banks. Reduction order inside a step: lane group h = lane / 32
// supplies elements k0 + 16h + 8s + (0..7) in substep s, for both operands.
//
// Dequantization role of a thread: tile row dr = 32w + lane/2, half
// hb = lane % 2 of a step's 32 elements (16 codes = 8 bytes). The lane's
// 16-entry table (bf16(L[e] c1_hat) of the row's current block) is a 4-byte
// column of its wave's 4 KB LDS region: entry e at 256 e + 4 lane, the value
// in the low half. A lookup instruction touches 64 distinct banks; its
// address is one byte permute of the code word. The two lanes of a row build
// 8 entries each and write both columns.
//
// Step kb reads x tile kb % 3 and bf16 tile kb % 3; it stores x(kb+2) (loaded
// last step) and dequantizes step kb+2 into the rings, and prefetches the
// fragments of (kb+1, substep 0), whose tiles were completed before the
// previous barrier:
//   issue x(kb+3) loads, codes(kb+3), (odd steps) scales of step kb+3; wait
//   for the previous step's loads; store x(kb+2); on even steps build the
//   tables of the block starting at step kb+2; substep 0: read the fragments
//   of substep 1, issue the lookups of code word 0 of step kb+2, 16 MFMAs,
//   pack and store; substep 1: read the fragments of (kb+1, 0), lookups of
//   code word 1, 16 MFMAs, pack and store; barrier.
constexpr int kF2BM = 512;
constexpr int kF2BN = 128;
constexpr int kF2Ld = 40;  // bf16 weight tile row stride (80 B): B reads of one instruction hit distinct banks
constexpr int kF2Tile = kF2BN * kF2Ld;
constexpr int kF2XTile = kF2BM * 32;  // x tile, bf16 elements

template <bool kOutBf16>
__global__ __launch_bounds__(256, 1) void gemm_fwd_kernel(FwdArgs p, Codebook cb) {
  // The tables come first in LDS (largest alignment): lookup addresses then
  // need no base added.
  __shared__ __attribute__((aligned(16384))) uint32_t tabs[4][16][64];
  __shared__ __attribute__((aligned(1024))) uint16_t xs[3 * kF2XTile];
  __shared__ __attribute__((aligned(16))) uint16_t wt[3 * kF2Tile];
  __shared__ __attribute__((aligned(16))) float levels[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, i = lane & 31, h = lane >> 5;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t m0 = (int64_t)blockIdx.y * kF2BM, n0 = (int64_t)blockIdx.x * kF2BN;
  const int64_t KB = K / 64;
  // this workgroup's blocks [kblk0, kblk0 + nsteps/2): whole blocks, so the
  // local step parity is the global one
  const int split = (int)blockIdx.z;
  const int64_t bper = (KB + p.nsplit - 1) / p.nsplit;
  const int64_t kblk0 = split * bper;
  const int nsteps = (int)(2 * (bper < KB - kblk0 ? bper : KB - kblk0));
  const int64_t kstep0 = 2 * kblk0;  // first global step
  if (tid < 16) levels[tid] = cb.level[tid];
  auto clamp = [&](int kb) { return kb < nsteps ? kb : nsteps - 1; };

  // x staging role: chunk q = tid + 256 j (j < 8) of the tile -> row q / 4,
  // 16-byte chunk q % 4. Rows past M are not loaded: their LDS rows keep
  // whatever they held and only feed accumulator rows that are never stored
  // (at small M this saves all but M of the tile's 512 rows of traffic).
  // Every step waits for all of its loads, so skipping some costs no wait.
  const uint16_t* xsrc[8];
  int xdst[8];
  bool xok[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int q = tid + 256 * j, row = q >> 2, c = q & 3;
    xok[j] = m0 + row < M;
    const int64_t grow = xok[j] ? m0 + row : M - 1;
    xsrc[j] = p.x + grow * K + 8 * c;
    xdst[j] = row * 32 + 8 * (c ^ ((row >> 2) & 3));
  }
  u32x4_t xr[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) xr[j] = zero4();
  auto load_x = [&](int kb) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (xok[j]) xr[j] = *reinterpret_cast<const u32x4_t*>(xsrc[j] + 32 * (kstep0 + kb));
  };
  auto store_x = [&](int tile) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<u32x4_t*>(&xs[tile * kF2XTile + xdst[j]]) = xr[j];
  };
  // A fragment of row tile mt, substep s: row 128w + 32mt + i, chunk 2h + s.
  const int arow0 = 128 * w + i;
  auto read_afrag = [&](int tile, int s, u32x4_t (&af)[4]) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int row = arow0 + 32 * mt;
      af[mt] = *reinterpret_cast<const u32x4_t*>(
          &xs[tile * kF2XTile + row * 32 + 8 * ((2 * h + s) ^ ((row >> 2) & 3))]);
    }
  };

  // dequantization role
  const int dr = 32 * w + (lane >> 1), hb = lane & 1;
  const bool drow_ok = n0 + dr < N;
  const int64_t drow = drow_ok ? n0 + dr : N - 1;
  const uint8_t* dcode = p.codes + drow * (K / 2) + 8 * hb;
  const int64_t dblk = drow * KB;
  u32x2_t cr[2];  // codes of step j in cr[j % 2]
  int qv = 0;
  float sv = 0.0f;
  auto load_c = [&](int par, int kb) {
    cr[par] = *reinterpret_cast<const u32x2_t*>(dcode + 16 * (kstep0 + kb));
  };
  auto load_s = [&](int kb) {
    const int64_t bi = dblk + kblk0 + kb / 2;
    qv = (int)p.q8[bi];
    sv = p.s2[bi >> 8];
  };
  const uint32_t colbase = 4u * (uint32_t)lane;
  const uint32_t region = 0x10101010u * (uint32_t)w;
  const char* tb = reinterpret_cast<const char*>(&tabs[0][0][0]);
  auto build = [&]() {
    const float ch = drow_ok ? q8_value(qv, cb.dq_format) * sv : 0.0f;
    const f32x4_t la = *reinterpret_cast<const f32x4_t*>(&levels[8 * hb]);
    const f32x4_t lb = *reinterpret_cast<const f32x4_t*>(&levels[8 * hb + 4]);
    const float lv[8] = {la.x, la.y, la.z, la.w, lb.x, lb.y, lb.z, lb.w};
    uint32_t* col = &tabs[w][8 * hb][lane & ~1];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t v = pack_bf16x2(lv[j] * ch, 0.0f);
      *reinterpret_cast<u32x2_t*>(col + j * 64) = u32x2_t{v, v};
    }
  };
  // Lookups of the eight codes of code word cw (element e = nibble e).
  auto lookup_issue = [&](uint32_t cw, uint32_t (&v)[8]) {
    const uint32_t lo = (cw & 0x0F0F0F0Fu) | region;
    const uint32_t hi = ((cw >> 4) & 0x0F0F0F0Fu) | region;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t sel = 0x0C0C0000u | ((uint32_t)(4 + b) << 8);
      v[2 * b] = *reinterpret_cast<const uint16_t*>(tb + __builtin_amdgcn_perm(lo, colbase, sel));
      v[2 * b + 1] = *reinterpret_cast<const uint16_t*>(tb + __builtin_amdgcn_perm(hi, colbase, sel));
    }
  };
  auto pack = [&](const uint32_t (&v)[8]) {
    return u32x4_t{__builtin_amdgcn_perm(v[1], v[0], 0x05040100u),
                   __builtin_amdgcn_perm(v[3], v[2], 0x05040100u),
                   __builtin_amdgcn_perm(v[5], v[4], 0x05040100u),
                   __builtin_amdgcn_perm(v[7], v[6], 0x05040100u)};
  };
  const int wt_off = dr * kF2Ld + 16 * hb;  // this thread's 16 elements of a bf16 tile
  const int fr_off = i * kF2Ld + 16 * h;    // this lane's B fragment of column tile 0
  auto read_bfrag = [&](int tile, int s, u32x4_t (&bf)[4]) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      bf[nt] = *reinterpret_cast<const u32x4_t*>(&wt[tile * kF2Tile + fr_off + 32 * nt * kF2Ld + 8 * s]);
  };

  f32x16_t acc[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mt][nt][e] = 0.0f;

  // Prologue: x tiles 0, 1 and bf16 tiles 0, 1 (block 0) in LDS; x(2) in
  // registers; codes of step 2, scales of block 1; fragments of (0, 0).
  {
    load_c(0, 0);
    load_c(1, clamp(1));
    load_s(0);
    load_x(0);
    wait_vmem<0>();
    store_x(0);
    load_x(clamp(1));
    wait_vmem<0>();
    store_x(1);
    load_x(clamp(2));
    __syncthreads();  // codebook levels
    build();
    uint32_t v0[8], v1[8], v2[8], v3[8];
    lookup_issue(cr[0].x, v0);
    lookup_issue(cr[0].y, v1);
    lookup_issue(cr[1].x, v2);
    lookup_issue(cr[1].y, v3);
    *reinterpret_cast<u32x4_t*>(&wt[0 * kF2Tile + wt_off]) = pack(v0);
    *reinterpret_cast<u32x4_t*>(&wt[0 * kF2Tile + wt_off + 8]) = pack(v1);
    *reinterpret_cast<u32x4_t*>(&wt[1 * kF2Tile + wt_off]) = pack(v2);
    *reinterpret_cast<u32x4_t*>(&wt[1 * kF2Tile + wt_off + 8]) = pack(v3);
    load_c(0, clamp(2));
    load_s(clamp(2));
    wait_vmem<0>();
    __syncthreads();
  }
  u32x4_t afa[4], afb[4], bfa[4], bfb[4];
  read_afrag(0, 0, afa);
  read_bfrag(0, 0, bfa);

  // One substep: 16 MFMAs on fragments (ac, bc) while the fragments of the
  // next substep (tile ntile, substep ns) are read into (an, bn) and the eight
  // codes of word cw are looked up, packed and stored at wdst. Issue order
  // (pinned with scheduling groups): eight times {MFMA, fragment read,
  // address permute, lookup}, then four MFMAs, then four times {MFMA, pack},
  // so no LDS result is waited for while MFMAs remain to be issued.
  auto substep = [&](int ntile, int ns, uint32_t cw, const u32x4_t (&ac)[4], const u32x4_t (&bc)[4],
                     u32x4_t (&an)[4], u32x4_t (&bn)[4], uint16_t* wdst) {
    const uint32_t lo = (cw & 0x0F0F0F0Fu) | region;
    const uint32_t hi = ((cw >> 4) & 0x0F0F0F0Fu) | region;
    uint32_t v[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const int mt = g >> 2, nt = g & 3;
      acc[mt][nt] = mfma_32x32x16(ac[mt], bc[nt], acc[mt][nt]);
      if (g < 4) {
        const int row = arow0 + 32 * g;
        an[g] = *reinterpret_cast<const u32x4_t*>(
            &xs[ntile * kF2XTile + row * 32 + 8 * ((2 * h + ns) ^ ((row >> 2) & 3))]);
      } else {
        bn[g - 4] = *reinterpret_cast<const u32x4_t*>(
            &wt[ntile * kF2Tile + fr_off + 32 * (g - 4) * kF2Ld + 8 * ns]);
      }
      const uint32_t sel = 0x0C0C0000u | ((uint32_t)(4 + (g >> 1)) << 8);
      v[g] = *reinterpret_cast<const uint16_t*>(
          tb + __builtin_amdgcn_perm((g & 1) ? hi : lo, colbase, sel));
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // fragment read
      __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);  // address permute
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // lookup
    }
#pragma unroll
    for (int g = 8; g < 12; ++g) {
      acc[g >> 2][g & 3] = mfma_32x32x16(ac[g >> 2], bc[g & 3], acc[g >> 2][g & 3]);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    uint32_t pk[4];
#pragma unroll
    for (int g = 12; g < 16; ++g) {
      acc[g >> 2][g & 3] = mfma_32x32x16(ac[g >> 2], bc[g & 3], acc[g >> 2][g & 3]);
      const int b = g - 12;
      pk[b] = __builtin_amdgcn_perm(v[2 * b + 1], v[2 * b], 0x05040100u);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);  // pack
    }
    *reinterpret_cast<u32x4_t*>(wdst) = u32x4_t{pk[0], pk[1], pk[2], pk[3]};
    __builtin_amdgcn_sched_barrier(0);
  };
  auto step = [&](int kb, auto q6) {
    constexpr int Q = decltype(q6)::value;  // kb % 6
    constexpr int P2 = Q % 2, P3 = Q % 3;
    constexpr int T1 = (P3 + 1) % 3, T2 = (P3 + 2) % 3;
    // x(kb+2) is in registers (loaded last step): store it, then load x(kb+3)
    wait_vmem<0>();
    store_x(T2);
    __builtin_amdgcn_sched_barrier(0);
    load_x(clamp(kb + 3));
    load_c(P2 ^ 1, clamp(kb + 3));
    if (P2 == 1) load_s(clamp(kb + 3));
    __builtin_amdgcn_sched_barrier(0);
    if (P2 == 0) build();  // step kb+2 starts a block
    __builtin_amdgcn_sched_barrier(0);
    const u32x2_t cn = cr[P2];
    uint16_t* const wd = &wt[T2 * kF2Tile + wt_off];
    substep(P3, 1, cn.x, afa, bfa, afb, bfb, wd);   // substep 0: prefetch (kb, 1)
    substep(T1, 0, cn.y, afb, bfb, afa, bfa, wd + 8);  // substep 1: prefetch (kb+1, 0)
    __syncthreads();
  };
  int kb = 0;
  for (; kb + 6 <= nsteps; kb += 6) {
    step(kb, std::integral_constant<int, 0>());
    step(kb + 1, std::integral_constant<int, 1>());
    step(kb + 2, std::integral_constant<int, 2>());
    step(kb + 3, std::integral_constant<int, 3>());
    step(kb + 4, std::integral_constant<int, 4>());
    step(kb + 5, std::integral_constant<int, 5>());
  }
  if (kb < nsteps) {
    step(kb, std::integral_constant<int, 0>());
    step(kb + 1, std::integral_constant<int, 1>());
  }
  if (kb + 2 < nsteps) {
    step(kb + 2, std::integral_constant<int, 2>());
    step(kb + 3, std::integral_constant<int, 3>());
  }

  // Adapter term as 2r extra reduction elements, 16 per MFMA: lane group h
  // supplies elements 16q + 8h + (0..7) (split 0).
  const int r = p.r, r2 = 2 * r;
  for (int q = 0; q < (split == 0 ? r2 / 16 : 0); ++q) {
    const int jj = 16 * q + 8 * h;
    const int jb = jj % r;
    u32x4_t bfr[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int64_t n = n0 + 32 * nt + i;
      bfr[nt] = n < N ? *reinterpret_cast<const u32x4_t*>(p.Bt + n * r + jb) : zero4();
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int64_t m = m0 + 128 * w + 32 * mt + i;
      const u32x4_t a = m < M ? *reinterpret_cast<const u32x4_t*>(p.ulr + m * r2 + jj) : zero4();
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mfma_32x32x16(a, bfr[nt], acc[mt][nt]);
    }
  }

  float* const dst = p.nsplit > 1 ? p.part + (int64_t)split * M * N : nullptr;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int64_t n = n0 + 32 * nt + i;
    if (n < N) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t m = m0 + 128 * w + 32 * mt + 8 * (e >> 2) + 4 * h + (e & 3);
          if (m < M && dst) {
            dst[m * N + n] = acc[mt][nt][e];
          } else if (m < M) {
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
  // Reduction split (nsplit > 1): workgroup z takes the z-th range of whole
  // 64-row steps of N and stores fp32 sums for rows m < M to part + z*M*K
  // (the adapter term rides in split 0); a reduce launch adds the splits in
  // order into dX.
  int nsplit;
  float* part;
};

// Tile mapping (v_mfma_f32_32x32x16_bf16). Lane l = 32h + c of wave w:
//   MFMA (mt, nt) covers rows m0 + 32mt + (0..31) and output columns
//   kbase + 2c + nt (kbase = first column of wave w, a block boundary).
//   Step = 64 weight rows (the reduction) = 4 substeps s of 16; in substep s
//   lane group h supplies rows n0 + 32h + 8s + (0..7) of both operands. The
//   B fragment of (nt, s) holds, for each of those 8 rows, nibble nt of the
//   code byte of columns kbase + 2c, kbase + 2c + 1.
//
// Pipeline of one step ns, three buffers of dY, code blocks and tables:
//   top:   DMA dY(ns+2); DMA this wave's code block (64 rows x its 32 bytes)
//          of step ns+2; load the scales of ns+3 (12 vector-memory
//          instructions); build this wave's tables of step ns+1.
//   body:  32 groups (s, mt) of 2 MFMAs on the fragments of substep s while
//          the fragments of substep s+1 (or of step ns+1, substep 0) are
//          looked up, 2 LUT reads per group; the 8 code bytes of the next
//          substep are read at the start of each substep.
//   end:   wait until only this step's loads are in flight, then barrier.
// Wave w only reads the code bytes and tables of its own 64 columns, which
// its own lanes fetch and build, so those need only this wave's waits.
// kMT: 32-row MFMA row tiles of the 256-row output tile that carry rows of
// dY (8; 1 when M <= 32, so that a decode-size call issues one MFMA group
// per lookup group instead of eight).
template <bool kOutBf16, int kMT>
__global__ __launch_bounds__(256, 1) void gemm_bwd_kernel(BwdArgs p, Codebook cb) {
  static_assert(kMT == 1 || kMT == 8, "row tiles");
  __shared__ __attribute__((aligned(1024))) uint16_t ys0[kTileBytes / 2];
  __shared__ __attribute__((aligned(1024))) uint16_t ys1[kTileBytes / 2];
  __shared__ __attribute__((aligned(1024))) uint16_t ys2[kTileBytes / 2];
  __shared__ __attribute__((aligned(1024))) uint8_t cs0[64 * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t cs1[64 * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t cs2[64 * 128];
  __shared__ __attribute__((aligned(32))) uint16_t tab0[256 * 16];
  __shared__ __attribute__((aligned(32))) uint16_t tab1[256 * 16];
  __shared__ __attribute__((aligned(32))) uint16_t tab2[256 * 16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 31, h = lane >> 5;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t m0 = (int64_t)blockIdx.y * kBM;
  const int64_t kt0 = (int64_t)blockIdx.x * kBN;
  const int64_t KB = K / 64;
  // this workgroup's steps: [nsb, nsb + NS) of the (N + 63) / 64 steps of N
  const int64_t NS_all = (N + 63) / 64;
  const int split = (int)blockIdx.z;
  const int64_t per = (NS_all + p.nsplit - 1) / p.nsplit;
  const int64_t nsb = split * per;
  const int64_t NS = per < NS_all - nsb ? per : NS_all - nsb;
  const int64_t kbase = kt0 + 64 * w;
  const bool wave_live = kbase < K;

  // dY DMA: instruction j of wave w, lane l -> slot (w*8+j)*64 + l -> row
  // (w*8+j)*8 + l/8, chunk slot l%8 holding global chunk (l%8) ^ ((l/8)%8).
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
  // Code DMA of this wave: 64 rows x 32 bytes (columns kbase..kbase+63) =
  // 128 chunks of 16 B: instruction j, lane l -> chunk 64j + l -> row
  // (64j+l)/2, half (64j+l)%2, stored at byte (64j+l)*16 of the wave's 2 KB.
  const int64_t ccol = (wave_live ? kbase : K - 64) / 2;
  int crow[2], chalf[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    crow[j] = (64 * j + lane) >> 1;
    chalf[j] = (64 * j + lane) & 1;
  }
  const int64_t tblk = kt0 / 64 + (tid >> 6);
  const bool tblk_ok = tblk < KB;

  // 8 vector-memory instructions
  auto issue_y = [&](int64_t ns, uint16_t* ydst) {
    int64_t ccl = (nsb + ns) * 64 + ychunk * 8;
    if (ccl + 8 > N) ccl = N - 8;
    const uint16_t* ysrc = yrow0 + ccl;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      __builtin_amdgcn_global_load_lds(ysrc + yoff[j], ydst + (w * 8 + j) * 512, 16, 0, 0);
  };
  // 2 vector-memory instructions
  auto issue_codes = [&](int64_t ns, uint8_t* cdst) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      int64_t row = (nsb + ns) * 64 + crow[j];
      row = row < N ? row : N - 1;
      __builtin_amdgcn_global_load_lds(p.codes + row * (K / 2) + ccol + 16 * chalf[j],
                                       cdst + w * 2048 + 64 * j * 16, 16, 0, 0);
    }
  };
  // 2 vector-memory instructions (unconditional; masked when the table is built)
  auto load_scale = [&](int64_t ns, int& qv, float& sv) {
    const int64_t nn = (nsb + ns) * 64 + (tid & 63);
    const int64_t bi = (nn < N ? nn : N - 1) * KB + (tblk_ok ? tblk : KB - 1);
    qv = (int)p.q8[bi];
    sv = p.s2[bi >> 8];
  };
  auto scale_ok = [&](int64_t ns) { return (nsb + ns) * 64 + (tid & 63) < N && tblk_ok; };

  f32x16_t acc[kMT][2];
#pragma unroll
  for (int i = 0; i < kMT; ++i)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][nt][e] = 0.0f;

  int a_off[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) a_off[s] = c * 128 + (((4 * h + s) ^ (c & 7)) << 4);
  const uint32_t t_byte = (uint32_t)((w * 64 + 32 * h) * 32);  // table of this lane's row 0
  const int cb_off = w * 2048 + (32 * h) * 32 + c;             // its code byte of row 0

  // The 8 code bytes (rows 8s..8s+7 of this lane's half) of substep s.
  auto code_bytes = [&](const uint8_t* cbuf, int s, uint32_t (&b)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = cbuf[cb_off + (8 * s + i) * 32];
  };
  // One substep: 8 groups (A fragment of row tile mt, 2 MFMAs) on fragments
  // bc, while fragments bn of substep sn (code bytes b, table array tarr) are
  // looked up: group mt looks up dword mt%4 (rows 2(mt%4), 2(mt%4)+1) of
  // fragment mt/4.
  auto substep = [&](const char* ya, const u32x4_t (&bc)[2], u32x4_t (&bn)[2],
                     const uint32_t (&b)[8], const uint16_t* tarr, int sn) {
    const char* tb = reinterpret_cast<const char*>(tarr);
    u32x4_t a[3];
    a[0] = *reinterpret_cast<const u32x4_t*>(ya);
    if (kMT > 1) a[1] = *reinterpret_cast<const u32x4_t*>(ya + 4096);
    uint32_t lo[8], hi[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      if (mt + 2 < kMT) a[(mt + 2) % 3] = *reinterpret_cast<const u32x4_t*>(ya + (mt + 2) * 4096);
      if (mt < kMT) {
        constexpr int kLast = kMT - 1;
        const int mi = mt < kMT ? mt : kLast;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[mi][nt] = mfma_32x32x16(a[mt % 3], bc[nt], acc[mi][nt]);
      }
      {
        const int f = mt >> 2, q = mt & 3;
        const uint32_t r0 = t_byte + (uint32_t)(8 * sn + 2 * q) * 32;
        const uint32_t b0 = b[2 * q], b1 = b[2 * q + 1];
        const uint32_t o0 = f == 0 ? ((b0 << 1) & 30u) : ((b0 >> 3) & 30u);
        const uint32_t o1 = f == 0 ? ((b1 << 1) & 30u) : ((b1 >> 3) & 30u);
        lo[mt] = *reinterpret_cast<const uint16_t*>(tb + (r0 | o0));
        hi[mt] = *reinterpret_cast<const uint16_t*>(tb + ((r0 + 32) | o1));
      }
      if (mt >= 2) bn[(mt - 2) >> 2][(mt - 2) & 3] = lo[mt - 2] | (hi[mt - 2] << 16);
      if (kMT == 8) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      }
    }
    bn[1][2] = lo[6] | (hi[6] << 16);
    bn[1][3] = lo[7] | (hi[7] << 16);
  };

  // Prologue: dY(0), dY(1), code blocks 0 and 1, scales 0..2; table 0 built;
  // fragments of (step 0, substep 0) looked up.
  int qs[3] = {0, 0, 0};
  float ss[3] = {0.0f, 0.0f, 0.0f};
  const int64_t ns1 = NS > 1 ? 1 : 0, ns2 = NS > 2 ? 2 : NS - 1;
  issue_y(0, ys0);
  issue_y(ns1, ys1);
  issue_codes(0, cs0);
  issue_codes(ns1, cs1);
  load_scale(0, qs[0], ss[0]);
  load_scale(ns1, qs[1], ss[1]);
  load_scale(ns2, qs[2], ss[2]);
  wait_vmem<0>();
  build_table(cb, scale_ok(0) ? qs[0] : 0, ss[0], tab0 + tid * 16);
  u32x4_t bf0[2], bf1[2];
  {
    uint32_t b[8];
    code_bytes(cs0, 0, b);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      uint32_t v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        v[i] = *reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(tab0) + t_byte +
                                                  i * 32 + 2 * ((b[i] >> (4 * nt)) & 15u));
      bf0[nt] = u32x4_t{v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16),
                        v[6] | (v[7] << 16)};
    }
  }
  __syncthreads();  // dY(0), dY(1) visible everywhere

  // Every step issues the same 12 vector-memory instructions (indices past
  // the last step are clamped), so the wait counts are exact on every path.
  auto step = [&](int64_t ns, auto slot) {
    constexpr int S0 = decltype(slot)::value, S1 = (S0 + 1) % 3, S2 = (S0 + 2) % 3;
    const int64_t n2 = ns + 2 < NS ? ns + 2 : NS - 1;
    const int64_t n3 = ns + 3 < NS ? ns + 3 : NS - 1;
    const char* y0 = reinterpret_cast<const char*>(pick3<S0>(ys0, ys1, ys2));
    uint16_t* const y2 = pick3<S2>(ys0, ys1, ys2);
    const uint8_t* c0 = pick3<S0>(cs0, cs1, cs2);
    const uint8_t* c1 = pick3<S1>(cs0, cs1, cs2);
    uint8_t* const c2 = pick3<S2>(cs0, cs1, cs2);
    uint16_t* const t0 = pick3<S0>(tab0, tab1, tab2);
    uint16_t* const t1 = pick3<S1>(tab0, tab1, tab2);
    issue_y(n2, y2);
    issue_codes(n2, c2);
    load_scale(n3, qs[S0], ss[S0]);
    __builtin_amdgcn_sched_barrier(0);
    // scales(ns+1) came two steps ago: at least 24 younger loads
    wait_vmem<24>();
    build_table(cb, scale_ok(ns + 1) ? qs[S1] : 0, ss[S1], t1 + tid * 16);
    uint32_t b1[8], b2[8], b3[8], bn[8];
    code_bytes(c0, 1, b1);
    substep(y0 + a_off[0], bf0, bf1, b1, t0, 1);
    code_bytes(c0, 2, b2);
    substep(y0 + a_off[1], bf1, bf0, b2, t0, 2);
    code_bytes(c0, 3, b3);
    substep(y0 + a_off[2], bf0, bf1, b3, t0, 3);
    // this wave's code block of ns+1 came in the previous step
    wait_vmem<12>();
    code_bytes(c1, 0, bn);
    substep(y0 + a_off[3], bf1, bf0, bn, t1, 0);
    // only this step's 12 loads may be in flight: dY(ns+1) has landed
    wait_vmem<12>();
    __builtin_amdgcn_s_barrier();
  };
  int64_t ns = 0;
  for (; ns + 3 <= NS; ns += 3) {
    step(ns, std::integral_constant<int, 0>());
    step(ns + 1, std::integral_constant<int, 1>());
    step(ns + 2, std::integral_constant<int, 2>());
  }
  if (ns < NS) step(ns, std::integral_constant<int, 0>());
  if (ns + 1 < NS) step(ns + 1, std::integral_constant<int, 1>());

  // Adapter term as 2r extra reduction elements, 16 per MFMA (split 0).
  const int r = p.r, r2 = 2 * r;
  for (int q = 0; q < (split == 0 ? r2 / 16 : 0); ++q) {
    const int jj = 16 * q + 8 * h;
    const int jb = jj % r;
    u32x4_t bfr[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int64_t kc = kbase + 2 * c + nt;
      bfr[nt] = kc < K ? *reinterpret_cast<const u32x4_t*>(p.A + kc * r + jb) : zero4();
    }
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
      const int64_t m = m0 + 32 * mt + c;
      const u32x4_t a = m < M ? *reinterpret_cast<const u32x4_t*>(p.svlr + m * r2 + jj) : zero4();
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = mfma_32x32x16(a, bfr[nt], acc[mt][nt]);
    }
  }

  const int64_t kcol = kbase + 2 * c;
  if (wave_live && p.nsplit > 1) {  // fp32 partial sums of this split
    float* dst = p.part + (int64_t)split * M * K;
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t m = m0 + 32 * mt + 8 * (e >> 2) + 4 * h + (e & 3);
        if (m < M) store2<false>(dst, K, m, kcol, K, acc[mt][0][e], acc[mt][1][e]);
      }
  } else if (wave_live) {
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t m = m0 + 32 * mt + 8 * (e >> 2) + 4 * h + (e & 3);
        if (m < M) store2<kOutBf16>(p.dX, K, m, kcol, K, acc[mt][0][e], acc[mt][1][e]);
      }
  }
}

}  // namespace

int gemm_fwd_splits(int64_t M, int64_t N, int64_t K) {
  // Under half as many output tiles as CUs: split the reduction over K into
  // ranges of whole 64-weight blocks (at least two a range) so that the
  // launch fills more of the GPU (one workgroup per CU); the fp32 partial
  // sums (s * M * N * 4 bytes) stay within 24 MB. The count minimises rounds
  // of 256 workgroups times (blocks per range + 2, the fixed cost of a
  // workgroup in blocks). Measured at 16 < M < 512 before: every M took
  // 155-170 us on 4096-wide weights, each workgroup walking all of K.
  const int64_t tiles = ((N + kF2BN - 1) / kF2BN) * ((M + kF2BM - 1) / kF2BM);
  if (tiles >= 128) return 1;
  const int64_t blocks = K / 64;
  int64_t smax = blocks / 2;
  if (smax > 64) smax = 64;
  const int64_t cap = ((int64_t)24 << 20) / (M * N * 4);
  if (smax > cap) smax = cap;
  int best = 1;
  int64_t best_cost = blocks + 2;  // one range: one round
  for (int64_t s = 2; s <= smax; ++s) {
    if ((s - 1) * ((blocks + s - 1) / s) >= blocks) continue;  // an empty range
    const int64_t rounds = (tiles * s + 255) / 256;
    const int64_t cost = rounds * ((blocks + s - 1) / s + 2);
    if (cost < best_cost) {
      best_cost = cost;
      best = (int)s;
    }
  }
  return best;
}

hipError_t launch_gemm_fwd(const uint16_t* x, const uint8_t* codes, const int8_t* q8,
                           const float* s2, const uint16_t* ulr, const uint16_t* Bt, int64_t M,
                           int64_t N, int64_t K, int r, void* y, bool y_bf16, const Codebook& cb,
                           hipStream_t st, float* part) {
  const int nsplit = part ? gemm_fwd_splits(M, N, K) : 1;
  const FwdArgs a{x, codes, q8, s2, ulr, Bt, y, M, N, K, r, nsplit, part};
  const dim3 grid((unsigned)((N + kF2BN - 1) / kF2BN), (unsigned)((M + kF2BM - 1) / kF2BM),
                  (unsigned)nsplit);
  if (y_bf16)
    hipLaunchKernelGGL(gemm_fwd_kernel<true>, grid, dim3(256), 0, st, a, cb);
  else
    hipLaunchKernelGGL(gemm_fwd_kernel<false>, grid, dim3(256), 0, st, a, cb);
  if (nsplit > 1) {
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_split_reduce(part, nsplit, M * N, y, y_bf16, st);
  }
  return hipGetLastError();
}

int gemm_bwd_splits(int64_t M, int64_t N, int64_t K) {
  // Few output tiles (small M): split the reduction over N into ranges of
  // at least two 64-row steps so that the launch fills the GPU (measured
  // on the 1024 x 1024 layer at M = 16: 4 workgroups walking all 16 steps
  // took 45 us). The general kernel (N % 8 != 0) does not split.
  if (N % 8) return 1;
  const int64_t tiles = ((K + kBN - 1) / kBN) * ((M + kBM - 1) / kBM);
  if (tiles >= 64) return 1;
  const int64_t steps = (N + 63) / 64;
  int64_t s = 256 / tiles;
  if (s > steps / 2) s = steps / 2;
  if (s > 64) s = 64;
  // the fp32 partial sums (s * M * K * 4 bytes) stay within the size of the
  // NF4 weight (N * K / 2 bytes): small M only
  if (s > N / (8 * M)) s = N / (8 * M);
  if (s < 2) return 1;
  // no empty split: the last range must hold a step
  while (s > 1 && (s - 1) * ((steps + s - 1) / s) >= steps) --s;
  return (int)s;
}

hipError_t launch_gemm_bwd(const uint16_t* dY, const uint8_t* codes, const int8_t* q8,
                           const float* s2, const uint16_t* svlr, const uint16_t* A, int64_t M,
                           int64_t N, int64_t K, int r, void* dX, bool dx_bf16,
                           const Codebook& cb, hipStream_t st, float* part) {
  const int nsplit = part ? gemm_bwd_splits(M, N, K) : 1;
  if (N % 8 == 0) {
    const dim3 grid((unsigned)((K + kBN - 1) / kBN), (unsigned)((M + kBM - 1) / kBM),
                    (unsigned)nsplit);
    const BwdArgs a{dY, codes, q8, s2, svlr, A, dX, M, N, K, r, nsplit, part};
    // one 32-row MFMA row tile when M <= 32 (the other seven would hold only
    // the padding rows)
    if (M <= 32) {
      if (dx_bf16)
        hipLaunchKernelGGL((gemm_bwd_kernel<true, 1>), grid, dim3(256), 0, st, a, cb);
      else
        hipLaunchKernelGGL((gemm_bwd_kernel<false, 1>), grid, dim3(256), 0, st, a, cb);
    } else if (dx_bf16) {
      hipLaunchKernelGGL((gemm_bwd_kernel<true, 8>), grid, dim3(256), 0, st, a, cb);
    } else {
      hipLaunchKernelGGL((gemm_bwd_kernel<false, 8>), grid, dim3(256), 0, st, a, cb);
    }
    if (nsplit > 1) {
      const hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
      return launch_split_reduce(part, nsplit, M * K, dX, dx_bf16, st);
    }
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((K + kBN - 1) / kBN), (unsigned)((M + kBM - 1) / kBM));
  if (dx_bf16) {
    hipLaunchKernelGGL(gemm_bwd_general_kernel<true>, grid, dim3(256), 0, st, dY, codes, q8, s2,
                       svlr, A, M, N, K, r, dX, cb);
  } else {
    hipLaunchKernelGGL(gemm_bwd_general_kernel<false>, grid, dim3(256), 0, st, dY, codes, q8, s2,
                       svlr, A, M, N, K, r, dX, cb);
  }
  return hipGetLastError();
}

}  // namespace qlora
