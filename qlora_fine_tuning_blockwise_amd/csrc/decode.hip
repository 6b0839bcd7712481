// Decode path of the QLoRA layer (M <= 16 tokens) on gfx950: two launches.
//
// [P1] "QLoRA" forward equation: y = x doubleDequant(c1, c2, W) + s (x A) B
// with s = alpha / r; [P2] s2 (4-bit NormalFloat, Double Quantization).
//
//  1. lora_down_decode: per K slice (at most 16), part[slice][m][j] =
//     sum_k x[m,k] A[k,j] on MFMA (A read transposed from an LDS panel).
//  2. gemv: the frozen-weight product streams the NF4 codes once from HBM
//     and finishes the layer in its epilogue: the adapter term s (sum of the
//     slices) B is added before y is written.
//
// The weight stream is the roofline: per weight, 0.5 byte of code plus 1/64
// byte of block scale. Dequantization runs beside the loads: each lane owns a
// full 64-weight block of one row in each of two chunks of K and looks its
// codes up in a 16-entry table of its own. The tables live in LDS as one
// 4-byte column per lane (entry e of lane t at 256*e + 4*t inside the wave's
// 4 KB region), so a lookup instruction touches 64 distinct banks whatever
// the codes are; the two halves of an entry hold the bf16 values of the
// lane's two blocks. The lookup address is assembled with one byte permute
// per code.
#include <algorithm>

#include "device.h"

namespace qlora {
namespace {

// ------------------------------------------------------ adapter down, decode
constexpr int kDecMaxSlices = 16;  // K slices (partial sums) of the down projection
constexpr int kDecLd = 18;         // panel row stride in bf16 (36 B)

// grid: (slices, r / 16). Workgroup `slice` reduces k in [slice*L, (slice+1)*L)
// in 256-wide pieces (wave w: the piece's k 64w .. 64w+63) for the 16 adapter
// columns j0..j0+15; the four waves are summed in order. part[slice][m][j].
__global__ __launch_bounds__(256) void lora_down_decode_kernel(const uint16_t* __restrict__ x,
                                                               const uint16_t* __restrict__ A,
                                                               int64_t M, int64_t K, int r,
                                                               int64_t L,
                                                               float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint16_t as[4][64][kDecLd];
  __shared__ float red[4][16][17];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, i = lane & 15, g = lane >> 4;
  const int slice = blockIdx.x;
  const int j0 = blockIdx.y * 16;
  const int64_t k0 = (int64_t)slice * L, k1 = min(K, k0 + L);
  // x rows >= M are read from row M-1: they only feed output rows that are
  // never stored.
  const int64_t mrow = min((int64_t)i, M - 1);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int64_t kp = k0; kp < k1; kp += 256) {
    const int64_t kw = kp + 64 * w;
    // Panel A[kw .. kw+63][j0 .. j0+15]: 128 chunks of 16 bytes, 2 per lane;
    // then the x fragments, so that both loads are in flight together.
    u32x4_t pv[2], xa[2];
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int q = lane + 64 * it, row = q >> 1, half = q & 1;
      const int64_t k = kw + row;
      pv[it] = k < k1 ? *reinterpret_cast<const u32x4_t*>(A + k * r + j0 + 8 * half) : zero4();
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int64_t k = kw + 32 * s + 8 * g;
      xa[s] = k < k1 ? *reinterpret_cast<const u32x4_t*>(x + mrow * K + k) : zero4();
    }
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int q = lane + 64 * it, row = q >> 1, half = q & 1;
      uint32_t* d = reinterpret_cast<uint32_t*>(&as[w][row][8 * half]);
      d[0] = pv[it].x;
      d[1] = pv[it].y;
      d[2] = pv[it].z;
      d[3] = pv[it].w;
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const u32x4_t a = xa[s];
      const uint16_t* pa = &as[w][32 * s + 8 * g][i];
      u32x4_t b;
      b.x = (uint32_t)pa[0 * kDecLd] | ((uint32_t)pa[1 * kDecLd] << 16);
      b.y = (uint32_t)pa[2 * kDecLd] | ((uint32_t)pa[3 * kDecLd] << 16);
      b.z = (uint32_t)pa[4 * kDecLd] | ((uint32_t)pa[5 * kDecLd] << 16);
      b.w = (uint32_t)pa[6 * kDecLd] | ((uint32_t)pa[7 * kDecLd] << 16);
      acc = mfma_16x16x32(a, b, acc);
    }
  }
  // acc[v] = partial sum for m = 4g + v, j = j0 + i.
#pragma unroll
  for (int v = 0; v < 4; ++v) red[w][4 * g + v][i] = acc[v];
  __syncthreads();
  const int m = tid >> 4, j = tid & 15;
  if (m < M)
    part[((int64_t)slice * M + m) * r + j0 + j] =
        ((red[0][m][j] + red[1][m][j]) + red[2][m][j]) + red[3][m][j];
}

// Slice length of the down projection: whole 256-wide pieces.
int64_t decode_down_len(int64_t K, int slices) {
  const int64_t pieces = (K + 255) / 256;
  return ((pieces + slices - 1) / slices) * 256;
}

// ----------------------------------------------------------------- GEMV
constexpr int kGvWaves = 8;  // waves per workgroup; 256-wide K chunks go round-robin to them

struct GemvArgs {
  const uint16_t* x;      // [M, K] bf16
  const uint8_t* codes;   // [N, K/2]
  const int8_t* q8;       // [N*K/64]
  const float* s2;        // [ceil(N*K/64/256)]
  const float* upart;     // [slices, M, r] from lora_down_decode
  const uint16_t* B;      // [r, N] bf16
  float* u_out;           // [M, r] fp32 or NULL
  void* y;                // [M, N] fp32 or bf16
  int64_t M, N, K;
  int r, slices;
  float s;
};

// Byte selectors of v_perm_b32 building a lookup address: byte 0 from the
// lane's column offset (src1 byte 0), byte 1 from byte b of the code word
// (src0 byte b), bytes 2 and 3 zero.
__device__ __forceinline__ uint32_t lut_addr(uint32_t codebytes, uint32_t colbase, int b) {
  return __builtin_amdgcn_perm(codebytes, colbase, 0x0C0C0000u | ((uint32_t)(4 + b) << 8));
}

// Issue the eight table reads for code word `cw` (element e = nibble e) from
// half `half` of the lane's table entries. `region` carries the wave's
// region bits in the high nibble of every byte.
__device__ __forceinline__ void lookup_issue(const char* tab, uint32_t cw, uint32_t region,
                                             uint32_t colbase, int half, uint32_t v[8]) {
  const uint32_t lo = (cw & 0x0F0F0F0Fu) | region;
  const uint32_t hi = ((cw >> 4) & 0x0F0F0F0Fu) | region;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    v[2 * b] = *reinterpret_cast<const uint16_t*>(tab + lut_addr(lo, colbase, b) + 2 * half);
    v[2 * b + 1] = *reinterpret_cast<const uint16_t*>(tab + lut_addr(hi, colbase, b) + 2 * half);
  }
}

// Pack eight 16-bit table values into an MFMA operand (value e to bf16 slot e).
__device__ __forceinline__ u32x4_t lookup_pack(const uint32_t v[8]) {
  return u32x4_t{__builtin_amdgcn_perm(v[1], v[0], 0x05040100u),
                 __builtin_amdgcn_perm(v[3], v[2], 0x05040100u),
                 __builtin_amdgcn_perm(v[5], v[4], 0x05040100u),
                 __builtin_amdgcn_perm(v[7], v[6], 0x05040100u)};
}

// grid: ceil(N / 16), 512 threads, two workgroups per CU. Workgroup rows
// n0 .. n0+15 form one 16-row MFMA tile; 256-wide chunk G of K goes to wave
// G % 8, and a wave takes its chunks in pairs. Within a chunk, lane group
// g = lane / 16 owns block 4G + g of row n0 + i (i = lane % 16); the two
// halves of a table entry hold the lane's blocks of the two chunks of a
// pair. MFMA rows are the tokens (rows >= M are zero and never stored).
// Dynamic LDS: s*u [M][r] fp32, then the B columns of the workgroup [r][16]
// bf16.
template <bool kOutBf16>
__global__ __launch_bounds__(512, 4) void gemv_kernel(GemvArgs p, Codebook cb) {
  __shared__ __attribute__((aligned(16))) uint32_t tabs[kGvWaves][16][64];
  extern __shared__ __attribute__((aligned(16))) float dyn[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, i = lane & 15, g = lane >> 4;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int r = p.r;
  const int mr = (int)M * r;
  float* us = dyn;
  uint16_t* bs = reinterpret_cast<uint16_t*>(dyn + mr);
  const int64_t KB = K / 64;                                  // blocks per row
  const int64_t nchunk = (KB + 3) / 4;                        // 256-wide chunks
  const int64_t nch = (nchunk - w + kGvWaves - 1) / kGvWaves; // chunks of this wave
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t nrow = min(n0 + i, N - 1);

  u32x4_t cw[2][2];  // [chunk of the pair][half of the 32-byte block]
  int qv[2];
  float sv[2];
  u32x4_t xa[2][4];  // [buffer][k-step within a half chunk]

  auto block_of = [&](int64_t ci) { return 4 * (kGvWaves * ci + w) + g; };
  auto load_codes = [&](int slot, int64_t ci) {
    const int64_t b = min(block_of(ci), KB - 1);
    const uint8_t* cp = p.codes + nrow * (K / 2) + 32 * b;
    cw[slot][0] = *reinterpret_cast<const u32x4_t*>(cp);
    cw[slot][1] = *reinterpret_cast<const u32x4_t*>(cp + 16);
    const int64_t bi = nrow * KB + b;
    qv[slot] = p.q8[bi];
    sv[slot] = p.s2[bi >> 8];
  };
  // x through a buffer resource: lanes of tokens >= M and blocks past the
  // row end (or past the wave's last chunk) use an out-of-range offset and
  // read zeros without a memory access.
  const __amdgpu_buffer_rsrc_t xres =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.x, (short)0, (int)(M * K * 2), 0x00020000);
  auto load_x = [&](int buf, int64_t ci, int hh) {  // k-steps 4hh .. 4hh+3 of chunk ci
    const int64_t blk = block_of(ci);
    const uint32_t off = (i < M && blk < KB) ? (uint32_t)((i * K + 64 * blk + 32 * hh) * 2)
                                             : 0x80000000u;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      xa[buf][s] = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(xres, (int)(off + 16 * s), 0, 0));
  };

  // Region bits of this wave's tables (address bits 12..14 = wave), or-ed
  // into the high nibble of each code byte.
  const uint32_t region = 0x10101010u * (uint32_t)w;
  const uint32_t colbase = 4u * (uint32_t)lane;
  const char* tab = reinterpret_cast<const char*>(&tabs[0][0][0]);

  // One pair of chunks, straight-line: every load is issued unconditionally
  // (code indices clamped to the wave's last chunk) so that the wait counts
  // stay exact; a chunk past the wave's end gets a zero table.
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  auto pair = [&](int64_t c0, bool reload) {
    // Entry e = {bf16(L[e] c1_hat(block of chunk c0)), bf16(L[e] c1_hat(block of chunk c0+1))};
    // a block past the end of the row gets zeros.
    const float ch0 =
        c0 < nch && block_of(c0) < KB ? q8_value(qv[0], cb.dq_format) * sv[0] : 0.0f;
    const float ch1 =
        c0 + 1 < nch && block_of(c0 + 1) < KB ? q8_value(qv[1], cb.dq_format) * sv[1] : 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e)
      tabs[w][e][lane] = pack_bf16x2(cb.level[e] * ch0, cb.level[e] * ch1);
    const uint32_t cwd[2][8] = {{cw[0][0].x, cw[0][0].y, cw[0][0].z, cw[0][0].w, cw[0][1].x,
                                 cw[0][1].y, cw[0][1].z, cw[0][1].w},
                                {cw[1][0].x, cw[1][0].y, cw[1][0].z, cw[1][0].w, cw[1][1].x,
                                 cw[1][1].y, cw[1][1].z, cw[1][1].w}};
    // 16 lookup groups j = (chunk j/8 of the pair, k-step j%8), software
    // pipelined: the reads of group j+1 are in flight while group j is packed
    // and fed to the MFMA. x streams in half chunks (four groups each), one
    // half chunk ahead.
    uint32_t v[2][8];
    lookup_issue(tab, cwd[0][0], region, colbase, 0, v[0]);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if ((j & 3) == 0) {
        const int q = (j >> 2) + 1;  // next half chunk
        if (q < 4)
          load_x(q & 1, c0 + (q >> 1), q & 1);
        else
          load_x(0, c0 + 2, 0);
      }
      if (j + 1 < 16)
        lookup_issue(tab, cwd[(j + 1) >> 3][(j + 1) & 7], region, colbase, (j + 1) >> 3,
                     v[(j + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      const u32x4_t bop = lookup_pack(v[j & 1]);
      acc = mfma_16x16x32(xa[(j >> 2) & 1][j & 3], bop, acc);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (reload) {
      load_codes(0, min(c0 + 2, nch - 1));
      load_codes(1, min(c0 + 3, nch - 1));
    }
  };

  // The weight stream is issued first; the adapter operands (read only in
  // the epilogue) load behind it into registers and are consumed after the
  // weight work, so their latency overlaps it.
  if (nch > 0) {
    load_codes(0, 0);
    load_codes(1, min((int64_t)1, nch - 1));
    load_x(0, 0, 0);
  }
  // u = sum of the slices in order (same bits as the finalize kernel's sum);
  // the loads use clamped slice indices so that they are issued
  // unconditionally, the padding terms are +0.
  auto uload = [&](int idx, float (&t)[kDecMaxSlices]) {
#pragma unroll
    for (int k = 0; k < kDecMaxSlices; ++k) t[k] = p.upart[(int64_t)min(k, p.slices - 1) * mr + idx];
  };
  auto ustore = [&](int idx, const float (&t)[kDecMaxSlices]) {
    float u = 0.0f;
#pragma unroll
    for (int k = 0; k < kDecMaxSlices; ++k) u += k < p.slices ? t[k] : 0.0f;
    us[idx] = p.s * u;
    if (p.u_out && blockIdx.x == 0) p.u_out[idx] = u;
  };
  auto bval = [&](int idx) {
    const int j = idx >> 4, nl = idx & 15;
    return p.B[(int64_t)j * N + min(n0 + nl, N - 1)];
  };
  float ut[kDecMaxSlices];
  uint16_t bv = 0;
  if (tid < mr) uload(tid, ut);
  if (tid < r * 16) bv = bval(tid);
  if (nch > 0) {
    if (nch <= 2) {
      pair(0, false);
    } else {
      for (int64_t c0 = 0; c0 < nch; c0 += 2) pair(c0, true);
    }
  }
  if (tid < mr) ustore(tid, ut);
  if (tid < r * 16) bs[tid] = bv;
  for (int idx = tid + 512; idx < mr; idx += 512) {  // M * r > 512
    uload(idx, ut);
    ustore(idx, ut);
  }
  for (int idx = tid + 512; idx < r * 16; idx += 512) bs[idx] = bval(idx);  // r > 32

  // Cross-wave sum (each wave's partial tile goes to its own table region,
  // which only it reads), adapter term, store. acc[v] = y partial for token
  // m = 4g + v and row n0 + i.
  float* red = reinterpret_cast<float*>(&tabs[w][0][0]);  // [16][17] per wave
#pragma unroll
  for (int v = 0; v < 4; ++v) red[(4 * g + v) * 17 + i] = acc[v];
  __syncthreads();
  if (tid < 256) {
    const int m = tid >> 4, nl = tid & 15;
    const int64_t n = n0 + nl;
    if (m < M && n < N) {
      const int o = m * 17 + nl;
      float v = reinterpret_cast<const float*>(&tabs[0][0][0])[o];
#pragma unroll
      for (int ww = 1; ww < kGvWaves; ++ww) v += reinterpret_cast<const float*>(&tabs[ww][0][0])[o];
      float lo = 0.0f;
      for (int j = 0; j < r; ++j) lo = __builtin_fmaf(us[m * r + j], bf16_lo(bs[j * 16 + nl]), lo);
      v += lo;
      if (kOutBf16)
        static_cast<uint16_t*>(p.y)[m * N + n] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
      else
        static_cast<float*>(p.y)[m * N + n] = v;
    }
  }
}

__device__ __forceinline__ const void* gv_uniform(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
}

// Buffer resource over `bytes` bytes at `base` (uniform): loads past the end
// return zeros without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t gv_rsrc(const void* base, int64_t bytes) {
  const int n = (int)(bytes < (int64_t)0x7FFFFFFF ? (bytes > 0 ? bytes : 0) : 0x7FFFFFFF);
  return __builtin_amdgcn_make_buffer_rsrc((void*)gv_uniform(base), (short)0, n, 0x00020000);
}

__device__ __forceinline__ u32x4_t gv_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

template <int kFmt>
__device__ __forceinline__ float gv_absmax(int b) {  // b: the byte, zero-extended
  if constexpr (kFmt == kDqInt8) {
    return (float)(b ^ 0x80) - 128.0f;
  } else {
    return q8_value(b, kFmt);
  }
}


// ------------------------------------------- one-round-trip GEMV (K <= 4096)
// Under the full weight stream a memory round trip takes microseconds, so
// gemv_tiles_kernel makes exactly one: every wave issues all of its loads
// (the B columns of the tile and, in wave 0, the down projection's slices,
// which only the epilogue reads; its slice of x by direct-to-LDS loads; its
// absmax bytes, group scale and codes) before its first wait, so that
// every resident workgroup's share of the weight is requested at once. The first lookups wait only for the x slice and the
// codes they read. Per weight a lane does one address permute, one 16-bit
// LDS lookup and half a packing permute; each pair of blocks costs 32
// multiplies and 16 conversions for its table. Measured on the 11008 x 4096
// weight at M = 1 (a ring of 24 weights, each call with the down
// projection): 13.4 us per call against 15.9 us for gemv_kernel; a plain
// read of the codes and absmax bytes with the same grid and load pattern (a
// timing probe) takes 6.2 us, an empty launch of the grid 1.9 us.
constexpr int kTlMaxR = 32;
constexpr int kTlMaxM = 4;  // tokens; a launch is built for at most 2 or at most 4

struct TilesArgs {
  const uint16_t* x;      // [M, K] bf16
  const uint8_t* codes;   // [N, K/2]
  const int8_t* q8;       // [N*K/64]
  const float* s2;        // [ceil(N*K/64/256)]
  const float* upart;     // [slices, M, r] from lora_down_decode
  const uint16_t* B;      // [r, N] bf16
  float* u_out;           // [M, r] fp32 or NULL (written by workgroup 0)
  void* y;                // [M, N] fp32 or bf16
  int64_t M, N, K;
  int r, slices;
  float s;
};

__device__ __forceinline__ uint32_t tl_lookup(const char* tab, uint32_t addr) {
  return *reinterpret_cast<const uint16_t*>(tab + addr);
}

// grid: ceil(N / 16) workgroups of 64 kWaves threads (kWaves = 8 for
// weights with under 1024 tiles, else 4). Workgroup rows n0 .. n0+15 form one 16-row
// MFMA tile. With bpl = 16 / kWaves, lane (i, g) of wave w owns row n0 + i
// and the blocks bpl (4 w + g) .. + bpl - 1, two per table; the table
// (bf16(L[e] c1_hat) for both blocks of a pair, one in each half of an LDS
// dword) sits in a bank-private column: entry e of lane t at 256 e + 4 t in
// the wave's 4 KB region. MFMA rows are the tokens; MFMA step s of a block
// takes, in every lane, the block's weights 8 s .. 8 s + 7, and the x
// operand of the same k comes from the wave's LDS slice of x (the 256 bpl k
// its blocks cover, M <= kMaxM; tokens >= M read a zero row).
template <int kFmt, bool kOutBf16, int kWaves, int kMaxM>
__global__ __launch_bounds__(64 * kWaves) void gemv_tiles_kernel(TilesArgs p, Codebook cb) {
  constexpr int kTlWaves = kWaves;
  // Staged slices (at most 16 x M r floats). The two-token build holds 512
  // (M r <= 32), so that its eight-wave workgroup fits three to a CU.
  constexpr int kTlUp = kMaxM == 2 ? 512 : 16 * kMaxM * kTlMaxR;
  constexpr int kTlBpl = 16 / kWaves;                          // blocks per lane (K <= 4096)
  constexpr int kSpan = 64 * 4 * kTlBpl;                       // k covered by one wave
  constexpr int kXw = 2 * kSpan * kMaxM;                       // x slice bytes per wave
  __shared__ __attribute__((aligned(16))) uint32_t tabs[kTlWaves][16][64];
  __shared__ __attribute__((aligned(16))) unsigned char xs[kTlWaves][kXw + 16];
  __shared__ __attribute__((aligned(16))) float ups[kTlUp];  // wave 0's staged slices
  __shared__ __attribute__((aligned(16))) float usm[kMaxM * kTlMaxR];  // s*u [M][r]
  __shared__ __attribute__((aligned(16))) uint16_t bsm[kTlMaxR * 16];  // B tile [r][16]
  typedef __attribute__((address_space(3))) void lds_void;
  const int tid = threadIdx.x, lane = tid & 63, i = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t M = p.M, N = p.N, K = p.K;
  const int r = p.r;
  const int mr = (int)M * r;
  const int64_t KB = K >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int rows = (int)min((int64_t)16, N - n0);
  const uint32_t nl = (uint32_t)min(i, rows - 1);  // rows past N read row N-1 (never stored)
  const int64_t b0 = kTlBpl * (4 * w + g);          // the lane's first block

  // 1. wave 0: the down projection's slices (slices x M r floats, 1 KB per
  //    instruction) and the tile's B columns, issued first: they are read
  //    only in the epilogue, so the waits before the first lookups skip
  //    them.
  const int upb = p.slices * mr * 4;
  if (w == 0) {
    const __amdgpu_buffer_rsrc_t ures = gv_rsrc(p.upart, upb);
    for (int q = 0; q < (upb + 1023) / 1024; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ures, (lds_void*)(ups + 256 * q), 16,
                                               (uint32_t)(1024 * q + 16 * lane), 0, 0, 0);
  }
  uint16_t bv[kTlMaxR / 16];
#pragma unroll
  for (int q = 0; q < kTlMaxR / 16; ++q) {  // 16 r values over 256 threads
    const int idx = tid + 256 * q;
    const uint32_t bj = (uint32_t)min(idx >> 4, r - 1);
    const uint32_t bc = (uint32_t)min((int64_t)(idx & 15), N - 1 - n0);
    if (q == 0 || idx < 16 * r) bv[q] = (p.B + n0)[bj * (uint32_t)N + bc];
  }


  // 2. x slice of this wave (M <= kMaxM tokens x kSpan k) by direct-to-LDS
  //    loads: instruction q covers 512 k (piece q % kXq) of token q / kXq;
  //    the zero row behind it is written first.
  unsigned char* xw = xs[w];
  if (lane < 4) reinterpret_cast<uint32_t*>(xw + kXw)[lane] = 0u;
  const __amdgpu_buffer_rsrc_t xres = gv_rsrc(p.x, M * K * 2);
  constexpr int kXq = kSpan / 512;  // 1 KB (512 k) pieces per token
#pragma unroll
  for (int q = 0; q < kXq * kMaxM; ++q) {
    const int m = q / kXq, hk = q % kXq;
    const int64_t k = (int64_t)kSpan * w + 512 * hk + 8 * lane;
    const uint32_t off = (m < M && k < K) ? (uint32_t)((m * K + k) * 2) : 0x80000000u;
    if (q < kXq * M)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xres, (lds_void*)(xw + 1024 * q), 16, off, 0, 0, 0);
  }
  // The wait before the first lookups counts the loads issued after the x
  // slices: none may move above them.
  __builtin_amdgcn_sched_barrier(0);
  // 3. codes, absmax bytes and group scales of the lane's four blocks
  //    (blocks past the row end read the row's last block and get zeros).
  const uint32_t kb32 = (uint32_t)KB;
  const __amdgpu_buffer_rsrc_t cres = gv_rsrc(p.codes + n0 * (K >> 1), (int64_t)rows * (K >> 1));
  const __amdgpu_buffer_rsrc_t qres = gv_rsrc(p.q8 + n0 * KB, (int64_t)rows * KB);
  //    Every load instruction costs the CU's load pipeline about the same
  //    whatever its width, so each is as wide as the data allows: the four
  //    blocks' 128 bytes of codes in eight 16-byte loads, their absmax bytes
  //    in one dword (K % 256 == 0: the four bytes are aligned), and one
  //    group scale (four blocks from a multiple of four never straddle a
  //    256-block group).
  u32x4_t cw[kTlBpl][2];
  const uint32_t bq = (uint32_t)min(b0, KB - kTlBpl);  // lanes past the row end: the last blocks
#pragma unroll
  for (int h = 0; h < kTlBpl; ++h) {
    const uint32_t off = nl * (32u * kb32) + 32u * (bq + h);
    cw[h][0] = gv_load16(cres, off);
    cw[h][1] = gv_load16(cres, off + 16);
  }
  const uint32_t qi = nl * kb32 + bq;
  uint32_t q4;
  if constexpr (kTlBpl == 4)
    q4 = __builtin_amdgcn_raw_buffer_load_b32(qres, (int)qi, 0, 0);
  else
    q4 = __builtin_amdgcn_raw_buffer_load_b16(qres, (int)qi, 0, 0);
  const float sv = (p.s2 + ((n0 * KB) >> 8))[((uint32_t)((n0 * KB) & 255) + qi) >> 8];
  const uint32_t region = __builtin_amdgcn_mbcnt_lo(0u, 0u) + 0x10101010u * (uint32_t)w;
  const uint32_t colbase = 4u * (uint32_t)lane;
  const char* tab = reinterpret_cast<const char*>(&tabs[0][0][0]);
  // x operand of step s of block h: x[i][64 (b0 + h) + 8 s .. + 8] from the
  // wave's slice (k within the slice: 256 g + 64 h + 8 s), zeros for i >= M.
  const bool xok = i < M;
  const unsigned char* xrow = xok ? xw + 2 * kSpan * i + 2 * (64 * kTlBpl * g) : xw + kXw;
  const int xstep = xok ? 16 : 0;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  bool first = true;
#pragma unroll
  for (int pr = 0; pr < kTlBpl / 2; ++pr) {
    const int q0 = (int)((q4 >> (16 * pr)) & 0xFFu), q1 = (int)((q4 >> (16 * pr + 8)) & 0xFFu);
    const float ch0 = b0 + 2 * pr < KB ? gv_absmax<kFmt>(q0) * sv : 0.0f;
    const float ch1 = b0 + 2 * pr + 1 < KB ? gv_absmax<kFmt>(q1) * sv : 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) tabs[w][e][lane] = pack_bf16x2(cb.level[e] * ch0, cb.level[e] * ch1);
    if (first) {  // the x slice: every load but the codes, q4 and sv has landed
      constexpr int kYounger = 2 * kTlBpl + 2;
      __builtin_amdgcn_s_waitcnt((kYounger & 15) | ((kYounger >> 4) << 14) | (0x7 << 4));
      first = false;
    }
    const uint32_t dw[16] = {cw[2 * pr][0].x, cw[2 * pr][0].y, cw[2 * pr][0].z, cw[2 * pr][0].w,
                             cw[2 * pr][1].x, cw[2 * pr][1].y, cw[2 * pr][1].z, cw[2 * pr][1].w,
                             cw[2 * pr + 1][0].x, cw[2 * pr + 1][0].y, cw[2 * pr + 1][0].z,
                             cw[2 * pr + 1][0].w, cw[2 * pr + 1][1].x, cw[2 * pr + 1][1].y,
                             cw[2 * pr + 1][1].z, cw[2 * pr + 1][1].w};
    uint32_t va[2][8];
    auto issue = [&](int s, uint32_t (&v)[8]) {  // step s of the pair: block s / 8
      const uint32_t d = dw[s];
      const uint32_t lo = (d & 0x0F0F0F0Fu) | region;
      const uint32_t hi = ((d >> 4) & 0x0F0F0F0Fu) | region;
      const int hh = s >> 3;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        v[2 * b] = tl_lookup(tab, lut_addr(lo, colbase, b) + 2 * hh);
        v[2 * b + 1] = tl_lookup(tab, lut_addr(hi, colbase, b) + 2 * hh);
      }
    };
    issue(0, va[0]);
    issue(1, va[1]);
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      __builtin_amdgcn_sched_barrier(0);
      uint32_t (&v)[8] = va[s & 1];
      const u32x4_t bop{__builtin_amdgcn_perm(v[1], v[0], 0x05040100u),
                        __builtin_amdgcn_perm(v[3], v[2], 0x05040100u),
                        __builtin_amdgcn_perm(v[5], v[4], 0x05040100u),
                        __builtin_amdgcn_perm(v[7], v[6], 0x05040100u)};
      const u32x4_t xop = *reinterpret_cast<const u32x4_t*>(
          xrow + xstep * (8 * (2 * pr + (s >> 3)) + (s & 7)));
      if (s + 2 < 16) issue(s + 2, v);
      acc = mfma_16x16x32(xop, bop, acc);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // u = sum of the slices in order from +0 (the same bits as the finalize
  // kernel's sum), s*u for the epilogue; wave 0 staged the slices.
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): the staged slices
  if (w == 0)
    for (int idx = lane; idx < mr; idx += 64) {
      float t[kDecMaxSlices];
#pragma unroll
      for (int k = 0; k < kDecMaxSlices; ++k) t[k] = ups[min(k, p.slices - 1) * mr + idx];
      float u = 0.0f;
#pragma unroll
      for (int k = 0; k < kDecMaxSlices; ++k) u += k < p.slices ? t[k] : 0.0f;
      usm[idx] = p.s * u;
      if (p.u_out && blockIdx.x == 0) p.u_out[idx] = u;
    }
#pragma unroll
  for (int q = 0; q < kTlMaxR / 16; ++q)
    if (tid + 256 * q < 16 * r) bsm[tid + 256 * q] = bv[q];
  // cross-wave sum (each wave's partial tile in its own table region, which
  // only it reads), adapter term, store. acc[v]: token 4 g + v, row n0 + i.
  float* red = reinterpret_cast<float*>(&tabs[w][0][0]);  // [16][17] per wave
#pragma unroll
  for (int v = 0; v < 4; ++v) red[(4 * g + v) * 17 + i] = acc[v];
  __syncthreads();
  {
    const int m = tid >> 4, c = tid & 15;
    const int64_t n = n0 + c;
    if (m < M && n < N) {
      const int o = m * 17 + c;
      float v = reinterpret_cast<const float*>(&tabs[0][0][0])[o];
#pragma unroll
      for (int ww = 1; ww < kTlWaves; ++ww) v += reinterpret_cast<const float*>(&tabs[ww][0][0])[o];
      float lo = 0.0f;
      for (int j0 = 0; j0 < r; j0 += 16) {
        float uv[16], bw[16];
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          uv[jj] = usm[m * r + j0 + jj];
          bw[jj] = bf16_lo(bsm[(j0 + jj) * 16 + c]);
        }
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) lo = __builtin_fmaf(uv[jj], bw[jj], lo);
      }
      v += lo;
      if (kOutBf16)
        static_cast<uint16_t*>(p.y)[m * N + n] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
      else
        static_cast<float*>(p.y)[m * N + n] = v;
    }
  }
}

}  // namespace

int decode_down_slices(int64_t K) {
  const int64_t pieces = (K + 255) / 256;
  const int64_t per = (pieces + kDecMaxSlices - 1) / kDecMaxSlices;
  return (int)((pieces + per - 1) / per);
}

hipError_t launch_lora_down_decode(const uint16_t* x, const uint16_t* A, int64_t M, int64_t K,
                                   int r, float* part, hipStream_t st) {
  const int slices = decode_down_slices(K);
  const dim3 grid((unsigned)slices, (unsigned)(r / 16));
  hipLaunchKernelGGL(lora_down_decode_kernel, grid, dim3(256), 0, st, x, A, M, K, r,
                     decode_down_len(K, slices), part);
  return hipGetLastError();
}

hipError_t launch_gemv(const uint16_t* x, const uint8_t* codes, const int8_t* q8,
                       const float* s2, const float* upart, int slices, const uint16_t* B,
                       int64_t M, int64_t N, int64_t K, int r, float s, float* u_out, void* y,
                       bool y_bf16, const Codebook& cb, hipStream_t st) {
  const GemvArgs a{x, codes, q8, s2, upart, B, u_out, y, M, N, K, r, slices, s};
  const dim3 grid((unsigned)((N + 15) / 16));
  const size_t dyn = (size_t)M * r * 4 + (size_t)r * 16 * 2;  // s*u and the B columns
  if (y_bf16)
    hipLaunchKernelGGL(gemv_kernel<true>, grid, dim3(64 * kGvWaves), dyn, st, a, cb);
  else
    hipLaunchKernelGGL(gemv_kernel<false>, grid, dim3(64 * kGvWaves), dyn, st, a, cb);
  return hipGetLastError();
}


bool decode_tiles_ok(int64_t M, int64_t N, int64_t K, int r) {
  (void)N;
  // x slice in LDS (up to 4 tokens x the wave's k), the down projection's
  // slices in LDS (16 x M r floats), B tile and s*u in LDS
  return M >= 1 && M <= kTlMaxM && K <= 4096 && K % 256 == 0 && r <= kTlMaxR &&
         (int64_t)decode_down_slices(K) * M * r <= 16 * kTlMaxM * kTlMaxR;
}

hipError_t launch_gemv_tiles(const uint16_t* x, const uint8_t* codes, const int8_t* q8,
                             const float* s2, const float* upart, int slices, const uint16_t* B,
                             int64_t M, int64_t N, int64_t K, int r, float s, float* u_out,
                             void* y, bool y_bf16, const Codebook& cb, hipStream_t st) {
  const TilesArgs a{x, codes, q8, s2, upart, B, u_out, y, M, N, K, r, slices, s};
  const int64_t tiles = (N + 15) / 16;
  const dim3 grid((unsigned)tiles);
  // Eight waves per tile up to 1023 tiles, four beyond. Measured on the
  // 11008 x 4096 weight at M = 1 (688 tiles, a ring of 24 weights): 10.8 us
  // per GEMV with eight waves against 11.4 us with four when two eight-wave
  // workgroups fit a CU (two rounds): each wave has half the chunks, so a
  // wave's compute after its data lands is half as long. With the two-token
  // build's LDS trimmed so that three fit (one round for 688 tiles) the call
  // went 13.5 -> 12.4-12.7 us.
  const bool eight = tiles < 1024;
  // x slices (and staged slices of u) for at most two tokens (M r <= 32), or
  // for three or four tokens (twice the LDS).
  const bool four = M > 2 || (int64_t)slices * M * r > 512;
#define QLORA_TL(F, B16)                                                                      \
  do {                                                                                        \
    if (eight && four)                                                                        \
      hipLaunchKernelGGL((gemv_tiles_kernel<F, B16, 8, 4>), grid, dim3(512), 0, st, a, cb);  \
    else if (eight)                                                                           \
      hipLaunchKernelGGL((gemv_tiles_kernel<F, B16, 8, 2>), grid, dim3(512), 0, st, a, cb);  \
    else if (four)                                                                            \
      hipLaunchKernelGGL((gemv_tiles_kernel<F, B16, 4, 4>), grid, dim3(256), 0, st, a, cb);  \
    else                                                                                      \
      hipLaunchKernelGGL((gemv_tiles_kernel<F, B16, 4, 2>), grid, dim3(256), 0, st, a, cb);  \
  } while (0)
  switch (cb.dq_format) {
    case kDqInt8: if (y_bf16) QLORA_TL(kDqInt8, true); else QLORA_TL(kDqInt8, false); break;
    case kDqUint8: if (y_bf16) QLORA_TL(kDqUint8, true); else QLORA_TL(kDqUint8, false); break;
    default: if (y_bf16) QLORA_TL(kDqE4m3, true); else QLORA_TL(kDqE4m3, false); break;
  }
#undef QLORA_TL
  return hipGetLastError();
}

}  // namespace qlora
