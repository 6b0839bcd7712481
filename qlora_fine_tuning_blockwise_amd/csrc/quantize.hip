// Blockwise NF4 quantization with double quantization, and dequantization to
// bf16 (row-major, and transposed for the input gradient), for gfx950.
//
// [P1] "QLoRA", "controlled rounding": per block of weights find the absmax,
// normalise, store the index of the nearest grid point plus one scale per
// block; bullets: blocks of 64, NF4 levels, and the block constants quantized
// again to 8 bits ("double quantization"). [P2] s1 "Double Quantization".
//
// Quantize: one workgroup per group of 256 blocks (16384 weights). Each thread
// loads 8 consecutive weights per pass (a 16-byte bf16 load, coalesced across
// the wave), 8 lanes cover one block; the block absmax is reduced across those
// 8 lanes with DPP moves. Codes come from a 65-bucket table in LDS: the bucket
// of x in [-1,1] (width 1/32) holds at most one decision threshold, so one
// compare finishes the search. For bf16 weights the compare is made on the
// weight itself, w > t' c1 (the sign of one FMA), with the quotient threshold
// t' of the codebook, so no quotient is formed. The 8 codes of a thread are
// packed into one dword and stored. After all passes the 256 block constants
// are in LDS and the workgroup writes their 8-bit codes and the group's fp32
// scale.
#include "device.h"

namespace qlora {
namespace {

constexpr int kLut = 128;  // 65 live buckets, padded so a masked index stays in bounds
// Threads per group: 512 (4 passes). Measured against 256 threads x 8 passes
// on one GPU: equal or faster for every layer shape (8192 x 8192: 31.3 ->
// 28.4 us; 8192 x 28672: 115.5 -> 109.8 us; 28672 x 8192: 117.0 -> 115.7
// us), and it fills the GPU when there are few groups.
constexpr int kQThreadsUsed = 512;
static_assert(kGroup == 4 * 64 && 2 * kLut == 256, "");

// Max of a non-negative value over each aligned group of 8 lanes.
__device__ __forceinline__ uint32_t max_over_8_lanes(uint32_t v) {
  // quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  return v;
}

// Code of a normalised value x in [-1,1]: bucket b = floor(32x + 32), then
// code = (#thresholds below the bucket) + (x > the bucket's threshold).
// The byte offset 8b of the bucket's 8-byte entry is floor(256x + 256) with
// its low three bits cleared (scaling by 8 commutes with the rounding, and
// floor(8y) & ~7 = 8 floor(y) for y >= 0), so one AND both scales and masks;
// the mask keeps a non-finite x inside the table.
__device__ __forceinline__ uint32_t nf4_code(float x, const u32x2_t* lut) {
  const uint32_t off = ((uint32_t)(int)__builtin_fmaf(x, 256.0f, 256.0f)) & (8u * kLut - 8u);
  const u32x2_t e = *reinterpret_cast<const u32x2_t*>(reinterpret_cast<const char*>(lut) + off);
  return e.y + (x > __uint_as_float(e.x) ? 1u : 0u);
}

typedef __attribute__((ext_vector_type(2))) unsigned short u16x2_t;

// Largest |w| bit pattern of the bf16 pairs in four words, as fp32 bits:
// packed 16-bit maxima of the magnitudes, then the larger half.
__device__ __forceinline__ uint32_t absmax_bf16x8(const uint32_t (&v)[4]) {
  u16x2_t m[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) m[j] = __builtin_bit_cast(u16x2_t, v[j] & 0x7FFF7FFFu);
  const u16x2_t a = __builtin_elementwise_max(__builtin_elementwise_max(m[0], m[1]),
                                              __builtin_elementwise_max(m[2], m[3]));
  return (uint32_t)max(a.x, a.y) << 16;
}

// Nearest FP8 E4M3 code of x >= 0 (or +inf), ties to the even code,
// saturating at 448 (code 0x7E). Below 2^-6 the values are the subnormals
// m * 2^-9, so the code is x * 2^9 rounded to an integer (exact scaling,
// rint rounds ties to even; 8 lands on the smallest normal, code 0x08).
// Above, rounding the fp32 pattern at mantissa bit 20 to nearest-even keeps
// 3 mantissa bits (a carry moves into the exponent), and the exponent field
// is rebased from 127 to 7.
__device__ __forceinline__ int e4m3_code(float x) {
  if (!(x < 448.0f)) return 0x7E;
  if (x < 0x1p-6f) return (int)__builtin_rintf(x * 0x1p9f);
  uint32_t b = __float_as_uint(x);
  b += 0x7FFFFu + ((b >> 20) & 1u);
  const int q = (int)((((b >> 23) - 120u) << 3) | ((b >> 20) & 7u));
  return q < 0x7E ? q : 0x7E;
}

template <bool kF32In, int kQThreads>
__global__ __launch_bounds__(kQThreads) void quantize_kernel(const void* __restrict__ W,
                                                             int64_t nblocks,
                                                             uint8_t* __restrict__ codes,
                                                             int8_t* __restrict__ q8,
                                                             float* __restrict__ s2, Codebook cb) {
  __shared__ u32x2_t lut[kLut];
  __shared__ u32x2_t lutq[kLut];  // entry j: bucket j - 1, quotient threshold
  __shared__ float c1s[kGroup];
  __shared__ float red[4];
  constexpr int kQPasses = kGroup * kBlock / (8 * kQThreads);  // passes per thread
  constexpr int kQBlocksPerPass = kQThreads / 8;
  static_assert(kQPasses >= 1 && kQPasses <= 8 && kQBlocksPerPass * kQPasses == kGroup, "");
  const int tid = threadIdx.x;
  const int64_t g = blockIdx.x;
  const int64_t b0 = g * kGroup;
  const int nbg = (int)min((int64_t)kGroup, nblocks - b0);

  if (tid < 2 * kLut) {
    // bucket [lo, lo + 1/32); buckets past 64 repeat bucket 64. lutq is the
    // same table shifted up one entry (entry 0 repeats bucket 0) and holding
    // the quotient threshold in place of the threshold. Threads kLut.. build
    // lutq, so each wave builds half a table.
    auto entry = [&](int b, bool quotient) {
      const float lo = -1.0f + (float)b * 0.03125f;
      const float hi = lo + 0.03125f;
      uint32_t below = 0;
      float inside = 2.0f;
#pragma unroll
      for (int i = 0; i < 15; ++i) {
        const float t = cb.thr[i];
        below += (t < lo) ? 1u : 0u;
        if (t >= lo && t < hi) inside = quotient ? cb.thr_q[i] : t;
      }
      return u32x2_t{__float_as_uint(inside), below};
    };
    if (tid < kLut)
      lut[tid] = entry(min(tid, 64), false);
    else
      lutq[tid - kLut] = entry(min(max(tid - kLut - 1, 0), 64), true);
  }

  // Issue every load of the group up front (kQPasses passes x 8 weights).
  // Blocks past the group's end (last group only) load the group's last
  // block instead: no branch around the loads, so each pass waits only for
  // its own. Their constants and codes are never stored. The weight is read
  // once, so the loads carry the nontemporal hint: on the 8192 x 28672 bf16
  // tensor 106 -> 90 us (0.70 -> 0.82 of HBM peak), the codes unchanged.
  constexpr int kWords = kF32In ? 8 : 4;  // dwords per 8 weights
  uint32_t raw[kQPasses][kWords];
#pragma unroll
  for (int it = 0; it < kQPasses; ++it) {
    const int bl = min(it * kQBlocksPerPass + (tid >> 3), nbg - 1);
    const int64_t e0 = (b0 + bl) * kBlock + (tid & 7) * 8;
    if (kF32In) {
      const u32x4_t* p = reinterpret_cast<const u32x4_t*>(static_cast<const float*>(W) + e0);
      const u32x4_t a = __builtin_nontemporal_load(p), b = __builtin_nontemporal_load(p + 1);
      raw[it][0] = a.x; raw[it][1] = a.y; raw[it][2] = a.z; raw[it][3] = a.w;
      raw[it][4] = b.x; raw[it][5] = b.y; raw[it][6] = b.z; raw[it][7] = b.w;
    } else {
      const u32x4_t a = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(W) + e0));
      raw[it][0] = a.x; raw[it][1] = a.y; raw[it][2] = a.z; raw[it][3] = a.w;
    }
  }
  // The table is ready once every wave's LDS writes are done. A plain
  // barrier after an LDS-only wait: a full __syncthreads would also wait for
  // the weight loads above, and each pass should start when its own arrive.
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt untouched
  __builtin_amdgcn_s_barrier();

  // Block constants of all passes first: lane j < kQPasses of each 8-lane
  // group then computes the correctly rounded reciprocal for pass j alone,
  // and every pass fetches its reciprocal from that lane (one division per
  // lane instead of one per pass).
  float c1v[kQPasses];
#pragma unroll
  for (int it = 0; it < kQPasses; ++it) {
    uint32_t amax = 0;
    if (kF32In) {
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = max(amax, raw[it][j] & 0x7FFFFFFFu);
    } else {
      amax = absmax_bf16x8(*reinterpret_cast<const uint32_t(*)[4]>(&raw[it][0]));
    }
    c1v[it] = __uint_as_float(max_over_8_lanes(amax));
    const int bl = it * kQBlocksPerPass + (tid >> 3);
    if (bl < nbg && (tid & 7) == 0) c1s[bl] = c1v[it];
  }
  float rc_mine = 1.0f;
  if (!kF32In) {
    float c1_mine = c1v[0];
#pragma unroll
    for (int it = 1; it < kQPasses; ++it)
      if ((tid & 7) == it) c1_mine = c1v[it];
    rc_mine = 1.0f / c1_mine;  // +inf for an all-zero block (unused)
  }

  // This thread's code word of pass `it`: block it*kQBlocksPerPass + tid/8 of
  // the group, word tid%8, i.e. dword tid + kQThreads*it of the group's codes.
  uint32_t* const cwp = reinterpret_cast<uint32_t*>(codes + b0 * (kBlock / 2)) + tid;
#pragma unroll
  for (int it = 0; it < kQPasses; ++it) {
    const int bl = it * kQBlocksPerPass + (tid >> 3);
    float w[8];
    if (kF32In) {
#pragma unroll
      for (int j = 0; j < 8; ++j) w[j] = __uint_as_float(raw[it][j]);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t v = raw[it][j];
        w[2 * j] = __uint_as_float(v << 16);
        w[2 * j + 1] = __uint_as_float(v & 0xFFFF0000u);
      }
    }
    const float c1 = c1v[it];

    uint32_t word = 0;
    if (c1 == 0.0f) {
      word = 0x77777777u;  // all-zero block: every weight at the zero level
    } else if (!kF32In && c1 >= 0x1p-60f && c1 <= 0x1p60f) {
      // No quotient: the bucket comes from w * (256 r) + (2^23 + 264) in one
      // FMA (r the correctly rounded 1/c1, from lane it of this lane's
      // group); at that magnitude the fp32 ulp is 1, so the low mantissa bits
      // hold round(256x + 264) and clearing the low three gives the byte
      // offset 8 (bucket + 1) of lutq. Rounding to nearest instead of down
      // can move x up one bucket from the last 1/16 of its bucket, where the
      // codebook has no threshold, so the code is unchanged. The one compare
      // is then w > t' c1 for the bucket's quotient threshold t': the sign of
      // fma(-t', c1, w), exact. Checked exhaustively on the host over every
      // bf16 pair with c1 in this range and |w| <= c1 against the code of the
      // IEEE quotient.
      const float rc256 = __shfl(rc_mine, (tid & 56) | it) * 256.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float f = __builtin_fmaf(w[j], rc256, 8388872.0f);
        const u32x2_t e = *reinterpret_cast<const u32x2_t*>(
            reinterpret_cast<const char*>(lutq) + (__float_as_uint(f) & 0x3F8u));
        const float d = __builtin_fmaf(-__uint_as_float(e.x), c1, w[j]);
        word |= (e.y + (d > 0.0f ? 1u : 0u)) << (4 * j);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) word |= nf4_code(w[j] / c1, lut) << (4 * j);
    }
    if (bl < nbg) cwp[kQThreads * it] = word;
  }
  __syncthreads();  // c1s complete

  // Second level: c2 = max c1 over the group, s2 = c2/top with top = 127,
  // 255 or 448 by format; q8 = the nearest integer of c1/s2 (ties to the
  // lower) clamped to [0, top], or its nearest E4M3 value (ties to even).
  // The first kGroup threads (whole waves) hold one block constant each.
  const float c1 = tid < nbg ? c1s[tid] : 0.0f;
  if (tid < kGroup) {
    float m = c1;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if ((tid & 63) == 0) red[tid >> 6] = m;
  }
  __syncthreads();
  const float c2 = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int fmt = cb.dq_format;
  const float top = fmt == kDqInt8 ? 127.0f : fmt == kDqUint8 ? 255.0f : 448.0f;
  const float sc = c2 / top;
  if (tid < nbg) {
    int q = 0;
    if (c1 != 0.0f) {
      const float v = c1 / sc;  // +inf when sc underflowed to 0
      if (fmt == kDqE4m3) {
        q = e4m3_code(v);
      } else {
        float t = ceilf(v - 0.5f);  // v - 0.5 is exact for v >= 0.5
        t = fminf(fmaxf(t, 0.0f), top);
        q = (int)t;
      }
    }
    q8[b0 + tid] = (int8_t)(uint8_t)q;
  }
  if (tid == 0) s2[g] = sc;
}

// Dequantize. Lane j (0..7) of an 8-lane group takes code word j (codes
// 8j..8j+7) of one block, so a wave covers 8 consecutive blocks per pass:
// 256 bytes of codes in and 1 KB of bf16 out, both contiguous. Each block's
// 16-entry bf16 table (bf16(L[i] * c1_hat)) sits at bytes 32g of the pass's
// 256-byte LDS region (g = block within the pass): the 8 tables fill one row
// of the 64 LDS banks, and a group only reads its own table, so every lookup
// instruction is free of bank conflicts. Lane j writes entries 2j and 2j+1;
// its group reads them back in the same wave (LDS keeps a wave's order). A
// lookup address is one v_perm: byte 0 = 32g + 2*code (computed four codes
// at a time), bytes 1..3 = the region's offset. Each wave runs kDqPasses
// passes with every load issued first. Lanes past the last block redo the
// last block (same values to the same place), so no lane branches. The
// row-major output (the standalone dequantization) is written with the
// nontemporal hint: on the 8192 x 28672 weight 101 -> 83 us. The K-slab
// copy keeps plain stores: the dense GEMM reads it right after, and with
// the hint the layer's calls measured 0.5-1% slower (one box, alternating
// runs), although the copy alone was faster (120 -> 87 us).
// With kKSlab the output is the K-slab layout [K/32][rows][32] of a weight
// with `rows` rows of kb blocks, and a wave takes 8 consecutive rows (one per
// group) by kDqPasses consecutive blocks (one per pass) instead: per pass,
// lanes 0-3 of the 8 groups write slab 2*blk for the 8 rows, 512 contiguous
// bytes, and lanes 4-7 the next slab, so every store fills whole cache
// lines; the passes walk along each row's 128-byte line of codes. Rows and
// blocks past the end are clamped to the last (same values, same place).
constexpr int kDqPasses = 4;

template <bool kKSlab>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ codes,
                                                      const int8_t* __restrict__ q8,
                                                      const float* __restrict__ s2,
                                                      int64_t nblocks, uint16_t* __restrict__ out,
                                                      uint32_t rows, uint32_t kb, Codebook cb) {
  __shared__ __attribute__((aligned(1024))) uint32_t tab[4 * kDqPasses * 64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 3, j = lane & 7;
  const int64_t b0 = ((int64_t)blockIdx.x * 4 + w) * (8 * kDqPasses) + g;
  uint32_t srow = 0, sblk0 = 0;  // K-slab mode: this group's row, the wave's first block
  if (kKSlab) {
    // Consecutive waves take consecutive block groups of one row group, so
    // the waves that run together read each row's codes as one contiguous
    // run. (Row groups first would make them read 128 bytes per row at the
    // row stride of the codes, K/2 bytes: measured 148 against 122 us on a
    // 28672 x 8192 weight, although the slabs then fill sequentially.)
    const uint32_t wid = (uint32_t)blockIdx.x * 4 + (uint32_t)__builtin_amdgcn_readfirstlane(w);
    const uint32_t ncg = (kb + kDqPasses - 1) / kDqPasses;  // block groups
    const uint32_t rg = wid / ncg;
    srow = min(8 * rg + (uint32_t)g, rows - 1);
    sblk0 = min((wid - rg * ncg) * kDqPasses, kb - 1);
  }
  int64_t bk[kDqPasses];
  uint32_t cw[kDqPasses];
  float ch[kDqPasses];
#pragma unroll
  for (int p = 0; p < kDqPasses; ++p) {
    if (kKSlab)
      bk[p] = (int64_t)srow * kb + min(sblk0 + (uint32_t)p, kb - 1);
    else
      bk[p] = b0 + 8 * p < nblocks ? b0 + 8 * p : nblocks - 1;
    cw[p] = reinterpret_cast<const uint32_t*>(codes)[bk[p] * 8 + j];
    ch[p] = q8_value(q8[bk[p]], cb.dq_format) * s2[bk[p] >> 8];
  }
  // levels 2j and 2j+1 of this lane (uniform values, selected per lane)
  float l0 = cb.level[0], l1 = cb.level[1];
#pragma unroll
  for (int jj = 1; jj < 8; ++jj)
    if (j == jj) {
      l0 = cb.level[2 * jj];
      l1 = cb.level[2 * jj + 1];
    }
  const char* tb = reinterpret_cast<const char*>(tab);
  const uint32_t gb = 0x01010101u * (uint32_t)(32 * g);
#pragma unroll
  for (int p = 0; p < kDqPasses; ++p)
    tab[(w * kDqPasses + p) * 64 + 8 * g + j] = pack_bf16x2(l0 * ch[p], l1 * ch[p]);
#pragma unroll
  for (int p = 0; p < kDqPasses; ++p) {
    const uint32_t region = (uint32_t)(w * kDqPasses + p) * 256u;  // low byte 0
    const uint32_t tl = ((cw[p] & 0x0F0F0F0Fu) << 1) + gb;        // 32g + 2*code, per byte
    const uint32_t th = (((cw[p] >> 4) & 0x0F0F0F0Fu) << 1) + gb;
    uint32_t v[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t sel = 0x03020104u + (uint32_t)k;
      v[2 * k] = *reinterpret_cast<const uint16_t*>(tb + __builtin_amdgcn_perm(tl, region, sel));
      v[2 * k + 1] = *reinterpret_cast<const uint16_t*>(tb + __builtin_amdgcn_perm(th, region, sel));
    }
    uint16_t* dst;
    if (kKSlab) {
      const uint32_t s = 2 * min(sblk0 + (uint32_t)p, kb - 1) + (uint32_t)(j >> 2);
      dst = out + ((int64_t)s * rows + srow) * 32 + 8 * (j & 3);
    } else {
      dst = out + bk[p] * 64 + 8 * j;
    }
    const u32x4_t ov{__builtin_amdgcn_perm(v[1], v[0], 0x05040100u),
                     __builtin_amdgcn_perm(v[3], v[2], 0x05040100u),
                     __builtin_amdgcn_perm(v[5], v[4], 0x05040100u),
                     __builtin_amdgcn_perm(v[7], v[6], 0x05040100u)};
    if (kKSlab)
      *reinterpret_cast<u32x4_t*>(dst) = ov;
    else
      __builtin_nontemporal_store(ov, reinterpret_cast<u32x4_t*>(dst));
  }
}

// w_hat^T in the K-slab layout [N/32][K][32]: out[s][k][j] =
// bf16(L[code(32 s + j, k)] * c1_hat(32 s + j, k / 64)), c1_hat = fp32(q8 * s2)
// (the same roundings as the row-major dequantization). A workgroup owns one
// slab s and the 256 columns [k0, k0 + 256): its output is one contiguous
// 16 KB run, and its 16 KB LDS tile leaves room for eight workgroups on a CU.
// Thread t owns the row pair (32 s + 2p, 32 s + 2p + 1), p = t / 16, and the
// 16 columns [k0 + 16c, +16), c = t % 16, so sixteen consecutive lanes read a
// row's 128 bytes of codes. It packs the pair of each column into one dword
// of the transposed tile (row k: 16 dwords, the slab row's 64 bytes), dword p
// at position p ^ (4 ((k >> 2) & 3)), which keeps aligned groups of four
// dwords together for the 16-byte reads. In write step j a lane takes column
// (j + c) % 16 of its own 16, so the 64 lanes of a write cover every residue
// of k mod 16 and, with the swizzle, spread over all banks two lanes a bank.
// The stores carry no nontemporal hint: the dense GEMM reads the copy next.
constexpr int kDtCols = 256;  // tile columns (k)

__global__ __launch_bounds__(256) void dequant_t_kernel(const uint8_t* __restrict__ codes,
                                                        const int8_t* __restrict__ q8,
                                                        const float* __restrict__ s2, int64_t K,
                                                        uint16_t* __restrict__ out, Codebook cb) {
  __shared__ __attribute__((aligned(16))) uint32_t tile[kDtCols * 16];
  __shared__ float levels[16];
  const int tid = threadIdx.x;
  const int64_t KB = K / 64, ktiles = (K + kDtCols - 1) / kDtCols;
  const int64_t slab = blockIdx.x / ktiles, k0 = (int64_t)(blockIdx.x % ktiles) * kDtCols;
  const int p = tid >> 4, c = tid & 15;
  const int64_t na = 32 * slab + 2 * p, nb = na + 1;  // < N: the grid covers whole slabs
  const int64_t kk = k0 + 16 * c;
  uint64_t wa = 0, wb = 0;
  float cha = 0.0f, chb = 0.0f;
  if (kk < K) {
    const int64_t blk = kk / 64;
    wa = *reinterpret_cast<const uint64_t*>(codes + na * (K / 2) + kk / 2);
    wb = *reinterpret_cast<const uint64_t*>(codes + nb * (K / 2) + kk / 2);
    cha = q8_value(q8[na * KB + blk], cb.dq_format) * s2[(na * KB + blk) >> 8];
    chb = q8_value(q8[nb * KB + blk], cb.dq_format) * s2[(nb * KB + blk) >> 8];
  }
  if (tid < 16) levels[tid] = cb.level[tid];
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int jj = (j + c) & 15;  // weight kk + jj: code nibble jj
    const int k = 16 * c + jj;
    const float va = levels[(uint32_t)(wa >> (4 * jj)) & 15u] * cha;
    const float vb = levels[(uint32_t)(wb >> (4 * jj)) & 15u] * chb;
    tile[16 * k + (p ^ (4 * ((k >> 2) & 3)))] = pack_bf16x2(va, vb);
  }
  __syncthreads();
  // Pass i: thread t copies slab row k = 64 i + t / 4, 16-byte piece q = t % 4
  // (weight rows 8q .. 8q + 7 of the slab); the workgroup writes 4 KB of
  // consecutive bytes per pass.
  const int q = tid & 3;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = 64 * i + (tid >> 2);
    if (k0 + k >= K) break;
    const u32x4_t v =
        *reinterpret_cast<const u32x4_t*>(&tile[16 * k + 4 * (q ^ ((k >> 2) & 3))]);
    *reinterpret_cast<u32x4_t*>(out + (slab * K + k0 + k) * 32 + 8 * q) = v;
  }
}

}  // namespace

hipError_t launch_quantize(const void* W, bool f32_in, int64_t n, uint8_t* codes, int8_t* q8,
                           float* s2, const Codebook& cb, hipStream_t st) {
  const int64_t nb = n / kBlock;
  const int64_t ng = (nb + kGroup - 1) / kGroup;
  if (ng == 0) return hipSuccess;
  const dim3 grid((unsigned)ng);
  if (f32_in)
    hipLaunchKernelGGL((quantize_kernel<true, kQThreadsUsed>), grid, dim3(kQThreadsUsed), 0, st, W,
                       nb, codes, q8, s2, cb);
  else
    hipLaunchKernelGGL((quantize_kernel<false, kQThreadsUsed>), grid, dim3(kQThreadsUsed), 0, st, W,
                       nb, codes, q8, s2, cb);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* codes, const int8_t* q8, const float* s2, int64_t n,
                          uint16_t* out, int64_t rows, const Codebook& cb, hipStream_t st) {
  const int64_t nb = n / kBlock;
  const int64_t per_wg = 4 * 8 * kDqPasses;  // blocks per workgroup
  const int64_t grid = (nb + per_wg - 1) / per_wg;
  if (grid == 0) return hipSuccess;
  if (rows > 0) {
    if (nb >= ((int64_t)1 << 32) || nb % rows) return hipErrorInvalidValue;
    const int64_t kb = nb / rows;
    const int64_t waves = (rows + 7) / 8 * ((kb + kDqPasses - 1) / kDqPasses);
    hipLaunchKernelGGL(dequant_kernel<true>, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st,
                       codes, q8, s2, nb, out, (uint32_t)rows, (uint32_t)kb, cb);
  } else {
    hipLaunchKernelGGL(dequant_kernel<false>, dim3((unsigned)grid), dim3(256), 0, st, codes, q8,
                       s2, nb, out, 0u, 0u, cb);
  }
  return hipGetLastError();
}


hipError_t launch_dequant_t(const uint8_t* codes, const int8_t* q8, const float* s2, int64_t N,
                            int64_t K, uint16_t* out, const Codebook& cb, hipStream_t st) {
  if (N % 32 || K % 64) return hipErrorInvalidValue;
  if (N == 0 || K == 0) return hipSuccess;
  // Tiles along K first: consecutive workgroups read each row's codes as one
  // run and write each slab in order.
  const int64_t tiles = N / 32 * ((K + kDtCols - 1) / kDtCols);
  if (tiles >= ((int64_t)1 << 32)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(dequant_t_kernel, dim3((unsigned)tiles), dim3(256), 0, st, codes, q8, s2, K,
                     out, cb);
  return hipGetLastError();
}

}  // namespace qlora
