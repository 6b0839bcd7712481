// Device-side helpers for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace qlora {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// Two fp32 values to a packed bf16 pair, round-to-nearest-even
// (one v_cvt_pk_bf16_f32 on gfx950). `a` goes to the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// D = A(16x32) * B(32x16) + C with bf16 inputs and fp32 accumulation.
// Lane l supplies row (l%16) of A and column (l%16) of B, each as the 8
// consecutive reduction elements 8*(l/16)..8*(l/16)+7; it receives rows
// 4*(l/16)..4*(l/16)+3 of column (l%16) of D.
__device__ __forceinline__ f32x4_t mfma_16x16x32(const u32x4_t a, const u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

typedef __attribute__((ext_vector_type(16))) float f32x16_t;

// D = A(32x16) * B(16x32) + C with bf16 inputs and fp32 accumulation (the
// full-rate bf16 MFMA of gfx950: 32K flops in 32 cycles). Lane l supplies row
// (l%32) of A and column (l%32) of B as the 8 consecutive reduction elements
// 8*(l/32)..8*(l/32)+7; its accumulator element e holds
// D[8*(e/4) + 4*(l/32) + e%4][l%32].
__device__ __forceinline__ f32x16_t mfma_32x32x16(const u32x4_t a, const u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Dequantized values of the 8 NF4 codes in one little-endian dword through a
// 16-entry bf16 table in LDS (the table of one block: bf16(L[i] * c1_hat)).
// Element i (nibble i) lands in bf16 slot i of the result.
__device__ __forceinline__ u32x4_t lut8(uint32_t w, const uint16_t* tab) {
  u32x4_t r;
  r.x = (uint32_t)tab[w & 15u] | ((uint32_t)tab[(w >> 4) & 15u] << 16);
  r.y = (uint32_t)tab[(w >> 8) & 15u] | ((uint32_t)tab[(w >> 12) & 15u] << 16);
  r.z = (uint32_t)tab[(w >> 16) & 15u] | ((uint32_t)tab[(w >> 20) & 15u] << 16);
  r.w = (uint32_t)tab[(w >> 24) & 15u] | ((uint32_t)tab[w >> 28] << 16);
  return r;
}

// Value of a stored 8-bit absmax code (the byte, loaded as int8 into `raw`)
// in second-level format `fmt`: the signed byte, the unsigned byte, or the
// FP8 E4M3 value (exponent bias 7, subnormals m * 2^-9). Exact in fp32.
// Branch-free: all three readings are formed and the uniform format picks
// one by bit masks, so a caller's loads stay batched (a branch on the format
// would wait for them inside each arm).
__device__ __forceinline__ float q8_value(int raw, int fmt) {
  const uint32_t b = (uint32_t)raw & 0xFFu;
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  const uint32_t nrm = ((e + 120u) << 23) | (m << 20);
  const uint32_t sub = __float_as_uint((float)m * 0x1p-9f);
  const uint32_t fp8 = (e ? nrm : sub) | ((b & 0x80u) << 24);
  const uint32_t i8 = __float_as_uint((float)raw);
  const uint32_t u8 = __float_as_uint((float)b);
  const uint32_t sel_i8 = 0u - (uint32_t)(fmt == kDqInt8);
  const uint32_t sel_u8 = 0u - (uint32_t)(fmt == kDqUint8);
  return __uint_as_float((i8 & sel_i8) | (u8 & sel_u8) | (fp8 & ~(sel_i8 | sel_u8)));
}

// Build the 16-entry bf16 dequantization table of one block from its
// 8-bit absmax code and the group scale: entry i = bf16(fp32(L[i] * c1_hat)),
// c1_hat = fp32(value(q8) * s2). Writes 32 bytes at `dst` (16-byte aligned).
__device__ __forceinline__ void build_table(const Codebook& cb, int q8, float s2, uint16_t* dst) {
  const float ch = q8_value(q8, cb.dq_format) * s2;
  u32x4_t t0, t1;
  t0.x = pack_bf16x2(cb.level[0] * ch, cb.level[1] * ch);
  t0.y = pack_bf16x2(cb.level[2] * ch, cb.level[3] * ch);
  t0.z = pack_bf16x2(cb.level[4] * ch, cb.level[5] * ch);
  t0.w = pack_bf16x2(cb.level[6] * ch, cb.level[7] * ch);
  t1.x = pack_bf16x2(cb.level[8] * ch, cb.level[9] * ch);
  t1.y = pack_bf16x2(cb.level[10] * ch, cb.level[11] * ch);
  t1.z = pack_bf16x2(cb.level[12] * ch, cb.level[13] * ch);
  t1.w = pack_bf16x2(cb.level[14] * ch, cb.level[15] * ch);
  *reinterpret_cast<u32x4_t*>(dst) = t0;
  *reinterpret_cast<u32x4_t*>(dst + 8) = t1;
}

// Byte address of an LDS location (for explicit address arithmetic).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)p;
}

// Wait until at most `n` vector-memory operations of this wave are in flight
// (loads, including direct-to-LDS loads, complete in issue order). Other
// counters are left alone; the scheduler may not move instructions across
// it. gfx9 s_waitcnt encoding: vmcnt in bits [3:0] and
// [15:14], expcnt [6:4] (7 = no wait), lgkmcnt [11:8] (15 = no wait).
template <int n>
__device__ __forceinline__ void wait_vmem() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  __builtin_amdgcn_sched_barrier(0);  // nothing may be scheduled across the wait
}

__device__ __forceinline__ u32x4_t zero4() { return u32x4_t{0u, 0u, 0u, 0u}; }

// sum_{k < n} p[k * stride], added in order k = 0, 1, ... starting from +0.
// The loads of U consecutive terms are issued together (a plain loop with a
// run-time trip count waits for each load in turn); the padding terms are +0
// and leave the sum unchanged, so every U gives the same bits.
template <int U>
__device__ __forceinline__ float sum_strided(const float* __restrict__ p, int64_t stride, int n) {
  float v = 0.0f;
  for (int k0 = 0; k0 < n; k0 += U) {
    float t[U];
#pragma unroll
    for (int k = 0; k < U; ++k) t[k] = k0 + k < n ? p[(int64_t)(k0 + k) * stride] : 0.0f;
#pragma unroll
    for (int k = 0; k < U; ++k) v += t[k];
  }
  return v;
}

}  // namespace qlora
