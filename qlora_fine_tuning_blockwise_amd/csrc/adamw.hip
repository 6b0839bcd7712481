// AdamW step on the adapter parameters on gfx950.
//
// [P2] precision table: the Adam state of an adapter parameter is fp32, 12
// bytes, read as the fp32 master value p and the two fp32 moments m and v;
// [P4] "The memory term LoRA does not remove" names master copies and
// optimizer moments as what a trained parameter carries. The bf16 adapter
// the layer reads is RNbf16(p) after the step. [P1] paragraph on paged
// optimizers and [P3] "How it works": the state may live in pinned host
// memory; the kernel then reads and writes it across the host link.
//
// Per element in binary32, every operation rounded, nothing fused (the file
// is built with FP contraction off and correctly rounded sqrt and division):
//   p <- p*decay
//   m <- b1*m + c1*g
//   v <- b2*v + c2*(g*g)
//   p <- p - step_size * (m / (sqrt(v)/bc2_sqrt + eps))
// with the step's scalars computed on the host (AdamScalars).
//
// Streaming layout: one thread updates 8 consecutive parameters, so every
// access is a 16-byte vector (p, m, v: two each; a bf16 gradient or the bf16
// copy: one), all loads issued before any arithmetic. 28 bytes move per
// parameter with a bf16 gradient, 30 with fp32. The last thread of a ragged
// tail takes its elements one by one.
#include "device.h"

namespace qlora {
namespace {

__device__ __forceinline__ void adam_elem(float& p, float& m, float& v, float g,
                                          const AdamScalars& s) {
  const float pd = p * s.decay;
  const float mb = s.b1 * m;
  const float mg = s.c1 * g;
  const float mi = mb + mg;
  const float vb = s.b2 * v;
  const float gg = g * g;
  const float vg = s.c2 * gg;
  const float vi = vb + vg;
  const float sq = __builtin_sqrtf(vi);
  const float dn = sq / s.bc2_sqrt;
  const float de = dn + s.eps;
  const float q = mi / de;
  const float up = s.step_size * q;
  p = pd - up;
  m = mi;
  v = vi;
}

__device__ __forceinline__ uint16_t bf16_bits(float x) { return (uint16_t)pack_bf16x2(x, 0.0f); }

template <bool kGradBf16>
__global__ __launch_bounds__(256) void adamw_kernel(float* __restrict__ p,
                                                    const void* __restrict__ g,
                                                    float* __restrict__ m, float* __restrict__ v,
                                                    uint16_t* __restrict__ pb, int64_t n,
                                                    AdamScalars s) {
  const int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (e0 >= n) return;
  if (e0 + 8 <= n) {
    f32x4_t pv[2], mv[2], vv[2];
    float gv[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      pv[h] = *reinterpret_cast<const f32x4_t*>(p + e0 + 4 * h);
      mv[h] = *reinterpret_cast<const f32x4_t*>(m + e0 + 4 * h);
      vv[h] = *reinterpret_cast<const f32x4_t*>(v + e0 + 4 * h);
    }
    if (kGradBf16) {
      const u32x4_t gq = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(g) + e0);
      const uint32_t gw[4] = {gq.x, gq.y, gq.z, gq.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        gv[2 * i] = bf16_lo(gw[i]);
        gv[2 * i + 1] = bf16_hi(gw[i]);
      }
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f32x4_t gq = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(g) + e0 + 4 * h);
        gv[4 * h] = gq.x;
        gv[4 * h + 1] = gq.y;
        gv[4 * h + 2] = gq.z;
        gv[4 * h + 3] = gq.w;
      }
    }
    float pe[8], me[8], ve[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      pe[4 * h] = pv[h].x; pe[4 * h + 1] = pv[h].y; pe[4 * h + 2] = pv[h].z; pe[4 * h + 3] = pv[h].w;
      me[4 * h] = mv[h].x; me[4 * h + 1] = mv[h].y; me[4 * h + 2] = mv[h].z; me[4 * h + 3] = mv[h].w;
      ve[4 * h] = vv[h].x; ve[4 * h + 1] = vv[h].y; ve[4 * h + 2] = vv[h].z; ve[4 * h + 3] = vv[h].w;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) adam_elem(pe[i], me[i], ve[i], gv[i], s);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      *reinterpret_cast<f32x4_t*>(p + e0 + 4 * h) =
          f32x4_t{pe[4 * h], pe[4 * h + 1], pe[4 * h + 2], pe[4 * h + 3]};
      *reinterpret_cast<f32x4_t*>(m + e0 + 4 * h) =
          f32x4_t{me[4 * h], me[4 * h + 1], me[4 * h + 2], me[4 * h + 3]};
      *reinterpret_cast<f32x4_t*>(v + e0 + 4 * h) =
          f32x4_t{ve[4 * h], ve[4 * h + 1], ve[4 * h + 2], ve[4 * h + 3]};
    }
    if (pb)
      *reinterpret_cast<u32x4_t*>(pb + e0) =
          u32x4_t{pack_bf16x2(pe[0], pe[1]), pack_bf16x2(pe[2], pe[3]),
                  pack_bf16x2(pe[4], pe[5]), pack_bf16x2(pe[6], pe[7])};
  } else {
    for (int64_t e = e0; e < n; ++e) {
      const float ge = kGradBf16 ? bf16_lo(static_cast<const uint16_t*>(g)[e])
                                 : static_cast<const float*>(g)[e];
      float pe = p[e], me = m[e], ve = v[e];
      adam_elem(pe, me, ve, ge, s);
      p[e] = pe;
      m[e] = me;
      v[e] = ve;
      if (pb) pb[e] = bf16_bits(pe);
    }
  }
}

}  // namespace

hipError_t launch_adamw(float* p, const void* g, bool g_bf16, float* m, float* v, uint16_t* pb,
                        int64_t n, const AdamScalars& s, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int64_t threads = (n + 7) / 8;
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (g_bf16)
    hipLaunchKernelGGL(adamw_kernel<true>, grid, dim3(256), 0, st, p, g, m, v, pb, n, s);
  else
    hipLaunchKernelGGL(adamw_kernel<false>, grid, dim3(256), 0, st, p, g, m, v, pb, n, s);
  return hipGetLastError();
}

}  // namespace qlora
