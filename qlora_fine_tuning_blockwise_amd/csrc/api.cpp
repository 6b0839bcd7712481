// C ABI of the library: argument validation, workspace layout and the launch
// sequence of each entry point. Every check runs on the host before anything
// is enqueued; the compute entry points only enqueue kernels on the caller's
// stream.
#include <cmath>
#include <cstring>

#include "../../include/qlora_amd.h"
#include "internal.h"

namespace qlora {
namespace {

constexpr int64_t kGemvMaxM = 16;  // decode sizes take the GEMV path
// From this many rows on (training batches) the forward has two routes:
//  - fast: the weight is dequantized once into the caller's workspace (one
//    layer's worth of bf16, K-slab layout) and a plain bf16 MFMA GEMM runs on
//    it; needs N*K*2 bytes more workspace;
//  - lean: the fused kernel dequantizes each weight tile in registers right
//    before its MFMAs, so no bf16 copy of the weight ever exists.
// The call takes the fast route when the workspace holds it, else the lean
// one (qlora_workspace_bytes with QLORA_OP_FWD or QLORA_OP_FWD_LEAN).
// Below 512 rows the 512 x 128-tile kernel dequantizes in LDS.
constexpr int64_t kPlainMinM = 512;

bool fwd_plain(int64_t M, int64_t N, int64_t K) {
  return M >= kPlainMinM && gemm_nt_supported(K, K, 0, N, true);
}
bool fwd_fused(int64_t M, int64_t N, int64_t K) {
  return M >= kPlainMinM && gemm_nf4_supported(M, N, K);
}
// The backward's dX from 512 rows on: the weight is dequantized once,
// transposed, into the workspace (K-slab layout: whole cache lines per
// direct-to-LDS load of the GEMM's b operand), then a plain bf16 GEMM.
bool bwd_plain(int64_t M, int64_t N, int64_t K) {
  return M >= kPlainMinM && N % 32 == 0 && gemm_nt_supported(N, N, 0, K, true);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Every product of two of M, N and K stays at most 2^40 (a bf16 matrix of
// 2 TiB, far beyond one GPU's memory), so no byte count, workspace size or
// offset formed from them can overflow 64 bits.
constexpr int64_t kMaxElems = int64_t(1) << 40;

bool shape_ok(int64_t N, int64_t K) {
  return N >= 1 && K >= 64 && K % 64 == 0 && N <= kMaxElems / K;
}

// M rows against a weight of shape_ok (N, K >= 1); M >= 0 is checked first.
bool rows_ok(int64_t M, int64_t N, int64_t K) { return M <= kMaxElems / N && M <= kMaxElems / K; }

bool rank_ok(int r) { return r >= 16 && r <= 256 && r % 16 == 0; }

size_t round_up(size_t v) { return (v + 255) & ~(size_t)255; }

// Workspace carve-up, shared by the size query and the entry points.
struct Carve {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off += round_up(bytes);
    return o;
  }
};

struct FwdLayout {
  size_t At = 0, Bt = 0, u = 0, ulr = 0, down = 0, W = 0, part = 0, total = 0;
  size_t fpart = 0;  // split sums of the tile kernel (fsplit > 1)
  int fsplit = 1;
  bool gemv_path = false, plain = false, fused = false;
  int splits = 1;  // reduction splits of the dense stage (fp32 partials at `part`)
};

// lean: the layout of the lean route (no bf16 copy of the weight); nosplit:
// without the tile kernel's split sums (it then walks all of K).
FwdLayout fwd_layout(int64_t M, int64_t N, int64_t K, int r, bool need_u, bool lean = false,
                     bool nosplit = false) {
  FwdLayout L;
  Carve c;
  L.gemv_path = M <= kGemvMaxM;
  if (L.gemv_path) {
    L.down = c.take((size_t)decode_down_slices(K) * M * r * 4);
  } else {
    L.At = c.take((size_t)r * K * 2);
    L.u = need_u ? c.take((size_t)M * r * 4) : 0;
    L.down = c.take((size_t)lora_down_slices(M, K, r) * M * r * 4);
    L.Bt = c.take((size_t)N * r * 2);
    L.ulr = c.take((size_t)M * 2 * r * 2);
    L.plain = !lean && fwd_plain(M, N, K);
    L.fused = !L.plain && fwd_fused(M, N, K);
    if (L.plain) {
      L.W = c.take((size_t)N * K * 2);
      L.splits = gemm_nt_splits(M, N, K);
      if (L.splits > 1) L.part = c.take((size_t)L.splits * M * N * 4);
    } else if (!L.fused && !nosplit) {
      L.fsplit = gemm_fwd_splits(M, N, K);
      if (L.fsplit > 1) L.fpart = c.take((size_t)L.fsplit * M * N * 4);
    }
  }
  L.total = c.off;
  return L;
}

struct BwdLayout {
  size_t At = 0, down = 0, v = 0, svlr = 0, vT = 0, uT = 0, col = 0, Wt = 0, part = 0, total = 0;
  size_t dxpart = 0;  // split sums of the in-register dX kernel (dxsplit > 1)
  int dxsplit = 1;
  bool plain = false;
  int splits = 1;  // reduction splits of the dense stage for dX
};

// lean: the layout of the lean route (dX through the in-register kernel, no
// bf16 copy of the weight).
BwdLayout bwd_layout(int64_t M, int64_t N, int64_t K, int r, bool need_u, bool lean = false) {
  BwdLayout L;
  Carve c;
  // u is recomputed with the kernels of the forward pass for this M, so that
  // it has the same bits as the u the forward pass returns.
  if (need_u && M > kGemvMaxM) L.At = c.take((size_t)r * K * 2);
  int down_slices = decode_down_slices(K);
  if (lora_down_slices(M, K, r) > down_slices) down_slices = lora_down_slices(M, K, r);
  if (lora_down_slices(M, N, r) > down_slices) down_slices = lora_down_slices(M, N, r);
  L.down = c.take((size_t)down_slices * M * r * 4);
  L.v = c.take((size_t)M * r * 4);
  L.svlr = c.take((size_t)M * 2 * r * 2);
  const size_t Mp = (size_t)((M + 7) & ~(int64_t)7);
  L.vT = c.take(2 * (size_t)r * Mp * 2);
  L.uT = c.take(2 * (size_t)r * Mp * 2);
  L.col = c.take((size_t)colred_splits(M) * (K + N) * r * 4);  // dA's partials, then dB's
  L.plain = !lean && bwd_plain(M, N, K);
  if (L.plain) {
    L.Wt = c.take((size_t)K * N * 2);
    L.splits = gemm_nt_splits(M, K, N);
    if (L.splits > 1) L.part = c.take((size_t)L.splits * M * K * 4);
  } else if (M > 0) {
    L.dxsplit = gemm_bwd_splits(M, N, K);
    if (L.dxsplit > 1) L.dxpart = c.take((size_t)L.dxsplit * M * K * 4);
  }
  L.total = c.off;
  return L;
}

struct MergeLayout {
  size_t At = 0, Bt = 0, total = 0;
};

MergeLayout merge_layout(int64_t N, int64_t K, int r) {
  MergeLayout L;
  Carve c;
  L.At = c.take((size_t)r * K * 2);
  L.Bt = c.take((size_t)N * r * 2);
  L.total = c.off;
  return L;
}

template <typename T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

int launch_status(hipError_t e) { return e == hipSuccess ? QLORA_OK : QLORA_ERR_LAUNCH; }

bool format_ok(int dq_format) {
  return dq_format == QLORA_DQ_INT8 || dq_format == QLORA_DQ_UINT8 || dq_format == QLORA_DQ_E4M3;
}

// Host check of a weight descriptor (the rules of qlora_nf4_check).
int nf4_check(const qlora_nf4* w) {
  if (!w || !w->codes || !w->absmax_q || !w->absmax_scale || w->reserved != 0 ||
      !format_ok(w->dq_format))
    return QLORA_ERR_INVALID_ARG;
  if (!shape_ok(w->N, w->K)) return QLORA_ERR_SHAPE;
  if (!aligned16(w->codes) || !aligned16(w->absmax_q) || !aligned16(w->absmax_scale))
    return QLORA_ERR_ALIGN;
  const uint32_t id = setup_id(w->dq_format);
  if (id == 0) return QLORA_ERR_INTERNAL;
  if (w->format_version != QLORA_FORMAT_VERSION || w->setup_id != id) return QLORA_ERR_SETUP;
  return QLORA_OK;
}

// The codebook as one call's kernels receive it, with that call's
// second-level format. QLORA_ERR_INVALID_ARG for an unknown format.
int call_codebook(int dq_format, Codebook* out) {
  if (!format_ok(dq_format)) return QLORA_ERR_INVALID_ARG;
  const Codebook* cb = nullptr;
  if (get_codebook(&cb, nullptr) != QLORA_OK) return QLORA_ERR_INTERNAL;
  *out = *cb;
  out->dq_format = dq_format;
  return QLORA_OK;
}

// The address a kernel uses for p: device memory as it is; host memory only
// if the runtime has pinned it and mapped it for the device (hipHostMalloc),
// translated to its device-side address; managed memory as it is. Returns
// NULL for anything else (pageable host memory is not reachable).
void* device_view(void* p) {
  hipPointerAttribute_t a{};
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();  // clear the lookup failure; it is not a launch error
    return nullptr;
  }
  if (a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged || a.isManaged)
    return p;
  if (a.type == hipMemoryTypeHost && a.devicePointer && a.hostPointer)
    return static_cast<char*>(a.devicePointer) +
           (static_cast<char*>(p) - static_cast<char*>(a.hostPointer));
  return nullptr;
}

}  // namespace

size_t fwd_workspace_nosplit(int64_t M, int64_t N, int64_t K, int r) {
  if (M < 0 || !shape_ok(N, K) || !rows_ok(M, N, K) || !rank_ok(r)) return 0;
  return fwd_layout(M, N, K, r, true, true, true).total;
}

}  // namespace qlora

using namespace qlora;

extern "C" {

const char* qlora_strerror(int status) {
  switch (status) {
    case QLORA_OK: return "ok";
    case QLORA_ERR_INVALID_ARG: return "invalid argument (NULL pointer, negative size or bad enum)";
    case QLORA_ERR_SHAPE: return "unsupported shape (need N >= 1, K >= 64, K % 64 == 0)";
    case QLORA_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case QLORA_ERR_DTYPE: return "unsupported dtype";
    case QLORA_ERR_RANK: return "unsupported LoRA rank (need 16 <= r <= 256, r % 16 == 0)";
    case QLORA_ERR_WORKSPACE: return "workspace too small";
    case QLORA_ERR_LAUNCH: return "kernel launch failed";
    case QLORA_ERR_INTERNAL: return "codebook self-check failed";
    case QLORA_ERR_TOO_LARGE:
      return "the call needs more workspace than the allocation-free entry point holds";
    case QLORA_ERR_SETUP:
      return "weight descriptor does not match this library's format version or quantization "
             "setup";
    default: return "unknown status";
  }
}

int qlora_nf4_sizes(int64_t N, int64_t K, size_t* codes_bytes, size_t* absmax_q_bytes,
                    size_t* absmax_scale_bytes) {
  if (!shape_ok(N, K)) return QLORA_ERR_SHAPE;
  const int64_t n = N * K, nb = n / kBlock;
  if (codes_bytes) *codes_bytes = (size_t)(n / 2);
  if (absmax_q_bytes) *absmax_q_bytes = (size_t)nb;
  if (absmax_scale_bytes) *absmax_scale_bytes = (size_t)((nb + kGroup - 1) / kGroup) * 4;
  return QLORA_OK;
}

int qlora_codebook(float levels[16], float thresholds[15]) {
  const Codebook* cb = nullptr;
  const int st = get_codebook(&cb, nullptr);
  if (st != QLORA_OK) return st;
  if (levels) std::memcpy(levels, cb->level, sizeof cb->level);
  if (thresholds) std::memcpy(thresholds, cb->thr, sizeof cb->thr);
  return QLORA_OK;
}

int qlora_codebook_quotient_thresholds(float thresholds_q[15]) {
  const Codebook* cb = nullptr;
  const int st = get_codebook(&cb, nullptr);
  if (st != QLORA_OK) return st;
  if (!thresholds_q) return QLORA_ERR_INVALID_ARG;
  std::memcpy(thresholds_q, cb->thr_q, sizeof cb->thr_q);
  return QLORA_OK;
}

uint32_t qlora_codebook_id(void) {
  uint32_t id = 0;
  return get_codebook(nullptr, &id) == QLORA_OK ? id : 0u;
}

uint32_t qlora_setup_id(int dq_format) { return setup_id(dq_format); }

int qlora_nf4_check(const qlora_nf4* w) { return nf4_check(w); }

size_t qlora_workspace_bytes(int op, int64_t M, int64_t N, int64_t K, int r) {
  if (M < 0 || !shape_ok(N, K) || !rows_ok(M, N, K) || !rank_ok(r)) return 0;
  if (op == QLORA_OP_FWD) return fwd_layout(M, N, K, r, true).total;
  if (op == QLORA_OP_FWD_LEAN) return fwd_layout(M, N, K, r, true, true).total;
  if (op == QLORA_OP_BWD) return bwd_layout(M, N, K, r, true).total;
  if (op == QLORA_OP_BWD_LEAN) return bwd_layout(M, N, K, r, true, true).total;
  if (op == QLORA_OP_MERGE) return merge_layout(N, K, r).total;
  return 0;
}

int qlora_quantize_nf4_dq(const void* W, int w_dtype, int64_t N, int64_t K, int dq_format,
                          qlora_nf4* out, void* stream) {
  Codebook cb;
  if (const int st = call_codebook(dq_format, &cb)) return st;
  if (!W || !out || !out->codes || !out->absmax_q || !out->absmax_scale)
    return QLORA_ERR_INVALID_ARG;
  if (!shape_ok(N, K)) return QLORA_ERR_SHAPE;
  if (w_dtype != QLORA_DTYPE_F32 && w_dtype != QLORA_DTYPE_BF16) return QLORA_ERR_DTYPE;
  if (!aligned16(W) || !aligned16(out->codes) || !aligned16(out->absmax_q) ||
      !aligned16(out->absmax_scale))
    return QLORA_ERR_ALIGN;
  const uint32_t id = setup_id(dq_format);
  if (id == 0) return QLORA_ERR_INTERNAL;
  out->N = N;
  out->K = K;
  out->dq_format = dq_format;
  out->format_version = QLORA_FORMAT_VERSION;
  out->setup_id = id;
  out->reserved = 0;
  return launch_status(launch_quantize(W, w_dtype == QLORA_DTYPE_F32, N * K, out->codes,
                                       out->absmax_q, out->absmax_scale, cb,
                                       static_cast<hipStream_t>(stream)));
}

int qlora_dequant_bf16(const qlora_nf4* w, uint16_t* W_out, int layout, void* stream) {
  if (const int st = nf4_check(w)) return st;
  Codebook cb;
  if (const int st = call_codebook(w->dq_format, &cb)) return st;
  if (!W_out) return QLORA_ERR_INVALID_ARG;
  if (layout != QLORA_LAYOUT_ROWS && layout != QLORA_LAYOUT_KSLAB32) return QLORA_ERR_INVALID_ARG;
  const int64_t N = w->N, K = w->K;
  if (layout == QLORA_LAYOUT_KSLAB32 && N * (K / kBlock) >= ((int64_t)1 << 32))
    return QLORA_ERR_SHAPE;
  if (!aligned16(W_out)) return QLORA_ERR_ALIGN;
  return launch_status(launch_dequant(w->codes, w->absmax_q, w->absmax_scale, N * K, W_out,
                                      layout == QLORA_LAYOUT_KSLAB32 ? N : 0, cb,
                                      static_cast<hipStream_t>(stream)));
}

int qlora_linear_fwd(const qlora_nf4* w, const uint16_t* x, int64_t M, const uint16_t* A,
                     const uint16_t* B, int r, float alpha, void* y, int y_dtype, float* u_out,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (const int st = nf4_check(w)) return st;
  Codebook cb;
  if (const int st = call_codebook(w->dq_format, &cb)) return st;
  const int64_t N = w->N, K = w->K;
  const uint8_t* codes = w->codes;
  const int8_t* absmax_q = w->absmax_q;
  const float* absmax_scale = w->absmax_scale;
  if (M < 0) return QLORA_ERR_INVALID_ARG;
  if (!rows_ok(M, N, K)) return QLORA_ERR_SHAPE;
  if (y_dtype != QLORA_DTYPE_F32 && y_dtype != QLORA_DTYPE_BF16) return QLORA_ERR_DTYPE;
  if (!rank_ok(r)) return QLORA_ERR_RANK;
  if (M == 0) return QLORA_OK;
  if (!x || !A || !B || !y) return QLORA_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(A) || !aligned16(B) || !aligned16(y) ||
      (u_out && !aligned16(u_out)) || (workspace && !aligned16(workspace)))
    return QLORA_ERR_ALIGN;
  FwdLayout L = fwd_layout(M, N, K, r, u_out == nullptr);
  if (L.plain && workspace_bytes < L.total) L = fwd_layout(M, N, K, r, u_out == nullptr, true);
  if (L.fsplit > 1 && workspace_bytes < L.total)
    L = fwd_layout(M, N, K, r, u_out == nullptr, true, true);
  if (!workspace || workspace_bytes < L.total) return QLORA_ERR_WORKSPACE;

  hipStream_t st = static_cast<hipStream_t>(stream);
  const float s = alpha / (float)r;
  const bool ybf = y_dtype == QLORA_DTYPE_BF16;
  float* down = at<float>(workspace, L.down);
  hipError_t e = hipSuccess;
  if (L.gemv_path) {
    e = launch_lora_down_decode(x, A, M, K, r, down, st);
    if (e == hipSuccess && decode_tiles_ok(M, N, K, r))
      e = launch_gemv_tiles(x, codes, absmax_q, absmax_scale, down, decode_down_slices(K), B, M, N,
                            K, r, s, u_out, y, ybf, cb, st);
    else if (e == hipSuccess)
      e = launch_gemv(x, codes, absmax_q, absmax_scale, down, decode_down_slices(K), B, M, N, K, r,
                      s, u_out, y, ybf, cb, st);
  } else {
    uint16_t* At = at<uint16_t>(workspace, L.At);
    float* u = u_out ? u_out : at<float>(workspace, L.u);
    uint16_t* Bt = at<uint16_t>(workspace, L.Bt);
    uint16_t* ulr = at<uint16_t>(workspace, L.ulr);
    e = launch_transpose2_bf16(A, K, r, At, B, r, N, Bt, st);  // A^T [r,K], B^T [N,r]
    if (e == hipSuccess && lora_down_full_ok(M, K, r)) {
      e = launch_lora_down_full(x, At, M, K, r, s, u, ulr, nullptr, nullptr, nullptr, st);
    } else {
      if (e == hipSuccess) e = launch_lora_down_parts(x, At, M, K, r, down, st);
      if (e == hipSuccess)
        e = launch_lora_down_finalize(down, lora_down_slices(M, K, r), M, r, s, u, ulr, nullptr,
                                      st);
    }
    if (e == hipSuccess && L.plain) {
      uint16_t* W = at<uint16_t>(workspace, L.W);
      e = launch_dequant(codes, absmax_q, absmax_scale, N * K, W, N, cb, st);  // K-slab
      if (e == hipSuccess)
        e = launch_gemm_nt(x, K, W, 0, ulr, Bt, M, N, K, r, y, ybf, true, st, L.splits,
                           at<float>(workspace, L.part));
    } else if (e == hipSuccess && L.fused) {
      e = launch_gemm_nf4_fwd(x, codes, absmax_q, absmax_scale, ulr, Bt, M, N, K, r, y, ybf, cb,
                              st);
    } else if (e == hipSuccess) {
      e = launch_gemm_fwd(x, codes, absmax_q, absmax_scale, ulr, Bt, M, N, K, r, y, ybf, cb, st,
                          L.fsplit > 1 ? at<float>(workspace, L.fpart) : nullptr);
    }
  }
  return launch_status(e);
}

int qlora_linear_bwd(const qlora_nf4* w, const uint16_t* x, const uint16_t* dY, int64_t M,
                     const uint16_t* A, const uint16_t* B, int r, float alpha,
                     const float* u_saved, void* dX, int dx_dtype, void* dA, void* dB,
                     int grad_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (const int st = nf4_check(w)) return st;
  Codebook cb;
  if (const int st = call_codebook(w->dq_format, &cb)) return st;
  const int64_t N = w->N, K = w->K;
  const uint8_t* codes = w->codes;
  const int8_t* absmax_q = w->absmax_q;
  const float* absmax_scale = w->absmax_scale;
  if (M < 0) return QLORA_ERR_INVALID_ARG;
  if (!rows_ok(M, N, K)) return QLORA_ERR_SHAPE;
  if ((dx_dtype != QLORA_DTYPE_F32 && dx_dtype != QLORA_DTYPE_BF16) ||
      (grad_dtype != QLORA_DTYPE_F32 && grad_dtype != QLORA_DTYPE_BF16))
    return QLORA_ERR_DTYPE;
  if (!rank_ok(r)) return QLORA_ERR_RANK;
  if (!A || !B) return QLORA_ERR_INVALID_ARG;
  if (M > 0 && !dY) return QLORA_ERR_INVALID_ARG;
  if ((dA || dB) && M > 0 && !x) return QLORA_ERR_INVALID_ARG;
  const void* ptrs[] = {x, dY, A, B, u_saved, dX, dA, dB, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return QLORA_ERR_ALIGN;

  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool gbf = grad_dtype == QLORA_DTYPE_BF16;
  const size_t gsz = gbf ? 2 : 4;
  if (M == 0) {  // empty sums: zero adapter gradients, nothing else to do
    hipError_t e = hipSuccess;
    if (dA) e = launch_zero(dA, (size_t)K * r * gsz, st);
    if (e == hipSuccess && dB) e = launch_zero(dB, (size_t)r * N * gsz, st);
    return launch_status(e);
  }
  const bool need_u = dB && !u_saved;
  BwdLayout L = bwd_layout(M, N, K, r, need_u);
  if (L.plain && workspace_bytes < L.total) L = bwd_layout(M, N, K, r, need_u, true);
  if (!workspace || workspace_bytes < L.total) return QLORA_ERR_WORKSPACE;

  const float s = alpha / (float)r;
  float* down = at<float>(workspace, L.down);
  float* v = at<float>(workspace, L.v);
  uint16_t* svlr = at<uint16_t>(workspace, L.svlr);
  uint16_t* vT = at<uint16_t>(workspace, L.vT);
  uint16_t* uT = at<uint16_t>(workspace, L.uT);
  float* col = at<float>(workspace, L.col);
  hipError_t e = hipSuccess;
  // v = dY B^T (B [r,N] is already contiguous along N); the finalize writes
  // the split of s*v both row-major (dX tiles) and transposed (dA). With a
  // saved u, the transposed split of s u for dB shares that launch.
  bool uT_done = false;
  if (lora_down_full_ok(M, N, r)) {
    uT_done = dB && !need_u;
    e = launch_lora_down_full(dY, B, M, N, r, s, v, svlr, dA ? vT : nullptr,
                              uT_done ? u_saved : nullptr, uT_done ? uT : nullptr, st);
  } else {
    e = launch_lora_down_parts(dY, B, M, N, r, down, st);
    uT_done = dB && !need_u;
    if (e == hipSuccess)
      e = launch_lora_down_finalize2(down, lora_down_slices(M, N, r), v, svlr, dA ? vT : nullptr,
                                     uT_done ? u_saved : nullptr, 1, nullptr, nullptr, uT, M, r,
                                     s, st);
  }
  if (e == hipSuccess && dX && L.plain) {  // dX = dY w_hat through w_hat^T [K,N]
    uint16_t* Wt = at<uint16_t>(workspace, L.Wt);
    e = launch_dequant_t(codes, absmax_q, absmax_scale, N, K, Wt, cb, st);  // K-slab
    if (e == hipSuccess)
      e = launch_gemm_nt(dY, N, Wt, 0, svlr, A, M, K, N, r, dX, dx_dtype == QLORA_DTYPE_BF16, true,
                         st, L.splits, at<float>(workspace, L.part));
  } else if (e == hipSuccess && dX) {
    e = launch_gemm_bwd(dY, codes, absmax_q, absmax_scale, svlr, A, M, N, K, r, dX,
                        dx_dtype == QLORA_DTYPE_BF16, cb, st,
                        L.dxsplit > 1 ? at<float>(workspace, L.dxpart) : nullptr);
  }
  // The split of s u first (it depends only on x, A or the saved u), so that
  // both reductions over M, dA = x^T (s v) and dB = (s u)^T dY, run as one
  // launch and one finalize.
  if (e == hipSuccess && dB) {
    if (need_u && M <= kGemvMaxM) {
      e = launch_lora_down_decode(x, A, M, K, r, down, st);
      if (e == hipSuccess)
        e = launch_lora_down_finalize(down, decode_down_slices(K), M, r, s, nullptr, nullptr, uT,
                                      st);
    } else if (need_u) {
      uint16_t* At = at<uint16_t>(workspace, L.At);
      e = launch_transpose_bf16(A, K, r, At, st);
      if (e == hipSuccess && lora_down_full_ok(M, K, r)) {
        e = launch_lora_down_full(x, At, M, K, r, s, nullptr, nullptr, uT, nullptr, nullptr,
                                  st);
      } else {
        if (e == hipSuccess) e = launch_lora_down_parts(x, At, M, K, r, down, st);
        if (e == hipSuccess)
          e = launch_lora_down_finalize(down, lora_down_slices(M, K, r), M, r, s, nullptr, nullptr,
                                        uT,
                                        st);
      }
    } else if (!uT_done) {
      e = launch_lora_down_finalize(u_saved, 1, M, r, s, nullptr, nullptr, uT, st);
    }
  }
  // The route depends on the shape alone, so that dA or dB asked for alone
  // has the bits of the call that asks for both.
  const int cg = colred_direct_cg(M, K, N, r);
  if (e == hipSuccess && (dA || dB) && cg) {
    // One launch writes dA [K, r] and dB [r, N] (transposed) directly.
    e = launch_colred_direct2(dA ? x : dY, dA ? vT : uT, dA ? K : N, dA ? dA : dB, !dA,
                              dA && dB ? dY : nullptr, uT, N, dB, true, M, r, cg, gbf, st);
  } else if (e == hipSuccess && (dA || dB)) {
    // Partial sums: dA's [splits, K, r] at col, dB's [splits, N, r] after it.
    float* colB = col + (size_t)colred_splits(M) * K * r;
    e = launch_colred2(dA ? x : dY, dA ? vT : uT, dA ? K : N, dA ? col : colB,
                       dA && dB ? dY : nullptr, uT, N, colB, M, r, st);
    if (e == hipSuccess)
      e = launch_colred_finalize2(dA ? col : colB, dA ? K : N, !dA, dA ? dA : dB,
                                  dA && dB ? colB : nullptr, N, true, dB, colred_splits(M), r,
                                  1.0f, gbf, st);
  }
  return launch_status(e);
}

int qlora_gemm_bf16_nt(const uint16_t* a, int64_t lda, const uint16_t* b, int64_t ldb,
                       int b_layout, const uint16_t* e, const uint16_t* f, int64_t M, int64_t N,
                       int64_t K, int r, void* y, int y_dtype, void* stream) {
  if (M < 0 || N < 1 || K < 1) return M < 0 ? QLORA_ERR_INVALID_ARG : QLORA_ERR_SHAPE;
  if (N > kMaxElems / K || !rows_ok(M, N, K)) return QLORA_ERR_SHAPE;
  if (b_layout != QLORA_LAYOUT_ROWS && b_layout != QLORA_LAYOUT_KSLAB32) return QLORA_ERR_INVALID_ARG;
  const bool kslab = b_layout == QLORA_LAYOUT_KSLAB32;
  if (lda < K || (!kslab && ldb < K) || !gemm_nt_supported(K, lda, ldb, N, kslab))
    return QLORA_ERR_SHAPE;
  if (y_dtype != QLORA_DTYPE_F32 && y_dtype != QLORA_DTYPE_BF16) return QLORA_ERR_DTYPE;
  if (!rank_ok(r)) return QLORA_ERR_RANK;
  if (M == 0) return QLORA_OK;
  if (!a || !b || !e || !f || !y) return QLORA_ERR_INVALID_ARG;
  if (!aligned16(a) || !aligned16(b) || !aligned16(e) || !aligned16(f) || !aligned16(y))
    return QLORA_ERR_ALIGN;
  return launch_status(launch_gemm_nt(a, lda, b, ldb, e, f, M, N, K, r, y,
                                      y_dtype == QLORA_DTYPE_BF16, kslab,
                                      static_cast<hipStream_t>(stream)));
}

int qlora_merge_lora(const qlora_nf4* w, const uint16_t* W, int64_t N, int64_t K,
                     const uint16_t* A, const uint16_t* B, int r, float alpha, float* merged,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (!W && !w) return QLORA_ERR_INVALID_ARG;
  if (!W)
    if (const int st = nf4_check(w)) return st;
  Codebook cb;
  if (const int st = call_codebook(W ? QLORA_DQ_INT8 : w->dq_format, &cb)) return st;
  if (!shape_ok(N, K)) return QLORA_ERR_SHAPE;
  if (!W && (w->N != N || w->K != K)) return QLORA_ERR_SHAPE;
  if (!rank_ok(r)) return QLORA_ERR_RANK;
  if (!A || !B || !merged) return QLORA_ERR_INVALID_ARG;
  const uint8_t* codes = W ? nullptr : w->codes;
  const int8_t* absmax_q = W ? nullptr : w->absmax_q;
  const float* absmax_scale = W ? nullptr : w->absmax_scale;
  const void* ptrs[] = {W, A, B, merged, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return QLORA_ERR_ALIGN;
  const MergeLayout L = merge_layout(N, K, r);
  if (!workspace || workspace_bytes < L.total) return QLORA_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint16_t* At = at<uint16_t>(workspace, L.At);
  uint16_t* Bt = at<uint16_t>(workspace, L.Bt);
  hipError_t e = launch_transpose2_bf16(A, K, r, At, B, r, N, Bt, st);  // A^T [r,K], B^T [N,r]
  if (e == hipSuccess)
    e = launch_merge(codes, absmax_q, absmax_scale, W, N, K, At, Bt, r,
                     alpha / (float)r, merged, cb, st);
  return launch_status(e);
}

int qlora_adamw_step(float* param, const void* grad, int grad_dtype, float* exp_avg,
                     float* exp_avg_sq, uint16_t* param_bf16, int64_t n, double lr, double beta1,
                     double beta2, double eps, double weight_decay, int64_t step, void* stream) {
  if (n < 0 || step < 1) return QLORA_ERR_INVALID_ARG;
  if (grad_dtype != QLORA_DTYPE_F32 && grad_dtype != QLORA_DTYPE_BF16) return QLORA_ERR_DTYPE;
  if (!(beta1 >= 0.0 && beta1 < 1.0 && beta2 >= 0.0 && beta2 < 1.0)) return QLORA_ERR_INVALID_ARG;
  if (!std::isfinite(lr) || !std::isfinite(eps) || !std::isfinite(weight_decay))
    return QLORA_ERR_INVALID_ARG;
  if (n == 0) return QLORA_OK;
  if (!param || !grad || !exp_avg || !exp_avg_sq) return QLORA_ERR_INVALID_ARG;
  const void* ptrs[] = {param, grad, exp_avg, exp_avg_sq, param_bf16};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return QLORA_ERR_ALIGN;
  void* view[5] = {param, const_cast<void*>(grad), exp_avg, exp_avg_sq, param_bf16};
  for (void*& p : view) {
    if (p && !(p = device_view(p))) return QLORA_ERR_INVALID_ARG;
    if (p && !aligned16(p)) return QLORA_ERR_ALIGN;  // the mapped address, too
  }
  const double b1t = std::pow(beta1, (double)step), b2t = std::pow(beta2, (double)step);
  AdamScalars s;
  s.b1 = (float)beta1;
  s.b2 = (float)beta2;
  s.eps = (float)eps;
  s.decay = (float)(1.0 - lr * weight_decay);
  s.c1 = (float)(1.0 - beta1);
  s.c2 = (float)(1.0 - beta2);
  s.step_size = (float)(lr / (1.0 - b1t));
  s.bc2_sqrt = (float)std::sqrt(1.0 - b2t);
  return launch_status(launch_adamw(static_cast<float*>(view[0]), view[1],
                                    grad_dtype == QLORA_DTYPE_BF16, static_cast<float*>(view[2]),
                                    static_cast<float*>(view[3]), static_cast<uint16_t*>(view[4]),
                                    n, s, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
