// The forward for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid allocation): the
// same launches as qlora_linear_fwd, with the workspace taken from a
// file-scope device array instead of the caller.
//
// Each GPU the library runs on holds its own copy of `scratch` from module
// load until the process ends. Host code never uses the array's name as an
// address (on the host it names a stand-in, not device memory): the device
// address comes from hipGetSymbolAddress, once per device with that device
// current, and is kept per device. Every call on one GPU shares that GPU's
// array: calls that overlap on one GPU (two streams, two threads) race, and
// the caller orders them. The forward's kernels write every workspace region
// before they read it, so nothing needs clearing between calls.
#include <mutex>

#include "../../include/qlora_amd.h"
#include "internal.h"

namespace qlora {
namespace {

static __device__ __align__(256) unsigned char scratch[QLORA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_ptr[kMaxDevices];  // device address of `scratch`, per device ordinal

// Device address of this device's scratch array (NULL on failure).
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace
}  // namespace qlora

extern "C" int qlora_linear_fwd_noalloc(const qlora_nf4* w, const uint16_t* x, int64_t M,
                                        const uint16_t* A, const uint16_t* B, int r,
                                        float alpha, void* y, int y_dtype, float* u_out,
                                        void* stream) {
  if (const int st = qlora_nf4_check(w)) return st;
  if (M < 0) return QLORA_ERR_INVALID_ARG;
  if (M == 0) return QLORA_OK;
  size_t need = qlora_workspace_bytes(QLORA_OP_FWD_LEAN, M, w->N, w->K, r);
  // No size for these arguments: the forward's own checks name the error
  // (they all come before its workspace check, so nothing is enqueued).
  if (need == 0)
    return qlora_linear_fwd(w, x, M, A, B, r, alpha, y, y_dtype, u_out, nullptr, 0, stream);
  // Too large with the tile kernel's split sums: without them (the kernel
  // then walks all of K in each workgroup).
  if (need > QLORA_NOALLOC_SCRATCH_BYTES) need = qlora::fwd_workspace_nosplit(M, w->N, w->K, r);
  if (need > QLORA_NOALLOC_SCRATCH_BYTES) return QLORA_ERR_TOO_LARGE;
  void* ws = qlora::scratch_ptr();
  if (!ws) return QLORA_ERR_LAUNCH;  // the runtime could not give the array's address
  return qlora_linear_fwd(w, x, M, A, B, r, alpha, y, y_dtype, u_out, ws, need, stream);
}
