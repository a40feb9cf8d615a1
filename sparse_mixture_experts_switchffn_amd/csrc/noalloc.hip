// The allocation-free forward: switch_ffn_forward with its workspace in a
// file-scope device array, for callers that cannot allocate device memory
// (code under stream capture, tight serving loops, harnesses that forbid
// allocation).  Nothing here allocates: the array is part of the library's
// code object, and each GPU the library runs on holds its own copy from the
// first use until the process ends.
#include <mutex>

#include "sffn_internal.h"
#include "../../include/switch_ffn.h"

namespace {

constexpr size_t kScratchBytes = (size_t)SFFN_NOALLOC_SCRATCH_MIB << 20;
constexpr int kMaxDevices = 64;

// The workspace of every allocation-free call on one GPU.  In host code this
// name stands for the host-side shadow, not a device address: kernels get the
// device address that hipGetSymbolAddress returns for the current device.
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up

// Device address of this device's `scratch` (looked up once per device, with
// that device current).  Returns a HIP error code.
hipError_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

size_t switch_ffn_noalloc_scratch_bytes(void) { return kScratchBytes; }

int switch_ffn_forward_noalloc(const void* x, const float* Wr, const void* W1, const void* b1,
                               const void* W2, const void* b2, int64_t T, int64_t d, int64_t F,
                               int64_t N, double CF, int dtype, void* y, int32_t* expert_idx,
                               int32_t* slot, float* gate, float* aux_loss, void* stream) {
  // Every argument check of the forward but the workspace's, before any device
  // call: without a workspace the forward returns SFFN_EWORKSPACE exactly when
  // all its other checks pass (it checks the workspace last and enqueues
  // nothing on an error).
  const int rc = switch_ffn_forward(x, Wr, W1, b1, W2, b2, T, d, F, N, CF, dtype, y, expert_idx,
                                    slot, gate, aux_loss, nullptr, 0, stream);
  if (rc != SFFN_EWORKSPACE) return rc;
  if (switch_ffn_workspace_bytes(T, d, F, N, CF, dtype) > kScratchBytes) return SFFN_ESCRATCH;
  void* ws = nullptr;
  const hipError_t e = scratch_ptr(&ws);
  if (e != hipSuccess) return sffn::record_hip_error(e, "scratch address lookup");
  return switch_ffn_forward(x, Wr, W1, b1, W2, b2, T, d, F, N, CF, dtype, y, expert_idx, slot,
                            gate, aux_loss, ws, kScratchBytes, stream);
}

}  // extern "C"
