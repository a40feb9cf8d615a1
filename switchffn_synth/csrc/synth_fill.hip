// Device (HIP) filler for the counter-based synthetic input generator: the
// same element definition as the host filler (synth_common.h), evaluated in
// place on the GPU so that multi-GB weight tensors never cross PCIe.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "synth_common.h"

__global__ void __launch_bounds__(256) synth_fill_kernel(void* __restrict__ out, int64_t n,
                                                         int64_t start, uint64_t key, float sigma,
                                                         int as_bf16) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) {
    float v = synth_value(key, (uint64_t)(start + i), sigma);
    if (as_bf16)
      ((uint16_t*)out)[i] = synth_f32_to_bf16(v);
    else
      ((float*)out)[i] = v;
  }
}

extern "C" int synth_fill_device(void* out, int64_t n, int64_t start, uint64_t seed,
                                 uint64_t stream_id, float sigma, int as_bf16, void* stream) {
  if (!out || n < 0 || start < 0) return -1;
  if (n == 0) return 0;
  const uint64_t key = synth_key(seed, stream_id);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(synth_fill_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     (hipStream_t)stream, out, n, start, key, sigma, as_bf16);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? 0 : (int)e;  // the HIP error code (positive)
}

extern "C" const char* synth_error_string(int code) {
  return hipGetErrorString((hipError_t)code);
}
