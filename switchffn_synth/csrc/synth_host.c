/*
 * Host (CPU) filler for the counter-based synthetic input generator.
 * The element definition lives in synth_common.h; this file only loops.
 */
#include <stdint.h>
#include <stddef.h>
#include "synth_common.h"

/* Fill out[0..n) with elements start..start+n-1 of (seed, stream).
 * as_bf16 != 0 writes uint16 bf16 bits, else fp32.  Returns 0, or -1 on bad
 * arguments. */
int synth_fill_host(void* out, int64_t n, int64_t start, uint64_t seed, uint64_t stream,
                    float sigma, int as_bf16, int nthreads) {
  if (!out || n < 0 || start < 0) return -1;
  uint64_t key = synth_key(seed, stream);
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    float v = synth_value(key, (uint64_t)(start + i), sigma);
    if (as_bf16)
      ((uint16_t*)out)[i] = synth_f32_to_bf16(v);
    else
      ((float*)out)[i] = v;
  }
  return 0;
}
