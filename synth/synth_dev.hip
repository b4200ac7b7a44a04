/*
 * synth_dev.hip -- device fills for the counter-based generator in synth.h.
 * Produces the same bits as the host fills (integer arithmetic plus one
 * correctly rounded float multiply per value).
 */
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "synth.h"

__global__ void synth_fill_normal_kernel(uint64_t key, uint64_t start, uint64_t n, float scale,
                                         float *__restrict__ out) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = synth_normal(key, start + i, scale);
}

extern "C" int synth_dev_fill_normal(uint64_t seed, uint64_t stream, uint64_t start, uint64_t n,
                                     float scale, float *out, hipStream_t st) {
  if (n == 0) return 0;
  if (!out) return -1;
  uint64_t key = synth_key(seed, stream);
  uint64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(synth_fill_normal_kernel, dim3((unsigned)blocks), dim3(256), 0, st, key,
                     start, n, scale, out);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
