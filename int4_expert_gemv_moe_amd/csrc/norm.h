// norm.h -- RMSNorm (section 04 of the reader.mx article "惊呆了！25GB 内存上运行
// GLM 5.2 744B 模型") as pieces that other kernels can run in front of their
// own work: the row's factor r = 1 / sqrt(mean(x^2) + eps) with the squares
// summed in double in one fixed order, and the element rule (x * r) * gamma.
// moe_rmsnorm's kernel and the fused callers use the same functions, so a
// normalized row has the same bits wherever it is formed.
#pragma once

#include "moe_common.h"

namespace moe {

// Block sum of one double per thread (256 threads): a shuffle tree per wave,
// then the four wave sums as (w0 + w1) + (w2 + w3).  red: 4 doubles of LDS.
__device__ __forceinline__ double block_sum_f64(double v, double *red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  const double t = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();  // red may be reused right after
  return t;
}

// Rows that the vector form takes: D % 4 == 0, D <= 8192 (8 float4 per
// thread of a 256-thread block), 16-byte aligned rows.
inline bool rms_vec_ok(int D, const void *x, const void *gamma) {
  return D % 4 == 0 && D <= 8192 && ((uintptr_t)x % 16) == 0 && ((uintptr_t)gamma % 16) == 0;
}

// One row in the registers of a 256-thread block: thread t holds float4s
// t, t + 256, ... (up to 8) of x and of gamma.  norm_row_load only issues
// the loads, so that a caller can put other loads behind them.
struct NormRow {
  float4 xv[8], gv[8];
};

__device__ __forceinline__ void norm_row_load(const float *x, const float *gamma, int D,
                                              NormRow &nr) {
  const int n4 = D / 4;
#pragma unroll
  for (int k = 0; k < 8; k++) {
    const int i = min((int)threadIdx.x + 256 * k, n4 - 1);
    nr.xv[k] = reinterpret_cast<const float4 *>(x)[i];
    nr.gv[k] = reinterpret_cast<const float4 *>(gamma)[i];
  }
}

// The factor r = 1 / sqrt(mean(x^2) + eps) of the loaded row, on every
// thread.  Thread t sums the squares of its float4s in order (components
// x, y, z, w), then block_sum_f64.
__device__ inline float norm_row_factor(const NormRow &nr, int D, float eps, double *red) {
  const int n4 = D / 4;
  double ms = 0.0;
#pragma unroll
  for (int k = 0; k < 8; k++) {
    if ((int)threadIdx.x + 256 * k < n4) {
      ms += (double)nr.xv[k].x * (double)nr.xv[k].x;
      ms += (double)nr.xv[k].y * (double)nr.xv[k].y;
      ms += (double)nr.xv[k].z * (double)nr.xv[k].z;
      ms += (double)nr.xv[k].w * (double)nr.xv[k].w;
    }
  }
  const double t = block_sum_f64(ms, red);
  return 1.f / sqrtf((float)(t / D) + eps);
}

__device__ __forceinline__ float4 norm4(float4 x, float4 g, float r) {
  return make_float4(x.x * r * g.x, x.y * r * g.y, x.z * r * g.z, x.w * r * g.w);
}

// The normalized row (x * r) * gamma to dst (global or shared memory).
__device__ __forceinline__ void norm_row_store(const NormRow &nr, int D, float r, float *dst) {
  const int n4 = D / 4;
#pragma unroll
  for (int k = 0; k < 8; k++) {
    const int i = threadIdx.x + 256 * k;
    if (i < n4) reinterpret_cast<float4 *>(dst)[i] = norm4(nr.xv[k], nr.gv[k], r);
  }
}

// Loaded row -> RMSNorm row in shared memory dst (D floats, 16-byte
// aligned), complete for every thread on return.
__device__ inline void prenorm_finish_lds(const NormRow &nr, int D, float eps, float *dst) {
  __shared__ double red[4];
  norm_row_store(nr, D, norm_row_factor(nr, D, eps, red), dst);
  __syncthreads();
}

}  // namespace moe
