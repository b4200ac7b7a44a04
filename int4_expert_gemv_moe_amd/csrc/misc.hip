// misc.hip -- the int4 weight packer (section 06 of the reader.mx article
// "惊呆了！25GB 内存上运行 GLM 5.2 744B 模型") and RMSNorm (section 04).
#include "moe_kernels.h"
#include "norm.h"

namespace moe {

// One wave per row: s = max(amax/7, 1e-8); q = clamp(rint(w/s), -8, 7);
// byte j = (q[2j]+8) | (q[2j+1]+8) << 4.  Division, not a reciprocal, as in the
// article's packer.
__global__ __launch_bounds__(256) void pack_kernel(PackArgs a) {
  const int lane = threadIdx.x & 63;
  const int o = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (o >= a.O) return;
  const float *wr = a.w + (int64_t)o * a.C;
  const int npairs = a.C >> 1;
  const float2 *w2 = reinterpret_cast<const float2 *>(wr);
  float m = 0.f;
  for (int j = lane; j < npairs; j += 64) {
    float2 v = w2[j];
    float t0 = fabsf(v.x), t1 = fabsf(v.y);
    m = (t0 > m) ? t0 : m;
    m = (t1 > m) ? t1 : m;
  }
  m = wave_max_f32(m);
  float s = m / 7.f;
  if (s < 1e-8f) s = 1e-8f;
  uint8_t *qr = a.q4 + (int64_t)o * npairs;
  for (int j = lane; j < npairs; j += 64) {
    float2 v = w2[j];
    float r0 = fminf(fmaxf(rintf(v.x / s), -8.f), 7.f);
    float r1 = fminf(fmaxf(rintf(v.y / s), -8.f), 7.f);
    qr[j] = (uint8_t)(((int)r0 + 8) | (((int)r1 + 8) << 4));
  }
  if (lane == 0) a.scale[o] = s;
}

// One block per row: mean of squares in double, r = 1/sqrtf(ms + eps),
// y = x * r * gamma.  With a.vec (D <= 8192, D % 4 == 0, 16-byte aligned
// rows) each row is read once, all of a thread's loads issued together (the
// row is then in registers); otherwise the plain loop.
__global__ __launch_bounds__(256) void rmsnorm_kernel(RmsArgs a) {
  __shared__ double red[4];
  const int tid = threadIdx.x;
  const float *x = a.x + (int64_t)blockIdx.x * a.D;
  float *y = a.y + (int64_t)blockIdx.x * a.D;
  if (a.vec) {
    NormRow nr;
    norm_row_load(x, a.gamma, a.D, nr);
    norm_row_store(nr, a.D, norm_row_factor(nr, a.D, a.eps, red), y);
    return;
  }
  double ms = 0.0;
  for (int i = tid; i < a.D; i += blockDim.x) ms += (double)x[i] * (double)x[i];
  const double t = block_sum_f64(ms, red);
  const float r = 1.f / sqrtf((float)(t / a.D) + a.eps);
  for (int i = tid; i < a.D; i += blockDim.x) y[i] = x[i] * r * a.gamma[i];
}

hipError_t launch_pack(const PackArgs &a, hipStream_t st) {
  hipLaunchKernelGGL(pack_kernel, dim3((a.O + 3) / 4), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const RmsArgs &a, int S, hipStream_t st) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(S), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
