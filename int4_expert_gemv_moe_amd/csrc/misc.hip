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

// Read-only streaming reference: every byte of buf read once with 16-byte
// nontemporal loads, 8 lanes per 128-byte segment, four loads in flight per
// thread; one xor word per workgroup keeps the loads live.
constexpr int kStreamBlocks = 4096;

__global__ __launch_bounds__(256) void stream_read_kernel(const uint4 *buf, size_t n16,
                                                          uint32_t *sink) {
  typedef unsigned int u4v __attribute__((ext_vector_type(4)));
  const u4v *p = reinterpret_cast<const u4v *>(buf);
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u4v a = __builtin_nontemporal_load(p + i), b = __builtin_nontemporal_load(p + i + stride),
              c = __builtin_nontemporal_load(p + i + 2 * stride),
              d = __builtin_nontemporal_load(p + i + 3 * stride);
    acc ^= (a.x ^ b.y) + (c.z ^ d.w) + (a.w ^ b.x) + (c.y ^ d.z);
  }
  for (; i < n16; i += stride) {
    const u4v a = __builtin_nontemporal_load(p + i);
    acc ^= a.x + a.y + a.z + a.w;
  }
  __shared__ uint32_t red[4];
  for (int d = 32; d >= 1; d >>= 1) acc ^= __shfl_xor(acc, d, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t st) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(kStreamBlocks), dim3(256), 0, st,
                     reinterpret_cast<const uint4 *>(buf), bytes / 16, sink);
  return hipGetLastError();
}

int stream_read_sink_words() { return kStreamBlocks; }

hipError_t launch_pack(const PackArgs &a, hipStream_t st) {
  hipLaunchKernelGGL(pack_kernel, dim3((a.O + 3) / 4), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const RmsArgs &a, int S, hipStream_t st) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(S), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
