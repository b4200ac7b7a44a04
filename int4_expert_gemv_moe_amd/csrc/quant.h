// quant.h -- per-row int8 activation quantization by one block of 256
// threads (section 12 of the reader.mx article "惊呆了！25GB 内存上运行 GLM 5.2
// 744B 模型"): s = max(amax/127, 1e-12), q = rint(x * (1/s)).  Shared by the
// quantization kernel and the per-token path so both produce the same codes.
#pragma once

#include "moe_common.h"
#include "norm.h"

namespace moe {

// ---- activation quantization (one block per row) ---------------------------

// gamma (optional, with xf): quantize the RMSNorm (x * r) * gamma of the row.
__device__ inline void quant_row_block(const float *xf, const uint16_t *xb, int D, int8_t *xq_perm,
                                int8_t *xq_nat, float *sx_out, int32_t *sumx_out,
                                const float *gamma = nullptr, float r = 0.f) {
  __shared__ float red_f[16];  // one slot per wave, blocks of up to 1024 threads
  __shared__ int red_i[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ngroups = D >> 3;
  float m = 0.f;
  for (int g = tid; g < ngroups; g += blockDim.x) {
    float v[8];
    if (xf) {
      float4 a = reinterpret_cast<const float4 *>(xf)[2 * g];
      float4 b = reinterpret_cast<const float4 *>(xf)[2 * g + 1];
      if (gamma) {
        a = norm4(a, reinterpret_cast<const float4 *>(gamma)[2 * g], r);
        b = norm4(b, reinterpret_cast<const float4 *>(gamma)[2 * g + 1], r);
      }
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
      uint4 r = reinterpret_cast<const uint4 *>(xb)[g];
      uint32_t wds[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int i = 0; i < 4; i++) {
        v[2 * i] = __uint_as_float(wds[i] << 16);
        v[2 * i + 1] = __uint_as_float(wds[i] & 0xFFFF0000u);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; i++) {
      float a = fabsf(v[i]);
      m = (a > m) ? a : m;
    }
  }
  m = wave_max_f32(m);
  if (lane == 0) red_f[wave] = m;
  __syncthreads();
  float amax = red_f[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); i++) amax = (red_f[i] > amax) ? red_f[i] : amax;
  const float s = quant_scale(amax);
  const float inv = 1.f / s;
  int sum = 0;
  for (int g = tid; g < ngroups; g += blockDim.x) {
    float v[8];
    if (xf) {
      float4 a = reinterpret_cast<const float4 *>(xf)[2 * g];
      float4 b = reinterpret_cast<const float4 *>(xf)[2 * g + 1];
      if (gamma) {
        a = norm4(a, reinterpret_cast<const float4 *>(gamma)[2 * g], r);
        b = norm4(b, reinterpret_cast<const float4 *>(gamma)[2 * g + 1], r);
      }
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
      uint4 r = reinterpret_cast<const uint4 *>(xb)[g];
      uint32_t wds[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int i = 0; i < 4; i++) {
        v[2 * i] = __uint_as_float(wds[i] << 16);
        v[2 * i + 1] = __uint_as_float(wds[i] & 0xFFFF0000u);
      }
    }
    int q[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
      q[i] = quant_code(v[i], inv);
      sum += q[i];
    }
    uint32_t pe = (q[0] & 0xFF) | ((q[2] & 0xFF) << 8) | ((q[4] & 0xFF) << 16) | ((uint32_t)(q[6] & 0xFF) << 24);
    uint32_t po = (q[1] & 0xFF) | ((q[3] & 0xFF) << 8) | ((q[5] & 0xFF) << 16) | ((uint32_t)(q[7] & 0xFF) << 24);
    if (xq_perm) reinterpret_cast<uint2 *>(xq_perm)[g] = make_uint2(pe, po);
    if (xq_nat) {
      uint32_t n0 = (q[0] & 0xFF) | ((q[1] & 0xFF) << 8) | ((q[2] & 0xFF) << 16) | ((uint32_t)(q[3] & 0xFF) << 24);
      uint32_t n1 = (q[4] & 0xFF) | ((q[5] & 0xFF) << 8) | ((q[6] & 0xFF) << 16) | ((uint32_t)(q[7] & 0xFF) << 24);
      reinterpret_cast<uint2 *>(xq_nat)[g] = make_uint2(n0, n1);
    }
  }
  sum = wave_sum_i32(sum);
  if (lane == 0) red_i[wave] = sum;
  __syncthreads();
  if (tid == 0) {
    int t = 0;
    for (int i = 0; i < (int)(blockDim.x >> 6); i++) t += red_i[i];
    if (sx_out) *sx_out = s;
    if (sumx_out) *sumx_out = t;
  }
}

// The same quantization of a row of D <= 8*NT*NCH floats by a block of NT
// threads into shared memory (permuted codes, D bytes at `codes`).  Thread t
// owns groups t + NT*k: quant_row_load issues its loads (so the caller can
// put other loads behind them), quant_row_block_lds does the rest.
// Returns the code sum on every thread; *sx receives the scale.
// NORM: the row is x's RMSNorm (x * r) * gamma.
template <int NCH, int NT = 256, bool NORM = false>
__device__ __forceinline__ void quant_row_load(const float *x, int D, float4 (&v)[NCH][2],
                                               const float *gamma = nullptr, float r = 0.f) {
  const int ngroups = D >> 3;
#pragma unroll
  for (int k = 0; k < NCH; k++) {
    const int g = min((int)threadIdx.x + NT * k, ngroups - 1);
    v[k][0] = reinterpret_cast<const float4 *>(x)[2 * g];
    v[k][1] = reinterpret_cast<const float4 *>(x)[2 * g + 1];
    if (NORM) {
      v[k][0] = norm4(v[k][0], reinterpret_cast<const float4 *>(gamma)[2 * g], r);
      v[k][1] = norm4(v[k][1], reinterpret_cast<const float4 *>(gamma)[2 * g + 1], r);
    }
  }
}

template <int NCH, int NT = 256>
__device__ inline int quant_row_block_lds(const float4 (&v)[NCH][2], int D, int8_t *codes,
                                          float *sx) {
  constexpr int NW = NT / 64;
  __shared__ float red_f[NW];
  __shared__ int red_i[NW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ngroups = D >> 3;
  float m = 0.f;
#pragma unroll
  for (int k = 0; k < NCH; k++) {
    const bool ok = tid + NT * k < ngroups;
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const float4 t = v[k][j];
      float a = fmax_nan_skip(fmax_nan_skip(fabsf(t.x), fabsf(t.y)), fmax_nan_skip(fabsf(t.z), fabsf(t.w)));
      a = ok ? a : 0.f;
      m = fmax_nan_skip(m, a);
    }
  }
  m = wave_max_f32(m);
  if (lane == 0) red_f[wave] = m;
  __syncthreads();
  float amax = red_f[0];
#pragma unroll
  for (int i = 1; i < NW; i++) amax = fmax_nan_skip(amax, red_f[i]);
  const float s = quant_scale(amax);
  const float inv = 1.f / s;
  int sum = 0;
#pragma unroll
  for (int k = 0; k < NCH; k++) {
    const int g = tid + NT * k;
    const float4 a = v[k][0], b = v[k][1];
    const int q0 = quant_code(a.x, inv), q1 = quant_code(a.y, inv), q2 = quant_code(a.z, inv),
              q3 = quant_code(a.w, inv), q4 = quant_code(b.x, inv), q5 = quant_code(b.y, inv),
              q6 = quant_code(b.z, inv), q7 = quant_code(b.w, inv);
    if (g < ngroups) {
      sum += ((q0 + q1) + (q2 + q3)) + ((q4 + q5) + (q6 + q7));
      const uint32_t pe = (q0 & 0xFF) | ((q2 & 0xFF) << 8) | ((q4 & 0xFF) << 16) | ((uint32_t)(q6 & 0xFF) << 24);
      const uint32_t po = (q1 & 0xFF) | ((q3 & 0xFF) << 8) | ((q5 & 0xFF) << 16) | ((uint32_t)(q7 & 0xFF) << 24);
      reinterpret_cast<uint2 *>(codes)[g] = make_uint2(pe, po);
    }
  }
  sum = wave_sum_i32(sum);
  if (lane == 0) red_i[wave] = sum;
  __syncthreads();
  *sx = s;
  int t = 0;
#pragma unroll
  for (int i = 0; i < NW; i++) t += red_i[i];
  return t;
}

}  // namespace moe
