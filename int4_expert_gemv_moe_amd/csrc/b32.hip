// b32.hip -- block-32 activation scales: the "Q8_0 style" activation format
// that the summaries of the reader.mx article "惊呆了！25GB 内存上运行 GLM
// 5.2 744B 模型" name (its section 12 listing scales whole rows).  Each run of
// 32 values of a row is quantized like a section 12 row (s = max(amax/127,
// 1e-12), q = rint(x * (1/s))), and an int4 matmul row becomes
// s_w * sum_b acc_b * s_b over its blocks, acc_b the exact int32 sum of
// block b.
//
// The int4 GEMV layout fits the format exactly: a lane's 16-byte piece of a
// packed row is 32 columns, one block.  A lane forms its block's int32 sum
// (nibbles taken as unsigned, minus 8 times the block's code sum), scales it
// by the block's activation scale in float, and the wave adds the lanes'
// floats.  Launches: gate/up + SwiGLU; then per-block requantization of h in
// shared memory + down.
#include "moe_kernels.h"
#include "rowops.h"

namespace moe {

// One thread per block of 32 values.
__global__ __launch_bounds__(256) void quant_b32_kernel(QuantB32Args a) {
  const int64_t blk = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int nb = a.D / 32;
  if (blk >= (int64_t)a.S * nb) return;
  const int64_t s = blk / nb;
  const int64_t off = s * a.D + (blk - s * nb) * 32;
  const float4 *xr = reinterpret_cast<const float4 *>(a.x + off);
  float4 v[8];
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    v[i] = xr[i];
    m = fmax_nan_skip(m, fabsf(v[i].x));
    m = fmax_nan_skip(m, fabsf(v[i].y));
    m = fmax_nan_skip(m, fabsf(v[i].z));
    m = fmax_nan_skip(m, fabsf(v[i].w));
  }
  const float sc = quant_scale(m);
  const float inv = 1.f / sc;
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; i++)
    w[i] = pack4(quant_code(v[i].x, inv), quant_code(v[i].y, inv), quant_code(v[i].z, inv),
                 quant_code(v[i].w, inv));
  uint4 *dst = reinterpret_cast<uint4 *>(a.xq + off);
  dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
  dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  a.sxb[blk] = sc;
}

// 32 natural-order codes (two uint4) regrouped for dot32_i4: per 8 columns
// the even columns, then the odd ones.  __builtin_amdgcn_perm(a, b, sel):
// selector byte values 0-3 pick b's bytes, 4-7 pick a's.
__device__ __forceinline__ void split_even_odd(const uint4 &n0, const uint4 &n1, uint4 &x0,
                                               uint4 &x1) {
  auto ev = [](uint32_t lo, uint32_t hi) { return __builtin_amdgcn_perm(hi, lo, 0x06040200u); };
  auto od = [](uint32_t lo, uint32_t hi) { return __builtin_amdgcn_perm(hi, lo, 0x07050301u); };
  x0 = make_uint4(ev(n0.x, n0.y), od(n0.x, n0.y), ev(n0.z, n0.w), od(n0.z, n0.w));
  x1 = make_uint4(ev(n1.x, n1.y), od(n1.x, n1.y), ev(n1.z, n1.w), od(n1.z, n1.w));
}

__device__ __forceinline__ int sum32(const uint4 &n0, const uint4 &n1) {
  int s = dot4((int)n0.x, 0x01010101, 0);
  s = dot4((int)n0.y, 0x01010101, s);
  s = dot4((int)n0.z, 0x01010101, s);
  s = dot4((int)n0.w, 0x01010101, s);
  s = dot4((int)n1.x, 0x01010101, s);
  s = dot4((int)n1.y, 0x01010101, s);
  s = dot4((int)n1.z, 0x01010101, s);
  return dot4((int)n1.w, 0x01010101, s);
}

// Gate/up: wave w of block b owns row o = 4b + w; chunk c of a row is its
// bytes [1024c, 1024c + 1024) (columns [2048c, 2048c + 2048)); lane l's piece
// is activation block 64c + l.  D % 256 == 0: a piece is whole or past the end.
template <int NCH, bool MASKED>
__global__ __launch_bounds__(256) void gu_b32_kernel(SwigluB32Args a) {
  const int lane = threadIdx.x & 63;
  const int o = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (o >= a.I) return;
  const int rb = a.D >> 1, nb = a.D >> 5;
  const uint8_t *gr = a.G + (int64_t)o * rb;
  const uint8_t *ur = a.U + (int64_t)o * rb;
  uint4 g[NCH], u[NCH];
#pragma unroll
  for (int c = 0; c < NCH; c++) {
    const int off = 1024 * c + 16 * lane;
    const bool ok = !MASKED || off < rb;
    g[c] = ldnt16(gr + off, ok, gr);
    u[c] = ldnt16(ur + off, ok, ur);
  }
  const float gs = a.gs[o], us = a.us[o];
  for (int s = 0; s < a.S; s++) {
    const int8_t *xs = a.xq + (int64_t)s * a.D;
    const float *sb = a.sxb + (int64_t)s * nb;
    float pg = 0.f, pu = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; c++) {
      const int col = 2048 * c + 32 * lane;
      const bool ok = !MASKED || col < a.D;
      const uint4 n0 = ld16(xs + col, ok, xs), n1 = ld16(xs + col + 16, ok, xs);
      const float bs = ok ? sb[64 * c + lane] : 0.f;
      uint4 x0, x1;
      split_even_odd(n0, n1, x0, x1);
      const int corr = 8 * sum32(n0, n1);
      const int ag = dot32_i4(g[c], x0, x1, 0) - corr;
      const int au = dot32_i4(u[c], x0, x1, 0) - corr;
      pg = pg + (float)ag * bs;
      pu = pu + (float)au * bs;
    }
    const float gv = wave_sum_f32(pg) * gs;
    const float uv = wave_sum_f32(pu) * us;
    if (lane == 0) a.h[(int64_t)s * a.I + o] = silu(gv) * uv;
  }
}

// Down: wave w of block b owns rows d0 .. d0+R-1, d0 = (4b + w) R.  For each
// token the block first requantizes h in blocks of 32 into shared memory
// (codes regrouped for dot32_i4, each block's scale and code sum); the weight
// loads are issued before, so their latency overlaps it.  I <= 8192.
constexpr int kB32MaxI = 8192;

template <int NCH, bool MASKED, int R>
__global__ __launch_bounds__(256) void dn_b32_kernel(SwigluB32Args a) {
  __shared__ __align__(16) int8_t codes[kB32MaxI];
  __shared__ float bsc[kB32MaxI / 32];
  __shared__ int bsum[kB32MaxI / 32];
  const int tid = threadIdx.x, lane = tid & 63;
  const int d0 = (blockIdx.x * 4 + (tid >> 6)) * R;
  // no early exit: every wave takes part in the block's barriers
  const int rb = a.I >> 1, nb = a.I >> 5, ngroups = a.I >> 3;
  uint4 w[R][NCH];
  float dsc[R];
#pragma unroll
  for (int r = 0; r < R; r++) {
    const int d = min(d0 + r, a.D - 1);
    const uint8_t *row = a.Dn + (int64_t)d * rb;
#pragma unroll
    for (int c = 0; c < NCH; c++) {
      const int off = 1024 * c + 16 * lane;
      w[r][c] = ldnt16(row + off, !MASKED || off < rb, row);
    }
    dsc[r] = a.ds[d];
  }
  for (int s = 0; s < a.S; s++) {
    __syncthreads();  // the previous token's codes are consumed
    // thread t takes groups of 8 values g = t + 256k; the four groups of a
    // block of 32 sit in one quad of lanes
    const float *hr = a.h + (int64_t)s * a.I;
    for (int g0 = 0; g0 < ngroups; g0 += 256) {
      const int g = g0 + tid;
      const bool ok = g < ngroups;  // ngroups % 4 == 0: quads are all in or all out
      const int gc = ok ? g : 0;
      const float4 p = reinterpret_cast<const float4 *>(hr)[2 * gc];
      const float4 q = reinterpret_cast<const float4 *>(hr)[2 * gc + 1];
      float m = fmax_nan_skip(fmax_nan_skip(fmax_nan_skip(fabsf(p.x), fabsf(p.y)),
                                            fmax_nan_skip(fabsf(p.z), fabsf(p.w))),
                              fmax_nan_skip(fmax_nan_skip(fabsf(q.x), fabsf(q.y)),
                                            fmax_nan_skip(fabsf(q.z), fabsf(q.w))));
      m = fmax_nan_skip(m, dpp_f<MOE_DPP_QUAD_X1>(m));
      m = fmax_nan_skip(m, dpp_f<MOE_DPP_QUAD_X2>(m));
      const float sc = quant_scale(m);
      const float inv = 1.f / sc;
      const int q0 = quant_code(p.x, inv), q1 = quant_code(p.y, inv), q2 = quant_code(p.z, inv),
                q3 = quant_code(p.w, inv), q4 = quant_code(q.x, inv), q5 = quant_code(q.y, inv),
                q6 = quant_code(q.z, inv), q7 = quant_code(q.w, inv);
      int sum = ((q0 + q1) + (q2 + q3)) + ((q4 + q5) + (q6 + q7));
      sum += dpp_i<MOE_DPP_QUAD_X1>(sum);
      sum += dpp_i<MOE_DPP_QUAD_X2>(sum);
      if (ok) {
        reinterpret_cast<uint2 *>(codes)[g] =
            make_uint2(pack4(q0, q2, q4, q6), pack4(q1, q3, q5, q7));
        if ((g & 3) == 0) {
          bsc[g >> 2] = sc;
          bsum[g >> 2] = sum;
        }
        if (blockIdx.x == 0) {
          if (a.hq_out)
            reinterpret_cast<uint2 *>(a.hq_out + (int64_t)s * a.I)[g] =
                make_uint2(pack4(q0, q1, q2, q3), pack4(q4, q5, q6, q7));
          if (a.shb_out && (g & 3) == 0) a.shb_out[(int64_t)s * nb + (g >> 2)] = sc;
        }
      }
    }
    __syncthreads();
    float part[R];
#pragma unroll
    for (int r = 0; r < R; r++) part[r] = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; c++) {
      const int b = 64 * c + lane;
      const bool ok = !MASKED || b < nb;
      const int bc = ok ? b : 0;
      const uint4 x0 = reinterpret_cast<const uint4 *>(codes)[2 * bc];
      const uint4 x1 = reinterpret_cast<const uint4 *>(codes)[2 * bc + 1];
      const float bs = ok ? bsc[bc] : 0.f;
      const int corr = 8 * bsum[bc];
#pragma unroll
      for (int r = 0; r < R; r++) {
        const int acc = dot32_i4(w[r][c], x0, x1, 0) - corr;
        part[r] = part[r] + (float)acc * bs;
      }
    }
#pragma unroll
    for (int r = 0; r < R; r++) {
      const float v = wave_sum_f32(part[r]) * dsc[r];
      if (lane == r && d0 + r < a.D) a.y[(int64_t)s * a.D + d0 + r] = v;
    }
  }
}

hipError_t launch_quant_b32(const QuantB32Args &a, hipStream_t st) {
  const int64_t n = (int64_t)a.S * (a.D / 32);
  hipLaunchKernelGGL(quant_b32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int NCH>
static void launch_gu_b32(const SwigluB32Args &a, hipStream_t st) {
  const dim3 grid((a.I + 3) / 4);
  if (a.D % 2048)
    hipLaunchKernelGGL((gu_b32_kernel<NCH, true>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((gu_b32_kernel<NCH, false>), grid, dim3(256), 0, st, a);
}

// D and I are at most 8192 (checked by the caller): at most 4 chunks.
hipError_t launch_swiglu_b32_gateup(const SwigluB32Args &a, hipStream_t st) {
  switch ((a.D + 2047) / 2048) {
    case 1: launch_gu_b32<1>(a, st); break;
    case 2: launch_gu_b32<2>(a, st); break;
    case 3: launch_gu_b32<3>(a, st); break;
    case 4: launch_gu_b32<4>(a, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int NCH, int R>
static void launch_dn_b32(const SwigluB32Args &a, hipStream_t st) {
  const dim3 grid((a.D + 4 * R - 1) / (4 * R));
  if (a.I % 2048)
    hipLaunchKernelGGL((dn_b32_kernel<NCH, true, R>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((dn_b32_kernel<NCH, false, R>), grid, dim3(256), 0, st, a);
}

hipError_t launch_swiglu_b32_down(const SwigluB32Args &a, hipStream_t st) {
  switch ((a.I + 2047) / 2048) {
    case 1: launch_dn_b32<1, 4>(a, st); break;
    case 2: launch_dn_b32<2, 2>(a, st); break;
    case 3: launch_dn_b32<3, 2>(a, st); break;
    case 4: launch_dn_b32<4, 2>(a, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
