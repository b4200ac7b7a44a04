// fmt2.hip -- packed int2 weights: the 2-bit path that section 12 of the
// reader.mx article "惊呆了！25GB 内存上运行 GLM 5.2 744B 模型" keeps beside
// int8 and int4 (its summaries list packed int2 with per-row scales).  The
// codes are the section 05 quantizer's at 2 bits (scale = amax, values -1, 0,
// 1); the byte layout carries the int4 container's rule to 2 bits: four codes
// per byte, each stored as code + 2, column 4j + k in bits 2k..2k+1 of byte j.
//
// Dot products: the stored fields u = q + 2 (0..3) are masked out four at a
// time ((w >> 2k) & 0x03030303) and met with the activation codes of the
// same columns by v_dot4; sum (u - 2) x = sum u x - 2 sum x, exact integer
// algebra.  A lane's 16 weight bytes cover 64 consecutive columns; field k of
// the four bytes of weight dword t covers columns 16t + k, +4, +8, +12, so the
// lane's 64 activation codes are transposed in registers (4 x 4 bytes per 16
// columns, v_perm_b32) once per token and reused for every row of the wave.
//
// Launches as for the int8 format: gate/up + SwiGLU, then the per-row
// requantization of h in shared memory + down.
#include "moe_kernels.h"
#include "quant.h"
#include "rowops.h"

namespace moe {

// One wave per row: s = max(amax, 1e-8) (amax / qmax with qmax = 1),
// q = clamp(rint(w/s), -2, 1), packed four per byte.
__global__ __launch_bounds__(256) void pack_int2_kernel(Pack2Args a) {
  const int lane = threadIdx.x & 63;
  const int o = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (o >= a.O) return;
  const float *wr = a.w + (int64_t)o * a.C;
  float m = 0.f;
  for (int j = lane; j < a.C; j += 64) m = fmax_nan_skip(m, fabsf(wr[j]));
  m = wave_max_f32(m);
  float s = m / 1.f;
  if (s < 1e-8f) s = 1e-8f;
  const int rb = (a.C + 3) / 4;
  uint8_t *qr = a.q2 + (int64_t)o * rb;
  for (int j = lane; j < rb; j += 64) {
    unsigned b = 0;
#pragma unroll
    for (int k = 0; k < 4; k++) {
      const int c = 4 * j + k;
      const int v = c < a.C ? (int)fminf(fmaxf(rintf(wr[c] / s), -2.f), 1.f) : 0;
      b |= (unsigned)(v + 2) << (2 * k);
    }
    qr[j] = (uint8_t)b;
  }
  if (lane == 0) a.scale[o] = s;
}

// The 16 activation codes of x0..x3 (columns 4m .. 4m+3 in dword m) regrouped
// so that dword k holds columns k, 4+k, 8+k, 12+k: a 4 x 4 byte transpose.
// __builtin_amdgcn_perm(a, b, sel): selector byte values 0-3 pick b's bytes,
// 4-7 pick a's.
__device__ __forceinline__ void transpose4x4(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3,
                                             uint32_t (&t)[4]) {
  const uint32_t lo01 = __builtin_amdgcn_perm(x1, x0, 0x05010400u);  // x0b0 x1b0 x0b1 x1b1
  const uint32_t hi01 = __builtin_amdgcn_perm(x1, x0, 0x07030602u);  // x0b2 x1b2 x0b3 x1b3
  const uint32_t lo23 = __builtin_amdgcn_perm(x3, x2, 0x05010400u);
  const uint32_t hi23 = __builtin_amdgcn_perm(x3, x2, 0x07030602u);
  t[0] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);  // x0b0 x1b0 x2b0 x3b0
  t[1] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);  // x0b1 x1b1 x2b1 x3b1
  t[2] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
  t[3] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
}

// A lane's 64 activation codes (four uint4, natural order) in dot order:
// xt[t][k] meets field k of weight dword t.
struct X64 {
  uint32_t t[4][4];
};

__device__ __forceinline__ void regroup64(const uint4 (&xv)[4], X64 &x) {
#pragma unroll
  for (int t = 0; t < 4; t++) transpose4x4(xv[t].x, xv[t].y, xv[t].z, xv[t].w, x.t[t]);
}

// sum over 64 columns of u * x (u = stored fields 0..3).
__device__ __forceinline__ int dot64_u2(const uint4 &w, const X64 &x, int acc) {
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int t = 0; t < 4; t++)
#pragma unroll
    for (int k = 0; k < 4; k++)
      acc = dot4((int)((wd[t] >> (2 * k)) & 0x03030303u), (int)x.t[t][k], acc);
  return acc;
}

__device__ __forceinline__ int sum64(const uint4 (&xv)[4]) {
  int s = 0;
#pragma unroll
  for (int t = 0; t < 4; t++) {
    s = dot4((int)xv[t].x, 0x01010101, s);
    s = dot4((int)xv[t].y, 0x01010101, s);
    s = dot4((int)xv[t].z, 0x01010101, s);
    s = dot4((int)xv[t].w, 0x01010101, s);
  }
  return s;
}

// Gate/up: wave w of block b owns row o = 4b + w.  Chunk c of a row is its
// bytes [1024c, 1024c + 1024) = columns [4096c, 4096c + 4096); lane l takes
// bytes 1024c + 16l .. +16.  D % 256 == 0, so a lane's piece is either whole
// or past the row end.
template <int NCH, bool MASKED>
__global__ __launch_bounds__(256) void gu2_kernel(Swiglu2Args a) {
  const int lane = threadIdx.x & 63;
  const int o = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (o >= a.I) return;
  const int rb = a.D >> 2;
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
    int ag = 0, au = 0, sx = 0;
#pragma unroll
    for (int c = 0; c < NCH; c++) {
      const int col = 4096 * c + 64 * lane;
      const bool ok = !MASKED || col < a.D;
      uint4 xv[4];
#pragma unroll
      for (int m = 0; m < 4; m++) xv[m] = ld16(xs + col + 16 * m, ok, xs);
      X64 xt;
      regroup64(xv, xt);
      ag = dot64_u2(g[c], xt, ag);
      au = dot64_u2(u[c], xt, au);
      sx = sum64(xv) + sx;
    }
    sx = wave_sum_i32(sx);
    ag = wave_sum_i32(ag) - 2 * sx;
    au = wave_sum_i32(au) - 2 * sx;
    if (lane == 0) {
      const float sxs = a.sx[s];
      const float gv = ((float)ag * gs) * sxs;
      const float uv = ((float)au * us) * sxs;
      a.h[(int64_t)s * a.I + o] = silu(gv) * uv;
      if (a.acc_gu) {
        a.acc_gu[(int64_t)s * 2 * a.I + o] = ag;
        a.acc_gu[((int64_t)s * 2 + 1) * a.I + o] = au;
      }
    }
  }
}

// Down: wave w of block b owns rows d0 .. d0+R-1, d0 = (4b + w) R; the block
// requantizes h into shared memory first (code sums included), as the int8
// format's down kernel does.  I % 64 == 0 (whole 16-byte pieces).
constexpr int kDn2CodeBytes = 32768;

template <int NCH, bool MASKED, int R>
__global__ __launch_bounds__(256) void dn2_kernel(Swiglu2Args a) {
  __shared__ __align__(16) int8_t codes[kDn2CodeBytes];
  __shared__ float shs[kDn2CodeBytes / 64];  // I >= 64
  __shared__ int sums[kDn2CodeBytes / 64];
  const int lane = threadIdx.x & 63;
  const int d0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * R;
  // no early exit: every wave takes part in the block's barriers
  const int rb = a.I >> 2;
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
  const int TS = kDn2CodeBytes / a.I;
  for (int s0 = 0; s0 < a.S; s0 += TS) {
    const int ns = min(TS, a.S - s0);
    __syncthreads();  // the previous chunk's codes are consumed
    for (int j = 0; j < ns; j++)
      quant_row_block(a.h + (int64_t)(s0 + j) * a.I, nullptr, a.I, nullptr, codes + j * a.I,
                      &shs[j], &sums[j]);
    __syncthreads();  // scales and sums are written by thread 0 after the last barrier
    if (blockIdx.x == 0) {
      if (a.hq_out)
        for (int i = threadIdx.x; i < ns * a.I / 16; i += 256)
          reinterpret_cast<uint4 *>(a.hq_out + (int64_t)s0 * a.I)[i] =
              reinterpret_cast<const uint4 *>(codes)[i];
      if (a.sh_out && (int)threadIdx.x < ns) a.sh_out[s0 + threadIdx.x] = shs[threadIdx.x];
    }
    for (int j = 0; j < ns; j++) {
      const int8_t *hs = codes + j * a.I;
      X64 ht[NCH];
#pragma unroll
      for (int c = 0; c < NCH; c++) {
        const int col = 4096 * c + 64 * lane;
        const bool ok = !MASKED || col < a.I;
        uint4 hv[4];
#pragma unroll
        for (int m = 0; m < 4; m++)
          hv[m] = ok ? *reinterpret_cast<const uint4 *>(hs + col + 16 * m) : make_uint4(0u, 0u, 0u, 0u);
        regroup64(hv, ht[c]);
      }
      const float sh = shs[j];
      const int corr = 2 * sums[j];
      const int64_t s = s0 + j;
#pragma unroll
      for (int r = 0; r < R; r++) {
        int acc = 0;
#pragma unroll
        for (int c = 0; c < NCH; c++) acc = dot64_u2(w[r][c], ht[c], acc);
        acc = wave_sum_i32(acc) - corr;
        if (lane == r && d0 + r < a.D) {
          a.y[s * a.D + d0 + r] = ((float)acc * dsc[r]) * sh;
          if (a.acc_d) a.acc_d[s * a.D + d0 + r] = acc;
        }
      }
    }
  }
}

hipError_t launch_pack_int2(const Pack2Args &a, hipStream_t st) {
  hipLaunchKernelGGL(pack_int2_kernel, dim3((a.O + 3) / 4), dim3(256), 0, st, a);
  return hipGetLastError();
}

// D and I are at most 8192 (checked by the caller): at most two chunks.
hipError_t launch_swiglu2_gateup(const Swiglu2Args &a, hipStream_t st) {
  const dim3 grid((a.I + 3) / 4), block(256);
  const bool masked = a.D % 4096 != 0;
  if (a.D <= 4096) {
    if (masked) hipLaunchKernelGGL((gu2_kernel<1, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((gu2_kernel<1, false>), grid, block, 0, st, a);
  } else {
    if (masked) hipLaunchKernelGGL((gu2_kernel<2, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((gu2_kernel<2, false>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_swiglu2_down(const Swiglu2Args &a, hipStream_t st) {
  constexpr int R = 4;
  const dim3 grid((a.D + 4 * R - 1) / (4 * R)), block(256);
  const bool masked = a.I % 4096 != 0;
  if (a.I <= 4096) {
    if (masked) hipLaunchKernelGGL((dn2_kernel<1, true, R>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((dn2_kernel<1, false, R>), grid, block, 0, st, a);
  } else {
    if (masked) hipLaunchKernelGGL((dn2_kernel<2, true, R>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((dn2_kernel<2, false, R>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace moe
