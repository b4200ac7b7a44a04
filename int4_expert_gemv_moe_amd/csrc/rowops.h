// rowops.h -- device building blocks of the per-token MoE kernels (see
// decode.hip): unconditional 16-byte loads, row splitting, the router dot
// product, the token row held across the lanes of one wave, and the gate/up
// pipeline stages.
#pragma once

#include "moe_common.h"
#include "norm.h"

namespace moe {

typedef unsigned v4u __attribute__((ext_vector_type(4)));

// Unconditional 16-byte nontemporal load of p, or of `safe` when ok is false
// (the result is then replaced by zeros).  Keeping every load unconditional
// leaves the wave's code straight-line, so the compiler can wait for exactly
// the loads a step needs instead of draining all of them at a branch.
__device__ __forceinline__ uint4 ldnt16(const void *p, bool ok, const void *safe) {
  const v4u t = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(ok ? p : safe));
  return ok ? make_uint4(t.x, t.y, t.z, t.w) : make_uint4(0u, 0u, 0u, 0u);
}

__device__ __forceinline__ uint4 ld16(const void *p, bool ok, const void *safe) {
  const uint4 t = *reinterpret_cast<const uint4 *>(ok ? p : safe);
  return ok ? t : make_uint4(0u, 0u, 0u, 0u);
}

// 16 int8 weights in natural column order against 16 activation codes in the
// permuted layout (see moe_common.h): each 8-column group of weights
// w0..w7 is reordered with byte permutes into the words [w0 w2 w4 w6] and
// [w1 w3 w5 w7] that meet the two code words of the group.
__device__ __forceinline__ int dot16_i8p(const uint4 &w, const uint4 &x, int acc) {
  acc = dot4((int)__builtin_amdgcn_perm(w.y, w.x, 0x06040200u), (int)x.x, acc);
  acc = dot4((int)__builtin_amdgcn_perm(w.y, w.x, 0x07050301u), (int)x.y, acc);
  acc = dot4((int)__builtin_amdgcn_perm(w.w, w.z, 0x06040200u), (int)x.z, acc);
  acc = dot4((int)__builtin_amdgcn_perm(w.w, w.z, 0x07050301u), (int)x.w, acc);
  return acc;
}

__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d) {
  return (uint32_t)(a & 0xFF) | ((uint32_t)(b & 0xFF) << 8) | ((uint32_t)(c & 0xFF) << 16) |
         ((uint32_t)(d & 0xFF) << 24);
}

// Rows [r0, r1) of block b when n rows are split over nb blocks.
__device__ __forceinline__ void split_rows(int n, int nb, int b, int &r0, int &r1) {
  r0 = (int)(((int64_t)n * b) / nb);
  r1 = (int)(((int64_t)n * (b + 1)) / nb);
}

// ---- router: one wave computes one logit ----------------------------------------
//
// Same arithmetic as router_kernel (router.hip): lane p accumulates
// fmaf(x[k], W[e][k], acc) for k = 4p + 256j + q, j then q ascending, and the
// lanes are summed by wave_sum_f32.  D % 256 == 0.  Every lane returns the
// logit.
// NORM: x is the raw row and the dot uses its RMSNorm (x * r) * gamma.
template <bool NORM = false>
__device__ inline float router_dot(const float *x, const float *w, int D,
                                   const float *gamma = nullptr, float r = 0.f) {
  const int lane = threadIdx.x & 63;
  constexpr int JB = 24;
  const float4 *wr = reinterpret_cast<const float4 *>(w);
  const float4 *xr = reinterpret_cast<const float4 *>(x);
  const float4 *gr = reinterpret_cast<const float4 *>(gamma);
  const int nj = D >> 8;
  float acc = 0.f;
  for (int j0 = 0; j0 < nj; j0 += JB) {
    float4 wv[JB], xv[JB];
#pragma unroll
    for (int jj = 0; jj < JB; jj++) {
      wv[jj] = make_float4(0.f, 0.f, 0.f, 0.f);
      xv[jj] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (j0 + jj < nj) {
        const uint4 t = ldnt16(wr + lane + 64 * (j0 + jj), true, wr);
        wv[jj] = make_float4(__uint_as_float(t.x), __uint_as_float(t.y), __uint_as_float(t.z),
                             __uint_as_float(t.w));
        xv[jj] = xr[lane + 64 * (j0 + jj)];
        if (NORM) xv[jj] = norm4(xv[jj], gr[lane + 64 * (j0 + jj)], r);
      }
    }
#pragma unroll
    for (int jj = 0; jj < JB; jj++) {
      if (j0 + jj < nj) {
        acc = fmaf(xv[jj].x, wv[jj].x, acc);
        acc = fmaf(xv[jj].y, wv[jj].y, acc);
        acc = fmaf(xv[jj].z, wv[jj].z, acc);
        acc = fmaf(xv[jj].w, wv[jj].w, acc);
      }
    }
  }
  return wave_sum_f32(acc);
}

// ---- token activations in the gate/up lanes ---------------------------------------

// Lane l holds x[2048c + 32l .. +32) for chunk c < NCH.
template <int NCH, bool MASKED>
__device__ __forceinline__ void load_x_f32(const float *x, int D, float4 (&xf)[NCH][8]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int c = 0; c < NCH; c++) {
    const int col = 2048 * c + 32 * lane;
    const bool ok = !MASKED || col < D;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      xf[c][i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (ok) xf[c][i] = reinterpret_cast<const float4 *>(x + col)[i];
    }
  }
}

// The matching 32 permuted codes per chunk from an already quantized row.
template <int NCH, bool MASKED>
__device__ __forceinline__ void load_x_codes(const int8_t *xq, int D, uint4 (&xv)[NCH][2]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int c = 0; c < NCH; c++) {
    const int col = 2048 * c + 32 * lane;
    const bool ok = !MASKED || col < D;
    xv[c][0] = ld16(xq + col, ok, xq);
    xv[c][1] = ld16(xq + col + 16, ok, xq);
  }
}

// Section 12 quantization of the whole row by one wave (its lanes cover the
// row, so the maximum is a wave reduction).  Gives the permuted codes of the
// lane, the scale and the row's code sum; the same bits as quant_row_block.
template <int NCH>
__device__ __forceinline__ int quant_x_wave(const float4 (&xf)[NCH][8], uint4 (&xv)[NCH][2],
                                            float *sx) {
  float m = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; c++)
#pragma unroll
    for (int i = 0; i < 8; i++) {
      m = fmax_nan_skip(m, fabsf(xf[c][i].x));
      m = fmax_nan_skip(m, fabsf(xf[c][i].y));
      m = fmax_nan_skip(m, fabsf(xf[c][i].z));
      m = fmax_nan_skip(m, fabsf(xf[c][i].w));
    }
  m = wave_max_f32(m);
  const float s = quant_scale(m);
  const float inv = 1.f / s;
  int sum = 0;
#pragma unroll
  for (int c = 0; c < NCH; c++) {
    uint32_t w[8];
#pragma unroll
    for (int g = 0; g < 4; g++) {
      const float4 p = xf[c][2 * g], q = xf[c][2 * g + 1];
      const int q0 = quant_code(p.x, inv), q1 = quant_code(p.y, inv), q2 = quant_code(p.z, inv),
                q3 = quant_code(p.w, inv), q4 = quant_code(q.x, inv), q5 = quant_code(q.y, inv),
                q6 = quant_code(q.z, inv), q7 = quant_code(q.w, inv);
      sum += ((q0 + q1) + (q2 + q3)) + ((q4 + q5) + (q6 + q7));
      w[2 * g] = pack4(q0, q2, q4, q6);
      w[2 * g + 1] = pack4(q1, q3, q5, q7);
    }
    xv[c][0] = make_uint4(w[0], w[1], w[2], w[3]);
    xv[c][1] = make_uint4(w[4], w[5], w[6], w[7]);
  }
  *sx = s;
  return wave_sum_i32(sum);
}

// ---- gate/up pipeline stages ------------------------------------------------------
//
// Items are (slot, row) pairs of a concatenated list: item i is row i % I of
// slot i / I.  Res maps a slot to its gate and up matrices and hidden row.

struct GuMats {
  RowPtr G, U;
  float *h;  // hidden row of the slot
};

// One pipeline stage: ROWS gate and up rows of the wave, plus the row scales
// of item (first + lane) for lanes < ROWS (they are only needed after the
// stage's dot products, so they travel with its loads).
template <int NCH, int ROWS>
struct GuStage {
  uint4 g[ROWS][NCH], u[ROWS][NCH];
  float gs, us;
};

template <int NCH, bool MASKED, int ROWS, class Res>
__device__ __forceinline__ void gu_load(Res res, int I, int rowbytes, int item, int hi,
                                        const uint8_t *dummy, GuStage<NCH, ROWS> &st) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int r = 0; r < ROWS; r++) {
    const int it = item + r;
    const bool live = it < hi;  // uniform across the wave
    const int itc = max(min(it, hi - 1), 0);
    const int slot = itc / I;
    const int row = itc - slot * I;
    const GuMats m = res(slot);
    const uint8_t *gr = live ? m.G.q + (int64_t)row * rowbytes : dummy;
    const uint8_t *ur = live ? m.U.q + (int64_t)row * rowbytes : dummy;
#pragma unroll
    for (int c = 0; c < NCH; c++) {
      const int off = c * 1024 + lane * 16;
      const bool ok = !MASKED || off < rowbytes;
      st.g[r][c] = ldnt16(gr + off, ok, gr);
      st.u[r][c] = ldnt16(ur + off, ok, ur);
    }
  }
  const int itc = max(min(item + min(lane, ROWS - 1), hi - 1), 0);
  const int slot = itc / I;
  const int row = itc - slot * I;
  const GuMats m = res(slot);
  st.gs = m.G.s[row];
  st.us = m.U.s[row];
}

// W8: the rows are int8 codes (16 columns per lane and 1 KB chunk, codes
// xv[c][0]; corr is 0); otherwise packed int4 (32 columns, xv[c][0..1]).
template <int NCH, int ROWS, bool W8 = false>
__device__ __forceinline__ void gu_step(const GuStage<NCH, ROWS> &st, const uint4 (&xv)[NCH][2],
                                        int corr, float sxs, int item, int lo, int hi,
                                        float *hout, int *acco) {
  const int lane = threadIdx.x & 63;
  int ag[ROWS], au[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; r++) {
    ag[r] = 0;
    au[r] = 0;
#pragma unroll
    for (int c = 0; c < NCH; c++) {
      if constexpr (W8) {
        ag[r] = dot16_i8p(st.g[r][c], xv[c][0], ag[r]);
        au[r] = dot16_i8p(st.u[r][c], xv[c][0], au[r]);
      } else {
        ag[r] = dot32_i4(st.g[r][c], xv[c][0], xv[c][1], ag[r]);
        au[r] = dot32_i4(st.u[r][c], xv[c][0], xv[c][1], au[r]);
      }
    }
    ag[r] = wave_sum_i32(ag[r]);
    au[r] = wave_sum_i32(au[r]);
  }
  int myg = ag[0], myu = au[0];
#pragma unroll
  for (int r = 1; r < ROWS; r++)
    if (lane == r) {
      myg = ag[r];
      myu = au[r];
    }
  const int it = item + lane;
  if (lane < ROWS && it < hi) {
    const int t = it - lo;
    const int accg = myg - corr, accu = myu - corr;
    const float g = ((float)accg * st.gs) * sxs;
    const float u = ((float)accu * st.us) * sxs;
    hout[t] = silu(g) * u;
    if (acco) {
      acco[2 * t] = accg;
      acco[2 * t + 1] = accu;
    }
  }
}

}  // namespace moe
