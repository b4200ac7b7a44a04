// moe_common.h -- device helpers and argument structs shared by the gfx950
// kernels of the int4 MoE block.
//
// Activation layout used by the integer kernels ("permuted int8 rows"): every
// group of 8 consecutive values x0..x7 is stored as x0 x2 x4 x6 x1 x3 x5 x7.
// A 32-bit word of packed int4 weights holds columns 8m..8m+7, even columns in
// the low nibbles; masking the low nibbles gives the four even columns and
// shifting by 4 gives the four odd ones, so each half meets one 32-bit word of
// permuted activations in a 4-way int8 dot product.  The nibbles are used as
// the unsigned values q+8 (0..15); the -8 offset is removed afterwards as
// acc - 8 * sum(x), which is exact in int32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_i4.h"

#define MOE_WAVE 64

namespace moe {

__device__ __forceinline__ int dot4(int a, int b, int c) {
  return __builtin_amdgcn_sdot4(a, b, c, false);
}

// 8 int4 columns (one packed word) against 8 permuted int8 activations.
__device__ __forceinline__ int dot8_i4(uint32_t w, int xe, int xo, int acc) {
  acc = dot4((int)(w & 0x0F0F0F0Fu), xe, acc);
  acc = dot4((int)((w >> 4) & 0x0F0F0F0Fu), xo, acc);
  return acc;
}

// 32 int4 columns held in one uint4 against 32 permuted activations (two uint4).
__device__ __forceinline__ int dot32_i4(const uint4 &w, const uint4 &x0, const uint4 &x1, int acc) {
  acc = dot8_i4(w.x, (int)x0.x, (int)x0.y, acc);
  acc = dot8_i4(w.y, (int)x0.z, (int)x0.w, acc);
  acc = dot8_i4(w.z, (int)x1.x, (int)x1.y, acc);
  acc = dot8_i4(w.w, (int)x1.z, (int)x1.w, acc);
  return acc;
}

// 16-byte load, or zeros when ok is false (the address is not touched then).
__device__ __forceinline__ uint4 load16(const void *p, bool ok) {
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (ok) v = *reinterpret_cast<const uint4 *>(p);
  return v;
}

// Cross-lane steps inside a 16-lane row use DPP: quad permutations [1,0,3,2]
// and [2,3,0,1], then the half-row mirror (lane i <-> 7-i) and the row mirror
// (i <-> 15-i).  After the four steps every lane of a row holds the row's
// value; the four rows are then read with readlane and combined as
// (row0 + row1) + (row2 + row3).  Every lane ends with the same result, and
// the order of operations is fixed, so float sums are reproducible.
#define MOE_DPP_QUAD_X1 0xB1
#define MOE_DPP_QUAD_X2 0x4E
#define MOE_DPP_HALF_MIRROR 0x141
#define MOE_DPP_ROW_MIRROR 0x140

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ int lane_i(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

__device__ __forceinline__ int wave_sum_i32(int v) {
  v += dpp_i<MOE_DPP_QUAD_X1>(v);
  v += dpp_i<MOE_DPP_QUAD_X2>(v);
  v += dpp_i<MOE_DPP_HALF_MIRROR>(v);
  v += dpp_i<MOE_DPP_ROW_MIRROR>(v);
  return (lane_i(v, 0) + lane_i(v, 16)) + (lane_i(v, 32) + lane_i(v, 48));
}

__device__ __forceinline__ float wave_sum_f32(float v) {
  v = v + dpp_f<MOE_DPP_QUAD_X1>(v);
  v = v + dpp_f<MOE_DPP_QUAD_X2>(v);
  v = v + dpp_f<MOE_DPP_HALF_MIRROR>(v);
  v = v + dpp_f<MOE_DPP_ROW_MIRROR>(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}

__device__ __forceinline__ float fmax_nan_skip(float a, float b) { return (b > a) ? b : a; }

// Maximum that ignores NaN (a NaN never compares greater); same on all lanes.
__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmax_nan_skip(v, dpp_f<MOE_DPP_QUAD_X1>(v));
  v = fmax_nan_skip(v, dpp_f<MOE_DPP_QUAD_X2>(v));
  v = fmax_nan_skip(v, dpp_f<MOE_DPP_HALF_MIRROR>(v));
  v = fmax_nan_skip(v, dpp_f<MOE_DPP_ROW_MIRROR>(v));
  return fmax_nan_skip(fmax_nan_skip(lane_f(v, 0), lane_f(v, 16)),
                       fmax_nan_skip(lane_f(v, 32), lane_f(v, 48)));
}

// Wave-wide maximum of an int32 through DPP only: the row steps above, then
// the two GFX9 row broadcasts (lane 15 of each row into the next row, lane 31
// into rows 2 and 3), after which lane 63 holds the maximum.
#define MOE_DPP_ROW_BCAST15 0x142
#define MOE_DPP_ROW_BCAST31 0x143
__device__ __forceinline__ int wave_max_i32(int v) {
  v = max(v, dpp_i<MOE_DPP_QUAD_X1>(v));
  v = max(v, dpp_i<MOE_DPP_QUAD_X2>(v));
  v = max(v, dpp_i<MOE_DPP_HALF_MIRROR>(v));
  v = max(v, dpp_i<MOE_DPP_ROW_MIRROR>(v));
  v = max(v, __builtin_amdgcn_update_dpp(v, v, MOE_DPP_ROW_BCAST15, 0xA, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(v, v, MOE_DPP_ROW_BCAST31, 0xC, 0xF, false));
  return lane_i(v, 63);
}

// Minimum over the wave, same on every lane.
__device__ __forceinline__ int wave_min_i32(int v) {
  v = min(v, dpp_i<MOE_DPP_QUAD_X1>(v));
  v = min(v, dpp_i<MOE_DPP_QUAD_X2>(v));
  v = min(v, dpp_i<MOE_DPP_HALF_MIRROR>(v));
  v = min(v, dpp_i<MOE_DPP_ROW_MIRROR>(v));
  return min(min(lane_i(v, 0), lane_i(v, 16)), min(lane_i(v, 32), lane_i(v, 48)));
}

// Position of value j (0 <= j < 8) of an 8-group in the permuted layout.
__device__ __host__ __forceinline__ int perm8(int j) { return (j & 1) ? 4 + (j >> 1) : (j >> 1); }

__device__ __forceinline__ float silu(float g) { return g / (1.f + expf(-g)); }

__device__ __forceinline__ float sigmoid(float v) { return 1.f / (1.f + expf(-v)); }

// Per-row int8 quantization scale from the row's max |x| (section 12).
__device__ __forceinline__ float quant_scale(float amax) {
  float s = amax / 127.f;
  return (s < 1e-12f) ? 1e-12f : s;
}

__device__ __forceinline__ int quant_code(float x, float inv) {
  float r = rintf(x * inv);
  r = fminf(fmaxf(r, -127.f), 127.f);
  return (int)r;
}

// Device view of one stacked int4 matrix.
struct QMat {
  const uint8_t *q4;
  const float *scale;
  int64_t q4_stride;  // bytes between experts
  int64_t s_stride;   // floats between experts
  __device__ __forceinline__ const uint8_t *rows(int e) const { return q4 + (int64_t)e * q4_stride; }
  __device__ __forceinline__ const float *scales(int e) const { return scale + (int64_t)e * s_stride; }
};

struct ExpertSet {
  QMat gate, up, down;
};

// Rows and scales of one expert's matrix, chosen field by field between two
// stacks (choosing whole structs by a runtime condition would make the
// compiler copy them to private memory).
struct RowPtr {
  const uint8_t *q;
  const float *s;
};

__device__ __forceinline__ RowPtr pick(const QMat &a, const QMat &b, bool use_b, int e) {
  const uint8_t *q = use_b ? b.q4 : a.q4;
  const int64_t qs = use_b ? b.q4_stride : a.q4_stride;
  const float *sc = use_b ? b.scale : a.scale;
  const int64_t ss = use_b ? b.s_stride : a.s_stride;
  return RowPtr{q + (int64_t)e * qs, sc + (int64_t)e * ss};
}

// Scratch buffers carved out of the caller's workspace.
struct Work {
  int8_t *xq;       // [S][D] permuted activations
  float *sx;        // [S]
  int32_t *sumx;    // [S]
  float *logits;    // [S][E]
  int32_t *idx;     // [S][K]
  float *w;         // [S][K]
  int32_t *keff;    // [S] experts kept per token
  float *h;         // [S][P][I]
  int8_t *hq;       // [S][P][I] permuted
  float *sh;        // [S][P]
  int32_t *sumh;    // [S][P]
  float *ysh;       // [S][D] shared-expert output
  float *tmp;       // [S][D] running combine
  int32_t *gcount;  // [E+1] tokens per group (batch path)
  int32_t *gfill;   // [E+1]
  int32_t *goff;    // [E+2]
  int32_t *pairs;   // [S*P] (s*P + slot) grouped by expert
  float *stage;     // [S][P][D]
  int2 *tiles;      // MFMA tiles of the grouped pairs
  int32_t *ntiles;
  float *xn;        // [S][D] normalized rows (batch path with MOE_F_PRENORM)
};

}  // namespace moe
