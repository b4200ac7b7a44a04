// router.hip -- sigmoid router, correction-bias top-K and per-row int8
// activation quantization (sections 11 and 12 of the reader.mx article
// "惊呆了！25GB 内存上运行 GLM 5.2 744B 模型").
//
// Logit arithmetic is fixed independently of the launch shape, so a token
// gets the same bits whether it is routed alone or inside a batch: lane p of
// a wave accumulates, with fused multiply-adds in ascending order, the
// products x[k]*W[e][k] for k = 4p + 256j + q (j ascending, q = 0..3); the 64
// lane partials are then summed by the fixed DPP tree of wave_sum_f32.  This
// needs D to be a multiple of 256.
//
// No kernel here communicates between workgroups inside a launch: on this
// chip a device-scope fence writes back and invalidates the issuing XCD's L2,
// which costs about a microsecond per workgroup, so every cross-workgroup
// dependency goes through a kernel boundary instead.
#include "moe_kernels.h"
#include "dma.h"
#include "topk.h"
#include "quant.h"
#include "norm.h"

namespace moe {

// Four consecutive activations of row `row` (element offset 4 i): float32
// rows, or bf16 rows (XB) widened exactly (a bf16 value is the top half of
// its float32), so both give the router the same float operands.
template <bool XB>
__device__ __forceinline__ float4 ldx4(const RouterArgs &a, const float *row, int64_t rowi, int i) {
  if constexpr (XB) {
    const uint2 w = reinterpret_cast<const uint2 *>(a.xb + rowi * a.D)[i];
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                       __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u));
  } else {
    return reinterpret_cast<const float4 *>(row)[i];
  }
}

__global__ __launch_bounds__(256) void quant_kernel(QuantArgs a) {
  const int s = blockIdx.x;
  quant_row_block(a.xf ? a.xf + (int64_t)s * a.D : nullptr,
                  a.xb ? a.xb + (int64_t)s * a.D : nullptr, a.D,
                  a.xq_perm ? a.xq_perm + (int64_t)s * a.D : nullptr,
                  a.xq_nat ? a.xq_nat + (int64_t)s * a.D : nullptr, a.sx ? a.sx + s : nullptr,
                  a.sumx ? a.sumx + s : nullptr);
}

// Natural-order int8 rows -> permuted layout plus the row's code sum.
__global__ __launch_bounds__(256) void prep_xq_kernel(PrepArgs a) {
  __shared__ int red[4];
  const int s = blockIdx.x, tid = threadIdx.x;
  const uint2 *src = reinterpret_cast<const uint2 *>(a.xq + (int64_t)s * a.D);
  uint2 *dst = reinterpret_cast<uint2 *>(a.xq_perm + (int64_t)s * a.D);
  int sum = 0;
  for (int g = tid; g < (a.D >> 3); g += blockDim.x) {
    uint2 v = src[g];
    int q[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      q[i] = (int)(int8_t)((v.x >> (8 * i)) & 0xFF);
      q[4 + i] = (int)(int8_t)((v.y >> (8 * i)) & 0xFF);
    }
#pragma unroll
    for (int i = 0; i < 8; i++) sum += q[i];
    uint32_t pe = (q[0] & 0xFF) | ((q[2] & 0xFF) << 8) | ((q[4] & 0xFF) << 16) | ((uint32_t)(q[6] & 0xFF) << 24);
    uint32_t po = (q[1] & 0xFF) | ((q[3] & 0xFF) << 8) | ((q[5] & 0xFF) << 16) | ((uint32_t)(q[7] & 0xFF) << 24);
    dst[g] = make_uint2(pe, po);
  }
  sum = wave_sum_i32(sum);
  if ((tid & 63) == 0) red[tid >> 6] = sum;
  if (a.amax && tid < a.P) a.amax[(int64_t)s * a.P + tid] = 0u;
  __syncthreads();
  if (tid == 0) a.sumx[s] = red[0] + red[1] + red[2] + red[3];
}

// ---- top-K over one token's logits by one wave -----------------------------

__global__ __launch_bounds__(256) void topk_kernel(TopkArgs a) {
  const int s = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (s >= a.S) return;
  topk_rounds(a.logits + (int64_t)s * a.E, a.bias, a.E, a.K, a.scale, a.idx + (int64_t)s * a.K,
              a.w + (int64_t)s * a.K, nullptr, a.topp, a.keff ? a.keff + s : nullptr);
}

// ---- router logits (+ quantization blocks) -----------------------------------

// Block = 4 waves = 4 experts; TS tokens per block; JB 16-byte loads of the
// expert row per lane issued together.  Blocks with index >= n_router
// quantize token (index - n_router) and clear its amax slots.
// With a.gamma (TS == 1 launches) every workgroup first forms its token's
// RMSNorm row in dynamic shared memory and works on that.
// XB: the tokens are bf16 rows a.xb (no RMSNorm with them).
template <int TS, int JB, bool XB = false>
__global__ __launch_bounds__(256) void router_kernel(RouterArgs a) {
  extern __shared__ __align__(16) float xn_dyn[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ne4 = (a.E + 3) >> 2;
  const int n_router = ne4 * ((a.S + TS - 1) / TS);
  const bool quant = (int)blockIdx.x >= n_router;
  const int e = (blockIdx.x % ne4) * 4 + wave;
  const int s0 = quant ? blockIdx.x - n_router : (blockIdx.x / ne4) * TS;
  const bool normed = !XB && TS == 1 && a.gamma;
  if (normed) {
    NormRow nr;
    norm_row_load(a.x + (int64_t)s0 * a.D, a.gamma, a.D, nr);
    prenorm_finish_lds(nr, a.D, a.eps, xn_dyn);
  }
  // token row s as the block sees it (the normalized row of token s0 when normed)
  auto xrow = [&](int s) { return normed ? (const float *)xn_dyn : a.x + (int64_t)s * a.D; };
  if (quant) {
    const int s = s0;
    if (a.amax && threadIdx.x < a.P) a.amax[(int64_t)s * a.P + threadIdx.x] = 0u;
    quant_row_block(XB ? nullptr : xrow(s), XB ? a.xb + (int64_t)s * a.D : nullptr, a.D,
                    a.xq_perm + (int64_t)s * a.D, nullptr, a.sx + s, a.sumx + s);
    return;
  }
  if (e >= a.E) return;
  float acc[TS];
#pragma unroll
  for (int t = 0; t < TS; t++) acc[t] = 0.f;
  const float4 *wr = reinterpret_cast<const float4 *>(a.W + (int64_t)e * a.D);
  const int nj = a.D >> 8;
  for (int j0 = 0; j0 < nj; j0 += JB) {
    float4 wv[JB];
#pragma unroll
    for (int jj = 0; jj < JB; jj++) {
      wv[jj] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (j0 + jj < nj) wv[jj] = wr[lane + 64 * (j0 + jj)];
    }
#pragma unroll
    for (int t = 0; t < TS; t++) {
      if (s0 + t < a.S) {
        const float *xr = XB ? nullptr : xrow(s0 + t);
        float4 xv[JB];
#pragma unroll
        for (int jj = 0; jj < JB; jj++) {
          xv[jj] = make_float4(0.f, 0.f, 0.f, 0.f);
          if (j0 + jj < nj) xv[jj] = ldx4<XB>(a, xr, s0 + t, lane + 64 * (j0 + jj));
        }
#pragma unroll
        for (int jj = 0; jj < JB; jj++) {
          if (j0 + jj < nj) {
            acc[t] = fmaf(xv[jj].x, wv[jj].x, acc[t]);
            acc[t] = fmaf(xv[jj].y, wv[jj].y, acc[t]);
            acc[t] = fmaf(xv[jj].z, wv[jj].z, acc[t]);
            acc[t] = fmaf(xv[jj].w, wv[jj].w, acc[t]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TS; t++) {
    const float v = wave_sum_f32(acc[t]);
    if (lane == 0 && s0 + t < a.S) {
      a.logits[(int64_t)(s0 + t) * a.E + e] = v;
      if (a.logits_out) a.logits_out[(int64_t)(s0 + t) * a.E + e] = v;
    }
  }
}

// Many tokens: a register tile per wave, TT tokens x EE experts, so each
// loaded x vector serves EE experts and each weight vector TT tokens.  Block
// = TG x 4 waves over TG * TT tokens and 4 * EE consecutive experts.  Every logit
// is still lane p's ascending FMA chain over k = 4p + 256j + q followed by
// wave_sum_f32, i.e. the same bits as router_kernel.  The operands of step
// j + 1 are loaded while step j is multiplied.
template <int TT, int EE, int TG, bool XB = false>
__global__ __launch_bounds__(256 * TG) void router_tile_kernel(RouterArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int neb = (a.E + 4 * EE - 1) / (4 * EE);
  const int n_router = neb * ((a.S + TG * TT - 1) / (TG * TT));
  if ((int)blockIdx.x >= n_router) {
    const int s = blockIdx.x - n_router;
    if (a.amax && threadIdx.x < a.P) a.amax[(int64_t)s * a.P + threadIdx.x] = 0u;
    quant_row_block(XB ? nullptr : a.x + (int64_t)s * a.D, XB ? a.xb + (int64_t)s * a.D : nullptr,
                    a.D, a.xq_perm + (int64_t)s * a.D, nullptr, a.sx + s, a.sumx + s);
    return;
  }
  // TG groups of 4 waves: group g takes tokens s0 + TT g .. +TT, wave w % 4
  // of a group takes experts e0 + EE (w % 4) .. +EE; the groups share each
  // weight vector through the cache
  const int e0 = (blockIdx.x % neb) * 4 * EE + (wave & 3) * EE;
  const int s0 = (blockIdx.x / neb) * TG * TT + (wave >> 2) * TT;
  if (e0 >= a.E || s0 >= a.S) return;
  const float4 *wr[EE];
  int64_t xs[TT];  // token rows (clamped)
#pragma unroll
  for (int t = 0; t < TT; t++) xs[t] = min(s0 + t, a.S - 1);
  const float *xbase = XB ? nullptr : a.x;
#pragma unroll
  for (int e = 0; e < EE; e++)
    wr[e] = reinterpret_cast<const float4 *>(a.W + (int64_t)min(e0 + e, a.E - 1) * a.D) + lane;
  float acc[TT][EE];
#pragma unroll
  for (int t = 0; t < TT; t++)
#pragma unroll
    for (int e = 0; e < EE; e++) acc[t][e] = 0.f;
  const int nj = a.D >> 8;
  float4 xv[TT], wv[EE];
#pragma unroll
  for (int t = 0; t < TT; t++) xv[t] = ldx4<XB>(a, XB ? nullptr : xbase + xs[t] * a.D, xs[t], lane);
#pragma unroll
  for (int e = 0; e < EE; e++) wv[e] = wr[e][0];
  for (int j = 0; j < nj; j++) {
    const int jn = min(j + 1, nj - 1) * 64;
    float4 xn[TT], wn[EE];
#pragma unroll
    for (int t = 0; t < TT; t++)
      xn[t] = ldx4<XB>(a, XB ? nullptr : xbase + xs[t] * a.D, xs[t], lane + jn);
#pragma unroll
    for (int e = 0; e < EE; e++) wn[e] = wr[e][jn];
#pragma unroll
    for (int t = 0; t < TT; t++)
#pragma unroll
      for (int e = 0; e < EE; e++) {
        float c = acc[t][e];
        c = fmaf(xv[t].x, wv[e].x, c);
        c = fmaf(xv[t].y, wv[e].y, c);
        c = fmaf(xv[t].z, wv[e].z, c);
        c = fmaf(xv[t].w, wv[e].w, c);
        acc[t][e] = c;
      }
#pragma unroll
    for (int t = 0; t < TT; t++) xv[t] = xn[t];
#pragma unroll
    for (int e = 0; e < EE; e++) wv[e] = wn[e];
  }
#pragma unroll
  for (int t = 0; t < TT; t++)
#pragma unroll
    for (int e = 0; e < EE; e++) {
      const float v = wave_sum_f32(acc[t][e]);
      if (lane == 0 && s0 + t < a.S && e0 + e < a.E) {
        a.logits[(int64_t)(s0 + t) * a.E + e0 + e] = v;
        if (a.logits_out) a.logits_out[(int64_t)(s0 + t) * a.E + e0 + e] = v;
      }
    }
}

// Mid-size batches: a workgroup of 4 waves over 8 tokens x 8 experts, each
// wave a 4 x 4 register tile of logits (wave w: tokens 4 (w / 2) .., experts
// 4 (w % 2) ..), with the step's 8 token rows and 8 weight rows copied into
// shared memory once per workgroup
// (global_load_lds_dwordx4, a three-stage ring, two steps of 256 columns
// requested ahead) instead of once per wave.  Every logit is lane p's
// ascending FMA chain over k = 4p + 256j + q followed by wave_sum_f32: the
// same bits as router_kernel.
constexpr int kRmT = 8, kRmE = 8;  // tokens and experts of a workgroup

template <bool XB>
struct RouterMid {
  static constexpr int XR = XB ? 512 : 1024;             // shared bytes of a token row per step
  static constexpr int XI = kRmT * XR / 1024;            // token-row requests per step
  static constexpr int PIECES = (XI + kRmE) / 4;         // per wave and step (4, or 3 with bf16)
  static constexpr int STAGE = kRmT * XR + kRmE * 1024;  // shared bytes of a stage
};

template <bool XB>
__global__ __launch_bounds__(256) void router_mid_kernel(RouterArgs a) {
  using R = RouterMid<XB>;
  static_assert((R::XI + kRmE) % 4 == 0, "requests per wave");
  __shared__ __align__(1024) int8_t S0[R::STAGE], S1[R::STAGE], S2[R::STAGE];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int neb = (a.E + kRmE - 1) / kRmE;
  const int n_router = neb * ((a.S + kRmT - 1) / kRmT);
  if ((int)blockIdx.x >= n_router) {
    const int s = blockIdx.x - n_router;
    if (a.amax && threadIdx.x < a.P) a.amax[(int64_t)s * a.P + threadIdx.x] = 0u;
    quant_row_block(XB ? nullptr : a.x + (int64_t)s * a.D, XB ? a.xb + (int64_t)s * a.D : nullptr,
                    a.D, a.xq_perm + (int64_t)s * a.D, nullptr, a.sx + s, a.sumx + s);
    return;
  }
  const int eb = (blockIdx.x % neb) * kRmE, sb = (blockIdx.x / neb) * kRmT;
  // request n = PIECES wave + u of a step: n < XI token rows (XR bytes each,
  // 1024 / XR rows per request), otherwise weight row n - XI; lane l copies
  // bytes 16 (l % (XR / 16)) of its row
  const int8_t *src[R::PIECES];
  int step_bytes[R::PIECES], dst[R::PIECES];
#pragma unroll
  for (int u = 0; u < R::PIECES; u++) {
    const int n = R::PIECES * wave + u;
    if (n < R::XI) {
      const int r = (1024 / R::XR) * n + lane / (R::XR / 16);
      const int srow = min(sb + r, a.S - 1);
      const int8_t *base = XB ? reinterpret_cast<const int8_t *>(a.xb) + (int64_t)srow * a.D * 2
                              : reinterpret_cast<const int8_t *>(a.x) + (int64_t)srow * a.D * 4;
      src[u] = base + 16 * (lane % (R::XR / 16));
      step_bytes[u] = R::XR;
      dst[u] = 1024 * n;
    } else {
      const int r = n - R::XI;
      const int erow = min(eb + r, a.E - 1);
      src[u] = reinterpret_cast<const int8_t *>(a.W) + (int64_t)erow * a.D * 4 + 16 * lane;
      step_bytes[u] = 1024;
      dst[u] = kRmT * R::XR + 1024 * r;
    }
  }
  const int nj = a.D >> 8;
  auto stage = [&](auto bc) __attribute__((always_inline)) {
    constexpr int B = decltype(bc)::value;
    return B == 0 ? S0 : (B == 1 ? S1 : S2);
  };
  auto issue = [&](int j, auto bc) __attribute__((always_inline)) {
    const int jj = min(j, nj - 1);
    int8_t *st = stage(bc);
#pragma unroll
    for (int u = 0; u < R::PIECES; u++) dma16(src[u] + (int64_t)jj * step_bytes[u], st + dst[u]);
  };
  const int tg = wave >> 1, eg = wave & 1;
  float acc[4][4];
#pragma unroll
  for (int t = 0; t < 4; t++)
#pragma unroll
    for (int e = 0; e < 4; e++) acc[t][e] = 0.f;
  issue(0, std::integral_constant<int, 0>{});
  issue(1, std::integral_constant<int, 1>{});
  auto step = [&](int j, auto bc) __attribute__((always_inline)) {
    constexpr int B = decltype(bc)::value;
    dma_step_barrier<R::PIECES>();
    issue(j + 2, std::integral_constant<int, (B + 2) % 3>{});
    const int8_t *st = stage(bc);
    float4 xv[4], wv[4];
#pragma unroll
    for (int t = 0; t < 4; t++) {
      const int8_t *row = st + (4 * tg + t) * R::XR;
      if constexpr (XB) {
        const uint2 w = reinterpret_cast<const uint2 *>(row)[lane];
        xv[t] = make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                            __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u));
      } else {
        xv[t] = reinterpret_cast<const float4 *>(row)[lane];
      }
    }
#pragma unroll
    for (int e = 0; e < 4; e++)
      wv[e] = reinterpret_cast<const float4 *>(st + kRmT * R::XR + (4 * eg + e) * 1024)[lane];
#pragma unroll
    for (int t = 0; t < 4; t++)
#pragma unroll
      for (int e = 0; e < 4; e++) {
        float c = acc[t][e];
        c = fmaf(xv[t].x, wv[e].x, c);
        c = fmaf(xv[t].y, wv[e].y, c);
        c = fmaf(xv[t].z, wv[e].z, c);
        c = fmaf(xv[t].w, wv[e].w, c);
        acc[t][e] = c;
      }
  };
  int j = 0;
  for (; j + 2 < nj; j += 3) {
    step(j, std::integral_constant<int, 0>{});
    step(j + 1, std::integral_constant<int, 1>{});
    step(j + 2, std::integral_constant<int, 2>{});
  }
  if (j < nj) step(j, std::integral_constant<int, 0>{});
  if (j + 1 < nj) step(j + 1, std::integral_constant<int, 1>{});
  // the last requests (repeats of the last step) land in stages no step
  // reads; none may still be in flight when the workgroup ends
  wait_vm_at_most<0>();
  const int s0 = sb + 4 * tg, e0 = eb + 4 * eg;
#pragma unroll
  for (int t = 0; t < 4; t++)
#pragma unroll
    for (int e = 0; e < 4; e++) {
      const float v = wave_sum_f32(acc[t][e]);
      if (lane == 0 && s0 + t < a.S && e0 + e < a.E) {
        a.logits[(int64_t)(s0 + t) * a.E + e0 + e] = v;
        if (a.logits_out) a.logits_out[(int64_t)(s0 + t) * a.E + e0 + e] = v;
      }
    }
}

}  // namespace moe

namespace moe {

hipError_t launch_quant(const QuantArgs &a, int S, hipStream_t st) {
  hipLaunchKernelGGL(quant_kernel, dim3(S), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_router(const RouterArgs &a, bool with_quant, hipStream_t st) {
  const int ne4 = (a.E + 3) / 4;
  const int nq = with_quant ? a.S : 0;
  // a few tokens: one token per wave, the whole weight row in one batch of
  // loads (rows are re-read per token from L2); up to 255: 8 x 8 tiles staged
  // in shared memory; more: 8 x 8 register tiles per wave
  const bool xb = a.xb != nullptr;  // bf16 tokens (no RMSNorm with them)
  if (a.S <= 8) {
    const size_t lds = a.gamma ? (size_t)a.D * 4 : 0;  // the normalized row
    if (xb)
      hipLaunchKernelGGL((router_kernel<1, 24, true>), dim3(ne4 * a.S + nq), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((router_kernel<1, 24>), dim3(ne4 * a.S + nq), dim3(256), lds, st, a);
  } else if (a.S < kRouterTileMinTokens) {
    // 8 tokens x 8 experts per workgroup through shared memory (against the
    // 4 x 4 register tiles of router_tile_kernel, 4 tokens x 16 experts per
    // workgroup: 14.0 against 20.5 us at 64 tokens)
    const dim3 grid(((a.E + kRmE - 1) / kRmE) * ((a.S + kRmT - 1) / kRmT) + nq);
    if (xb)
      hipLaunchKernelGGL((router_mid_kernel<true>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((router_mid_kernel<false>), grid, dim3(256), 0, st, a);
  } else {
    // 4-wave workgroups of 8 tokens x 32 experts (swept against 8-wave
    // workgroups of 16 x 32 and other tiles: 188 against 209 us at 2048 tokens)
    const int neb = (a.E + 31) / 32;
    const dim3 grid(neb * ((a.S + 7) / 8) + nq);
    if (xb)
      hipLaunchKernelGGL((router_tile_kernel<8, 8, 1, true>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((router_tile_kernel<8, 8, 1>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_prep_xq(const PrepArgs &a, int S, hipStream_t st) {
  hipLaunchKernelGGL(prep_xq_kernel, dim3(S), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs &a, hipStream_t st) {
  hipLaunchKernelGGL(topk_kernel, dim3((a.S + 3) / 4), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
