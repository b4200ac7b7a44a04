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

// Lane partner l ^ MASK of every lane, for a value in each lane.
template <int MASK>
__device__ __forceinline__ float xor_lane(float v) {
  if constexpr (MASK == 1) {
    return dpp_f<MOE_DPP_QUAD_X1>(v);
  } else if constexpr (MASK == 2) {
    return dpp_f<MOE_DPP_QUAD_X2>(v);
  } else if constexpr (MASK == 4 || MASK == 8) {
    // lanes with the bit clear read lane + MASK (row shift left), the others
    // lane - MASK (row shift right); the bank masks pick the 4-lane groups
    constexpr int clear = MASK == 4 ? 0x5 : 0x3, set = MASK == 4 ? 0xA : 0xC;
    const int x = __float_as_int(v);
    int r = __builtin_amdgcn_update_dpp(0, x, 0x100 + MASK, 0xF, clear, false);
    r = __builtin_amdgcn_update_dpp(r, x, 0x110 + MASK, 0xF, set, false);
    return __int_as_float(r);
  } else {
    return __shfl_xor(v, MASK);
  }
}

// Wave sums of N values per lane at once.  Step L adds lane l and lane
// l ^ 2^L, as wave_sum_f32 does (its half-row and row mirrors pair the same
// groups of 4 and 8 lanes, whose lanes hold equal bits by then), so every
// sum has wave_sum_f32's bits.  While a lane holds more than one value, step
// L keeps half of them: lanes with bit L set keep the upper half and send
// the lower half to their partner, the others the reverse.  On return v[0]
// of lane l is the sum of value m, m the low log2(N) bits of l reversed.
template <int L, int N>
__device__ __forceinline__ void wave_sum_many(float (&v)[N], int lane) {
  constexpr int MASK = 1 << L, n = N >> L;
  if constexpr (n > 1) {
    const bool up = (lane & MASK) != 0;
#pragma unroll
    for (int k = 0; k < n / 2; k++) {
      const float send = up ? v[k] : v[k + n / 2];
      const float keep = up ? v[k + n / 2] : v[k];
      v[k] = keep + xor_lane<MASK>(send);
    }
  } else {
    v[0] = v[0] + xor_lane<MASK>(v[0]);
  }
  if constexpr (L < 5) wave_sum_many<L + 1, N>(v, lane);
}

// Batches through shared memory: a workgroup of 4 waves over 2TT tokens x
// 2TT experts, each wave a TT x TT register tile of logits (wave w: tokens
// TT (w / 2) .., experts TT (w % 2) ..), with the step's token rows and
// weight rows copied into shared memory once per workgroup
// (global_load_lds_dwordx4 into a ring of stages, steps of 256 columns
// requested ahead) instead of once per wave.  Every logit is lane p's
// ascending FMA chain over k = 4p + 256j + q followed by the additions of
// wave_sum_f32 (all TT x TT at once through wave_sum_many): the same bits as
// router_kernel.
template <bool XB, int TT>
struct RouterShared {
  static constexpr int T = 2 * TT, E = 2 * TT;      // tokens and experts of a workgroup
  static constexpr int XR = XB ? 512 : 1024;        // shared bytes of a token row per step
  static constexpr int XI = T * XR / 1024;          // token-row requests per step
  static constexpr int PIECES = (XI + E) / 4;       // per wave and step
  static constexpr int STAGE = T * XR + E * 1024;   // shared bytes of a stage
  static_assert((XI + E) % 4 == 0, "requests per wave");
};

// NS stages in the ring (NS - 1 steps requested ahead); WPE caps the
// registers so that WPE waves fit on a SIMD.
template <bool XB, int TT, int NS, int WPE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE)))
void router_shared_kernel(RouterArgs a) {
  using R = RouterShared<XB, TT>;
  static_assert(NS >= 2 && NS <= 6 && R::PIECES * (NS - 2) < 16, "ring stages");
  constexpr int SZ = R::STAGE;
  __shared__ __align__(1024) int8_t S0[SZ], S1[SZ], S2[NS > 2 ? SZ : 16], S3[NS > 3 ? SZ : 16],
      S4[NS > 4 ? SZ : 16], S5[NS > 5 ? SZ : 16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int neb = (a.E + R::E - 1) / R::E;
  const int n_router = neb * ((a.S + R::T - 1) / R::T);
  if ((int)blockIdx.x >= n_router) {
    const int s = blockIdx.x - n_router;
    if (a.amax && threadIdx.x < a.P) a.amax[(int64_t)s * a.P + threadIdx.x] = 0u;
    quant_row_block(XB ? nullptr : a.x + (int64_t)s * a.D, XB ? a.xb + (int64_t)s * a.D : nullptr,
                    a.D, a.xq_perm + (int64_t)s * a.D, nullptr, a.sx + s, a.sumx + s);
    return;
  }
  const int eb = (blockIdx.x % neb) * R::E, sb = (blockIdx.x / neb) * R::T;
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
      dst[u] = R::T * R::XR + 1024 * r;
    }
  }
  const int nj = a.D >> 8;
  auto stage = [&](auto bc) __attribute__((always_inline)) {
    constexpr int B = decltype(bc)::value;
    return B == 0 ? S0 : B == 1 ? S1 : B == 2 ? S2 : B == 3 ? S3 : B == 4 ? S4 : S5;
  };
  auto issue = [&](int j, auto bc) __attribute__((always_inline)) {
    const int jj = min(j, nj - 1);
    int8_t *st = stage(bc);
#pragma unroll
    for (int u = 0; u < R::PIECES; u++) dma16(src[u] + (int64_t)jj * step_bytes[u], st + dst[u]);
  };
  const int tg = wave >> 1, eg = wave & 1;
  float acc[TT][TT];
#pragma unroll
  for (int t = 0; t < TT; t++)
#pragma unroll
    for (int e = 0; e < TT; e++) acc[t][e] = 0.f;
  // steps 0 .. NS - 2 requested ahead; step j waits for its own pieces (the
  // NS - 2 later steps stay in flight), then requests step j + NS - 1 into
  // the stage step j - 1 read
  issue(0, std::integral_constant<int, 0>{});
  if constexpr (NS > 2) issue(1, std::integral_constant<int, 1>{});
  if constexpr (NS > 3) issue(2, std::integral_constant<int, 2>{});
  if constexpr (NS > 4) issue(3, std::integral_constant<int, 3>{});
  if constexpr (NS > 5) issue(4, std::integral_constant<int, 4>{});
  auto step = [&](int j, auto bc) __attribute__((always_inline)) {
    constexpr int B = decltype(bc)::value;
    dma_step_barrier<R::PIECES * (NS - 2)>();
    issue(j + NS - 1, std::integral_constant<int, (B + NS - 1) % NS>{});
    const int8_t *st = stage(bc);
    float4 xv[TT], wv[TT];
#pragma unroll
    for (int t = 0; t < TT; t++) {
      const int8_t *row = st + (TT * tg + t) * R::XR;
      if constexpr (XB) {
        const uint2 w = reinterpret_cast<const uint2 *>(row)[lane];
        xv[t] = make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                            __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u));
      } else {
        xv[t] = reinterpret_cast<const float4 *>(row)[lane];
      }
    }
#pragma unroll
    for (int e = 0; e < TT; e++)
      wv[e] = reinterpret_cast<const float4 *>(st + R::T * R::XR + (TT * eg + e) * 1024)[lane];
#pragma unroll
    for (int t = 0; t < TT; t++)
#pragma unroll
      for (int e = 0; e < TT; e++) {
        float c = acc[t][e];
        c = fmaf(xv[t].x, wv[e].x, c);
        c = fmaf(xv[t].y, wv[e].y, c);
        c = fmaf(xv[t].z, wv[e].z, c);
        c = fmaf(xv[t].w, wv[e].w, c);
        acc[t][e] = c;
      }
  };
  // NS steps per turn of the ring, then the rest (fewer than NS)
  auto steps = [&](int j, int n) __attribute__((always_inline)) {
    if (n > 0) step(j, std::integral_constant<int, 0>{});
    if (n > 1) step(j + 1, std::integral_constant<int, 1>{});
    if constexpr (NS > 2) if (n > 2) step(j + 2, std::integral_constant<int, 2 % NS>{});
    if constexpr (NS > 3) if (n > 3) step(j + 3, std::integral_constant<int, 3 % NS>{});
    if constexpr (NS > 4) if (n > 4) step(j + 4, std::integral_constant<int, 4 % NS>{});
    if constexpr (NS > 5) if (n > 5) step(j + 5, std::integral_constant<int, 5 % NS>{});
  };
  int j = 0;
  for (; j + NS <= nj; j += NS) steps(j, NS);
  steps(j, nj - j);
  // the last requests (repeats of the last step) land in stages no step
  // reads; none may still be in flight when the workgroup ends
  wait_vm_at_most<0>();
  const int s0 = sb + TT * tg, e0 = eb + TT * eg;
  // all TT x TT wave sums at once; lane l then holds logit m (token m / TT,
  // expert m % TT of the wave's tile)
  constexpr int N = TT * TT, LOGN = TT == 8 ? 6 : 4;
  float v[N];
#pragma unroll
  for (int t = 0; t < TT; t++)
#pragma unroll
    for (int e = 0; e < TT; e++) v[t * TT + e] = acc[t][e];
  wave_sum_many<0, N>(v, lane);
  const int m = (int)(__builtin_bitreverse32((uint32_t)lane) >> (32 - LOGN));
  const int s = s0 + m / TT, e = e0 + m % TT;
  if (lane < N && s < a.S && e < a.E) {
    a.logits[(int64_t)s * a.E + e] = v[0];
    if (a.logits_out) a.logits_out[(int64_t)s * a.E + e] = v[0];
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
  // in shared memory; more: 16 x 16 tiles staged in shared memory
  const bool xb = a.xb != nullptr;  // bf16 tokens (no RMSNorm with them)
  if (a.S <= 8) {
    const size_t lds = a.gamma ? (size_t)a.D * 4 : 0;  // the normalized row
    if (xb)
      hipLaunchKernelGGL((router_kernel<1, 24, true>), dim3(ne4 * a.S + nq), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((router_kernel<1, 24>), dim3(ne4 * a.S + nq), dim3(256), lds, st, a);
  } else if (a.S < kRouterTileMinTokens) {
    // 8 tokens x 8 experts per workgroup, 4 x 4 logits per wave, three stages
    const dim3 grid(((a.E + 7) / 8) * ((a.S + 7) / 8) + nq);
    if (xb)
      hipLaunchKernelGGL((router_shared_kernel<true, 4, 3, 1>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((router_shared_kernel<false, 4, 3, 1>), grid, dim3(256), 0, st, a);
  } else {
    // 16 tokens x 16 experts per workgroup, 8 x 8 logits per wave, two
    // stages (48 KB with bf16 rows) and at most 168 registers, so three
    // workgroups share a CU (two with float32 rows, 64 KB).  2048 bf16
    // tokens: 136 us, against 147 with one wave sum at a time, 175 with
    // three stages and 189 with 8 x 8 register tiles loaded by every wave
    // for itself
    const dim3 grid(((a.E + 15) / 16) * ((a.S + 15) / 16) + nq);
    if (xb)
      hipLaunchKernelGGL((router_shared_kernel<true, 8, 2, 3>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((router_shared_kernel<false, 8, 2, 3>), grid, dim3(256), 0, st, a);
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
