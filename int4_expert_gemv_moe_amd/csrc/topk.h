// topk.h -- the section 11 top-K selection (reader.mx article "惊呆了！25GB
// 内存上运行 GLM 5.2 744B 模型") run by one wave; used by the top-K kernel and
// by the per-token gate/up kernel, so both select identically.
#pragma once

#include <climits>

#include "moe_common.h"

namespace moe {

// Integer key with the order of a non-NaN float (-0 taken as +0 first, so
// that equal choices give equal keys).
__device__ __forceinline__ int topk_key(float c) {
  const int b = __float_as_int(c == 0.f ? 0.f : c);
  return b >= 0 ? b : (b ^ 0x7FFFFFFF);
}

// Runs `rounds` selection rounds of the section 11 rule over E experts held
// MAXM per lane (expert e in lane e % 64, slot e / 64; E <= 64*MAXM).
// Round k picks the largest choice not taken yet, ties to the lowest index;
// candidates need choice > -1e30 (a NaN never qualifies); with no candidate
// left, the lowest untaken index.  Choices become order-preserving integer
// keys (non-candidates the key of -inf; padding past E the lowest key of all,
// index INT_MAX) and each lane sorts its own entries by (key descending,
// index ascending), so a round only compares the 64 list heads: one DPP
// maximum, a ballot of the lanes holding it (a tie between lanes takes an
// integer minimum over their indices), and the winning lane pops its head.
// Lanes 0..rounds-1 then write their round's expert to idx_out / sel_out and
// weight sigmoid(logit) * scale to w_out (each pointer optional; sel_out may
// be shared memory).  Returns the expert of the last round on every lane.
// Adaptive expert top-p over the weights of one token's selection (lane k
// holds the weight of round k, k < K): the smallest k whose running sum, in
// round order, reaches p times the sum of all K (float32, one rounding per
// addition and one product); K when p is not in (0, 1).  Same on every lane.
// (k is uniform, so each weight is read with a lane read into a scalar
// register, a few cycles, rather than a cross-lane permute through LDS.)
__device__ inline int topk_keff(float wk, int K, float p) {
  if (!(p > 0.f && p < 1.f)) return K;
  const int wb = __float_as_int(wk);
  if (K <= 8) {
    // unrolled, constant lanes: the eight reads issue back to back; the sums
    // are the same left-to-right additions over k < K
    float w[8];
#pragma unroll
    for (int k = 0; k < 8; k++) w[k] = __int_as_float(__builtin_amdgcn_readlane(wb, k));
    float total = 0.f;
#pragma unroll
    for (int k = 0; k < 8; k++)
      if (k < K) total = total + w[k];
    const float thr = p * total;
    float run = 0.f;
    int keff = K;
#pragma unroll
    for (int k = 0; k < 8; k++) {
      if (k < K) {
        run = run + w[k];
        if (run >= thr && keff == K) keff = k + 1;
      }
    }
    return keff;
  }
  float total = 0.f;
  for (int k = 0; k < K; k++) total = total + __int_as_float(__builtin_amdgcn_readlane(wb, k));
  const float thr = p * total;
  float run = 0.f;
  for (int k = 0; k < K; k++) {
    run = run + __int_as_float(__builtin_amdgcn_readlane(wb, k));
    if (run >= thr) return k + 1;
  }
  return K;
}

template <int MAXM>
__device__ inline int topk_rounds_m(const float *logits, const float *bias, int E, int rounds,
                                   float scale, int32_t *idx_out, float *w_out, int *sel_out,
                                   float topp = 0.f, int *keff_out = nullptr) {
  constexpr int kNone = static_cast<int>(0x807FFFFF);  // key of -inf
  constexpr int kPad = INT_MIN;
  const int lane = threadIdx.x & 63;
  int v[MAXM], ix[MAXM];
  {
    float lg[MAXM], bs[MAXM];
#pragma unroll
    for (int m = 0; m < MAXM; m++) {
      const int e = min(lane + 64 * m, E - 1);
      lg[m] = logits[e];
      bs[m] = bias[e];
    }
#pragma unroll
    for (int m = 0; m < MAXM; m++) {
      const int e = lane + 64 * m;
      const float c = sigmoid(lg[m]) + bs[m];
      v[m] = e < E ? (c > -1e30f ? topk_key(c) : kNone) : kPad;
      ix[m] = e < E ? e : INT_MAX;
    }
  }
  // odd-even transposition sort of the lane's list (indices ascend with m,
  // so keeping equal keys in place keeps them in index order)
#pragma unroll
  for (int r = 0; r < MAXM; r++) {
#pragma unroll
    for (int m = r & 1; m + 1 < MAXM; m += 2) {
      const bool sw = v[m + 1] > v[m];
      const int tv = v[m], ti = ix[m];
      v[m] = sw ? v[m + 1] : tv;
      ix[m] = sw ? ix[m + 1] : ti;
      v[m + 1] = sw ? tv : v[m + 1];
      ix[m + 1] = sw ? ti : ix[m + 1];
    }
  }
  int mine = 0, sel = 0;
  for (int k = 0; k < rounds; k++) {
    const int mx = wave_max_i32(v[0]);
    const unsigned long long ties = __ballot(v[0] == mx);
    if (__popcll(ties) == 1) {
      sel = lane_i(ix[0], __builtin_ctzll(ties));
    } else {
      // several heads hold the maximum: the lowest index among them
      sel = wave_min_i32(v[0] == mx ? ix[0] : INT_MAX);
    }
    if (lane == k) mine = sel;
    const bool pop = (ix[0] == sel);
#pragma unroll
    for (int m = 0; m + 1 < MAXM; m++) {
      v[m] = pop ? v[m + 1] : v[m];
      ix[m] = pop ? ix[m + 1] : ix[m];
    }
    v[MAXM - 1] = pop ? kPad : v[MAXM - 1];
    ix[MAXM - 1] = pop ? INT_MAX : ix[MAXM - 1];
  }
  const float wk = lane < rounds ? sigmoid(logits[mine]) * scale : 0.f;
  if (lane < rounds) {
    if (sel_out) sel_out[lane] = mine;
    if (idx_out) {
      idx_out[lane] = mine;
      w_out[lane] = wk;
    }
  }
  if (keff_out) {
    const int ke = topk_keff(wk, rounds, topp);
    if (lane == 0) *keff_out = ke;
  }
  return sel;
}

// sel_out (optional, e.g. shared memory) receives every round's expert; the
// caller synchronizes before reading it.
__device__ inline int topk_rounds(const float *logits, const float *bias, int E, int rounds,
                                  float scale, int32_t *idx_out, float *w_out,
                                  int *sel_out = nullptr, float topp = 0.f,
                                  int *keff_out = nullptr) {
  if (E <= 256)
    return topk_rounds_m<4>(logits, bias, E, rounds, scale, idx_out, w_out, sel_out, topp,
                            keff_out);
  return topk_rounds_m<16>(logits, bias, E, rounds, scale, idx_out, w_out, sel_out, topp,
                           keff_out);
}

}  // namespace moe
