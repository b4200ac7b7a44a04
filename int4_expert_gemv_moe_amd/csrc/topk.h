// topk.h -- the section 11 top-K selection (reader.mx article "惊呆了！25GB
// 内存上运行 GLM 5.2 744B 模型") run by one wave; used by the top-K kernel and
// by the per-token gate/up kernel, so both select identically.
#pragma once

#include "moe_common.h"

namespace moe {

// Runs `rounds` selection rounds of the section 11 rule over E experts held
// MAXM per lane (expert e in lane e % 64, slot e / 64; E <= 64*MAXM).
// Round k picks the largest choice not taken yet, ties to the lowest index;
// candidates need choice > -1e30 (a NaN never qualifies); with no candidate
// left, the lowest untaken index.  Each round is one wave-wide float maximum
// (DPP) followed by ballots that find the lowest index holding that maximum,
// so the whole selection is branch-free except for the uniform fallback.
// If idx_out is given, lane 0 writes every round's expert and weight;
// sel_out (e.g. shared memory) receives every round's expert.  Returns the
// expert of the last round on every lane.
template <int MAXM, bool CACHE>
__device__ inline int topk_rounds_m(const float *logits, const float *bias, int E, int rounds,
                                   float scale, int32_t *idx_out, float *w_out, int *sel_out) {
  const int lane = threadIdx.x & 63;
  const int nm = (E + 63) >> 6;
  // choice values (-inf when not a candidate); held in registers when CACHE,
  // else recomputed each round from the same expression (same bits)
  float c[CACHE ? MAXM : 1];
  if (CACHE) {
    float lg[CACHE ? MAXM : 1], bs[CACHE ? MAXM : 1];
#pragma unroll
    for (int m = 0; m < MAXM; m++) {
      const int e = min(lane + 64 * m, E - 1);
      lg[CACHE ? m : 0] = logits[e];
      bs[CACHE ? m : 0] = bias[e];
    }
#pragma unroll
    for (int m = 0; m < MAXM; m++) {
      const int e = lane + 64 * m;
      const float v = sigmoid(lg[CACHE ? m : 0]) + bs[CACHE ? m : 0];
      c[CACHE ? m : 0] = (m < nm && e < E && v > -1e30f) ? v : -INFINITY;
    }
  }
  uint32_t taken = 0;
  int sel = 0;
  for (int k = 0; k < rounds; k++) {
    float cv[MAXM];
#pragma unroll
    for (int m = 0; m < MAXM; m++) {
      const int e = lane + 64 * m;
      float v;
      if (CACHE) {
        v = c[CACHE ? m : 0];
      } else {
        const int ec = min(e, E - 1);
        const float t = sigmoid(logits[ec]) + bias[ec];
        v = (m < nm && e < E && t > -1e30f) ? t : -INFINITY;
      }
      cv[m] = ((taken >> m) & 1u) ? -INFINITY : v;
    }
    float mx = cv[0];
#pragma unroll
    for (int m = 1; m < MAXM; m++) mx = fmax_nan_skip(mx, cv[m]);
    mx = wave_max_f32(mx);
    sel = -1;
    if (mx > -INFINITY) {
#pragma unroll
      for (int m = 0; m < MAXM; m++) {
        const unsigned long long b = __ballot(cv[m] == mx);
        if (sel < 0 && b) sel = 64 * m + __builtin_ctzll(b);
      }
    } else {
#pragma unroll
      for (int m = 0; m < MAXM; m++) {
        const int e = lane + 64 * m;
        const unsigned long long b = __ballot(m < nm && e < E && !((taken >> m) & 1u));
        if (sel < 0 && b) sel = 64 * m + __builtin_ctzll(b);
      }
    }
    if ((sel & 63) == lane) taken |= 1u << (sel >> 6);
    if (idx_out && lane == 0) {
      idx_out[k] = sel;
      w_out[k] = sigmoid(logits[sel]) * scale;
    }
    if (sel_out && lane == 0) sel_out[k] = sel;
  }
  return sel;
}

// sel_out (optional, e.g. shared memory) receives every round's expert.
__device__ inline int topk_rounds(const float *logits, const float *bias, int E, int rounds,
                                  float scale, int32_t *idx_out, float *w_out,
                                  int *sel_out = nullptr) {
  if (E <= 256)
    return topk_rounds_m<4, true>(logits, bias, E, rounds, scale, idx_out, w_out, sel_out);
  return topk_rounds_m<16, false>(logits, bias, E, rounds, scale, idx_out, w_out, sel_out);
}

}  // namespace moe
