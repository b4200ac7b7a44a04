/*
 * moe_ref.c -- CPU oracle for the routed-expert int4 MoE block.
 *
 * TEST INFRASTRUCTURE ONLY (see moe_ref.h).  Plain single-threaded C, built
 * with -O2 -ffp-contract=off so that every float expression is evaluated as
 * written: one rounding per operation, no fused multiply-add.
 *
 * Rounding of float to integer uses lrintf in the default rounding mode
 * (round half to even), as the article's listings do in sections 05, 06
 * and 12.
 */
#include "moe_ref.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static int bad_cfg(const moe_ref_config *c) {
  return !c || c->D < 1 || c->I < 1 || c->E < 1 || c->K < 1 || c->K > c->E || c->K > 64 ||
         c->n_shared < 0 || c->n_shared > 1 || !(c->expert_topp >= 0.f && c->expert_topp <= 1.f);
}

int moe_ref_expert_keff(const float *w, int K, float p) {
  float total = 0.f, run = 0.f, thr;
  int k;
  if (!w || K < 1) return -1;
  if (!(p > 0.f && p < 1.f)) return K;
  for (k = 0; k < K; k++) total = total + w[k];
  thr = p * total;
  for (k = 0; k < K; k++) {
    run = run + w[k];
    if (run >= thr) return k + 1;
  }
  return K;
}

/* ---- section 06: int4 weight container ------------------------------------ */

int moe_ref_pack_int4(const float *w, int O, int C, uint8_t *q4, float *scale) {
  if (!w || !q4 || !scale || O < 1 || C < 1) return -1;
  const int qmax = 7, rb = (C + 1) / 2;
  for (int o = 0; o < O; o++) {
    const float *wr = w + (int64_t)o * C;
    float amax = 0.f;
    for (int i = 0; i < C; i++) {
      float a = fabsf(wr[i]);
      if (a > amax) amax = a;
    }
    float s = amax / (float)qmax;
    if (s < 1e-8f) s = 1e-8f;
    scale[o] = s;
    uint8_t *qr = q4 + (int64_t)o * rb;
    for (int i = 0; i < C; i += 2) {
      int v0 = (int)lrintf(wr[i] / s);
      if (v0 > qmax) v0 = qmax;
      if (v0 < -8) v0 = -8;
      int v1 = 0;
      if (i + 1 < C) {
        v1 = (int)lrintf(wr[i + 1] / s);
        if (v1 > qmax) v1 = qmax;
        if (v1 < -8) v1 = -8;
      }
      qr[i >> 1] = (uint8_t)((v0 + 8) | ((v1 + 8) << 4));
    }
  }
  return 0;
}

static inline int nibble_value(const uint8_t *row, int c) {
  uint8_t b = row[c >> 1];
  int n = (c & 1) ? (b >> 4) : (b & 0x0F);
  return n - 8;
}

int moe_ref_unpack_int4(const uint8_t *q4, int O, int C, int8_t *q) {
  if (!q4 || !q || O < 1 || C < 1) return -1;
  const int rb = (C + 1) / 2;
  for (int o = 0; o < O; o++)
    for (int c = 0; c < C; c++) q[(int64_t)o * C + c] = (int8_t)nibble_value(q4 + (int64_t)o * rb, c);
  return 0;
}

/* ---- section 12: activation quantization and integer dots ---------------- */

float moe_ref_quant_row_i8(const float *x, int n, int8_t *q) {
  float amax = 0.f;
  for (int i = 0; i < n; i++) {
    float a = fabsf(x[i]);
    if (a > amax) amax = a;
  }
  float s = amax / 127.f;
  if (s < 1e-12f) s = 1e-12f;
  float inv = 1.f / s;
  for (int i = 0; i < n; i++) {
    long v = lrintf(x[i] * inv);
    /* |x * inv| <= 127 up to rounding, so this clamp never changes a value. */
    if (v > 127) v = 127;
    if (v < -127) v = -127;
    q[i] = (int8_t)v;
  }
  return s;
}

int moe_ref_quant_act_i8(const float *x, int S, int D, int8_t *xq, float *sx) {
  if (!x || !xq || !sx || S < 1 || D < 1) return -1;
  for (int s = 0; s < S; s++)
    sx[s] = moe_ref_quant_row_i8(x + (int64_t)s * D, D, xq + (int64_t)s * D);
  return 0;
}

static float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

int moe_ref_quant_act_i8_bf16(const uint16_t *x, int S, int D, int8_t *xq, float *sx) {
  if (!x || !xq || !sx || S < 1 || D < 1) return -1;
  float *row = (float *)malloc((size_t)D * sizeof(float));
  if (!row) return -2;
  for (int s = 0; s < S; s++) {
    for (int i = 0; i < D; i++) row[i] = bf16_to_f32(x[(int64_t)s * D + i]);
    sx[s] = moe_ref_quant_row_i8(row, D, xq + (int64_t)s * D);
  }
  free(row);
  return 0;
}

int32_t moe_ref_dot_i4_i8(const uint8_t *q4row, const int8_t *x, int C) {
  int32_t acc = 0;
  for (int c = 0; c < C; c++) acc += (int32_t)nibble_value(q4row, c) * (int32_t)x[c];
  return acc;
}

/* ---- section 11: router ---------------------------------------------------- */

static float sigmoid_ref(float v) { return 1.f / (1.f + expf(-v)); }

/* Top-K by repeated argmax over the experts not yet taken.  An expert is a
 * candidate when choice > -1e30 (the article's initial best value; a NaN is
 * never greater, so NaN choices are never picked).  If fewer than K experts are
 * candidates, the remaining slots take the lowest-numbered experts not yet
 * taken (the article leaves this case undefined). */
static void topk_row(const float *choice, const float *sig, int E, int K, float scale,
                     int32_t *idx, float *w) {
  for (int kk = 0; kk < K; kk++) {
    int best = -1;
    float bv = -1e30f;
    for (int e = 0; e < E; e++) {
      int taken = 0;
      for (int j = 0; j < kk; j++)
        if (idx[j] == e) { taken = 1; break; }
      if (!taken && choice[e] > bv) { bv = choice[e]; best = e; }
    }
    if (best < 0) {
      for (int e = 0; e < E && best < 0; e++) {
        int taken = 0;
        for (int j = 0; j < kk; j++)
          if (idx[j] == e) { taken = 1; break; }
        if (!taken) best = e;
      }
    }
    idx[kk] = best;
    w[kk] = sig[best];
  }
  for (int kk = 0; kk < K; kk++) w[kk] *= scale;
}

int moe_ref_router_topk(const moe_ref_config *cfg, const float *x, int S, const float *router_w,
                        const float *router_b, int32_t *idx, float *w, float *logits,
                        float *choice) {
  if (bad_cfg(cfg) || !x || !router_w || !router_b || !idx || !w || S < 1) return -1;
  const int D = cfg->D, E = cfg->E, K = cfg->K;
  float *sig = (float *)malloc((size_t)E * sizeof(float));
  float *ch = (float *)malloc((size_t)E * sizeof(float));
  if (!sig || !ch) { free(sig); free(ch); return -2; }
  for (int s = 0; s < S; s++) {
    const float *xs = x + (int64_t)s * D;
    for (int e = 0; e < E; e++) {
      const float *we = router_w + (int64_t)e * D;
      double acc = 0.0;
      for (int i = 0; i < D; i++) acc += (double)xs[i] * (double)we[i];
      float lg = (float)acc;
      if (logits) logits[(int64_t)s * E + e] = lg;
      sig[e] = sigmoid_ref(lg);
      ch[e] = sig[e] + router_b[e];
      if (choice) choice[(int64_t)s * E + e] = ch[e];
    }
    topk_row(ch, sig, E, K, cfg->routed_scale, idx + (int64_t)s * K, w + (int64_t)s * K);
  }
  free(sig);
  free(ch);
  return 0;
}

/* ---- sections 11 and 12: one SwiGLU expert ---------------------------------- */

static float silu_ref(float v) { return v / (1.f + expf(-v)); }

static int qmat_ok(const moe_ref_qmat *m) { return m->q4 && m->scale; }

int moe_ref_expert_swiglu_i4(const moe_ref_config *cfg, const int8_t *xq, const float *sx, int S,
                             const moe_ref_expert *e, float *y, int32_t *acc_gu, int8_t *hq,
                             float *sh, int32_t *acc_d) {
  if (bad_cfg(cfg) || !xq || !sx || !e || !y || S < 1) return -1;
  if (!qmat_ok(&e->gate) || !qmat_ok(&e->up) || !qmat_ok(&e->down)) return -1;
  const int D = cfg->D, I = cfg->I;
  const int rbD = (D + 1) / 2, rbI = (I + 1) / 2;
  float *h = (float *)malloc((size_t)I * sizeof(float));
  int8_t *hqr = (int8_t *)malloc((size_t)I);
  if (!h || !hqr) { free(h); free(hqr); return -2; }
  for (int s = 0; s < S; s++) {
    const int8_t *xs = xq + (int64_t)s * D;
    const float sxs = sx[s];
    /* gate and up: integer dots, then (acc * row scale) * activation scale */
    for (int o = 0; o < I; o++) {
      int32_t ag = moe_ref_dot_i4_i8(e->gate.q4 + (int64_t)o * rbD, xs, D);
      int32_t au = moe_ref_dot_i4_i8(e->up.q4 + (int64_t)o * rbD, xs, D);
      if (acc_gu) {
        acc_gu[((int64_t)s * 2 + 0) * I + o] = ag;
        acc_gu[((int64_t)s * 2 + 1) * I + o] = au;
      }
      float g = ((float)ag * e->gate.scale[o]) * sxs;
      float u = ((float)au * e->up.scale[o]) * sxs;
      h[o] = silu_ref(g) * u;
    }
    /* the down projection is an integer matmul too, so its input is quantized */
    float shs = moe_ref_quant_row_i8(h, I, hqr);
    if (hq) memcpy(hq + (int64_t)s * I, hqr, (size_t)I);
    if (sh) sh[s] = shs;
    for (int d = 0; d < D; d++) {
      int32_t ad = moe_ref_dot_i4_i8(e->down.q4 + (int64_t)d * rbI, hqr, I);
      if (acc_d) acc_d[(int64_t)s * D + d] = ad;
      y[(int64_t)s * D + d] = ((float)ad * e->down.scale[d]) * shs;
    }
  }
  free(h);
  free(hqr);
  return 0;
}

/* ---- section 05: int8 weight rows; section 12: the int8 integer path ------ */

int moe_ref_quantize_rows(const float *w, int O, int C, int bits, int8_t *q, float *scale) {
  if (!w || !q || !scale || O < 1 || C < 1 || bits < 2 || bits > 8) return -1;
  const int qmax = (1 << (bits - 1)) - 1;
  for (int o = 0; o < O; o++) {
    const float *wr = w + (int64_t)o * C;
    float amax = 0.f;
    for (int i = 0; i < C; i++) {
      float a = fabsf(wr[i]);
      if (a > amax) amax = a;
    }
    float s = amax / (float)qmax;
    if (s < 1e-8f) s = 1e-8f;
    scale[o] = s;
    int8_t *qr = q + (int64_t)o * C;
    for (int i = 0; i < C; i++) {
      long v = lrintf(wr[i] / s);
      if (v > qmax) v = qmax;
      if (v < -qmax - 1) v = -qmax - 1;
      qr[i] = (int8_t)v;
    }
  }
  return 0;
}

int32_t moe_ref_dot_i8_i8(const int8_t *w, const int8_t *x, int C) {
  int32_t acc = 0;
  for (int c = 0; c < C; c++) acc += (int32_t)w[c] * (int32_t)x[c];
  return acc;
}

static int q8mat_ok(const moe_ref_q8mat *m) { return m->q && m->scale; }

int moe_ref_expert_swiglu_i8(const moe_ref_config *cfg, const int8_t *xq, const float *sx, int S,
                             const moe_ref_expert_i8 *e, float *y, int32_t *acc_gu, int8_t *hq,
                             float *sh, int32_t *acc_d) {
  if (bad_cfg(cfg) || !xq || !sx || !e || !y || S < 1) return -1;
  if (!q8mat_ok(&e->gate) || !q8mat_ok(&e->up) || !q8mat_ok(&e->down)) return -1;
  const int D = cfg->D, I = cfg->I;
  float *h = (float *)malloc((size_t)I * sizeof(float));
  int8_t *hqr = (int8_t *)malloc((size_t)I);
  if (!h || !hqr) { free(h); free(hqr); return -2; }
  for (int s = 0; s < S; s++) {
    const int8_t *xs = xq + (int64_t)s * D;
    const float sxs = sx[s];
    for (int o = 0; o < I; o++) {
      int32_t ag = moe_ref_dot_i8_i8(e->gate.q + (int64_t)o * D, xs, D);
      int32_t au = moe_ref_dot_i8_i8(e->up.q + (int64_t)o * D, xs, D);
      if (acc_gu) {
        acc_gu[((int64_t)s * 2 + 0) * I + o] = ag;
        acc_gu[((int64_t)s * 2 + 1) * I + o] = au;
      }
      float g = ((float)ag * e->gate.scale[o]) * sxs;
      float u = ((float)au * e->up.scale[o]) * sxs;
      h[o] = silu_ref(g) * u;
    }
    float shs = moe_ref_quant_row_i8(h, I, hqr);
    if (hq) memcpy(hq + (int64_t)s * I, hqr, (size_t)I);
    if (sh) sh[s] = shs;
    for (int d = 0; d < D; d++) {
      int32_t ad = moe_ref_dot_i8_i8(e->down.q + (int64_t)d * I, hqr, I);
      if (acc_d) acc_d[(int64_t)s * D + d] = ad;
      y[(int64_t)s * D + d] = ((float)ad * e->down.scale[d]) * shs;
    }
  }
  free(h);
  free(hqr);
  return 0;
}

/* ---- packed int2 (reading: the int4 container's rule at 2 bits) --------- */

int moe_ref_pack_int2(const float *w, int O, int C, uint8_t *q2, float *scale) {
  if (!w || !q2 || !scale || O < 1 || C < 1) return -1;
  int8_t *q = (int8_t *)malloc((size_t)O * C);
  if (!q) return -2;
  int rc = moe_ref_quantize_rows(w, O, C, 2, q, scale);
  const int rb = (C + 3) / 4;
  for (int o = 0; rc == 0 && o < O; o++)
    for (int j = 0; j < rb; j++) {
      unsigned b = 0;
      for (int k = 0; k < 4; k++) {
        const int c = 4 * j + k;
        const int v = c < C ? q[(int64_t)o * C + c] : 0;
        b |= (unsigned)(v + 2) << (2 * k);
      }
      q2[(int64_t)o * rb + j] = (uint8_t)b;
    }
  free(q);
  return rc;
}

int moe_ref_unpack_int2(const uint8_t *q2, int O, int C, int8_t *q) {
  if (!q2 || !q || O < 1 || C < 1) return -1;
  const int rb = (C + 3) / 4;
  for (int o = 0; o < O; o++)
    for (int c = 0; c < C; c++) {
      const uint8_t b = q2[(int64_t)o * rb + c / 4];
      q[(int64_t)o * C + c] = (int8_t)(((b >> (2 * (c % 4))) & 3) - 2);
    }
  return 0;
}

static int widen_int2(const moe_ref_qmat *m, int O, int C, int8_t **out) {
  *out = (int8_t *)malloc((size_t)O * C);
  if (!*out) return -2;
  return moe_ref_unpack_int2(m->q4, O, C, *out);
}

int moe_ref_expert_swiglu_i2(const moe_ref_config *cfg, const int8_t *xq, const float *sx, int S,
                             const moe_ref_expert_i2 *e, float *y, int32_t *acc_gu, int8_t *hq,
                             float *sh, int32_t *acc_d) {
  if (bad_cfg(cfg) || !xq || !sx || !e || !y || S < 1) return -1;
  if (!qmat_ok(&e->gate) || !qmat_ok(&e->up) || !qmat_ok(&e->down)) return -1;
  const int D = cfg->D, I = cfg->I;
  int8_t *g = NULL, *u = NULL, *d = NULL;
  int rc = widen_int2(&e->gate, I, D, &g);
  if (rc == 0) rc = widen_int2(&e->up, I, D, &u);
  if (rc == 0) rc = widen_int2(&e->down, D, I, &d);
  if (rc == 0) {
    moe_ref_expert_i8 e8 = {{g, e->gate.scale}, {u, e->up.scale}, {d, e->down.scale}};
    rc = moe_ref_expert_swiglu_i8(cfg, xq, sx, S, &e8, y, acc_gu, hq, sh, acc_d);
  }
  free(g);
  free(u);
  free(d);
  return rc;
}

/* ---- block-32 activation scales (reading of the "Q8_0 style" remark) ---- */

int moe_ref_quant_act_b32(const float *x, int S, int D, int8_t *xq, float *sxb) {
  if (!x || !xq || !sxb || S < 1 || D < 32 || D % 32) return -1;
  const int nb = D / 32;
  for (int s = 0; s < S; s++)
    for (int b = 0; b < nb; b++) {
      const int64_t off = (int64_t)s * D + 32 * b;
      sxb[(int64_t)s * nb + b] = moe_ref_quant_row_i8(x + off, 32, xq + off);
    }
  return 0;
}

/* s_w * sum_b acc_b * s_b for one packed int4 row against block-quantized q. */
static float dot_b32(const uint8_t *q4row, const int8_t *q, const float *sb, int C, float sw) {
  double t = 0.0;
  for (int b = 0; b < C / 32; b++) {
    int32_t acc = 0;
    for (int c = 32 * b; c < 32 * b + 32; c++) acc += nibble_value(q4row, c) * (int32_t)q[c];
    t += (double)acc * (double)sb[b];
  }
  return (float)(t * (double)sw);
}

int moe_ref_expert_swiglu_i4_b32(const moe_ref_config *cfg, const int8_t *xq, const float *sxb,
                                 int S, const moe_ref_expert *e, float *y, int8_t *hq,
                                 float *shb) {
  if (bad_cfg(cfg) || !xq || !sxb || !e || !y || S < 1) return -1;
  if (!qmat_ok(&e->gate) || !qmat_ok(&e->up) || !qmat_ok(&e->down)) return -1;
  const int D = cfg->D, I = cfg->I;
  if (D % 32 || I % 32) return -1;
  const int rbD = D / 2, rbI = I / 2;
  float *h = (float *)malloc((size_t)I * sizeof(float));
  int8_t *hqr = (int8_t *)malloc((size_t)I);
  float *hs = (float *)malloc((size_t)(I / 32) * sizeof(float));
  if (!h || !hqr || !hs) { free(h); free(hqr); free(hs); return -2; }
  for (int s = 0; s < S; s++) {
    const int8_t *xs = xq + (int64_t)s * D;
    const float *sb = sxb + (int64_t)s * (D / 32);
    for (int o = 0; o < I; o++) {
      const float g = dot_b32(e->gate.q4 + (int64_t)o * rbD, xs, sb, D, e->gate.scale[o]);
      const float u = dot_b32(e->up.q4 + (int64_t)o * rbD, xs, sb, D, e->up.scale[o]);
      h[o] = silu_ref(g) * u;
    }
    moe_ref_quant_act_b32(h, 1, I, hqr, hs);
    if (hq) memcpy(hq + (int64_t)s * I, hqr, (size_t)I);
    if (shb) memcpy(shb + (int64_t)s * (I / 32), hs, (size_t)(I / 32) * sizeof(float));
    for (int d = 0; d < D; d++)
      y[(int64_t)s * D + d] = dot_b32(e->down.q4 + (int64_t)d * rbI, hqr, hs, I, e->down.scale[d]);
  }
  free(h);
  free(hqr);
  free(hs);
  return 0;
}

/* ---- section 09: MLA decode attention with weight absorption -------------- */

int moe_ref_mla_decode(const moe_ref_mla_config *c, const float *q, int S, const float *kv_b,
                       const float *L, const float *R, int T, float *ctx) {
  if (!c || !q || !kv_b || !L || !R || !ctx || S < 1 || T < S) return -1;
  if (c->H < 1 || c->kvl < 1 || c->nope < 1 || c->rope < 0 || c->vdim < 1) return -1;
  const int H = c->H, kvl = c->kvl, nope = c->nope, rope = c->rope, vd = c->vdim;
  const int qh = nope + rope, rows = nope + vd;
  double *qabs = (double *)malloc((size_t)kvl * sizeof(double));
  double *clat = (double *)malloc((size_t)kvl * sizeof(double));
  double *sc = (double *)malloc((size_t)T * sizeof(double));
  if (!qabs || !clat || !sc) { free(qabs); free(clat); free(sc); return -2; }
  for (int s = 0; s < S; s++) {
    const int n = T - S + 1 + s;
    for (int h = 0; h < H; h++) {
      const float *qp = q + ((int64_t)s * H + h) * qh;
      const float *wk = kv_b + (int64_t)h * rows * kvl;
      const float *wv = wk + (int64_t)nope * kvl;
      for (int i = 0; i < kvl; i++) qabs[i] = 0.0;
      for (int d = 0; d < nope; d++)
        for (int i = 0; i < kvl; i++) qabs[i] += (double)qp[d] * (double)wk[(int64_t)d * kvl + i];
      double mx = -INFINITY;
      for (int t = 0; t < n; t++) {
        double a = 0.0;
        for (int i = 0; i < kvl; i++) a += qabs[i] * (double)L[(int64_t)t * kvl + i];
        for (int d = 0; d < rope; d++) a += (double)qp[nope + d] * (double)R[(int64_t)t * rope + d];
        sc[t] = a * (double)c->scale;
        if (sc[t] > mx) mx = sc[t];
      }
      double sum = 0.0;
      for (int t = 0; t < n; t++) {
        sc[t] = exp(sc[t] - mx);
        sum += sc[t];
      }
      for (int i = 0; i < kvl; i++) clat[i] = 0.0;
      for (int t = 0; t < n; t++)
        for (int i = 0; i < kvl; i++) clat[i] += (sc[t] / sum) * (double)L[(int64_t)t * kvl + i];
      float *out = ctx + ((int64_t)s * H + h) * vd;
      for (int v = 0; v < vd; v++) {
        double a = 0.0;
        for (int i = 0; i < kvl; i++) a += (double)wv[(int64_t)v * kvl + i] * clat[i];
        out[v] = (float)a;
      }
    }
  }
  free(qabs);
  free(clat);
  free(sc);
  return 0;
}

/* ---- the block ------------------------------------------------------------ */

static int layer_ok(const moe_ref_config *cfg, const moe_ref_layer *L) {
  if (bad_cfg(cfg) || !L || !L->router_w || !L->router_b || !L->experts) return 0;
  if (cfg->n_shared == 1 && !L->shared) return 0;
  return 1;
}

static void combine_row(const moe_ref_config *cfg, const float *w, int keff, const float *stage,
                        float *out, unsigned flags) {
  /* stage holds K (+1 shared) rows of D floats for one token; the first keff
   * routed rows take part */
  const int D = cfg->D, K = cfg->K;
  for (int d = 0; d < D; d++) {
    float acc = 0.f;
    for (int k = 0; k < keff; k++) acc += w[k] * stage[(int64_t)k * D + d];
    if (cfg->n_shared == 1) acc += stage[(int64_t)K * D + d];
    if (flags & MOE_REF_ACCUMULATE)
      out[d] = out[d] + acc;
    else
      out[d] = acc;
  }
}

/* shared8 (optional): the shared expert in the int8 format, used in place of
 * layer->shared. */
static int layer_forward_impl(const moe_ref_config *cfg, const moe_ref_layer *layer,
                              const moe_ref_expert_i8 *shared8, const float *x, int S, float *out,
                              unsigned flags) {
  if (!x || !out || S < 1) return -1;
  const int D = cfg->D, K = cfg->K, slots = cfg->K + cfg->n_shared;
  int32_t idx[64];
  float w[64];
  int8_t *xq = (int8_t *)malloc((size_t)D);
  float *stage = (float *)malloc((size_t)slots * D * sizeof(float));
  if (!xq || !stage) { free(xq); free(stage); return -2; }
  int rc = 0;
  for (int s = 0; s < S && rc == 0; s++) {
    const float *xs = x + (int64_t)s * D;
    rc = moe_ref_router_topk(cfg, xs, 1, layer->router_w, layer->router_b, idx, w, NULL, NULL);
    if (rc) break;
    float sxs = moe_ref_quant_row_i8(xs, D, xq);
    const int keff = moe_ref_expert_keff(w, K, cfg->expert_topp);
    for (int k = 0; k < keff && rc == 0; k++)
      rc = moe_ref_expert_swiglu_i4(cfg, xq, &sxs, 1, &layer->experts[idx[k]],
                                    stage + (int64_t)k * D, NULL, NULL, NULL, NULL);
    if (rc == 0 && cfg->n_shared == 1)
      rc = shared8 ? moe_ref_expert_swiglu_i8(cfg, xq, &sxs, 1, shared8, stage + (int64_t)K * D,
                                              NULL, NULL, NULL, NULL)
                   : moe_ref_expert_swiglu_i4(cfg, xq, &sxs, 1, layer->shared,
                                              stage + (int64_t)K * D, NULL, NULL, NULL, NULL);
    if (rc == 0) combine_row(cfg, w, keff, stage, out + (int64_t)s * D, flags);
  }
  free(xq);
  free(stage);
  return rc;
}

int moe_ref_layer_forward(const moe_ref_config *cfg, const moe_ref_layer *layer, const float *x,
                          int S, float *out, unsigned flags) {
  if (!layer_ok(cfg, layer)) return -1;
  return layer_forward_impl(cfg, layer, NULL, x, S, out, flags);
}

int moe_ref_layer_forward_shared_i8(const moe_ref_config *cfg, const moe_ref_layer *layer,
                                    const moe_ref_expert_i8 *shared8, const float *x, int S,
                                    float *out, unsigned flags) {
  if (!cfg || cfg->n_shared != 1 || !shared8) return -1;
  if (!q8mat_ok(&shared8->gate) || !q8mat_ok(&shared8->up) || !q8mat_ok(&shared8->down)) return -1;
  moe_ref_config c0 = *cfg;
  c0.n_shared = 0;  /* the routed experts and the router are checked as usual */
  if (!layer_ok(&c0, layer)) return -1;
  return layer_forward_impl(cfg, layer, shared8, x, S, out, flags);
}

int moe_ref_layer_forward_batch(const moe_ref_config *cfg, const moe_ref_layer *layer,
                                const float *x, int S, float *out, unsigned flags, int32_t *idx_out,
                                float *w_out, int32_t *uniq_out, int32_t *n_uniq_out) {
  if (!layer_ok(cfg, layer) || !x || !out || S < 1) return -1;
  const int D = cfg->D, E = cfg->E, K = cfg->K, slots = cfg->K + cfg->n_shared;
  int32_t *idx = (int32_t *)malloc((size_t)S * K * sizeof(int32_t));
  float *w = (float *)malloc((size_t)S * K * sizeof(float));
  int8_t *xq = (int8_t *)malloc((size_t)S * D);
  float *sx = (float *)malloc((size_t)S * sizeof(float));
  float *stage = (float *)malloc((size_t)S * slots * D * sizeof(float));
  int32_t *uniq = (int32_t *)malloc((size_t)E * sizeof(int32_t));
  unsigned char *seen = (unsigned char *)calloc((size_t)E, 1);
  int32_t *rows = (int32_t *)malloc((size_t)S * sizeof(int32_t));
  int32_t *slot = (int32_t *)malloc((size_t)S * sizeof(int32_t));
  int8_t *xg = (int8_t *)malloc((size_t)S * D);
  float *sg = (float *)malloc((size_t)S * sizeof(float));
  float *yg = (float *)malloc((size_t)S * D * sizeof(float));
  int32_t *keff = (int32_t *)malloc((size_t)S * sizeof(int32_t));
  int rc = -2;
  if (!idx || !w || !xq || !sx || !stage || !uniq || !seen || !rows || !slot || !xg || !sg || !yg ||
      !keff)
    goto done;
  rc = moe_ref_router_topk(cfg, x, S, layer->router_w, layer->router_b, idx, w, NULL, NULL);
  if (rc) goto done;
  moe_ref_quant_act_i8(x, S, D, xq, sx);
  /* keff[s] experts per token; the union of the kept experts, in order of
   * first appearance */
  for (int s = 0; s < S; s++) keff[s] = moe_ref_expert_keff(w + (int64_t)s * K, K, cfg->expert_topp);
  int nu = 0;
  for (int s = 0; s < S; s++)
    for (int k = 0; k < keff[s]; k++) {
      int e = idx[(int64_t)s * K + k];
      if (!seen[e]) { seen[e] = 1; uniq[nu++] = e; }
    }
  for (int u = 0; u < nu && rc == 0; u++) {
    int e = uniq[u], nr = 0;
    for (int s = 0; s < S; s++)
      for (int k = 0; k < keff[s]; k++)
        if (idx[(int64_t)s * K + k] == e) { rows[nr] = s; slot[nr] = k; nr++; }
    for (int r = 0; r < nr; r++) {
      memcpy(xg + (int64_t)r * D, xq + (int64_t)rows[r] * D, (size_t)D);
      sg[r] = sx[rows[r]];
    }
    rc = moe_ref_expert_swiglu_i4(cfg, xg, sg, nr, &layer->experts[e], yg, NULL, NULL, NULL, NULL);
    for (int r = 0; r < nr && rc == 0; r++)
      memcpy(stage + ((int64_t)rows[r] * slots + slot[r]) * D, yg + (int64_t)r * D,
             (size_t)D * sizeof(float));
  }
  if (rc == 0 && cfg->n_shared == 1) {
    /* the shared expert is read once and applied to every row */
    rc = moe_ref_expert_swiglu_i4(cfg, xq, sx, S, layer->shared, yg, NULL, NULL, NULL, NULL);
    for (int s = 0; s < S && rc == 0; s++)
      memcpy(stage + ((int64_t)s * slots + K) * D, yg + (int64_t)s * D, (size_t)D * sizeof(float));
  }
  if (rc == 0)
    for (int s = 0; s < S; s++)
      combine_row(cfg, w + (int64_t)s * K, keff[s], stage + (int64_t)s * slots * D,
                  out + (int64_t)s * D, flags);
  if (rc == 0) {
    if (idx_out) memcpy(idx_out, idx, (size_t)S * K * sizeof(int32_t));
    if (w_out) memcpy(w_out, w, (size_t)S * K * sizeof(float));
    if (uniq_out) memcpy(uniq_out, uniq, (size_t)nu * sizeof(int32_t));
    if (n_uniq_out) *n_uniq_out = nu;
  }
done:
  free(idx); free(w); free(xq); free(sx); free(stage); free(uniq); free(seen);
  free(rows); free(slot); free(xg); free(sg); free(yg); free(keff);
  return rc;
}

/* ---- section 04: RMSNorm ---------------------------------------------------- */

int moe_ref_rmsnorm(const float *x, const float *gamma, int S, int D, float eps, float *y) {
  if (!x || !gamma || !y || S < 1 || D < 1) return -1;
  for (int s = 0; s < S; s++) {
    const float *xs = x + (int64_t)s * D;
    float *ys = y + (int64_t)s * D;
    double ms = 0.0;
    for (int i = 0; i < D; i++) ms += (double)xs[i] * xs[i];
    float r = 1.f / sqrtf((float)(ms / D) + eps);
    for (int i = 0; i < D; i++) ys[i] = xs[i] * r * gamma[i];
  }
  return 0;
}

/* ---- section 05 expert cache and section 13 tier policy ---------------- */

int moe_ref_expert_get(int32_t *slot_eid, uint64_t *slot_used, int cap, int *n_used,
                       uint64_t *clock, uint64_t *hits, uint64_t *misses, int32_t eid,
                       int *loaded) {
  int i, victim;
  if (!slot_eid || !slot_used || !n_used || !clock || !hits || !misses || !loaded) return -1;
  if (cap < 1 || *n_used < 0 || *n_used > cap) return -1;
  /* lookup: a hit refreshes the slot's use */
  for (i = 0; i < *n_used; i++) {
    if (slot_eid[i] == eid) {
      *hits += 1;
      *clock += 1;
      slot_used[i] = *clock;
      *loaded = 0;
      return i;
    }
  }
  *misses += 1;
  if (*n_used < cap) {
    victim = *n_used;
    *n_used += 1;
  } else {
    /* least recently used slot */
    victim = 0;
    for (i = 1; i < *n_used; i++)
      if (slot_used[i] < slot_used[victim]) victim = i;
  }
  slot_eid[victim] = eid;
  *clock += 1;
  slot_used[victim] = *clock;
  *loaded = 1;
  return victim;
}

int moe_ref_tier_pick_swap(const uint32_t *heat, int nexpert, const int32_t *pinned, int npin,
                           int32_t *slot, int32_t *eid, int64_t *gain) {
  int z, e, cold = 0, hot = -1;
  uint32_t fh = 0;
  uint64_t fc;
  if (!heat || !pinned || !slot || !eid || !gain || npin < 1 || nexpert < 1) return 0;
  for (z = 0; z < npin; z++)
    if (pinned[z] < 0 || pinned[z] >= nexpert) return 0;
  for (z = 1; z < npin; z++)
    if (heat[pinned[z]] < heat[pinned[cold]]) cold = z;
  for (e = 0; e < nexpert; e++) {
    int resident = 0;
    for (z = 0; z < npin; z++) {
      if (pinned[z] == e) {
        resident = 1;
        break;
      }
    }
    if (!resident && heat[e] > fh) {
      fh = heat[e];
      hot = e;
    }
  }
  if (hot < 0) return 0;
  fc = heat[pinned[cold]];
  if ((uint64_t)fh <= fc + fc / 4 + 4) return 0;
  *slot = cold;
  *eid = hot;
  *gain = (int64_t)fh - (int64_t)fc;
  return 1;
}

uint64_t moe_ref_tier_lfru_score(uint32_t heat, uint32_t last, uint32_t clock) {
  uint32_t age = clock - last;
  uint32_t recent = age < 255u ? 255u - age : 0u;
  return ((uint64_t)heat << 8) | (uint64_t)recent;
}
