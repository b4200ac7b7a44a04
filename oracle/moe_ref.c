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

/* Codes of one row: the row's scale is its largest magnitude over qmax,
 * floored at floor_s; sections 05 and 06 divide each weight by that scale,
 * section 12 multiplies each activation by its reciprocal.  Every code is
 * rounded half to even and clamped into [lo, hi]. */
static float row_absmax(const float *v, int n) {
  float m = 0.f;
  for (int i = 0; i < n; i++)
    if (fabsf(v[i]) > m) m = fabsf(v[i]); /* a NaN never compares greater */
  return m;
}

static float row_scale(float amax, int qmax, float floor_s) {
  const float s = amax / (float)qmax;
  return s < floor_s ? floor_s : s;
}

static int clamp_code(long v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : (int)v); }

int moe_ref_pack_int4(const float *w, int O, int C, uint8_t *q4, float *scale) {
  if (!w || !q4 || !scale || O < 1 || C < 1) return -1;
  /* the section 06 container is the section 05 quantizer at 4 bits, then two
   * codes per byte as code + 8 (even column low) */
  int8_t *codes = (int8_t *)malloc((size_t)O * C);
  if (!codes) return -2;
  moe_ref_quantize_rows(w, O, C, 4, codes, scale);
  const int rb = (C + 1) / 2;
  for (int o = 0; o < O; o++) {
    const int8_t *cr = codes + (int64_t)o * C;
    for (int j = 0; j < rb; j++) {
      const int lo = cr[2 * j] + 8;
      const int hi = (2 * j + 1 < C ? cr[2 * j + 1] : 0) + 8;
      q4[(int64_t)o * rb + j] = (uint8_t)(lo | (hi << 4));
    }
  }
  free(codes);
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
  const float s = row_scale(row_absmax(x, n), 127, 1e-12f);
  const float inv = 1.f / s;
  /* |x * inv| <= 127 up to rounding, so the clamp never changes a code */
  for (int i = 0; i < n; i++) q[i] = (int8_t)clamp_code(lrintf(x[i] * inv), -127, 127);
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

/* Top-K selection.  Each pass of the section 11 rule takes the largest
 * choice among the experts not yet taken, scanning the experts in ascending
 * order with a strict comparison, so the K passes return the experts ranked
 * by (choice descending, index ascending).  The listing's running best starts
 * at -1e30 and a NaN never compares greater, so only choices > -1e30 are
 * candidates; if fewer than K experts are candidates, the remaining passes
 * find none and (a reading: the article leaves this case undefined) take the
 * lowest-numbered experts not yet taken.  The ranking below sorts by exactly
 * that order: candidates first, by choice then index, then the others by
 * index. */
typedef struct {
  float choice;
  int expert;
  int candidate;
} ranked;

static int rank_order(const void *pa, const void *pb) {
  const ranked *a = (const ranked *)pa, *b = (const ranked *)pb;
  if (a->candidate != b->candidate) return b->candidate - a->candidate;
  if (a->candidate && a->choice != b->choice) return a->choice > b->choice ? -1 : 1;
  return a->expert - b->expert;
}

static int select_top_k(const float *choice, const float *sig, int E, int K, float scale,
                        int32_t *idx, float *w) {
  ranked *r = (ranked *)malloc((size_t)E * sizeof(ranked));
  if (!r) return -2;
  for (int e = 0; e < E; e++) {
    r[e].choice = choice[e];
    r[e].expert = e;
    r[e].candidate = choice[e] > -1e30f;
  }
  qsort(r, (size_t)E, sizeof(ranked), rank_order);
  for (int k = 0; k < K; k++) {
    idx[k] = r[k].expert;
    w[k] = sig[idx[k]] * scale; /* the unbiased sigmoid times the routed scale */
  }
  free(r);
  return 0;
}

int moe_ref_router_topk(const moe_ref_config *cfg, const float *x, int S, const float *router_w,
                        const float *router_b, int32_t *idx, float *w, float *logits,
                        float *choice) {
  if (bad_cfg(cfg) || !x || !router_w || !router_b || !idx || !w || S < 1) return -1;
  const int D = cfg->D, E = cfg->E, K = cfg->K;
  float *sig = (float *)malloc((size_t)E * sizeof(float));
  float *ch = (float *)malloc((size_t)E * sizeof(float));
  int rc = (sig && ch) ? 0 : -2;
  for (int s = 0; s < S && rc == 0; s++) {
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
    rc = select_top_k(ch, sig, E, K, cfg->routed_scale, idx + (int64_t)s * K, w + (int64_t)s * K);
  }
  free(sig);
  free(ch);
  return rc;
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
    const float s = row_scale(row_absmax(wr, C), qmax, 1e-8f);
    scale[o] = s;
    for (int i = 0; i < C; i++)
      q[(int64_t)o * C + i] = (int8_t)clamp_code(lrintf(wr[i] / s), -qmax - 1, qmax);
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

static int layer_ok(const moe_ref_config *cfg, const moe_ref_layer *L, int need_router) {
  if (bad_cfg(cfg) || !L || !L->experts) return 0;
  if (need_router && (!L->router_w || !L->router_b)) return 0;
  if (cfg->n_shared == 1 && !L->shared) return 0;
  return 1;
}

static int routing_ok(const moe_ref_config *cfg, const int32_t *idx, const float *w, int S) {
  if (!idx || !w) return 0;
  for (int64_t p = 0; p < (int64_t)S * cfg->K; p++)
    if (idx[p] < 0 || idx[p] >= cfg->E) return 0;
  return 1;
}

/* Section 11's combine for one token: the first keff routed results weighted
 * by their combine weights, added in slot order starting from 0, then the
 * shared expert's result with weight 1 (a reading: the article's listing
 * shows the routed sum only).  stage holds K (+1 shared) rows of D floats. */
static void combine_row(const moe_ref_config *cfg, const float *w, int keff, const float *stage,
                        float *out, unsigned flags) {
  const int D = cfg->D, K = cfg->K;
  for (int d = 0; d < D; d++) {
    float acc = 0.f;
    for (int k = 0; k < keff; k++) acc += w[k] * stage[(int64_t)k * D + d];
    if (cfg->n_shared == 1) acc += stage[(int64_t)K * D + d];
    out[d] = (flags & MOE_REF_ACCUMULATE) ? out[d] + acc : acc;
  }
}

/* The shared expert on S quantized rows, in the int4 format or (shared8 set)
 * the int8 one. */
static int shared_rows(const moe_ref_config *cfg, const moe_ref_layer *layer,
                       const moe_ref_expert_i8 *shared8, const int8_t *xq, const float *sx, int S,
                       float *y) {
  return shared8 ? moe_ref_expert_swiglu_i8(cfg, xq, sx, S, shared8, y, NULL, NULL, NULL, NULL)
                 : moe_ref_expert_swiglu_i4(cfg, xq, sx, S, layer->shared, y, NULL, NULL, NULL,
                                            NULL);
}

/* The experts of the block for one token whose routing is known: quantize
 * the token, run the first keff selected experts and the shared expert on
 * it, combine.  stage: (K + 1) * D floats of scratch. */
static int token_block(const moe_ref_config *cfg, const moe_ref_layer *layer,
                       const moe_ref_expert_i8 *shared8, const float *xs, const int32_t *idx,
                       const float *w, int keff, float *stage, int8_t *xq, float *out,
                       unsigned flags) {
  const int D = cfg->D, K = cfg->K;
  float sxs = moe_ref_quant_row_i8(xs, D, xq);
  int rc = 0;
  for (int k = 0; k < keff && rc == 0; k++)
    rc = moe_ref_expert_swiglu_i4(cfg, xq, &sxs, 1, &layer->experts[idx[k]],
                                  stage + (int64_t)k * D, NULL, NULL, NULL, NULL);
  if (rc == 0 && cfg->n_shared == 1)
    rc = shared_rows(cfg, layer, shared8, xq, &sxs, 1, stage + (int64_t)K * D);
  if (rc == 0) combine_row(cfg, w, keff, stage, out, flags);
  return rc;
}

/* Per-token path.  With given_idx/given_w the routing is the caller's and all
 * K experts run; otherwise each token is routed first (section 11: routing,
 * then the experts) and keeps keff experts. */
static int per_token(const moe_ref_config *cfg, const moe_ref_layer *layer,
                     const moe_ref_expert_i8 *shared8, const float *x, int S,
                     const int32_t *given_idx, const float *given_w, float *out, unsigned flags) {
  if (!x || !out || S < 1) return -1;
  const int D = cfg->D, K = cfg->K;
  int32_t idx[64];
  float w[64];
  int8_t *xq = (int8_t *)malloc((size_t)D);
  float *stage = (float *)malloc((size_t)(K + 1) * D * sizeof(float));
  int rc = (xq && stage) ? 0 : -2;
  for (int s = 0; s < S && rc == 0; s++) {
    const float *xs = x + (int64_t)s * D;
    const int32_t *ti = idx;
    const float *tw = w;
    int keff = K;
    if (given_idx) {
      ti = given_idx + (int64_t)s * K;
      tw = given_w + (int64_t)s * K;
    } else {
      rc = moe_ref_router_topk(cfg, xs, 1, layer->router_w, layer->router_b, idx, w, NULL, NULL);
      keff = moe_ref_expert_keff(w, K, cfg->expert_topp);
    }
    if (rc == 0)
      rc = token_block(cfg, layer, shared8, xs, ti, tw, keff, stage, xq, out + (int64_t)s * D,
                       flags);
  }
  free(xq);
  free(stage);
  return rc;
}

int moe_ref_layer_forward(const moe_ref_config *cfg, const moe_ref_layer *layer, const float *x,
                          int S, float *out, unsigned flags) {
  if (!layer_ok(cfg, layer, 1)) return -1;
  return per_token(cfg, layer, NULL, x, S, NULL, NULL, out, flags);
}

int moe_ref_layer_forward_routed(const moe_ref_config *cfg, const moe_ref_layer *layer,
                                 const float *x, int S, const int32_t *idx, const float *w,
                                 float *out, unsigned flags) {
  if (!layer_ok(cfg, layer, 0) || S < 1 || !routing_ok(cfg, idx, w, S)) return -1;
  return per_token(cfg, layer, NULL, x, S, idx, w, out, flags);
}

static int shared8_ok(const moe_ref_config *cfg, const moe_ref_expert_i8 *e) {
  return cfg && cfg->n_shared == 1 && e && q8mat_ok(&e->gate) && q8mat_ok(&e->up) &&
         q8mat_ok(&e->down);
}

int moe_ref_layer_forward_shared_i8(const moe_ref_config *cfg, const moe_ref_layer *layer,
                                    const moe_ref_expert_i8 *shared8, const float *x, int S,
                                    float *out, unsigned flags) {
  if (!shared8_ok(cfg, shared8)) return -1;
  moe_ref_config c0 = *cfg;
  c0.n_shared = 0; /* layer->shared is not read */
  if (!layer_ok(&c0, layer, 1)) return -1;
  return per_token(cfg, layer, shared8, x, S, NULL, NULL, out, flags);
}

/* Section 11 unique-expert union for S tokens whose routing is known (the
 * first keff[s] of the K selected experts of token s take part).  Each
 * expert selected by any kept pair is visited once, in order of its first
 * appearance scanning the pairs token by token and slot by slot; its rows are
 * gathered, run through the expert together, and scattered to a staging
 * area indexed by (token, slot).  The shared expert runs once on all S
 * rows.  Each row's arithmetic is that of the per-token path, and the staged
 * rows are combined per token in the same order, so the result equals the
 * per-token path bit for bit. */
static int union_block(const moe_ref_config *cfg, const moe_ref_layer *layer,
                       const moe_ref_expert_i8 *shared8, const float *x, int S, const int32_t *idx,
                       const float *w, const int32_t *keff, float *out, unsigned flags,
                       int32_t *uniq_out, int32_t *n_uniq_out) {
  const int D = cfg->D, E = cfg->E, K = cfg->K, P = cfg->K + 1;
  int8_t *xq = (int8_t *)malloc((size_t)S * D);
  float *sx = (float *)malloc((size_t)S * sizeof(float));
  float *stage = (float *)malloc((size_t)S * P * D * sizeof(float));
  int64_t *first = (int64_t *)malloc((size_t)E * sizeof(int64_t));
  int32_t *order = (int32_t *)malloc((size_t)E * sizeof(int32_t));
  int32_t *rows = (int32_t *)malloc((size_t)S * K * sizeof(int32_t));
  int8_t *xg = NULL;
  float *sg = NULL, *yg = NULL;
  int rc = -2, nu = 0;
  if (!xq || !sx || !stage || !first || !order || !rows) goto done;
  rc = moe_ref_quant_act_i8(x, S, D, xq, sx);
  if (rc) goto done;
  /* first[e]: the first kept pair p = s*K + k that selects e (-1: none) */
  for (int e = 0; e < E; e++) first[e] = -1;
  for (int64_t p = (int64_t)S * K - 1; p >= 0; p--)
    if (p % K < keff[p / K]) first[idx[p]] = p;
  /* the selected experts ordered by first appearance (counting the pairs in
   * order, each expert at its first pair) */
  for (int64_t p = 0; p < (int64_t)S * K; p++)
    if (p % K < keff[p / K] && first[idx[p]] == p) order[nu++] = idx[p];
  for (int u = 0; u < nu && rc == 0; u++) {
    const int e = order[u];
    int nr = 0; /* the expert's kept (token, slot) pairs */
    for (int64_t p = first[e]; p < (int64_t)S * K; p++)
      if (idx[p] == e && p % K < keff[p / K]) rows[nr++] = (int32_t)p;
    xg = (int8_t *)malloc((size_t)nr * D);
    sg = (float *)malloc((size_t)nr * sizeof(float));
    yg = (float *)malloc((size_t)nr * D * sizeof(float));
    rc = (xg && sg && yg) ? 0 : -2;
    for (int r = 0; r < nr && rc == 0; r++) { /* gather */
      memcpy(xg + (int64_t)r * D, xq + (int64_t)(rows[r] / K) * D, (size_t)D);
      sg[r] = sx[rows[r] / K];
    }
    if (rc == 0)
      rc = moe_ref_expert_swiglu_i4(cfg, xg, sg, nr, &layer->experts[e], yg, NULL, NULL, NULL, NULL);
    for (int r = 0; r < nr && rc == 0; r++) { /* scatter to (token, slot) */
      const int64_t s = rows[r] / K, k = rows[r] % K;
      memcpy(stage + (s * P + k) * D, yg + (int64_t)r * D, (size_t)D * sizeof(float));
    }
    free(xg); free(sg); free(yg);
    xg = NULL; sg = NULL; yg = NULL;
  }
  if (rc == 0 && cfg->n_shared == 1) {
    /* staged in place: row s of the shared expert's output is (s, K) */
    float *ys = (float *)malloc((size_t)S * D * sizeof(float));
    rc = ys ? shared_rows(cfg, layer, shared8, xq, sx, S, ys) : -2;
    for (int s = 0; s < S && rc == 0; s++)
      memcpy(stage + ((int64_t)s * P + K) * D, ys + (int64_t)s * D, (size_t)D * sizeof(float));
    free(ys);
  }
  if (rc == 0)
    for (int s = 0; s < S; s++)
      combine_row(cfg, w + (int64_t)s * K, keff[s], stage + (int64_t)s * P * D,
                  out + (int64_t)s * D, flags);
  if (rc == 0) {
    if (uniq_out) memcpy(uniq_out, order, (size_t)nu * sizeof(int32_t));
    if (n_uniq_out) *n_uniq_out = nu;
  }
done:
  free(xq); free(sx); free(stage); free(first); free(order); free(rows);
  return rc;
}

/* The union path with the router: route all S tokens (section 11 routes
 * before it forms the union), keff per token, then union_block. */
static int routed_union(const moe_ref_config *cfg, const moe_ref_layer *layer,
                        const moe_ref_expert_i8 *shared8, const float *x, int S, float *out,
                        unsigned flags, int32_t *idx_out, float *w_out, int32_t *uniq_out,
                        int32_t *n_uniq_out) {
  if (!x || !out || S < 1) return -1;
  const int K = cfg->K;
  int32_t *idx = (int32_t *)malloc((size_t)S * K * sizeof(int32_t));
  float *w = (float *)malloc((size_t)S * K * sizeof(float));
  int32_t *keff = (int32_t *)malloc((size_t)S * sizeof(int32_t));
  int rc = (idx && w && keff) ? 0 : -2;
  if (rc == 0) rc = moe_ref_router_topk(cfg, x, S, layer->router_w, layer->router_b, idx, w, NULL, NULL);
  for (int s = 0; s < S && rc == 0; s++)
    keff[s] = moe_ref_expert_keff(w + (int64_t)s * K, K, cfg->expert_topp);
  if (rc == 0) rc = union_block(cfg, layer, shared8, x, S, idx, w, keff, out, flags, uniq_out, n_uniq_out);
  if (rc == 0) {
    if (idx_out) memcpy(idx_out, idx, (size_t)S * K * sizeof(int32_t));
    if (w_out) memcpy(w_out, w, (size_t)S * K * sizeof(float));
  }
  free(idx);
  free(w);
  free(keff);
  return rc;
}

int moe_ref_layer_forward_batch(const moe_ref_config *cfg, const moe_ref_layer *layer,
                                const float *x, int S, float *out, unsigned flags, int32_t *idx_out,
                                float *w_out, int32_t *uniq_out, int32_t *n_uniq_out) {
  if (!layer_ok(cfg, layer, 1)) return -1;
  return routed_union(cfg, layer, NULL, x, S, out, flags, idx_out, w_out, uniq_out, n_uniq_out);
}

int moe_ref_layer_forward_batch_shared_i8(const moe_ref_config *cfg, const moe_ref_layer *layer,
                                          const moe_ref_expert_i8 *shared8, const float *x, int S,
                                          float *out, unsigned flags, int32_t *uniq_out,
                                          int32_t *n_uniq_out) {
  if (!shared8_ok(cfg, shared8)) return -1;
  moe_ref_config c0 = *cfg;
  c0.n_shared = 0;
  if (!layer_ok(&c0, layer, 1)) return -1;
  return routed_union(cfg, layer, shared8, x, S, out, flags, NULL, NULL, uniq_out, n_uniq_out);
}

int moe_ref_layer_forward_batch_routed(const moe_ref_config *cfg, const moe_ref_layer *layer,
                                       const float *x, int S, const int32_t *idx, const float *w,
                                       float *out, unsigned flags, int32_t *uniq_out,
                                       int32_t *n_uniq_out) {
  if (!layer_ok(cfg, layer, 0) || !x || !out || S < 1 || !routing_ok(cfg, idx, w, S)) return -1;
  int32_t *keff = (int32_t *)malloc((size_t)S * sizeof(int32_t));
  if (!keff) return -2;
  for (int s = 0; s < S; s++) keff[s] = cfg->K;
  const int rc = union_block(cfg, layer, NULL, x, S, idx, w, keff, out, flags, uniq_out, n_uniq_out);
  free(keff);
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

/* The slot holding eid among the n_used filled ones, or -1. */
static int cache_lookup(const int32_t *slot_eid, int n_used, int32_t eid) {
  for (int z = 0; z < n_used; z++)
    if (slot_eid[z] == eid) return z;
  return -1;
}

/* Where a missing expert goes: the next unfilled slot while there is one,
 * else the least recently used slot (the smallest use value, the lowest slot
 * among equals). */
static int cache_victim(const uint64_t *slot_used, int n_used, int cap) {
  if (n_used < cap) return n_used;
  int v = 0;
  for (int z = 1; z < n_used; z++)
    if (slot_used[z] < slot_used[v]) v = z;
  return v;
}

int moe_ref_expert_get(int32_t *slot_eid, uint64_t *slot_used, int cap, int *n_used,
                       uint64_t *clock, uint64_t *hits, uint64_t *misses, int32_t eid,
                       int *loaded) {
  if (!slot_eid || !slot_used || !n_used || !clock || !hits || !misses || !loaded) return -1;
  if (cap < 1 || *n_used < 0 || *n_used > cap) return -1;
  int z = cache_lookup(slot_eid, *n_used, eid);
  *loaded = z < 0;
  if (z >= 0) {
    *hits += 1;
  } else {
    *misses += 1;
    z = cache_victim(slot_used, *n_used, cap);
    if (z == *n_used) *n_used += 1;
    slot_eid[z] = eid;
  }
  /* every use, hit or load, stamps the slot with the next clock value */
  *clock += 1;
  slot_used[z] = *clock;
  return z;
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
