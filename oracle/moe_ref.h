/*
 * moe_ref.h -- CPU oracle for the routed-expert int4 MoE block.
 *
 * TEST INFRASTRUCTURE ONLY.  This is a plain, slow, single-threaded C model of
 * what the block computes, used to check the GPU library.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it; the product
 * library never calls it and shares no code with it.
 *
 * Source: the reader.mx article "惊呆了！25GB 内存上运行 GLM 5.2 744B 模型"
 * (called "the article" below), whose listings define every step:
 *   - section 04 (RMSNorm, SiLU, layer order),
 *   - section 05 (per-row absmax quantization to int8, the expert cache's
 *     int8 weight format),
 *   - section 06 (per-row int4 quantization and nibble packing; the packed
 *     int2 layout below is a reading of the same rule at 2 bits, parity with
 *     the article unpinned),
 *   - section 09 (MLA decode attention with weight absorption, the step
 *     after the MoE block),
 *   - section 11 (sigmoid router with correction bias, top-K, unique-expert
 *     union, SwiGLU expert, weighted scatter),
 *   - the summaries' "Q8_0 style" activation remark (block-32 scales below,
 *     a reading; parity with the article unpinned),
 *   - section 12 (per-row int8 activation quantization; integer dot products
 *     scaled by the weight and activation scales; activations are quantized in
 *     front of every integer matmul).
 * Readings of points the article leaves open are stated next to the function
 * that takes them.
 *
 * All pointers are host pointers.  Matrices are row-major.  A packed int4
 * matrix with O rows and C columns is q4[O][(C+1)/2] bytes plus scale[O];
 * byte j of a row holds column 2j in its low nibble and column 2j+1 in its high
 * nibble, each stored as q + 8.
 *
 * Functions return 0 on success and a negative value on invalid arguments.
 */
#ifndef MOE_REF_H
#define MOE_REF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t D;          /* hidden size */
  int32_t I;          /* expert intermediate size */
  int32_t E;          /* routed experts */
  int32_t K;          /* experts per token */
  int32_t n_shared;   /* 0 or 1 shared expert */
  float routed_scale; /* routed scaling factor (2.5 for the GLM shape) */
  float expert_topp;  /* adaptive expert top-p in (0, 1); 0 or 1 = all K experts */
} moe_ref_config;

typedef struct {
  const uint8_t *q4;  /* [O][(C+1)/2] */
  const float *scale; /* [O] */
} moe_ref_qmat;

typedef struct {
  moe_ref_qmat gate; /* O = I, C = D */
  moe_ref_qmat up;   /* O = I, C = D */
  moe_ref_qmat down; /* O = D, C = I */
} moe_ref_expert;

typedef struct {
  const float *router_w;         /* [E][D] */
  const float *router_b;         /* [E] correction bias */
  const moe_ref_expert *experts; /* [E]; an entry may hold NULLs if never selected */
  const moe_ref_expert *shared;  /* used when n_shared == 1 */
} moe_ref_layer;

enum { MOE_REF_ACCUMULATE = 1 };

/* Section 06: per-row symmetric int4 quantization, s = max(amax/7, 1e-8),
 * q = clamp(lrint(w/s), -8, 7), two nibbles per byte as q+8, even column in
 * the low nibble.  An odd last column is padded with nibble 8 (value 0). */
int moe_ref_pack_int4(const float *w, int O, int C, uint8_t *q4, float *scale);

/* Inverse of the nibble packing: q[o][c] = nibble - 8. */
int moe_ref_unpack_int4(const uint8_t *q4, int O, int C, int8_t *q);

/* Section 12: per-row int8 activation quantization of n floats,
 * s = max(amax/127, 1e-12), q = lrint(x * (1/s)).  Returns s. */
float moe_ref_quant_row_i8(const float *x, int n, int8_t *q);

/* Row-wise quantization of x[S][D] (f32) or of bf16 bit patterns widened to
 * f32 exactly (section 08 widens bf16 by a 16-bit shift). */
int moe_ref_quant_act_i8(const float *x, int S, int D, int8_t *xq, float *sx);
int moe_ref_quant_act_i8_bf16(const uint16_t *x, int S, int D, int8_t *xq, float *sx);

/* Exact integer dot of one packed int4 row of C columns with C int8 values. */
int32_t moe_ref_dot_i4_i8(const uint8_t *q4row, const int8_t *x, int C);

/* Section 11 router for S tokens: logits[s][e] = x[s] . W[e] (accumulated in
 * double, rounded once to float), sig = 1/(1+exp(-logit)), choice = sig + b;
 * K passes pick the largest choice not yet taken (strict >, experts scanned in
 * ascending order, so ties go to the lowest index); weight = sig * scale.
 * Outputs: idx[S][K], w[S][K]; logits[S][E] and choice[S][E] are optional. */
int moe_ref_router_topk(const moe_ref_config *cfg, const float *x, int S, const float *router_w,
                        const float *router_b, int32_t *idx, float *w, float *logits,
                        float *choice);

/* One SwiGLU expert applied to S quantized rows (sections 11 and 12).
 * y[S][D] is the unweighted expert output.  Optional outputs: acc_gu[S][2][I]
 * (gate then up int32 accumulators), hq[S][I] and sh[S] (requantized SwiGLU
 * output), acc_d[S][D] (down-projection int32 accumulators). */
int moe_ref_expert_swiglu_i4(const moe_ref_config *cfg, const int8_t *xq, const float *sx, int S,
                             const moe_ref_expert *e, float *y, int32_t *acc_gu, int8_t *hq,
                             float *sh, int32_t *acc_d);

/* Section 05 (the expert cache's per-row absmax quantizer, one int8 per
 * value): qmax = 2^(bits-1) - 1 for bits in 2..8, s = max(amax/qmax, 1e-8),
 * q = clamp(lrint(w/s), -qmax-1, qmax), w divided by s as in the article.
 * bits = 8 gives the article's int8 expert format; bits = 4 gives the codes
 * that moe_ref_pack_int4 packs. */
int moe_ref_quantize_rows(const float *w, int O, int C, int bits, int8_t *q, float *scale);

/* Exact integer dot of two int8 rows of C values (section 12 dot_i8i8: its
 * sign folding is exact, so the result is the plain sum of products). */
int32_t moe_ref_dot_i8_i8(const int8_t *w, const int8_t *x, int C);

typedef struct {
  const int8_t *q;    /* [O][C] */
  const float *scale; /* [O] */
} moe_ref_q8mat;

typedef struct {
  moe_ref_q8mat gate; /* O = I, C = D */
  moe_ref_q8mat up;   /* O = I, C = D */
  moe_ref_q8mat down; /* O = D, C = I */
} moe_ref_expert_i8;

/* moe_ref_expert_swiglu_i4 with int8 weight rows (section 12's integer path
 * for the int8 format: int8 weights times int8 activation codes, the int32
 * sum scaled by the weight row scale, then by the activation scale).  Same
 * outputs and optional probes. */
int moe_ref_expert_swiglu_i8(const moe_ref_config *cfg, const int8_t *xq, const float *sx, int S,
                             const moe_ref_expert_i8 *e, float *y, int32_t *acc_gu, int8_t *hq,
                             float *sh, int32_t *acc_d);

/* Packed int2 weights (the article's 2-bit format; its section 12 keeps an
 * int2 path beside int8 and int4, and its summary lists packed int2 with
 * per-row scales).  The article gives no int2 byte layout.  Reading, the
 * int4 container's rule at 2 bits: codes from moe_ref_quantize_rows with
 * bits = 2 (values in [-2, 1]), four per byte, each stored as q + 2, column
 * 4j + k in bits 2k..2k+1 of byte j.  A row of C columns takes (C+3)/4
 * bytes; missing columns of the last byte hold 2 (value 0). */
int moe_ref_pack_int2(const float *w, int O, int C, uint8_t *q2, float *scale);
int moe_ref_unpack_int2(const uint8_t *q2, int O, int C, int8_t *q);

typedef struct {
  moe_ref_qmat gate; /* q4 field holds the packed int2 rows: O = I, C = D */
  moe_ref_qmat up;
  moe_ref_qmat down; /* O = D, C = I */
} moe_ref_expert_i2;

/* moe_ref_expert_swiglu_i8 with packed int2 weight rows (each code unpacked,
 * then the same integer path).  Same outputs and optional probes. */
int moe_ref_expert_swiglu_i2(const moe_ref_config *cfg, const int8_t *xq, const float *sx, int S,
                             const moe_ref_expert_i2 *e, float *y, int32_t *acc_gu, int8_t *hq,
                             float *sh, int32_t *acc_d);

/* Block-32 activation scales (the summaries call the activation format
 * "Q8_0 style", a format with one scale per 32 values; the section 12 listing
 * itself scales whole rows).  Reading: each run of 32 values of a row is
 * quantized like a section 12 row, s = max(amax/127, 1e-12),
 * q = lrint(x * (1/s)).  D % 32 == 0.  Outputs xq[S][D], sxb[S][D/32]. */
int moe_ref_quant_act_b32(const float *x, int S, int D, int8_t *xq, float *sxb);

/* One int4 SwiGLU expert on block-32 quantized rows: for each output row,
 * acc_b = sum over block b of q_w * q_x (exact int32), the matmul value is
 * s_w * sum_b acc_b * s_b (in double, rounded once to float); h = silu(g) * u
 * in float; h is requantized in blocks of 32 the same way (hq[S][I],
 * shb[S][I/32], both optional outputs) and the down projection is formed the
 * same way.  y[S][D] is the unweighted expert output. */
int moe_ref_expert_swiglu_i4_b32(const moe_ref_config *cfg, const int8_t *xq, const float *sxb,
                                 int S, const moe_ref_expert *e, float *y, int8_t *hq,
                                 float *shb);

/* Section 09 MLA decode attention with weight absorption.  The cache keeps
 * per token a latent row L[t][kvl] and a rotary key R[t][rope] shared by all
 * heads.  kv_b holds, per head h, nope rows (key up-projection) and then
 * vdim rows (value up-projection) of kvl columns: rows h*(nope+vdim) + d.
 * For query s, head h (q[s][h] = nope values, then rope values):
 *   qabs[i]  = sum_d q_nope[d] * kv_b[h, d][i]          (key absorbed into q)
 *   score[t] = (sum_i qabs[i] L[t][i] + sum_d q_rope[d] R[t][d]) * scale
 *   p        = softmax(score) over the visible rows
 *   clat[i]  = sum_t p[t] L[t][i]
 *   ctx[s][h][v] = sum_i kv_b[h, nope + v][i] * clat[i]  (value absorbed after)
 * Visible rows (reading: the S queries are the last S cache rows, in order,
 * each seeing itself and everything before it): t < T - S + 1 + s.
 * All arithmetic in double, each output rounded once to float. */
typedef struct {
  int32_t H, kvl, nope, rope, vdim;
  float scale;
} moe_ref_mla_config;

int moe_ref_mla_decode(const moe_ref_mla_config *c, const float *q, int S, const float *kv_b,
                       const float *L, const float *R, int T, float *ctx);

/* The block for S tokens, one token at a time: route, quantize the token,
 * run its K experts and the shared expert, and combine
 * out = sum_k w_k * y_k (k ascending, from 0) + y_shared.
 * With MOE_REF_ACCUMULATE the result is added to out (residual). */
int moe_ref_layer_forward(const moe_ref_config *cfg, const moe_ref_layer *layer, const float *x,
                          int S, float *out, unsigned flags);

/* moe_ref_layer_forward with the shared expert in the int8 format (the
 * article keeps the shared experts at higher precision than the routed ones:
 * they belong to its quantization-sensitive dense class).  cfg->n_shared must
 * be 1; layer->shared is not read. */
int moe_ref_layer_forward_shared_i8(const moe_ref_config *cfg, const moe_ref_layer *layer,
                                    const moe_ref_expert_i8 *shared8, const float *x, int S,
                                    float *out, unsigned flags);

/* Same block through the section 11 unique-expert union: the experts selected
 * by any token are visited once each in order of first appearance, each one
 * applied to all its rows; per-(token, slot) results are staged and combined
 * in the same order as layer_forward, so the two agree bit for bit.
 * Optional outputs: idx[S][K], w[S][K], uniq[E] and n_uniq. */
int moe_ref_layer_forward_batch(const moe_ref_config *cfg, const moe_ref_layer *layer,
                                const float *x, int S, float *out, unsigned flags, int32_t *idx,
                                float *w, int32_t *uniq, int32_t *n_uniq);

/* The per-token block with the routing given instead of the router's
 * (section 11 routes first and runs the experts after; section 13 fetches the
 * selected experts in between): idx[S][K] in [0, E) and w[S][K]; all K
 * experts of every token run (expert_topp does not apply); router_w and
 * router_b are not read.  Fed the routing moe_ref_router_topk selects, it
 * returns moe_ref_layer_forward's bits. */
int moe_ref_layer_forward_routed(const moe_ref_config *cfg, const moe_ref_layer *layer,
                                 const float *x, int S, const int32_t *idx, const float *w,
                                 float *out, unsigned flags);

/* The unique-expert union with the routing given, as
 * moe_ref_layer_forward_routed is to moe_ref_layer_forward.  A token may name
 * an expert more than once; each (token, slot) pair is then a row of its own.
 * Optional outputs uniq[E] (first-appearance order) and n_uniq. */
int moe_ref_layer_forward_batch_routed(const moe_ref_config *cfg, const moe_ref_layer *layer,
                                       const float *x, int S, const int32_t *idx, const float *w,
                                       float *out, unsigned flags, int32_t *uniq,
                                       int32_t *n_uniq);

/* The unique-expert union with the shared expert in the int8 format: the
 * union of moe_ref_layer_forward_batch for the routed experts, the int8
 * shared expert read once for all S rows, the per-token combine; equal bit
 * for bit to moe_ref_layer_forward_shared_i8.  cfg->n_shared must be 1. */
int moe_ref_layer_forward_batch_shared_i8(const moe_ref_config *cfg, const moe_ref_layer *layer,
                                          const moe_ref_expert_i8 *shared8, const float *x, int S,
                                          float *out, unsigned flags, int32_t *uniq,
                                          int32_t *n_uniq);

/* Section 04 RMSNorm: ms = mean of squares in double, r = 1/sqrtf(ms + eps),
 * y = x * r * gamma. */
int moe_ref_rmsnorm(const float *x, const float *gamma, int S, int D, float eps, float *y);

/* Adaptive expert top-p (section 11 runs keff[s] experts per token; the
 * article's --topp option, its reduced-reads figures in the summary pages).
 * The article gives no formula; reading: keff is the smallest k in 1..K
 * whose running sum w[0] + ... + w[k-1] (float32, in selection order) reaches
 * p * (w[0] + ... + w[K-1]) (float32 total in the same order, one float32
 * product); p <= 0 or p >= 1 keeps all K.  The kept experts keep their
 * weights (no renormalization, as in the section 11 listing).  The tests pin
 * this function to the rule as stated; the rule itself is a reading, so its
 * parity with the article is unpinned. */
int moe_ref_expert_keff(const float *w, int K, float p);

/* Section 05 per-layer expert cache, one lookup (the article's expert_get):
 * the layer's cache has cap slots, of which *n_used are filled; slot_eid[z]
 * is the expert held by slot z and slot_used[z] the clock value of its last
 * use.  A held expert is a hit: its slot gets the next clock value.  Else it
 * is a miss: the next unused slot if any, otherwise the slot with the
 * smallest use value found first scanning from slot 0, gets the expert and
 * the next clock value.  *clock, *hits and *misses are the counters the
 * article keeps in its model (shared by all layers).  Returns the slot and
 * sets *loaded to 1 for a miss, 0 for a hit. */
int moe_ref_expert_get(int32_t *slot_eid, uint64_t *slot_used, int cap, int *n_used,
                       uint64_t *clock, uint64_t *hits, uint64_t *misses, int32_t eid,
                       int *loaded);

/* Section 13 swap decision for the pinned tier: the coldest pinned expert (by
 * heat, first of equals) against the hottest expert not pinned (first of
 * equals; heat must exceed 0).  Swap when the newcomer's heat exceeds
 * fc + fc/4 + 4 (fc = the coldest one's heat, fc/4 rounded down).  Reading:
 * that bound is evaluated without wrap-around (the article's listing adds in
 * 32 bits; heats that large never occur in a run).  Returns 1 with the pinned
 * position, the expert and the heat gain, else 0. */
int moe_ref_tier_pick_swap(const uint32_t *heat, int nexpert, const int32_t *pinned, int npin,
                           int32_t *slot, int32_t *eid, int64_t *gain);

/* Section 13 frequency-first score: (heat << 8) | recent, recent = 255 - age
 * for age = clock - last below 255, else 0 (unsigned 32-bit age). */
uint64_t moe_ref_tier_lfru_score(uint32_t heat, uint32_t last, uint32_t clock);

#ifdef __cplusplus
}
#endif

#endif /* MOE_REF_H */
