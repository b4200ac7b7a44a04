/*
 * moe_i4.h -- C ABI of the MI355X (gfx950) routed-expert int4 MoE block.
 *
 * The block is the one described by the reader.mx article "惊呆了！25GB 内存上
 * 运行 GLM 5.2 744B 模型" (cited below as "the article"):
 *   - section 02: the GLM-5.2 shape (hidden 6144, 256 routed experts, top-8,
 *     one shared expert, expert intermediate size 2048, sigmoid scoring,
 *     routed scaling factor 2.5);
 *   - section 06: the int4 weight container (per-row symmetric scale
 *     amax/7, values clamped to [-8, 7], two per byte as value+8, even column
 *     in the low nibble, one float scale per row);
 *   - section 11: the router (sigmoid of the logits plus a correction bias
 *     picks the top K experts; the weight is the unbiased sigmoid times the
 *     routed scaling factor), the SwiGLU expert, and the unique-expert union
 *     used to run a batch of tokens with each selected expert read once;
 *   - section 12: per-row int8 activation quantization (scale amax/127,
 *     floored at 1e-12, round half to even) in front of every integer matmul,
 *     integer dot products rescaled by the weight and activation scales;
 *   - beside the int4 block: the section 05 int8 weight format, a packed int2
 *     format, block-32 activation scales (one SwiGLU expert each) and the
 *     section 09 MLA decode attention with weight absorption.
 *
 * Conventions
 *   - Every pointer is a DEVICE pointer unless its comment says "host".
 *   - Matrices are row-major.  A packed int4 matrix with O rows and C columns
 *     is q4[O][C/2] bytes plus scale[O] floats.
 *   - All calls are asynchronous on the given HIP stream and return a
 *     moe_status.  Arguments are validated on the host before anything is
 *     enqueued; an invalid call enqueues nothing.  No call allocates, frees or
 *     keeps device memory: scratch space comes from the caller's workspace
 *     (moe_layer_forward_noalloc: from a library-held array, see there).
 *   - A workspace holds only values written and read within one call: its
 *     contents before a call do not matter (no zero fill is needed) and are
 *     undefined after it.  Calls that share one workspace must not overlap
 *     (use one workspace per concurrent stream).
 *   - Shape limits: D a multiple of 256 (the router's lane order), I a
 *     multiple of 32, D/2 and I/2 at most 4096 bytes per packed row,
 *     1 <= K <= E <= 1024, K <= 64, n_shared 0 or 1, S >= 1 (MOE_ESHAPE
 *     otherwise).  q4, scale and activation buffers must be 16-byte aligned.
 *     The device must be a gfx950.
 */
#ifndef MOE_I4_H
#define MOE_I4_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,     /* null pointer or bad scalar argument */
  MOE_ESHAPE = -2,     /* shape outside the supported limits */
  MOE_EALIGN = -3,     /* a buffer is not 16-byte aligned */
  MOE_EWORKSPACE = -4, /* workspace too small */
  MOE_EHIP = -5,       /* a HIP launch or runtime call failed */
  MOE_EDEVICE = -6     /* current device is not a gfx950 */
} moe_status;

/* Element types of activation inputs (passed as int: any other value is
 * refused with MOE_EINVAL). */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Flags of the layer calls. */
#define MOE_F_ACCUMULATE 1u /* out += block(x) instead of out = block(x) */
/* The block's input is RMSNorm(x) with layer->norm_gamma and norm_eps
 * (section 04 RMSNorm, the same bits as moe_rmsnorm) instead of x.  With
 * MOE_F_ACCUMULATE and out == x this is one decoder-layer update
 * x <- x + block(rmsnorm(x)) in place.  Needs D % 4 == 0, D <= 8192 and
 * 16-byte aligned x and gamma (MOE_EALIGN otherwise). */
#define MOE_F_PRENORM 2u
/* x holds bf16 values (uint16 bit patterns, [S][D], 16-byte aligned) instead
 * of float32.  Section 08 reads bf16 tensors by widening them to float32; the
 * widening is exact (a bf16 value is the top 16 bits of its float32), and the
 * router and the section 12 quantization do it as they load, so the call
 * returns the bits it returns for the widened float32 rows while x costs half
 * the bytes.  Union-path calls only (moe_layer_forward_batch,
 * moe_layer_forward_batch_routed), not with MOE_F_PRENORM; MOE_EINVAL
 * otherwise. */
#define MOE_F_X_BF16 4u

typedef struct {
  int32_t D;          /* hidden size (6144 for the GLM shape) */
  int32_t I;          /* expert intermediate size (2048) */
  int32_t E;          /* routed experts (256) */
  int32_t K;          /* experts per token (8) */
  int32_t n_shared;   /* shared experts, 0 or 1 */
  float routed_scale; /* routed scaling factor (2.5) */
  /* Adaptive expert top-p (section 11 runs keff[s] experts per token).  In
   * (0, 1): token s keeps its first keff selected experts, keff the smallest
   * k in 1..K whose float32 running weight sum (selection order) reaches
   * expert_topp * the float32 sum of its K weights; the kept experts keep
   * their weights.  0 or 1: all K experts.  Other values: MOE_EINVAL.
   * moe_layer_forward_routed always runs all K given experts. */
  float expert_topp;
} moe_config;

/* One packed int4 matrix per expert, stacked over experts.  Expert e's matrix
 * starts at q4 + e*q4_stride bytes and its scales at scale + e*scale_stride
 * floats.  A stride of 0 means densely stacked (O*C/2 bytes, O floats), so
 * e.g. gate.q4 may point at a [E][I][D/2] array.  Non-zero strides allow the
 * article's section 13 slab layout (gate, up and down of one expert adjacent). */
typedef struct {
  const uint8_t *q4;
  const float *scale;
  int64_t q4_stride;
  int64_t scale_stride;
} moe_qmat;

typedef struct {
  moe_qmat gate; /* O = I, C = D */
  moe_qmat up;   /* O = I, C = D */
  moe_qmat down; /* O = D, C = I */
} moe_experts;

typedef struct {
  const float *router_w; /* [E][D] float32 */
  const float *router_b; /* [E] float32 correction bias */
  moe_experts routed;    /* E experts */
  moe_experts shared;    /* one expert; read only when n_shared == 1 */
  const float *norm_gamma; /* [D] RMSNorm gain; read only with MOE_F_PRENORM */
  float norm_eps;          /* RMSNorm epsilon (> 0); read only with MOE_F_PRENORM */
} moe_layer;

/* Optional outputs of the layer calls (host struct; any member may be NULL). */
typedef struct {
  int32_t *topk_idx;    /* [S][K] experts chosen for each token, in selection order */
  float *topk_w;        /* [S][K] their weights */
  /* If both events of a pair are set they time that kernel.  moe_layer_forward
   * launches its gate/up kernel (routed gate/up + shared down) and its down
   * kernel(s) with hipExtLaunchKernel, so the events take the kernels' own
   * start and end timestamps; moe_layer_forward_batch records them on the
   * stream around its grouped gate/up and grouped down kernels. */
  hipEvent_t ev_gateup[2];
  hipEvent_t ev_down[2];
  int32_t *keff;        /* [S] experts kept per token (K unless expert_topp is in (0, 1)) */
} moe_probe;

/* The article's int8 weight format (section 05: the expert cache holds each
 * matrix as one int8 code per weight plus one float scale per row; section 12
 * runs it on the integer path).  One int8 matrix per expert, stacked over
 * experts: expert e's codes q[O][C] start at q + e*q_stride bytes and its
 * scales at scale + e*scale_stride floats; a stride of 0 means densely
 * stacked (O*C bytes, O floats).  q and q_stride must be 16-byte aligned. */
typedef struct {
  const int8_t *q;
  const float *scale;
  int64_t q_stride;
  int64_t scale_stride;
} moe_q8mat;

typedef struct {
  moe_q8mat gate; /* O = I, C = D */
  moe_q8mat up;   /* O = I, C = D */
  moe_q8mat down; /* O = D, C = I */
} moe_experts_i8;

/* Human-readable name of a status code (static string). */
const char *moe_status_str(int status);

/* Workspace bytes needed by a call with S tokens.  which: 0 = moe_layer_forward,
 * 1 = moe_layer_forward_batch, 2 = moe_expert_swiglu_i4, 3 = moe_router_topk,
 * 4 = moe_expert_swiglu_i8, moe_expert_swiglu_i2 and moe_expert_swiglu_i4_b32,
 * 5 = moe_layer_forward_shared_i8 (0 unless n_shared == 1).
 * Returns 0 for invalid arguments. */
size_t moe_workspace_bytes(const moe_config *cfg, int S, int which);

/* Zero-fill a workspace.  Not needed by any call (a workspace's contents
 * before a call do not matter); kept for callers that want defined memory. */
int moe_workspace_init(void *ws, size_t ws_bytes, hipStream_t stream);

/* Section 06 converter: quantize w[O][C] (float32) to the int4 container,
 * q4[O][C/2] and scale[O].  C must be even.  Bit-exact with the article's
 * packer (division by the scale, round half to even, clamp to [-8, 7]). */
int moe_pack_int4(const float *w, int O, int C, uint8_t *q4, float *scale, hipStream_t stream);

/* Section 05 per-row weight quantization to int8 codes: for each row of
 * w[O][C] (float32), s = max(amax/127, 1e-8), q = clamp(rint(w/s), -128, 127)
 * (division by the scale, round half to even, as the article's quantizer
 * does with bits = 8).  Outputs q[O][C] and scale[O].  Any C >= 1; w and
 * scale 4-byte aligned.  Bit-exact with the article's quantizer. */
int moe_quantize_rows_i8(const float *w, int O, int C, int8_t *q, float *scale,
                         hipStream_t stream);

/* Section 12: per-row int8 quantization of x[S][D] (float32, or bf16 widened
 * exactly).  Outputs xq[S][D] and sx[S].  D must be a multiple of 8. */
int moe_quant_act_i8(const void *x, int dtype, int S, int D, int8_t *xq, float *sx,
                     hipStream_t stream);

/* Section 11 router for S tokens x[S][D]: logits = x . router_w^T in float32,
 * sig = 1/(1+exp(-logit)), choice = sig + router_b; K passes take the largest
 * choice not yet taken (ties to the lowest expert index; NaN choices and
 * choices <= -1e30 are never taken unless fewer than K candidates remain, in
 * which case the lowest untaken indices fill the rest).  Outputs
 * topk_idx[S][K] (selection order) and topk_w[S][K] = routed_scale * sig;
 * logits[S][E] is optional (NULL to skip).  D must be a multiple of 256. */
int moe_router_topk(const moe_config *cfg, const float *x, int S, const float *router_w,
                    const float *router_b, int32_t *topk_idx, float *topk_w, float *logits,
                    void *ws, size_t ws_bytes, hipStream_t stream);

/* One SwiGLU expert (sections 11 and 12) on S already-quantized rows
 * xq[S][D], sx[S]: g = (acc_g * s_g) * s_x, u likewise, h = silu(g) * u,
 * h requantized per row to (hq, sh), y = (acc_d * s_d) * sh.  The expert is
 * number `expert` of the stacked matrices in *w (host struct).  Outputs
 * y[S][D] (unweighted); optional integer probes acc_gu[S][2][I] (gate then
 * up), hq[S][I], sh[S], acc_d[S][D]. */
int moe_expert_swiglu_i4(const moe_config *cfg, const int8_t *xq, const float *sx, int S,
                         const moe_experts *w, int expert, float *y, int32_t *acc_gu, int8_t *hq,
                         float *sh, int32_t *acc_d, void *ws, size_t ws_bytes, hipStream_t stream);

/* moe_expert_swiglu_i4 for an expert in the int8 format (*w, host struct):
 * gate/up sums acc = sum_c q[o][c] * xq[s][c] over int8 weight codes, then
 * g = (acc_g * s_g) * s_x, u likewise, h = silu(g) * u, h requantized per
 * row (section 12, as for the int4 format), y = (acc_d * s_d) * sh.  Same
 * outputs and probes as moe_expert_swiglu_i4; xq and hq (if given) must be
 * 16-byte aligned.  Workspace: moe_workspace_bytes(cfg, S, 4). */
int moe_expert_swiglu_i8(const moe_config *cfg, const int8_t *xq, const float *sx, int S,
                         const moe_experts_i8 *w, int expert, float *y, int32_t *acc_gu,
                         int8_t *hq, float *sh, int32_t *acc_d, void *ws, size_t ws_bytes,
                         hipStream_t stream);

/* Packed int2 weights (section 12 keeps a 2-bit integer path beside int8
 * and int4; the summaries list packed int2 with per-row scales).  The
 * article gives no int2 byte layout; this library carries the section 06
 * int4 rule to 2 bits: per row s = max(amax, 1e-8) (amax/qmax, qmax = 1),
 * q = clamp(rint(w/s), -2, 1), four codes per byte, each stored as q + 2,
 * column 4j + k in bits 2k..2k+1 of byte j; a row of C columns takes
 * (C+3)/4 bytes, missing columns of its last byte hold 2 (value 0).
 * moe_pack_int2 converts w[O][C] (float32) to q2[O][(C+3)/4] and scale[O];
 * any C >= 1; w and scale 4-byte aligned. */
int moe_pack_int2(const float *w, int O, int C, uint8_t *q2, float *scale, hipStream_t stream);

/* moe_expert_swiglu_i8 for an expert in the packed int2 format: *w (host
 * struct) holds packed int2 rows in the q4 fields (gate/up [I][D/4], down
 * [D][I/4]; a stride of 0 means densely stacked, O*C/4 bytes per expert).
 * Needs I % 64 == 0 (MOE_ESHAPE otherwise).  Same arithmetic after the codes
 * are unpacked, same outputs and probes.  Workspace:
 * moe_workspace_bytes(cfg, S, 4). */
int moe_expert_swiglu_i2(const moe_config *cfg, const int8_t *xq, const float *sx, int S,
                         const moe_experts *w, int expert, float *y, int32_t *acc_gu, int8_t *hq,
                         float *sh, int32_t *acc_d, void *ws, size_t ws_bytes, hipStream_t stream);

/* Block-32 activation scales (the summaries call the activation format
 * "Q8_0 style", one scale per 32 values; the section 12 listing scales whole
 * rows).  moe_quant_act_b32 quantizes every run of 32 values of x[S][D]
 * (float32) like a section 12 row: s = max(amax/127, 1e-12),
 * q = rint(x * (1/s)).  Outputs xq[S][D] (natural order) and sxb[S][D/32].
 * D % 32 == 0; x and xq 16-byte aligned. */
int moe_quant_act_b32(const float *x, int S, int D, int8_t *xq, float *sxb, hipStream_t stream);

/* One int4 SwiGLU expert (packed as in moe_expert_swiglu_i4) on block-32
 * quantized rows xq[S][D], sxb[S][D/32]: each gate/up/down output is
 * s_w * sum_b acc_b * s_b over the blocks b of its row, acc_b the exact int32
 * sum of block b, the block terms added in float; h = silu(g) * u is
 * requantized in blocks of 32 the same way before the down projection.
 * Outputs y[S][D] (unweighted); optional hq[S][I] (natural order, 16-byte
 * aligned) and shb[S][I/32].  Workspace: moe_workspace_bytes(cfg, S, 4). */
int moe_expert_swiglu_i4_b32(const moe_config *cfg, const int8_t *xq, const float *sxb, int S,
                             const moe_experts *w, int expert, float *y, int8_t *hq, float *shb,
                             void *ws, size_t ws_bytes, hipStream_t stream);

/* Section 09 MLA decode attention with weight absorption (the step after the
 * MoE block in a decoder layer).  The cache keeps per token one latent row
 * L[t][kvl] and one rotary key R[t][rope] shared by all heads.  kv_b holds,
 * per head h, nope rows of the key up-projection and then vdim rows of the
 * value up-projection, kvl columns each: kv_b[h][nope + vdim][kvl].  For
 * query s and head h, with q[s][h] = (q_nope[nope], q_rope[rope]):
 * qabs = W_UK[h]^T q_nope, score[t] = (qabs . L[t] + q_rope . R[t]) * scale,
 * p = softmax(score) over the visible rows, ctx[s][h] = W_UV[h] (sum_t p[t]
 * L[t]).  The S queries are the last S cache rows, in order: query s sees
 * rows t < T - S + 1 + s.  All float32; kv_b 16-byte aligned, every other
 * pointer 4-byte aligned.
 * Limits: kvl a multiple of 64 up to 1024, rope <= 64, S <= T <= 16384
 * (MOE_ESHAPE otherwise). */
typedef struct {
  int32_t H;     /* heads (64 for the GLM shape) */
  int32_t kvl;   /* latent width (512) */
  int32_t nope;  /* non-rotary query/key dims per head (192) */
  int32_t rope;  /* rotary dims (64) */
  int32_t vdim;  /* value dims per head (256) */
  float scale;   /* score scale, e.g. 1/sqrt(nope + rope) */
} moe_mla_config;

/* Workspace bytes of moe_mla_decode for S queries over T cache rows
 * (0 for invalid arguments). */
size_t moe_mla_workspace_bytes(const moe_mla_config *cfg, int S, int T);

/* q[S][H][nope + rope], kv_b as above, L[T][kvl], R[T][rope] (may be NULL
 * when rope == 0) -> ctx[S][H][vdim].  Launches: query absorption; per
 * cache chunk (32, 64 or 128 rows) and four heads, the chunk softmax statistics
 * and weighted latent sums; the merge of the chunks; the value
 * up-projection. */
int moe_mla_decode(const moe_mla_config *cfg, const float *q, int S, const float *kv_b,
                   const float *L, const float *R, int T, float *ctx, void *ws, size_t ws_bytes,
                   hipStream_t stream);

/* moe_layer_forward with the shared expert in the int8 format (the article
 * keeps shared experts in its quantization-sensitive dense class, at higher
 * precision than the routed int4 experts): out[s] = sum_k w_k y_k + y_shared
 * with y_shared from the int8 expert *shared8 (host struct, expert 0 of its
 * stacks); layer->shared is not read.  cfg->n_shared must be 1 (MOE_ESHAPE);
 * flags: MOE_F_ACCUMULATE only (MOE_EINVAL otherwise); x 16-byte aligned.
 * With D % 2048 == 0, D <= 8192, I % 1024 == 0 and I <= 4096 (the GLM shape)
 * the int8 expert runs inside the per-token path's launches, its gate/up
 * beside the router and its down beside the routed gate/up, exactly as the
 * int4 shared expert does.  Other shapes run the launches of
 * moe_layer_forward_batch_shared_i8 (which return the same bits).  Workspace:
 * moe_workspace_bytes(cfg, S, 5). */
int moe_layer_forward_shared_i8(const moe_config *cfg, const moe_layer *layer,
                                const moe_experts_i8 *shared8, const float *x, int S, float *out,
                                unsigned flags, void *ws, size_t ws_bytes, hipStream_t stream);

/* The block, one token at a time (each token reads its own K experts):
 * route, quantize, run the K routed experts and the shared expert, and
 * combine out[s] = sum_k w_k * y_k (k in selection order, from 0) + y_shared.
 * With MOE_F_ACCUMULATE the result is added to out.  x and out must not
 * overlap, except out == x with MOE_F_PRENORM (in-place residual update;
 * the first launch then normalizes each token inside every workgroup).
 * Unknown flag bits give MOE_EINVAL.  probe is optional (host struct).
 * Launches: router + token quantization + shared gate/up; routed gate/up +
 * shared down; routed down + combine (one launch per batch of 8 slots). */
int moe_layer_forward(const moe_config *cfg, const moe_layer *layer, const float *x, int S,
                      float *out, unsigned flags, const moe_probe *probe, void *ws,
                      size_t ws_bytes, hipStream_t stream);

/* moe_layer_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The workspace is a library-held device
 * array of MOE_NOALLOC_WS_BYTES per GPU, allocated with the library's code
 * object and kept until the process ends; the call itself allocates nothing.
 * Calls whose moe_workspace_bytes(cfg, S, 0) exceeds MOE_NOALLOC_WS_BYTES
 * return MOE_EWORKSPACE (16 MiB holds a GLM-shape call of up to 128 tokens).
 * Every call on one GPU uses the same array: calls that overlap on one GPU
 * (different streams, or different host threads) race and must be
 * serialized by the caller.  Arguments, flags and results are as in
 * moe_layer_forward with no probe. */
#define MOE_NOALLOC_WS_BYTES (16u << 20)
int moe_layer_forward_noalloc(const moe_config *cfg, const moe_layer *layer, const float *x,
                              int S, float *out, unsigned flags, hipStream_t stream);

/* The same block through the unique-expert union (section 11): tokens are
 * grouped by selected expert and every selected expert's weights are read
 * once for all its tokens.  Per-(token, slot) results are staged and combined
 * in the same order as moe_layer_forward, so the two calls return identical
 * bits for the same inputs.  Flags and the x/out rule as moe_layer_forward
 * (with MOE_F_PRENORM the normalized rows go to the workspace first). */
int moe_layer_forward_batch(const moe_config *cfg, const moe_layer *layer, const float *x, int S,
                            float *out, unsigned flags, const moe_probe *probe, void *ws,
                            size_t ws_bytes, hipStream_t stream);

/* The unique-expert union (moe_layer_forward_batch) with the shared expert in
 * the int8 format, as moe_layer_forward_shared_i8 is to moe_layer_forward:
 * the routed experts are grouped and read once as in the union path, the
 * int8 expert *shared8 (host struct, expert 0 of its stacks) is read once
 * for all S tokens (its gate/up and down each one launch on the int8 matrix
 * cores, the same int32 sums as the per-token path), its results are staged
 * as the shared slot, and the per-token combine adds it last.  Returns the bits of
 * moe_layer_forward_shared_i8 for the same inputs.  cfg->n_shared must be 1
 * (MOE_ESHAPE); flags: MOE_F_ACCUMULATE only; layer->shared is not read.
 * Workspace: moe_workspace_bytes(cfg, S, 1). */
int moe_layer_forward_batch_shared_i8(const moe_config *cfg, const moe_layer *layer,
                                      const moe_experts_i8 *shared8, const float *x, int S,
                                      float *out, unsigned flags, void *ws, size_t ws_bytes,
                                      hipStream_t stream);

/* The per-token block with the routing given by the caller instead of the
 * router (section 11 computes the routing first and the experts after it;
 * section 13 fetches the selected experts between the two).  topk_idx[S][K]
 * (int32) are expert indices into layer->routed and topk_w[S][K] (float32)
 * their combine weights, both device arrays read by the call; indices outside
 * [0, E) are clamped into it, so no access leaves the expert stack.
 * layer->router_w and router_b are not read and may be NULL.  Everything else
 * (flags, x/out rule, workspace of moe_workspace_bytes(cfg, S, 0)) is as in
 * moe_layer_forward; with the routing that moe_layer_forward selects, the two
 * calls return identical bits. */
int moe_layer_forward_routed(const moe_config *cfg, const moe_layer *layer, const float *x, int S,
                             const int32_t *topk_idx, const float *topk_w, float *out,
                             unsigned flags, void *ws, size_t ws_bytes, hipStream_t stream);

/* The unique-expert union with the routing given by the caller, as
 * moe_layer_forward_routed is to moe_layer_forward: topk_idx[S][K] and
 * topk_w[S][K] (device, read by the call; indices clamped into [0, E)), all
 * K experts of every token; layer->router_w and router_b are not read.  With
 * MOE_F_PRENORM the normalized rows go to the workspace first.  With the
 * routing that moe_layer_forward_batch selects, the two calls return
 * identical bits. */
int moe_layer_forward_batch_routed(const moe_config *cfg, const moe_layer *layer, const float *x,
                                   int S, const int32_t *topk_idx, const float *topk_w, float *out,
                                   unsigned flags, void *ws, size_t ws_bytes, hipStream_t stream);

/* ---- Expert residency tiers (section 05 expert cache, section 13 tiers) ----
 * Every expert of a layer is kept as one slab, the three packed matrices
 * followed by the three scale vectors (section 13 reads an expert with a
 * single ~19 MB read for this reason); moe_slab_layout_of gives the byte
 * offsets.  A layer's routed stack in moe_experts form over such slabs uses
 * q4 = base + offset, scale = base + offset, q4_stride = bytes and
 * scale_stride = bytes / 4.  All experts live in pinned host memory
 * (hipHostMalloc); each layer has n_slots HBM slab slots.  A call's experts
 * are mapped to slots by moe_tier_map, the missing slabs are copied in by
 * moe_tier_fetch, and moe_layer_forward_routed then runs on the slot stack
 * with the routing rewritten to slot numbers. */
typedef struct {
  int64_t gate_q4, up_q4, down_q4; /* byte offsets of the packed matrices */
  int64_t gate_s, up_s, down_s;    /* byte offsets of the float32 scales */
  int64_t bytes;                   /* slab size (a multiple of 16) */
} moe_slab_layout;

/* Offsets of one expert slab for cfg's D and I (host; MOE_ESHAPE unless both
 * are multiples of 32). */
int moe_slab_layout_of(const moe_config *cfg, moe_slab_layout *out);

/* Host bookkeeping of the HBM slots of n_layers layers of n_experts experts,
 * n_slots per layer, all empty.  Returns NULL on invalid sizes or when host
 * memory runs out.  The object holds no device memory. */
typedef struct moe_tier moe_tier;
moe_tier *moe_tier_create(int n_layers, int n_experts, int n_slots);
void moe_tier_destroy(moe_tier *t);

/* As moe_tier_create, plus n_pinned heat-managed slots per layer (0 <=
 * n_pinned < n_experts; the section 13 pinned tier): slots 0 .. n_pinned-1 of
 * a layer are pinned slots, its n_lru LRU slots follow.  Every lookup of
 * moe_tier_map adds 1 to the expert's heat; a pinned expert is a hit in its
 * pinned slot before the LRU slots are searched.  moe_tier_rebalance decides
 * what the pinned slots hold. */
moe_tier *moe_tier_create_pinned(int n_layers, int n_experts, int n_lru, int n_pinned);

/* One pinned-slot change for a layer, after its calls: an empty pinned slot
 * takes the hottest expert not pinned (heat > 0, first of equals); with all
 * filled, moe_tier_pick_swap over the layer's heat and pinned experts.
 * Returns 1 with the pinned slot, the new expert and the one it replaces (-1
 * when the slot was empty) -- the caller copies the new expert's slab into the
 * slot (moe_tier_fetch) before the layer's next call -- or 0 (no change), or a
 * negative status. */
int moe_tier_rebalance(moe_tier *t, int layer, int32_t *slot, int32_t *eid, int32_t *old_eid);

/* Section 05 expert_get for each of eids[0..n) of one call, in order (host
 * arrays): a resident expert is a hit and its slot's use clock is refreshed;
 * a missing one takes the next unused slot, else the least recently used slot
 * (ties: the lowest slot), and loads[i] = 1 says its slab must be copied in
 * before the call.  slots[i] receives the slot.  With n <= n_slots (checked,
 * MOE_ESHAPE otherwise) no slot of the call is evicted by the same call.
 * Returns the number of misses, or a negative status (eids outside [0,
 * n_experts) or a bad layer: MOE_EINVAL, nothing changed). */
int moe_tier_map(moe_tier *t, int layer, const int32_t *eids, int n, int32_t *slots,
                 int32_t *loads);

/* (With pinned slots, the LRU slot numbers start at n_pinned.) */

/* Hits and misses of every moe_tier_map so far (either pointer may be NULL). */
int moe_tier_stats(const moe_tier *t, uint64_t *hits, uint64_t *misses);

/* Enqueue one host-to-device copy of slab_bytes per i with loads[i] != 0:
 * host_slabs + eids[i]*slab_bytes (pinned host memory) to hbm_slots +
 * slots[i]*slab_bytes (device).  eids, slots and loads are host arrays.  The
 * copies are ordered on stream before the work queued after them. */
int moe_tier_fetch(const void *host_slabs, void *hbm_slots, size_t slab_bytes,
                   const int32_t *eids, const int32_t *slots, const int32_t *loads, int n,
                   hipStream_t stream);

/* One call of a tiered layer, the steps above in native code: the router and
 * the K selection rounds on the device (layer->router_w, router_b), one
 * synchronization of stream to read the selection into host_idx (pinned host
 * memory, S*K int32, owned by the caller and overwritten), moe_tier_map of the
 * call's experts in order of first appearance, moe_tier_fetch of the missing
 * slabs, the routing rewritten to slot numbers and copied back, then
 * moe_layer_forward_routed (union_path = 0; ws of moe_workspace_bytes(cfg, S, 0))
 * or moe_layer_forward_batch_routed (union_path = 1; which = 1) with
 * layer->routed describing the slot stack over hbm_slots.  ws_router: a
 * workspace of moe_workspace_bytes(cfg, S, 3).  Flags: MOE_F_ACCUMULATE only.
 * *misses (optional) receives the call's misses.  The call returns after the
 * selection has been read; the rest is queued on stream.  All K experts of
 * every token are used (expert_topp does not apply). */
int moe_tier_forward(moe_tier *t, int layer_index, const moe_config *cfg, const moe_layer *layer,
                     const void *host_slabs, void *hbm_slots, size_t slab_bytes, const float *x,
                     int S, float *out, unsigned flags, int union_path, int32_t *host_idx,
                     int32_t *misses, void *ws_router, size_t ws_router_bytes, void *ws,
                     size_t ws_bytes, hipStream_t stream);

/* Section 13 swap rule for a frequency-managed tier holding pinned[0..n_pinned)
 * (host arrays, expert ids): take the coldest held expert by heat (first of
 * equals) and the hottest expert not held (first of equals, heat > 0); swap
 * only if the newcomer's heat exceeds the coldest's by more than a quarter of
 * it plus 4.  Returns 1 and the held position, the newcomer and the heat gain,
 * or 0 (no swap, or invalid arguments). */
int moe_tier_pick_swap(const uint32_t *heat, int n_experts, const int32_t *pinned, int n_pinned,
                       int32_t *slot, int32_t *eid, int64_t *gain);

/* Section 13 frequency-first score: heat in the high bits, then recency
 * (255 - age for ages below 255, else 0) so that recency only orders experts
 * of equal heat. */
uint64_t moe_tier_lfru_score(uint32_t heat, uint32_t last, uint32_t clock);

/* Section 04 RMSNorm: y = x * (1/sqrt(mean(x^2) + eps)) * gamma per row,
 * with the mean of squares accumulated in double. */
int moe_rmsnorm(const float *x, const float *gamma, int S, int D, float eps, float *y,
                hipStream_t stream);

/* Measurement reference, not part of the block: reads buf[bytes] once with
 * the library's streaming load pattern (16-byte nontemporal loads, 8 lanes
 * per 128-byte segment) and leaves one xor word per workgroup in
 * sink[moe_stream_read_sink_words()].  bytes must be a non-zero multiple of
 * 16 and buf 16-byte aligned.  Timing it on a buffer far larger than the
 * 256 MB MALL gives the device's read rate to compare the block's rates
 * with. */
int moe_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream);
int moe_stream_read_sink_words(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_I4_H */
