// moe_kernels.h -- kernel argument structs and kernel declarations.
#pragma once

#include "moe_common.h"

namespace moe {

struct QuantArgs {
  const float *xf;     // [S][D] float32, or null
  const uint16_t *xb;  // [S][D] bf16 bits, or null
  int D;
  int8_t *xq_perm;     // optional permuted output
  int8_t *xq_nat;      // optional natural-order output
  float *sx;
  int32_t *sumx;
};

struct RouterArgs {
  const float *x;      // [S][D] float32 tokens, or
  const uint16_t *xb;  // [S][D] bf16 tokens (bit patterns; then x is unused)
  const float *W;      // [E][D]
  int S, D, E;
  float *logits;       // [S][E] scratch (always written)
  float *logits_out;   // optional caller copy
  int8_t *xq_perm;     // quantization blocks write these
  float *sx;
  int32_t *sumx;
  uint32_t *amax;      // optional [S][P]: cleared by the quantization blocks
  int P;
  const float *gamma;  // optional [D] (one-token-per-block launches only): work on RMSNorm(x)
  float eps;
};

struct PrepArgs {
  const int8_t *xq;    // [S][D] natural order
  int D;
  int8_t *xq_perm;
  int32_t *sumx;
  uint32_t *amax;      // optional [S][P]: cleared
  int P;
};

struct TopkArgs {
  const float *logits;
  const float *bias;
  int S, E, K;
  float scale;
  int32_t *idx;
  float *w;
  float topp;             // adaptive expert top-p (keff per token)
  int32_t *keff;          // [S] out
};

// Per-token ("decode") path: three launches, see decode.hip.
struct DecodeArgs {
  int S, D, I, E, K, P;     // P = K + n_shared slots per token
  float scale;              // routed scaling factor
  const float *x;           // [S][D] float32 tokens (phase A)
  const float *W;           // [E][D] router
  const float *bias;        // [E]
  ExpertSet rt;             // routed stack
  ExpertSet fx;             // stack holding the fixed expert (shared, or the single expert)
  int fx_index;             // its index in fx
  int fx_slot;              // its slot number (K for the shared expert)
  const int8_t *xq;         // [S][D] permuted codes (phase B; also phase A single-expert calls)
  const float *sx;          // [S]
  const int32_t *sumx;      // [S]
  // phase A single-expert calls: xq holds natural-order codes (16-byte
  // aligned rows); the gate/up blocks permute them and form their sum
  int xq_natural;
  float *logits;            // [S][E]
  int32_t *idx;             // [S][K]
  float *w;                 // [S][K]
  float *h;                 // [S][P][I]
  float *ysh;               // [S][D] output of the fixed expert's down projection
  float *tmp;               // [S][D] running combine between slot batches
  int n_router;             // phase A: router blocks per token
  int n_quant;              // phase A: quantization blocks (one per token, column 0)
  int n_gu_fx;              // phase A: fixed-expert gate/up blocks per token
  int n_gu_rt;              // phase B: routed gate/up blocks per token
  int n_dn_fx;              // phase B: fixed-expert down blocks per token
  int n_dn;                 // phase C: down blocks per token
  int p_lo, p_hi;           // phase C: routed slots of this launch
  int c_first, c_last;      // phase C: first / last slot batch of the combine
  float *out;               // [S][D]
  unsigned flags;
  int32_t *acc_gu;          // optional [S][2][I] (single-expert calls)
  int32_t *acc_d;           // optional [S][D]
  int8_t *hq_nat;           // optional [S][I]
  float *sh_out;            // optional [S]
  const float *gamma;       // optional [D]: phase A works on RMSNorm(x) with gamma, eps
  float eps;
  int given;                // routing given by the caller: idx and w are inputs
  int fx8;                  // the fixed expert is in the int8 format: rows f8g, f8u, f8d
  RowPtr f8g, f8u, f8d;     // its int8 gate/up [I][D] and down [D][I] codes and row scales
  float topp;               // adaptive expert top-p (0: all K)
  int32_t *keff;            // [S] experts kept per token (phase B writes, C reads); null: K
};

// Grouped (unique-expert union) kernels.
struct GroupArgs {
  int32_t *idx;           // [S][K]: read, or written when with_topk
  int S, E, K, P, n_shared;
  int32_t *gcount, *goff, *pairs;
  int2 *tiles;            // optional: (group, first pair) of every tile of tile_rows pairs
  int32_t *ntiles;        // number of tiles
  int tile_rows;
  // with_topk: the kernel first runs each token's top-K rounds itself (one
  // wave per token) from logits and bias into idx and wts
  int with_topk;
  const float *logits, *bias;
  float scale;
  float *wts;
  float topp;             // adaptive expert top-p
  int32_t *keff;          // [S]: written with the selection (with_topk), else read
  int use_keff;           // drop pairs past keff (top-p on); else keep all K
};

// Grouped int8 MFMA GEMM of the union path (grouped_mfma.hip); mode 0 is
// gate/up + SwiGLU, mode 1 is down.
struct GroupedMfmaArgs {
  ExpertSet rt, sh;
  int E, P;
  int C, O;               // contraction length and output rows of the matrix
  const int32_t *gcount, *goff, *pairs;
  const int2 *tiles;
  const int32_t *ntiles;
  const int8_t *act;      // mode 0: xq [S][D]; mode 1: hq [S*P][I] (permuted codes)
  const float *ascale;    // sx [S] or sh [S*P]
  const int32_t *asum;    // sumx [S] or sumh [S*P]
  float *out;             // h [S*P][I] or stage [S*P][D]
};

struct GroupedGateUpArgs {
  ExpertSet rt, sh;
  int D, I, E, P;
  const int32_t *gcount, *goff, *pairs;
  const int8_t *xq;
  const float *sx;
  const int32_t *sumx;
  float *h;               // [S][P][I]
};

struct RequantArgs {
  const float *h;         // [rows][I]
  int I;
  int8_t *hq;             // [rows][I] permuted
  float *sh_scale;
  int32_t *sumh;
};

struct GroupedDownArgs {
  ExpertSet rt, sh;
  int D, I, E, P;
  const int32_t *gcount, *goff, *pairs;
  const int8_t *hq;
  const float *sh_scale;
  const int32_t *sumh;
  float *stage;           // [S][P][D]
};

struct CombineArgs {
  const float *stage;
  const float *w;
  int S, D, K, P, n_shared;
  float *out;
  unsigned flags;
  const int32_t *keff;  // [S] routed slots combined per token
};

struct PackArgs {
  const float *w;
  int O, C;
  uint8_t *q4;
  float *scale;
};

struct RmsArgs {
  const float *x, *gamma;
  int D;
  float eps;
  float *y;
  int vec;  // float4 path: D <= 8192, D % 4 == 0, all three 16-byte aligned
};

// Host launchers, each defined next to its kernels.  They return the launch
// status (hipGetLastError after the launch).
// The int8 weight format (fmt8.hip).
struct Q8QuantArgs {
  const float *w;  // [O][C]
  int O, C;
  int8_t *q;       // [O][C]
  float *scale;    // [O]
};

struct Swiglu8Args {
  const int8_t *xq;        // [S][D] natural-order activation codes
  const float *sx;         // [S]
  int S, D, I;
  const int8_t *G, *U;     // [I][D] this expert's gate and up codes
  const int8_t *Dn;        // [D][I] down codes
  const float *gs, *us;    // [I]
  const float *ds;         // [D]
  float *h;                // [S][I] SwiGLU output
  int32_t *acc_gu;         // optional [S][2][I]
  int8_t *hq_out;          // optional [S][I] requantized h (natural order)
  float *sh_out;           // optional [S]
  float *y;                // [S][D]
  int32_t *acc_d;          // optional [S][D]
  int accumulate;          // y += result instead of y = result
  int x_perm;              // xq holds permuted-layout codes (the union path's) instead
  int64_t h_stride;        // floats between the tokens' h rows (0: I)
  int64_t y_stride;        // floats between the tokens' y rows (0: D)
};

// The int8 shared expert of the union path on int8 matrix cores (fmt8.hip):
// MODE 0 gate/up + SwiGLU into h, MODE 1 down into y, on all S tokens.
struct Shared8MfmaArgs {
  const int8_t *act;       // token codes, permuted layout; token t's row at act + t * act_stride
  int64_t act_stride;      // bytes between token rows
  const float *ascale;     // token t's scale at ascale[t * ascale_stride]
  int64_t ascale_stride;
  const int8_t *W0, *W1;   // MODE 0: gate and up codes [O][C]; MODE 1: down codes [O][C] (W0)
  const float *ws0, *ws1;  // their row scales [O]
  int S, O, C;             // tokens, output rows (MODE 0: hidden units), columns
  float *out;              // token t's output row at out + t * out_stride (h or y)
  int64_t out_stride;      // floats between output rows
};

// Packed int2 weights (fmt2.hip): four codes per byte, code + 2, column
// 4j + k in bits 2k..2k+1 of byte j.
struct Pack2Args {
  const float *w;  // [O][C]
  int O, C;
  uint8_t *q2;     // [O][(C+3)/4]
  float *scale;    // [O]
};

struct Swiglu2Args {
  const int8_t *xq;        // [S][D] natural-order activation codes
  const float *sx;         // [S]
  int S, D, I;
  const uint8_t *G, *U;    // [I][D/4] this expert's packed gate and up rows
  const uint8_t *Dn;       // [D][I/4] packed down rows
  const float *gs, *us;    // [I]
  const float *ds;         // [D]
  float *h;                // [S][I]
  int32_t *acc_gu;         // optional [S][2][I]
  int8_t *hq_out;          // optional [S][I]
  float *sh_out;           // optional [S]
  float *y;                // [S][D]
  int32_t *acc_d;          // optional [S][D]
};

// Block-32 activation scales (b32.hip).
struct QuantB32Args {
  const float *x;  // [S][D]
  int S, D;
  int8_t *xq;      // [S][D] natural order
  float *sxb;      // [S][D/32]
};

struct SwigluB32Args {
  const int8_t *xq;        // [S][D] natural-order codes
  const float *sxb;        // [S][D/32]
  int S, D, I;
  const uint8_t *G, *U;    // [I][D/2] this expert's packed int4 gate and up rows
  const uint8_t *Dn;       // [D][I/2]
  const float *gs, *us;    // [I]
  const float *ds;         // [D]
  float *h;                // [S][I]
  int8_t *hq_out;          // optional [S][I] natural order
  float *shb_out;          // optional [S][I/32]
  float *y;                // [S][D]
};

hipError_t launch_quant_b32(const QuantB32Args &a, hipStream_t st);
hipError_t launch_swiglu_b32_gateup(const SwigluB32Args &a, hipStream_t st);
hipError_t launch_swiglu_b32_down(const SwigluB32Args &a, hipStream_t st);

// MLA decode attention with weight absorption (mla.hip).
// Cache rows per attention workgroup, swept at the GLM shape: 32 up to 2048
// rows (40.6 against 45.5 us at 1024 rows with 64), 64 up to 4096 (73.8
// against 83.6 with 32), 128 beyond (the merge of 256 chunks per (query,
// head) costs more than the longer chunks).
constexpr int kMlaMaxChunk = 128;
constexpr int kMlaMaxSplit = 128;  // chunks per query: T <= 16384
__host__ __device__ inline int mla_chunk_rows(int T) { return T <= 2048 ? 32 : T <= 4096 ? 64 : 128; }
constexpr int kMlaAbsorbParts = 8; // workgroups per (query, head) in the absorption
constexpr int kMlaValueParts = 8;  // workgroups per (query, head) in the value projection
constexpr int kMlaMergeParts = 8;  // workgroups per (query, head) in the chunk merge
constexpr int kMlaHeads = 4;       // heads per attention workgroup (8 measured slower: fewer workgroups, 171 VGPRs)
struct MlaArgs {
  int S, T, H, kvl, nope, rope, vdim, nsplit, chunk;
  float scale;
  const float *q;      // [S][H][nope + rope]
  const float *kv_b;   // [H][nope + vdim][kvl]
  const float *L;      // [T][kvl]
  const float *R;      // [T][rope]
  float *qabs;         // [S][H][kvl] absorbed queries
  float *pclat;        // [S][H][nsplit][kvl] per-chunk latent sums
  float *pm, *pl;      // [S][H][nsplit] per-chunk max and exp sum
  float *clat;         // [S][H][kvl] merged, normalized latent
  float *ctx;          // [S][H][vdim]
};

hipError_t launch_mla_decode(const MlaArgs &a, hipStream_t st);
// The matrix-core attention applies when kvl + rope (rounded up to 16) <= 576,
// rope % 4 == 0 and the cache arrays are 16-byte aligned; it splits each
// query's cache into mla_mfma_splits parts.
bool mla_mfma_fits(int kvl, int rope, const float *L, const float *R);
int mla_mfma_splits(int S, int T, int H);

hipError_t launch_pack_int2(const Pack2Args &a, hipStream_t st);
hipError_t launch_swiglu2_gateup(const Swiglu2Args &a, hipStream_t st);
hipError_t launch_swiglu2_down(const Swiglu2Args &a, hipStream_t st);

hipError_t launch_quant_rows_i8(const Q8QuantArgs &a, hipStream_t st);
hipError_t launch_swiglu8_gateup(const Swiglu8Args &a, hipStream_t st);
hipError_t launch_swiglu8_down(const Swiglu8Args &a, hipStream_t st);
hipError_t launch_shared8_mfma(const Shared8MfmaArgs &a, int mode, hipStream_t st);

hipError_t launch_quant(const QuantArgs &a, int S, hipStream_t st);
hipError_t launch_router(const RouterArgs &a, bool with_quant, hipStream_t st);
hipError_t launch_topk(const TopkArgs &a, hipStream_t st);
hipError_t launch_prep_xq(const PrepArgs &a, int S, hipStream_t st);
// Phase launchers of the per-token path (decode.hip).
hipError_t launch_decode_a(const DecodeArgs &a, bool local_quant, hipStream_t st);
// e0 / e1 (optional): events that take the kernel's own start / end timestamps
hipError_t launch_decode_b(const DecodeArgs &a, hipStream_t st, hipEvent_t e0 = nullptr,
                           hipEvent_t e1 = nullptr);
hipError_t launch_decode_c(const DecodeArgs &a, hipStream_t st, hipEvent_t e0 = nullptr,
                           hipEvent_t e1 = nullptr);
// Slots per phase-C launch for rows of I columns.
int decode_c_slots(int I);
// Output rows a phase C workgroup computes per pass.
int decode_c_rows_per_pass(int I);
hipError_t launch_requant(const RequantArgs &a, int rows, hipStream_t st);
hipError_t launch_group(const GroupArgs &a, hipStream_t st);
hipError_t launch_grouped_gateup(const GroupedGateUpArgs &a, hipStream_t st);
// The MFMA form applies when the contraction length is a multiple of 256.
bool grouped_mfma_fits(int C);
constexpr int kGroupedMfmaTile = 128;  // pairs per tile
// logits per phase-A router workgroup (one per wave)
constexpr int kARouterWaves = 4;
constexpr int kRouterTileMinTokens = 256;  // batches from this size use the 8x8 router tiles
// batches up to this size select inside group_kernel (one wave per token)
constexpr int kGroupTopkMaxTokens = 16;
int grouped_mfma_tile_rows(int S);
int grouped_mfma_max_tiles(int S, int P, int E);
hipError_t launch_grouped_mfma(const GroupedMfmaArgs &a, int mode, int max_tiles, int S, hipStream_t st);
hipError_t launch_grouped_down(const GroupedDownArgs &a, hipStream_t st);
hipError_t launch_combine(const CombineArgs &a, hipStream_t st);
hipError_t launch_pack(const PackArgs &a, hipStream_t st);
hipError_t launch_rmsnorm(const RmsArgs &a, int S, hipStream_t st);
hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t st);
int stream_read_sink_words();

// Row length C (int4 columns) supported by the GEMV kernels: C % 32 == 0 and
// C/2 bytes either below 1024 or up to 4096.
inline bool gemv_cols_ok(int C) { return C > 0 && C % 32 == 0 && C / 2 <= 4096; }

}  // namespace moe
