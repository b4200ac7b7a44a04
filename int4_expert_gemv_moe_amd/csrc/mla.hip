// mla.hip -- MLA decode attention with weight absorption (section 09 of the
// reader.mx article "惊呆了！25GB 内存上运行 GLM 5.2 744B 模型"): the cache
// keeps one latent row and one rotary key per token; the key up-projection
// is absorbed into the query and the value up-projection is applied to the
// attention-weighted latent.
//
// Four launches, split over the cache like flash decoding:
//   1. absorb: qabs[s][h] = W_UK[h]^T q_nope[s][h] (eight workgroups per
//      query and head, each an eighth of the key rows; 16-byte loads);
//   2. splits: workgroup (s, 16 heads, k) walks cache rows [k R, (k + 1) R)
//      of the query's window 16 rows at a time and forms, per head, the
//      split's max m_k, exp sum l_k and latent sum sum_t e^(score_t - m_k) L[t]
//      (online softmax), both products on fp32 matrix cores
//      (mla_attn_mfma_kernel, latent + rotary width up to 576); wider latents
//      use mla_chunk_kernel (four heads per workgroup, v_fma);
//   3. merge: per (s, h) the chunks merge with weights e^(m_k - m) and the
//      latent is normalized (eight workgroups per query and head, each an
//      eighth of the latent columns);
//   4. value: the value up-projection gives ctx (eight workgroups per query
//      and head, each an eighth of the value rows).
// All float32; the oracle computes in double.
#include <algorithm>

#include "moe_kernels.h"
#include "dma.h"

namespace moe {

// Workgroup (s, h, part) forms latent columns [c0, c1) = kvl part / P ..
// (P = kMlaAbsorbParts) of qabs[s][h] over all key rows d < nope.  Thread t
// takes columns c0 + 4 (t % tpr) .. +3 (16-byte loads, tpr = (c1 - c0) / 4
// threads per row) of rows d = t / tpr, t / tpr + nph, ... (nph = 256 / tpr
// row phases), all its loads issued before the sums; the row phases are
// added through shared memory in a fixed order.
__global__ __launch_bounds__(256) void mla_absorb_kernel(MlaArgs a) {
  __shared__ float4 red[256];
  const int sh = blockIdx.x / kMlaAbsorbParts, part = blockIdx.x % kMlaAbsorbParts;
  const int h = sh % a.H;
  const int c0 = a.kvl * part / kMlaAbsorbParts, c1 = a.kvl * (part + 1) / kMlaAbsorbParts;
  const float *qp = a.q + (int64_t)sh * (a.nope + a.rope);
  const float *wk = a.kv_b + (int64_t)h * (a.nope + a.vdim) * a.kvl + c0;
  const int tpr = (c1 - c0) >> 2;       // threads per row (2 .. 32)
  const int nph = 256 / tpr;            // row phases (8 .. 128)
  const int c4 = threadIdx.x % tpr, ph = threadIdx.x / tpr;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  constexpr int U = 12;  // rows per batch of loads in flight (a GLM head: 192 / 16 phases)
  for (int d0 = ph; d0 < a.nope; d0 += U * nph) {
    float4 w[U];
    float qd[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int d = min(d0 + u * nph, a.nope - 1);
      w[u] = reinterpret_cast<const float4 *>(wk + (int64_t)d * a.kvl)[c4];
      qd[u] = d0 + u * nph < a.nope ? qp[d] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      acc.x = fmaf(qd[u], w[u].x, acc.x);
      acc.y = fmaf(qd[u], w[u].y, acc.y);
      acc.z = fmaf(qd[u], w[u].z, acc.z);
      acc.w = fmaf(qd[u], w[u].w, acc.w);
    }
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  if (ph == 0) {
    float4 t = red[c4];
    for (int p = 1; p < nph; p++) {
      const float4 u = red[p * tpr + c4];
      t.x += u.x;
      t.y += u.y;
      t.z += u.z;
      t.w += u.w;
    }
    reinterpret_cast<float4 *>(a.qabs + (int64_t)sh * a.kvl + c0)[c4] = t;
  }
}

// kvl % 64 == 0 and kvl <= 1024: lane l holds latent columns l + 64j.
constexpr int kMlaMaxJ = 16;

// Workgroup (s, hg, k): heads kMlaHeads hg .. +kMlaHeads-1 of query s over
// cache rows [ck, ck + c) of its window (c = 64 or 128 rows).  Each cache row
// is loaded once, by one wave, for all the heads: the wave scores it against
// their absorbed queries (lanes over latent columns, rotary part on the first
// lanes, a DPP sum per head) and folds it into per-head running softmax
// statistics and latent sums (online softmax: when the running max grows the
// sums are rescaled).  The four waves' partial results merge through shared
// memory in a fixed order.
// MAXJ >= kvl / 64 bounds the latent columns per lane (register arrays).
template <int MAXJ>
__global__ __launch_bounds__(256) void mla_chunk_kernel(MlaArgs a) {
  __shared__ float wacc[4][kMlaHeads][64 * MAXJ];
  __shared__ float wm[4][kMlaHeads], wl[4][kMlaHeads];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ngroups = (a.H + kMlaHeads - 1) / kMlaHeads;
  const int k = blockIdx.x % a.nsplit;
  const int sg = blockIdx.x / a.nsplit;  // s * ngroups + hg
  const int s = sg / ngroups, h0 = (sg % ngroups) * kMlaHeads;
  const int n = a.T - a.S + 1 + s;  // visible cache rows of query s
  const int t0 = k * a.chunk;
  const int nt = max(0, min(a.chunk, n - t0));
  const int nj = a.kvl >> 6;
  if (nt == 0) {  // the chunk lies past this query's window
    for (int hb = 0; hb < kMlaHeads && h0 + hb < a.H; hb++) {
      const int64_t part = ((int64_t)s * a.H + h0 + hb) * a.nsplit + k;
      for (int i = tid; i < a.kvl; i += 256) a.pclat[part * a.kvl + i] = 0.f;
      if (tid == 0) {
        a.pm[part] = -INFINITY;
        a.pl[part] = 0.f;
      }
    }
    return;
  }
  // the heads' absorbed queries into shared memory, then every wave reads them
  __shared__ float qsum[kMlaHeads][64 * MAXJ];
  for (int idx = tid; idx < kMlaHeads * a.kvl; idx += 256) {
    const int hb = idx / a.kvl, i = idx - hb * a.kvl;
    const int64_t sh = (int64_t)s * a.H + min(h0 + hb, a.H - 1);
    qsum[hb][i] = a.qabs[sh * a.kvl + i];
  }
  __syncthreads();
  float qa[kMlaHeads][MAXJ], qr[kMlaHeads];
#pragma unroll
  for (int hb = 0; hb < kMlaHeads; hb++) {
    const int64_t sh = (int64_t)s * a.H + min(h0 + hb, a.H - 1);
#pragma unroll
    for (int j = 0; j < MAXJ; j++) qa[hb][j] = j < nj ? qsum[hb][lane + 64 * j] : 0.f;
    qr[hb] = lane < a.rope ? a.q[sh * (a.nope + a.rope) + a.nope + lane] : 0.f;
  }
  float m[kMlaHeads], l[kMlaHeads], acc[kMlaHeads][MAXJ];
#pragma unroll
  for (int hb = 0; hb < kMlaHeads; hb++) {
    m[hb] = -INFINITY;
    l[hb] = 0.f;
#pragma unroll
    for (int j = 0; j < MAXJ; j++) acc[hb][j] = 0.f;
  }
  for (int tt = wave; tt < nt; tt += 4) {
    const int t = t0 + tt;
    const float *lr = a.L + (int64_t)t * a.kvl;
    float lv[MAXJ];
#pragma unroll
    for (int j = 0; j < MAXJ; j++) lv[j] = j < nj ? lr[lane + 64 * j] : 0.f;
    const float rv = lane < a.rope ? a.R[(int64_t)t * a.rope + lane] : 0.f;
#pragma unroll
    for (int hb = 0; hb < kMlaHeads; hb++) {
      float d = 0.f;
#pragma unroll
      for (int j = 0; j < MAXJ; j++)
        if (j < nj) d = fmaf(qa[hb][j], lv[j], d);
      if (lane < a.rope) d = fmaf(qr[hb], rv, d);
      const float sc = wave_sum_f32(d) * a.scale;
      const float mn = fmaxf(m[hb], sc);
      const float c = expf(m[hb] - mn);  // 0 for the first row (m = -inf)
      const float e = expf(sc - mn);
      l[hb] = fmaf(l[hb], c, e);
#pragma unroll
      for (int j = 0; j < MAXJ; j++)
        if (j < nj) acc[hb][j] = fmaf(e, lv[j], acc[hb][j] * c);
      m[hb] = mn;
    }
  }
#pragma unroll
  for (int hb = 0; hb < kMlaHeads; hb++) {
#pragma unroll
    for (int j = 0; j < MAXJ; j++)
      if (j < nj) wacc[wave][hb][lane + 64 * j] = acc[hb][j];
    if (lane == 0) {
      wm[wave][hb] = m[hb];
      wl[wave][hb] = l[hb];
    }
  }
  __syncthreads();
  for (int hb = 0; hb < kMlaHeads && h0 + hb < a.H; hb++) {
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; w++) mm = fmaxf(mm, wm[w][hb]);
    float cw[4], ll = 0.f;
#pragma unroll
    for (int w = 0; w < 4; w++) {
      cw[w] = wl[w][hb] > 0.f ? expf(wm[w][hb] - mm) : 0.f;
      ll = fmaf(cw[w], wl[w][hb], ll);
    }
    const int64_t part = ((int64_t)s * a.H + h0 + hb) * a.nsplit + k;
    for (int i = tid; i < a.kvl; i += 256) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < 4; w++) v = fmaf(cw[w], wacc[w][hb][i], v);
      a.pclat[part * a.kvl + i] = v;
    }
    if (tid == 0) {
      a.pm[part] = mm;
      a.pl[part] = ll;
    }
  }
}

// ---- attention on fp32 matrix cores ----------------------------------------------
//
// v_mfma_f32_16x16x4_f32: lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16]
// and receives C[4 (l / 16) + i][l % 16], i = 0..3.  The contraction index is
// permuted consistently for A and B: MFMA number s (0..3) of a 16-column block q
// takes column 16 q + 4 (l / 16) + s, so one 16-byte read gives a lane its
// operands of four MFMAs.
//
// A workgroup (four waves) takes 16 heads of one query and one split of its
// window, 16 cache rows per step; two workgroups share a CU (77 KB of shared
// memory, about 110 registers per lane).  Per step:
//   rows    the step's 16 cache rows (latent and rotary columns) arrive in a
//           shared-memory stage by DMA (global_load_lds_dwordx4; two stages,
//           the next step's rows requested while this one computes);
//   scores  S[row][head] = L_row . qabs_head + R_row . qrope_head, one 16 x 16
//           tile: wave w takes a quarter of the columns, its queries held in
//           registers for the whole split; the four partial tiles meet in
//           shared memory and every wave adds them in the same order;
//   softmax every wave forms the same running max, exp sum and weights
//           (online softmax; the latent sums are rescaled by e^(m_old - m_new)),
//           the weights staying in the registers that the next products read;
//   latent  clat[head][col] += sum_row p[head][row] L[row][col]: wave w takes
//           columns w kvl / 4 .. (kvl / 64 tiles of 16).
// Stage layout: row r of a stage is 145 pieces of 16 bytes (latent, rotary,
// padding to 576 columns, one spare piece), so the 16 lanes of a score read,
// one row each, hit 16 distinct bank groups and the 64 lanes of a latent-sum
// read 64 distinct banks.
constexpr int kMlaMH = 16;               // heads per workgroup
constexpr int kMlaMR = 16;               // cache rows per step
constexpr int kMlaMK = 576;              // latent + rotary (rounded up to 16) columns at most
constexpr int kMlaRowP = kMlaMK / 4 + 1; // 16-byte pieces per shared row (144 + 1 of padding)
constexpr int kMlaRowB = 16 * kMlaRowP;  // 2320 bytes
constexpr int kMlaDmaN = (kMlaMR * kMlaRowP + 63) / 64;  // DMA requests of a stage (37)
constexpr int kMlaStage = 1024 * kMlaDmaN;               // 37 KB
constexpr int kMlaDma = (kMlaDmaN + 3) / 4;  // at most per wave and step (10)
constexpr int kMlaQB = kMlaMK / 16 / 4;  // 16-column blocks of a wave's score quarter (9)

typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4f mfma_f32(float a, float b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

bool mla_mfma_fits(int kvl, int rope, const float *L, const float *R) {
  // the cache rows are read in 16-byte pieces
  const bool al = ((uintptr_t)L & 15u) == 0 && (rope == 0 || ((uintptr_t)R & 15u) == 0);
  return al && rope % 4 == 0 && kvl + (rope + 15) / 16 * 16 <= kMlaMK;
}

// Splits per query (16-row steps): at most kMlaMaxSplit and about 512
// workgroups (hi), and between that and about 256 workgroups (lo) as few as
// leave every split four steps.  Swept at the GLM shape (64 heads, one
// query): 1024 rows 64 splits 25.1 us (16 or 32 splits 30.1, 26.1); 4096
// rows 64 splits 31.8-32.1 us (128: 34.1); 16384 rows 128 splits 54.3 us
// (64: 58.1).
int mla_mfma_splits(int S, int T, int H) {
  const int groups = (H + kMlaMH - 1) / kMlaMH;
  const int sg = std::max(1, S * groups);
  const int one_step = (T + kMlaMR - 1) / kMlaMR, four_steps = (T + 4 * kMlaMR - 1) / (4 * kMlaMR);
  const int hi = std::max(1, std::min(std::min(kMlaMaxSplit, one_step), 512 / sg));
  const int lo = std::max(1, std::min(hi, 256 / sg));
  return std::max(lo, std::min(hi, four_steps));
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void mla_attn_mfma_kernel(MlaArgs a) {
  __shared__ __align__(1024) int8_t st0[kMlaStage], st1[kMlaStage];
  __shared__ __align__(16) float4 part[4][64];  // the waves' partial score tiles
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  const int groups = (a.H + kMlaMH - 1) / kMlaMH;
  const int k = blockIdx.x % a.nsplit;
  const int sg = blockIdx.x / a.nsplit;
  const int s = sg / groups, h0 = (sg % groups) * kMlaMH;
  const int kv4 = a.kvl / 4, ro4 = a.rope / 4;
  const int n = a.T - a.S + 1 + s;                 // visible rows of query s
  const int per = (a.T + a.nsplit - 1) / a.nsplit;
  const int rows = (per + kMlaMR - 1) / kMlaMR * kMlaMR;
  const int r0 = k * rows, r1 = min(n, r0 + rows);
  const int steps = r1 > r0 ? (r1 - r0 + kMlaMR - 1) / kMlaMR : 0;

  // the wave's quarter of the queries: blocks q = kQB wave .. (columns 16 q +
  // 4 lg + 0..3 of head h0 + ln), zero past the head count and the columns
  const int h = h0 + ln;
  const int64_t shq = (int64_t)s * a.H + min(h, a.H - 1);
  float4 qv[kMlaQB];
#pragma unroll
  for (int b = 0; b < kMlaQB; b++) {
    const int c = 16 * (kMlaQB * wave + b) + 4 * lg;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (h < a.H) {
      if (c < a.kvl) {
        v = *reinterpret_cast<const float4 *>(a.qabs + shq * a.kvl + c);
      } else if (c < a.kvl + a.rope) {
        const float *qr = a.q + shq * (a.nope + a.rope) + a.nope + (c - a.kvl);
        v = make_float4(qr[0], qr[1], qr[2], qr[3]);
      }
    }
    qv[b] = v;
  }

  // DMA request n = 4 u + wave of a stage (n < kMlaDmaN): slot g = 64 n +
  // lane, row g / 145, piece g % 145 (pieces past the row's columns, the
  // spare piece and the slots past the last row copy the row's first latent
  // piece: a finite value that no product uses)
  int roff[kMlaDma];   // byte offset of the piece within its row
  int rrow[kMlaDma];   // row of the step
  bool rrot[kMlaDma];  // rotary piece (R) rather than latent (L)
#pragma unroll
  for (int u = 0; u < kMlaDma; u++) {
    const int g = 64 * (4 * u + wave) + lane;
    const int r = g / kMlaRowP, lp = g % kMlaRowP;
    rrow[u] = min(r, kMlaMR - 1);
    rrot[u] = r < kMlaMR && lp >= kv4 && lp < kv4 + ro4;
    roff[u] = r < kMlaMR && lp < kv4 ? 16 * lp : (rrot[u] ? 16 * (lp - kv4) : 0);
  }
  auto issue = [&](int st, int8_t *dst) __attribute__((always_inline)) {
    // rows past the split's window repeat its last row (their weights are 0)
    const int tb = r0 + st * kMlaMR;
#pragma unroll
    for (int u = 0; u < kMlaDma; u++) {
      if (4 * u + wave < kMlaDmaN) {  // uniform across the wave
        const int64_t t = max(min(tb + rrow[u], r1 - 1), 0);
        const float *row = rrot[u] ? a.R + t * a.rope : a.L + t * a.kvl;
        dma16(reinterpret_cast<const int8_t *>(row) + roff[u], dst + 1024 * (4 * u + wave));
      }
    }
  };

  v4f acc[8];  // latent sums: heads 4 lg + i, columns cw0 + 16 ct + ln
#pragma unroll
  for (int ct = 0; ct < 8; ct++) acc[ct] = v4f{0.f, 0.f, 0.f, 0.f};
  float mrun = -INFINITY, lrun = 0.f;  // of head h0 + ln (every lane group alike)
  const int nct = a.kvl / 64;
  const int cw0 = wave * (a.kvl / 4);
  if (steps > 0) issue(0, st0);
  auto step = [&](int st, int8_t *cur, int8_t *nxt) __attribute__((always_inline)) {
    // this step's rows are in (the wave's only requests in flight) and every
    // wave is done with the previous step, whose stage now takes the next rows
    dma_step_barrier<0>();
    if (st + 1 < steps) issue(st + 1, nxt);
    const int t0 = r0 + st * kMlaMR;
    // scores of rows ln (A) against heads ln (B) over the wave's quarter
    v4f c0 = v4f{0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0;
    const int8_t *arow = cur + ln * kMlaRowB;
    // blocks past the contraction columns read padding pieces against zero queries
#pragma unroll
    for (int b = 0; b < kMlaQB; b++) {
      const int q = kMlaQB * wave + b;
      const float4 av = *reinterpret_cast<const float4 *>(arow + 16 * (4 * q + lg));
      c0 = mfma_f32(av.x, qv[b].x, c0);
      c1 = mfma_f32(av.y, qv[b].y, c1);
      c2 = mfma_f32(av.z, qv[b].z, c2);
      c3 = mfma_f32(av.w, qv[b].w, c3);
    }
    const v4f pw = (c0 + c1) + (c2 + c3);
    part[wave][lane] = make_float4(pw[0], pw[1], pw[2], pw[3]);
    lds_barrier();  // every wave's partial tile is in place (the next rows stay in flight)
    const float4 p0 = part[0][lane], p1 = part[1][lane], p2 = part[2][lane], p3 = part[3][lane];
    // lane: rows 4 lg + i of head h0 + ln
    float sv[4];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float pa = i == 0 ? p0.x : (i == 1 ? p0.y : (i == 2 ? p0.z : p0.w));
      const float pb = i == 0 ? p1.x : (i == 1 ? p1.y : (i == 2 ? p1.z : p1.w));
      const float pc = i == 0 ? p2.x : (i == 1 ? p2.y : (i == 2 ? p2.z : p2.w));
      const float pd = i == 0 ? p3.x : (i == 1 ? p3.y : (i == 2 ? p3.z : p3.w));
      const float sc = (pa + pb) + (pc + pd);
      const int t = t0 + 4 * lg + i;
      sv[i] = t < r1 ? sc * a.scale : -INFINITY;
      mx = fmaxf(mx, sv[i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(mrun, mx);
    const float al = mrun == -INFINITY ? 0.f : expf(mrun - mn);
    float pv[4], sum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      pv[i] = sv[i] == -INFINITY ? 0.f : expf(sv[i] - mn);
      sum += pv[i];
    }
    sum += __shfl_xor(sum, 16, 64);
    sum += __shfl_xor(sum, 32, 64);
    lrun = fmaf(lrun, al, sum);
    mrun = mn;
    // the latent sums hold heads 4 lg + i: their rescale factors from lanes 4 lg + i
    float ali[4];
#pragma unroll
    for (int i = 0; i < 4; i++) ali[i] = __shfl(al, 4 * lg + i, 64);
#pragma unroll
    for (int ct = 0; ct < 8; ct++)
#pragma unroll
      for (int i = 0; i < 4; i++) acc[ct][i] *= ali[i];
    // the weights p[head ln][rows 4 lg + i] are this lane's A operands; all 8
    // column tiles run (with a latent narrower than 512 the tiles past kvl / 64
    // read other finite columns and are not written)
#pragma unroll
    for (int ct = 0; ct < 8; ct++) {
      const int c = cw0 + 16 * ct + ln;
      float b[4];
#pragma unroll
      for (int i = 0; i < 4; i++)
        b[i] = *reinterpret_cast<const float *>(cur + (4 * lg + i) * kMlaRowB + 4 * c);
#pragma unroll
      for (int i = 0; i < 4; i++) acc[ct] = mfma_f32(pv[i], b[i], acc[ct]);
    }
  };
  int st = 0;
  for (; st + 1 < steps; st += 2) {
    step(st, st0, st1);
    step(st + 1, st1, st0);
  }
  if (st < steps) step(st, st0, st1);
  wait_vm_at_most<0>();  // no request may still be in flight when the workgroup ends

  // the split's partial results: lane holds heads h0 + 4 lg + i, columns cw0 + 16 ct + ln
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int hh = h0 + 4 * lg + i;
    if (hh < a.H) {
      float *dst = a.pclat + (((int64_t)s * a.H + hh) * a.nsplit + k) * a.kvl + cw0 + ln;
#pragma unroll
      for (int ct = 0; ct < 8; ct++)
        if (ct < nct) dst[16 * ct] = acc[ct][i];
    }
  }
  if (wave == 0 && lg == 0 && h < a.H) {
    const int64_t pidx = ((int64_t)s * a.H + h) * a.nsplit + k;
    a.pm[pidx] = mrun;
    a.pl[pidx] = lrun;
  }
}

// Workgroup (s, h, cp) merges the chunks of (s, h) for latent columns
// [kvl cp / P, kvl (cp + 1) / P) (P = kMlaMergeParts): weights e^(m_k - m),
// normalized by the merged exp sum.  Wave 0 forms the weights; thread t
// takes four columns (16-byte loads) and every nsl-th chunk from slice t /
// (columns / 4), its loads issued together (8 at a time), and the slices are
// added in a fixed order.
__global__ __launch_bounds__(256) void mla_merge_kernel(MlaArgs a) {
  __shared__ float wk[kMlaMaxSplit];
  __shared__ float4 part[256];
  __shared__ float inv_l;
  const int tid = threadIdx.x, lane = tid & 63;
  const int sh = blockIdx.x / kMlaMergeParts, cp = blockIdx.x % kMlaMergeParts;
  const float *pm = a.pm + (int64_t)sh * a.nsplit;
  const float *pl = a.pl + (int64_t)sh * a.nsplit;
  if (tid < 64) {
    float m = -INFINITY;
    for (int k = lane; k < a.nsplit; k += 64) m = fmaxf(m, pm[k]);
    m = wave_max_f32(m);
    float l = 0.f;
    for (int k = lane; k < a.nsplit; k += 64) {
      const float w = pl[k] > 0.f ? expf(pm[k] - m) : 0.f;
      wk[k] = w;
      l = fmaf(w, pl[k], l);
    }
    l = wave_sum_f32(l);
    if (lane == 0) inv_l = 1.f / l;
  }
  __syncthreads();
  const int c0 = a.kvl * cp / kMlaMergeParts, c1 = a.kvl * (cp + 1) / kMlaMergeParts;
  const int nq = (c1 - c0) / 4;           // column quads: 2 .. 64 (kvl % 64 == 0)
  const int nsl = 256 / nq;               // chunk slices
  const int q = tid % nq, sl = tid / nq;
  const float *pc = a.pclat + (int64_t)sh * a.nsplit * a.kvl + c0 + 4 * q;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (sl < nsl) {
    constexpr int U = 8;
    for (int k0 = sl; k0 < a.nsplit; k0 += U * nsl) {
      float4 v[U];
      float w[U];
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int k = k0 + u * nsl;
        const bool ok = k < a.nsplit;
        v[u] = *reinterpret_cast<const float4 *>(pc + (int64_t)(ok ? k : k0) * a.kvl);
        w[u] = ok ? wk[k] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < U; u++) {
        acc.x = fmaf(w[u], v[u].x, acc.x);
        acc.y = fmaf(w[u], v[u].y, acc.y);
        acc.z = fmaf(w[u], v[u].z, acc.z);
        acc.w = fmaf(w[u], v[u].w, acc.w);
      }
    }
  }
  part[tid] = acc;
  __syncthreads();
  if (tid < nq) {
    float4 v = part[tid];
    for (int k = 1; k < nsl; k++) {
      const float4 u = part[k * nq + tid];
      v.x += u.x;
      v.y += u.y;
      v.z += u.z;
      v.w += u.w;
    }
    const float il = inv_l;
    reinterpret_cast<float4 *>(a.clat + (int64_t)sh * a.kvl + c0)[tid] =
        make_float4(v.x * il, v.y * il, v.z * il, v.w * il);
  }
}

// Workgroup (s, h, vb): value rows [vdim vb / 8, vdim (vb + 1) / 8) of ctx,
// four rows per wave in flight (the first four requested before the merged
// latent is read).
__global__ __launch_bounds__(256) void mla_value_kernel(MlaArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sh = blockIdx.x / kMlaValueParts, vb = blockIdx.x % kMlaValueParts;
  const int h = sh % a.H;
  const int nj = a.kvl >> 6;
  const float *wv = a.kv_b + ((int64_t)h * (a.nope + a.vdim) + a.nope) * a.kvl;
  const int v0 = a.vdim * vb / kMlaValueParts, v1 = a.vdim * (vb + 1) / kMlaValueParts;
  float wr[4][kMlaMaxJ];
  {
    const int vg = v0 + 4 * wave;
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const float *row = wv + (int64_t)max(min(vg + r, v1 - 1), 0) * a.kvl;
#pragma unroll
      for (int j = 0; j < kMlaMaxJ; j++) wr[r][j] = j < nj ? row[lane + 64 * j] : 0.f;
    }
  }
  float cl[kMlaMaxJ];
  const float *clat = a.clat + (int64_t)sh * a.kvl;
#pragma unroll
  for (int j = 0; j < kMlaMaxJ; j++) cl[j] = j < nj ? clat[lane + 64 * j] : 0.f;
  for (int vg = v0 + 4 * wave; vg < v1; vg += 16) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 4; r++) {
      if (vg != v0 + 4 * wave) {  // later groups: load now
        const float *row = wv + (int64_t)min(vg + r, v1 - 1) * a.kvl;
#pragma unroll
        for (int j = 0; j < kMlaMaxJ; j++) wr[r][j] = j < nj ? row[lane + 64 * j] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < kMlaMaxJ; j++)
        if (j < nj) acc[r] = fmaf(wr[r][j], cl[j], acc[r]);
    }
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const float v = wave_sum_f32(acc[r]);
      if (lane == 0 && vg + r < v1) a.ctx[(int64_t)sh * a.vdim + vg + r] = v;
    }
  }
}

// kvl % 256 == 0: lane l holds latent columns 4l + 256c .. +4 (c < NJ4) of a
// row as 16-byte loads, and a wave requests all of its up to 8 value rows of
// the part at once before any product.
template <int NJ4>
__global__ __launch_bounds__(256) void mla_value4_kernel(MlaArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sh = blockIdx.x / kMlaValueParts, vb = blockIdx.x % kMlaValueParts;
  const int h = sh % a.H;
  const float *wv = a.kv_b + ((int64_t)h * (a.nope + a.vdim) + a.nope) * a.kvl;
  const int v0 = a.vdim * vb / kMlaValueParts, v1 = a.vdim * (vb + 1) / kMlaValueParts;
  const float4 *cl4 = reinterpret_cast<const float4 *>(a.clat + (int64_t)sh * a.kvl);
  float4 cl[NJ4];
#pragma unroll
  for (int c = 0; c < NJ4; c++) cl[c] = cl4[lane + 64 * c];
  constexpr int RW = 8;  // rows per wave in flight
  for (int vg = v0 + RW * wave; vg < v1; vg += 4 * RW) {
    float4 w[RW][NJ4];
#pragma unroll
    for (int r = 0; r < RW; r++) {
      const float4 *row = reinterpret_cast<const float4 *>(wv + (int64_t)min(vg + r, v1 - 1) * a.kvl);
#pragma unroll
      for (int c = 0; c < NJ4; c++) w[r][c] = row[lane + 64 * c];
    }
#pragma unroll
    for (int r = 0; r < RW; r++) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < NJ4; c++) {
        acc = fmaf(w[r][c].x, cl[c].x, acc);
        acc = fmaf(w[r][c].y, cl[c].y, acc);
        acc = fmaf(w[r][c].z, cl[c].z, acc);
        acc = fmaf(w[r][c].w, cl[c].w, acc);
      }
      const float v = wave_sum_f32(acc);
      if (lane == 0 && vg + r < v1) a.ctx[(int64_t)sh * a.vdim + vg + r] = v;
    }
  }
}

// The value projection: 16-byte loads when the latent width allows them
// (kv_b rows then start 16-byte aligned: kv_b itself is checked on the host).
static void launch_mla_value(const MlaArgs &a, hipStream_t st) {
  const dim3 grid(a.S * a.H * kMlaValueParts);
  switch (a.kvl % 256 == 0 ? a.kvl / 256 : 0) {
    case 1: hipLaunchKernelGGL((mla_value4_kernel<1>), grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((mla_value4_kernel<2>), grid, dim3(256), 0, st, a); break;
    case 3: hipLaunchKernelGGL((mla_value4_kernel<3>), grid, dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL((mla_value4_kernel<4>), grid, dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL(mla_value_kernel, grid, dim3(256), 0, st, a); break;
  }
}

hipError_t launch_mla_decode(const MlaArgs &a, hipStream_t st) {
  const int sh = a.S * a.H;
  hipLaunchKernelGGL(mla_absorb_kernel, dim3(sh * kMlaAbsorbParts), dim3(256), 0, st, a);
  if (mla_mfma_fits(a.kvl, a.rope, a.L, a.R)) {
    const int groups = (a.H + kMlaMH - 1) / kMlaMH;
    hipLaunchKernelGGL(mla_attn_mfma_kernel, dim3(a.S * groups * a.nsplit), dim3(256), 0, st, a);
    hipLaunchKernelGGL(mla_merge_kernel, dim3(sh * kMlaMergeParts), dim3(256), 0, st, a);
    launch_mla_value(a, st);
    return hipGetLastError();
  }
  const int ngroups = (a.H + kMlaHeads - 1) / kMlaHeads;
  const dim3 grid(a.S * ngroups * a.nsplit);
  const int nj = a.kvl >> 6;
  if (nj <= 2) hipLaunchKernelGGL((mla_chunk_kernel<2>), grid, dim3(256), 0, st, a);
  else if (nj <= 4) hipLaunchKernelGGL((mla_chunk_kernel<4>), grid, dim3(256), 0, st, a);
  else if (nj <= 8) hipLaunchKernelGGL((mla_chunk_kernel<8>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((mla_chunk_kernel<kMlaMaxJ>), grid, dim3(256), 0, st, a);
  hipLaunchKernelGGL(mla_merge_kernel, dim3(sh * kMlaMergeParts), dim3(256), 0, st, a);
  launch_mla_value(a, st);
  return hipGetLastError();
}

}  // namespace moe
