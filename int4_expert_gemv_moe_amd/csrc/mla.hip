// mla.hip -- MLA decode attention with weight absorption (section 09 of the
// reader.mx article "惊呆了！25GB 内存上运行 GLM 5.2 744B 模型"): the cache
// keeps one latent row and one rotary key per token; the key up-projection
// is absorbed into the query and the value up-projection is applied to the
// attention-weighted latent.
//
// Four launches, split over the cache like flash decoding:
//   1. absorb: qabs[s][h] = W_UK[h]^T q_nope[s][h] (eight workgroups per
//      query and head, each an eighth of the key rows; 16-byte loads);
//   2. splits: workgroup (s, 32 heads, k) walks cache rows [k R, (k + 1) R)
//      of the query's window 32 rows at a time and forms, per head, the
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
// v_mfma_f32_16x16x4_f32: lane l supplies A[l % 16][k] and B[k][l % 16] for
// its k-group l / 16 and receives C[4 (l / 16) + i][l % 16], i = 0..3.  The
// contraction index is permuted consistently for A and B: MFMA number s
// (0..3) of a 16-column block q takes column 16 q + 4 (l / 16) + s, so one
// 16-byte shared-memory read gives a lane its operands of four MFMAs.
//
// Per 32-row step of a workgroup (32 heads, four waves):
//   scores  S[row][head] = L_row . qabs_head + R_row . qrope_head: wave w
//           takes rows 16 (w % 2) .., heads 16 (w / 2) .. (one 16x16 tile,
//           Kp / 4 MFMAs);
//   softmax per head over the step's rows, folded into the running max and
//           exp sum (the running latent sums are rescaled by e^(m_old - m_new));
//   latent  clat[head][col] += sum_row p[head][row] L[row][col]: wave w takes
//           columns w kvl / 4 .., both 16-head tiles (kvl / 64 column tiles).
// The step's cache rows (latent and rotary columns, row stride kMlaMS floats,
// 4 banks apart so the 16 lanes of a read hit distinct banks) are read from
// global memory once per workgroup; the next step's rows are loaded into
// registers while the step computes.
constexpr int kMlaMH = 32;               // heads per workgroup
constexpr int kMlaMR = 32;               // cache rows per step
constexpr int kMlaMK = 576;              // latent + rotary (rounded up to 16) columns at most
constexpr int kMlaMS = kMlaMK + 4;       // shared row stride (floats)
constexpr int kMlaPS = kMlaMR + 4;       // softmax-weight row stride (floats)
constexpr int kMlaLoads = kMlaMR * kMlaMK / 4 / 256;  // 16-byte row loads per thread per step

typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4f mfma_f32(float a, float b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

bool mla_mfma_fits(int kvl, int rope, const float *L, const float *R) {
  // the cache rows are read in 16-byte pieces
  const bool al = ((uintptr_t)L & 15u) == 0 && (rope == 0 || ((uintptr_t)R & 15u) == 0);
  return al && rope % 4 == 0 && kvl + (rope + 15) / 16 * 16 <= kMlaMK;
}

int mla_mfma_splits(int S, int T, int H) {
  const int groups = (H + kMlaMH - 1) / kMlaMH;
  const int target = std::max(1, 256 / std::max(1, S * groups));
  return std::max(1, std::min(std::min(kMlaMaxSplit, (T + kMlaMR - 1) / kMlaMR), target));
}

__global__ __launch_bounds__(256) void mla_attn_mfma_kernel(MlaArgs a) {
  __shared__ __align__(16) float qs[kMlaMH * kMlaMS];  // [head][column]
  __shared__ __align__(16) float ls[kMlaMR * kMlaMS];  // [row][column]
  __shared__ __align__(16) float ps[kMlaMH * kMlaPS];  // [head][row]
  __shared__ float cmax[2][kMlaMH], csum[2][kMlaMH];
  __shared__ float mrun[kMlaMH], lrun[kMlaMH], mnew[kMlaMH], alpha[kMlaMH];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  const int groups = (a.H + kMlaMH - 1) / kMlaMH;
  const int k = blockIdx.x % a.nsplit;
  const int sg = blockIdx.x / a.nsplit;
  const int s = sg / groups, h0 = (sg % groups) * kMlaMH;
  const int kp = a.kvl + (a.rope + 15) / 16 * 16;  // contraction columns
  const int c4n = kp / 4, kv4 = a.kvl / 4, ro4 = a.rope / 4;
  const int n = a.T - a.S + 1 + s;                  // visible rows of query s
  const int per = (a.T + a.nsplit - 1) / a.nsplit;
  const int rows = (per + kMlaMR - 1) / kMlaMR * kMlaMR;
  const int r0 = k * rows, r1 = min(n, r0 + rows);
  const int steps = r1 > r0 ? (r1 - r0 + kMlaMR - 1) / kMlaMR : 0;

  // the absorbed queries, the same pieces as a step's rows (head for row),
  // every load unconditional (a piece outside the queries reads qabs[0] and
  // is replaced by zeros); then the rotary queries (4-byte aligned, scalar
  // loads) and zeros in the padding columns
  {
    const float *qbase = a.qabs;
    float4 qv[kMlaLoads];
#pragma unroll
    for (int i = 0; i < kMlaLoads; i++) {
      const int f = tid + 256 * i;
      const int hb = f / c4n, c4 = f - hb * c4n, h = h0 + hb;
      const bool ok = hb < kMlaMH && h < a.H && c4 < kv4;
      const float *src = ok ? a.qabs + ((int64_t)s * a.H + h) * a.kvl + 4 * c4 : qbase;
      const float4 v = *reinterpret_cast<const float4 *>(src);
      qv[i] = ok ? v : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int i = 0; i < kMlaLoads; i++) {
      const int f = tid + 256 * i;
      const int hb = f / c4n, c4 = f - hb * c4n;
      if (hb < kMlaMH) *reinterpret_cast<float4 *>(qs + hb * kMlaMS + 4 * c4) = qv[i];
    }
    __syncthreads();
    const int pad = kp - a.kvl;  // rotary columns and their padding
    for (int i = tid; i < kMlaMH * pad; i += 256) {
      const int hb = i / pad, d = i - hb * pad, h = h0 + hb;
      float v = 0.f;
      if (h < a.H && d < a.rope) v = a.q[((int64_t)s * a.H + h) * (a.nope + a.rope) + a.nope + d];
      qs[hb * kMlaMS + a.kvl + d] = v;
    }
  }
  if (tid < kMlaMH) {
    mrun[tid] = -INFINITY;
    lrun[tid] = 0.f;
  }
  // the rows of a step into registers: load i of thread t is 16-byte piece
  // f = t + 256 i of the step, row f / c4n, column piece f % c4n
  float4 pre[kMlaLoads];
  // every load unconditional: pieces past the step's rows or the row's
  // columns read L[0] and are replaced by zeros
  auto load_rows = [&](int t0) {
#pragma unroll
    for (int i = 0; i < kMlaLoads; i++) {
      const int f = tid + 256 * i;
      const int r = f / c4n, c4 = f - r * c4n;
      const int t = t0 + r;
      const bool ok = r < kMlaMR && t < r1 && c4 < kv4 + ro4;
      const float *src = c4 < kv4 ? a.L + (int64_t)t * a.kvl + 4 * c4
                                  : a.R + (int64_t)t * a.rope + 4 * (c4 - kv4);
      const float4 v = *reinterpret_cast<const float4 *>(ok ? src : a.L);
      pre[i] = ok ? v : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  v4f acc[2][8];  // running latent sums: head tile, column tile
#pragma unroll
  for (int mt = 0; mt < 2; mt++)
#pragma unroll
    for (int ct = 0; ct < 8; ct++) acc[mt][ct] = v4f{0.f, 0.f, 0.f, 0.f};
  const int nct = a.kvl / 64;            // column tiles per wave (kvl / 4 columns)
  const int cw0 = wave * (a.kvl / 4);
  const int rt = wave & 1, ht = wave >> 1;
  if (steps > 0) load_rows(r0);
  for (int st = 0; st < steps; st++) {
    const int t0 = r0 + st * kMlaMR;
#pragma unroll
    for (int i = 0; i < kMlaLoads; i++) {
      const int f = tid + 256 * i;
      const int r = f / c4n, c4 = f - r * c4n;
      if (r < kMlaMR) *reinterpret_cast<float4 *>(ls + r * kMlaMS + 4 * c4) = pre[i];
    }
    __syncthreads();  // the rows (and, on the first step, the queries) are in place
    if (st + 1 < steps) load_rows(t0 + kMlaMR);
    // scores of rows 16 rt + .., heads 16 ht + ..
    // four independent accumulators (one per MFMA of a column block), added
    // at the end in a fixed order
    v4f sc;
    {
      const float *arow = ls + (16 * rt + ln) * kMlaMS + 4 * lg;
      const float *brow = qs + (16 * ht + ln) * kMlaMS + 4 * lg;
      v4f s0 = v4f{0.f, 0.f, 0.f, 0.f}, s1 = s0, s2 = s0, s3 = s0;
#pragma unroll 4
      for (int q = 0; q < kp / 16; q++) {
        const float4 av = *reinterpret_cast<const float4 *>(arow + 16 * q);
        const float4 bv = *reinterpret_cast<const float4 *>(brow + 16 * q);
        s0 = mfma_f32(av.x, bv.x, s0);
        s1 = mfma_f32(av.y, bv.y, s1);
        s2 = mfma_f32(av.z, bv.z, s2);
        s3 = mfma_f32(av.w, bv.w, s3);
      }
      sc = (s0 + s1) + (s2 + s3);
    }
    // lane holds rows 16 rt + 4 lg + i of head 16 ht + ln
    const int hh = 16 * ht + ln;
    float sv[4];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int t = t0 + 16 * rt + 4 * lg + i;
      sv[i] = t < r1 ? sc[i] * a.scale : -INFINITY;
      mx = fmaxf(mx, sv[i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (lg == 0) cmax[rt][hh] = mx;
    __syncthreads();
    if (tid < kMlaMH) {
      const float mo = mrun[tid];
      const float mn = fmaxf(mo, fmaxf(cmax[0][tid], cmax[1][tid]));
      alpha[tid] = mo == -INFINITY ? 0.f : expf(mo - mn);
      mnew[tid] = mn;
      mrun[tid] = mn;
    }
    __syncthreads();
    {
      const float mn = mnew[hh];
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const float pv = sv[i] == -INFINITY ? 0.f : expf(sv[i] - mn);
        ps[hh * kMlaPS + 16 * rt + 4 * lg + i] = pv;
        sum += pv;
      }
      sum += __shfl_xor(sum, 16, 64);
      sum += __shfl_xor(sum, 32, 64);
      if (lg == 0) csum[rt][hh] = sum;
    }
    __syncthreads();  // the weights and row sums are in place
    if (tid < kMlaMH) lrun[tid] = fmaf(lrun[tid], alpha[tid], csum[0][tid] + csum[1][tid]);
    // latent sums of columns cw0 + 16 ct + ln, heads 16 mt + 4 lg + i
#pragma unroll
    for (int mt = 0; mt < 2; mt++) {
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; i++) al[i] = alpha[16 * mt + 4 * lg + i];
#pragma unroll
      for (int ct = 0; ct < 8; ct++)
        if (ct < nct)
#pragma unroll
          for (int i = 0; i < 4; i++) acc[mt][ct][i] *= al[i];
    }
#pragma unroll
    for (int q = 0; q < kMlaMR / 16; q++) {
      float4 pa[2];
#pragma unroll
      for (int mt = 0; mt < 2; mt++)
        pa[mt] = *reinterpret_cast<const float4 *>(ps + (16 * mt + ln) * kMlaPS + 16 * q + 4 * lg);
      const float *lrow = ls + (16 * q + 4 * lg) * kMlaMS + cw0 + ln;
#pragma unroll
      for (int ct = 0; ct < 8; ct++) {
        if (ct < nct) {
          const float b0 = lrow[16 * ct], b1 = lrow[kMlaMS + 16 * ct];
          const float b2 = lrow[2 * kMlaMS + 16 * ct], b3 = lrow[3 * kMlaMS + 16 * ct];
#pragma unroll
          for (int mt = 0; mt < 2; mt++) {
            acc[mt][ct] = mfma_f32(pa[mt].x, b0, acc[mt][ct]);
            acc[mt][ct] = mfma_f32(pa[mt].y, b1, acc[mt][ct]);
            acc[mt][ct] = mfma_f32(pa[mt].z, b2, acc[mt][ct]);
            acc[mt][ct] = mfma_f32(pa[mt].w, b3, acc[mt][ct]);
          }
        }
      }
    }
    __syncthreads();  // every wave is done with the step's rows and weights
  }
  // the split's partial results
#pragma unroll
  for (int mt = 0; mt < 2; mt++)
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int h = h0 + 16 * mt + 4 * lg + i;
      if (h < a.H) {
        float *dst = a.pclat + (((int64_t)s * a.H + h) * a.nsplit + k) * a.kvl + cw0 + ln;
#pragma unroll
        for (int ct = 0; ct < 8; ct++)
          if (ct < nct) dst[16 * ct] = acc[mt][ct][i];
      }
    }
  if (tid < kMlaMH && h0 + tid < a.H) {
    const int64_t part = ((int64_t)s * a.H + h0 + tid) * a.nsplit + k;
    a.pm[part] = mrun[tid];
    a.pl[part] = lrun[tid];
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
