// mla.hip -- MLA decode attention with weight absorption (section 09 of the
// reader.mx article "惊呆了！25GB 内存上运行 GLM 5.2 744B 模型"): the cache
// keeps one latent row and one rotary key per token; the key up-projection
// is absorbed into the query and the value up-projection is applied to the
// attention-weighted latent.
//
// Four launches, split over the cache like flash decoding:
//   1. absorb: qabs[s][h] = W_UK[h]^T q_nope[s][h] (eight workgroups per
//      query and head, each an eighth of the key rows; 16-byte loads);
//   2. chunks: workgroup (s, four heads, k) reads cache rows [ck, ck + c)
//      (c = 64 or 128) of the query's window once and forms, per head, the
//      chunk's max m_k, exp sum l_k and latent sum sum_t e^(score_t - m_k) L[t]
//      in one pass (online softmax);
//   3. merge: per (s, h) the chunks merge with weights e^(m_k - m) and the
//      latent is normalized (eight workgroups per query and head, each an
//      eighth of the latent columns);
//   4. value: the value up-projection gives ctx (eight workgroups per query
//      and head, each an eighth of the value rows).
// All float32; the oracle computes in double.
#include "moe_kernels.h"

namespace moe {

// Workgroup (s, h, part) sums the key rows d of its share of [0, nope).
// Thread t takes latent columns 4 (t % (kvl/4)) .. +3 (16-byte loads) of rows
// d0 + t / (kvl/4), stepping by floor(1024 / kvl) rows;
// the row phases are added through shared memory in a fixed order.  The
// chunk kernel adds the parts' vectors in a fixed order.
__global__ __launch_bounds__(256) void mla_absorb_kernel(MlaArgs a) {
  __shared__ float4 red[256];
  const int sh = blockIdx.x / kMlaAbsorbParts, part = blockIdx.x % kMlaAbsorbParts;
  const int h = sh % a.H;
  const int d0 = a.nope * part / kMlaAbsorbParts, d1 = a.nope * (part + 1) / kMlaAbsorbParts;
  const float *qp = a.q + (int64_t)sh * (a.nope + a.rope);
  const float *wk = a.kv_b + (int64_t)h * (a.nope + a.vdim) * a.kvl;
  const int tpr = a.kvl >> 2;           // threads per row (16 .. 256)
  const int nph = 256 / tpr;            // row phases (1 .. 16); threads past nph * tpr idle
  const int c4 = threadIdx.x % tpr, ph = threadIdx.x / tpr;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
  for (int d = d0 + ph; ph < nph && d < d1; d += nph) {
    const float qd = qp[d];
    const float4 w = reinterpret_cast<const float4 *>(wk + (int64_t)d * a.kvl)[c4];
    acc.x = fmaf(qd, w.x, acc.x);
    acc.y = fmaf(qd, w.y, acc.y);
    acc.z = fmaf(qd, w.z, acc.z);
    acc.w = fmaf(qd, w.w, acc.w);
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
    reinterpret_cast<float4 *>(a.qabs + ((int64_t)sh * kMlaAbsorbParts + part) * a.kvl)[c4] = t;
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
  // the heads' absorbed queries: the workgroup adds the absorption parts
  // once into shared memory (fixed order), then every wave reads them
  __shared__ float qsum[kMlaHeads][64 * MAXJ];
  for (int idx = tid; idx < kMlaHeads * a.kvl; idx += 256) {
    const int hb = idx / a.kvl, i = idx - hb * a.kvl;
    const int64_t sh = (int64_t)s * a.H + min(h0 + hb, a.H - 1);
    const float *qab = a.qabs + sh * kMlaAbsorbParts * a.kvl + i;
    float v = 0.f;
#pragma unroll
    for (int p = 0; p < kMlaAbsorbParts; p++) v += qab[p * a.kvl];
    qsum[hb][i] = v;
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

// Workgroup (s, h, cp) merges the chunks of (s, h) for latent columns
// [kvl cp / P, kvl (cp + 1) / P) (P = kMlaMergeParts): weights e^(m_k - m),
// normalized by the merged exp sum.  Wave 0 forms the weights; the threads
// split the chunks into 256 / ncols slices per column (so each issues a few
// loads, not nsplit), and the slices are added in a fixed order.
__global__ __launch_bounds__(256) void mla_merge_kernel(MlaArgs a) {
  __shared__ float wk[kMlaMaxSplit];
  __shared__ float part[256];
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
  const int ncols = c1 - c0;              // kvl / P: 8 .. 256 (kvl % 64 == 0)
  const int nsl = 256 / ncols;            // chunk slices per column
  const int c = tid % ncols, sl = tid / ncols;
  const float *pc = a.pclat + (int64_t)sh * a.nsplit * a.kvl + c0 + c;
  float acc = 0.f;
  if (sl < nsl)
    for (int k = sl; k < a.nsplit; k += nsl) acc = fmaf(wk[k], pc[(int64_t)k * a.kvl], acc);
  part[tid] = acc;
  __syncthreads();
  if (tid < ncols) {
    float v = part[tid];
    for (int q = 1; q < nsl; q++) v += part[q * ncols + tid];
    a.clat[(int64_t)sh * a.kvl + c0 + tid] = v * inv_l;
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

hipError_t launch_mla_decode(const MlaArgs &a, hipStream_t st) {
  const int sh = a.S * a.H;
  hipLaunchKernelGGL(mla_absorb_kernel, dim3(sh * kMlaAbsorbParts), dim3(256), 0, st, a);
  const int ngroups = (a.H + kMlaHeads - 1) / kMlaHeads;
  const dim3 grid(a.S * ngroups * a.nsplit);
  const int nj = a.kvl >> 6;
  if (nj <= 2) hipLaunchKernelGGL((mla_chunk_kernel<2>), grid, dim3(256), 0, st, a);
  else if (nj <= 4) hipLaunchKernelGGL((mla_chunk_kernel<4>), grid, dim3(256), 0, st, a);
  else if (nj <= 8) hipLaunchKernelGGL((mla_chunk_kernel<8>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((mla_chunk_kernel<kMlaMaxJ>), grid, dim3(256), 0, st, a);
  hipLaunchKernelGGL(mla_merge_kernel, dim3(sh * kMlaMergeParts), dim3(256), 0, st, a);
  hipLaunchKernelGGL(mla_value_kernel, dim3(sh * kMlaValueParts), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
