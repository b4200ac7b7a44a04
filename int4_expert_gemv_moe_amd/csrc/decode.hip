// decode.hip -- the per-token ("decode") MoE block in three launches
// (sections 11 and 12 of the reader.mx article "惊呆了！25GB 内存上运行
// GLM 5.2 744B 模型"):
//
//   phase A  router logits, token quantization    | shared-expert gate/up
//   phase B  routed gate/up (each block selects   | shared-expert down
//            its expert from the logits)          |   -> y_shared
//   phase C  routed down + weighted combine (+ y_shared) -> out
//
// The shared expert does not depend on the routing, so its gate/up runs
// beside the router and its down beside the routed gate/up.  No workgroup
// waits for another inside a launch (no fences, no shared-address atomics):
// on this chip a device-scope fence writes back and invalidates the issuing
// XCD's L2 and a same-address atomic serializes at about 13 ns, so every
// cross-workgroup hand-off goes through a launch boundary.  The max |h| of a
// hidden row, needed for its requantization, is kept as one partial maximum
// per gate/up workgroup and reduced by the consumer.
//
// Weight rows stream with 16-byte nontemporal loads: lane l reads bytes
// 16l + 1024c of a row (c = 1 KB chunk), so one wave instruction covers 1 KB
// of contiguous HBM.  Each wave walks its rows ROWS at a time and keeps the
// next step's loads in flight while it computes the current one.
#include <hip/hip_ext.h>

#include "moe_kernels.h"
#include "quant.h"
#include "norm.h"
#include "rowops.h"
#include "topk.h"

namespace moe {

// Every kernel here runs 256-thread workgroups (4 waves).
constexpr int kWaves = 4;

// ---- router: one wave computes one logit ----------------------------------------

__device__ void router_logit(const DecodeArgs &a, const float *xrow, int s, int e) {
  if (e >= a.E) return;
  const float v = router_dot(xrow, a.W + (int64_t)e * a.D, a.D);
  if ((threadIdx.x & 63) == 0) a.logits[(int64_t)s * a.E + e] = v;
}

// An expert index read back from memory (the caller's, when the routing is
// given), kept inside the stack.
__device__ __forceinline__ int expert_at(const DecodeArgs &a, int64_t i) {
  return min(max((int)a.idx[i], 0), a.E - 1);
}

// ---- gate/up rows -----------------------------------------------------------------
//
// A block works through a contiguous range of "items" of a concatenated list
// of (slot, row) pairs: item i is row i % I of slot i / I.  Wave w takes
// items lo + w*ROWS + k*4*ROWS, ROWS at a time, with the loads of the next
// step in flight while it computes the current one.
//
// The loop body is free of branches around memory instructions: every stage
// load is issued (past the end of the range it reads a row of the token's
// own codes, which sit in L2, and the result is unused), and results go to
// LDS and reach global memory once, after the loop.  Stores count in the same
// counter as loads here and vector loads complete in issue order, so this is
// what lets the compiler wait for exactly one stage at a time.

// Most rows a gate/up block may own (its row scales and outputs sit in LDS).
#define MOE_GU_MAX_ROWS 512

// Shared-memory buffers of a gate/up block.
struct GuLds {
  float h[MOE_GU_MAX_ROWS];
};

// Walks this wave's items with a two-stage pipeline (the caller issued the
// first stage into sa), then writes the block's
// hidden values (and accumulators when acc_gu is set) to global memory.
template <int NCH, bool MASKED, int ROWS, class Res, bool W8 = false>
__device__ __forceinline__ void gu_items(Res res, int I, int rowbytes, int lo, int hi,
                                         const uint4 (&xv)[NCH][2], int corr, float sxs,
                                         GuLds &L, int *acco, int32_t *acc_gu,
                                         const uint8_t *dummy, GuStage<NCH, ROWS> &sa) {
  const int wave = threadIdx.x >> 6;
  const int stride = kWaves * ROWS;
  const int first = lo + wave * ROWS;
  const int nsteps = (first < hi) ? (hi - first + stride - 1) / stride : 0;
  GuStage<NCH, ROWS> sb;
  for (int i = 0; i < nsteps; i += 2) {
    const int ra = first + i * stride, rb = ra + stride;
    gu_load<NCH, MASKED, ROWS>(res, I, rowbytes, rb, hi, dummy, sb);
    gu_step<NCH, ROWS, W8>(sa, xv, corr, sxs, ra, lo, hi, L.h, acco);
    gu_load<NCH, MASKED, ROWS>(res, I, rowbytes, rb + stride, hi, dummy, sa);
    if (i + 1 < nsteps) gu_step<NCH, ROWS, W8>(sb, xv, corr, sxs, rb, lo, hi, L.h, acco);
  }
  __syncthreads();
  for (int t = threadIdx.x; t < hi - lo; t += 64 * kWaves) {
    const int it = lo + t;
    const int slot = it / I;
    const int row = it - slot * I;
    res(slot).h[row] = L.h[t];
    if (acc_gu) {
      acc_gu[row] = acco[2 * t];
      acc_gu[I + row] = acco[2 * t + 1];
    }
  }
}

// Fixed expert (the shared one, or the single expert of a one-expert call) for
// token s, rows of block gb.  LOCALQ: quantize the float token row in the
// block; otherwise read its codes.  W8: the fixed expert is in the int8
// format (a.f8g, a.f8u; NCH = 1 KB chunks of a D-byte row; LOCALQ only).
template <int NCH, bool MASKED, int ROWS, bool LOCALQ, bool W8 = false>
__device__ void gateup_fixed(const DecodeArgs &a, int s, int gb, float *xn) {
  static_assert(!W8 || LOCALQ, "the int8 fixed expert quantizes its token in the block");
  // chunks of 2048 columns held per thread by the row quantization
  constexpr int NX = W8 ? (NCH + 1) / 2 : NCH;
  __shared__ GuLds L;
  __shared__ int acco[2 * MOE_GU_MAX_ROWS];
  const int wave = threadIdx.x >> 6;
  const int rowbytes = W8 ? a.D : a.D >> 1;
  const int pair = s * a.P + a.fx_slot;
  GuMats m;
  if constexpr (W8) {
    m.G = a.f8g;
    m.U = a.f8u;
  } else {
    m.G = pick(a.fx.gate, a.fx.gate, false, a.fx_index);
    m.U = pick(a.fx.up, a.fx.up, false, a.fx_index);
  }
  m.h = a.h + (int64_t)pair * a.I;
  auto res = [m](int) { return m; };
  int lo, hi;
  split_rows(a.I, a.n_gu_fx, gb, lo, hi);
  const int first = lo + wave * ROWS;
  const uint8_t *dummy = reinterpret_cast<const uint8_t *>(a.xq + (int64_t)s * a.D);
  uint4 xv[NCH][2];
  GuStage<NCH, ROWS> sa;
  float sxs;
  int sumx;
  int32_t *acc_gu = a.acc_gu ? a.acc_gu + (int64_t)s * 2 * a.I : nullptr;
  if (LOCALQ) {
    // the block quantizes the token row once into shared memory (each wave
    // then reads its lanes' codes); the first weight stage is already in
    // flight while it does
    __shared__ __align__(16) int8_t xcodes[2048 * 4];
    float4 xr[NX][2];
    if (a.gamma) {
      // the token row and gain, then the first weight stage, are in flight
      // together; the normalization waits only for the former
      NormRow nr;
      norm_row_load(a.x + (int64_t)s * a.D, a.gamma, a.D, nr);
      gu_load<NCH, MASKED, ROWS>(res, a.I, rowbytes, first, hi, dummy, sa);
      prenorm_finish_lds(nr, a.D, a.eps, xn);
      quant_row_load<NX>(xn, a.D, xr);
    } else {
      quant_row_load<NX>(a.x + (int64_t)s * a.D, a.D, xr);
      gu_load<NCH, MASKED, ROWS>(res, a.I, rowbytes, first, hi, dummy, sa);
    }
    sumx = quant_row_block_lds<NX>(xr, a.D, xcodes, &sxs);
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int c = 0; c < NCH; c++) {
      // int4 rows: lane l of chunk c covers columns 2048c + 32l .. +32;
      // int8 rows: 1024c + 16l .. +16
      const int col = W8 ? 1024 * c + 16 * lane : 2048 * c + 32 * lane;
      const bool ok = !MASKED || col < a.D;
      const int cc = ok ? col : 0;
      const uint4 v0 = *reinterpret_cast<const uint4 *>(xcodes + cc);
      const uint4 v1 = W8 ? v0 : *reinterpret_cast<const uint4 *>(xcodes + cc + 16);
      xv[c][0] = ok ? v0 : make_uint4(0u, 0u, 0u, 0u);
      xv[c][1] = ok ? v1 : make_uint4(0u, 0u, 0u, 0u);
    }
  } else if (a.xq_natural) {
    // natural-order codes: each wave holds the whole row, so it reorders
    // every 8 codes into the permuted layout and sums the row itself
    load_x_codes<NCH, MASKED>(a.xq + (int64_t)s * a.D, a.D, xv);
    sxs = a.sx[s];
    gu_load<NCH, MASKED, ROWS>(res, a.I, rowbytes, first, hi, dummy, sa);
    int part = 0;
#pragma unroll
    for (int c = 0; c < NCH; c++)
#pragma unroll
      for (int h = 0; h < 2; h++) {
        uint4 &v = xv[c][h];
        const uint32_t e0 = __builtin_amdgcn_perm(v.y, v.x, 0x06040200u);
        const uint32_t o0 = __builtin_amdgcn_perm(v.y, v.x, 0x07050301u);
        const uint32_t e1 = __builtin_amdgcn_perm(v.w, v.z, 0x06040200u);
        const uint32_t o1 = __builtin_amdgcn_perm(v.w, v.z, 0x07050301u);
        v = make_uint4(e0, o0, e1, o1);
        part = dot4((int)e0, 0x01010101, part);
        part = dot4((int)o0, 0x01010101, part);
        part = dot4((int)e1, 0x01010101, part);
        part = dot4((int)o1, 0x01010101, part);
      }
    sumx = wave_sum_i32(part);
  } else {
    load_x_codes<NCH, MASKED>(a.xq + (int64_t)s * a.D, a.D, xv);
    sxs = a.sx[s];
    sumx = a.sumx[s];
    gu_load<NCH, MASKED, ROWS>(res, a.I, rowbytes, first, hi, dummy, sa);
  }
  // int8 codes are signed: no offset to remove
  gu_items<NCH, MASKED, ROWS, decltype(res), W8>(res, a.I, rowbytes, lo, hi, xv,
                                                 W8 ? 0 : 8 * sumx, sxs, L,
                                                 acc_gu ? acco : nullptr, acc_gu, dummy, sa);
}

// Routed experts of token s: the block runs the token's K selection rounds
// once (block 0 publishes them), or reads the caller's selection, then works
// through its share of the concatenated rows of the K selected experts.
template <int NCH, bool MASKED, int ROWS>
__device__ void gateup_routed(const DecodeArgs &a, int s, int gb) {
  __shared__ int sel[64];
  __shared__ int keff;
  __shared__ GuLds L;
  const int wave = threadIdx.x >> 6;
  const int rowbytes = a.D >> 1;
  uint4 xv[NCH][2];
  load_x_codes<NCH, MASKED>(a.xq + (int64_t)s * a.D, a.D, xv);
  const int corr = 8 * a.sumx[s];
  const float sxs = a.sx[s];
  if (a.given) {
    if ((int)threadIdx.x < a.K) sel[threadIdx.x] = expert_at(a, (int64_t)s * a.K + threadIdx.x);
    if (threadIdx.x == 0) keff = a.K;
  } else if (wave == 0) {
    const bool pub = (gb == 0);
    topk_rounds(a.logits + (int64_t)s * a.E, a.bias, a.E, a.K, a.scale,
                pub ? a.idx + (int64_t)s * a.K : nullptr, pub ? a.w + (int64_t)s * a.K : nullptr,
                sel, a.topp, &keff);
  }
  __syncthreads();
  // with top-p the block's share is taken from the kept slots only (every
  // block computed the same keff); block 0 publishes it for phase C
  if (gb == 0 && threadIdx.x == 0 && a.keff) a.keff[s] = keff;
  const ExpertSet &rt = a.rt;
  float *hbase = a.h + (int64_t)s * a.P * a.I;
  const int I = a.I;
  auto res = [&](int slot) {
    GuMats m;
    const int e = sel[slot];
    m.G = pick(rt.gate, rt.gate, false, e);
    m.U = pick(rt.up, rt.up, false, e);
    m.h = hbase + (int64_t)slot * I;
    return m;
  };
  int lo, hi;
  split_rows(keff * a.I, a.n_gu_rt, gb, lo, hi);
  const int first = lo + wave * ROWS;
  const uint8_t *dummy = reinterpret_cast<const uint8_t *>(a.xq + (int64_t)s * a.D);
  GuStage<NCH, ROWS> sa;
  gu_load<NCH, MASKED, ROWS>(res, I, rowbytes, first, hi, dummy, sa);
  gu_items<NCH, MASKED, ROWS>(res, I, rowbytes, lo, hi, xv, corr, sxs, L, nullptr, nullptr, dummy,
                              sa);
}

// ---- down rows ----------------------------------------------------------------------

#define MOE_DOWN_MAXP 8
// Most rows a down block may own (its scales, combine inputs and outputs sit
// in LDS).
#define MOE_DN_MAX_ROWS 256

struct DownTask {
  int np;                         // slots (<= PMAX of the kernel)
  RowPtr M[MOE_DOWN_MAXP];        // down matrices (all valid, also past np)
  float wgt[MOE_DOWN_MAXP];       // combine weights
  bool weighted[MOE_DOWN_MAXP];   // false: added with weight 1
  const float *h[MOE_DOWN_MAXP];  // hidden rows (I floats; all valid)
  int d0, d1;                     // rows of this block
  const float *init;              // optional running combine to continue (D floats)
  const float *extra;             // optional row added after the slots (D floats)
  float *out;                     // D floats
  bool accumulate;                // out = out + result
  int32_t *acc_d;                 // optional (single slot)
  int8_t *hq_nat;                 // optional (single slot), first block only
  float *sh_out;                  // optional (single slot), first block only
  bool first_block;
};

// Requantize the slots' hidden rows (section 12 rule) into LDS codes in the
// permuted layout: one round of loads for all slots, the row maxima reduced
// across the block, then the codes.  Scales go to sh[], code sums to sums[].
// NCH bounds the groups of 8 per thread: I <= 2048*NCH with 256 threads.
template <int PMAX, int NCH>
__device__ void requant_to_lds(const DownTask &t, int I, int8_t *lds, float *sh, int *sums) {
  __shared__ float redm[PMAX][kWaves];
  __shared__ int reds[PMAX][kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ngroups = I >> 3;
  float4 hv[PMAX][NCH][2];
#pragma unroll
  for (int p = 0; p < PMAX; p++)
#pragma unroll
    for (int k = 0; k < NCH; k++) {
      // unconditional loads (index clamped; every t.h[p] is a valid row)
      const int g = tid + k * 64 * kWaves;
      const bool ok = (p < t.np) && (g < ngroups);
      const int gc = min(g, ngroups - 1);
      const float4 v0 = reinterpret_cast<const float4 *>(t.h[p])[2 * gc];
      const float4 v1 = reinterpret_cast<const float4 *>(t.h[p])[2 * gc + 1];
      const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
      hv[p][k][0] = ok ? v0 : z;
      hv[p][k][1] = ok ? v1 : z;
    }
#pragma unroll
  for (int p = 0; p < PMAX; p++) {
    float m = 0.f;
#pragma unroll
    for (int k = 0; k < NCH; k++)
#pragma unroll
      for (int j = 0; j < 2; j++) {
        m = fmax_nan_skip(m, fabsf(hv[p][k][j].x));
        m = fmax_nan_skip(m, fabsf(hv[p][k][j].y));
        m = fmax_nan_skip(m, fabsf(hv[p][k][j].z));
        m = fmax_nan_skip(m, fabsf(hv[p][k][j].w));
      }
    m = wave_max_f32(m);
    if (lane == 0) redm[p][wave] = m;
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < PMAX; p++) {
    const float m = fmax_nan_skip(fmax_nan_skip(redm[p][0], redm[p][1]),
                                  fmax_nan_skip(redm[p][2], redm[p][3]));
    const float sc = quant_scale(m);
    const float inv = 1.f / sc;
    uint2 *dst = reinterpret_cast<uint2 *>(lds + p * I);
    int sum = 0;
#pragma unroll
    for (int k = 0; k < NCH; k++) {
      const int g = tid + k * 64 * kWaves;
      const float4 x0 = hv[p][k][0], x1 = hv[p][k][1];
      const int q0 = quant_code(x0.x, inv), q1 = quant_code(x0.y, inv), q2 = quant_code(x0.z, inv),
                q3 = quant_code(x0.w, inv), q4 = quant_code(x1.x, inv), q5 = quant_code(x1.y, inv),
                q6 = quant_code(x1.z, inv), q7 = quant_code(x1.w, inv);
      sum += ((q0 + q1) + (q2 + q3)) + ((q4 + q5) + (q6 + q7));
      if (g < ngroups) {
        dst[g] = make_uint2(pack4(q0, q2, q4, q6), pack4(q1, q3, q5, q7));
        if (t.hq_nat && t.first_block)
          reinterpret_cast<uint2 *>(t.hq_nat)[g] =
              make_uint2(pack4(q0, q1, q2, q3), pack4(q4, q5, q6, q7));
      }
    }
    sum = wave_sum_i32(sum);
    if (lane == 0) reds[p][wave] = sum;
    if (tid == 0) {
      sh[p] = sc;
      if (t.sh_out && t.first_block) *t.sh_out = sc;
    }
  }
  __syncthreads();
  if (tid < PMAX) sums[tid] = (reds[tid][0] + reds[tid][1]) + (reds[tid][2] + reds[tid][3]);
  __syncthreads();
}

// One pipeline stage of the down projection: ROWS rows of every slot's
// weights (the only global loads of the loop body, see the gate/up notes).
template <int NCH, int ROWS, int PMAX>
struct DnStage {
  uint4 w[PMAX][ROWS][NCH];
};

template <int NCH, bool MASKED, int ROWS, int PMAX>
__device__ __forceinline__ void dn_load(const DownTask &t, int rowbytes, int row,
                                        const uint8_t *dummy, DnStage<NCH, ROWS, PMAX> &st) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int p = 0; p < PMAX; p++) {
#pragma unroll
    for (int r = 0; r < ROWS; r++) {
      const int d = row + r;
      const bool live = (d < t.d1) && (p < t.np);  // uniform across the wave
      const uint8_t *wr = live ? t.M[p].q + (int64_t)d * rowbytes : dummy;
#pragma unroll
      for (int c = 0; c < NCH; c++) {
        const int off = c * 1024 + lane * 16;
        const bool ok = !MASKED || off < rowbytes;
        st.w[p][r][c] = ldnt16(wr + off, ok, wr);
      }
    }
  }
}

// Row scales of every slot for the block's rows, and the combine's running
// value and final addend, into LDS (one round of loads).
template <int PMAX>
__device__ __forceinline__ void dn_scales(const DownTask &t, float (*dsc)[MOE_DN_MAX_ROWS],
                                          float *init, float *extra) {
  const int n = t.d1 - t.d0;
  for (int i0 = 0; i0 < n; i0 += 64 * kWaves) {
    const int i = i0 + threadIdx.x;
    const int d = t.d0 + min(i, n - 1);
    float v[PMAX];
#pragma unroll
    for (int p = 0; p < PMAX; p++) v[p] = t.M[p].s[d];
    const float vi = t.init ? t.init[d] : 0.f;
    const float ve = t.extra ? t.extra[d] : 0.f;
    if (i < n) {
#pragma unroll
      for (int p = 0; p < PMAX; p++) dsc[p][i] = v[p];
      init[i] = vi;
      extra[i] = ve;
    }
  }
}

struct DnLds {
  float sh[MOE_DOWN_MAXP];
  int sums[MOE_DOWN_MAXP];
  float dsc[MOE_DOWN_MAXP][MOE_DN_MAX_ROWS];
  float init[MOE_DN_MAX_ROWS], extra[MOE_DN_MAX_ROWS], out[MOE_DN_MAX_ROWS];
  int accd[MOE_DN_MAX_ROWS];
};

// W8: the rows are int8 codes (lane l of chunk c: columns 1024c + 16l .. +16).
template <int NCH, bool MASKED, int ROWS, int PMAX, bool W8 = false>
__device__ __forceinline__ void dn_step(const DownTask &t, const DnStage<NCH, ROWS, PMAX> &st,
                                        const int8_t *codes, DnLds &L, int I, int row) {
  const int lane = threadIdx.x & 63;
  const int rowbytes = W8 ? I : I >> 1;
  const int i0 = row - t.d0;
  const int n = t.d1 - t.d0;
  float comb[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; r++) comb[r] = L.init[min(i0 + r, n - 1)];
#pragma unroll
  for (int p = 0; p < PMAX; p++) {
    uint4 hv[NCH][2];
#pragma unroll
    for (int c = 0; c < NCH; c++) {
      const int off = c * 1024 + lane * 16;
      const int offc = (!MASKED || off < rowbytes) ? off : 0;
      const int col = W8 ? offc : 2 * offc;  // first column of the lane's bytes
      hv[c][0] = *reinterpret_cast<const uint4 *>(codes + p * I + col);
      hv[c][1] = W8 ? hv[c][0] : *reinterpret_cast<const uint4 *>(codes + p * I + col + 16);
      if (MASKED && off >= rowbytes) {
        hv[c][0] = make_uint4(0u, 0u, 0u, 0u);
        hv[c][1] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
    const int corr = W8 ? 0 : 8 * L.sums[p];  // int8 codes are signed
    const float shs = L.sh[p];
    const bool use = p < t.np;
#pragma unroll
    for (int r = 0; r < ROWS; r++) {
      int acc = 0;
#pragma unroll
      for (int c = 0; c < NCH; c++)
        acc = W8 ? dot16_i8p(st.w[p][r][c], hv[c][0], acc)
                 : dot32_i4(st.w[p][r][c], hv[c][0], hv[c][1], acc);
      acc = wave_sum_i32(acc) - corr;
      const float y = ((float)acc * L.dsc[p][min(i0 + r, n - 1)]) * shs;
      const float nc = t.weighted[p] ? comb[r] + t.wgt[p] * y : comb[r] + y;
      comb[r] = use ? nc : comb[r];
      if (lane == r && i0 + r < n) L.accd[i0 + r] = acc;  // meaningful for single-slot calls
    }
  }
  float mine = comb[0];
#pragma unroll
  for (int r = 1; r < ROWS; r++)
    if (lane == r) mine = comb[r];
  if (lane < ROWS && i0 + lane < n) L.out[i0 + lane] = mine;
}

template <int NCH, bool MASKED, int ROWS, int PMAX, bool W8 = false>
__device__ void down_block(const DownTask &t, int I) {
  // chunks of 2048 columns per thread in the requantization
  constexpr int NR = W8 ? (NCH + 1) / 2 : NCH;
  extern __shared__ __align__(16) int8_t codes[];
  __shared__ DnLds L;
  const int wave = threadIdx.x >> 6;
  const int rowbytes = W8 ? I : I >> 1;
  const int stride = kWaves * ROWS;
  const int first = t.d0 + wave * ROWS;
  const int nsteps = (first < t.d1) ? (t.d1 - first + stride - 1) / stride : 0;
  const uint8_t *dummy = reinterpret_cast<const uint8_t *>(t.h[0]);
  DnStage<NCH, ROWS, PMAX> sa, sb;
  dn_scales<PMAX>(t, L.dsc, L.init, L.extra);
  // the first step's weights do not depend on the hidden rows: issue them early
  dn_load<NCH, MASKED, ROWS, PMAX>(t, rowbytes, first, dummy, sa);
  requant_to_lds<PMAX, NR>(t, I, codes, L.sh, L.sums);  // ends with a barrier
  for (int i = 0; i < nsteps; i += 2) {
    const int ra = first + i * stride, rb = ra + stride;
    dn_load<NCH, MASKED, ROWS, PMAX>(t, rowbytes, rb, dummy, sb);
    dn_step<NCH, MASKED, ROWS, PMAX, W8>(t, sa, codes, L, I, ra);
    dn_load<NCH, MASKED, ROWS, PMAX>(t, rowbytes, rb + stride, dummy, sa);
    if (i + 1 < nsteps) dn_step<NCH, MASKED, ROWS, PMAX, W8>(t, sb, codes, L, I, rb);
  }
  __syncthreads();
  const int n = t.d1 - t.d0;
  for (int i = threadIdx.x; i < n; i += 64 * kWaves) {
    const int d = t.d0 + i;
    float v = L.out[i];
    if (t.extra) v = v + L.extra[i];
    t.out[d] = t.accumulate ? (t.out[d] + v) : v;
    if (t.acc_d) t.acc_d[d] = L.accd[i];
  }
}

// Down projection of the fixed expert for token s, rows of block db (W8: the
// int8 fixed expert a.f8d; NCH = 1 KB chunks of an I-byte row).
template <int NCH, bool MASKED, int ROWS, bool W8 = false>
__device__ void down_fixed(const DecodeArgs &a, int s, int db) {
  DownTask t;
  const int pair = s * a.P + a.fx_slot;
  t.np = 1;
#pragma unroll
  for (int j = 0; j < MOE_DOWN_MAXP; j++) {
    t.M[j] = W8 ? a.f8d : pick(a.fx.down, a.fx.down, false, a.fx_index);
    t.wgt[j] = 1.f;
    t.weighted[j] = false;
    t.h[j] = a.h + (int64_t)pair * a.I;
  }
  split_rows(a.D, a.n_dn_fx, db, t.d0, t.d1);
  t.init = nullptr;
  t.extra = nullptr;
  t.out = a.ysh + (int64_t)s * a.D;
  t.accumulate = false;
  t.acc_d = a.acc_d ? a.acc_d + (int64_t)s * a.D : nullptr;
  t.hq_nat = a.hq_nat ? a.hq_nat + (int64_t)s * a.I : nullptr;
  t.sh_out = a.sh_out ? a.sh_out + s : nullptr;
  t.first_block = (db == 0);
  down_block<NCH, MASKED, ROWS, 1, W8>(t, a.I);
}

#ifndef MOE_DNFX_ROWS
#define MOE_DNFX_ROWS 2
#endif

// ---- the three launches ----------------------------------------------------------------

#ifndef MOE_GU_ROWS
#define MOE_GU_ROWS 1
#endif

// With a.gamma set every workgroup of phase A first forms the token's RMSNorm
// row in dynamic shared memory (D floats) and works on that.
// W8: the fixed expert is in the int8 format (NCHD = 1 KB chunks of its
// D-byte rows).
template <int NCHD, bool MD, bool LOCALQ, bool W8 = false>
__global__ __launch_bounds__(256) void decode_a_kernel(DecodeArgs a) {
  extern __shared__ __align__(16) float xn_dyn[];
  const int s = blockIdx.y, b = blockIdx.x;
  const float *xrow = a.x + (int64_t)s * a.D;
  if (b < a.n_router + a.n_quant && a.gamma) {
    NormRow nr;
    norm_row_load(xrow, a.gamma, a.D, nr);
    prenorm_finish_lds(nr, a.D, a.eps, xn_dyn);
    xrow = xn_dyn;
  }
  if (b < a.n_router) {
    const int wave = threadIdx.x >> 6;
    if (wave < kARouterWaves) router_logit(a, xrow, s, b * kARouterWaves + wave);
    return;
  }
  if (b < a.n_router + a.n_quant) {
    quant_row_block(xrow, nullptr, a.D, const_cast<int8_t *>(a.xq) + (int64_t)s * a.D, nullptr,
                    const_cast<float *>(a.sx) + s, const_cast<int32_t *>(a.sumx) + s);
    return;
  }
  gateup_fixed<NCHD, MD, MOE_GU_ROWS, LOCALQ, W8>(a, s, b - a.n_router - a.n_quant, xn_dyn);
}

// W8: the fixed expert's down rows are int8 (NCHI = 1 KB chunks of I bytes).
template <int NCHD, bool MD, int NCHI, bool MI, bool W8 = false>
__global__ __launch_bounds__(256) void decode_b_kernel(DecodeArgs a) {
  const int s = blockIdx.y, b = blockIdx.x;
  if (b < a.n_gu_rt) {
    gateup_routed<NCHD, MD, MOE_GU_ROWS>(a, s, b);
    return;
  }
  down_fixed<NCHI, MI, MOE_DNFX_ROWS, W8>(a, s, b - a.n_gu_rt);
}

// ---- phase C: routed down + combine ---------------------------------------------
//
// A phase C workgroup has 8 waves, one per routed slot of the launch, and
// owns RB consecutive output rows per pass.  Wave p holds slot p's whole
// hidden row across its lanes (lane l: columns 2048c + 32l .. +32), so it
// requantizes the row by itself (section 12 rule, the same bits as any other
// quantization of that row) and keeps the codes in registers: no workgroup
// barrier until the combine.  The hidden row is loaded first and all of the
// pass's weight rows right after it, so the requantization runs while the
// weights stream in.  Each wave leaves its RB partial outputs y_p in LDS;
// then lane r of the workgroup forms row r's combine: running value, slots
// in ascending order (weight * y_p), then the extra row.
constexpr int kCWaves = 8;

int decode_c_slots(int) { return kCWaves; }

#ifndef MOE_C_RB1
#define MOE_C_RB1 24
#endif
// rows per pass for NCH 1 KB chunks of a weight row (at most 96 registers of
// weights)
template <int NCH>
struct CRows {
  static constexpr int value = NCH == 1 ? MOE_C_RB1 : (NCH == 2 ? 12 : (NCH == 3 ? 6 : 4));
};

int decode_c_rows_per_pass(int I) {
  const int nch = (I / 2 + 1023) / 1024;
  return nch == 1 ? MOE_C_RB1 : (nch == 2 ? 12 : (nch == 3 ? 6 : 4));
}

template <int NCH, bool MASKED>
__global__ __launch_bounds__(64 * kCWaves) void decode_c_kernel(DecodeArgs a) {
  constexpr int RB = CRows<NCH>::value;
  __shared__ float ys[kCWaves][RB];
  // lane partial sums of the wave's rows, summed across lanes by lane r
  // (one read of 64 values instead of a reduction tree per row)
  __shared__ __align__(16) int part[kCWaves][RB][64];
  const int s = blockIdx.y, db = blockIdx.x;
  const int lane = threadIdx.x & 63, p = threadIdx.x >> 6;
  // routed slots of this launch that the token keeps (top-p); the wave's
  // slot does not depend on it, so the index and keff loads go out together
  const int keff = a.keff ? a.keff[s] : a.K;
  const int np = max(0, min(a.p_hi, keff) - a.p_lo);
  const bool live = p < np;  // uniform across the wave
  const int slot = a.p_lo + min(p, a.p_hi - a.p_lo - 1);
  const int e = expert_at(a, (int64_t)s * a.K + slot);
  const RowPtr M = pick(a.rt.down, a.rt.down, false, e);
  const float *hrow = a.h + ((int64_t)s * a.P + slot) * a.I;
  const int rowbytes = a.I >> 1;
  int d0, d1;
  split_rows(a.D, a.n_dn, db, d0, d1);

  float4 xf[NCH][8];
  load_x_f32<NCH, MASKED>(hrow, a.I, xf);
  uint4 w[RB][NCH];
  float dsc;
  auto load_pass = [&](int base) {
#pragma unroll
    for (int r = 0; r < RB; r++) {
      const int d = base + r;
      const uint8_t *wr = (live && d < d1) ? M.q + (int64_t)d * rowbytes
                                           : reinterpret_cast<const uint8_t *>(hrow);
#pragma unroll
      for (int c = 0; c < NCH; c++) {
        const int off = c * 1024 + lane * 16;
        const bool ok = !MASKED || off < rowbytes;
        w[r][c] = ldnt16(wr + off, ok, wr);
      }
    }
    dsc = M.s[min(base + min(lane, RB - 1), d1 - 1)];
  };
  int base = d0;
  load_pass(base);
  uint4 xv[NCH][2];
  float sh;
  const int corr = 8 * quant_x_wave<NCH>(xf, xv, &sh);
  const float *init = a.c_first ? nullptr : a.tmp + (int64_t)s * a.D;
  const bool last = a.c_last;
  const float *extra = (last && a.P > a.K) ? a.ysh + (int64_t)s * a.D : nullptr;
  float *out = last ? a.out + (int64_t)s * a.D : a.tmp + (int64_t)s * a.D;
  const bool accumulate = last && (a.flags & MOE_F_ACCUMULATE);
  for (;;) {
#pragma unroll
    for (int r = 0; r < RB; r++) {
      int acc = 0;
#pragma unroll
      for (int c = 0; c < NCH; c++) acc = dot32_i4(w[r][c], xv[c][0], xv[c][1], acc);
      part[p][r][lane] = acc;
    }
    // shared memory is in order within a wave: lane r reads its row's 64
    // partial sums after the wave's writes
    int mine = 0;
    if (lane < RB) {
      const int4 *pr = reinterpret_cast<const int4 *>(part[p][lane]);
      int4 t[16];
#pragma unroll
      for (int i = 0; i < 16; i++) t[i] = pr[i];
#pragma unroll
      for (int i = 0; i < 16; i++) mine += (t[i].x + t[i].y) + (t[i].z + t[i].w);
      ys[p][lane] = ((float)(mine - corr) * dsc) * sh;
    }
    __syncthreads();
    const int d = base + threadIdx.x;
    if (threadIdx.x < RB && d < d1) {
      float comb = init ? init[d] : 0.f;
      for (int q = 0; q < np; q++) comb = comb + a.w[s * a.K + a.p_lo + q] * ys[q][threadIdx.x];
      float v = comb;
      if (extra) v = v + extra[d];
      out[d] = accumulate ? (out[d] + v) : v;
    }
    base += RB;
    if (base >= d1) break;
    __syncthreads();  // ys is rewritten by the next pass
    load_pass(base);
  }
}

// ---- launchers -----------------------------------------------------------------------

// Plain launch, or, when an event is given, a launch whose dispatch itself
// records the kernel's start (e0) and end (e1) timestamps.
template <class F>
static void launch_timed(F kernel, dim3 grid, dim3 block, size_t lds, hipStream_t st, hipEvent_t e0,
                         hipEvent_t e1, const DecodeArgs &a) {
  if (e0 || e1)
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, st, e0, e1, 0u, a);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, st, a);
}

// Column dispatch: NCH 1 KB chunks per row, masked when the row is not a whole
// number of chunks.
#define MOE_COLS(RB, F)                                         \
  do {                                                          \
    const int nch_ = ((RB) + 1023) / 1024;                      \
    const bool msk_ = ((RB) % 1024) != 0;                       \
    if (msk_) {                                                 \
      if (nch_ == 1) F(1, true); else if (nch_ == 2) F(2, true); \
      else if (nch_ == 3) F(3, true); else F(4, true);          \
    } else {                                                    \
      if (nch_ == 1) F(1, false); else if (nch_ == 2) F(2, false); \
      else if (nch_ == 3) F(3, false); else F(4, false);        \
    }                                                           \
  } while (0)


hipError_t launch_decode_a(const DecodeArgs &a, bool local_quant, hipStream_t st) {
  const dim3 grid(a.n_router + a.n_quant + a.n_gu_fx, a.S);
  const int rb = a.D / 2;
  const size_t lds = a.gamma ? (size_t)a.D * 4 : 0;  // the normalized row
  if (a.fx8) {
    // int8 fixed expert: D-byte rows, D % 2048 == 0 and D <= 8192 (checked
    // by the caller), so 2, 4, 6 or 8 whole 1 KB chunks
    switch (a.D / 1024) {
      case 2: hipLaunchKernelGGL((decode_a_kernel<2, false, true, true>), grid, dim3(256), lds, st, a); break;
      case 4: hipLaunchKernelGGL((decode_a_kernel<4, false, true, true>), grid, dim3(256), lds, st, a); break;
      case 6: hipLaunchKernelGGL((decode_a_kernel<6, false, true, true>), grid, dim3(256), lds, st, a); break;
      case 8: hipLaunchKernelGGL((decode_a_kernel<8, false, true, true>), grid, dim3(256), lds, st, a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
#define MOE_FA(N, M)                                                                     \
  do {                                                                                   \
    if (local_quant)                                                                     \
      hipLaunchKernelGGL((decode_a_kernel<N, M, true>), grid, dim3(256), lds, st, a);    \
    else                                                                                 \
      hipLaunchKernelGGL((decode_a_kernel<N, M, false>), grid, dim3(256), lds, st, a);   \
  } while (0)
  MOE_COLS(rb, MOE_FA);
#undef MOE_FA
  return hipGetLastError();
}

template <int ND>
static hipError_t launch_decode_b8(const DecodeArgs &a, dim3 grid, size_t lds, hipStream_t st,
                                   hipEvent_t e0, hipEvent_t e1) {
  // int8 fixed expert: I-byte down rows, I % 1024 == 0 and I <= 4096
  switch (a.I / 1024) {
    case 1: launch_timed((decode_b_kernel<ND, false, 1, false, true>), grid, dim3(256), lds, st, e0, e1, a); break;
    case 2: launch_timed((decode_b_kernel<ND, false, 2, false, true>), grid, dim3(256), lds, st, e0, e1, a); break;
    case 3: launch_timed((decode_b_kernel<ND, false, 3, false, true>), grid, dim3(256), lds, st, e0, e1, a); break;
    case 4: launch_timed((decode_b_kernel<ND, false, 4, false, true>), grid, dim3(256), lds, st, e0, e1, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_b(const DecodeArgs &a, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  const dim3 grid(a.n_gu_rt + a.n_dn_fx, a.S);
  const size_t lds = (size_t)a.I;  // one hidden row of codes
  const int rbd = a.D / 2, rbi = a.I / 2;
  if (a.fx8) {
    // routed int4 rows of D/2 bytes, D % 2048 == 0 and D <= 8192: 1 to 4 whole chunks
    switch (a.D / 2048) {
      case 1: return launch_decode_b8<1>(a, grid, lds, st, e0, e1);
      case 2: return launch_decode_b8<2>(a, grid, lds, st, e0, e1);
      case 3: return launch_decode_b8<3>(a, grid, lds, st, e0, e1);
      case 4: return launch_decode_b8<4>(a, grid, lds, st, e0, e1);
      default: return hipErrorInvalidValue;
    }
  }
#define MOE_FBI(NI, MI, ND, MD) \
  launch_timed((decode_b_kernel<ND, MD, NI, MI>), grid, dim3(256), lds, st, e0, e1, a)
#define MOE_FBD(ND, MD)                                          \
  do {                                                           \
    const int nchi_ = (rbi + 1023) / 1024;                       \
    const bool mski_ = (rbi % 1024) != 0;                        \
    if (mski_) {                                                 \
      if (nchi_ == 1) MOE_FBI(1, true, ND, MD);                  \
      else if (nchi_ == 2) MOE_FBI(2, true, ND, MD);             \
      else if (nchi_ == 3) MOE_FBI(3, true, ND, MD);             \
      else MOE_FBI(4, true, ND, MD);                             \
    } else {                                                     \
      if (nchi_ == 1) MOE_FBI(1, false, ND, MD);                 \
      else if (nchi_ == 2) MOE_FBI(2, false, ND, MD);            \
      else if (nchi_ == 3) MOE_FBI(3, false, ND, MD);            \
      else MOE_FBI(4, false, ND, MD);                            \
    }                                                            \
  } while (0)
  MOE_COLS(rbd, MOE_FBD);
#undef MOE_FBD
#undef MOE_FBI
  return hipGetLastError();
}

template <int N, bool M>
static void launch_c(const DecodeArgs &a, dim3 grid, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  launch_timed((decode_c_kernel<N, M>), grid, dim3(64 * kCWaves), 0, st, e0, e1, a);
}

hipError_t launch_decode_c(const DecodeArgs &a, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  const dim3 grid(a.n_dn, a.S);
  const int rb = a.I / 2;
#define MOE_FC(N, M) launch_c<N, M>(a, grid, st, e0, e1)
  MOE_COLS(rb, MOE_FC);
#undef MOE_FC
  return hipGetLastError();
}

}  // namespace moe
