// grouped.hip -- the unique-expert union path (section 11 of the reader.mx
// article "惊呆了！25GB 内存上运行 GLM 5.2 744B 模型"): the (token, slot)
// pairs of a batch are grouped by expert on the device, each selected expert's
// weight rows are loaded once into registers and applied to every token of its
// group, and the per-pair outputs are staged and combined per token in
// selection order.
#include "moe_kernels.h"
#include "topk.h"

namespace moe {

// Requantize one hidden row h[0..I) (section 12 rule) into the permuted int8
// layout; the whole block takes part.  Returns nothing; thread 0 writes the
// scale and the code sum.
__device__ void requant_row_block(const float *h, int I, int8_t *hq_perm, int8_t *hq_nat,
                                  float *sh_out, float *sh_out2, int32_t *sumh_out) {
  __shared__ float red_f[4];
  __shared__ int red_i[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ngroups = I >> 3;
  const float4 *h4 = reinterpret_cast<const float4 *>(h);
  float m = 0.f;
  for (int g = tid; g < ngroups; g += blockDim.x) {
    float4 a = h4[2 * g], b = h4[2 * g + 1];
    float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; i++) {
      float t = fabsf(v[i]);
      m = (t > m) ? t : m;
    }
  }
  m = wave_max_f32(m);
  if (lane == 0) red_f[wave] = m;
  __syncthreads();
  float amax = red_f[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); i++) amax = (red_f[i] > amax) ? red_f[i] : amax;
  const float s = quant_scale(amax);
  const float inv = 1.f / s;
  int sum = 0;
  for (int g = tid; g < ngroups; g += blockDim.x) {
    float4 a = h4[2 * g], b = h4[2 * g + 1];
    float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    int q[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
      q[i] = quant_code(v[i], inv);
      sum += q[i];
    }
    uint32_t pe = (q[0] & 0xFF) | ((q[2] & 0xFF) << 8) | ((q[4] & 0xFF) << 16) | ((uint32_t)(q[6] & 0xFF) << 24);
    uint32_t po = (q[1] & 0xFF) | ((q[3] & 0xFF) << 8) | ((q[5] & 0xFF) << 16) | ((uint32_t)(q[7] & 0xFF) << 24);
    reinterpret_cast<uint2 *>(hq_perm)[g] = make_uint2(pe, po);
    if (hq_nat) {
      uint32_t n0 = (q[0] & 0xFF) | ((q[1] & 0xFF) << 8) | ((q[2] & 0xFF) << 16) | ((uint32_t)(q[3] & 0xFF) << 24);
      uint32_t n1 = (q[4] & 0xFF) | ((q[5] & 0xFF) << 8) | ((q[6] & 0xFF) << 16) | ((uint32_t)(q[7] & 0xFF) << 24);
      reinterpret_cast<uint2 *>(hq_nat)[g] = make_uint2(n0, n1);
    }
  }
  sum = wave_sum_i32(sum);
  if (lane == 0) red_i[wave] = sum;
  __syncthreads();
  if (tid == 0) {
    int t = 0;
    for (int i = 0; i < (int)(blockDim.x >> 6); i++) t += red_i[i];
    *sh_out = s;
    if (sh_out2) *sh_out2 = s;
    *sumh_out = t;
  }
}

__global__ __launch_bounds__(256) void requant_kernel(RequantArgs a) {
  const int64_t r = blockIdx.x;
  requant_row_block(a.h + r * a.I, a.I, a.hq + r * a.I, nullptr, a.sh_scale + r, nullptr,
                    a.sumh + r);
}

// Exclusive prefix sums over up to 2048 slots in a workgroup of 1024 threads:
// thread t holds the values of slots 2t and 2t + 1 and receives their
// offsets; every wave scans its 128 slots at once (shuffles), then adds the
// totals of the waves before it.  Returns the total to every thread.
__device__ __forceinline__ int scan_2048(int v0, int v1, int *wtot, int &e0, int &e1) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int two = v0 + v1;
  int incl = two;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(incl, d, 64);
    if (lane >= d) incl += t;
  }
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < 16; w++) {
    const int x = wtot[w];
    before += w < wave ? x : 0;
    total += x;
  }
  e0 = before + incl - two;
  e1 = e0 + v0;
  __syncthreads();  // wtot may be reused
  return total;
}

// One block of 1024 threads: (optionally the top-K of every token, then) a
// counting sort of the S*K routed pairs by expert, plus the shared expert as
// group E holding every token.  The order of pairs
// inside a group is whatever the shared-memory atomics produce; it does not
// affect any result, because each pair is computed on its own.  Each thread
// requests the expert ids of up to 8 pairs before it counts or places them,
// so the global loads overlap; a long list is assembled in shared memory
// when it fits, so that it reaches global memory in coalesced stores.
constexpr int kGroupStage = 24576;  // pairs the shared-memory list holds (96 KB)

__global__ __launch_bounds__(1024) void group_kernel(GroupArgs a) {
  constexpr int U = 8;  // pairs per thread and round
  __shared__ int cnt[2048];
  __shared__ int fill[2048];
  __shared__ int off[2048];
  __shared__ int wtot[16];
  __shared__ int pstage[kGroupStage];
  const int G = a.E + 1;  // group E is the shared expert (empty without one)
  const int t = threadIdx.x;
  if (a.with_topk) {
    // the tokens' selections (E <= 256), one wave per token; the writes are
    // visible to the whole workgroup after the barrier below
    for (int s = t >> 6; s < a.S; s += blockDim.x >> 6)
      topk_rounds_m<4>(a.logits + (int64_t)s * a.E, a.bias, a.E, a.K, a.scale,
                       a.idx + (int64_t)s * a.K, a.wts + (int64_t)s * a.K, nullptr, a.topp,
                       a.keff ? a.keff + s : nullptr);
  }
  cnt[2 * t] = cnt[2 * t + 1] = 0;
  fill[2 * t] = fill[2 * t + 1] = 0;
  __syncthreads();
  const int np = a.S * a.K;
  // the expert of pair p (kept inside [0, E)), or -1 for a pair past its
  // token's keff (adaptive top-p) or past the end
  auto expert = [&](int p) {
    if (p >= np || (a.use_keff && (p % a.K) >= a.keff[p / a.K])) return -1;
    return min(max((int)a.idx[p], 0), a.E - 1);
  };
  for (int p0 = t; p0 < np; p0 += U * 1024) {
    int ex[U];
#pragma unroll
    for (int u = 0; u < U; u++) ex[u] = expert(p0 + 1024 * u);
#pragma unroll
    for (int u = 0; u < U; u++)
      if (ex[u] >= 0) atomicAdd(&cnt[ex[u]], 1);
  }
  if (t == 0) cnt[a.E] = a.n_shared ? a.S : 0;
  __syncthreads();
  int e0, e1;
  const int np_kept = scan_2048(cnt[2 * t], cnt[2 * t + 1], wtot, e0, e1);
  off[2 * t] = e0;
  off[2 * t + 1] = e1;
  __syncthreads();
  // a long pair list is built in shared memory when it fits and then
  // written out in order (2048 tokens: about 2 us less); short ones, and
  // lists too long for it, are placed in global memory pair by pair
  const bool staged = np_kept >= 4096 && np_kept <= kGroupStage;
  auto place = [&](int pos, int v) {
    if (staged) pstage[pos] = v;
    else a.pairs[pos] = v;
  };
  for (int p0 = t; p0 < np; p0 += U * 1024) {
    int ex[U];
#pragma unroll
    for (int u = 0; u < U; u++) ex[u] = expert(p0 + 1024 * u);
#pragma unroll
    for (int u = 0; u < U; u++) {
      if (ex[u] < 0) continue;
      const int p = p0 + 1024 * u;
      place(off[ex[u]] + atomicAdd(&fill[ex[u]], 1), (p / a.K) * a.P + (p % a.K));
    }
  }
  if (a.n_shared)
    for (int s = t; s < a.S; s += blockDim.x) place(off[a.E] + s, s * a.P + a.K);
  if (staged) {
    __syncthreads();
    for (int i = t; i < np_kept; i += blockDim.x) a.pairs[i] = pstage[i];
  }
  for (int g = t; g <= G; g += blockDim.x) {
    if (g < G) a.gcount[g] = cnt[g];
    a.goff[g] = g < G ? off[g] : np_kept;
  }
  if (!a.tiles) return;
  // tiles of up to tile_rows pairs, groups in order: the same scan over the
  // tile counts of the groups
  auto ntile = [&](int g) { return g < G ? (cnt[g] + a.tile_rows - 1) / a.tile_rows : 0; };
  const int total = scan_2048(ntile(2 * t), ntile(2 * t + 1), wtot, e0, e1);
  if (t == 0) *a.ntiles = total;
#pragma unroll
  for (int h = 0; h < 2; h++) {
    const int g = 2 * t + h;
    const int nt = ntile(g);
    for (int i = 0; i < nt; i++) a.tiles[(h ? e1 : e0) + i] = make_int2(g, i * a.tile_rows);
  }
}

template <int NCH, bool MASKED, int ROWS>
__global__ __launch_bounds__(256) void grouped_gateup_kernel(GroupedGateUpArgs a) {
  const int g = blockIdx.y;
  const int n = a.gcount[g];
  if (n == 0) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool shared = (g == a.E);
  const int e = shared ? 0 : g;
  const RowPtr G = pick(a.rt.gate, a.sh.gate, shared, e);
  const RowPtr U = pick(a.rt.up, a.sh.up, shared, e);
  const int rowbytes = a.D >> 1;
  const int o0 = (blockIdx.x * 4 + wave) * ROWS;
  const uint8_t *gb = G.q, *ub = U.q;
  const int *plist = a.pairs + a.goff[g];

  uint4 wg[ROWS][NCH], wu[ROWS][NCH];
#pragma unroll
  for (int r = 0; r < ROWS; r++) {
    const int o = o0 + r;
#pragma unroll
    for (int c = 0; c < NCH; c++) {
      const int off = c * 1024 + lane * 16;
      const bool ok = (o < a.I) && (!MASKED || off < rowbytes);
      wg[r][c] = load16(gb + (int64_t)o * rowbytes + off, ok);
      wu[r][c] = load16(ub + (int64_t)o * rowbytes + off, ok);
    }
  }
  float gs = 0.f, us = 0.f;
  if (lane < ROWS && o0 + lane < a.I) {
    gs = G.s[o0 + lane];
    us = U.s[o0 + lane];
  }
  for (int t = 0; t < n; t++) {
    const int pr = plist[t];
    const int s = pr / a.P;
    const int8_t *xs = a.xq + (int64_t)s * a.D;
    uint4 xv[NCH][2];
#pragma unroll
    for (int c = 0; c < NCH; c++) {
      const int off = c * 1024 + lane * 16;
      const bool ok = !MASKED || off < rowbytes;
      xv[c][0] = load16(xs + 2 * off, ok);
      xv[c][1] = load16(xs + 2 * off + 16, ok);
    }
    int ag[ROWS], au[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; r++) {
      ag[r] = 0;
      au[r] = 0;
#pragma unroll
      for (int c = 0; c < NCH; c++) {
        ag[r] = dot32_i4(wg[r][c], xv[c][0], xv[c][1], ag[r]);
        au[r] = dot32_i4(wu[r][c], xv[c][0], xv[c][1], au[r]);
      }
      ag[r] = wave_sum_i32(ag[r]);
      au[r] = wave_sum_i32(au[r]);
    }
    int myg = ag[0], myu = au[0];
#pragma unroll
    for (int r = 1; r < ROWS; r++)
      if (lane == r) { myg = ag[r]; myu = au[r]; }
    const int o = o0 + lane;
    if (lane < ROWS && o < a.I) {
      const int corr = 8 * a.sumx[s];
      const float sxs = a.sx[s];
      const float gv = ((float)(myg - corr) * gs) * sxs;
      const float uv = ((float)(myu - corr) * us) * sxs;
      a.h[(int64_t)pr * a.I + o] = silu(gv) * uv;
    }
  }
}

template <int NCH, bool MASKED, int ROWS>
__global__ __launch_bounds__(256) void grouped_down_kernel(GroupedDownArgs a) {
  const int g = blockIdx.y;
  const int n = a.gcount[g];
  if (n == 0) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool shared = (g == a.E);
  const int e = shared ? 0 : g;
  const RowPtr M = pick(a.rt.down, a.sh.down, shared, e);
  const int rowbytes = a.I >> 1;
  const int d0 = (blockIdx.x * 4 + wave) * ROWS;
  const uint8_t *base = M.q;
  const int *plist = a.pairs + a.goff[g];

  uint4 wd[ROWS][NCH];
#pragma unroll
  for (int r = 0; r < ROWS; r++) {
    const int d = d0 + r;
#pragma unroll
    for (int c = 0; c < NCH; c++) {
      const int off = c * 1024 + lane * 16;
      const bool ok = (d < a.D) && (!MASKED || off < rowbytes);
      wd[r][c] = load16(base + (int64_t)d * rowbytes + off, ok);
    }
  }
  float ds = 0.f;
  if (lane < ROWS && d0 + lane < a.D) ds = M.s[d0 + lane];
  for (int t = 0; t < n; t++) {
    const int pr = plist[t];
    const int8_t *hs = a.hq + (int64_t)pr * a.I;
    uint4 hv[NCH][2];
#pragma unroll
    for (int c = 0; c < NCH; c++) {
      const int off = c * 1024 + lane * 16;
      const bool ok = !MASKED || off < rowbytes;
      hv[c][0] = load16(hs + 2 * off, ok);
      hv[c][1] = load16(hs + 2 * off + 16, ok);
    }
    int acc[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; r++) {
      acc[r] = 0;
#pragma unroll
      for (int c = 0; c < NCH; c++) acc[r] = dot32_i4(wd[r][c], hv[c][0], hv[c][1], acc[r]);
      acc[r] = wave_sum_i32(acc[r]);
    }
    int mine = acc[0];
#pragma unroll
    for (int r = 1; r < ROWS; r++)
      if (lane == r) mine = acc[r];
    const int d = d0 + lane;
    if (lane < ROWS && d < a.D) {
      const float y = ((float)(mine - 8 * a.sumh[pr]) * ds) * a.sh_scale[pr];
      a.stage[(int64_t)pr * a.D + d] = y;
    }
  }
}

// out[s] = sum_k w[s][k] * stage[s][k] (k ascending, from 0) + stage[s][K]
// VEC: 4 consecutive columns per thread (D % 4 == 0); the stage rows of a
// column group are loaded 4 slots at a time before they are summed, in the
// same order and with the same roundings as the scalar form.
typedef float f4v __attribute__((ext_vector_type(4)));

template <bool VEC>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int s = blockIdx.y;
  const float *wts = a.w + s * a.K;
  const int K = a.keff ? a.keff[s] : a.K;  // routed slots kept (top-p)
  if (!VEC) {
    const int d = blockIdx.x * blockDim.x + threadIdx.x;
    if (d >= a.D) return;
    const float *st = a.stage + (int64_t)s * a.P * a.D + d;
    float acc = 0.f;
    for (int k = 0; k < K; k++) acc = acc + wts[k] * st[(int64_t)k * a.D];
    if (a.n_shared) acc = acc + st[(int64_t)a.K * a.D];
    float *o = a.out + (int64_t)s * a.D + d;
    *o = (a.flags & MOE_F_ACCUMULATE) ? (*o + acc) : acc;
    return;
  }
  const int d = 4 * (blockIdx.x * blockDim.x + threadIdx.x);
  if (d >= a.D) return;
  const f4v *st = reinterpret_cast<const f4v *>(a.stage + (int64_t)s * a.P * a.D + d);
  const int64_t step = a.D / 4;
  f4v acc = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < K; k0 += 4) {
    f4v v[4];
#pragma unroll
    for (int i = 0; i < 4; i++)
      if (k0 + i < K) v[i] = __builtin_nontemporal_load(st + (int64_t)(k0 + i) * step);
#pragma unroll
    for (int i = 0; i < 4; i++)
      if (k0 + i < K) {
        const float w = wts[k0 + i];
        acc.x = acc.x + w * v[i].x;
        acc.y = acc.y + w * v[i].y;
        acc.z = acc.z + w * v[i].z;
        acc.w = acc.w + w * v[i].w;
      }
  }
  if (a.n_shared) {
    const f4v v = __builtin_nontemporal_load(st + (int64_t)a.K * step);
    acc.x = acc.x + v.x;
    acc.y = acc.y + v.y;
    acc.z = acc.z + v.z;
    acc.w = acc.w + v.w;
  }
  f4v *o = reinterpret_cast<f4v *>(a.out + (int64_t)s * a.D + d);
  if (a.flags & MOE_F_ACCUMULATE) {
    const f4v p = *o;
    acc.x = p.x + acc.x;
    acc.y = p.y + acc.y;
    acc.z = p.z + acc.z;
    acc.w = p.w + acc.w;
  }
  *o = acc;
}

#define MOE_DISPATCH_COLS(RB, LAUNCH)                         \
  do {                                                        \
    const int nch_ = ((RB) + 1023) / 1024;                    \
    if ((RB) % 1024) {                                        \
      switch (nch_) {                                         \
        case 1: LAUNCH(1, true, 1); break;                    \
        case 2: LAUNCH(2, true, 1); break;                    \
        case 3: LAUNCH(3, true, 1); break;                    \
        default: LAUNCH(4, true, 1); break;                   \
      }                                                       \
    } else {                                                  \
      switch (nch_) {                                         \
        case 1: LAUNCH(1, false, 2); break;                   \
        case 2: LAUNCH(2, false, 2); break;                   \
        case 3: LAUNCH(3, false, 2); break;                   \
        default: LAUNCH(4, false, 2); break;                  \
      }                                                       \
    }                                                         \
  } while (0)

static inline int rows_for(int rb) { return (rb % 1024) ? 1 : 2; }

hipError_t launch_requant(const RequantArgs &a, int rows, hipStream_t st) {
  hipLaunchKernelGGL(requant_kernel, dim3(rows), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_group(const GroupArgs &a, hipStream_t st) {
  hipLaunchKernelGGL(group_kernel, dim3(1), dim3(1024), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_grouped_gateup(const GroupedGateUpArgs &a, hipStream_t st) {
  const int rb = a.D / 2, rows = rows_for(rb);
  const dim3 grid((a.I + 4 * rows - 1) / (4 * rows), a.E + 1);
#define MOE_L(N, M, R) hipLaunchKernelGGL((grouped_gateup_kernel<N, M, R>), grid, dim3(256), 0, st, a)
  MOE_DISPATCH_COLS(rb, MOE_L);
#undef MOE_L
  return hipGetLastError();
}

hipError_t launch_grouped_down(const GroupedDownArgs &a, hipStream_t st) {
  const int rb = a.I / 2, rows = rows_for(rb);
  const dim3 grid((a.D + 4 * rows - 1) / (4 * rows), a.E + 1);
#define MOE_L(N, M, R) hipLaunchKernelGGL((grouped_down_kernel<N, M, R>), grid, dim3(256), 0, st, a)
  MOE_DISPATCH_COLS(rb, MOE_L);
#undef MOE_L
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs &a, hipStream_t st) {
  // the vector form needs 16-byte aligned rows of stage and out
  const bool vec = a.D % 4 == 0 && ((uintptr_t)a.stage % 16) == 0 && ((uintptr_t)a.out % 16) == 0;
  if (vec)
    hipLaunchKernelGGL(combine_kernel<true>, dim3((a.D / 4 + 255) / 256, a.S), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3((a.D + 255) / 256, a.S), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
