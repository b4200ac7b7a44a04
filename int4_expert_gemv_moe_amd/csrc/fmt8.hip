// fmt8.hip -- the int8 weight format of the reader.mx article "惊呆了！25GB
// 内存上运行 GLM 5.2 744B 模型": the section 05 per-row quantizer (one int8
// code per weight, one float scale per row) and the section 12 integer path
// for that format (int8 weights times int8 activation codes, the int32 sum
// scaled by the row scale and then by the activation scale), as a SwiGLU
// expert.
//
// The one-expert call runs in two launches: gate/up + SwiGLU (one wave per
// output row, the row's gate and up codes held in registers while the wave
// walks the tokens), then the per-row requantization of h and down (one wave
// per one to four output rows, same scheme).  Every weight byte is read once
// per call; the token codes are re-read per wave from the cache.  Rows are
// split into 16-byte pieces, lane l taking piece l of every 1024-column
// chunk, so each load instruction of a wave covers 1 KiB of one row.  That
// suits a token or a few; the union path's int8 shared expert, which sees
// every token of a batch, runs on the int8 matrix cores instead
// (shared8_mfma_kernel, shared8_tile_kernel below).
#include "moe_kernels.h"
#include "dma.h"
#include "quant.h"
#include "rowops.h"

namespace moe {

// One wave per row: s = max(amax/127, 1e-8), q = clamp(rint(w/s), -128, 127),
// w divided by s as in the article's quantizer.
__global__ __launch_bounds__(256) void quant_rows_i8_kernel(Q8QuantArgs a) {
  const int lane = threadIdx.x & 63;
  const int o = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (o >= a.O) return;
  const float *wr = a.w + (int64_t)o * a.C;
  float m = 0.f;
  for (int j = lane; j < a.C; j += 64) m = fmax_nan_skip(m, fabsf(wr[j]));
  m = wave_max_f32(m);
  float s = m / 127.f;
  if (s < 1e-8f) s = 1e-8f;
  int8_t *qr = a.q + (int64_t)o * a.C;
  for (int j = lane; j < a.C; j += 64)
    qr[j] = (int8_t)(int)fminf(fmaxf(rintf(wr[j] / s), -128.f), 127.f);
  if (lane == 0) a.scale[o] = s;
}

// 16 int8 weights against 16 int8 activation codes.
__device__ __forceinline__ int dot16_i8(const uint4 &w, const uint4 &x, int acc) {
  acc = dot4((int)w.x, (int)x.x, acc);
  acc = dot4((int)w.y, (int)x.y, acc);
  acc = dot4((int)w.z, (int)x.z, acc);
  acc = dot4((int)w.w, (int)x.w, acc);
  return acc;
}

// Gate/up: wave w of block b owns row o = 4b + w of both matrices.
// NCH = ceil(D / 1024) chunks; MASKED when D is not a multiple of 1024.
// XPERM: the token codes are in the permuted layout (the weight bytes are
// reordered to meet them, dot16_i8p).
template <int NCH, bool MASKED, bool XPERM = false>
__global__ __launch_bounds__(256) void gu8_kernel(Swiglu8Args a) {
  const int lane = threadIdx.x & 63;
  const int o = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (o >= a.I) return;
  const int8_t *gr = a.G + (int64_t)o * a.D;
  const int8_t *ur = a.U + (int64_t)o * a.D;
  uint4 g[NCH], u[NCH];
#pragma unroll
  for (int c = 0; c < NCH; c++) {
    const int col = 1024 * c + 16 * lane;
    const bool ok = !MASKED || col < a.D;
    g[c] = ldnt16(gr + col, ok, gr);
    u[c] = ldnt16(ur + col, ok, ur);
  }
  const float gs = a.gs[o], us = a.us[o];
  for (int s = 0; s < a.S; s++) {
    const int8_t *xs = a.xq + (int64_t)s * a.D;
    int ag = 0, au = 0;
#pragma unroll
    for (int c = 0; c < NCH; c++) {
      const int col = 1024 * c + 16 * lane;
      const uint4 xv = ld16(xs + col, !MASKED || col < a.D, xs);
      ag = XPERM ? dot16_i8p(g[c], xv, ag) : dot16_i8(g[c], xv, ag);
      au = XPERM ? dot16_i8p(u[c], xv, au) : dot16_i8(u[c], xv, au);
    }
    ag = wave_sum_i32(ag);
    au = wave_sum_i32(au);
    if (lane == 0) {
      const float sxs = a.sx[s];
      const float gv = ((float)ag * gs) * sxs;
      const float uv = ((float)au * us) * sxs;
      a.h[(int64_t)s * (a.h_stride ? a.h_stride : a.I) + o] = silu(gv) * uv;
      if (a.acc_gu) {
        a.acc_gu[(int64_t)s * 2 * a.I + o] = ag;
        a.acc_gu[((int64_t)s * 2 + 1) * a.I + o] = au;
      }
    }
  }
}

// Down: wave w of block b owns rows d0 .. d0+R-1, d0 = (4b + w) R.  Every
// block requantizes the rows of h it needs into shared memory (the section 12
// quantization of the down projection's input, the same bits as the
// activation quantizer), kDn8CodeBytes of codes at a time: the weight loads
// are issued first, so their latency overlaps the requantization.  Block 0
// also writes the codes and scales out when the caller asks for them.
constexpr int kDn8CodeBytes = 32768;

template <int NCH, bool MASKED, int R>
__global__ __launch_bounds__(256) void dn8_kernel(Swiglu8Args a) {
  __shared__ __align__(16) int8_t codes[kDn8CodeBytes];
  __shared__ float shs[kDn8CodeBytes / 32];  // I >= 32
  const int lane = threadIdx.x & 63;
  const int d0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * R;
  // no early exit: every wave takes part in the block's barriers
  uint4 w[R][NCH];
  float dsc[R];
#pragma unroll
  for (int r = 0; r < R; r++) {
    const int d = min(d0 + r, a.D - 1);
    const int8_t *row = a.Dn + (int64_t)d * a.I;
#pragma unroll
    for (int c = 0; c < NCH; c++) {
      const int col = 1024 * c + 16 * lane;
      w[r][c] = ldnt16(row + col, !MASKED || col < a.I, row);
    }
    dsc[r] = a.ds[d];
  }
  const int TS = kDn8CodeBytes / a.I;
  for (int s0 = 0; s0 < a.S; s0 += TS) {
    const int ns = min(TS, a.S - s0);
    __syncthreads();  // the previous chunk's codes are consumed
    const int64_t hs = a.h_stride ? a.h_stride : a.I;
    for (int j = 0; j < ns; j++)
      quant_row_block(a.h + (int64_t)(s0 + j) * hs, nullptr, a.I, nullptr, codes + j * a.I,
                      &shs[j], nullptr);
    __syncthreads();  // the scales are written by thread 0 after the last barrier
    if (blockIdx.x == 0) {
      if (a.hq_out)
        for (int i = threadIdx.x; i < ns * a.I / 16; i += 256)
          reinterpret_cast<uint4 *>(a.hq_out + (int64_t)s0 * a.I)[i] =
              reinterpret_cast<const uint4 *>(codes)[i];
      if (a.sh_out && (int)threadIdx.x < ns) a.sh_out[s0 + threadIdx.x] = shs[threadIdx.x];
    }
    for (int j = 0; j < ns; j++) {
      const int8_t *hs = codes + j * a.I;
      uint4 hv[NCH];
#pragma unroll
      for (int c = 0; c < NCH; c++) {
        const int col = 1024 * c + 16 * lane;
        hv[c] = (!MASKED || col < a.I) ? *reinterpret_cast<const uint4 *>(hs + col)
                                       : make_uint4(0u, 0u, 0u, 0u);
      }
      const float sh = shs[j];
      const int64_t s = s0 + j;
#pragma unroll
      for (int r = 0; r < R; r++) {
        int acc = 0;
#pragma unroll
        for (int c = 0; c < NCH; c++) acc = dot16_i8(w[r][c], hv[c], acc);
        acc = wave_sum_i32(acc);
        if (lane == r && d0 + r < a.D) {
          const float v = ((float)acc * dsc[r]) * sh;
          float *yp = a.y + s * (a.y_stride ? a.y_stride : a.D) + d0 + r;
          *yp = a.accumulate ? *yp + v : v;
          if (a.acc_d) a.acc_d[s * a.D + d0 + r] = acc;
        }
      }
    }
  }
}

// The int8 shared expert of the union path on int8 matrix cores
// (v_mfma_i32_16x16x64_i8; lane l supplies A[l % 16][16 (l / 16) ..] and
// B[16 (l / 16) ..][l % 16] and receives C[4 (l / 16) + i][l % 16]).  A
// workgroup takes 16 weight rows (MODE 0: the gate rows of 8 hidden units in
// columns 0..7 of the tile and their up rows in columns 8..15; MODE 1: 16
// down rows) and up to 64 tokens (16-token subtiles).  Its waves split the
// contraction, wave w of W taking 64-column steps w, w + W, ..., and add
// their int32 tiles in shared memory: integer sums, so the split changes no
// bit.
// The token codes are in the permuted layout (per 8 columns the even columns,
// then the odd ones); each 8-column group of weight bytes is permuted alike
// before the product.  Operands come straight from global memory, 16 bytes
// per lane (a weight load covers 16 rows x 64 bytes, a token load 16 tokens x
// 64 bytes), several steps of loads in flight.  Row blocks vary fastest over the
// grid, so each XCD's L2 keeps the weight rows of its blocks across token
// chunks.  The epilogues are those of gu8_kernel and dn8_kernel.
typedef int v4i8x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4i8x4 perm_i8x16(const uint4 &w) {
  return v4i8x4{(int)__builtin_amdgcn_perm(w.y, w.x, 0x06040200u),
                (int)__builtin_amdgcn_perm(w.y, w.x, 0x07050301u),
                (int)__builtin_amdgcn_perm(w.w, w.z, 0x06040200u),
                (int)__builtin_amdgcn_perm(w.w, w.z, 0x07050301u)};
}

constexpr int kS8Tokens = 64;  // tokens of a workgroup (at most four 16-token subtiles)
constexpr int kS8U = 2;        // steps of a wave with loads in flight together

// MS: 16-token subtiles of a workgroup (1..4; fewer when S is small); NW:
// waves of a workgroup, the contraction split; R: 16-row weight tiles of a
// workgroup (each token load feeds all R).
template <int MODE, int MS, int NW, int R>
__global__ __launch_bounds__(64 * NW) void shared8_mfma_kernel(Shared8MfmaArgs a) {
  constexpr int kS8Waves = NW, kS8R = R;
  __shared__ v4i8x4 part[kS8Waves][MS * kS8R][64];  // [wave][tile][lane]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  constexpr int RB = (MODE == 0 ? 8 : 16) * kS8R;  // output rows of a workgroup
  const int nrb = (a.O + RB - 1) / RB;
  const int rb = blockIdx.x % nrb, s0 = (blockIdx.x / nrb) * (16 * MS);
  // the lane's weight row (B column n) of row tile r
  const int8_t *wrow[kS8R];
  int orow[kS8R];
#pragma unroll
  for (int r = 0; r < kS8R; r++) {
    orow[r] = MODE == 0 ? rb * RB + 8 * r + (n & 7) : rb * RB + 16 * r + n;
    wrow[r] = (MODE == 0 && n >= 8 ? a.W1 : a.W0) + (int64_t)min(orow[r], a.O - 1) * a.C;
  }
  const int8_t *xrow[MS];  // A row n of subtile ms: token s0 + 16 ms + n (past S: the last token)
#pragma unroll
  for (int ms = 0; ms < MS; ms++)
    xrow[ms] = a.act + (int64_t)min(s0 + 16 * ms + n, a.S - 1) * a.act_stride;
  v4i8x4 acc[MS][kS8R];
#pragma unroll
  for (int ms = 0; ms < MS; ms++)
#pragma unroll
    for (int r = 0; r < kS8R; r++) acc[ms][r] = v4i8x4{0, 0, 0, 0};
  const int nsteps = (a.C + 63) / 64;
  for (int st0 = wave; st0 < nsteps; st0 += kS8Waves * kS8U) {
    uint4 wv[kS8U][kS8R], xv[kS8U][MS];
#pragma unroll
    for (int u = 0; u < kS8U; u++) {
      // columns 64 st + 16 g .. +16 (C % 32 == 0: a piece is whole or past the end)
      const int col = 64 * (st0 + kS8Waves * u) + 16 * g;
      const bool ok = col < a.C;
#pragma unroll
      for (int r = 0; r < kS8R; r++) wv[u][r] = ldnt16(wrow[r] + col, ok, wrow[r]);
#pragma unroll
      for (int ms = 0; ms < MS; ms++) xv[u][ms] = ld16(xrow[ms] + col, ok, xrow[ms]);
    }
#pragma unroll
    for (int u = 0; u < kS8U; u++) {
#pragma unroll
      for (int r = 0; r < kS8R; r++) {
        const v4i8x4 b = perm_i8x16(wv[u][r]);
#pragma unroll
        for (int ms = 0; ms < MS; ms++) {
          const v4i8x4 x = v4i8x4{(int)xv[u][ms].x, (int)xv[u][ms].y, (int)xv[u][ms].z,
                                  (int)xv[u][ms].w};
          acc[ms][r] = __builtin_amdgcn_mfma_i32_16x16x64_i8(x, b, acc[ms][r], 0, 0, 0);
        }
      }
    }
  }
#pragma unroll
  for (int ms = 0; ms < MS; ms++)
#pragma unroll
    for (int r = 0; r < kS8R; r++) part[wave][ms * kS8R + r][lane] = acc[ms][r];
  __syncthreads();
  // wave w finishes tile w (token subtile w / R, row tile w % R): lane holds
  // tokens s0 + 16 (w / R) + 4 g + i of column n
  for (int tile = wave; tile < MS * kS8R; tile += kS8Waves) {
    v4i8x4 tot = part[0][tile][lane];
#pragma unroll
    for (int w = 1; w < kS8Waves; w++) tot += part[w][tile][lane];
    const int ms = tile / kS8R, r = tile % kS8R;
    const int o = MODE == 0 ? rb * RB + 8 * r + (n & 7) : rb * RB + 16 * r + n;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int t = s0 + 16 * ms + 4 * g + i;
      if (MODE == 0) {
        const int au = __shfl_xor(tot[i], 8, 64);  // the up sum of the lane's hidden unit
        if (n < 8 && t < a.S && o < a.O) {
          const float sxs = a.ascale[(int64_t)t * a.ascale_stride];
          const float gv = ((float)tot[i] * a.ws0[o]) * sxs;
          const float uv = ((float)au * a.ws1[o]) * sxs;
          a.out[(int64_t)t * a.out_stride + o] = silu(gv) * uv;
        }
      } else if (t < a.S && o < a.O) {
        const float v = ((float)tot[i] * a.ws0[o]) * a.ascale[(int64_t)t * a.ascale_stride];
        a.out[(int64_t)t * a.out_stride + o] = v;
      }
    }
  }
}

// Larger batches: a workgroup (four waves) takes 128 tokens x 128 weight rows
// (MODE 0: 64 hidden units, each wave two 16-row tiles of the gate rows of 8
// units beside their up rows; MODE 1: 128 down rows) over the whole
// contraction, in steps of 128 columns.  A step's token rows (16 KB) and the
// waves' weight rows (4 KB each) travel from global memory into shared memory
// by DMA (global_load_lds_dwordx4, two stages: the next step is requested
// while this one computes), so each token row is fetched once per 128 weight
// rows and each weight row once per 128 tokens.  The 128-byte rows of a stage
// have their 16-byte pieces XOR-swizzled by row (piece q of row R holds
// logical piece q ^ ((R >> 1) & 7)).  MFMA chunk c of a step covers columns
// 64 c .. +64, lane group g logical piece 4 c + g.  Pieces past C read the
// row's first piece and meet zeroed weights.  Row blocks vary fastest over the
// grid, so each XCD keeps the weight rows of its blocks in L2 across the token
// chunks.  The epilogues are those of shared8_mfma_kernel.
constexpr int kS8TT = 128;             // tokens of a workgroup
constexpr int kS8TR = 32;              // weight rows of a wave (two 16-row tiles)
constexpr int kS8TK = 128;             // columns of a step
constexpr int kS8TA = kS8TT * kS8TK;   // token bytes of a stage (16 KB)
constexpr int kS8TW = kS8TR * kS8TK;   // weight bytes of a wave's stage (4 KB)

template <int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void shared8_tile_kernel(Shared8MfmaArgs a) {
  __shared__ __align__(1024) int8_t A0[kS8TA], A1[kS8TA], B0[4 * kS8TW], B1[4 * kS8TW];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  constexpr int RB = MODE == 0 ? 64 : 128;  // output rows (MODE 0: hidden units) of a workgroup
  const int nrb = (a.O + RB - 1) / RB;
  const int rb = blockIdx.x % nrb, s0 = (blockIdx.x / nrb) * kS8TT;
  // output row of the wave's local weight row R (0..31): tile R / 16, row R % 16
  auto out_row = [&](int R) {
    return MODE == 0 ? rb * 64 + wave * 16 + 8 * (R >> 4) + (R & 7) : rb * 128 + wave * 32 + R;
  };
  // DMA request k of a stage: token rows 8 (wave + 4 k) + lane / 8 and local
  // weight rows 8 k + lane / 8; the lane fetches logical piece
  // (lane % 8) ^ ((row >> 1) & 7) of its row into slot lane
  const int8_t *asrc[4], *wsrc[4];
  int apc[4], wpc[4];  // column of the fetched piece within a step
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const int ra = 8 * (wave + 4 * k) + (lane >> 3);
    asrc[k] = a.act + (int64_t)min(s0 + ra, a.S - 1) * a.act_stride;
    apc[k] = 16 * ((lane & 7) ^ ((ra >> 1) & 7));
    const int rw = 8 * k + (lane >> 3);
    wsrc[k] = (MODE == 0 && (rw & 8) ? a.W1 : a.W0) + (int64_t)min(out_row(rw), a.O - 1) * a.C;
    wpc[k] = 16 * ((lane & 7) ^ ((rw >> 1) & 7));
  }
  const int nsteps = (a.C + kS8TK - 1) / kS8TK;
  auto issue = [&](int st, int8_t *As, int8_t *Bs) __attribute__((always_inline)) {
    const int k0 = st * kS8TK;
#pragma unroll
    for (int k = 0; k < 4; k++) {
      const int ca = k0 + apc[k], cw = k0 + wpc[k];
      dma16(asrc[k] + (ca < a.C ? ca : 0), As + 1024 * (wave + 4 * k));
      dma16(wsrc[k] + (cw < a.C ? cw : 0), Bs + wave * kS8TW + 1024 * k);
    }
  };
  v4i8x4 acc[8][2];
#pragma unroll
  for (int ms = 0; ms < 8; ms++)
#pragma unroll
    for (int r = 0; r < 2; r++) acc[ms][r] = v4i8x4{0, 0, 0, 0};
  issue(0, A0, B0);
  auto step = [&](int st, int8_t *As, int8_t *Bs, int8_t *An, int8_t *Bn)
                  __attribute__((always_inline)) {
    // this step's pieces are in and every wave is done with the other stage
    dma_step_barrier<0>();
    if (st + 1 < nsteps) issue(st + 1, An, Bn);
#pragma unroll
    for (int c = 0; c < 2; c++) {
      const int q = 4 * c + g;  // logical piece of the lane
      const bool ok = st * kS8TK + 16 * q < a.C;
      v4i8x4 b[2];
#pragma unroll
      for (int r = 0; r < 2; r++) {
        const int R = 16 * r + n;
        const uint4 v = *reinterpret_cast<const uint4 *>(Bs + wave * kS8TW + R * kS8TK +
                                                         16 * (q ^ ((R >> 1) & 7)));
        b[r] = ok ? perm_i8x16(v) : v4i8x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int ms = 0; ms < 8; ms++) {
        const int R = 16 * ms + n;
        const uint4 v = *reinterpret_cast<const uint4 *>(As + R * kS8TK + 16 * (q ^ ((R >> 1) & 7)));
        const v4i8x4 x = v4i8x4{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
#pragma unroll
        for (int r = 0; r < 2; r++)
          acc[ms][r] = __builtin_amdgcn_mfma_i32_16x16x64_i8(x, b[r], acc[ms][r], 0, 0, 0);
      }
    }
  };
  int st = 0;
  for (; st + 1 < nsteps; st += 2) {
    step(st, A0, B0, A1, B1);
    step(st + 1, A1, B1, A0, B0);
  }
  if (st < nsteps) step(st, A0, B0, A1, B1);
  wait_vm_at_most<0>();  // nothing in flight when the workgroup ends
  // lane: tokens s0 + 16 ms + 4 g + i of column n of tile (ms, r)
#pragma unroll
  for (int ms = 0; ms < 8; ms++)
#pragma unroll
    for (int r = 0; r < 2; r++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int t = s0 + 16 * ms + 4 * g + i;
        const int o = out_row(16 * r + n);
        if (MODE == 0) {
          const int au = __shfl_xor(acc[ms][r][i], 8, 64);  // the up sum of the lane's unit
          if (n < 8 && t < a.S && o < a.O) {
            const float sxs = a.ascale[(int64_t)t * a.ascale_stride];
            const float gv = ((float)acc[ms][r][i] * a.ws0[o]) * sxs;
            const float uv = ((float)au * a.ws1[o]) * sxs;
            a.out[(int64_t)t * a.out_stride + o] = silu(gv) * uv;
          }
        } else if (t < a.S && o < a.O) {
          const float v = ((float)acc[ms][r][i] * a.ws0[o]) * a.ascale[(int64_t)t * a.ascale_stride];
          a.out[(int64_t)t * a.out_stride + o] = v;
        }
      }
}

template <int MODE, int MS, int NW, int R>
static void launch_s8(const Shared8MfmaArgs &a, hipStream_t st) {
  constexpr int RB = (MODE == 0 ? 8 : 16) * R;
  const int nrb = (a.O + RB - 1) / RB;
  const dim3 grid(nrb * ((a.S + 16 * MS - 1) / (16 * MS))), block(64 * NW);
  hipLaunchKernelGGL((shared8_mfma_kernel<MODE, MS, NW, R>), grid, block, 0, st, a);
}

// Swept at the GLM shape (int8 gate/up, down): up to 64 tokens 16 waves and
// 2 row tiles (64 tokens: 27.8, 11.6 us; 8 waves and 1 or 4 row tiles:
// 23.8, 15.9 and 38.3, 16.6 us); 65 to 511 tokens 8 waves and 4 row tiles
// (at 2048 tokens: 254, 154 us; 2 row tiles 334-352, 178-198 us; 1 row tile
// 543, 272 us), every token load feeding more weight rows.
// Batches from this size take shared8_tile_kernel (GLM shape, int8 gate/up +
// down: 256 tokens 104 against 59 us with shared8_mfma_kernel<., 4, 8, 4>,
// 384 112 against 111, 512 105 against 105, 768 108 against 157, 1024 112
// against 206, 2048 163 against 410).
constexpr int kS8TileMinTokens = 512;

template <int MODE>
static void launch_s8_mode(const Shared8MfmaArgs &a, hipStream_t st) {
  if (a.S >= kS8TileMinTokens) {
    const int nrb = (a.O + (MODE == 0 ? 63 : 127)) / (MODE == 0 ? 64 : 128);
    const dim3 grid(nrb * ((a.S + kS8TT - 1) / kS8TT));
    hipLaunchKernelGGL(shared8_tile_kernel<MODE>, grid, dim3(256), 0, st, a);
    return;
  }
  if (a.S > 64) {
    launch_s8<MODE, 4, 8, 4>(a, st);
    return;
  }
  switch ((a.S + 15) / 16) {
    case 1: launch_s8<MODE, 1, 16, 2>(a, st); break;
    case 2: launch_s8<MODE, 2, 16, 2>(a, st); break;
    case 3: launch_s8<MODE, 3, 16, 2>(a, st); break;
    default: launch_s8<MODE, 4, 16, 2>(a, st); break;
  }
}

hipError_t launch_shared8_mfma(const Shared8MfmaArgs &a, int mode, hipStream_t st) {
  if (mode == 0)
    launch_s8_mode<0>(a, st);
  else
    launch_s8_mode<1>(a, st);
  return hipGetLastError();
}

hipError_t launch_quant_rows_i8(const Q8QuantArgs &a, hipStream_t st) {
  hipLaunchKernelGGL(quant_rows_i8_kernel, dim3((a.O + 3) / 4), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int NCH>
static void launch_gu8(const Swiglu8Args &a, hipStream_t st) {
  const dim3 grid((a.I + 3) / 4);
  if (a.x_perm) {
    if (a.D % 1024)
      hipLaunchKernelGGL((gu8_kernel<NCH, true, true>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((gu8_kernel<NCH, false, true>), grid, dim3(256), 0, st, a);
  } else if (a.D % 1024) {
    hipLaunchKernelGGL((gu8_kernel<NCH, true>), grid, dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL((gu8_kernel<NCH, false>), grid, dim3(256), 0, st, a);
  }
}

// D and I are at most 8192 (checked by the caller): at most 8 chunks.
hipError_t launch_swiglu8_gateup(const Swiglu8Args &a, hipStream_t st) {
  switch ((a.D + 1023) / 1024) {
    case 1: launch_gu8<1>(a, st); break;
    case 2: launch_gu8<2>(a, st); break;
    case 3: launch_gu8<3>(a, st); break;
    case 4: launch_gu8<4>(a, st); break;
    case 5: launch_gu8<5>(a, st); break;
    case 6: launch_gu8<6>(a, st); break;
    case 7: launch_gu8<7>(a, st); break;
    case 8: launch_gu8<8>(a, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int NCH, int R>
static void launch_dn8(const Swiglu8Args &a, hipStream_t st) {
  const dim3 grid((a.D + 4 * R - 1) / (4 * R));
  if (a.I % 1024)
    hipLaunchKernelGGL((dn8_kernel<NCH, true, R>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((dn8_kernel<NCH, false, R>), grid, dim3(256), 0, st, a);
}

// Rows per wave swept at the GLM shape (I = 2048, one token): 1, 2, 4, 8 rows
// gave 12.7, 11.5, 11.7, 11.9 us per expert call.
hipError_t launch_swiglu8_down(const Swiglu8Args &a, hipStream_t st) {
  switch ((a.I + 1023) / 1024) {
    case 1: launch_dn8<1, 4>(a, st); break;
    case 2: launch_dn8<2, 2>(a, st); break;
    case 3: launch_dn8<3, 2>(a, st); break;
    case 4: launch_dn8<4, 2>(a, st); break;
    case 5: launch_dn8<5, 2>(a, st); break;
    case 6: launch_dn8<6, 2>(a, st); break;
    case 7: launch_dn8<7, 1>(a, st); break;
    case 8: launch_dn8<8, 1>(a, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
