// grouped_mfma.hip -- the unique-expert union's expert matmuls as grouped
// int8 MFMA GEMMs (sections 11 and 12 of the reader.mx article "惊呆了！25GB
// 内存上运行 GLM 5.2 744B 模型": each selected expert's weights are read once
// for all of its tokens; integer products, then the weight and activation
// scales).  Used when the contraction length is a multiple of 256; the
// results are the same integers, and the same floats, as the GEMV kernels of
// grouped.hip.
//
// Work unit: a tile of up to 128 (token, slot) pairs of one expert group (the
// tile list is built by group_kernel; a routed expert of a 2048-token prefill
// gets about 64 pairs, so its weights are read once) times 64 (gate/up) or
// 128 (down) output rows.  A workgroup has 4 waves; wave w owns 16 gate rows
// and the 16 up rows with the same indices (gate/up), or 32 down rows, for
// all pairs of the tile.
//
// v_mfma_i32_16x16x64_i8 (layout checked on the device): lane l supplies row
// l % 16 of A (a pair) and column l % 16 of B (an output row), each 16 int8
// values of the k-range 16 * (l / 16) .. +16, and receives C for column
// l % 16, rows 4 * (l / 16) .. +4.  Here lane group j = l / 16 of an MFMA
// covers columns 64j + 16c .. +16 of the 256-column step (c = the step's 4
// MFMAs), so a lane's weight bytes of one step are 32 contiguous bytes of its
// row and its activation bytes 64 contiguous bytes of its pair's row.
//
// The int4 nibbles n = q + 8 are used as unsigned int8 values (0..15) against
// the permuted activation codes [x0 x2 x4 x6 x1 x3 x5 x7] of each group of 8
// (the low nibbles of a word are the even columns): acc - 8 * sum(x) is the
// exact signed product.
#include "moe_kernels.h"
#include "rowops.h"

namespace moe {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kMT = kGroupedMfmaTile;  // pairs per tile (128)
constexpr int kKS = 256;        // columns per pipeline step
constexpr int kAStride = 272;   // LDS bytes per pair row (256 + 16: no bank conflicts)

// 16 int4 columns (two packed words) as 16 unsigned int8 nibbles in the
// order of the permuted activation layout.
__device__ __forceinline__ v4i unpack16(uint32_t w0, uint32_t w1) {
  v4i b;
  b[0] = (int)(w0 & 0x0F0F0F0Fu);
  b[1] = (int)((w0 >> 4) & 0x0F0F0F0Fu);
  b[2] = (int)(w1 & 0x0F0F0F0Fu);
  b[3] = (int)((w1 >> 4) & 0x0F0F0F0Fu);
  return b;
}

// MODE 0: gate/up (A = token codes xq[s], B = gate and up rows, epilogue
// h = silu(g) * u into h[pair]); MODE 1: down (A = hidden codes hq[pair],
// B = down rows, epilogue y into stage[pair]).  MSV: 16-pair subtiles the
// tile needs (1 to 8); only those rows are loaded and multiplied.
struct MfmaTile {
  int rows;          // pairs of the tile
  int j, lane, wave;
  RowPtr Bm[2];
  int ob[2];         // output rows of the lane's two B subtiles
  const uint8_t *bp[2];
};

template <int MODE, int MSV>
__device__ __forceinline__ void mfma_tile(const GroupedMfmaArgs &a, const MfmaTile &t,
                                          int8_t (*As)[kMT * kAStride], const int *pr_l,
                                          const int *sum_l, const float *scl_l) {
  constexpr int NS = 2;
  const int C = a.C, O = a.O;
  const int lane = t.lane, j = t.j, rows = t.rows;
  // A loads: per step, load i of a thread copies 16 bytes (column piece
  // tid % 16) of pair row 16 i + tid / 16; rows past the tile are zero
  const int ar = threadIdx.x >> 4, aq = threadIdx.x & 15;
  const int8_t *arow[MSV];
#pragma unroll
  for (int i = 0; i < MSV; i++) {
    const int apr = pr_l[min(16 * i + ar, rows - 1)];
    arow[i] = (MODE == 0 ? a.act + (int64_t)(apr / a.P) * C : a.act + (int64_t)apr * C) + 16 * aq;
  }
  uint4 av[MSV], avn[MSV];
  auto load_a = [&](int k0, uint4 (&v)[MSV]) {
#pragma unroll
    for (int i = 0; i < MSV; i++) v[i] = *reinterpret_cast<const uint4 *>(arow[i] + k0);
  };
  auto store_a = [&](int buf, const uint4 (&v)[MSV]) {
#pragma unroll
    for (int i = 0; i < MSV; i++)
      *reinterpret_cast<uint4 *>(&As[buf][(16 * i + ar) * kAStride + 16 * aq]) =
          (16 * i + ar < rows) ? v[i] : make_uint4(0u, 0u, 0u, 0u);
  };
  uint4 bcur[NS][2], bnext[NS][2], bnext2[NS][2];
  auto load_b = [&](int k0, uint4 (&bv)[NS][2]) {
#pragma unroll
    for (int s = 0; s < NS; s++) {
      bv[s][0] = ldnt16(t.bp[s] + k0 / 2, true, t.bp[s]);
      bv[s][1] = ldnt16(t.bp[s] + k0 / 2 + 16, true, t.bp[s]);
    }
  };
  v4i acc[MSV][NS];
#pragma unroll
  for (int ms = 0; ms < MSV; ms++)
#pragma unroll
    for (int s = 0; s < NS; s++) acc[ms][s] = v4i{0, 0, 0, 0};
  float sc[NS];  // row scales of the lane's output rows
#pragma unroll
  for (int s = 0; s < NS; s++) sc[s] = t.Bm[s].s[min(t.ob[s], O - 1)];
  const int nsteps = C / kKS;

  // weights and activations both run two steps ahead: the activation rows
  // of step s + 1 wait in registers during step s and go to shared memory at
  // its end
  load_a(0, avn);
  load_b(0, bcur);
  load_a(min(1, nsteps - 1) * kKS, av);
  load_b(min(1, nsteps - 1) * kKS, bnext);
  store_a(0, avn);
  __syncthreads();
  for (int step = 0; step < nsteps; step++) {
    const int buf = step & 1;
    const bool more = step + 1 < nsteps;
    load_a(min(step + 2, nsteps - 1) * kKS, avn);
    load_b(min(step + 2, nsteps - 1) * kKS, bnext2);
    // per 64-column slice c: the operands first (one wait for shared
    // memory), then the MFMAs
    const int8_t *abase = &As[buf][(lane & 15) * kAStride + 64 * j];
#pragma unroll
    for (int c = 0; c < 4; c++) {
      v4i bb[NS];
#pragma unroll
      for (int s = 0; s < NS; s++) {
        const uint4 w = bcur[s][c >> 1];
        bb[s] = (c & 1) ? unpack16(w.z, w.w) : unpack16(w.x, w.y);
      }
      v4i aa[MSV];
#pragma unroll
      for (int ms = 0; ms < MSV; ms++) {
        const uint4 v = *reinterpret_cast<const uint4 *>(abase + ms * 16 * kAStride + 16 * c);
        aa[ms] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
      }
#pragma unroll
      for (int ms = 0; ms < MSV; ms++)
#pragma unroll
        for (int s = 0; s < NS; s++)
          acc[ms][s] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aa[ms], bb[s], acc[ms][s], 0, 0, 0);
    }
    if (more) store_a(buf ^ 1, av);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < MSV; i++) av[i] = avn[i];
#pragma unroll
    for (int s = 0; s < NS; s++) {
      bcur[s][0] = bnext[s][0];
      bcur[s][1] = bnext[s][1];
      bnext[s][0] = bnext2[s][0];
      bnext[s][1] = bnext2[s][1];
    }
  }

  // epilogue: lane holds output row ob[s] for pairs 16 ms + 4 j + i
#pragma unroll
  for (int ms = 0; ms < MSV; ms++) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int r = 16 * ms + 4 * j + i;
      if (r < rows) {
        const int pr = pr_l[r];
        const int corr = 8 * sum_l[r];
        const float as = scl_l[r];
        if (MODE == 0) {
          const int o = t.ob[0];
          if (o < O) {
            const float gv = ((float)(acc[ms][0][i] - corr) * sc[0]) * as;
            const float uv = ((float)(acc[ms][1][i] - corr) * sc[1]) * as;
            a.out[(int64_t)pr * O + o] = silu(gv) * uv;
          }
        } else {
#pragma unroll
          for (int s = 0; s < NS; s++) {
            const int o = t.ob[s];
            if (o < O) a.out[(int64_t)pr * O + o] = ((float)(acc[ms][s][i] - corr) * sc[s]) * as;
          }
        }
      }
    }
  }
}

template <int MODE>
__global__ __launch_bounds__(256) void grouped_mfma_kernel(GroupedMfmaArgs a) {
  constexpr int ROWS_PER_BLOCK = MODE == 0 ? 64 : 128;
  __shared__ __align__(16) int8_t As[2][kMT * kAStride];
  __shared__ int pr_l[kMT];
  __shared__ int sum_l[kMT];    // code sum of each pair's activation row
  __shared__ float scl_l[kMT];  // scale of each pair's activation row
  const int tile = blockIdx.y;
  if (tile >= *a.ntiles) return;
  const int2 tg = a.tiles[tile];
  const int g = tg.x, m0 = tg.y;
  MfmaTile t;
  t.rows = min(kMT, a.gcount[g] - m0);
  t.lane = threadIdx.x & 63;
  t.wave = threadIdx.x >> 6;
  t.j = t.lane >> 4;  // lane group: columns 64j .. 64j + 64 of a step
  const bool shared = (g == a.E);
  const int e = shared ? 0 : g;
  const int o_blk = blockIdx.x * ROWS_PER_BLOCK;
  if (MODE == 0) {
    t.Bm[0] = pick(a.rt.gate, a.sh.gate, shared, e);
    t.Bm[1] = pick(a.rt.up, a.sh.up, shared, e);
    t.ob[0] = t.ob[1] = o_blk + 16 * t.wave + (t.lane & 15);
  } else {
    t.Bm[0] = pick(a.rt.down, a.sh.down, shared, e);
    t.Bm[1] = t.Bm[0];
    t.ob[0] = o_blk + 32 * t.wave + (t.lane & 15);
    t.ob[1] = t.ob[0] + 16;
  }
  const int rowbytes = a.C >> 1;
#pragma unroll
  for (int s = 0; s < 2; s++)
    t.bp[s] = t.Bm[s].q + (int64_t)min(t.ob[s], a.O - 1) * rowbytes + 32 * t.j;

  // pair list of the tile and the scale and code sum of each pair's row
  const int *plist = a.pairs + a.goff[g] + m0;
  if (threadIdx.x < kMT) {
    const int pr = plist[min((int)threadIdx.x, t.rows - 1)];
    const int ar = MODE == 0 ? pr / a.P : pr;  // activation row
    pr_l[threadIdx.x] = pr;
    sum_l[threadIdx.x] = a.asum[ar];
    scl_l[threadIdx.x] = a.ascale[ar];
  }
  __syncthreads();
  switch ((t.rows + 15) >> 4) {  // 16-pair subtiles in use, uniform across the block
    case 1: mfma_tile<MODE, 1>(a, t, As, pr_l, sum_l, scl_l); break;
    case 2: mfma_tile<MODE, 2>(a, t, As, pr_l, sum_l, scl_l); break;
    case 3: mfma_tile<MODE, 3>(a, t, As, pr_l, sum_l, scl_l); break;
    case 4: mfma_tile<MODE, 4>(a, t, As, pr_l, sum_l, scl_l); break;
    case 5: mfma_tile<MODE, 5>(a, t, As, pr_l, sum_l, scl_l); break;
    case 6: mfma_tile<MODE, 6>(a, t, As, pr_l, sum_l, scl_l); break;
    case 7: mfma_tile<MODE, 7>(a, t, As, pr_l, sum_l, scl_l); break;
    default: mfma_tile<MODE, 8>(a, t, As, pr_l, sum_l, scl_l); break;
  }
}

bool grouped_mfma_fits(int C) { return C % kKS == 0; }

int grouped_mfma_max_tiles(int S, int P, int E) { return (S * P + kMT - 1) / kMT + E + 1; }

hipError_t launch_grouped_mfma(const GroupedMfmaArgs &a, int mode, int max_tiles, hipStream_t st) {
  if (mode == 0) {
    const dim3 grid((a.O + 63) / 64, max_tiles);
    hipLaunchKernelGGL(grouped_mfma_kernel<0>, grid, dim3(256), 0, st, a);
  } else {
    const dim3 grid((a.O + 127) / 128, max_tiles);
    hipLaunchKernelGGL(grouped_mfma_kernel<1>, grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace moe
