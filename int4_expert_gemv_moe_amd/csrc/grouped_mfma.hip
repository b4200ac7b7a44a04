// grouped_mfma.hip -- the unique-expert union's expert matmuls as grouped
// int8 MFMA GEMMs (sections 11 and 12 of the reader.mx article "惊呆了！25GB
// 内存上运行 GLM 5.2 744B 模型": each selected expert's weights are read once
// for all of its tokens; integer products, then the weight and activation
// scales).  Used when the contraction length is a multiple of 256; the
// results are the same integers, and the same floats, as the GEMV kernels of
// grouped.hip.
//
// Work unit: a tile of up to 64 (token, slot) pairs of one expert group (the
// tile list is built by group_kernel) times 64 (gate/up) or 128 (down) output
// rows.  A workgroup has 4 waves; wave w owns 16 gate rows and the 16 up rows
// with the same indices (gate/up), or 32 down rows, for all 64 pairs.
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

constexpr int kMT = 64;         // pairs per tile
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
// B = down rows, epilogue y into stage[pair]).
template <int MODE>
__global__ __launch_bounds__(256) void grouped_mfma_kernel(GroupedMfmaArgs a) {
  constexpr int NS = 2;                    // B subtiles of 16 rows per wave
  constexpr int ROWS_PER_BLOCK = MODE == 0 ? 64 : 128;
  __shared__ __align__(16) int8_t As[2][kMT * kAStride];
  __shared__ int pr_l[kMT];
  const int tile = blockIdx.y;
  if (tile >= *a.ntiles) return;
  const int2 tg = a.tiles[tile];
  const int g = tg.x, m0 = tg.y;
  const int n = a.gcount[g];
  const int rows = min(kMT, n - m0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool shared = (g == a.E);
  const int e = shared ? 0 : g;
  const int C = a.C;                       // contraction length
  const int O = a.O;                       // output rows of the matrix
  const int rowbytes = C >> 1;
  const int o_blk = blockIdx.x * ROWS_PER_BLOCK;

  // B rows of this lane: subtile ns covers 16 rows
  RowPtr Bm[NS];
  int ob[NS];
  if (MODE == 0) {
    Bm[0] = pick(a.rt.gate, a.sh.gate, shared, e);
    Bm[1] = pick(a.rt.up, a.sh.up, shared, e);
    ob[0] = ob[1] = o_blk + 16 * wave + (lane & 15);
  } else {
    Bm[0] = pick(a.rt.down, a.sh.down, shared, e);
    Bm[1] = Bm[0];
    ob[0] = o_blk + 32 * wave + (lane & 15);
    ob[1] = ob[0] + 16;
  }
  const int j = lane >> 4;  // lane group: columns 64j .. 64j + 64 of a step
  const uint8_t *bp[NS];
#pragma unroll
  for (int s = 0; s < NS; s++) {
    const int oc = min(ob[s], O - 1);
    bp[s] = Bm[s].q + (int64_t)oc * rowbytes + 32 * j;
  }

  // pair list of the tile
  const int *plist = a.pairs + a.goff[g] + m0;
  if (threadIdx.x < kMT) pr_l[threadIdx.x] = plist[min((int)threadIdx.x, rows - 1)];
  __syncthreads();

  // A loads: thread t copies 64 bytes (4 x 16) of pair row t / 4, piece t % 4
  const int ar = threadIdx.x >> 2, aq = threadIdx.x & 3;
  const int apr = pr_l[min(ar, rows - 1)];
  const int8_t *arow = (MODE == 0 ? a.act + (int64_t)(apr / a.P) * C : a.act + (int64_t)apr * C) +
                       64 * aq;
  const bool alive = ar < rows;
  uint4 av[4];
  auto load_a = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; i++) av[i] = *reinterpret_cast<const uint4 *>(arow + k0 + 16 * i);
  };
  auto store_a = [&](int buf) {
    int8_t *dst = &As[buf][ar * kAStride + 64 * aq];
#pragma unroll
    for (int i = 0; i < 4; i++)
      *reinterpret_cast<uint4 *>(dst + 16 * i) = alive ? av[i] : make_uint4(0u, 0u, 0u, 0u);
  };
  uint4 bcur[NS][2], bnext[NS][2];
  auto load_b = [&](int k0, uint4 (&bv)[NS][2]) {
#pragma unroll
    for (int s = 0; s < NS; s++) {
      bv[s][0] = ldnt16(bp[s] + k0 / 2, true, bp[s]);
      bv[s][1] = ldnt16(bp[s] + k0 / 2 + 16, true, bp[s]);
    }
  };

  v4i acc[4][NS];
#pragma unroll
  for (int ms = 0; ms < 4; ms++)
#pragma unroll
    for (int s = 0; s < NS; s++) acc[ms][s] = v4i{0, 0, 0, 0};
  const int msa = (rows + 15) >> 4;  // active 16-pair subtiles (uniform)
  const int nsteps = C / kKS;

  load_a(0);
  load_b(0, bcur);
  store_a(0);
  __syncthreads();
  for (int step = 0; step < nsteps; step++) {
    const int buf = step & 1;
    const bool more = step + 1 < nsteps;
    const int kn = more ? (step + 1) * kKS : step * kKS;
    load_a(kn);
    load_b(kn, bnext);
    const int8_t *abase = &As[buf][(lane & 15) * kAStride + 64 * j];
#pragma unroll
    for (int c = 0; c < 4; c++) {
      v4i bb[NS];
#pragma unroll
      for (int s = 0; s < NS; s++) {
        const uint4 w = bcur[s][c >> 1];
        bb[s] = (c & 1) ? unpack16(w.z, w.w) : unpack16(w.x, w.y);
      }
#pragma unroll
      for (int ms = 0; ms < 4; ms++) {
        if (ms < msa) {
          const uint4 av4 = *reinterpret_cast<const uint4 *>(abase + ms * 16 * kAStride + 16 * c);
          const v4i aa = v4i{(int)av4.x, (int)av4.y, (int)av4.z, (int)av4.w};
#pragma unroll
          for (int s = 0; s < NS; s++)
            acc[ms][s] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aa, bb[s], acc[ms][s], 0, 0, 0);
        }
      }
    }
    if (more) store_a(buf ^ 1);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < NS; s++) {
      bcur[s][0] = bnext[s][0];
      bcur[s][1] = bnext[s][1];
    }
  }

  // epilogue: lane holds output row ob[s] for pairs 16 ms + 4 j + i
  float sc[NS];
#pragma unroll
  for (int s = 0; s < NS; s++) sc[s] = Bm[s].s[min(ob[s], O - 1)];
#pragma unroll
  for (int ms = 0; ms < 4; ms++) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int r = 16 * ms + 4 * j + i;
      if (ms < msa && r < rows) {
        const int pr = pr_l[r];
        if (MODE == 0) {
          const int s = pr / a.P;
          const int o = ob[0];
          if (o < O) {
            const int corr = 8 * a.asum[s];
            const float sx = a.ascale[s];
            const float gv = ((float)(acc[ms][0][i] - corr) * sc[0]) * sx;
            const float uv = ((float)(acc[ms][1][i] - corr) * sc[1]) * sx;
            a.out[(int64_t)pr * O + o] = silu(gv) * uv;
          }
        } else {
          const int corr = 8 * a.asum[pr];
          const float shs = a.ascale[pr];
#pragma unroll
          for (int s = 0; s < NS; s++) {
            const int o = ob[s];
            if (o < O) a.out[(int64_t)pr * O + o] = ((float)(acc[ms][s][i] - corr) * sc[s]) * shs;
          }
        }
      }
    }
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
