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
#include <type_traits>

#include "moe_kernels.h"
#include "rowops.h"

namespace moe {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int u4v __attribute__((ext_vector_type(4)));  // 16 staged bytes

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
// B = down rows, epilogue y into stage[pair]).  NW waves per workgroup; MSV:
// 16-pair subtiles the tile needs (1 to 8); only those rows are loaded and
// multiplied.
struct MfmaTile {
  int rows;          // pairs of the tile
  int j, lane, wave;
  RowPtr Bm[2];
  int ob[2];         // output rows of the lane's two B subtiles
  const uint8_t *bp[4];  // the lane's 16-byte piece of each coalesced weight load
  int8_t *bs;        // the wave's weight transpose buffer in shared memory
};

constexpr int kBStride = 144;  // shared bytes per weight row of a step (128 + 16)

// As: two activation buffers of ABUF bytes each.
template <int MODE, int NW, int MSV, int ABUF>
__device__ __forceinline__ void mfma_tile(const GroupedMfmaArgs &a, const MfmaTile &t, int8_t *As,
                                          const int *pr_l, const int *sum_l, const float *scl_l) {
  constexpr int NS = 2;
  constexpr int RPL = NW * 4;                  // pair rows staged per load round
  constexpr int NA = (MSV * 16 + RPL - 1) / RPL;  // 16-byte activation loads per thread per step
  const int C = a.C, O = a.O;
  const int lane = t.lane, j = t.j, rows = t.rows;
  // activation staging: load i of a thread copies 16 bytes (column piece
  // tid % 16) of pair row RPL * i + tid / 16.  Rows from `rows` up to
  // 16 * MSV repeat the tile's last pair: their products land only in
  // output rows that the epilogue skips.
  const int ar = threadIdx.x >> 4, aq = threadIdx.x & 15;
  const int8_t *arow[NA];
#pragma unroll
  for (int i = 0; i < NA; i++) {
    const int apr = pr_l[min(RPL * i + ar, rows - 1)];
    arow[i] = (MODE == 0 ? a.act + (int64_t)(apr / a.P) * C : a.act + (int64_t)apr * C) + 16 * aq;
  }
  auto load_a = [&](int k0, u4v (&v)[NA]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NA; i++) v[i] = *reinterpret_cast<const u4v *>(arow[i] + k0);
  };
  auto store_a = [&](int buf, const u4v (&v)[NA]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NA; i++)
      if (RPL * (i + 1) <= MSV * 16 || RPL * i + ar < MSV * 16)
        *reinterpret_cast<u4v *>(As + buf * ABUF + (RPL * i + ar) * kAStride + 16 * aq) = v[i];
  };
  // Weights: the wave's 32 rows of a step (128 bytes each) arrive in four
  // coalesced loads, load i holding rows 8 i .. 8 i + 7 with 8 lanes per
  // row, and pass through the wave's own shared-memory buffer to reach the
  // MFMA operand layout (lane: one row, 32 bytes).
  auto load_b = [&](int k0, uint4 (&bv)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; i++) bv[i] = ldnt16(t.bp[i] + k0 / 2, true, t.bp[i]);
  };
  auto transpose_b = [&](const uint4 (&bv)[4], uint4 (&bm)[NS][2]) __attribute__((always_inline)) {
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < 4; i++)
      *reinterpret_cast<uint4 *>(t.bs + (8 * i + (lane >> 3)) * kBStride + 16 * (lane & 7)) = bv[i];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int s = 0; s < NS; s++)
#pragma unroll
      for (int h = 0; h < 2; h++)
        bm[s][h] = *reinterpret_cast<const uint4 *>(t.bs + (16 * s + (lane & 15)) * kBStride + 32 * j +
                                                    16 * h);
    __builtin_amdgcn_wave_barrier();
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

  // Two register sets each for weights (bw0, bw1) and activations (ra0,
  // ra1), named statically by unrolling the step loop twice, so that no
  // load is waited for before the step that uses it.  At the start of step
  // s: bw[s % 2] holds the weights of step s, ra[(s + 1) % 2] the
  // activations of step s + 1 and ra[s % 2] those of step s + 2; shared
  // buffer s % 2 holds the activations of step s.  Step s unpacks its
  // weights and refills their set with step s + 2, moves the activations of
  // step s + 1 to shared memory and refills their set with step s + 3, and
  // only then multiplies.
  uint4 bw0[4], bw1[4];
  u4v ra0[NA], ra1[NA];
  // Loads past the last step repeat the last step's addresses: every load
  // is issued unconditionally, so the compiler's count of loads in flight
  // is exact and its waits name only the data a step needs.
  const int last = (nsteps - 1) * kKS;
  load_b(0, bw0);
  load_a(0, ra0);
  load_b(min(kKS, last), bw1);
  load_a(min(kKS, last), ra1);
  store_a(0, ra0);
  load_a(min(2 * kKS, last), ra0);
  __syncthreads();
  // one step; H = st % 2 is a template constant, so every register set is
  // named statically
  auto step = [&](int st, auto hc) __attribute__((always_inline)) {
    constexpr int H = decltype(hc)::value;
    // the step's weights, unpacked at once so that their registers take
    // the loads of step s + 2 before the multiplications start
    uint4 bm[NS][2];
    if constexpr (H == 0)
      transpose_b(bw0, bm);
    else
      transpose_b(bw1, bm);
    v4i bb[4][NS];
#pragma unroll
    for (int c = 0; c < 4; c++)
#pragma unroll
      for (int s = 0; s < NS; s++) {
        const uint4 w = bm[s][c >> 1];
        bb[c][s] = (c & 1) ? unpack16(w.z, w.w) : unpack16(w.x, w.y);
      }
    const int kb = min((st + 2) * kKS, last), ka = min((st + 3) * kKS, last);
    // shared buffer (s + 1) % 2 was last read in step s - 1, which ended
    // with a barrier
    if constexpr (H == 0) {
      load_b(kb, bw0);
      if (st + 1 < nsteps) store_a(1, ra1);
      load_a(ka, ra1);
    } else {
      load_b(kb, bw1);
      if (st + 1 < nsteps) store_a(0, ra0);
      load_a(ka, ra0);
    }
    // keep the compiler from sinking those loads below the multiplications
    __builtin_amdgcn_sched_barrier(0);
    const int8_t *abase = As + H * ABUF + (lane & 15) * kAStride + 64 * j;
#pragma unroll
    for (int c = 0; c < 4; c++) {
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
          acc[ms][s] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aa[ms], bb[c][s], acc[ms][s], 0, 0, 0);
    }
    __syncthreads();
  };
  int st = 0;
  for (; st + 1 < nsteps; st += 2) {
    step(st, std::integral_constant<int, 0>{});
    step(st + 1, std::integral_constant<int, 1>{});
  }
  if (st < nsteps) step(st, std::integral_constant<int, 0>{});

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

constexpr int cmin(int x, int y) { return x < y ? x : y; }

// Rows of B per workgroup: NW waves of 16 gate + 16 up rows (MODE 0) or
// 32 down rows (MODE 1).
template <int MODE, int NW>
constexpr int mfma_block_rows() { return MODE == 0 ? 16 * NW : 32 * NW; }

// MSVMAX: the largest subtile count the launch can meet (tiles never hold
// more pairs than the batch has tokens); it bounds the registers the
// compiler reserves.
template <int MODE, int NW, int MSVMAX>
__global__ __launch_bounds__(NW * 64) void grouped_mfma_kernel(GroupedMfmaArgs a) {
  constexpr int ABUF = 16 * MSVMAX * kAStride;
  __shared__ __align__(16) int8_t As[2 * ABUF];
  __shared__ __align__(16) int8_t Bs[NW][32 * kBStride];
  __shared__ int pr_l[kMT];
  __shared__ int sum_l[kMT];    // code sum of each pair's activation row
  __shared__ float scl_l[kMT];  // scale of each pair's activation row
  const int tile = blockIdx.y;
  if (tile >= *a.ntiles) return;
  const int2 tg = a.tiles[tile];
  const int g = tg.x, m0 = tg.y;
  MfmaTile t;
  t.rows = min(16 * MSVMAX, a.gcount[g] - m0);
  t.lane = threadIdx.x & 63;
  t.wave = threadIdx.x >> 6;
  t.j = t.lane >> 4;  // lane group: columns 64j .. 64j + 64 of a step
  const bool shared = (g == a.E);
  const int e = shared ? 0 : g;
  const int o_blk = blockIdx.x * mfma_block_rows<MODE, NW>();
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
  // coalesced load i: wave row r = 8 i + lane / 8 (rows 0..15 are subtile
  // 0, 16..31 subtile 1), bytes 16 (lane % 8) of the step's 128
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int r = 8 * i + (t.lane >> 3);
    const int s = r >> 4;
    const int o = (MODE == 0 ? o_blk + 16 * t.wave : o_blk + 32 * t.wave + 16 * s) + (r & 15);
    t.bp[i] = t.Bm[s].q + (int64_t)min(o, a.O - 1) * rowbytes + 16 * (t.lane & 7);
  }
  t.bs = &Bs[t.wave][0];

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
    case 1: mfma_tile<MODE, NW, 1, ABUF>(a, t, As, pr_l, sum_l, scl_l); break;
    case 2: mfma_tile<MODE, NW, cmin(2, MSVMAX), ABUF>(a, t, As, pr_l, sum_l, scl_l); break;
    case 3: mfma_tile<MODE, NW, cmin(3, MSVMAX), ABUF>(a, t, As, pr_l, sum_l, scl_l); break;
    case 4: mfma_tile<MODE, NW, cmin(4, MSVMAX), ABUF>(a, t, As, pr_l, sum_l, scl_l); break;
    case 5: mfma_tile<MODE, NW, cmin(5, MSVMAX), ABUF>(a, t, As, pr_l, sum_l, scl_l); break;
    case 6: mfma_tile<MODE, NW, cmin(6, MSVMAX), ABUF>(a, t, As, pr_l, sum_l, scl_l); break;
    case 7: mfma_tile<MODE, NW, cmin(7, MSVMAX), ABUF>(a, t, As, pr_l, sum_l, scl_l); break;
    default: mfma_tile<MODE, NW, MSVMAX, ABUF>(a, t, As, pr_l, sum_l, scl_l); break;
  }
}

bool grouped_mfma_fits(int C) { return C % kKS == 0; }

int grouped_mfma_max_tiles(int S, int P, int E) { return (S * P + kMT - 1) / kMT + E + 1; }

// Batches of up to 64 tokens (at most 4 subtiles per tile): 4-wave
// workgroups, so that a few experts still spread over many workgroups;
// larger batches: 8-wave workgroups, which stage each activation tile for
// twice as many weight rows.
hipError_t launch_grouped_mfma(const GroupedMfmaArgs &a, int mode, int max_tiles, int S,
                               hipStream_t st) {
  if (S <= 64) {
    const dim3 grid((a.O + mfma_block_rows<0, 4>() - 1) / mfma_block_rows<0, 4>(), max_tiles);
    if (mode == 0)
      hipLaunchKernelGGL((grouped_mfma_kernel<0, 4, 4>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((grouped_mfma_kernel<1, 4, 4>),
                         dim3((a.O + mfma_block_rows<1, 4>() - 1) / mfma_block_rows<1, 4>(), max_tiles),
                         dim3(256), 0, st, a);
  } else {
    if (mode == 0)
      hipLaunchKernelGGL((grouped_mfma_kernel<0, 8, 8>),
                         dim3((a.O + mfma_block_rows<0, 8>() - 1) / mfma_block_rows<0, 8>(), max_tiles),
                         dim3(512), 0, st, a);
    else
      hipLaunchKernelGGL((grouped_mfma_kernel<1, 8, 8>),
                         dim3((a.O + mfma_block_rows<1, 8>() - 1) / mfma_block_rows<1, 8>(), max_tiles),
                         dim3(512), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace moe
