// grouped_mfma.hip -- the unique-expert union's expert matmuls as grouped
// int8 MFMA GEMMs (sections 11 and 12 of the reader.mx article "惊呆了！25GB
// 内存上运行 GLM 5.2 744B 模型": each selected expert's weights are read once
// for all of its tokens; integer products, then the weight and activation
// scales).  Used when the contraction length is a multiple of 256; the
// results are the same integers, and the same floats, as the GEMV kernels of
// grouped.hip.
//
// Work unit: a tile of up to 64 (batches of at most 64 tokens) or 80 (larger
// batches) (token, slot) pairs of one expert group (the tile list is built by
// group_kernel; a routed expert of a 2048-token prefill gets about 64 pairs,
// so its weights are read once) times a chunk of output rows.  Each wave
// owns 8 NS gate rows and the 8 NS up rows with the same indices (gate/up),
// or 16 NS down rows, for all pairs of the tile.  Up to 64
// tokens grouped_mfma_kernel (operands staged through registers, NS = 2,
// 4-wave workgroups); larger batches operands copied into shared memory by
// DMA, NS = 4: gate/up grouped_mfma_dma2_kernel (8-wave workgroups, weights
// requested two steps at a time), down grouped_mfma_dma_kernel (4-wave).
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
#include "dma.h"
#include "rowops.h"

namespace moe {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int u4v __attribute__((ext_vector_type(4)));  // 16 staged bytes

constexpr int kMT = kGroupedMfmaTile;  // bound on the pairs of a tile (128)
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
  RowPtr Bm[4];      // matrix of each of the wave's 16-row B subtiles
  int ob[4];         // output row of the lane in each B subtile
  const uint8_t *bbase[4];  // matrix base of each subtile (uniform)
  int boff[8];       // byte offset of the lane's piece of each coalesced weight load
  int8_t *bs;        // the wave's weight transpose buffer in shared memory
};

constexpr int kBStride = 144;  // shared bytes per weight row of a step (128 + 16)

// As: three activation buffers of ABUF bytes each.  NS: 16-row B subtiles
// per wave (2: 16 gate + 16 up rows, or 32 down rows; 4: twice that, so each
// activation fragment read from shared memory feeds four MFMAs).
template <int MODE, int NW, int NS, int MSV, int ABUF>
__device__ __forceinline__ void mfma_tile(const GroupedMfmaArgs &a, const MfmaTile &t, int8_t *As,
                                          const int *pr_l, const int *sum_l, const float *scl_l) {
  constexpr int NI = 2 * NS;  // coalesced weight loads per step (8 rows each)
  constexpr int RPL = NW * 4;                  // pair rows staged per load round
  constexpr int NA = (MSV * 16 + RPL - 1) / RPL;  // 16-byte activation loads per thread per step
  const int C = a.C, O = a.O;
  const int lane = t.lane, j = t.j, rows = t.rows;
  // activation staging: load i of a thread copies 16 bytes (column piece
  // tid % 16) of pair row RPL * i + tid / 16.  Rows from `rows` up to
  // 16 * MSV repeat the tile's last pair: their products land only in
  // output rows that the epilogue skips.
  const int ar = threadIdx.x >> 4, aq = threadIdx.x & 15;
  int aoff[NA];  // byte offsets into a.act (rows * C < 2^31, checked on the host)
#pragma unroll
  for (int i = 0; i < NA; i++) {
    const int apr = pr_l[min(RPL * i + ar, rows - 1)];
    aoff[i] = (MODE == 0 ? apr / a.P : apr) * C + 16 * aq;
  }
  auto load_a = [&](int k0, u4v (&v)[NA]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NA; i++) v[i] = *reinterpret_cast<const u4v *>(a.act + aoff[i] + k0);
  };
  auto store_a = [&](int buf, const u4v (&v)[NA]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NA; i++)
      if (RPL * (i + 1) <= MSV * 16 || RPL * i + ar < MSV * 16)
        *reinterpret_cast<u4v *>(As + buf * ABUF + (RPL * i + ar) * kAStride + 16 * aq) = v[i];
  };
  // Weights: the wave's 16 NS rows of a step (128 bytes each) arrive in NI
  // coalesced loads, load i holding rows 8 i .. 8 i + 7 with 8 lanes per
  // row, and pass through the wave's own shared-memory buffer to reach the
  // MFMA operand layout (lane: one row, 32 bytes).
  auto load_b = [&](int k0, uint4 (&bv)[NI]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NI; i++) {
      const uint8_t *p = t.bbase[i >> 1] + t.boff[i] + k0 / 2;  // load i is subtile i / 2
      bv[i] = ldnt16(p, true, p);
    }
  };
  auto write_b = [&](const uint4 (&bv)[NI]) __attribute__((always_inline)) {
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < NI; i++)
      *reinterpret_cast<uint4 *>(t.bs + (8 * i + (lane >> 3)) * kBStride + 16 * (lane & 7)) = bv[i];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  // half h of the step's weights in the MFMA layout: lane holds 16 bytes of
  // row 16 s + lane % 16 of each subtile s
  auto read_b = [&](int h, uint4 (&bm)[NS]) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < NS; s++)
      bm[s] = *reinterpret_cast<const uint4 *>(t.bs + (16 * s + (lane & 15)) * kBStride + 32 * j + 16 * h);
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
  // B1 (NS == 4, where registers are scarce): one register set of weights;
  // the step's weights wait in the wave's shared buffer instead.  At the
  // start of step s the buffer holds step s and bw step s + 1; after its
  // multiplications the step moves bw to the buffer and loads step s + 2.
  constexpr bool B1 = NS == 4;
  uint4 bw0[NI], bw1[B1 ? 1 : NI];
  u4v ra0[NA], ra1[B1 ? 1 : NA];
  // Loads past the last step repeat the last step's addresses: every load
  // is issued unconditionally, so the compiler's count of loads in flight
  // is exact and its waits name only the data a step needs.
  const int last = (nsteps - 1) * kKS;
  load_b(0, bw0);
  load_a(0, ra0);
  if constexpr (B1) {
    write_b(bw0);
    load_b(min(kKS, last), bw0);
  } else {
    load_b(min(kKS, last), bw1);
  }
  if constexpr (B1) {
    // one activation register set: step s + 1 waits in it during step s
    store_a(0, ra0);
    load_a(min(kKS, last), ra0);
  } else {
    load_a(min(kKS, last), ra1);
    store_a(0, ra0);
    load_a(min(2 * kKS, last), ra0);
  }
  __syncthreads();
  // one step; H = st % 2 is a template constant, so every register set is
  // named statically.  The activations sit in a ring of three shared
  // buffers (step s in buffer s % 3): step s reads its first operands,
  // stores step s + 1, then passes the workgroup barrier and multiplies.
  // Buffer (s + 1) % 3 was last read in step s - 2, which every wave
  // finished before the barrier of step s - 1; step s's operands were
  // stored before the barrier of step s - 1.  One barrier per step, and
  // the first reads of a step wait out the barrier instead of following it.
  auto step = [&](int st, auto hc) __attribute__((always_inline)) {
    constexpr int H = decltype(hc)::value;
    // the step's weights in the MFMA layout; without B1 this frees their
    // load registers for step s + 2 before the multiplications start
    if constexpr (!B1) {
      if constexpr (H == 0)
        write_b(bw0);
      else
        write_b(bw1);
    }
    const int8_t *abase = As + (st % 3) * ABUF + (lane & 15) * kAStride + 64 * j;
    auto read_a = [&](int c, v4i (&aa)[MSV]) __attribute__((always_inline)) {
#pragma unroll
      for (int ms = 0; ms < MSV; ms++) {
        const uint4 v = *reinterpret_cast<const uint4 *>(abase + ms * 16 * kAStride + 16 * c);
        aa[ms] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
      }
    };
    // the first operands before the barrier, where registers allow (not B1)
    constexpr bool EARLY = !B1;
    uint4 bm[NS];
    v4i aa[MSV];
    if constexpr (EARLY) {
      read_b(0, bm);
      read_a(0, aa);
    }
    const int kb = min((st + 2) * kKS, last), ka = min((st + 3) * kKS, last);
    if constexpr (B1) {
      if (st + 1 < nsteps) store_a((st + 1) % 3, ra0);
      load_a(min((st + 2) * kKS, last), ra0);
    } else if constexpr (H == 0) {
      load_b(kb, bw0);
      if (st + 1 < nsteps) store_a((st + 1) % 3, ra1);
      load_a(ka, ra1);
    } else {
      load_b(kb, bw1);
      if (st + 1 < nsteps) store_a((st + 1) % 3, ra0);
      load_a(ka, ra0);
    }
    // keep the compiler from sinking those loads below the multiplications
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 4; c++) {
      if (c > 0 || !EARLY) {
        if ((c & 1) == 0) read_b(c >> 1, bm);
        read_a(c, aa);
      }
      v4i bb[NS];
#pragma unroll
      for (int s = 0; s < NS; s++) {
        const uint4 w = bm[s];
        bb[s] = (c & 1) ? unpack16(w.z, w.w) : unpack16(w.x, w.y);
      }
#pragma unroll
      for (int ms = 0; ms < MSV; ms++)
#pragma unroll
        for (int s = 0; s < NS; s++)
          acc[ms][s] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aa[ms], bb[s], acc[ms][s], 0, 0, 0);
    }
    if constexpr (B1) {
      // after this wave's reads of its buffer (shared-memory operations of a
      // wave complete in order): step s + 1 into it, step s + 2 into bw
      write_b(bw0);
      load_b(kb, bw0);
    }
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
          // subtile s holds gate rows, s + NS / 2 the up rows of the same outputs
#pragma unroll
          for (int s = 0; s < NS / 2; s++) {
            const int o = t.ob[s];
            if (o < O) {
              const float gv = ((float)(acc[ms][s][i] - corr) * sc[s]) * as;
              const float uv = ((float)(acc[ms][s + NS / 2][i] - corr) * sc[s + NS / 2]) * as;
              a.out[(int64_t)pr * O + o] = silu(gv) * uv;
            }
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

// Rows of B per workgroup: NW waves of 8 NS gate + 8 NS up rows (MODE 0) or
// 16 NS down rows (MODE 1).
template <int MODE, int NW, int NS>
constexpr int mfma_block_rows() { return MODE == 0 ? 8 * NS * NW : 16 * NS * NW; }

// MSVMAX: the largest subtile count of the launch's tiles; it bounds the
// registers the compiler reserves.
template <int MODE, int NW, int NS, int MSVMAX>
__global__ __launch_bounds__(NW * 64) void grouped_mfma_kernel(GroupedMfmaArgs a) {
  constexpr int ABUF = 16 * MSVMAX * kAStride;
  __shared__ __align__(16) int8_t As[3 * ABUF];
  __shared__ __align__(16) int8_t Bs[NW][16 * NS * kBStride];
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
  const int o_blk = blockIdx.x * mfma_block_rows<MODE, NW, NS>();
  // B subtile s of the wave: MODE 0: gate rows (s < NS / 2) or up rows,
  // 16 (s mod NS / 2) .. +16 of the wave's 8 NS outputs; MODE 1: down rows
  // 16 s .. +16 of the wave's 16 NS.
  const RowPtr G = MODE == 0 ? pick(a.rt.gate, a.sh.gate, shared, e) : pick(a.rt.down, a.sh.down, shared, e);
  const RowPtr U = MODE == 0 ? pick(a.rt.up, a.sh.up, shared, e) : G;
  auto sub_row = [&](int s, int r) {  // output row of row r (0..15) of subtile s
    return MODE == 0 ? o_blk + 8 * NS * t.wave + 16 * (s % (NS / 2)) + r
                     : o_blk + 16 * NS * t.wave + 16 * s + r;
  };
#pragma unroll
  for (int s = 0; s < NS; s++) {
    t.Bm[s] = (MODE == 0 && s >= NS / 2) ? U : G;
    t.ob[s] = sub_row(s, t.lane & 15);
  }
  const int rowbytes = a.C >> 1;
  // coalesced load i: wave row r = 8 i + lane / 8 (subtile r / 16), bytes
  // 16 (lane % 8) of the step's 128
#pragma unroll
  for (int s = 0; s < NS; s++) t.bbase[s] = t.Bm[s].q;
#pragma unroll
  for (int i = 0; i < 2 * NS; i++) {
    const int r = 8 * i + (t.lane >> 3);  // subtile r / 16 == i / 2
    t.boff[i] = min(sub_row(i >> 1, r & 15), a.O - 1) * rowbytes + 16 * (t.lane & 7);
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
    case 1: mfma_tile<MODE, NW, NS, 1, ABUF>(a, t, As, pr_l, sum_l, scl_l); break;
    case 2: mfma_tile<MODE, NW, NS, cmin(2, MSVMAX), ABUF>(a, t, As, pr_l, sum_l, scl_l); break;
    case 3: mfma_tile<MODE, NW, NS, cmin(3, MSVMAX), ABUF>(a, t, As, pr_l, sum_l, scl_l); break;
    case 4: mfma_tile<MODE, NW, NS, cmin(4, MSVMAX), ABUF>(a, t, As, pr_l, sum_l, scl_l); break;
    case 5: mfma_tile<MODE, NW, NS, cmin(5, MSVMAX), ABUF>(a, t, As, pr_l, sum_l, scl_l); break;
    case 6: mfma_tile<MODE, NW, NS, cmin(6, MSVMAX), ABUF>(a, t, As, pr_l, sum_l, scl_l); break;
    case 7: mfma_tile<MODE, NW, NS, cmin(7, MSVMAX), ABUF>(a, t, As, pr_l, sum_l, scl_l); break;
    default: mfma_tile<MODE, NW, NS, MSVMAX, ABUF>(a, t, As, pr_l, sum_l, scl_l); break;
  }
}

// Subtiles (16 pairs each) of the two launch shapes: batches of up to 64
// tokens hold at most 4 per tile, larger batches at most 5.
constexpr int kSmallMsv = 4, kLargeMsv = 5;
// Larger batches, down: the shared-memory DMA kernel in 4-wave workgroups,
// two per CU (measured against one 8-wave workgroup per CU and against the
// register-staged grouped_mfma_kernel<.., 8, 4, 5>: down 486 against 545 and
// 567 us at 2048 tokens), with whole tiles per XCD.
constexpr int kPrefillDmaWaves = 4;
constexpr bool kDmaXcdTiles = true;

// ---- large batches: operands staged by shared-memory DMA ----------------------
//
// The same tiles, waves and MFMA layout as grouped_mfma_kernel<MODE, 8, 4, ..>
// (8 waves of 64 weight rows, tiles of up to 80 pairs), but the operands
// travel from global memory straight into shared memory
// (global_load_lds_dwordx4: each lane's 16 bytes land at the instruction's
// shared base + 16 lane), so no registers hold loads in flight and two steps
// of 128 columns are requested ahead through three-stage rings: weights in a
// ring per wave (only that wave reads them), activations in one ring per
// workgroup.  A step waits for its own loads (the next step's stay in
// flight), passes the workgroup barrier, requests the step after next into
// the buffer every wave finished with, and multiplies.
//
// Layouts (16-byte pieces XOR-swizzled by row, so the MFMA-layout reads of
// 16 lanes hit 16 distinct bank groups):
//   weights: a wave's stage is 64 rows x 64 bytes; piece q of row R holds
//            logical piece q ^ ((R >> 2) & 3);
//   activations: 16 MSV rows x 128 bytes; piece q of row R holds logical
//            piece q ^ ((R >> 1) & 7).
// Lane group j of an MFMA covers columns 32 j + 16 c .. +16 of the step
// (c = the step's two MFMAs): one 16-byte weight piece feeds both, the
// activation pieces are logical 2 j + c.

constexpr int kDKS = 128;                    // columns per step
constexpr int kDNS = 4;                      // 16-row weight subtiles per wave
constexpr int kDBWave = 16 * kDNS * kDKS / 2;  // weight bytes of a wave's stage (4 KB)
constexpr int kDARow = kDKS;                 // activation bytes of a pair row per step

// Activation pieces per wave and step: the 2 MSVMAX instructions of a stage
// spread over the NW waves, every wave issuing the same count (an
// instruction number past the last repeats an earlier one, same data into
// the same place), so one wait count fits every wave.
template <int NW, int MSVMAX>
constexpr int dma_a_per_wave() { return (2 * MSVMAX + NW - 1) / NW; }

// The three stages are separate shared arrays (A0..A2, B0..B2), so the
// compiler can tell a step's reads from the requests in flight into the
// other stages and does not wait for those.
template <int MODE, int NW, int MSVMAX, int MSV, int ABUF>
__device__ __forceinline__ void dma_tile(const GroupedMfmaArgs &a, const MfmaTile &t,
                                         int8_t *A0, int8_t *A1, int8_t *A2, int8_t *B0,
                                         int8_t *B1, int8_t *B2, const int *pr_l,
                                         const int *sum_l, const float *scl_l) {
  constexpr int NS = kDNS;
  constexpr int NA = 2 * MSV;  // activation DMA instructions of a stage (8 rows x 128 bytes each)
  constexpr int AW = dma_a_per_wave<NW, MSVMAX>();
  constexpr int PIECES = NS + AW;  // requests per wave and step
  const int C = a.C, O = a.O;
  const int lane = t.lane, j = t.j, rows = t.rows, wave = t.wave;
  const int ln = lane & 15;
  const int rowbytes = C >> 1;
  // weights: instruction i of a step is subtile i: row lane / 4 of it,
  // shared piece lane % 4 = logical piece (lane % 4) ^ (lane / 16)
  const uint8_t *bsrc[NS];
#pragma unroll
  for (int i = 0; i < NS; i++) {
    const int o = t.ob[i] - ln + (lane >> 2);  // first row of subtile i + lane / 4
    const int p = (lane & 3) ^ (lane >> 4);
    bsrc[i] = t.bbase[i] + (int64_t)min(o, O - 1) * rowbytes + 16 * p;
  }
  // activations: instruction n = wave + NW u: pair row 8 n + lane / 8, shared
  // piece lane % 8 = logical piece (lane % 8) ^ ((row >> 1) & 7)
  int asrc[AW], adst[AW];
#pragma unroll
  for (int u = 0; u < AW; u++) {
    const int n = (wave + NW * u) % NA;
    const int r = 8 * n + (lane >> 3);
    const int apr = pr_l[min(r, rows - 1)];
    const int p = (lane & 7) ^ ((r >> 1) & 7);
    asrc[u] = (MODE == 0 ? apr / a.P : apr) * C + 16 * p;
    adst[u] = 1024 * n;
  }
  const int nsteps = C / kDKS;
  auto stage_a = [&](auto bc) __attribute__((always_inline)) {
    constexpr int B = decltype(bc)::value;
    return B == 0 ? A0 : (B == 1 ? A1 : A2);
  };
  auto stage_b = [&](auto bc) __attribute__((always_inline)) {
    constexpr int B = decltype(bc)::value;
    return (B == 0 ? B0 : (B == 1 ? B1 : B2)) + wave * kDBWave;
  };
  auto issue = [&](int st, auto bc) __attribute__((always_inline)) {
    const int k0 = min(st, nsteps - 1) * kDKS;
    int8_t *bd = stage_b(bc);
#pragma unroll
    for (int i = 0; i < NS; i++) dma16(bsrc[i] + k0 / 2, bd + 1024 * i);
    int8_t *ad = stage_a(bc);
#pragma unroll
    for (int u = 0; u < AW; u++) dma16(a.act + asrc[u] + k0, ad + adst[u]);
  };
  v4i acc[MSV][NS];
#pragma unroll
  for (int ms = 0; ms < MSV; ms++)
#pragma unroll
    for (int s = 0; s < NS; s++) acc[ms][s] = v4i{0, 0, 0, 0};
  float sc[NS];
#pragma unroll
  for (int s = 0; s < NS; s++) sc[s] = t.Bm[s].s[min(t.ob[s], O - 1)];
  // shared offsets of the lane's MFMA-layout reads within a stage
  const int boff = ln * 64 + 16 * (j ^ ((ln >> 2) & 3));  // + subtile * 1024
  int aoff[2];
#pragma unroll
  for (int c = 0; c < 2; c++) aoff[c] = ln * kDARow + 16 * ((2 * j + c) ^ ((ln >> 1) & 7));

  issue(0, std::integral_constant<int, 0>{});
  issue(1, std::integral_constant<int, 1>{});
  auto step = [&](int st, auto bc) __attribute__((always_inline)) {
    constexpr int BUF = decltype(bc)::value;
    // after the barrier every wave's pieces of the step are in, and every
    // wave is done with the stage of step st - 1, which the request below
    // refills
    dma_step_barrier<PIECES>();
    issue(st + 2, std::integral_constant<int, (BUF + 2) % 3>{});
    const int8_t *bw = stage_b(bc) + boff;
    const int8_t *aw = stage_a(bc);
    uint4 bm[NS];
#pragma unroll
    for (int s = 0; s < NS; s++) bm[s] = *reinterpret_cast<const uint4 *>(bw + 1024 * s);
#pragma unroll
    for (int c = 0; c < 2; c++) {
      v4i aa[MSV];
#pragma unroll
      for (int ms = 0; ms < MSV; ms++) {
        const uint4 v = *reinterpret_cast<const uint4 *>(aw + ms * 16 * kDARow + aoff[c]);
        aa[ms] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
      }
      v4i bb[NS];
#pragma unroll
      for (int s = 0; s < NS; s++) bb[s] = c ? unpack16(bm[s].z, bm[s].w) : unpack16(bm[s].x, bm[s].y);
#pragma unroll
      for (int ms = 0; ms < MSV; ms++)
#pragma unroll
        for (int s = 0; s < NS; s++)
          acc[ms][s] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aa[ms], bb[s], acc[ms][s], 0, 0, 0);
    }
    // instruction order of the step: the weight reads and the first
    // activation reads, then each of the step's DMA requests between three
    // MFMAs and one shared read, then the remaining MFMAs (measured against
    // the compiler's own order: 857 against 883 us for gate/up, 474 against
    // 492 us for down at 2048 tokens)
    __builtin_amdgcn_sched_group_barrier(0x100, NS + 2, 0);  // shared-memory reads
#pragma unroll
    for (int g = 0; g < PIECES; g++) {
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);     // MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);     // global (DMA) request
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    constexpr int REST = 2 * MSV * NS - 3 * PIECES;  // small tiles have fewer MFMAs than the groups
    if constexpr (REST > 0) __builtin_amdgcn_sched_group_barrier(0x008, REST, 0);
  };
  int st = 0;
  for (; st + 2 < nsteps; st += 3) {
    step(st, std::integral_constant<int, 0>{});
    step(st + 1, std::integral_constant<int, 1>{});
    step(st + 2, std::integral_constant<int, 2>{});
  }
  if (st < nsteps) step(st, std::integral_constant<int, 0>{});
  if (st + 1 < nsteps) step(st + 1, std::integral_constant<int, 1>{});
  // the last requests (repeats of the last step) land in stages no step
  // reads; none may still be in flight when the workgroup ends
  wait_vm_at_most<0>();

  // epilogue as in mfma_tile
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
#pragma unroll
          for (int s = 0; s < NS / 2; s++) {
            const int o = t.ob[s];
            if (o < O) {
              const float gv = ((float)(acc[ms][s][i] - corr) * sc[s]) * as;
              const float uv = ((float)(acc[ms][s + NS / 2][i] - corr) * sc[s + NS / 2]) * as;
              a.out[(int64_t)pr * O + o] = silu(gv) * uv;
            }
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

// Two waves per SIMD: two 4-wave workgroups (80 KB of shared memory each)
// or one 8-wave workgroup per CU, at most 256 registers per wave.
template <int MODE, int NW, int MSVMAX>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void grouped_mfma_dma_kernel(GroupedMfmaArgs a) {
  constexpr int NS = kDNS;
  constexpr int ABUF = 16 * MSVMAX * kDARow;
  __shared__ __align__(1024) int8_t B0[NW * kDBWave], B1[NW * kDBWave], B2[NW * kDBWave];
  __shared__ __align__(1024) int8_t A0[ABUF], A1[ABUF], A2[ABUF];
  __shared__ int pr_l[16 * MSVMAX];
  __shared__ int sum_l[16 * MSVMAX];
  __shared__ float scl_l[16 * MSVMAX];
  // kDmaXcdTiles: a one-dimensional grid in which workgroup i reaches XCD
  // i % 8 (round-robin dispatch) and every XCD takes whole tiles, all row
  // chunks of one tile back to back, so a tile's activation rows are fetched
  // into one XCD's L2 once; otherwise blockIdx = (row chunk, tile)
  int tile, chunk;
  if (kDmaXcdTiles) {
    const int nx = (a.O + mfma_block_rows<MODE, NW, NS>() - 1) / mfma_block_rows<MODE, NW, NS>();
    const int xcd = blockIdx.x % 8, k = blockIdx.x / 8;
    tile = (k / nx) * 8 + xcd;
    chunk = k % nx;
  } else {
    tile = blockIdx.y;
    chunk = blockIdx.x;
  }
  if (tile >= *a.ntiles) return;
  const int2 tg = a.tiles[tile];
  const int g = tg.x, m0 = tg.y;
  MfmaTile t;
  t.rows = min(16 * MSVMAX, a.gcount[g] - m0);
  t.lane = threadIdx.x & 63;
  t.wave = threadIdx.x >> 6;
  t.j = t.lane >> 4;
  const bool shared = (g == a.E);
  const int e = shared ? 0 : g;
  const int o_blk = chunk * mfma_block_rows<MODE, NW, NS>();
  const RowPtr G = MODE == 0 ? pick(a.rt.gate, a.sh.gate, shared, e) : pick(a.rt.down, a.sh.down, shared, e);
  const RowPtr U = MODE == 0 ? pick(a.rt.up, a.sh.up, shared, e) : G;
  auto sub_row = [&](int s, int r) {
    return MODE == 0 ? o_blk + 8 * NS * t.wave + 16 * (s % (NS / 2)) + r
                     : o_blk + 16 * NS * t.wave + 16 * s + r;
  };
#pragma unroll
  for (int s = 0; s < NS; s++) {
    t.Bm[s] = (MODE == 0 && s >= NS / 2) ? U : G;
    t.ob[s] = sub_row(s, t.lane & 15);
    t.bbase[s] = t.Bm[s].q;
  }
  const int *plist = a.pairs + a.goff[g] + m0;
  for (int i = threadIdx.x; i < 16 * MSVMAX; i += NW * 64) {
    const int pr = plist[min(i, t.rows - 1)];
    const int ar = MODE == 0 ? pr / a.P : pr;
    pr_l[i] = pr;
    sum_l[i] = a.asum[ar];
    scl_l[i] = a.ascale[ar];
  }
  __syncthreads();
#define MOE_DMA_TILE(M) \
  dma_tile<MODE, NW, MSVMAX, M, ABUF>(a, t, A0, A1, A2, B0, B1, B2, pr_l, sum_l, scl_l)
  switch ((t.rows + 15) >> 4) {
    case 1: MOE_DMA_TILE(1); break;
    case 2: MOE_DMA_TILE(cmin(2, MSVMAX)); break;
    case 3: MOE_DMA_TILE(cmin(3, MSVMAX)); break;
    case 4: MOE_DMA_TILE(cmin(4, MSVMAX)); break;
    default: MOE_DMA_TILE(MSVMAX); break;
  }
#undef MOE_DMA_TILE
}

// ---- gate/up of large batches: 8-wave workgroups, 128-byte weight requests ----
//
// As grouped_mfma_dma_kernel<0, ..>, but one 8-wave workgroup per CU (8 x 64
// weight rows, so the activation ring serves 512 rows) and the weights
// requested two steps at a time: an instruction copies 8 rows x 128 bytes,
// a whole cache line of each row, where the single-step kernel copies 16
// rows x 64 bytes.  Weight ring: two double stages per wave (8 KB each);
// activations: the three-stage ring of single steps.  Step t requests, when
// t is even, the weights of steps t + 2 and t + 3 (requested first: 826-833
// against 831-839 us at 2048 tokens), then the activations of step t + 2.
// Layout of a wave's weight double stage: 64 rows x 128 bytes, row R (the
// wave's row; subtile R / 16) at 128 R; piece q of row R holds logical piece
// q ^ ((R >> 1) & 7), logical pieces 0-3 being the first step's 64 bytes.
constexpr int kD2Waves = 8;
constexpr int kD2BWave = 16 * kDNS * 128;  // weight bytes of a wave's double stage (8 KB)

template <int NW, int MSVMAX, int MSV, int ABUF>
__device__ __forceinline__ void dma2_tile(const GroupedMfmaArgs &a, const MfmaTile &t,
                                          int8_t *A0, int8_t *A1, int8_t *A2, int8_t *W0,
                                          int8_t *W1, const int *pr_l, const int *sum_l,
                                          const float *scl_l) {
  constexpr int NS = kDNS;
  constexpr int NA = 2 * MSV;  // activation DMA instructions of a stage (8 rows x 128 bytes each)
  constexpr int AW = dma_a_per_wave<NW, MSVMAX>();
  constexpr int NWI = 2 * NS;  // weight DMA instructions of a double stage (8 rows each)
  static_assert(AW + NWI < 16, "vmcnt field");
  const int C = a.C, O = a.O;
  const int lane = t.lane, j = t.j, rows = t.rows, wave = t.wave;
  const int ln = lane & 15;
  const int rowbytes = C >> 1;
  // weights: instruction i covers the wave's rows 8 i .. 8 i + 7; lane: row
  // 8 i + lane / 8, shared piece lane % 8
  const uint8_t *bsrc[NWI];
#pragma unroll
  for (int i = 0; i < NWI; i++) {
    const int R = 8 * i + (lane >> 3);
    const int s = R >> 4;
    const int o = t.ob[s] - ln + (R & 15);  // t.ob[s] is the output row of row ln of subtile s
    const int p = (lane & 7) ^ ((R >> 1) & 7);
    bsrc[i] = t.bbase[s] + (int64_t)min(o, O - 1) * rowbytes + 16 * p;
  }
  // activations: as in dma_tile
  int asrc[AW], adst[AW];
#pragma unroll
  for (int u = 0; u < AW; u++) {
    const int n = (wave + NW * u) % NA;
    const int r = 8 * n + (lane >> 3);
    const int apr = pr_l[min(r, rows - 1)];
    const int p = (lane & 7) ^ ((r >> 1) & 7);
    asrc[u] = (apr / a.P) * C + 16 * p;
    adst[u] = 1024 * n;
  }
  const int nsteps = C / kDKS, ndouble = nsteps / 2;
  auto stage_a = [&](auto bc) __attribute__((always_inline)) {
    constexpr int B = decltype(bc)::value;
    return B == 0 ? A0 : (B == 1 ? A1 : A2);
  };
  auto stage_w = [&](auto bc) __attribute__((always_inline)) {
    constexpr int B = decltype(bc)::value;
    return (B == 0 ? W0 : W1) + wave * kD2BWave;
  };
  auto issue_a = [&](int st, auto bc) __attribute__((always_inline)) {
    const int k0 = min(st, nsteps - 1) * kDKS;
    int8_t *ad = stage_a(bc);
#pragma unroll
    for (int u = 0; u < AW; u++) dma16(a.act + asrc[u] + k0, ad + adst[u]);
  };
  auto issue_w = [&](int d, auto bc) __attribute__((always_inline)) {
    const int k = min(d, ndouble - 1) * 128;
    int8_t *wd = stage_w(bc);
#pragma unroll
    for (int i = 0; i < NWI; i++) dma16(bsrc[i] + k, wd + 1024 * i);
  };
  v4i acc[MSV][NS];
#pragma unroll
  for (int ms = 0; ms < MSV; ms++)
#pragma unroll
    for (int s = 0; s < NS; s++) acc[ms][s] = v4i{0, 0, 0, 0};
  float sc[NS];
#pragma unroll
  for (int s = 0; s < NS; s++) sc[s] = t.Bm[s].s[min(t.ob[s], O - 1)];
  const int bswz = (ln >> 1) & 7;
  int aoff[2];
#pragma unroll
  for (int c = 0; c < 2; c++) aoff[c] = ln * kDARow + 16 * ((2 * j + c) ^ ((ln >> 1) & 7));

  // as if steps -2 and -1 had run: activations of steps 0 and 1, weights of 0 and 1
  issue_a(0, std::integral_constant<int, 0>{});
  issue_w(0, std::integral_constant<int, 0>{});
  issue_a(1, std::integral_constant<int, 1>{});
  // K = st % 12 fixes the activation stage (st % 3), the weight double
  // stage ((st / 2) % 2) and the half (st % 2)
  auto step = [&](int st, auto kc) __attribute__((always_inline)) {
    constexpr int K = decltype(kc)::value;
    constexpr int AB = K % 3, WB = (K / 2) % 2, H = K % 2;
    // in flight may stay what step st - 1 requested: activations, and on
    // odd st the weights requested by the even step before
    dma_step_barrier<H == 0 ? AW : AW + NWI>();
    if constexpr (H == 0) issue_w(st / 2 + 1, std::integral_constant<int, (WB + 1) % 2>{});
    issue_a(st + 2, std::integral_constant<int, (AB + 2) % 3>{});
    const int8_t *bw = stage_w(std::integral_constant<int, WB>{}) + 128 * ln + 16 * ((4 * H + j) ^ bswz);
    const int8_t *aw = stage_a(std::integral_constant<int, AB>{});
    uint4 bm[NS];
#pragma unroll
    for (int s = 0; s < NS; s++) bm[s] = *reinterpret_cast<const uint4 *>(bw + 2048 * s);
#pragma unroll
    for (int c = 0; c < 2; c++) {
      v4i aa[MSV];
#pragma unroll
      for (int ms = 0; ms < MSV; ms++) {
        const uint4 v = *reinterpret_cast<const uint4 *>(aw + ms * 16 * kDARow + aoff[c]);
        aa[ms] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
      }
      v4i bb[NS];
#pragma unroll
      for (int s = 0; s < NS; s++) bb[s] = c ? unpack16(bm[s].z, bm[s].w) : unpack16(bm[s].x, bm[s].y);
#pragma unroll
      for (int ms = 0; ms < MSV; ms++)
#pragma unroll
        for (int s = 0; s < NS; s++)
          acc[ms][s] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aa[ms], bb[s], acc[ms][s], 0, 0, 0);
    }
    constexpr int PIECES = H == 0 ? AW + NWI : AW;
    // the step's order as in dma_tile (the compiler's own: 847 against 835 us)
    __builtin_amdgcn_sched_group_barrier(0x100, NS + 2, 0);  // shared-memory reads
#pragma unroll
    for (int g = 0; g < PIECES; g++) {
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);     // MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);     // global (DMA) request
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    constexpr int REST = 2 * MSV * NS - 3 * PIECES;
    if constexpr (REST > 0) __builtin_amdgcn_sched_group_barrier(0x008, REST, 0);
  };
  auto steps = [&](int st, int n) __attribute__((always_inline)) {
    if (n > 0) step(st, std::integral_constant<int, 0>{});
    if (n > 1) step(st + 1, std::integral_constant<int, 1>{});
    if (n > 2) step(st + 2, std::integral_constant<int, 2>{});
    if (n > 3) step(st + 3, std::integral_constant<int, 3>{});
    if (n > 4) step(st + 4, std::integral_constant<int, 4>{});
    if (n > 5) step(st + 5, std::integral_constant<int, 5>{});
    if (n > 6) step(st + 6, std::integral_constant<int, 6>{});
    if (n > 7) step(st + 7, std::integral_constant<int, 7>{});
    if (n > 8) step(st + 8, std::integral_constant<int, 8>{});
    if (n > 9) step(st + 9, std::integral_constant<int, 9>{});
    if (n > 10) step(st + 10, std::integral_constant<int, 10>{});
    if (n > 11) step(st + 11, std::integral_constant<int, 11>{});
  };
  int st = 0;
  for (; st + 12 <= nsteps; st += 12) steps(st, 12);
  steps(st, nsteps - st);
  // the last requests (repeats of the last steps) land in stages no step
  // reads; none may still be in flight when the workgroup ends
  wait_vm_at_most<0>();

#pragma unroll
  for (int ms = 0; ms < MSV; ms++) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int r = 16 * ms + 4 * j + i;
      if (r < rows) {
        const int pr = pr_l[r];
        const int corr = 8 * sum_l[r];
        const float as = scl_l[r];
#pragma unroll
        for (int s = 0; s < NS / 2; s++) {
          const int o = t.ob[s];
          if (o < O) {
            const float gv = ((float)(acc[ms][s][i] - corr) * sc[s]) * as;
            const float uv = ((float)(acc[ms][s + NS / 2][i] - corr) * sc[s + NS / 2]) * as;
            a.out[(int64_t)pr * O + o] = silu(gv) * uv;
          }
        }
      }
    }
  }
}

// One 8-wave workgroup per CU (159 KB of shared memory), two waves per SIMD.
template <int MSVMAX>
__global__ __launch_bounds__(kD2Waves * 64) __attribute__((amdgpu_waves_per_eu(2)))
void grouped_mfma_dma2_kernel(GroupedMfmaArgs a) {
  constexpr int NW = kD2Waves, NS = kDNS;
  constexpr int ABUF = 16 * MSVMAX * kDARow;
  __shared__ __align__(1024) int8_t W0[NW * kD2BWave], W1[NW * kD2BWave];
  __shared__ __align__(1024) int8_t A0[ABUF], A1[ABUF], A2[ABUF];
  __shared__ int pr_l[16 * MSVMAX];
  __shared__ int sum_l[16 * MSVMAX];
  __shared__ float scl_l[16 * MSVMAX];
  // whole tiles per XCD, all row chunks of a tile back to back (as in
  // grouped_mfma_dma_kernel)
  const int nx = (a.O + mfma_block_rows<0, NW, NS>() - 1) / mfma_block_rows<0, NW, NS>();
  const int xcd = blockIdx.x % 8, k = blockIdx.x / 8;
  const int tile = (k / nx) * 8 + xcd, chunk = k % nx;
  if (tile >= *a.ntiles) return;
  const int2 tg = a.tiles[tile];
  const int g = tg.x, m0 = tg.y;
  MfmaTile t;
  t.rows = min(16 * MSVMAX, a.gcount[g] - m0);
  t.lane = threadIdx.x & 63;
  t.wave = threadIdx.x >> 6;
  t.j = t.lane >> 4;
  const bool shared = (g == a.E);
  const int e = shared ? 0 : g;
  const int o_blk = chunk * mfma_block_rows<0, NW, NS>();
  const RowPtr G = pick(a.rt.gate, a.sh.gate, shared, e);
  const RowPtr U = pick(a.rt.up, a.sh.up, shared, e);
#pragma unroll
  for (int s = 0; s < NS; s++) {
    t.Bm[s] = s >= NS / 2 ? U : G;
    t.ob[s] = o_blk + 8 * NS * t.wave + 16 * (s % (NS / 2)) + (t.lane & 15);
    t.bbase[s] = t.Bm[s].q;
  }
  const int *plist = a.pairs + a.goff[g] + m0;
  for (int i = threadIdx.x; i < 16 * MSVMAX; i += NW * 64) {
    const int pr = plist[min(i, t.rows - 1)];
    const int ar = pr / a.P;
    pr_l[i] = pr;
    sum_l[i] = a.asum[ar];
    scl_l[i] = a.ascale[ar];
  }
  __syncthreads();
#define MOE_DMA2_TILE(M) dma2_tile<NW, MSVMAX, M, ABUF>(a, t, A0, A1, A2, W0, W1, pr_l, sum_l, scl_l)
  switch ((t.rows + 15) >> 4) {
    case 1: MOE_DMA2_TILE(1); break;
    case 2: MOE_DMA2_TILE(cmin(2, MSVMAX)); break;
    case 3: MOE_DMA2_TILE(cmin(3, MSVMAX)); break;
    case 4: MOE_DMA2_TILE(cmin(4, MSVMAX)); break;
    default: MOE_DMA2_TILE(MSVMAX); break;
  }
#undef MOE_DMA2_TILE
}

bool grouped_mfma_fits(int C) { return C % kKS == 0; }

// Pairs per tile: as many as the launch's workgroups hold.  A group larger
// than that (a routed expert with more pairs, or the shared expert) is cut
// into several tiles.  With the router's selection no group of a batch of S
// <= 64 tokens exceeds 64 pairs, but given routing may repeat an expert
// within a token or clamp several ids onto one expert.
int grouped_mfma_tile_rows(int S) { return 16 * (S > 64 ? kLargeMsv : kSmallMsv); }

int grouped_mfma_max_tiles(int S, int P, int E) {
  const int tr = grouped_mfma_tile_rows(S);
  return (S * P + tr - 1) / tr + E + 1;
}

template <int MODE, int NW, int NS, int MSVMAX>
static void launch_mode(const GroupedMfmaArgs &a, int max_tiles, hipStream_t st) {
  constexpr int RPB = mfma_block_rows<MODE, NW, NS>();
  const dim3 grid((a.O + RPB - 1) / RPB, max_tiles);
  hipLaunchKernelGGL((grouped_mfma_kernel<MODE, NW, NS, MSVMAX>), grid, dim3(NW * 64), 0, st, a);
}

// Batches of up to 64 tokens (at most 4 subtiles per tile): 4-wave
// workgroups of 32 B rows per wave, so that a few experts still spread over
// many workgroups (the DMA kernel took the 64-token verify from 532 to 632
// us); larger batches: 64 B rows per wave, gate/up in grouped_mfma_dma2_kernel
// (against grouped_mfma_dma_kernel: 2048 tokens 829-839 against 857-862 us,
// the union call 1 to 4 % faster from 96 to 2048 tokens), down in
// grouped_mfma_dma_kernel (the double-step form was slower there, 1555-1561
// against 1540-1550 us per 2048-token call).
hipError_t launch_grouped_mfma(const GroupedMfmaArgs &a, int mode, int max_tiles, int S,
                               hipStream_t st) {
  if (S <= 64) {
    if (mode == 0)
      launch_mode<0, 4, 2, kSmallMsv>(a, max_tiles, st);
    else
      launch_mode<1, 4, 2, kSmallMsv>(a, max_tiles, st);
  } else if (mode == 0) {
    // gate/up: 8-wave workgroups, the weights requested two steps at a time
    constexpr int RPB = mfma_block_rows<0, kD2Waves, kDNS>();
    const int nx = (a.O + RPB - 1) / RPB;
    hipLaunchKernelGGL((grouped_mfma_dma2_kernel<kLargeMsv>), dim3(nx * ((max_tiles + 7) / 8) * 8),
                       dim3(kD2Waves * 64), 0, st, a);
  } else {
    constexpr int NW = kPrefillDmaWaves;
    constexpr int RPB = mfma_block_rows<1, NW, kDNS>();
    const int nx = (a.O + RPB - 1) / RPB;
    const dim3 grid = kDmaXcdTiles ? dim3(nx * ((max_tiles + 7) / 8) * 8) : dim3(nx, max_tiles);
    hipLaunchKernelGGL((grouped_mfma_dma_kernel<1, NW, kLargeMsv>), grid, dim3(NW * 64), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace moe
