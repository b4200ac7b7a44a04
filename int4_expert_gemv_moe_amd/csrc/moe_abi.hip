// moe_abi.hip -- the extern "C" entry points declared in include/moe_i4.h:
// host-side validation, workspace carving and the launch sequence of each
// call.  No call allocates device memory.
#include <algorithm>
#include <vector>
#include <atomic>
#include <mutex>
#include <cstdio>
#include <cstring>

#include "moe_kernels.h"
#include "norm.h"

using namespace moe;

namespace moe {
// host bookkeeping of the residency tiers (tier.hip)
void tier_sizes(const moe_tier *t, int *n_experts, int *n_slot_total);
void tier_unmap_loads(moe_tier *t, int layer, const int32_t *eids, const int32_t *slots,
                      const int32_t *loads, int n);
}  // namespace moe

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Per-device memo of "is this a gfx950" (read-only device property).
std::atomic<int> g_arch_ok[64];

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_EHIP;
  if (dev < 0 || dev >= 64) return MOE_EDEVICE;
  int v = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_EHIP;
    v = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_arch_ok[dev].store(v, std::memory_order_relaxed);
  }
  return v == 1 ? MOE_OK : MOE_EDEVICE;
}

int check_cfg(const moe_config *c) {
  if (!c) return MOE_EINVAL;
  if (c->D < 256 || c->I < 32 || c->D % 256 || c->I % 32) return MOE_ESHAPE;
  if (!gemv_cols_ok(c->D) || !gemv_cols_ok(c->I)) return MOE_ESHAPE;
  if (c->E < 1 || c->E > 1024 || c->K < 1 || c->K > c->E || c->K > 64) return MOE_ESHAPE;
  if (c->n_shared < 0 || c->n_shared > 1) return MOE_ESHAPE;
  if (!(c->routed_scale == c->routed_scale)) return MOE_EINVAL;
  if (!(c->expert_topp >= 0.f && c->expert_topp <= 1.f)) return MOE_EINVAL;
  return MOE_OK;
}

enum Which { W_FWD = 0, W_BATCH = 1, W_SWIGLU = 2, W_ROUTER = 3, W_SWIGLU8 = 4, W_SHARED8 = 5 };

// Shapes whose int8 shared expert runs inside the per-token path's launches
// (whole 1 KB chunks of its rows, within the kernels' instantiations):
// D % 2048 == 0 and D <= 8192, I % 1024 == 0 and I <= 4096.  Other shapes
// run it in launches of its own after the routed experts.
bool shared8_fused_ok(const moe_config &c) {
  return c.D % 2048 == 0 && c.D <= 8192 && c.I % 1024 == 0 && c.I <= 4096;
}

// Workspace of moe_layer_forward_shared_i8: the per-token path's with the
// shared slot (fused shapes), else the union path's.
size_t carve(const moe_config &c, int S, int which, char *base, struct Work *w);
size_t shared8_bytes(const moe_config &c, int S) {
  return carve(c, S, shared8_fused_ok(c) ? W_FWD : W_BATCH, nullptr, nullptr);
}

// Workgroup counts of the per-token path (rows of a phase are split evenly
// over its workgroups): shared gate/up (phase A), routed gate/up over the
// concatenated slots and shared down (phase B), routed down (phase C).  The
// counts were swept on the device at the GLM shape.
struct DecodeShape {
  int gu_fx, gu_rt, dn_fx, dn;
  int gu_fx8, dn_fx8;  // the same for an int8 fixed expert (rows twice as long)
  int gu_one, dn_one;  // a one-expert call (the expert has the chip to itself)
};

#ifndef MOE_ONE_GU
#define MOE_ONE_GU 256
#endif
#ifndef MOE_ONE_DN
#define MOE_ONE_DN 256
#endif

DecodeShape decode_shape(const moe_config &c) {
  DecodeShape d;
  d.gu_fx = 128;
  d.gu_rt = 256;
  d.dn_fx = 192;
  d.gu_fx8 = 256;
  d.dn_fx8 = 256;
  d.gu_one = MOE_ONE_GU;
  d.dn_one = MOE_ONE_DN;
  // phase C: one pass of rows per workgroup
  const int cr = decode_c_rows_per_pass(c.I);
  d.dn = (c.D + cr - 1) / cr;
  // at least 8 rows per workgroup, at most the rows whose scales fit in LDS
  // (512 for gate/up, 256 for down)
  auto clampn = [](int n, int rows, int maxrows) {
    const int lo = (rows + maxrows - 1) / maxrows, hi = std::max(1, rows / 8);
    return std::max(lo, std::min(n, hi));
  };
  d.gu_fx = clampn(d.gu_fx, c.I, 512);
  d.gu_rt = clampn(d.gu_rt, c.I * c.K, 512);
  d.dn_fx = clampn(d.dn_fx, c.D, 256);
  d.dn = clampn(d.dn, c.D, 256);
  d.gu_fx8 = clampn(d.gu_fx8, c.I, 512);
  d.dn_fx8 = clampn(d.dn_fx8, c.D, 256);
  d.gu_one = clampn(d.gu_one, c.I, 512);
  d.dn_one = clampn(d.dn_one, c.D, 256);
  return d;
}

// Workspace carving.  With base == nullptr only the size is computed.
size_t carve(const moe_config &c, int S, int which, char *base, Work *w) {
  const int P = (which == W_SWIGLU) ? 1 : c.K + c.n_shared;
  const size_t s = (size_t)S;
  size_t off = 0;
  auto take = [&](size_t bytes) -> char * {
    char *p = base ? base + off : nullptr;
    off += align_up(bytes);
    return p;
  };
  Work t{};
  if (which == W_SWIGLU8) {
    t.h = (float *)take(s * c.I * 4);
    if (w) *w = t;
    return off;
  }
  if (which != W_SWIGLU) {
    t.logits = (float *)take(s * c.E * 4);
    t.idx = (int32_t *)take(s * c.K * 4);
    t.w = (float *)take(s * c.K * 4);
    t.keff = (int32_t *)take(s * 4);
  }
  if (which != W_ROUTER) {
    t.xq = (int8_t *)take(s * c.D);
    t.sx = (float *)take(s * 4);
    t.sumx = (int32_t *)take(s * 4);
    t.h = (float *)take(s * P * c.I * 4);
  }
  if (which == W_FWD || which == W_SWIGLU) {
    t.ysh = (float *)take(s * c.D * 4);
    t.tmp = (float *)take(s * c.D * 4);
  }
  if (which == W_BATCH) {
    t.hq = (int8_t *)take(s * P * c.I);
    t.sh = (float *)take(s * P * 4);
    t.sumh = (int32_t *)take(s * P * 4);
    t.gcount = (int32_t *)take((size_t)(c.E + 1) * 4);
    t.goff = (int32_t *)take((size_t)(c.E + 2) * 4);
    t.pairs = (int32_t *)take(s * P * 4);
    t.stage = (float *)take(s * P * c.D * 4);
    t.tiles = (int2 *)take((size_t)grouped_mfma_max_tiles(S, P, c.E) * 8);
    t.ntiles = (int32_t *)take(4);
    t.xn = (float *)take(s * c.D * 4);
  }
  if (w) *w = t;
  return off;
}

QMat to_qmat(const moe_qmat &m, int O, int C) {
  QMat q;
  q.q4 = m.q4;
  q.scale = m.scale;
  q.q4_stride = m.q4_stride ? m.q4_stride : (int64_t)O * (C / 2);
  q.s_stride = m.scale_stride ? m.scale_stride : (int64_t)O;
  return q;
}

ExpertSet to_set(const moe_experts &e, const moe_config &c) {
  ExpertSet s;
  s.gate = to_qmat(e.gate, c.I, c.D);
  s.up = to_qmat(e.up, c.I, c.D);
  s.down = to_qmat(e.down, c.D, c.I);
  return s;
}

int check_qmat(const moe_qmat &m) {
  if (!m.q4 || !m.scale) return MOE_EINVAL;
  if (!aligned16(m.q4) || ((uintptr_t)m.scale & 3u)) return MOE_EALIGN;
  if (m.q4_stride < 0 || m.scale_stride < 0 || (m.q4_stride & 15)) return MOE_EALIGN;
  return MOE_OK;
}

int check_experts(const moe_experts &e) {
  int rc;
  if ((rc = check_qmat(e.gate)) || (rc = check_qmat(e.up)) || (rc = check_qmat(e.down))) return rc;
  return MOE_OK;
}

int check_q8mat(const moe_q8mat &m) {
  if (!m.q || !m.scale) return MOE_EINVAL;
  if (!aligned16(m.q) || ((uintptr_t)m.scale & 3u)) return MOE_EALIGN;
  if (m.q_stride < 0 || m.scale_stride < 0 || (m.q_stride & 15)) return MOE_EALIGN;
  return MOE_OK;
}

int check_experts_i8(const moe_experts_i8 &e) {
  int rc;
  if ((rc = check_q8mat(e.gate)) || (rc = check_q8mat(e.up)) || (rc = check_q8mat(e.down))) return rc;
  return MOE_OK;
}

// Expert e's codes and scales in a stacked int8 matrix of O x C.
void q8_rows(const moe_q8mat &m, int O, int C, int e, const int8_t **q, const float **s) {
  const int64_t qs = m.q_stride ? m.q_stride : (int64_t)O * C;
  const int64_t ss = m.scale_stride ? m.scale_stride : (int64_t)O;
  *q = m.q + (int64_t)e * qs;
  *s = m.scale + (int64_t)e * ss;
}

// shared_i4: the shared expert is layer->shared (otherwise the caller passes
// it in another format and checks it itself).
int check_layer(const moe_config &c, const moe_layer *L, bool router = true,
                bool shared_i4 = true) {
  if (!L) return MOE_EINVAL;
  if (router) {
    if (!L->router_w || !L->router_b) return MOE_EINVAL;
    if (!aligned16(L->router_w) || ((uintptr_t)L->router_b & 3u)) return MOE_EALIGN;
  }
  int rc = check_experts(L->routed);
  if (rc) return rc;
  if (c.n_shared && shared_i4) return check_experts(L->shared);
  return MOE_OK;
}

__global__ void moe_zero_kernel(uint4 *p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

int hip_rc(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

#define MOE_TRY(expr)             \
  do {                            \
    int rc_ = (expr);             \
    if (rc_ != MOE_OK) return rc_; \
  } while (0)

#define MOE_TRY_HIP(expr) MOE_TRY(hip_rc(expr))

// Router logits (+ activation quantization); the top-K runs in a kernel of
// its own when with_topk, otherwise inside the per-token gate/up kernel.
int run_router(const moe_config &c, const float *x, int S, const float *W, const float *b,
               const Work &w, bool with_quant, bool with_topk, float *logits_out, hipStream_t st,
               const float *gamma = nullptr, float eps = 0.f, const uint16_t *xb = nullptr) {
  RouterArgs r{};
  r.gamma = gamma;
  r.eps = eps;
  r.x = xb ? nullptr : x;
  r.xb = xb;
  r.W = W;
  r.S = S;
  r.D = c.D;
  r.E = c.E;
  r.logits = w.logits;
  r.logits_out = logits_out;
  r.xq_perm = w.xq;
  r.sx = w.sx;
  r.sumx = w.sumx;
  r.amax = nullptr;
  r.P = c.K + c.n_shared;
  MOE_TRY_HIP(launch_router(r, with_quant, st));
  if (with_topk) {
    TopkArgs t{w.logits, b, S, c.E, c.K, c.routed_scale, w.idx, w.w, c.expert_topp, w.keff};
    MOE_TRY_HIP(launch_topk(t, st));
  }
  return MOE_OK;
}

int copy_probe(const moe_config &c, int S, const moe_probe *probe, const Work &w,
               hipStream_t st) {
  if (!probe) return MOE_OK;
  const size_t n = (size_t)S * c.K;
  if (probe->topk_idx)
    MOE_TRY_HIP(hipMemcpyAsync(probe->topk_idx, w.idx, n * 4, hipMemcpyDeviceToDevice, st));
  if (probe->topk_w)
    MOE_TRY_HIP(hipMemcpyAsync(probe->topk_w, w.w, n * 4, hipMemcpyDeviceToDevice, st));
  if (probe->keff)
    MOE_TRY_HIP(hipMemcpyAsync(probe->keff, w.keff, (size_t)S * 4, hipMemcpyDeviceToDevice, st));
  return MOE_OK;
}

int record(const moe_probe *probe, int which, int side, hipStream_t st) {
  if (!probe) return MOE_OK;
  const hipEvent_t *ev = which == 0 ? probe->ev_gateup : probe->ev_down;
  if (!ev[0] || !ev[1]) return MOE_OK;
  return hip_rc(hipEventRecord(ev[side], st));
}

int layer_common_checks(const moe_config *cfg, const moe_layer *layer, const float *x, int S,
                        float *out, unsigned flags, void *ws, size_t ws_bytes, int which,
                        bool router = true, bool shared_i4 = true) {
  MOE_TRY(check_cfg(cfg));
  if (S < 1 || !x || !out || !ws) return MOE_EINVAL;
  if (flags & ~(MOE_F_ACCUMULATE | MOE_F_PRENORM | MOE_F_X_BF16)) return MOE_EINVAL;
  // bf16 tokens: union-path calls only, without the in-call RMSNorm
  if ((flags & MOE_F_X_BF16) && (which != W_BATCH || (flags & MOE_F_PRENORM))) return MOE_EINVAL;
  MOE_TRY(check_layer(*cfg, layer, router, shared_i4));
  if (!aligned16(x) || ((uintptr_t)out & 3u) || ((uintptr_t)ws & 255u)) return MOE_EALIGN;
  const bool prenorm = (flags & MOE_F_PRENORM) != 0;
  if (prenorm) {
    const float eps = layer->norm_eps;
    if (!layer->norm_gamma || !(eps > 0.f) || !(eps < INFINITY)) return MOE_EINVAL;
    if (!rms_vec_ok(cfg->D, x, layer->norm_gamma)) return MOE_EALIGN;
  }
  // out may be x itself only for the in-place residual update of PRENORM:
  // every read of x then precedes the first write of out
  const size_t xb = (size_t)S * cfg->D * ((flags & MOE_F_X_BF16) ? 2 : 4);
  const bool same = (const void *)out == (const void *)x;
  if ((const char *)out < (const char *)x + xb && (const char *)x < (const char *)out + xb &&
      !(prenorm && same))
    return MOE_EINVAL;
  if (ws_bytes < carve(*cfg, S, which, nullptr, nullptr)) return MOE_EWORKSPACE;
  return check_device();
}

}  // namespace

extern "C" {

const char *moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_ESHAPE: return "unsupported shape";
    case MOE_EALIGN: return "misaligned buffer";
    case MOE_EWORKSPACE: return "workspace too small";
    case MOE_EHIP: return "HIP error";
    case MOE_EDEVICE: return "device is not a gfx950";
    default: return "unknown status";
  }
}

size_t moe_workspace_bytes(const moe_config *cfg, int S, int which) {
  if (check_cfg(cfg) != MOE_OK || S < 1 || which < 0 || which > 5) return 0;
  if (which == W_SHARED8) return cfg->n_shared == 1 ? shared8_bytes(*cfg, S) : 0;
  return carve(*cfg, S, which, nullptr, nullptr);
}

int moe_workspace_init(void *ws, size_t ws_bytes, hipStream_t stream) {
  if (!ws) return MOE_EINVAL;
  if (((uintptr_t)ws & 255u) || (ws_bytes & 15u)) return MOE_EALIGN;
  MOE_TRY(check_device());
  const size_t n16 = ws_bytes / 16;
  if (n16 == 0) return MOE_OK;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(moe_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (uint4 *)ws, n16);
  return hip_rc(hipGetLastError());
}

int moe_pack_int4(const float *w, int O, int C, uint8_t *q4, float *scale, hipStream_t stream) {
  if (!w || !q4 || !scale) return MOE_EINVAL;
  if (O < 1 || C < 2 || (C & 1)) return MOE_ESHAPE;
  if (((uintptr_t)w & 7u) || ((uintptr_t)scale & 3u)) return MOE_EALIGN;
  MOE_TRY(check_device());
  PackArgs a{w, O, C, q4, scale};
  return hip_rc(launch_pack(a, stream));
}

int moe_quantize_rows_i8(const float *w, int O, int C, int8_t *q, float *scale,
                         hipStream_t stream) {
  if (!w || !q || !scale) return MOE_EINVAL;
  if (O < 1 || C < 1) return MOE_ESHAPE;
  if (((uintptr_t)w & 3u) || ((uintptr_t)scale & 3u)) return MOE_EALIGN;
  MOE_TRY(check_device());
  Q8QuantArgs a{w, O, C, q, scale};
  return hip_rc(launch_quant_rows_i8(a, stream));
}

int moe_expert_swiglu_i8(const moe_config *cfg, const int8_t *xq, const float *sx, int S,
                         const moe_experts_i8 *wts, int expert, float *y, int32_t *acc_gu,
                         int8_t *hq, float *sh, int32_t *acc_d, void *ws, size_t ws_bytes,
                         hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  if (S < 1 || !xq || !sx || !wts || !y || !ws) return MOE_EINVAL;
  if (expert < 0 || expert >= cfg->E) return MOE_EINVAL;
  MOE_TRY(check_experts_i8(*wts));
  if (!aligned16(xq) || ((uintptr_t)sx & 3u) || ((uintptr_t)y & 3u) || ((uintptr_t)ws & 255u))
    return MOE_EALIGN;
  if ((hq && !aligned16(hq)) || ((uintptr_t)sh & 3u) || ((uintptr_t)acc_gu & 3u) ||
      ((uintptr_t)acc_d & 3u))
    return MOE_EALIGN;
  if (ws_bytes < carve(*cfg, S, W_SWIGLU8, nullptr, nullptr)) return MOE_EWORKSPACE;
  MOE_TRY(check_device());
  Work w;
  carve(*cfg, S, W_SWIGLU8, (char *)ws, &w);
  Swiglu8Args a{};
  a.xq = xq;
  a.sx = sx;
  a.S = S;
  a.D = cfg->D;
  a.I = cfg->I;
  q8_rows(wts->gate, cfg->I, cfg->D, expert, &a.G, &a.gs);
  q8_rows(wts->up, cfg->I, cfg->D, expert, &a.U, &a.us);
  q8_rows(wts->down, cfg->D, cfg->I, expert, &a.Dn, &a.ds);
  a.h = w.h;
  a.acc_gu = acc_gu;
  a.hq_out = hq;
  a.sh_out = sh;
  a.y = y;
  a.acc_d = acc_d;
  MOE_TRY_HIP(launch_swiglu8_gateup(a, stream));
  MOE_TRY_HIP(launch_swiglu8_down(a, stream));
  return MOE_OK;
}

int moe_pack_int2(const float *w, int O, int C, uint8_t *q2, float *scale, hipStream_t stream) {
  if (!w || !q2 || !scale) return MOE_EINVAL;
  if (O < 1 || C < 1) return MOE_ESHAPE;
  if (((uintptr_t)w & 3u) || ((uintptr_t)scale & 3u)) return MOE_EALIGN;
  MOE_TRY(check_device());
  Pack2Args a{w, O, C, q2, scale};
  return hip_rc(launch_pack_int2(a, stream));
}

int moe_expert_swiglu_i2(const moe_config *cfg, const int8_t *xq, const float *sx, int S,
                         const moe_experts *wts, int expert, float *y, int32_t *acc_gu,
                         int8_t *hq, float *sh, int32_t *acc_d, void *ws, size_t ws_bytes,
                         hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  if (cfg->I % 64) return MOE_ESHAPE;
  if (S < 1 || !xq || !sx || !wts || !y || !ws) return MOE_EINVAL;
  if (expert < 0 || expert >= cfg->E) return MOE_EINVAL;
  MOE_TRY(check_experts(*wts));
  if (!aligned16(xq) || ((uintptr_t)sx & 3u) || ((uintptr_t)y & 3u) || ((uintptr_t)ws & 255u))
    return MOE_EALIGN;
  if ((hq && !aligned16(hq)) || ((uintptr_t)sh & 3u) || ((uintptr_t)acc_gu & 3u) ||
      ((uintptr_t)acc_d & 3u))
    return MOE_EALIGN;
  if (ws_bytes < carve(*cfg, S, W_SWIGLU8, nullptr, nullptr)) return MOE_EWORKSPACE;
  MOE_TRY(check_device());
  Work w;
  carve(*cfg, S, W_SWIGLU8, (char *)ws, &w);
  auto rows = [&](const moe_qmat &m, int O, int C, const uint8_t **q, const float **sc) {
    const int64_t qs = m.q4_stride ? m.q4_stride : (int64_t)O * (C / 4);
    const int64_t ss = m.scale_stride ? m.scale_stride : (int64_t)O;
    *q = m.q4 + (int64_t)expert * qs;
    *sc = m.scale + (int64_t)expert * ss;
  };
  Swiglu2Args a{};
  a.xq = xq;
  a.sx = sx;
  a.S = S;
  a.D = cfg->D;
  a.I = cfg->I;
  rows(wts->gate, cfg->I, cfg->D, &a.G, &a.gs);
  rows(wts->up, cfg->I, cfg->D, &a.U, &a.us);
  rows(wts->down, cfg->D, cfg->I, &a.Dn, &a.ds);
  a.h = w.h;
  a.acc_gu = acc_gu;
  a.hq_out = hq;
  a.sh_out = sh;
  a.y = y;
  a.acc_d = acc_d;
  MOE_TRY_HIP(launch_swiglu2_gateup(a, stream));
  MOE_TRY_HIP(launch_swiglu2_down(a, stream));
  return MOE_OK;
}

namespace {
int mla_check(const moe_mla_config *c, int S, int T) {
  if (!c) return MOE_EINVAL;
  if (c->H < 1 || c->kvl < 64 || c->kvl % 64 || c->kvl > 1024) return MOE_ESHAPE;
  if (c->nope < 1 || c->rope < 0 || c->rope > 64 || c->vdim < 1) return MOE_ESHAPE;
  if (S < 1 || T < S || T > kMlaMaxChunk * kMlaMaxSplit) return MOE_ESHAPE;
  if (!(c->scale == c->scale)) return MOE_EINVAL;
  return MOE_OK;
}

// L and R: the call's cache arrays (their alignment chooses the attention
// kernel); moe_mla_workspace_bytes sizes for the larger of the two layouts.
size_t mla_carve(const moe_mla_config &c, int S, int T, char *base, MlaArgs *a,
                 const float *L = nullptr, const float *R = nullptr, bool size_max = false) {
  const int chunk = mla_chunk_rows(T);
  const size_t ns_v = (size_t)((T + chunk - 1) / chunk);
  const size_t ns_m = (size_t)mla_mfma_splits(S, T, c.H);
  const bool mf = mla_mfma_fits(c.kvl, c.rope, L, R);
  const size_t sh = (size_t)S * c.H;
  const size_t ns = size_max ? std::max(ns_v, ns_m) : (mf ? ns_m : ns_v);
  size_t off = 0;
  auto take = [&](size_t bytes) -> float * {
    float *p = base ? (float *)(base + off) : nullptr;
    off += align_up(bytes);
    return p;
  };
  float *qabs = take(sh * c.kvl * 4);
  float *pclat = take(sh * ns * c.kvl * 4);
  float *pm = take(sh * ns * 4);
  float *pl = take(sh * ns * 4);
  float *clat = take(sh * c.kvl * 4);
  if (a) {
    a->clat = clat;
    a->qabs = qabs;
    a->pclat = pclat;
    a->pm = pm;
    a->pl = pl;
    a->nsplit = (int)ns;
    a->chunk = chunk;
  }
  return off;
}
}  // namespace

size_t moe_mla_workspace_bytes(const moe_mla_config *cfg, int S, int T) {
  if (mla_check(cfg, S, T) != MOE_OK) return 0;
  return mla_carve(*cfg, S, T, nullptr, nullptr, nullptr, nullptr, true);
}

int moe_mla_decode(const moe_mla_config *cfg, const float *q, int S, const float *kv_b,
                   const float *L, const float *R, int T, float *ctx, void *ws, size_t ws_bytes,
                   hipStream_t stream) {
  MOE_TRY(mla_check(cfg, S, T));
  if (!q || !kv_b || !L || (cfg->rope > 0 && !R) || !ctx || !ws) return MOE_EINVAL;
  if (((uintptr_t)q & 3u) || !aligned16(kv_b) || ((uintptr_t)L & 3u) ||
      ((uintptr_t)R & 3u) || ((uintptr_t)ctx & 3u) || ((uintptr_t)ws & 255u))
    return MOE_EALIGN;
  if (ws_bytes < mla_carve(*cfg, S, T, nullptr, nullptr, L, R)) return MOE_EWORKSPACE;
  MOE_TRY(check_device());
  MlaArgs a{};
  mla_carve(*cfg, S, T, (char *)ws, &a, L, R);
  a.S = S;
  a.T = T;
  a.H = cfg->H;
  a.kvl = cfg->kvl;
  a.nope = cfg->nope;
  a.rope = cfg->rope;
  a.vdim = cfg->vdim;
  a.scale = cfg->scale;
  a.q = q;
  a.kv_b = kv_b;
  a.L = L;
  a.R = R;
  a.ctx = ctx;
  return hip_rc(launch_mla_decode(a, stream));
}

int moe_quant_act_b32(const float *x, int S, int D, int8_t *xq, float *sxb, hipStream_t stream) {
  if (!x || !xq || !sxb) return MOE_EINVAL;
  if (S < 1 || D < 32 || (D & 31)) return MOE_ESHAPE;
  if (!aligned16(x) || !aligned16(xq) || ((uintptr_t)sxb & 3u)) return MOE_EALIGN;
  MOE_TRY(check_device());
  QuantB32Args a{x, S, D, xq, sxb};
  return hip_rc(launch_quant_b32(a, stream));
}

int moe_expert_swiglu_i4_b32(const moe_config *cfg, const int8_t *xq, const float *sxb, int S,
                             const moe_experts *wts, int expert, float *y, int8_t *hq, float *shb,
                             void *ws, size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  if (S < 1 || !xq || !sxb || !wts || !y || !ws) return MOE_EINVAL;
  if (expert < 0 || expert >= cfg->E) return MOE_EINVAL;
  MOE_TRY(check_experts(*wts));
  if (!aligned16(xq) || ((uintptr_t)sxb & 3u) || ((uintptr_t)y & 3u) || ((uintptr_t)ws & 255u))
    return MOE_EALIGN;
  if ((hq && !aligned16(hq)) || ((uintptr_t)shb & 3u)) return MOE_EALIGN;
  if (ws_bytes < carve(*cfg, S, W_SWIGLU8, nullptr, nullptr)) return MOE_EWORKSPACE;
  MOE_TRY(check_device());
  Work w;
  carve(*cfg, S, W_SWIGLU8, (char *)ws, &w);
  const ExpertSet es = to_set(*wts, *cfg);
  SwigluB32Args a{};
  a.xq = xq;
  a.sxb = sxb;
  a.S = S;
  a.D = cfg->D;
  a.I = cfg->I;
  a.G = es.gate.q4 + (int64_t)expert * es.gate.q4_stride;
  a.U = es.up.q4 + (int64_t)expert * es.up.q4_stride;
  a.Dn = es.down.q4 + (int64_t)expert * es.down.q4_stride;
  a.gs = es.gate.scale + (int64_t)expert * es.gate.s_stride;
  a.us = es.up.scale + (int64_t)expert * es.up.s_stride;
  a.ds = es.down.scale + (int64_t)expert * es.down.s_stride;
  a.h = w.h;
  a.hq_out = hq;
  a.shb_out = shb;
  a.y = y;
  MOE_TRY_HIP(launch_swiglu_b32_gateup(a, stream));
  MOE_TRY_HIP(launch_swiglu_b32_down(a, stream));
  return MOE_OK;
}

int moe_quant_act_i8(const void *x, int dtype, int S, int D, int8_t *xq, float *sx,
                     hipStream_t stream) {
  if (!x || !xq || !sx) return MOE_EINVAL;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_EINVAL;
  if (S < 1 || D < 8 || (D & 7)) return MOE_ESHAPE;
  if (!aligned16(x) || ((uintptr_t)xq & 7u) || ((uintptr_t)sx & 3u)) return MOE_EALIGN;
  MOE_TRY(check_device());
  QuantArgs a{};
  a.xf = dtype == MOE_F32 ? (const float *)x : nullptr;
  a.xb = dtype == MOE_BF16 ? (const uint16_t *)x : nullptr;
  a.D = D;
  a.xq_nat = xq;
  a.sx = sx;
  return hip_rc(launch_quant(a, S, stream));
}

int moe_router_topk(const moe_config *cfg, const float *x, int S, const float *router_w,
                    const float *router_b, int32_t *topk_idx, float *topk_w, float *logits,
                    void *ws, size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  if (S < 1 || !x || !router_w || !router_b || !topk_idx || !topk_w || !ws) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(router_w) || ((uintptr_t)ws & 255u)) return MOE_EALIGN;
  if (ws_bytes < carve(*cfg, S, W_ROUTER, nullptr, nullptr)) return MOE_EWORKSPACE;
  MOE_TRY(check_device());
  Work w;
  carve(*cfg, S, W_ROUTER, (char *)ws, &w);
  MOE_TRY(run_router(*cfg, x, S, router_w, router_b, w, false, true, logits, stream));
  const size_t n = (size_t)S * cfg->K * 4;
  MOE_TRY_HIP(hipMemcpyAsync(topk_idx, w.idx, n, hipMemcpyDeviceToDevice, stream));
  MOE_TRY_HIP(hipMemcpyAsync(topk_w, w.w, n, hipMemcpyDeviceToDevice, stream));
  return MOE_OK;
}

int moe_expert_swiglu_i4(const moe_config *cfg, const int8_t *xq, const float *sx, int S,
                         const moe_experts *wts, int expert, float *y, int32_t *acc_gu,
                         int8_t *hq, float *sh, int32_t *acc_d, void *ws, size_t ws_bytes,
                         hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  if (S < 1 || !xq || !sx || !wts || !y || !ws) return MOE_EINVAL;
  if (expert < 0 || expert >= cfg->E) return MOE_EINVAL;
  MOE_TRY(check_experts(*wts));
  if (((uintptr_t)xq & 7u) || ((uintptr_t)ws & 255u)) return MOE_EALIGN;
  if (hq && ((uintptr_t)hq & 7u)) return MOE_EALIGN;
  if (ws_bytes < carve(*cfg, S, W_SWIGLU, nullptr, nullptr)) return MOE_EWORKSPACE;
  MOE_TRY(check_device());
  Work w;
  carve(*cfg, S, W_SWIGLU, (char *)ws, &w);
  // 16-byte aligned code rows are read as they are by the gate/up blocks
  // (each reorders and sums its row); others are first copied in the
  // permuted layout with their sums
  const bool natural = aligned16(xq) && cfg->D % 16 == 0;
  if (!natural) {
    PrepArgs pa{xq, cfg->D, w.xq, w.sumx, nullptr, 1};
    MOE_TRY_HIP(launch_prep_xq(pa, S, stream));
  }
  const DecodeShape ds = decode_shape(*cfg);
  DecodeArgs d{};
  d.S = S;
  d.D = cfg->D;
  d.I = cfg->I;
  d.E = cfg->E;
  d.K = 0;
  d.P = 1;
  d.scale = cfg->routed_scale;
  d.rt = to_set(*wts, *cfg);
  d.fx = d.rt;
  d.fx_index = expert;
  d.fx_slot = 0;
  d.xq = natural ? xq : w.xq;
  d.xq_natural = natural ? 1 : 0;
  d.sx = sx;
  d.sumx = w.sumx;
  d.h = w.h;
  d.ysh = y;
  d.n_router = 0;
  d.n_quant = 0;
  d.n_gu_fx = ds.gu_one;
  d.n_gu_rt = 0;
  d.n_dn_fx = ds.dn_one;
  d.acc_gu = acc_gu;
  d.acc_d = acc_d;
  d.hq_nat = hq;
  d.sh_out = sh;
  MOE_TRY_HIP(launch_decode_a(d, false, stream));
  MOE_TRY_HIP(launch_decode_b(d, stream));
  return MOE_OK;
}

}  // extern "C"

namespace {

// The per-token path; with given_idx / given_w the caller's routing replaces
// the router and the selection (phase A then has no router workgroups).  With
// shared8 the shared expert is that int8 expert (checked by the caller, and
// the shape by shared8_fused_ok), run inside phases A and B like the int4 one.
int layer_forward_impl(const moe_config *cfg, const moe_layer *layer, const float *x, int S,
                       const int32_t *given_idx, const float *given_w, float *out,
                       unsigned flags, const moe_probe *probe, void *ws, size_t ws_bytes,
                       hipStream_t stream, const moe_experts_i8 *shared8 = nullptr) {
  const bool given = given_idx != nullptr;
  if (given && !given_w) return MOE_EINVAL;
  if (given && (((uintptr_t)given_idx & 3u) || ((uintptr_t)given_w & 3u))) return MOE_EALIGN;
  if (shared8 && cfg->n_shared != 1) return MOE_ESHAPE;
  MOE_TRY(layer_common_checks(cfg, layer, x, S, out, flags, ws, ws_bytes, W_FWD, !given,
                              shared8 == nullptr));
  const moe_config &c = *cfg;
  Work w;
  carve(c, S, W_FWD, (char *)ws, &w);
  const DecodeShape ds = decode_shape(c);
  DecodeArgs d{};
  d.S = S;
  d.D = c.D;
  d.I = c.I;
  d.E = c.E;
  d.K = c.K;
  d.P = c.K + c.n_shared;
  d.scale = c.routed_scale;
  d.x = x;
  d.W = layer->router_w;
  d.bias = layer->router_b;
  d.rt = to_set(layer->routed, c);
  d.fx = (c.n_shared && !shared8) ? to_set(layer->shared, c) : d.rt;
  d.fx_index = 0;
  d.fx_slot = c.K;
  if (shared8) {
    const int8_t *q;
    const float *sc;
    d.fx8 = 1;
    q8_rows(shared8->gate, c.I, c.D, 0, &q, &sc);
    d.f8g = RowPtr{reinterpret_cast<const uint8_t *>(q), sc};
    q8_rows(shared8->up, c.I, c.D, 0, &q, &sc);
    d.f8u = RowPtr{reinterpret_cast<const uint8_t *>(q), sc};
    q8_rows(shared8->down, c.D, c.I, 0, &q, &sc);
    d.f8d = RowPtr{reinterpret_cast<const uint8_t *>(q), sc};
  }
  d.xq = w.xq;
  d.sx = w.sx;
  d.sumx = w.sumx;
  d.logits = w.logits;
  d.idx = given ? const_cast<int32_t *>(given_idx) : w.idx;
  d.w = given ? const_cast<float *>(given_w) : w.w;
  d.given = given ? 1 : 0;
  d.topp = given ? 0.f : c.expert_topp;
  d.keff = given ? nullptr : w.keff;
  d.h = w.h;
  d.ysh = w.ysh;
  d.tmp = w.tmp;
  d.n_router = given ? 0 : (c.E + kARouterWaves - 1) / kARouterWaves;
  d.n_quant = 1;
  d.n_gu_fx = c.n_shared ? (shared8 ? ds.gu_fx8 : ds.gu_fx) : 0;
  d.n_gu_rt = ds.gu_rt;
  d.n_dn_fx = c.n_shared ? (shared8 ? ds.dn_fx8 : ds.dn_fx) : 0;
  d.n_dn = ds.dn;
  d.out = out;
  d.flags = flags & MOE_F_ACCUMULATE;
  if (flags & MOE_F_PRENORM) {
    d.gamma = layer->norm_gamma;
    d.eps = layer->norm_eps;
  }
  MOE_TRY_HIP(launch_decode_a(d, true, stream));
  const bool tgu = probe && probe->ev_gateup[0] && probe->ev_gateup[1];
  const bool tdn = probe && probe->ev_down[0] && probe->ev_down[1];
  MOE_TRY_HIP(launch_decode_b(d, stream, tgu ? probe->ev_gateup[0] : nullptr,
                              tgu ? probe->ev_gateup[1] : nullptr));
  if (!given) MOE_TRY(copy_probe(c, S, probe, w, stream));
  const int batch = decode_c_slots(c.I);
  for (int p0 = 0; p0 < c.K; p0 += batch) {
    d.p_lo = p0;
    d.p_hi = std::min(c.K, p0 + batch);
    d.c_first = (p0 == 0);
    d.c_last = (d.p_hi == c.K);
    MOE_TRY_HIP(launch_decode_c(d, stream, (tdn && d.c_first) ? probe->ev_down[0] : nullptr,
                                (tdn && d.c_last) ? probe->ev_down[1] : nullptr));
  }
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_layer_forward(const moe_config *cfg, const moe_layer *layer, const float *x, int S,
                      float *out, unsigned flags, const moe_probe *probe, void *ws,
                      size_t ws_bytes, hipStream_t stream) {
  return layer_forward_impl(cfg, layer, x, S, nullptr, nullptr, out, flags, probe, ws, ws_bytes,
                            stream);
}

int moe_layer_forward_routed(const moe_config *cfg, const moe_layer *layer, const float *x, int S,
                             const int32_t *topk_idx, const float *topk_w, float *out,
                             unsigned flags, void *ws, size_t ws_bytes, hipStream_t stream) {
  if (!topk_idx) return MOE_EINVAL;
  return layer_forward_impl(cfg, layer, x, S, topk_idx, topk_w, out, flags, nullptr, ws,
                            ws_bytes, stream);
}

}  // extern "C"

// ---- moe_layer_forward_noalloc: the per-token path on a library-held scratch ----
//
// One file-scope device array per GPU serves as the workspace.  In host code
// `noalloc_scratch` names a host-side stand-in, not device memory: its device
// address is looked up once per device with hipGetSymbolAddress (with that
// device current) and only that address is ever passed to a kernel.  No
// kernel of the per-token path needs the workspace to start at zero, so the
// array is never cleared.
static __device__ __align__(256) unsigned char noalloc_scratch[MOE_NOALLOC_WS_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void *> g_noalloc_ptr[kMaxDevices];
std::mutex g_noalloc_mu;

int noalloc_ptr(void **p) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_EDEVICE;
  void *v = g_noalloc_ptr[dev].load(std::memory_order_acquire);
  if (!v) {
    std::lock_guard<std::mutex> lk(g_noalloc_mu);
    v = g_noalloc_ptr[dev].load(std::memory_order_relaxed);
    if (!v) {
      if (hipGetSymbolAddress(&v, HIP_SYMBOL(noalloc_scratch)) != hipSuccess || !v) return MOE_EHIP;
      g_noalloc_ptr[dev].store(v, std::memory_order_release);
    }
  }
  *p = v;
  return MOE_OK;
}

}  // namespace

extern "C" int moe_layer_forward_noalloc(const moe_config *cfg, const moe_layer *layer,
                                         const float *x, int S, float *out, unsigned flags,
                                         hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  if (S < 1) return MOE_EINVAL;
  if (carve(*cfg, S, W_FWD, nullptr, nullptr) > (size_t)MOE_NOALLOC_WS_BYTES) return MOE_EWORKSPACE;
  MOE_TRY(check_device());
  void *ws = nullptr;
  MOE_TRY(noalloc_ptr(&ws));
  return layer_forward_impl(cfg, layer, x, S, nullptr, nullptr, out, flags, nullptr, ws,
                            (size_t)MOE_NOALLOC_WS_BYTES, stream);
}

namespace {

// The int8 shared expert of the union path on all S tokens (int8 matrix
// cores): its gate/up (mode 0: codes xq in the permuted layout, h into slot K
// of every token's hidden rows) or its down (mode 1: the requantized slot K
// of the hidden rows, y into slot K of the staging rows).
int shared8_rows(const moe_config &c, const moe_experts_i8 &e, const Work &w, int S, int mode,
                 hipStream_t st) {
  const int P = c.K + 1;
  Shared8MfmaArgs a{};
  a.S = S;
  if (mode == 0) {
    a.act = w.xq;
    a.act_stride = c.D;
    a.ascale = w.sx;
    a.ascale_stride = 1;
    q8_rows(e.gate, c.I, c.D, 0, &a.W0, &a.ws0);
    q8_rows(e.up, c.I, c.D, 0, &a.W1, &a.ws1);
    a.O = c.I;
    a.C = c.D;
    a.out = w.h + (size_t)c.K * c.I;
    a.out_stride = (int64_t)P * c.I;
  } else {
    a.act = w.hq + (size_t)c.K * c.I;
    a.act_stride = (int64_t)P * c.I;
    a.ascale = w.sh + c.K;
    a.ascale_stride = P;
    q8_rows(e.down, c.D, c.I, 0, &a.W0, &a.ws0);
    a.O = c.D;
    a.C = c.I;
    a.out = w.stage + (size_t)c.K * c.D;
    a.out_stride = (int64_t)P * c.D;
  }
  return hip_rc(launch_shared8_mfma(a, mode, st));
}

// The union path; with given_idx / given_w the caller's routing replaces the
// router and the selection (the tokens are only quantized).  With shared8 the
// shared expert is that int8 expert (checked by the caller): the routed
// experts are grouped without a shared group, and the int8 expert runs on all
// tokens into the shared slot of the hidden and staging rows.
int layer_forward_batch_impl(const moe_config *cfg, const moe_layer *layer, const float *x, int S,
                             const int32_t *given_idx, const float *given_w, float *out,
                             unsigned flags, const moe_probe *probe, void *ws, size_t ws_bytes,
                             hipStream_t stream, const moe_experts_i8 *shared8 = nullptr) {
  const bool given = given_idx != nullptr;
  if (given && !given_w) return MOE_EINVAL;
  if (given && (((uintptr_t)given_idx & 3u) || ((uintptr_t)given_w & 3u))) return MOE_EALIGN;
  if (shared8 && cfg->n_shared != 1) return MOE_ESHAPE;
  MOE_TRY(layer_common_checks(cfg, layer, x, S, out, flags, ws, ws_bytes, W_BATCH, !given,
                              shared8 == nullptr));
  const moe_config &c = *cfg;
  const int P = c.K + c.n_shared;
  Work w;
  carve(c, S, W_BATCH, (char *)ws, &w);
  // x (maybe out itself) is read by the router launch and nowhere else.
  // With MOE_F_PRENORM, batches of up to 8 tokens normalize inside the
  // router's workgroups; larger ones (and calls with given routing) get the
  // normalized rows in the workspace first.
  const float *gamma = nullptr;
  if (flags & MOE_F_PRENORM) {
    if (S <= 8 && !given) {
      gamma = layer->norm_gamma;
    } else {
      RmsArgs ra{x, layer->norm_gamma, c.D, layer->norm_eps, w.xn, 1};
      MOE_TRY_HIP(launch_rmsnorm(ra, S, stream));
      x = w.xn;
    }
    flags &= ~MOE_F_PRENORM;
  }
  // small batches select inside the grouping kernel (one launch fewer)
  const bool topk_in_group = !given && S <= kGroupTopkMaxTokens && c.E <= 256;
  // bf16 tokens (MOE_F_X_BF16): x holds bf16 bit patterns
  const uint16_t *xbf = (flags & MOE_F_X_BF16) ? reinterpret_cast<const uint16_t *>(x) : nullptr;
  flags &= ~MOE_F_X_BF16;
  if (given) {
    QuantArgs q{xbf ? nullptr : x, xbf, c.D, w.xq, nullptr, w.sx, w.sumx};
    MOE_TRY_HIP(launch_quant(q, S, stream));
  } else {
    MOE_TRY(run_router(c, x, S, layer->router_w, layer->router_b, w, true, !topk_in_group, nullptr,
                       stream, gamma, layer->norm_eps, xbf));
  }
  int32_t *idx = given ? const_cast<int32_t *>(given_idx) : w.idx;
  const float *wts = given ? given_w : w.w;
  // keff is always computed with the selection (the probe reports it); the
  // grouping and the combine consult it only when top-p is on
  const bool topp_on = !given && c.expert_topp > 0.f && c.expert_topp < 1.f;
  int32_t *keff = given ? nullptr : w.keff;
  // the MFMA kernels address activation rows with 32-bit byte offsets
  const bool offs_ok = (int64_t)S * P * std::max(c.D, c.I) < INT32_MAX;
  const bool mfma_gu = grouped_mfma_fits(c.D) && offs_ok, mfma_dn = grouped_mfma_fits(c.I) && offs_ok;
  const int max_tiles = grouped_mfma_max_tiles(S, P, c.E);
  GroupArgs ga{idx,      S,     c.E,     c.K,      P, shared8 ? 0 : c.n_shared, w.gcount, w.goff,
               w.pairs, (mfma_gu || mfma_dn) ? w.tiles : nullptr, w.ntiles,
               grouped_mfma_tile_rows(S)};
  ga.with_topk = topk_in_group ? 1 : 0;
  ga.topp = c.expert_topp;
  ga.keff = keff;
  ga.use_keff = topp_on ? 1 : 0;
  ga.logits = w.logits;
  ga.bias = layer->router_b;
  ga.scale = c.routed_scale;
  ga.wts = w.w;
  MOE_TRY_HIP(launch_group(ga, stream));
  if (!given) MOE_TRY(copy_probe(c, S, probe, w, stream));
  const ExpertSet rt = to_set(layer->routed, c);
  const ExpertSet sh = (c.n_shared && !shared8) ? to_set(layer->shared, c) : rt;
  GroupedMfmaArgs m{};
  m.rt = rt;
  m.sh = sh;
  m.E = c.E;
  m.P = P;
  m.gcount = w.gcount;
  m.goff = w.goff;
  m.pairs = w.pairs;
  m.tiles = w.tiles;
  m.ntiles = w.ntiles;
  GroupedGateUpArgs g{};
  g.rt = rt;
  g.sh = sh;
  g.D = c.D;
  g.I = c.I;
  g.E = c.E;
  g.P = P;
  g.gcount = w.gcount;
  g.goff = w.goff;
  g.pairs = w.pairs;
  g.xq = w.xq;
  g.sx = w.sx;
  g.sumx = w.sumx;
  g.h = w.h;
  MOE_TRY(record(probe, 0, 0, stream));
  if (mfma_gu) {
    GroupedMfmaArgs mg = m;
    mg.C = c.D;
    mg.O = c.I;
    mg.act = w.xq;
    mg.ascale = w.sx;
    mg.asum = w.sumx;
    mg.out = w.h;
    MOE_TRY_HIP(launch_grouped_mfma(mg, 0, max_tiles, S, stream));
  } else {
    MOE_TRY_HIP(launch_grouped_gateup(g, stream));
  }
  if (shared8) MOE_TRY(shared8_rows(c, *shared8, w, S, 0, stream));
  MOE_TRY(record(probe, 0, 1, stream));
  RequantArgs rq{w.h, c.I, w.hq, w.sh, w.sumh};
  MOE_TRY_HIP(launch_requant(rq, S * P, stream));
  GroupedDownArgs d{};
  d.rt = rt;
  d.sh = sh;
  d.D = c.D;
  d.I = c.I;
  d.E = c.E;
  d.P = P;
  d.gcount = w.gcount;
  d.goff = w.goff;
  d.pairs = w.pairs;
  d.hq = w.hq;
  d.sh_scale = w.sh;
  d.sumh = w.sumh;
  d.stage = w.stage;
  MOE_TRY(record(probe, 1, 0, stream));
  if (mfma_dn) {
    GroupedMfmaArgs md = m;
    md.C = c.I;
    md.O = c.D;
    md.act = w.hq;
    md.ascale = w.sh;
    md.asum = w.sumh;
    md.out = w.stage;
    MOE_TRY_HIP(launch_grouped_mfma(md, 1, max_tiles, S, stream));
  } else {
    MOE_TRY_HIP(launch_grouped_down(d, stream));
  }
  if (shared8) MOE_TRY(shared8_rows(c, *shared8, w, S, 1, stream));
  MOE_TRY(record(probe, 1, 1, stream));
  CombineArgs cb{w.stage, wts, S, c.D, c.K, P, c.n_shared, out, flags, topp_on ? keff : nullptr};
  MOE_TRY_HIP(launch_combine(cb, stream));
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_layer_forward_batch(const moe_config *cfg, const moe_layer *layer, const float *x, int S,
                            float *out, unsigned flags, const moe_probe *probe, void *ws,
                            size_t ws_bytes, hipStream_t stream) {
  return layer_forward_batch_impl(cfg, layer, x, S, nullptr, nullptr, out, flags, probe, ws,
                                  ws_bytes, stream);
}

int moe_layer_forward_batch_shared_i8(const moe_config *cfg, const moe_layer *layer,
                                      const moe_experts_i8 *shared8, const float *x, int S,
                                      float *out, unsigned flags, void *ws, size_t ws_bytes,
                                      hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  if (cfg->n_shared != 1) return MOE_ESHAPE;
  if (!shared8) return MOE_EINVAL;
  if (flags & ~MOE_F_ACCUMULATE) return MOE_EINVAL;
  MOE_TRY(check_experts_i8(*shared8));
  return layer_forward_batch_impl(cfg, layer, x, S, nullptr, nullptr, out, flags, nullptr, ws,
                                  ws_bytes, stream, shared8);
}

int moe_layer_forward_batch_routed(const moe_config *cfg, const moe_layer *layer, const float *x,
                                   int S, const int32_t *topk_idx, const float *topk_w, float *out,
                                   unsigned flags, void *ws, size_t ws_bytes, hipStream_t stream) {
  if (!topk_idx) return MOE_EINVAL;
  return layer_forward_batch_impl(cfg, layer, x, S, topk_idx, topk_w, out, flags, nullptr, ws,
                                  ws_bytes, stream);
}

int moe_tier_forward(moe_tier *t, int layer_index, const moe_config *cfg, const moe_layer *layer,
                     const void *host_slabs, void *hbm_slots, size_t slab_bytes, const float *x,
                     int S, float *out, unsigned flags, int union_path, int32_t *host_idx,
                     int32_t *misses, void *ws_router, size_t ws_router_bytes, void *ws,
                     size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  const moe_config &c = *cfg;
  if (!t || !layer || !host_slabs || !hbm_slots || !x || !out || !host_idx || !ws_router || !ws ||
      S < 1)
    return MOE_EINVAL;
  if (flags & ~MOE_F_ACCUMULATE) return MOE_EINVAL;
  if (!layer->router_w || !layer->router_b) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(layer->router_w) || ((uintptr_t)ws_router & 255u))
    return MOE_EALIGN;
  if (ws_router_bytes < carve(c, S, W_ROUTER, nullptr, nullptr)) return MOE_EWORKSPACE;
  if (ws_bytes < carve(c, S, union_path ? W_BATCH : W_FWD, nullptr, nullptr)) return MOE_EWORKSPACE;
  // the slabs must hold this shape's layout, and every slot number must be a
  // valid expert index of the slot stack (the block clamps indices into
  // [0, E)); the router's experts must be experts of the tier
  moe_slab_layout lay;
  MOE_TRY(moe_slab_layout_of(cfg, &lay));
  if (slab_bytes == 0 || (slab_bytes & 15u)) return MOE_EALIGN;
  if (slab_bytes < (size_t)lay.bytes) return MOE_ESHAPE;
  int t_experts = 0, t_slots = 0;
  tier_sizes(t, &t_experts, &t_slots);
  if (t_slots > c.E || t_experts < c.E) return MOE_ESHAPE;
  if (layer_index < 0) return MOE_EINVAL;
  MOE_TRY(check_device());
  // 1. selection on the device (all K experts; top-p does not apply here)
  Work wr;
  carve(c, S, W_ROUTER, (char *)ws_router, &wr);
  MOE_TRY(run_router(c, x, S, layer->router_w, layer->router_b, wr, false, true, nullptr, stream));
  const size_t n = (size_t)S * c.K;
  MOE_TRY_HIP(hipMemcpyAsync(host_idx, wr.idx, n * 4, hipMemcpyDeviceToHost, stream));
  MOE_TRY_HIP(hipStreamSynchronize(stream));
  // 2. the call's experts in order of first appearance, mapped to slots
  std::vector<int32_t> eids, pos(n);
  eids.reserve(n);
  for (size_t i = 0; i < n; i++) {
    const int32_t e = host_idx[i];
    size_t u = 0;
    while (u < eids.size() && eids[u] != e) u++;
    if (u == eids.size()) eids.push_back(e);
    pos[i] = (int32_t)u;
  }
  std::vector<int32_t> slots(eids.size()), loads(eids.size());
  const int nm = moe_tier_map(t, layer_index, eids.data(), (int)eids.size(), slots.data(),
                              loads.data());
  if (nm < 0) return nm;
  if (misses) *misses = nm;
  // 3. the missing slabs, then the routing as slot numbers, both in stream order
  const int frc = moe_tier_fetch(host_slabs, hbm_slots, slab_bytes, eids.data(), slots.data(),
                                 loads.data(), (int)eids.size(), stream);
  if (frc != MOE_OK) {
    tier_unmap_loads(t, layer_index, eids.data(), slots.data(), loads.data(), (int)eids.size());
    return frc;
  }
  for (size_t i = 0; i < n; i++) host_idx[i] = slots[pos[i]];
  MOE_TRY_HIP(hipMemcpyAsync(wr.idx, host_idx, n * 4, hipMemcpyHostToDevice, stream));
  // 4. the block on the slot stack
  return union_path ? layer_forward_batch_impl(cfg, layer, x, S, wr.idx, wr.w, out, flags, nullptr,
                                               ws, ws_bytes, stream)
                    : layer_forward_impl(cfg, layer, x, S, wr.idx, wr.w, out, flags, nullptr, ws,
                                         ws_bytes, stream);
}

int moe_rmsnorm(const float *x, const float *gamma, int S, int D, float eps, float *y,
                hipStream_t stream) {
  if (!x || !gamma || !y) return MOE_EINVAL;
  if (S < 1 || D < 1) return MOE_ESHAPE;
  if (((uintptr_t)x & 3u) || ((uintptr_t)gamma & 3u) || ((uintptr_t)y & 3u)) return MOE_EALIGN;
  MOE_TRY(check_device());
  const int vec = (D % 4 == 0 && D <= 8192 && aligned16(x) && aligned16(gamma) && aligned16(y));
  RmsArgs a{x, gamma, D, eps, y, vec};
  return hip_rc(launch_rmsnorm(a, S, stream));
}

int moe_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream) {
  if (!buf || !sink) return MOE_EINVAL;
  if (bytes == 0 || bytes % 16) return MOE_ESHAPE;
  if (!aligned16(buf) || ((uintptr_t)sink & 3u)) return MOE_EALIGN;
  MOE_TRY(check_device());
  return hip_rc(launch_stream_read(buf, bytes, sink, stream));
}

int moe_stream_read_sink_words(void) { return stream_read_sink_words(); }

}  // extern "C"

extern "C" {

int moe_layer_forward_shared_i8(const moe_config *cfg, const moe_layer *layer,
                                const moe_experts_i8 *shared8, const float *x, int S, float *out,
                                unsigned flags, void *ws, size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  if (cfg->n_shared != 1) return MOE_ESHAPE;
  if (!shared8) return MOE_EINVAL;
  if (flags & ~MOE_F_ACCUMULATE) return MOE_EINVAL;
  MOE_TRY(check_experts_i8(*shared8));
  // shapes outside the fused kernels' instantiations take the union path's
  // launches, which return the per-token path's bits
  if (shared8_fused_ok(*cfg))
    return layer_forward_impl(cfg, layer, x, S, nullptr, nullptr, out, flags, nullptr, ws,
                              ws_bytes, stream, shared8);
  return layer_forward_batch_impl(cfg, layer, x, S, nullptr, nullptr, out, flags, nullptr, ws,
                                  ws_bytes, stream, shared8);
}

}  // extern "C"
