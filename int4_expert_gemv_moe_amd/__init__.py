"""Python binding of libmoe_i4.so, the gfx950 routed-expert int4 MoE block.

Argument marshalling only: every function here checks Python-side types,
passes device pointers of torch tensors and the current HIP stream to the
C ABI declared in include/moe_i4.h, and raises on a non-zero status.  All
arithmetic runs in the library's HIP kernels.  There is no fallback: if the
library is missing or the device is not a gfx950 the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_I4_LIB may name another build of the same library (e.g. a tuning variant).
LIB_PATH = os.environ.get("MOE_I4_LIB") or os.path.join(HERE, "libmoe_i4.so")

MOE_F32, MOE_BF16 = 0, 1
F_ACCUMULATE = 1
F_PRENORM = 2
F_X_BF16 = 4
WS_FORWARD, WS_BATCH, WS_SWIGLU, WS_ROUTER, WS_SWIGLU8, WS_SHARED8 = 0, 1, 2, 3, 4, 5

_lib = None


class Config(ctypes.Structure):
    _fields_ = [("D", ctypes.c_int32), ("I", ctypes.c_int32), ("E", ctypes.c_int32),
                ("K", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("routed_scale", ctypes.c_float), ("expert_topp", ctypes.c_float)]


class QMat(ctypes.Structure):
    _fields_ = [("q4", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("q4_stride", ctypes.c_int64), ("scale_stride", ctypes.c_int64)]


class Experts(ctypes.Structure):
    _fields_ = [("gate", QMat), ("up", QMat), ("down", QMat)]


class LayerC(ctypes.Structure):
    _fields_ = [("router_w", ctypes.c_void_p), ("router_b", ctypes.c_void_p),
                ("routed", Experts), ("shared", Experts),
                ("norm_gamma", ctypes.c_void_p), ("norm_eps", ctypes.c_float)]


class Probe(ctypes.Structure):
    _fields_ = [("topk_idx", ctypes.c_void_p), ("topk_w", ctypes.c_void_p),
                ("ev_gateup", ctypes.c_void_p * 2), ("ev_down", ctypes.c_void_p * 2),
                ("keff", ctypes.c_void_p)]


class MoeError(RuntimeError):
    pass


def lib():
    """Load libmoe_i4.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MoeError(f"{LIB_PATH} is not built; run int4_expert_gemv_moe_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz, f32, u32 = (ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float,
                                 ctypes.c_uint)
        L.moe_status_str.argtypes = [i32]
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_workspace_bytes.argtypes = [vp, i32, i32]
        L.moe_workspace_bytes.restype = sz
        L.moe_workspace_init.argtypes = [vp, sz, vp]
        L.moe_pack_int4.argtypes = [vp, i32, i32, vp, vp, vp]
        L.moe_quant_act_i8.argtypes = [vp, i32, i32, i32, vp, vp, vp]
        L.moe_router_topk.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_expert_swiglu_i4.argtypes = [vp, vp, vp, i32, vp, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_quantize_rows_i8.argtypes = [vp, i32, i32, vp, vp, vp]
        L.moe_expert_swiglu_i8.argtypes = [vp, vp, vp, i32, vp, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_pack_int2.argtypes = [vp, i32, i32, vp, vp, vp]
        L.moe_quant_act_b32.argtypes = [vp, i32, i32, vp, vp, vp]
        L.moe_mla_workspace_bytes.argtypes = [vp, i32, i32]
        L.moe_mla_workspace_bytes.restype = sz
        L.moe_mla_decode.argtypes = [vp, vp, i32, vp, vp, vp, i32, vp, vp, sz, vp]
        L.moe_layer_forward_shared_i8.argtypes = [vp, vp, vp, vp, i32, vp, u32, vp, sz, vp]
        L.moe_layer_forward_batch_shared_i8.argtypes = [vp, vp, vp, vp, i32, vp, u32, vp, sz, vp]
        L.moe_expert_swiglu_i4_b32.argtypes = [vp, vp, vp, i32, vp, i32, vp, vp, vp, vp, sz, vp]
        L.moe_expert_swiglu_i2.argtypes = [vp, vp, vp, i32, vp, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_layer_forward.argtypes = [vp, vp, vp, i32, vp, u32, vp, vp, sz, vp]
        L.moe_layer_forward_batch.argtypes = [vp, vp, vp, i32, vp, u32, vp, vp, sz, vp]
        L.moe_layer_forward_noalloc.argtypes = [vp, vp, vp, i32, vp, u32, vp]
        L.moe_rmsnorm.argtypes = [vp, vp, i32, i32, f32, vp, vp]
        L.moe_stream_read.argtypes = [vp, sz, vp, vp]
        L.moe_layer_forward_routed.argtypes = [vp, vp, vp, i32, vp, vp, vp, u32, vp, sz, vp]
        L.moe_layer_forward_batch_routed.argtypes = [vp, vp, vp, i32, vp, vp, vp, u32, vp, sz, vp]
        L.moe_slab_layout_of.argtypes = [vp, vp]
        L.moe_tier_create.argtypes = [i32, i32, i32]
        L.moe_tier_create.restype = vp
        L.moe_tier_create_pinned.argtypes = [i32, i32, i32, i32]
        L.moe_tier_create_pinned.restype = vp
        L.moe_tier_rebalance.argtypes = [vp, i32, vp, vp, vp]
        L.moe_tier_forward.argtypes = [vp, i32, vp, vp, vp, vp, sz, vp, i32, vp, u32, i32, vp, vp,
                                       vp, sz, vp, sz, vp]
        L.moe_tier_destroy.argtypes = [vp]
        L.moe_tier_destroy.restype = None
        L.moe_tier_map.argtypes = [vp, i32, vp, i32, vp, vp]
        L.moe_tier_stats.argtypes = [vp, vp, vp]
        L.moe_tier_fetch.argtypes = [vp, vp, sz, vp, vp, vp, i32, vp]
        L.moe_tier_pick_swap.argtypes = [vp, i32, vp, i32, vp, vp, vp]
        L.moe_tier_lfru_score.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32]
        L.moe_tier_lfru_score.restype = ctypes.c_uint64
        L.moe_stream_read_sink_words.argtypes = []
        for name in ("moe_workspace_init", "moe_pack_int4", "moe_quant_act_i8", "moe_router_topk",
                     "moe_expert_swiglu_i4", "moe_quantize_rows_i8", "moe_expert_swiglu_i8",
                     "moe_pack_int2", "moe_expert_swiglu_i2", "moe_quant_act_b32",
                     "moe_expert_swiglu_i4_b32", "moe_mla_decode", "moe_layer_forward_shared_i8",
                     "moe_layer_forward_batch_shared_i8",
                     "moe_layer_forward", "moe_layer_forward_batch", "moe_layer_forward_noalloc",
                     "moe_rmsnorm", "moe_stream_read", "moe_stream_read_sink_words",
                     "moe_layer_forward_routed", "moe_layer_forward_batch_routed",
                     "moe_slab_layout_of", "moe_tier_map",
                     "moe_tier_stats", "moe_tier_fetch", "moe_tier_pick_swap",
                     "moe_tier_rebalance", "moe_tier_forward"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def status_str(rc: int) -> str:
    return lib().moe_status_str(rc).decode()


def _check(rc: int, name: str) -> None:
    if rc != 0:
        raise MoeError(f"{name}: {status_str(rc)} ({rc})")


def _stream(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, dtype, name: str):
    if not t.is_cuda:
        raise MoeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise MoeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise MoeError(f"{name} must be contiguous")
    return t


def config(D: int, I: int, E: int, K: int, n_shared: int = 1, routed_scale: float = 2.5,
           expert_topp: float = 0.0) -> Config:
    return Config(D, I, E, K, n_shared, routed_scale, expert_topp)


# ---- device weights -----------------------------------------------------------

@dataclass
class DeviceExperts:
    """Stacked int4 experts on the device: gate/up q4 [n][I][D/2], scales
    [n][I]; down q4 [n][D][I/2], scales [n][D]."""
    gate_q4: torch.Tensor
    gate_s: torch.Tensor
    up_q4: torch.Tensor
    up_s: torch.Tensor
    down_q4: torch.Tensor
    down_s: torch.Tensor

    @staticmethod
    def empty(n: int, D: int, I: int, device="cuda") -> "DeviceExperts":
        u8, f32 = torch.uint8, torch.float32
        return DeviceExperts(torch.empty(n, I, D // 2, dtype=u8, device=device),
                             torch.empty(n, I, dtype=f32, device=device),
                             torch.empty(n, I, D // 2, dtype=u8, device=device),
                             torch.empty(n, I, dtype=f32, device=device),
                             torch.empty(n, D, I // 2, dtype=u8, device=device),
                             torch.empty(n, D, dtype=f32, device=device))

    def cstruct(self) -> Experts:
        def q(a, b):
            return QMat(a.data_ptr(), b.data_ptr(), 0, 0)
        return Experts(q(self.gate_q4, self.gate_s), q(self.up_q4, self.up_s),
                       q(self.down_q4, self.down_s))

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in
                   (self.gate_q4, self.gate_s, self.up_q4, self.up_s, self.down_q4, self.down_s))


class Q8Mat(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("q_stride", ctypes.c_int64),
                ("scale_stride", ctypes.c_int64)]


class ExpertsI8(ctypes.Structure):
    _fields_ = [("gate", Q8Mat), ("up", Q8Mat), ("down", Q8Mat)]


@dataclass
class DeviceExpertsI8:
    """Stacked experts in the int8 format on the device: gate/up codes
    [n][I][D], scales [n][I]; down codes [n][D][I], scales [n][D]."""
    gate_q: torch.Tensor
    gate_s: torch.Tensor
    up_q: torch.Tensor
    up_s: torch.Tensor
    down_q: torch.Tensor
    down_s: torch.Tensor

    @staticmethod
    def empty(n: int, D: int, I: int, device="cuda") -> "DeviceExpertsI8":
        i8, f32 = torch.int8, torch.float32
        return DeviceExpertsI8(torch.empty(n, I, D, dtype=i8, device=device),
                               torch.empty(n, I, dtype=f32, device=device),
                               torch.empty(n, I, D, dtype=i8, device=device),
                               torch.empty(n, I, dtype=f32, device=device),
                               torch.empty(n, D, I, dtype=i8, device=device),
                               torch.empty(n, D, dtype=f32, device=device))

    def cstruct(self) -> ExpertsI8:
        def q(a, b):
            return Q8Mat(a.data_ptr(), b.data_ptr(), 0, 0)
        return ExpertsI8(q(self.gate_q, self.gate_s), q(self.up_q, self.up_s),
                         q(self.down_q, self.down_s))

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in
                   (self.gate_q, self.gate_s, self.up_q, self.up_s, self.down_q, self.down_s))


@dataclass
class DeviceLayer:
    cfg: Config
    router_w: torch.Tensor  # [E][D] float32
    router_b: torch.Tensor  # [E] float32
    routed: DeviceExperts   # E experts
    shared: DeviceExperts | None  # 1 expert when cfg.n_shared == 1

    def cstruct(self, norm_gamma: torch.Tensor | None = None, norm_eps: float = 0.0) -> LayerC:
        """The C struct; norm_gamma / norm_eps are read by calls with F_PRENORM."""
        sh = self.shared.cstruct() if self.shared is not None else Experts()
        g = None if norm_gamma is None else norm_gamma.data_ptr()
        return LayerC(self.router_w.data_ptr(), self.router_b.data_ptr(), self.routed.cstruct(), sh,
                      g, float(norm_eps))


class Workspace:
    """Device scratch for the calls; zero-filled once on creation."""

    def __init__(self, cfg: Config, S: int, which: int, device="cuda"):
        n = lib().moe_workspace_bytes(ctypes.byref(cfg), S, which)
        if n == 0:
            raise MoeError("moe_workspace_bytes rejected the configuration")
        self.nbytes = int(n)
        self.buf = torch.empty(self.nbytes + 256, dtype=torch.uint8, device=device)
        off = (-self.buf.data_ptr()) % 256
        self.view = self.buf[off: off + self.nbytes]
        _check(lib().moe_workspace_init(ctypes.c_void_p(self.view.data_ptr()), self.nbytes,
                                        ctypes.c_void_p(_stream())), "moe_workspace_init")

    @property
    def ptr(self):
        return ctypes.c_void_p(self.view.data_ptr())


# ---- entry points ------------------------------------------------------------

def moe_pack_int4(w: torch.Tensor, q4: torch.Tensor | None = None, scale: torch.Tensor | None = None,
                  stream=None):
    """Section 06 converter on the device: w [O][C] float32 -> (q4 [O][C/2], scale [O])."""
    _dev(w, torch.float32, "w")
    O, C = w.shape
    q4 = torch.empty(O, C // 2, dtype=torch.uint8, device=w.device) if q4 is None else q4
    scale = torch.empty(O, dtype=torch.float32, device=w.device) if scale is None else scale
    _check(lib().moe_pack_int4(_ptr(w), O, C, _ptr(q4), _ptr(scale), ctypes.c_void_p(_stream(stream))),
           "moe_pack_int4")
    return q4, scale


def moe_quant_act_i8(x: torch.Tensor, stream=None):
    """Per-row int8 quantization of x [S][D] (float32 or bfloat16)."""
    if x.dtype == torch.float32:
        dt = MOE_F32
    elif x.dtype == torch.bfloat16:
        dt = MOE_BF16
    else:
        raise MoeError("x must be float32 or bfloat16")
    _dev(x, x.dtype, "x")
    S, D = x.shape
    xq = torch.empty(S, D, dtype=torch.int8, device=x.device)
    sx = torch.empty(S, dtype=torch.float32, device=x.device)
    _check(lib().moe_quant_act_i8(_ptr(x), dt, S, D, _ptr(xq), _ptr(sx),
                                  ctypes.c_void_p(_stream(stream))), "moe_quant_act_i8")
    return xq, sx


def moe_router_topk(cfg: Config, x: torch.Tensor, router_w: torch.Tensor, router_b: torch.Tensor,
                    ws: Workspace, want_logits: bool = False, stream=None):
    _dev(x, torch.float32, "x")
    S = x.shape[0]
    idx = torch.empty(S, cfg.K, dtype=torch.int32, device=x.device)
    w = torch.empty(S, cfg.K, dtype=torch.float32, device=x.device)
    logits = torch.empty(S, cfg.E, dtype=torch.float32, device=x.device) if want_logits else None
    _check(lib().moe_router_topk(ctypes.byref(cfg), _ptr(x), S, _ptr(router_w), _ptr(router_b),
                                 _ptr(idx), _ptr(w), _ptr(logits), ws.ptr, ws.nbytes,
                                 ctypes.c_void_p(_stream(stream))), "moe_router_topk")
    return idx, w, logits


def moe_expert_swiglu_i4(cfg: Config, xq: torch.Tensor, sx: torch.Tensor, experts: DeviceExperts,
                         expert: int, ws: Workspace, probes: bool = False, stream=None):
    _dev(xq, torch.int8, "xq")
    _dev(sx, torch.float32, "sx")
    S = xq.shape[0]
    dev = xq.device
    y = torch.empty(S, cfg.D, dtype=torch.float32, device=dev)
    acc_gu = hq = sh = acc_d = None
    if probes:
        acc_gu = torch.empty(S, 2, cfg.I, dtype=torch.int32, device=dev)
        hq = torch.empty(S, cfg.I, dtype=torch.int8, device=dev)
        sh = torch.empty(S, dtype=torch.float32, device=dev)
        acc_d = torch.empty(S, cfg.D, dtype=torch.int32, device=dev)
    es = experts.cstruct()
    _check(lib().moe_expert_swiglu_i4(ctypes.byref(cfg), _ptr(xq), _ptr(sx), S, ctypes.byref(es),
                                      expert, _ptr(y), _ptr(acc_gu), _ptr(hq), _ptr(sh), _ptr(acc_d),
                                      ws.ptr, ws.nbytes, ctypes.c_void_p(_stream(stream))),
           "moe_expert_swiglu_i4")
    return dict(y=y, acc_gu=acc_gu, hq=hq, sh=sh, acc_d=acc_d)


def moe_quantize_rows_i8(w: torch.Tensor, q: torch.Tensor | None = None,
                         scale: torch.Tensor | None = None, stream=None):
    """Section 05 quantizer on the device: w [O][C] float32 -> (q [O][C] int8, scale [O])."""
    _dev(w, torch.float32, "w")
    O, C = w.shape
    q = torch.empty(O, C, dtype=torch.int8, device=w.device) if q is None else q
    scale = torch.empty(O, dtype=torch.float32, device=w.device) if scale is None else scale
    _check(lib().moe_quantize_rows_i8(_ptr(w), O, C, _ptr(q), _ptr(scale),
                                      ctypes.c_void_p(_stream(stream))), "moe_quantize_rows_i8")
    return q, scale


def moe_expert_swiglu_i8(cfg: Config, xq: torch.Tensor, sx: torch.Tensor, experts: DeviceExpertsI8,
                         expert: int, ws: Workspace, probes: bool = False, stream=None, y=None):
    _dev(xq, torch.int8, "xq")
    _dev(sx, torch.float32, "sx")
    S = xq.shape[0]
    dev = xq.device
    y = torch.empty(S, cfg.D, dtype=torch.float32, device=dev) if y is None else y
    acc_gu = hq = sh = acc_d = None
    if probes:
        acc_gu = torch.empty(S, 2, cfg.I, dtype=torch.int32, device=dev)
        hq = torch.empty(S, cfg.I, dtype=torch.int8, device=dev)
        sh = torch.empty(S, dtype=torch.float32, device=dev)
        acc_d = torch.empty(S, cfg.D, dtype=torch.int32, device=dev)
    es = experts.cstruct()
    _check(lib().moe_expert_swiglu_i8(ctypes.byref(cfg), _ptr(xq), _ptr(sx), S, ctypes.byref(es),
                                      expert, _ptr(y), _ptr(acc_gu), _ptr(hq), _ptr(sh), _ptr(acc_d),
                                      ws.ptr, ws.nbytes, ctypes.c_void_p(_stream(stream))),
           "moe_expert_swiglu_i8")
    return dict(y=y, acc_gu=acc_gu, hq=hq, sh=sh, acc_d=acc_d)


@dataclass
class DeviceExpertsI2:
    """Stacked packed-int2 experts on the device: gate/up [n][I][D/4], scales
    [n][I]; down [n][D][I/4], scales [n][D]."""
    gate_q2: torch.Tensor
    gate_s: torch.Tensor
    up_q2: torch.Tensor
    up_s: torch.Tensor
    down_q2: torch.Tensor
    down_s: torch.Tensor

    @staticmethod
    def empty(n: int, D: int, I: int, device="cuda") -> "DeviceExpertsI2":
        u8, f32 = torch.uint8, torch.float32
        return DeviceExpertsI2(torch.empty(n, I, D // 4, dtype=u8, device=device),
                               torch.empty(n, I, dtype=f32, device=device),
                               torch.empty(n, I, D // 4, dtype=u8, device=device),
                               torch.empty(n, I, dtype=f32, device=device),
                               torch.empty(n, D, I // 4, dtype=u8, device=device),
                               torch.empty(n, D, dtype=f32, device=device))

    def cstruct(self) -> Experts:
        def q(a, b):
            return QMat(a.data_ptr(), b.data_ptr(), 0, 0)
        return Experts(q(self.gate_q2, self.gate_s), q(self.up_q2, self.up_s),
                       q(self.down_q2, self.down_s))


def moe_pack_int2(w: torch.Tensor, q2: torch.Tensor | None = None, scale: torch.Tensor | None = None,
                  stream=None):
    """Packed int2 on the device: w [O][C] float32 -> (q2 [O][(C+3)/4], scale [O])."""
    _dev(w, torch.float32, "w")
    O, C = w.shape
    q2 = torch.empty(O, (C + 3) // 4, dtype=torch.uint8, device=w.device) if q2 is None else q2
    scale = torch.empty(O, dtype=torch.float32, device=w.device) if scale is None else scale
    _check(lib().moe_pack_int2(_ptr(w), O, C, _ptr(q2), _ptr(scale), ctypes.c_void_p(_stream(stream))),
           "moe_pack_int2")
    return q2, scale


def moe_expert_swiglu_i2(cfg: Config, xq: torch.Tensor, sx: torch.Tensor, experts: DeviceExpertsI2,
                         expert: int, ws: Workspace, probes: bool = False, stream=None):
    _dev(xq, torch.int8, "xq")
    _dev(sx, torch.float32, "sx")
    S = xq.shape[0]
    dev = xq.device
    y = torch.empty(S, cfg.D, dtype=torch.float32, device=dev)
    acc_gu = hq = sh = acc_d = None
    if probes:
        acc_gu = torch.empty(S, 2, cfg.I, dtype=torch.int32, device=dev)
        hq = torch.empty(S, cfg.I, dtype=torch.int8, device=dev)
        sh = torch.empty(S, dtype=torch.float32, device=dev)
        acc_d = torch.empty(S, cfg.D, dtype=torch.int32, device=dev)
    es = experts.cstruct()
    _check(lib().moe_expert_swiglu_i2(ctypes.byref(cfg), _ptr(xq), _ptr(sx), S, ctypes.byref(es),
                                      expert, _ptr(y), _ptr(acc_gu), _ptr(hq), _ptr(sh), _ptr(acc_d),
                                      ws.ptr, ws.nbytes, ctypes.c_void_p(_stream(stream))),
           "moe_expert_swiglu_i2")
    return dict(y=y, acc_gu=acc_gu, hq=hq, sh=sh, acc_d=acc_d)


def moe_quant_act_b32(x: torch.Tensor, stream=None):
    """Block-32 activation quantization of x [S][D] float32: (xq [S][D], sxb [S][D/32])."""
    _dev(x, torch.float32, "x")
    S, D = x.shape
    xq = torch.empty(S, D, dtype=torch.int8, device=x.device)
    sxb = torch.empty(S, D // 32, dtype=torch.float32, device=x.device)
    _check(lib().moe_quant_act_b32(_ptr(x), S, D, _ptr(xq), _ptr(sxb),
                                   ctypes.c_void_p(_stream(stream))), "moe_quant_act_b32")
    return xq, sxb


def moe_expert_swiglu_i4_b32(cfg: Config, xq: torch.Tensor, sxb: torch.Tensor,
                             experts: DeviceExperts, expert: int, ws: Workspace, probes: bool = False,
                             stream=None):
    _dev(xq, torch.int8, "xq")
    _dev(sxb, torch.float32, "sxb")
    S = xq.shape[0]
    dev = xq.device
    y = torch.empty(S, cfg.D, dtype=torch.float32, device=dev)
    hq = shb = None
    if probes:
        hq = torch.empty(S, cfg.I, dtype=torch.int8, device=dev)
        shb = torch.empty(S, cfg.I // 32, dtype=torch.float32, device=dev)
    es = experts.cstruct()
    _check(lib().moe_expert_swiglu_i4_b32(ctypes.byref(cfg), _ptr(xq), _ptr(sxb), S,
                                          ctypes.byref(es), expert, _ptr(y), _ptr(hq), _ptr(shb),
                                          ws.ptr, ws.nbytes, ctypes.c_void_p(_stream(stream))),
           "moe_expert_swiglu_i4_b32")
    return dict(y=y, hq=hq, shb=shb)


def moe_layer_forward_shared_i8(layer: DeviceLayer, shared8: DeviceExpertsI8, x: torch.Tensor,
                                ws: Workspace, out=None, flags: int = 0, stream=None,
                                fn_name: str = "moe_layer_forward_shared_i8"):
    """The per-token block with the shared expert in the int8 format (workspace
    WS_SHARED8); fn_name="moe_layer_forward_batch_shared_i8": the union path
    instead (workspace WS_BATCH)."""
    _dev(x, torch.float32, "x")
    S = x.shape[0]
    out = torch.empty(S, layer.cfg.D, dtype=torch.float32, device=x.device) if out is None else out
    lc = layer.cstruct()
    e8 = shared8.cstruct()
    _check(getattr(lib(), fn_name)(ctypes.byref(layer.cfg), ctypes.byref(lc), ctypes.byref(e8),
                                   _ptr(x), S, _ptr(out), flags, ws.ptr, ws.nbytes,
                                   ctypes.c_void_p(_stream(stream))), fn_name)
    return out


class MlaConfig(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("kvl", ctypes.c_int32), ("nope", ctypes.c_int32),
                ("rope", ctypes.c_int32), ("vdim", ctypes.c_int32), ("scale", ctypes.c_float)]


class MlaWorkspace:
    """Device scratch of moe_mla_decode for up to S queries over T cache rows."""

    def __init__(self, cfg: MlaConfig, S: int, T: int, device="cuda"):
        n = lib().moe_mla_workspace_bytes(ctypes.byref(cfg), S, T)
        if n == 0:
            raise MoeError("moe_mla_workspace_bytes rejected the configuration")
        self.nbytes = int(n)
        self.buf = torch.empty(self.nbytes + 256, dtype=torch.uint8, device=device)
        off = (-self.buf.data_ptr()) % 256
        self.view = self.buf[off: off + self.nbytes]

    @property
    def ptr(self):
        return ctypes.c_void_p(self.view.data_ptr())


def moe_mla_decode(cfg: MlaConfig, q: torch.Tensor, kv_b: torch.Tensor, L: torch.Tensor,
                   R: torch.Tensor, ws: MlaWorkspace, out=None, stream=None):
    """Section 09 absorbed MLA decode: q [S][H][nope+rope], kv_b [H*(nope+vdim)][kvl],
    L [T][kvl], R [T][rope] (float32) -> ctx [S][H][vdim]."""
    for t, n in ((q, "q"), (kv_b, "kv_b"), (L, "L"), (R, "R")):
        _dev(t, torch.float32, n)
    S, T = q.shape[0], L.shape[0]
    ctx = torch.empty(S, cfg.H, cfg.vdim, dtype=torch.float32, device=q.device) if out is None else out
    _check(lib().moe_mla_decode(ctypes.byref(cfg), _ptr(q), S, _ptr(kv_b), _ptr(L), _ptr(R), T,
                                _ptr(ctx), ws.ptr, ws.nbytes, ctypes.c_void_p(_stream(stream))),
           "moe_mla_decode")
    return ctx


def _probe(topk_idx=None, topk_w=None, ev_gateup=None, ev_down=None, keff=None):
    p = Probe()
    p.topk_idx = None if topk_idx is None else topk_idx.data_ptr()
    p.topk_w = None if topk_w is None else topk_w.data_ptr()
    p.keff = None if keff is None else keff.data_ptr()
    if ev_gateup is not None:
        p.ev_gateup[0], p.ev_gateup[1] = ev_gateup
    if ev_down is not None:
        p.ev_down[0], p.ev_down[1] = ev_down
    return p


def _x_flags(x, flags, union: bool):
    """Checks x (float32, or bf16 on the union calls) and returns flags with
    F_X_BF16 set for bf16 rows."""
    if union and x.dtype == torch.bfloat16:
        _dev(x, torch.bfloat16, "x")
        return flags | F_X_BF16
    _dev(x, torch.float32, "x")
    return flags


def _layer_call(fn_name, layer: DeviceLayer, x, out, flags, ws, topk_idx, topk_w, ev_gateup,
                ev_down, stream, norm_gamma=None, norm_eps=1e-5, keff=None):
    flags = _x_flags(x, flags, fn_name == "moe_layer_forward_batch")
    S = x.shape[0]
    if out is None:
        out = torch.empty(S, layer.cfg.D, dtype=torch.float32, device=x.device)
    _dev(out, torch.float32, "out")
    if norm_gamma is not None:
        _dev(norm_gamma, torch.float32, "norm_gamma")
        flags |= F_PRENORM
    L = layer.cstruct(norm_gamma, norm_eps)
    probe = _probe(topk_idx, topk_w, ev_gateup, ev_down, keff)
    fn = getattr(lib(), fn_name)
    _check(fn(ctypes.byref(layer.cfg), ctypes.byref(L), _ptr(x), S, _ptr(out), flags,
              ctypes.byref(probe), ws.ptr, ws.nbytes, ctypes.c_void_p(_stream(stream))), fn_name)
    return out


def moe_layer_forward(layer: DeviceLayer, x: torch.Tensor, ws: Workspace, out=None, flags: int = 0,
                      topk_idx=None, topk_w=None, ev_gateup=None, ev_down=None, stream=None,
                      norm_gamma=None, norm_eps: float = 1e-5, keff=None):
    """Per-token path: each token reads its own K experts (keff with
    cfg.expert_topp) and the shared one.
    norm_gamma: run the block on RMSNorm(x) (flag F_PRENORM); out may then be x."""
    return _layer_call("moe_layer_forward", layer, x, out, flags, ws, topk_idx, topk_w, ev_gateup,
                       ev_down, stream, norm_gamma, norm_eps, keff)


def moe_layer_forward_batch(layer: DeviceLayer, x: torch.Tensor, ws: Workspace, out=None,
                            flags: int = 0, topk_idx=None, topk_w=None, ev_gateup=None,
                            ev_down=None, stream=None, norm_gamma=None, norm_eps: float = 1e-5,
                            keff=None):
    """Unique-expert union path: each selected expert is read once per call.
    x may be bf16 (flag F_X_BF16): the result is that of x.float()."""
    return _layer_call("moe_layer_forward_batch", layer, x, out, flags, ws, topk_idx, topk_w,
                       ev_gateup, ev_down, stream, norm_gamma, norm_eps, keff)


NOALLOC_WS_BYTES = 16 << 20


def moe_layer_forward_noalloc(layer: DeviceLayer, x: torch.Tensor, out=None, flags: int = 0,
                              stream=None, norm_gamma=None, norm_eps: float = 1e-5):
    """moe_layer_forward on the library's own device scratch (no workspace)."""
    _dev(x, torch.float32, "x")
    S = x.shape[0]
    if out is None:
        out = torch.empty(S, layer.cfg.D, dtype=torch.float32, device=x.device)
    _dev(out, torch.float32, "out")
    if norm_gamma is not None:
        _dev(norm_gamma, torch.float32, "norm_gamma")
        flags |= F_PRENORM
    L = layer.cstruct(norm_gamma, norm_eps)
    _check(lib().moe_layer_forward_noalloc(ctypes.byref(layer.cfg), ctypes.byref(L), _ptr(x), S,
                                           _ptr(out), flags, ctypes.c_void_p(_stream(stream))),
           "moe_layer_forward_noalloc")
    return out


def moe_stream_read(buf: torch.Tensor, stream=None) -> torch.Tensor:
    """Measurement reference: read buf once; returns the sink words."""
    n = lib().moe_stream_read_sink_words()
    sink = torch.empty(n, dtype=torch.int32, device=buf.device)
    _check(lib().moe_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                 ctypes.c_void_p(_stream(stream))), "moe_stream_read")
    return sink


def moe_rmsnorm(x: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-5, out=None, stream=None):
    _dev(x, torch.float32, "x")
    S, D = x.shape
    out = torch.empty_like(x) if out is None else out
    _check(lib().moe_rmsnorm(_ptr(x), _ptr(gamma), S, D, eps, _ptr(out),
                             ctypes.c_void_p(_stream(stream))), "moe_rmsnorm")
    return out


# ---- given routing and expert residency tiers ---------------------------------

def moe_layer_forward_routed(layer, x: torch.Tensor, topk_idx: torch.Tensor, topk_w: torch.Tensor,
                             ws: Workspace, out=None, flags: int = 0, stream=None,
                             norm_gamma=None, norm_eps: float = 1e-5,
                             fn_name: str = "moe_layer_forward_routed"):
    """Per-token path with the routing given: topk_idx [S][K] int32 indices
    into layer's routed stack, topk_w [S][K] float32 weights (device).
    fn_name="moe_layer_forward_batch_routed": the union path instead (its
    workspace is WS_BATCH; x may then be bf16)."""
    flags = _x_flags(x, flags, fn_name == "moe_layer_forward_batch_routed")
    _dev(topk_idx, torch.int32, "topk_idx")
    _dev(topk_w, torch.float32, "topk_w")
    S = x.shape[0]
    if out is None:
        out = torch.empty(S, layer.cfg.D, dtype=torch.float32, device=x.device)
    _dev(out, torch.float32, "out")
    if norm_gamma is not None:
        _dev(norm_gamma, torch.float32, "norm_gamma")
        flags |= F_PRENORM
    L = layer.cstruct(norm_gamma, norm_eps)
    _check(getattr(lib(), fn_name)(ctypes.byref(layer.cfg), ctypes.byref(L), _ptr(x), S,
                                   _ptr(topk_idx), _ptr(topk_w), _ptr(out), flags, ws.ptr,
                                   ws.nbytes, ctypes.c_void_p(_stream(stream))), fn_name)
    return out


def moe_layer_forward_batch_routed(layer, x: torch.Tensor, topk_idx: torch.Tensor,
                                   topk_w: torch.Tensor, ws: Workspace, out=None, flags: int = 0,
                                   stream=None, norm_gamma=None, norm_eps: float = 1e-5):
    """Unique-expert union path with the routing given (workspace WS_BATCH)."""
    return moe_layer_forward_routed(layer, x, topk_idx, topk_w, ws, out, flags, stream,
                                    norm_gamma, norm_eps, "moe_layer_forward_batch_routed")


class SlabLayout(ctypes.Structure):
    _fields_ = [("gate_q4", ctypes.c_int64), ("up_q4", ctypes.c_int64), ("down_q4", ctypes.c_int64),
                ("gate_s", ctypes.c_int64), ("up_s", ctypes.c_int64), ("down_s", ctypes.c_int64),
                ("bytes", ctypes.c_int64)]


def slab_layout(cfg: Config) -> SlabLayout:
    lay = SlabLayout()
    _check(lib().moe_slab_layout_of(ctypes.byref(cfg), ctypes.byref(lay)), "moe_slab_layout_of")
    return lay


class SlabExperts:
    """A stack of expert slabs (one slab per expert or slot) in the
    moe_experts form: base + offset, stride = slab bytes."""

    def __init__(self, buf: torch.Tensor, lay: SlabLayout):
        self.buf, self.lay = buf, lay

    def cstruct(self) -> Experts:
        b, L = self.buf.data_ptr(), self.lay

        def q(oq, os_):
            return QMat(b + oq, b + os_, L.bytes, L.bytes // 4)
        return Experts(q(L.gate_q4, L.gate_s), q(L.up_q4, L.up_s), q(L.down_q4, L.down_s))


def pack_slabs(experts: DeviceExperts, lay: SlabLayout, out: torch.Tensor) -> torch.Tensor:
    """Copy a stacked expert set into slab form (out: uint8 [n][lay.bytes],
    device or pinned host)."""
    n = experts.gate_q4.shape[0]
    parts = ((lay.gate_q4, experts.gate_q4), (lay.up_q4, experts.up_q4),
             (lay.down_q4, experts.down_q4), (lay.gate_s, experts.gate_s),
             (lay.up_s, experts.up_s), (lay.down_s, experts.down_s))
    for off, t in parts:
        flat = t.reshape(n, -1).view(torch.uint8)
        out[:, off:off + flat.shape[1]].copy_(flat)
    return out


class Tier:
    """Host bookkeeping of the HBM expert slots (moe_tier_*)."""

    def __init__(self, n_layers: int, n_experts: int, n_slots: int, n_pinned: int = 0):
        """n_slots LRU slots per layer, after n_pinned heat-managed ones."""
        h = (lib().moe_tier_create_pinned(n_layers, n_experts, n_slots, n_pinned) if n_pinned
             else lib().moe_tier_create(n_layers, n_experts, n_slots))
        if not h:
            raise MoeError("moe_tier_create failed")
        self.h, self.n_slots, self.n_pinned = h, n_slots, n_pinned

    def rebalance(self, layer: int):
        """(changed, pinned slot, new expert, replaced expert or -1)."""
        z, e, o = ctypes.c_int32(-1), ctypes.c_int32(-1), ctypes.c_int32(-1)
        r = lib().moe_tier_rebalance(self.h, layer, ctypes.byref(z), ctypes.byref(e),
                                     ctypes.byref(o))
        if r < 0:
            raise MoeError(f"moe_tier_rebalance: {status_str(r)}")
        return bool(r), z.value, e.value, o.value

    def __del__(self):
        if getattr(self, "h", None):
            lib().moe_tier_destroy(self.h)
            self.h = None

    def map(self, layer: int, eids):
        """(slots, loads, misses) for the experts of one call (host arrays)."""
        import numpy as np
        e = np.ascontiguousarray(eids, np.int32)
        slots = np.empty(e.size, np.int32)
        loads = np.empty(e.size, np.int32)
        r = lib().moe_tier_map(self.h, layer, e.ctypes.data, e.size, slots.ctypes.data,
                               loads.ctypes.data)
        if r < 0:
            raise MoeError(f"moe_tier_map: {status_str(r)}")
        return slots, loads, r

    def stats(self):
        h, m = ctypes.c_uint64(0), ctypes.c_uint64(0)
        _check(lib().moe_tier_stats(self.h, ctypes.byref(h), ctypes.byref(m)), "moe_tier_stats")
        return h.value, m.value

    @staticmethod
    def fetch(host_slabs: torch.Tensor, hbm_slots: torch.Tensor, slab_bytes: int, eids, slots,
              loads, stream=None):
        import numpy as np
        e = np.ascontiguousarray(eids, np.int32)
        sl = np.ascontiguousarray(slots, np.int32)
        ld = np.ascontiguousarray(loads, np.int32)
        _check(lib().moe_tier_fetch(_ptr(host_slabs), _ptr(hbm_slots), slab_bytes, e.ctypes.data,
                                    sl.ctypes.data, ld.ctypes.data, e.size,
                                    ctypes.c_void_p(_stream(stream))), "moe_tier_fetch")


def tier_pick_swap(heat, pinned):
    """(swap?, pinned position, expert, gain) by the section 13 rule."""
    import numpy as np
    h = np.ascontiguousarray(heat, np.uint32)
    p = np.ascontiguousarray(pinned, np.int32)
    slot, eid, gain = ctypes.c_int32(-1), ctypes.c_int32(-1), ctypes.c_int64(0)
    r = lib().moe_tier_pick_swap(h.ctypes.data, h.size, p.ctypes.data, p.size, ctypes.byref(slot),
                                 ctypes.byref(eid), ctypes.byref(gain))
    return bool(r), slot.value, eid.value, gain.value


def tier_lfru_score(heat: int, last: int, clock: int) -> int:
    return int(lib().moe_tier_lfru_score(heat, last, clock))


@dataclass
class TieredLayer:
    """One layer whose routed experts live in pinned host memory (all of them)
    and in n_slots HBM slots (those in use); router and shared expert in HBM.
    forward() routes on the device, maps the selected experts to slots on the
    host, copies the missing slabs in and runs the per-token block on the slot
    stack with the routing rewritten to slot numbers."""
    cfg: Config
    router_w: torch.Tensor
    router_b: torch.Tensor
    routed: SlabExperts        # the HBM slot stack
    shared: DeviceExperts | None
    host_slabs: torch.Tensor   # pinned uint8 [E][slab]
    tier: Tier
    layer_index: int = 0

    @staticmethod
    def from_device_layer(dl: DeviceLayer, n_slots: int, tier: Tier | None = None,
                          layer_index: int = 0, host_slabs: torch.Tensor | None = None,
                          n_pinned: int = 0) -> "TieredLayer":
        """host_slabs: reuse the pinned slabs of an earlier TieredLayer of the
        same layer instead of packing them again."""
        lay = slab_layout(dl.cfg)
        E = dl.cfg.E
        host = host_slabs
        if host is None:
            host = torch.empty(E, lay.bytes, dtype=torch.uint8, pin_memory=True)
            for e0 in range(0, E, 16):  # staged 16 experts at a time
                e1 = min(E, e0 + 16)
                part = DeviceExperts(*(t[e0:e1] for t in (
                    dl.routed.gate_q4, dl.routed.gate_s, dl.routed.up_q4, dl.routed.up_s,
                    dl.routed.down_q4, dl.routed.down_s)))
                staged = pack_slabs(part, lay, torch.empty(e1 - e0, lay.bytes, dtype=torch.uint8,
                                                           device=dl.router_w.device))
                host[e0:e1].copy_(staged)
            del staged
        slots = torch.empty(n_pinned + n_slots, lay.bytes, dtype=torch.uint8,
                            device=dl.router_w.device)
        tier = tier or Tier(1, E, n_slots, n_pinned)
        return TieredLayer(dl.cfg, dl.router_w, dl.router_b, SlabExperts(slots, lay), dl.shared,
                           host, tier, layer_index)

    def cstruct(self, norm_gamma=None, norm_eps: float = 0.0) -> LayerC:
        """Router and shared expert resident; routed experts = the slot stack."""
        sh = self.shared.cstruct() if self.shared is not None else Experts()
        g = None if norm_gamma is None else norm_gamma.data_ptr()
        return LayerC(self.router_w.data_ptr(), self.router_b.data_ptr(), self.routed.cstruct(), sh,
                      g, float(norm_eps))

    def forward(self, x: torch.Tensor, ws_router: Workspace, ws: Workspace, out=None,
                stream=None, union: bool = False):
        """Returns (out, misses of this call), through moe_tier_forward: the
        selection is read back once, the missing slabs are copied in and the
        block runs on the slot stack.  union: the unique-expert union path (ws
        must then be a WS_BATCH workspace); the union of the tokens' experts
        must fit in the layer's slots."""
        _dev(x, torch.float32, "x")
        S = x.shape[0]
        n = S * self.cfg.K
        if getattr(self, "_host_idx", None) is None or self._host_idx.numel() < n:
            self._host_idx = torch.empty(n, dtype=torch.int32, pin_memory=True)
        if out is None:
            out = torch.empty(S, self.cfg.D, dtype=torch.float32, device=x.device)
        L = self.cstruct()
        misses = ctypes.c_int32(0)
        _check(lib().moe_tier_forward(self.tier.h, self.layer_index, ctypes.byref(self.cfg),
                                      ctypes.byref(L), _ptr(self.host_slabs), _ptr(self.routed.buf),
                                      self.routed.lay.bytes, _ptr(x), S, _ptr(out), 0,
                                      1 if union else 0, _ptr(self._host_idx),
                                      ctypes.byref(misses), ws_router.ptr, ws_router.nbytes,
                                      ws.ptr, ws.nbytes, ctypes.c_void_p(_stream(stream))),
               "moe_tier_forward")
        o = out
        if self.tier.n_pinned:
            # one pinned-slot change by heat; its copy is ordered after the call
            changed, z, e, _ = self.tier.rebalance(self.layer_index)
            if changed:
                Tier.fetch(self.host_slabs, self.routed.buf, self.routed.lay.bytes, [e], [z], [1],
                           stream)
        return o, misses.value
