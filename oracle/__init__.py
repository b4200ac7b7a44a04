"""ctypes binding of the CPU oracle (oracle/moe_ref.c).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product package.  Everything here
works on host numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

ACCUMULATE = 1


class Config(ctypes.Structure):
    _fields_ = [("D", ctypes.c_int32), ("I", ctypes.c_int32), ("E", ctypes.c_int32),
                ("K", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("routed_scale", ctypes.c_float), ("expert_topp", ctypes.c_float)]


class QMat(ctypes.Structure):
    _fields_ = [("q4", ctypes.c_void_p), ("scale", ctypes.c_void_p)]


class Expert(ctypes.Structure):
    _fields_ = [("gate", QMat), ("up", QMat), ("down", QMat)]


class Layer(ctypes.Structure):
    _fields_ = [("router_w", ctypes.c_void_p), ("router_b", ctypes.c_void_p),
                ("experts", ctypes.c_void_p), ("shared", ctypes.c_void_p)]


def lib():
    global _lib
    if _lib is None:
        # MOE_REF_LIB may name another build of the same source (e.g. a sanitizer build)
        path = os.environ.get("MOE_REF_LIB") or os.path.join(HERE, "libmoe_ref.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run oracle/build.py (or __graft_entry__.build())")
        L = ctypes.CDLL(path)
        vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        L.moe_ref_pack_int4.argtypes = [vp, i32, i32, vp, vp]
        L.moe_ref_unpack_int4.argtypes = [vp, i32, i32, vp]
        L.moe_ref_quant_row_i8.argtypes = [vp, i32, vp]
        L.moe_ref_quant_row_i8.restype = f32
        L.moe_ref_quant_act_i8.argtypes = [vp, i32, i32, vp, vp]
        L.moe_ref_quant_act_i8_bf16.argtypes = [vp, i32, i32, vp, vp]
        L.moe_ref_dot_i4_i8.argtypes = [vp, vp, i32]
        L.moe_ref_dot_i4_i8.restype = ctypes.c_int32
        L.moe_ref_router_topk.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp, vp]
        L.moe_ref_expert_swiglu_i4.argtypes = [vp, vp, vp, i32, vp, vp, vp, vp, vp, vp]
        L.moe_ref_quantize_rows.argtypes = [vp, i32, i32, i32, vp, vp]
        L.moe_ref_dot_i8_i8.argtypes = [vp, vp, i32]
        L.moe_ref_dot_i8_i8.restype = ctypes.c_int32
        L.moe_ref_expert_swiglu_i8.argtypes = [vp, vp, vp, i32, vp, vp, vp, vp, vp, vp]
        L.moe_ref_pack_int2.argtypes = [vp, i32, i32, vp, vp]
        L.moe_ref_quant_act_b32.argtypes = [vp, i32, i32, vp, vp]
        L.moe_ref_mla_decode.argtypes = [vp, vp, i32, vp, vp, vp, i32, vp]
        L.moe_ref_layer_forward_shared_i8.argtypes = [vp, vp, vp, vp, i32, vp, ctypes.c_uint]
        L.moe_ref_expert_swiglu_i4_b32.argtypes = [vp, vp, vp, i32, vp, vp, vp, vp]
        L.moe_ref_unpack_int2.argtypes = [vp, i32, i32, vp]
        L.moe_ref_expert_swiglu_i2.argtypes = [vp, vp, vp, i32, vp, vp, vp, vp, vp, vp]
        L.moe_ref_layer_forward.argtypes = [vp, vp, vp, i32, vp, ctypes.c_uint]
        L.moe_ref_layer_forward_batch.argtypes = [vp, vp, vp, i32, vp, ctypes.c_uint, vp, vp, vp, vp]
        L.moe_ref_layer_forward_routed.argtypes = [vp, vp, vp, i32, vp, vp, vp, ctypes.c_uint]
        L.moe_ref_layer_forward_batch_routed.argtypes = [vp, vp, vp, i32, vp, vp, vp, ctypes.c_uint,
                                                         vp, vp]
        L.moe_ref_layer_forward_batch_shared_i8.argtypes = [vp, vp, vp, vp, i32, vp, ctypes.c_uint,
                                                            vp, vp]
        L.moe_ref_rmsnorm.argtypes = [vp, vp, i32, i32, f32, vp]
        L.moe_ref_expert_keff.argtypes = [vp, i32, f32]
        L.moe_ref_expert_get.argtypes = [vp, vp, i32, vp, vp, vp, vp, ctypes.c_int32, vp]
        L.moe_ref_tier_pick_swap.argtypes = [vp, i32, vp, i32, vp, vp, vp]
        L.moe_ref_tier_lfru_score.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32]
        L.moe_ref_tier_lfru_score.restype = ctypes.c_uint64
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name} returned {rc}")


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def make_config(D, I, E, K, n_shared=1, routed_scale=2.5, expert_topp=0.0) -> Config:
    return Config(D, I, E, K, n_shared, routed_scale, expert_topp)


# ---- primitives -------------------------------------------------------------

def pack_int4(w: np.ndarray):
    w = _c(w, np.float32)
    O, C = w.shape
    q4 = np.empty((O, (C + 1) // 2), np.uint8)
    s = np.empty(O, np.float32)
    _check(lib().moe_ref_pack_int4(_p(w), O, C, _p(q4), _p(s)), "pack_int4")
    return q4, s


def unpack_int4(q4: np.ndarray, C: int) -> np.ndarray:
    q4 = _c(q4, np.uint8)
    O = q4.shape[0]
    q = np.empty((O, C), np.int8)
    _check(lib().moe_ref_unpack_int4(_p(q4), O, C, _p(q)), "unpack_int4")
    return q


def quant_act_i8(x: np.ndarray):
    x = _c(x, np.float32)
    S, D = x.shape
    xq = np.empty((S, D), np.int8)
    sx = np.empty(S, np.float32)
    _check(lib().moe_ref_quant_act_i8(_p(x), S, D, _p(xq), _p(sx)), "quant_act_i8")
    return xq, sx


def quant_act_i8_bf16(xbits: np.ndarray):
    xbits = _c(xbits, np.uint16)
    S, D = xbits.shape
    xq = np.empty((S, D), np.int8)
    sx = np.empty(S, np.float32)
    _check(lib().moe_ref_quant_act_i8_bf16(_p(xbits), S, D, _p(xq), _p(sx)), "quant_act_i8_bf16")
    return xq, sx


def dot_i4_i8(q4row: np.ndarray, x: np.ndarray) -> int:
    q4row = _c(q4row, np.uint8)
    x = _c(x, np.int8)
    return int(lib().moe_ref_dot_i4_i8(_p(q4row), _p(x), x.shape[0]))


def router_topk(cfg: Config, x: np.ndarray, wr: np.ndarray, b: np.ndarray):
    x = _c(x, np.float32)
    S = x.shape[0]
    wr, b = _c(wr, np.float32), _c(b, np.float32)
    idx = np.empty((S, cfg.K), np.int32)
    w = np.empty((S, cfg.K), np.float32)
    logits = np.empty((S, cfg.E), np.float32)
    choice = np.empty((S, cfg.E), np.float32)
    _check(lib().moe_ref_router_topk(ctypes.byref(cfg), _p(x), S, _p(wr), _p(b), _p(idx), _p(w),
                                     _p(logits), _p(choice)), "router_topk")
    return idx, w, logits, choice


# ---- experts and layers -----------------------------------------------------

@dataclass
class HostExpert:
    """Packed int4 expert on the host: gate/up [I][D/2], down [D][I/2]."""
    gate_q4: np.ndarray
    gate_s: np.ndarray
    up_q4: np.ndarray
    up_s: np.ndarray
    down_q4: np.ndarray
    down_s: np.ndarray

    def cstruct(self) -> Expert:
        return Expert(QMat(_p(self.gate_q4), _p(self.gate_s)), QMat(_p(self.up_q4), _p(self.up_s)),
                      QMat(_p(self.down_q4), _p(self.down_s)))

    @staticmethod
    def from_f32(g, u, d) -> "HostExpert":
        gq, gs = pack_int4(g)
        uq, us = pack_int4(u)
        dq, ds = pack_int4(d)
        return HostExpert(gq, gs, uq, us, dq, ds)


def expert_swiglu(cfg: Config, xq: np.ndarray, sx: np.ndarray, e: HostExpert):
    xq = _c(xq, np.int8)
    sx = _c(sx, np.float32)
    S = xq.shape[0]
    y = np.empty((S, cfg.D), np.float32)
    acc_gu = np.empty((S, 2, cfg.I), np.int32)
    hq = np.empty((S, cfg.I), np.int8)
    sh = np.empty(S, np.float32)
    acc_d = np.empty((S, cfg.D), np.int32)
    es = e.cstruct()
    _check(lib().moe_ref_expert_swiglu_i4(ctypes.byref(cfg), _p(xq), _p(sx), S, ctypes.byref(es),
                                          _p(y), _p(acc_gu), _p(hq), _p(sh), _p(acc_d)),
           "expert_swiglu_i4")
    return dict(y=y, acc_gu=acc_gu, hq=hq, sh=sh, acc_d=acc_d)


def quantize_rows(w: np.ndarray, bits: int = 8):
    """Section 05 per-row quantizer: (q [O][C] int8, scale [O] float32)."""
    w = _c(w, np.float32)
    O, C = w.shape
    q = np.empty((O, C), np.int8)
    s = np.empty(O, np.float32)
    _check(lib().moe_ref_quantize_rows(_p(w), O, C, bits, _p(q), _p(s)), "quantize_rows")
    return q, s


def dot_i8_i8(w: np.ndarray, x: np.ndarray) -> int:
    w = _c(w, np.int8)
    x = _c(x, np.int8)
    return int(lib().moe_ref_dot_i8_i8(_p(w), _p(x), w.size))


class Q8Mat(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("scale", ctypes.c_void_p)]


class ExpertI8(ctypes.Structure):
    _fields_ = [("gate", Q8Mat), ("up", Q8Mat), ("down", Q8Mat)]


@dataclass
class HostExpertI8:
    """int8 expert on the host (section 05 format): gate/up [I][D], down [D][I]."""
    gate_q: np.ndarray
    gate_s: np.ndarray
    up_q: np.ndarray
    up_s: np.ndarray
    down_q: np.ndarray
    down_s: np.ndarray

    def cstruct(self) -> ExpertI8:
        return ExpertI8(Q8Mat(_p(self.gate_q), _p(self.gate_s)), Q8Mat(_p(self.up_q), _p(self.up_s)),
                        Q8Mat(_p(self.down_q), _p(self.down_s)))

    @staticmethod
    def from_f32(g, u, d) -> "HostExpertI8":
        gq, gs = quantize_rows(g, 8)
        uq, us = quantize_rows(u, 8)
        dq, ds = quantize_rows(d, 8)
        return HostExpertI8(gq, gs, uq, us, dq, ds)


def expert_swiglu_i8(cfg: Config, xq: np.ndarray, sx: np.ndarray, e: HostExpertI8):
    xq = _c(xq, np.int8)
    sx = _c(sx, np.float32)
    S = xq.shape[0]
    y = np.empty((S, cfg.D), np.float32)
    acc_gu = np.empty((S, 2, cfg.I), np.int32)
    hq = np.empty((S, cfg.I), np.int8)
    sh = np.empty(S, np.float32)
    acc_d = np.empty((S, cfg.D), np.int32)
    es = e.cstruct()
    _check(lib().moe_ref_expert_swiglu_i8(ctypes.byref(cfg), _p(xq), _p(sx), S, ctypes.byref(es),
                                          _p(y), _p(acc_gu), _p(hq), _p(sh), _p(acc_d)),
           "expert_swiglu_i8")
    return dict(y=y, acc_gu=acc_gu, hq=hq, sh=sh, acc_d=acc_d)


def pack_int2(w: np.ndarray):
    """Packed int2 rows: (q2 [O][(C+3)/4] uint8, scale [O] float32)."""
    w = _c(w, np.float32)
    O, C = w.shape
    q2 = np.empty((O, (C + 3) // 4), np.uint8)
    s = np.empty(O, np.float32)
    _check(lib().moe_ref_pack_int2(_p(w), O, C, _p(q2), _p(s)), "pack_int2")
    return q2, s


def unpack_int2(q2: np.ndarray, C: int) -> np.ndarray:
    q2 = _c(q2, np.uint8)
    O = q2.shape[0]
    q = np.empty((O, C), np.int8)
    _check(lib().moe_ref_unpack_int2(_p(q2), O, C, _p(q)), "unpack_int2")
    return q


@dataclass
class HostExpertI2:
    """Packed int2 expert on the host: gate/up [I][D/4], down [D][I/4]."""
    gate_q2: np.ndarray
    gate_s: np.ndarray
    up_q2: np.ndarray
    up_s: np.ndarray
    down_q2: np.ndarray
    down_s: np.ndarray

    def cstruct(self) -> Expert:
        return Expert(QMat(_p(self.gate_q2), _p(self.gate_s)), QMat(_p(self.up_q2), _p(self.up_s)),
                      QMat(_p(self.down_q2), _p(self.down_s)))

    @staticmethod
    def from_f32(g, u, d) -> "HostExpertI2":
        gq, gs = pack_int2(g)
        uq, us = pack_int2(u)
        dq, ds = pack_int2(d)
        return HostExpertI2(gq, gs, uq, us, dq, ds)


def expert_swiglu_i2(cfg: Config, xq: np.ndarray, sx: np.ndarray, e: HostExpertI2):
    xq = _c(xq, np.int8)
    sx = _c(sx, np.float32)
    S = xq.shape[0]
    y = np.empty((S, cfg.D), np.float32)
    acc_gu = np.empty((S, 2, cfg.I), np.int32)
    hq = np.empty((S, cfg.I), np.int8)
    sh = np.empty(S, np.float32)
    acc_d = np.empty((S, cfg.D), np.int32)
    es = e.cstruct()
    _check(lib().moe_ref_expert_swiglu_i2(ctypes.byref(cfg), _p(xq), _p(sx), S, ctypes.byref(es),
                                          _p(y), _p(acc_gu), _p(hq), _p(sh), _p(acc_d)),
           "expert_swiglu_i2")
    return dict(y=y, acc_gu=acc_gu, hq=hq, sh=sh, acc_d=acc_d)


def quant_act_b32(x: np.ndarray):
    """Block-32 activation quantization: (xq [S][D] int8, sxb [S][D/32] float32)."""
    x = _c(x, np.float32)
    S, D = x.shape
    xq = np.empty((S, D), np.int8)
    sxb = np.empty((S, D // 32), np.float32)
    _check(lib().moe_ref_quant_act_b32(_p(x), S, D, _p(xq), _p(sxb)), "quant_act_b32")
    return xq, sxb


def expert_swiglu_b32(cfg: Config, xq: np.ndarray, sxb: np.ndarray, e: HostExpert):
    xq = _c(xq, np.int8)
    sxb = _c(sxb, np.float32)
    S = xq.shape[0]
    y = np.empty((S, cfg.D), np.float32)
    hq = np.empty((S, cfg.I), np.int8)
    shb = np.empty((S, cfg.I // 32), np.float32)
    es = e.cstruct()
    _check(lib().moe_ref_expert_swiglu_i4_b32(ctypes.byref(cfg), _p(xq), _p(sxb), S,
                                              ctypes.byref(es), _p(y), _p(hq), _p(shb)),
           "expert_swiglu_i4_b32")
    return dict(y=y, hq=hq, shb=shb)


class MlaConfig(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("kvl", ctypes.c_int32), ("nope", ctypes.c_int32),
                ("rope", ctypes.c_int32), ("vdim", ctypes.c_int32), ("scale", ctypes.c_float)]


def mla_decode(cfg: MlaConfig, q: np.ndarray, kv_b: np.ndarray, L: np.ndarray, R: np.ndarray):
    """Section 09 absorbed MLA decode: q [S][H][nope+rope], kv_b [H*(nope+vdim)][kvl],
    L [T][kvl], R [T][rope] -> ctx [S][H][vdim]."""
    q, kv_b, L, R = (_c(a, np.float32) for a in (q, kv_b, L, R))
    S, T = q.shape[0], L.shape[0]
    ctx = np.empty((S, cfg.H, cfg.vdim), np.float32)
    _check(lib().moe_ref_mla_decode(ctypes.byref(cfg), _p(q), S, _p(kv_b), _p(L), _p(R), T, _p(ctx)),
           "mla_decode")
    return ctx


class HostLayer:
    """Router weights plus a dict of packed experts (any subset may be present;
    the oracle fails if routing selects an expert that is absent)."""

    def __init__(self, cfg: Config, router_w, router_b, experts: dict, shared: HostExpert | None):
        self.cfg = cfg
        self.router_w = _c(router_w, np.float32)
        self.router_b = _c(router_b, np.float32)
        self.experts = experts
        self.shared = shared

    def cstruct(self):
        arr = (Expert * self.cfg.E)()
        for e, ex in self.experts.items():
            arr[e] = ex.cstruct()
        sh = self.shared.cstruct() if self.shared is not None else None
        keep = (arr, sh)
        L = Layer(_p(self.router_w), _p(self.router_b), ctypes.addressof(arr),
                  ctypes.addressof(sh) if sh is not None else None)
        return L, keep


def layer_forward(layer: HostLayer, x: np.ndarray, out: np.ndarray | None = None, flags: int = 0):
    x = _c(x, np.float32)
    S = x.shape[0]
    out = np.zeros((S, layer.cfg.D), np.float32) if out is None else out
    L, keep = layer.cstruct()
    _check(lib().moe_ref_layer_forward(ctypes.byref(layer.cfg), ctypes.byref(L), _p(x), S, _p(out),
                                       flags), "layer_forward")
    return out


def layer_forward_shared_i8(layer: HostLayer, shared8: HostExpertI8, x: np.ndarray,
                            out: np.ndarray | None = None, flags: int = 0):
    """The per-token block with the shared expert in the int8 format."""
    x = _c(x, np.float32)
    S = x.shape[0]
    out = np.zeros((S, layer.cfg.D), np.float32) if out is None else out
    L, keep = layer.cstruct()
    e8 = shared8.cstruct()
    _check(lib().moe_ref_layer_forward_shared_i8(ctypes.byref(layer.cfg), ctypes.byref(L),
                                                 ctypes.byref(e8), _p(x), S, _p(out), flags),
           "layer_forward_shared_i8")
    return out


def layer_forward_batch(layer: HostLayer, x: np.ndarray, out: np.ndarray | None = None,
                        flags: int = 0):
    x = _c(x, np.float32)
    S = x.shape[0]
    cfg = layer.cfg
    out = np.zeros((S, cfg.D), np.float32) if out is None else out
    idx = np.empty((S, cfg.K), np.int32)
    w = np.empty((S, cfg.K), np.float32)
    uniq = np.empty(cfg.E, np.int32)
    nu = ctypes.c_int32(0)
    L, keep = layer.cstruct()
    _check(lib().moe_ref_layer_forward_batch(ctypes.byref(cfg), ctypes.byref(L), _p(x), S, _p(out),
                                             flags, _p(idx), _p(w), _p(uniq), ctypes.byref(nu)),
           "layer_forward_batch")
    return out, idx, w, uniq[: nu.value].copy()


def layer_forward_routed(layer: HostLayer, x: np.ndarray, idx: np.ndarray, w: np.ndarray,
                         out: np.ndarray | None = None, flags: int = 0):
    """The per-token block on the given routing idx [S][K] (in [0, E)), w [S][K]."""
    x = _c(x, np.float32)
    S = x.shape[0]
    cfg = layer.cfg
    idx = _c(idx, np.int32).reshape(S, cfg.K)
    w = _c(w, np.float32).reshape(S, cfg.K)
    out = np.zeros((S, cfg.D), np.float32) if out is None else out
    L, keep = layer.cstruct()
    _check(lib().moe_ref_layer_forward_routed(ctypes.byref(cfg), ctypes.byref(L), _p(x), S, _p(idx),
                                              _p(w), _p(out), flags), "layer_forward_routed")
    return out


def layer_forward_batch_routed(layer: HostLayer, x: np.ndarray, idx: np.ndarray, w: np.ndarray,
                               out: np.ndarray | None = None, flags: int = 0):
    """The unique-expert union on the given routing: (out, union in first-appearance order)."""
    x = _c(x, np.float32)
    S = x.shape[0]
    cfg = layer.cfg
    idx = _c(idx, np.int32).reshape(S, cfg.K)
    w = _c(w, np.float32).reshape(S, cfg.K)
    out = np.zeros((S, cfg.D), np.float32) if out is None else out
    uniq = np.empty(cfg.E, np.int32)
    nu = ctypes.c_int32(0)
    L, keep = layer.cstruct()
    _check(lib().moe_ref_layer_forward_batch_routed(ctypes.byref(cfg), ctypes.byref(L), _p(x), S,
                                                    _p(idx), _p(w), _p(out), flags, _p(uniq),
                                                    ctypes.byref(nu)), "layer_forward_batch_routed")
    return out, uniq[: nu.value].copy()


def layer_forward_batch_shared_i8(layer: HostLayer, shared8: HostExpertI8, x: np.ndarray,
                                  out: np.ndarray | None = None, flags: int = 0):
    """The unique-expert union with the shared expert in the int8 format."""
    x = _c(x, np.float32)
    S = x.shape[0]
    cfg = layer.cfg
    out = np.zeros((S, cfg.D), np.float32) if out is None else out
    uniq = np.empty(cfg.E, np.int32)
    nu = ctypes.c_int32(0)
    L, keep = layer.cstruct()
    e8 = shared8.cstruct()
    _check(lib().moe_ref_layer_forward_batch_shared_i8(ctypes.byref(cfg), ctypes.byref(L),
                                                       ctypes.byref(e8), _p(x), S, _p(out), flags,
                                                       _p(uniq), ctypes.byref(nu)),
           "layer_forward_batch_shared_i8")
    return out, uniq[: nu.value].copy()


def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float = 1e-5) -> np.ndarray:
    x = _c(x, np.float32)
    S, D = x.shape
    gamma = _c(gamma, np.float32)
    y = np.empty_like(x)
    _check(lib().moe_ref_rmsnorm(_p(x), _p(gamma), S, D, eps, _p(y)), "rmsnorm")
    return y


class ExpertCache:
    """Section 05 per-layer expert caches (cap slots per layer) with the
    article's shared clock and hit/miss counters, driven through the oracle's
    moe_ref_expert_get."""

    def __init__(self, n_layers: int, cap: int):
        self.cap = cap
        self.eid = np.full((n_layers, cap), -1, np.int32)
        self.used = np.zeros((n_layers, cap), np.uint64)
        self.n_used = np.zeros(n_layers, np.int32)
        self.counters = np.zeros(3, np.uint64)  # clock, hits, misses

    def get(self, layer: int, eid: int):
        """(slot, loaded) for one lookup."""
        loaded = ctypes.c_int(0)
        n = ctypes.c_int(int(self.n_used[layer]))
        c = self.counters
        cp = c.ctypes.data
        slot = lib().moe_ref_expert_get(self.eid[layer].ctypes.data, self.used[layer].ctypes.data,
                                        self.cap, ctypes.byref(n), cp, cp + 8, cp + 16,
                                        int(eid), ctypes.byref(loaded))
        if slot < 0:
            raise ValueError("moe_ref_expert_get rejected its arguments")
        self.n_used[layer] = n.value
        return slot, loaded.value

    @property
    def hits(self) -> int:
        return int(self.counters[1])

    @property
    def misses(self) -> int:
        return int(self.counters[2])


def tier_pick_swap(heat, pinned):
    """(swap?, pinned position, expert, gain) of the section 13 swap rule."""
    heat = np.ascontiguousarray(heat, np.uint32)
    pinned = np.ascontiguousarray(pinned, np.int32)
    slot, eid, gain = ctypes.c_int32(-1), ctypes.c_int32(-1), ctypes.c_int64(0)
    r = lib().moe_ref_tier_pick_swap(heat.ctypes.data, heat.size, pinned.ctypes.data, pinned.size,
                                     ctypes.byref(slot), ctypes.byref(eid), ctypes.byref(gain))
    return bool(r), slot.value, eid.value, gain.value


def tier_lfru_score(heat: int, last: int, clock: int) -> int:
    return int(lib().moe_ref_tier_lfru_score(heat, last, clock))


def expert_keff(w, p: float) -> int:
    """Adaptive expert top-p: experts kept for one token's weights w[K]."""
    w = np.ascontiguousarray(w, np.float32)
    return int(lib().moe_ref_expert_keff(w.ctypes.data, w.size, float(p)))
