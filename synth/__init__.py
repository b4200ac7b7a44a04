"""Seeded synthetic inputs for the routed-expert int4 MoE block.

One definition (synth.h) serves both sides: the host library fills numpy
arrays for the CPU oracle, the device library fills GPU buffers for the HIP
path, and the two produce identical bits.  This module holds none of the
block's arithmetic: no quantization, routing or expert math, only random
numbers and the input recipes built from them.

Recipes (shapes follow the GLM-5.2 configuration printed in section 02 of the
reader.mx article "惊呆了！25GB 内存上运行 GLM 5.2 744B 模型"):

* weights (router, gate, up, down): N(0, 0.02) in float32; the experts'
  float weights are later packed to int4 by the code under test;
* router correction bias: U(-0.1, 0.1), or 0 for the Zipf and uniform
  routing recipes, or the per-layer Zipf bias of the layer stack;
* activations: N(0, 1) float32, or rounded to bf16 for the prefill recipe;
* Zipf-skewed decode batch: token activations are solved so that the real
  router produces logits log p_e + Gumbel noise, p_e proportional to
  rank^-1.1 over a seeded permutation of the experts (Gumbel top-k, i.e.
  Plackett-Luce sampling without replacement from Zipf(1.1)).
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))

K_ROUTER_W, K_ROUTER_B, K_X, K_GATE, K_UP, K_DOWN, K_GAMMA, K_PERM, K_GUMBEL, K_Z = range(1, 11)
SHARED = 0xFFFF  # item id of the shared expert in stream ids

_host = None
_dev = None


def _load_host():
    global _host
    if _host is None:
        # SYNTH_HOST_LIB may name another build of the same source (e.g. a sanitizer build)
        path = os.environ.get("SYNTH_HOST_LIB") or os.path.join(HERE, "libsynth_host.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run synth/build.py (or __graft_entry__.build())")
        lib = ctypes.CDLL(path)
        u64, f32, f64, vp = ctypes.c_uint64, ctypes.c_float, ctypes.c_double, ctypes.c_void_p
        lib.synth_normal_scale.argtypes = [f64]
        lib.synth_normal_scale.restype = f32
        lib.synth_fill_normal.argtypes = [u64, u64, u64, u64, f32, vp]
        lib.synth_fill_uniform.argtypes = [u64, u64, u64, u64, f32, f32, vp]
        lib.synth_fill_unit_f64.argtypes = [u64, u64, u64, u64, vp]
        lib.synth_fill_ih8.argtypes = [u64, u64, u64, u64, vp]
        lib.synth_f32_to_bf16_array.argtypes = [vp, u64, vp]
        _host = lib
    return _host


def _load_dev():
    global _dev
    if _dev is None:
        path = os.path.join(HERE, "libsynth_dev.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run synth/build.py (or __graft_entry__.build())")
        lib = ctypes.CDLL(path)
        u64, f32, vp = ctypes.c_uint64, ctypes.c_float, ctypes.c_void_p
        lib.synth_dev_fill_normal.argtypes = [u64, u64, u64, u64, f32, vp, vp]
        lib.synth_dev_fill_normal.restype = ctypes.c_int
        _dev = lib
    return _dev


def stream(kind: int, layer: int = 0, item: int = 0) -> int:
    return ((kind & 0xFFFF) << 48) | ((layer & 0xFFFF) << 32) | (item & 0xFFFFFFFF)


def normal_scale(sigma: float) -> float:
    return float(_load_host().synth_normal_scale(float(sigma)))


def host_normal(seed: int, strm: int, n: int, sigma: float, start: int = 0) -> np.ndarray:
    out = np.empty(int(n), np.float32)
    lib = _load_host()
    lib.synth_fill_normal(seed, strm, start, int(n), lib.synth_normal_scale(float(sigma)),
                          out.ctypes.data)
    return out


def host_ih8(seed: int, strm: int, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(int(n), np.int32)
    _load_host().synth_fill_ih8(seed, strm, start, int(n), out.ctypes.data)
    return out


def host_uniform(seed: int, strm: int, n: int, lo: float, hi: float, start: int = 0) -> np.ndarray:
    out = np.empty(int(n), np.float32)
    _load_host().synth_fill_uniform(seed, strm, start, int(n), lo, hi, out.ctypes.data)
    return out


def host_unit_f64(seed: int, strm: int, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(int(n), np.float64)
    _load_host().synth_fill_unit_f64(seed, strm, start, int(n), out.ctypes.data)
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    _load_host().synth_f32_to_bf16_array(x.ctypes.data, x.size, out.ctypes.data)
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint32) << 16).view(np.float32)


def dev_fill_normal(ptr: int, seed: int, strm: int, n: int, sigma: float, hip_stream: int,
                    start: int = 0) -> None:
    """Fill n float32 values at device address ptr on the given HIP stream."""
    rc = _load_dev().synth_dev_fill_normal(seed, strm, start, int(n), normal_scale(sigma),
                                           ctypes.c_void_p(ptr), ctypes.c_void_p(hip_stream))
    if rc != 0:
        raise RuntimeError(f"synth_dev_fill_normal failed ({rc})")


# --------------------------------------------------------------------------
# Shapes and recipes
# --------------------------------------------------------------------------

WEIGHT_SIGMA = 0.02


@dataclass(frozen=True)
class Shape:
    D: int
    I: int
    E: int
    K: int
    n_shared: int = 1
    routed_scale: float = 2.5


TINY = Shape(D=256, I=128, E=8, K=2)
GLM = Shape(D=6144, I=2048, E=256, K=8)


def expert_streams(layer: int, expert: int):
    """Stream ids of the gate, up and down float weights of one expert
    (expert == SHARED for the shared expert)."""
    return (stream(K_GATE, layer, expert), stream(K_UP, layer, expert), stream(K_DOWN, layer, expert))


def host_expert_f32(seed: int, shape: Shape, layer: int, expert: int):
    """gate [I][D], up [I][D], down [D][I] float32 weights of one expert."""
    sg, su, sd = expert_streams(layer, expert)
    D, I = shape.D, shape.I
    g = host_normal(seed, sg, I * D, WEIGHT_SIGMA).reshape(I, D)
    u = host_normal(seed, su, I * D, WEIGHT_SIGMA).reshape(I, D)
    d = host_normal(seed, sd, D * I, WEIGHT_SIGMA).reshape(D, I)
    return g, u, d


def router_w(seed: int, shape: Shape, layer: int = 0) -> np.ndarray:
    return host_normal(seed, stream(K_ROUTER_W, layer), shape.E * shape.D, WEIGHT_SIGMA).reshape(
        shape.E, shape.D)


def router_b_uniform(seed: int, shape: Shape, layer: int = 0, half_width: float = 0.1) -> np.ndarray:
    return host_uniform(seed, stream(K_ROUTER_B, layer), shape.E, -half_width, half_width)


def activations(seed: int, S: int, D: int, item: int = 0) -> np.ndarray:
    return host_normal(seed, stream(K_X, 0, item), S * D, 1.0).reshape(S, D)


def zipf_probs(seed: int, E: int, s: float = 1.1, layer: int = 0) -> np.ndarray:
    """p_e proportional to rank(e)^-s, ranks assigned by a seeded permutation."""
    u = host_unit_f64(seed, stream(K_PERM, layer), E)
    perm = np.argsort(u, kind="stable")  # perm[r] = expert with rank r+1
    p = np.empty(E, np.float64)
    p[perm] = np.arange(1, E + 1, dtype=np.float64) ** (-s)
    return p / p.sum()


def zipf_activations(seed: int, shape: Shape, S: int, wr: np.ndarray, s: float = 1.1,
                     item: int = 1):
    """Token activations whose router logits are log p_e + Gumbel noise.

    x = z + Wr^T (Wr Wr^T)^-1 (l* - Wr z) with z ~ N(0,1), solved in float64 and
    rounded to float32; l* is centred per token so that sigmoid stays far from
    saturation.  Returns (x [S][D] float32, target logits [S][E] float64, p)."""
    E, D = shape.E, shape.D
    p = zipf_probs(seed, E, s)
    u = host_unit_f64(seed, stream(K_GUMBEL, 0, item), S * E).reshape(S, E)
    g = -np.log(-np.log(u))
    target = np.log(p)[None, :] + g
    target = target - target.mean(axis=1, keepdims=True)
    z = host_normal(seed, stream(K_Z, 0, item), S * D, 1.0).reshape(S, D).astype(np.float64)
    W = wr.astype(np.float64)
    gram = W @ W.T
    resid = target - z @ W.T
    x = z + np.linalg.solve(gram, resid.T).T @ W
    return x.astype(np.float32), target, p


def zipf_bias(seed: int, E: int, layer: int, beta: float, s: float = 1.1) -> np.ndarray:
    """Per-layer correction bias beta * (log p_e - mean) for the layer stack."""
    p = zipf_probs(seed, E, s, layer=layer)
    lp = np.log(p)
    return (beta * (lp - lp.mean())).astype(np.float32)


def fit_zipf_exponent(counts: np.ndarray) -> float:
    """Least-squares slope of log(frequency) against log(rank) over the
    experts hit at least once; returns the Zipf exponent estimate."""
    c = np.sort(np.asarray(counts, np.float64))[::-1]
    c = c[c > 0]
    if len(c) < 3:
        return float("nan")
    r = np.arange(1, len(c) + 1, dtype=np.float64)
    A = np.stack([np.log(r), np.ones_like(r)], axis=1)
    slope = np.linalg.lstsq(A, np.log(c), rcond=None)[0][0]
    return float(-slope)
