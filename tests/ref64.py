"""Float64 dequantized reference for the MoE block (independent of the oracle).

Used to pin the CPU oracle: it recomputes the block as plain dense algebra on
dequantized values (weights q*s, activations q*s_x) with numpy float64 matrix
products, instead of integer dot products with a float epilogue.  Its own
unpacking reads the nibbles with numpy bit operations.  A dropped term, a wrong
sign, a swapped nibble order, a transposed matrix or a misapplied scale in the
oracle shows up as a difference far above the 1e-3 bound.

Definitions follow the reader.mx article "惊呆了！25GB 内存上运行 GLM 5.2 744B
模型": section 11 (router, SwiGLU expert, weighted combine with the routed
scaling factor) and section 12 (int8 activation quantization before every
integer matmul, including the down projection).
"""
from __future__ import annotations

import numpy as np


def unpack64(q4: np.ndarray, C: int) -> np.ndarray:
    """Nibble-packed rows -> float64 integer values in [-8, 7]."""
    q4 = np.asarray(q4, np.uint8)
    lo = (q4 & 0x0F).astype(np.int64) - 8
    hi = (q4 >> 4).astype(np.int64) - 8
    out = np.empty((q4.shape[0], 2 * q4.shape[1]), np.int64)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out[:, :C].astype(np.float64)


def dequant(q4, scale, C) -> np.ndarray:
    return unpack64(q4, C) * np.asarray(scale, np.float64)[:, None]


def quant_rows64(x: np.ndarray):
    """Per-row int8 quantization evaluated in float64 (rounding half to even)."""
    x = np.asarray(x, np.float64)
    amax = np.abs(x).max(axis=1)
    s = np.maximum(amax / 127.0, 1e-12)
    q = np.clip(np.rint(x / s[:, None]), -127, 127)
    return q, s


def expert64(xdq: np.ndarray, e, D: int, I: int, requant: bool = True) -> np.ndarray:
    """SwiGLU expert on dequantized activations xdq [S][D] (float64)."""
    Wg = dequant(e.gate_q4, e.gate_s, D)
    Wu = dequant(e.up_q4, e.up_s, D)
    Wd = dequant(e.down_q4, e.down_s, I)
    g = xdq @ Wg.T
    u = xdq @ Wu.T
    h = g / (1.0 + np.exp(-g)) * u
    if requant:
        q, s = quant_rows64(h)
        h = q * s[:, None]
    return h @ Wd.T


def router64(x: np.ndarray, wr: np.ndarray, b: np.ndarray, K: int, scale: float):
    """Sigmoid router in float64: returns (idx [S][K], w [S][K], sorted choice [S][E])."""
    logits = np.asarray(x, np.float64) @ np.asarray(wr, np.float64).T
    sig = 1.0 / (1.0 + np.exp(-logits))
    c = sig + np.asarray(b, np.float64)[None, :]
    E = c.shape[1]
    # sort by (choice descending, expert ascending); lexsort's last key is primary
    order = np.stack([np.lexsort((np.arange(E), -c[s])) for s in range(c.shape[0])])
    idx = order[:, :K]
    w = np.take_along_axis(sig, idx, axis=1) * scale
    csorted = np.take_along_axis(c, order, axis=1)
    return idx, w, csorted


def layer64(x: np.ndarray, wr, b, experts: dict, shared, D: int, I: int, K: int, scale: float,
            quant: bool = True):
    """The block in float64 for tokens x [S][D]; returns (out, idx, sorted choice)."""
    x = np.asarray(x, np.float64)
    idx, w, csorted = router64(x, wr, b, K, scale)
    if quant:
        q, s = quant_rows64(x)
        xdq = q * s[:, None]
    else:
        xdq = x
    out = np.zeros((x.shape[0], D), np.float64)
    for t in range(x.shape[0]):
        for k in range(K):
            out[t] += w[t, k] * expert64(xdq[t:t + 1], experts[int(idx[t, k])], D, I, quant)[0]
        if shared is not None:
            out[t] += expert64(xdq[t:t + 1], shared, D, I, quant)[0]
    return out, idx, csorted


def max_rel_err(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Per-row max |a-b| / max |b|."""
    a = np.atleast_2d(np.asarray(a, np.float64))
    b = np.atleast_2d(np.asarray(b, np.float64))
    den = np.maximum(np.abs(b).max(axis=1), 1e-30)
    return np.abs(a - b).max(axis=1) / den
