"""Helpers shared by the GPU parity tests: device/oracle layer pairs built from
the same seeds, and comparison rules.

Comparison rules
* integer and byte results (quantized codes, int32 accumulators, packed
  weights, expert indices) must match bit for bit;
* float outputs: max_i |gpu_i - ref_i| / max_i |ref_i| <= 1e-3 per row;
* routing: where the oracle's choice values of a token leave a gap of at
  most NEAR_TIE between any two of its K+1 best experts, several selections
  are correct; there the GPU's selection is checked for validity (its experts
  are all within NEAR_TIE of the K-th best choice, in non-increasing order up
  to NEAR_TIE) and the token's float output is compared with the oracle's
  expert path run on the GPU's routing (oracle_block_ref).  Every token's
  floats are compared.
"""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

import oracle
import synth
from oracle.layers import LazyLayer, bias_for, config_of
from ref64 import max_rel_err

TOL = 1e-3
NEAR_TIE = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def device_layer(seed, shape, layer, router_b, router_w=None):
    from synth.device_layers import build_device_layer
    return build_device_layer(seed, shape, layer, router_b, router_w)


def oracle_layer(seed, shape, layer, router_b, router_w=None):
    return LazyLayer(seed, shape, layer, router_b, router_w)


def routing_unique(choice_ref: np.ndarray, K: int):
    """Per token: (is_unique, oracle order of experts by (choice desc, index asc))."""
    S, E = choice_ref.shape
    uniq = np.zeros(S, bool)
    orders = np.zeros((S, E), np.int64)
    for s in range(S):
        order = np.lexsort((np.arange(E), -choice_ref[s].astype(np.float64)))
        orders[s] = order
        cs = choice_ref[s].astype(np.float64)[order]
        n = min(K + 1, E)
        gaps = cs[: n - 1] - cs[1:n]
        uniq[s] = bool(np.all(gaps > NEAR_TIE))
    return uniq, orders


def check_routing(idx_gpu: np.ndarray, choice_ref: np.ndarray, K: int):
    """Assert the GPU routing is the oracle's where that is unique and valid
    elsewhere; returns the mask of unique tokens."""
    uniq, orders = routing_unique(choice_ref, K)
    for s in range(idx_gpu.shape[0]):
        if uniq[s]:
            assert idx_gpu[s].tolist() == orders[s, :K].tolist(), f"token {s}"
        else:
            c = choice_ref[s].astype(np.float64)
            kth = c[orders[s, K - 1]]
            sel = idx_gpu[s]
            assert len(set(sel.tolist())) == K
            assert np.all(c[sel] >= kth - NEAR_TIE), f"token {s}: invalid near-tie selection"
            assert np.all(c[sel[:-1]] >= c[sel[1:]] - NEAR_TIE)
    return uniq


def _routed_one(L, xs, idx, w, base_row, shared8):
    """The oracle's block for one token on the given routing (len(idx)
    experts), optionally with the int8 shared expert and accumulating."""
    c = L.cfg
    ns = c.n_shared if shared8 is None else 0
    sub = oracle.Config(c.D, c.I, c.E, len(idx), ns, c.routed_scale, 0.0)
    H = oracle.HostLayer(sub, L.router_w, L.router_b, L.experts, L.shared)
    out = oracle.layer_forward_routed(H, xs[None], np.asarray(idx, np.int32)[None],
                                      np.asarray(w, np.float32)[None])[0]
    if shared8 is not None:
        xq, sx = oracle.quant_act_i8(xs[None])
        out = out + oracle.expert_swiglu_i8(c, xq, sx, shared8)["y"][0]
    return out if base_row is None else base_row + out


def _workers():
    # at most 16 worker processes: a process may use a 16-CPU share of the host,
    # whatever os.cpu_count() says
    return max(1, min(16, os.cpu_count() or 1))


def _chunked(fn, n, workers):
    """fn(lo, hi) over [0, n) in chunks on threads (the oracle's C calls run
    outside the interpreter lock; each token's result is independent of the
    others, so the chunking changes no bit)."""
    if workers <= 1 or n < 2:
        fn(0, n)
        return
    from concurrent.futures import ThreadPoolExecutor
    step = (n + workers - 1) // workers
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(lambda lo: fn(lo, min(n, lo + step)), range(0, n, step)))


def oracle_block_ref(L, x, idx_gpu, w_gpu, keff_gpu=None, base=None, shared8=None):
    """Oracle reference rows for the GPU block's outputs on tokens x.

    The GPU routing is checked first (check_routing), and its weights against
    the routed scale times the sigmoid of the oracle's logits of the GPU's
    experts (relative 1e-5: the logits differ by float32 summation order).
    Tokens whose selection is unique (and, with top-p, whose kept count
    equals the oracle rule on the oracle's own weights) get the oracle's whole
    block; the others, where several selections are correct, get the oracle's
    expert path on the GPU's routing: its experts, weights and kept count.
    Returns (ref, unique mask)."""
    cfg = L.cfg
    S, K = idx_gpu.shape
    oidx, ow, logits, choice = oracle.router_topk(cfg, x, L.router_w, L.router_b)
    uniq = check_routing(idx_gpu, choice, K)
    sig = 1.0 / (1.0 + np.exp(-logits.astype(np.float64)))
    want_w = cfg.routed_scale * np.take_along_axis(sig, idx_gpu.astype(np.int64), axis=1)
    np.testing.assert_allclose(w_gpu, want_w, rtol=1e-5, atol=0)
    p = cfg.expert_topp
    if keff_gpu is not None:
        uniq = uniq & np.array([oracle.expert_keff(ow[s], p) == keff_gpu[s] for s in range(S)])
    nw = _workers()
    L.ensure(np.concatenate([oidx.ravel(), idx_gpu.ravel()]), workers=nw)
    flags = 0 if base is None else oracle.ACCUMULATE
    ref = np.zeros((S, cfg.D), np.float32) if base is None else np.array(base, np.float32, copy=True)

    def run(lo, hi):
        if hi <= lo:
            return
        part = ref[lo:hi]  # a view: the oracle writes (or adds) in place
        if shared8 is None:
            oracle.layer_forward(L, x[lo:hi], out=part, flags=flags)
        else:
            oracle.layer_forward_shared_i8(L, shared8, x[lo:hi], out=part, flags=flags)
    _chunked(run, S, nw)
    for s in np.flatnonzero(~uniq):
        ke = K if keff_gpu is None else int(keff_gpu[s])
        ref[s] = _routed_one(L, x[s], idx_gpu[s, :ke], w_gpu[s, :ke],
                             None if base is None else base[s], shared8)
    if (~uniq).any():
        say(f"  {int((~uniq).sum())}/{S} tokens near a routing tie: compared on the GPU's routing")
    return ref, uniq


def assert_close_rows(gpu: np.ndarray, ref: np.ndarray, mask=None, tol=TOL, what=""):
    err = max_rel_err(gpu, ref)
    if mask is not None:
        err = err[mask]
    worst = float(err.max()) if err.size else 0.0
    say(f"  {what}: max rel err {worst:.3e} over {err.size} rows")
    assert worst <= tol, f"{what}: max rel err {worst}"
    return worst


__all__ = ["TOL", "NEAR_TIE", "say", "to_np", "device_layer", "oracle_layer", "check_routing",
           "routing_unique", "assert_close_rows", "oracle_block_ref", "bias_for", "config_of",
           "oracle", "synth"]
