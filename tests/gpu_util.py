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
  to NEAR_TIE) and the token's float output is not compared.
"""
from __future__ import annotations

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


def assert_close_rows(gpu: np.ndarray, ref: np.ndarray, mask=None, tol=TOL, what=""):
    err = max_rel_err(gpu, ref)
    if mask is not None:
        err = err[mask]
    worst = float(err.max()) if err.size else 0.0
    say(f"  {what}: max rel err {worst:.3e} over {err.size} rows")
    assert worst <= tol, f"{what}: max rel err {worst}"
    return worst


__all__ = ["TOL", "NEAR_TIE", "say", "to_np", "device_layer", "oracle_layer", "check_routing",
           "routing_unique", "assert_close_rows", "bias_for", "config_of", "oracle", "synth"]
