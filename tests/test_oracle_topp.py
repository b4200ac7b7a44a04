"""Pins of the oracle's adaptive expert top-p (keff[s] experts per token,
section 11 union listing; the rule's reading is stated in the oracle
header): closed forms, exact rational brute force, the float64 reference
restricted to the kept experts, and union == per-token."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from oracle.layers import LazyLayer, bias_for
from ref64 import expert64, max_rel_err, quant_rows64, router64

MID = synth.Shape(D=512, I=256, E=64, K=8)


def test_keff_closed_forms():
    k = oracle.expert_keff
    w8 = np.ones(8, np.float32)
    assert k(w8, 0.0) == 8 and k(w8, 1.0) == 8         # off
    assert k(w8, 0.7) == 6                              # ceil(0.7 * 8)
    assert k(w8, 0.125) == 1 and k(w8, 0.126) == 2
    assert k(np.array([4, 2, 1, 1], np.float32), 0.5) == 1   # 4 >= 0.5 * 8
    assert k(np.array([4, 2, 1, 1], np.float32), 0.51) == 2
    assert k(np.array([1, 1, 1, 5], np.float32), 0.5) == 4   # order matters, not size
    assert k(np.array([3.0], np.float32), 0.3) == 1


def brute_keff(w, p):
    """Exact rational arithmetic on the float32 values; None when float32
    rounding could decide differently (a prefix within 1e-6 of the bound)."""
    ws = [Fraction(float(v)) for v in np.asarray(w, np.float32)]
    thr = Fraction(float(np.float32(p))) * sum(ws)
    run = Fraction(0)
    for i, v in enumerate(ws):
        run += v
        if abs(run - thr) <= Fraction(1, 10 ** 6) * sum(ws):
            return None
        if run >= thr:
            return i + 1
    return len(ws)


@pytest.mark.parametrize("seed", range(8))
def test_keff_brute_force(seed):
    rng = np.random.default_rng(seed)
    checked = 0
    for _ in range(200):
        K = int(rng.integers(1, 65))
        w = (rng.random(K) * 2.5).astype(np.float32)
        p = float(rng.choice([0.3, 0.5, 0.7, 0.9, 0.95]))
        ref = brute_keff(w, p)
        if ref is None:
            continue
        assert oracle.expert_keff(w, p) == ref
        checked += 1
    assert checked > 150


def _layer(p, seed=3):
    L = LazyLayer(seed, MID, 0, bias_for("uniform", seed, MID))
    L.cfg.expert_topp = p
    return L


@pytest.mark.parametrize("p", [0.5, 0.7, 0.9])
def test_topp_layer_within_1e3_of_float64_reference(p):
    L = _layer(p)
    x = synth.activations(4, 8, MID.D)
    L.ensure_for(x)
    out = oracle.layer_forward(L, x)
    idx64, w64, cs = router64(x, L.router_w, L.router_b, MID.K, MID.routed_scale)
    q, s = quant_rows64(x)
    xdq = q * s[:, None]
    compared = 0
    for t in range(x.shape[0]):
        keff = brute_keff(w64[t].astype(np.float32), p)
        if keff is None or not cs[t, MID.K - 1] - cs[t, MID.K] > 1e-5:
            continue
        ref = expert64(xdq[t:t + 1], L.shared, MID.D, MID.I)[0].copy()
        for k in range(keff):
            ref += w64[t, k] * expert64(xdq[t:t + 1], L.experts[int(idx64[t, k])], MID.D, MID.I)[0]
        assert max_rel_err(out[t], ref).max() <= 1e-3
        compared += 1
    assert compared >= 6


def test_topp_union_equals_per_token_and_drops_experts():
    L = _layer(0.6)
    x = synth.activations(5, 12, MID.D)
    L.ensure_for(x)
    a = oracle.layer_forward(L, x)
    b, idx, w, uniq = oracle.layer_forward_batch(L, x)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    keff = [oracle.expert_keff(w[s], 0.6) for s in range(x.shape[0])]
    assert max(keff) < MID.K
    kept = []
    for s in range(x.shape[0]):
        for e in idx[s, :keff[s]].tolist():
            if e not in kept:
                kept.append(e)
    assert uniq.tolist() == kept
    # top-p 1 is the full block, bit for bit
    L1 = _layer(1.0)
    L1.ensure_for(x)
    L0 = _layer(0.0)
    L0.ensure_for(x)
    assert np.array_equal(oracle.layer_forward(L1, x).view(np.uint32),
                          oracle.layer_forward(L0, x).view(np.uint32))
