"""Pins of the oracle's sigmoid router with correction-bias top-K (section 11 of
the reader.mx article "惊呆了！25GB 内存上运行 GLM 5.2 744B 模型").  CPU only."""
import ctypes
import itertools

import numpy as np

import oracle
import synth
from ref64 import router64

TINY = synth.TINY


def _cfg(shape=TINY, K=None, E=None):
    return oracle.make_config(shape.D, shape.I, E or shape.E, K or shape.K, shape.n_shared,
                              shape.routed_scale)


def test_logits_and_weights_match_float64():
    wr = synth.router_w(0, TINY)
    b = synth.router_b_uniform(0, TINY)
    x = synth.activations(0, 64, TINY.D)
    idx, w, logits, choice = oracle.router_topk(_cfg(), x, wr, b)
    l64 = x.astype(np.float64) @ wr.astype(np.float64).T
    assert np.allclose(logits, l64, rtol=0, atol=1e-6 * np.abs(l64).max())
    sig64 = 1.0 / (1.0 + np.exp(-logits.astype(np.float64)))
    assert np.allclose(choice, sig64 + b, rtol=0, atol=3e-7)
    # weight = routed_scale * sigmoid(logit) of the chosen expert, no renormalization
    want = 2.5 * np.take_along_axis(sig64, idx.astype(np.int64), axis=1)
    assert np.allclose(w, want, rtol=3e-7, atol=0)


def test_topk_equals_sort_by_choice_then_index():
    wr = synth.router_w(1, TINY)
    b = synth.router_b_uniform(1, TINY)
    x = synth.activations(1, 200, TINY.D)
    for K in (1, 2, 5, 8):
        idx, _, _, choice = oracle.router_topk(_cfg(K=K), x, wr, b)
        for s in range(x.shape[0]):
            order = sorted(range(TINY.E), key=lambda e: (-float(choice[s, e]), e))
            assert idx[s].tolist() == order[:K]


def test_tiny_pairs_brute_force():
    # with K=2 of 8 experts, the chosen pair must maximize the smaller choice
    # over all 28 pairs, and slot 0 holds the larger member
    wr = synth.router_w(2, TINY)
    b = synth.router_b_uniform(2, TINY)
    x = synth.activations(2, 50, TINY.D)
    idx, _, _, choice = oracle.router_topk(_cfg(), x, wr, b)
    for s in range(50):
        c = choice[s].astype(np.float64)
        best = max(itertools.combinations(range(8), 2), key=lambda p: (min(c[p[0]], c[p[1]]), -min(p)))
        assert set(idx[s].tolist()) == set(best)
        assert c[idx[s, 0]] >= c[idx[s, 1]]


def test_zero_bias_selects_largest_logits():
    # sigmoid is monotone, so with b = 0 the top-K of sigmoid is the top-K of
    # the logits computed independently in float64
    shape = synth.Shape(D=512, I=64, E=64, K=8)
    wr = synth.router_w(3, shape)
    b = np.zeros(shape.E, np.float32)
    x = synth.activations(3, 40, shape.D)
    idx, _, _, _ = oracle.router_topk(_cfg(shape), x, wr, b)
    idx64, _, cs = router64(x, wr, b, shape.K, 2.5)
    gaps = cs[:, shape.K - 1] - cs[:, shape.K]
    ok = gaps > 1e-5
    assert ok.sum() >= 35
    assert np.array_equal(idx[ok], idx64[ok])


def test_bias_changes_selection_but_not_weights():
    # the bias only picks experts; weights use the unbiased sigmoid
    wr = synth.router_w(4, TINY)
    x = synth.activations(4, 8, TINY.D)
    b = np.zeros(TINY.E, np.float32)
    b[7] = 0.9  # pushes expert 7 into every selection
    idx, w, logits, _ = oracle.router_topk(_cfg(), x, wr, b)
    assert np.all((idx == 7).any(axis=1))
    sig = 1.0 / (1.0 + np.exp(-logits.astype(np.float64)))
    assert np.allclose(w, 2.5 * np.take_along_axis(sig, idx.astype(np.int64), axis=1), rtol=3e-7)


def test_exact_ties_go_to_lowest_index():
    wr = synth.router_w(5, TINY).copy()
    wr[5] = wr[3]
    wr[6] = wr[3]
    b = np.zeros(TINY.E, np.float32)
    b[3] = b[5] = b[6] = 0.5
    x = synth.activations(5, 4, TINY.D)
    idx, _, _, _ = oracle.router_topk(_cfg(), x, wr, b)
    assert np.all(idx[:, 0] == 3) and np.all(idx[:, 1] == 5)


def test_nan_and_excluded_candidates():
    wr = synth.router_w(6, TINY)
    b = np.zeros(TINY.E, np.float32)
    x = np.full((1, TINY.D), np.nan, np.float32)
    idx, w, _, _ = oracle.router_topk(_cfg(), x, wr, b)
    assert idx[0].tolist() == [0, 1]  # no candidate: lowest untaken experts
    b2 = np.full(TINY.E, -1e31, np.float32)
    b2[6] = 0.0
    x2 = synth.activations(6, 1, TINY.D)
    idx2, _, _, _ = oracle.router_topk(_cfg(), x2, wr, b2)
    assert idx2[0].tolist() == [6, 0]


def test_rejects_bad_config():
    lib = oracle.lib()
    cfg = oracle.make_config(TINY.D, TINY.I, 4, 5)  # K > E
    z = np.zeros(4096, np.float32)
    i = np.zeros(64, np.int32)
    assert lib.moe_ref_router_topk(ctypes.byref(cfg), z.ctypes.data, 1, z.ctypes.data,
                                   z.ctypes.data, i.ctypes.data, z.ctypes.data, None, None) != 0
