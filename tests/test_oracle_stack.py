"""The 48-layer stack recipe on the CPU: the stored bias strength is what the
calibration gives, it does skew the selections toward a Zipf law, and one
stack layer is x + block(rmsnorm(x))."""
import json
import os

import numpy as np

import oracle
import synth
from oracle.layers import LazyLayer
from oracle.stack import calibrate_stack_beta, stack_layer

HERE = os.path.dirname(os.path.abspath(__file__))


def test_stored_beta_is_the_calibration_result():
    with open(os.path.join(HERE, "golden", "stack_beta.json")) as f:
        g = json.load(f)
    beta, fit = calibrate_stack_beta(g["seed"])
    assert beta == g["beta"]
    assert abs(fit - g["fitted_exponent"]) < 1e-3
    assert abs(fit - g["target_exponent"]) < 0.15


def test_zipf_bias_skews_selection():
    """With the stored beta, synthetic RMS-1 tokens against the real router
    select the experts of low Zipf rank far more often than uniform routing."""
    shape = synth.Shape(D=2048, I=128, E=256, K=8)
    with open(os.path.join(HERE, "golden", "stack_beta.json")) as f:
        beta = json.load(f)["beta"]
    b = synth.zipf_bias(0, shape.E, 3, beta)
    wr = synth.router_w(0, shape, 3)
    x = synth.activations(1, 512, shape.D)
    cfg = oracle.layers.config_of(shape)
    idx, _, _, _ = oracle.router_topk(cfg, x, wr, b)
    counts = np.bincount(idx.ravel(), minlength=shape.E)
    p = synth.zipf_probs(0, shape.E, 1.1, layer=3)
    top16 = np.argsort(-p)[:16]
    share = counts[top16].sum() / counts.sum()
    assert share > 3 * 16 / shape.E, share  # uniform routing would give 1/16


def test_stack_layer_definition():
    shape = synth.Shape(D=256, I=128, E=8, K=2)
    L = LazyLayer(0, shape, 0, synth.zipf_bias(0, shape.E, 0, 0.035))
    L.ensure(range(shape.E))
    x = synth.activations(2, 3, shape.D)
    gamma = np.ones(shape.D, np.float32)
    y = stack_layer(L, x, gamma)
    xn = oracle.rmsnorm(x, gamma, 1e-5)
    assert np.array_equal(y, x + oracle.layer_forward(L, xn))
    # accumulate flag of the block gives the same residual update
    acc = x.copy()
    oracle.layer_forward(L, xn, out=acc, flags=1)
    assert np.array_equal(acc.view(np.uint32), y.view(np.uint32))
