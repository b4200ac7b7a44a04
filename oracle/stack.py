"""Oracle side of the 48-layer stack recipe.

TEST INFRASTRUCTURE ONLY.  The stack applies, per layer, RMSNorm (section 04
of the reader.mx article "惊呆了！25GB 内存上运行 GLM 5.2 744B 模型") and the
MoE block with a residual add: x <- x + block(rmsnorm(x)).  Its routing is
skewed by a per-layer correction bias beta * (log p_e - mean), p_e a Zipf
law over a per-layer permutation of the experts (synth.zipf_bias); this
module picks beta, using the selection rule of section 11 on synthetic
logits, so that the realized rank-frequency slope is close to -s.
"""
from __future__ import annotations

import math

import numpy as np

import synth

from . import layer_forward, rmsnorm


def calibrate_stack_beta(seed: int, E: int = 256, K: int = 8, s: float = 1.1,
                         logit_sd: float = 0.02 * math.sqrt(6144), tokens: int = 4096):
    """Beta for which top-K selections over c = sigmoid(l) + beta*(log p - mean),
    l ~ N(0, logit_sd^2) independently per token (the logit spread of an RMS-1
    token against N(0, 0.02) router rows), have a rank-frequency slope closest
    to -s.  Returns (beta, fitted exponent)."""
    p = synth.zipf_probs(seed, E, s, layer=0)
    lp = np.log(p) - np.log(p).mean()
    rng_l = synth.host_normal(seed, synth.stream(synth.K_Z, 0xFFF0), tokens * E,
                              logit_sd).reshape(tokens, E)
    sig = 1.0 / (1.0 + np.exp(-rng_l.astype(np.float64)))
    best, best_err, best_fit = 0.0, float("inf"), float("nan")
    for beta in np.linspace(0.0, 0.5, 101):
        c = sig + beta * lp[None, :]
        top = np.argpartition(-c, K - 1, axis=1)[:, :K]
        counts = np.bincount(top.ravel(), minlength=E)
        fit = synth.fit_zipf_exponent(counts)
        if abs(fit - s) < best_err:
            best, best_err, best_fit = float(beta), abs(fit - s), fit
    return best, best_fit


def stack_layer(layer, x: np.ndarray, gamma: np.ndarray, eps: float = 1e-5) -> np.ndarray:
    """One layer of the stack on the residual stream x [S][D]: x + block(rmsnorm(x))."""
    xn = rmsnorm(x, gamma, eps)
    return x + layer_forward(layer, xn)
