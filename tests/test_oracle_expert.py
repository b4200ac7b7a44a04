"""Pins of the oracle's integer dot products and SwiGLU expert (sections 11
and 12 of the reader.mx article "惊呆了！25GB 内存上运行 GLM 5.2 744B 模型").
CPU only."""
import numpy as np
import pytest

import oracle
import synth
from oracle.layers import config_of, host_expert
from ref64 import expert64, max_rel_err, quant_rows64, unpack64

TINY = synth.TINY


@pytest.mark.parametrize("C", [1, 2, 7, 64, 6144])
def test_dot_equals_int64_loop(C):
    rng = np.random.default_rng(C)
    q4 = rng.integers(0, 256, size=(1, (C + 1) // 2), dtype=np.uint8)
    x = rng.integers(-127, 128, size=C).astype(np.int8)
    want = int((unpack64(q4, C)[0].astype(np.int64) * x.astype(np.int64)).sum())
    assert oracle.dot_i4_i8(q4[0], x) == want


def test_dot_extreme_bound_is_exact():
    # all weights -8 and all activations -127 reach the bound 8*127*6144
    q4 = np.zeros(3072, np.uint8)
    x = np.full(6144, -127, np.int8)
    assert oracle.dot_i4_i8(q4, x) == 8 * 127 * 6144 == 6_242_304


def test_expert_accumulators_equal_integer_matmul():
    e = host_expert(0, TINY, 0, 3)
    x = synth.activations(0, 4, TINY.D)
    xq, sx = oracle.quant_act_i8(x)
    r = oracle.expert_swiglu(config_of(TINY), xq, sx, e)
    xi = xq.astype(np.int64)
    assert np.array_equal(r["acc_gu"][:, 0], xi @ unpack64(e.gate_q4, TINY.D).astype(np.int64).T)
    assert np.array_equal(r["acc_gu"][:, 1], xi @ unpack64(e.up_q4, TINY.D).astype(np.int64).T)
    hi = r["hq"].astype(np.int64)
    assert np.array_equal(r["acc_d"], hi @ unpack64(e.down_q4, TINY.I).astype(np.int64).T)


def test_gate_up_lossless_special_case():
    # power-of-two row scales and x = m * 2^-j with max |m| = 127: the integer
    # path times its scales equals the float64 matrix-vector product exactly
    rng = np.random.default_rng(7)
    D, I = 256, 128
    shape = synth.Shape(D=D, I=I, E=1, K=1)
    qg = rng.integers(-7, 8, size=(I, D)).astype(np.float32)
    qg[:, 0] = 7
    qu = rng.integers(-7, 8, size=(I, D)).astype(np.float32)
    qu[:, 1] = -7
    sg = np.float32(2.0) ** -rng.integers(3, 9, size=I).astype(np.float32)
    su = np.float32(2.0) ** -rng.integers(3, 9, size=I).astype(np.float32)
    wg, wu = qg * sg[:, None], qu * su[:, None]
    wd = (rng.standard_normal((D, I)) * 0.02).astype(np.float32)
    e = oracle.HostExpert.from_f32(wg, wu, wd)
    m = rng.integers(-127, 128, size=(3, D)).astype(np.float32)
    m[:, 9] = 127
    x = m * np.float32(2.0 ** -5)
    xq, sx = oracle.quant_act_i8(x)
    r = oracle.expert_swiglu(config_of(shape), xq, sx, e)
    g = r["acc_gu"][:, 0].astype(np.float64) * e.gate_s[None, :] * sx[:, None]
    u = r["acc_gu"][:, 1].astype(np.float64) * e.up_s[None, :] * sx[:, None]
    assert np.array_equal(g, x.astype(np.float64) @ wg.astype(np.float64).T)
    assert np.array_equal(u, x.astype(np.float64) @ wu.astype(np.float64).T)


@pytest.mark.parametrize("shape,S", [(TINY, 4), (synth.Shape(D=1024, I=512, E=1, K=1), 3)])
def test_expert_within_1e3_of_float64_reference(shape, S):
    e = host_expert(1, shape, 0, 0)
    x = synth.activations(1, S, shape.D)
    xq, sx = oracle.quant_act_i8(x)
    r = oracle.expert_swiglu(config_of(shape), xq, sx, e)
    y64 = expert64(xq.astype(np.float64) * sx[:, None], e, shape.D, shape.I)
    assert max_rel_err(r["y"], y64).max() <= 1e-3


@pytest.mark.slow
def test_glm_expert_within_1e3_of_float64_reference():
    e = host_expert(0, synth.GLM, 0, 17)
    x = synth.activations(9, 2, synth.GLM.D)
    xq, sx = oracle.quant_act_i8(x)
    r = oracle.expert_swiglu(config_of(synth.GLM), xq, sx, e)
    y64 = expert64(xq.astype(np.float64) * sx[:, None], e, synth.GLM.D, synth.GLM.I)
    assert max_rel_err(r["y"], y64).max() <= 1e-3
    assert np.abs(r["acc_gu"]).max() <= 6_242_304


def test_requantized_hidden_matches_float64_hidden():
    e = host_expert(2, TINY, 0, 5)
    x = synth.activations(2, 4, TINY.D)
    xq, sx = oracle.quant_act_i8(x)
    r = oracle.expert_swiglu(config_of(TINY), xq, sx, e)
    xdq = xq.astype(np.float64) * sx[:, None]
    from ref64 import dequant
    g = xdq @ dequant(e.gate_q4, e.gate_s, TINY.D).T
    u = xdq @ dequant(e.up_q4, e.up_s, TINY.D).T
    h = g / (1.0 + np.exp(-g)) * u
    q64, s64 = quant_rows64(h)
    assert np.allclose(r["sh"], s64, rtol=1e-6, atol=0)
    # element-wise the codes agree except where h/s sits within rounding of a .5
    assert (r["hq"].astype(np.int64) != q64).mean() < 1e-2
    assert np.abs(r["hq"].astype(np.int64) - q64).max() <= 1


def test_quantization_noise_is_small():
    # the section 12 remark: int8 activations add a fraction of a percent of
    # RMS noise; the unquantized float64 expert is informational only
    e = host_expert(3, TINY, 0, 2)
    x = synth.activations(3, 4, TINY.D)
    xq, sx = oracle.quant_act_i8(x)
    r = oracle.expert_swiglu(config_of(TINY), xq, sx, e)
    y_noq = expert64(x.astype(np.float64), e, TINY.D, TINY.I, requant=False)
    rel = np.sqrt(((r["y"] - y_noq) ** 2).mean()) / np.sqrt((y_noq ** 2).mean())
    assert rel < 0.05
