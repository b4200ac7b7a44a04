"""Pins of the oracle's int8 weight format: the section 05 per-row quantizer
and the int8 SwiGLU expert on section 12's integer path (reader.mx article
"惊呆了！25GB 内存上运行 GLM 5.2 744B 模型").  CPU only."""
import numpy as np
import pytest

import oracle
import synth
from oracle.layers import config_of
from ref64 import max_rel_err, quant_rows64, unpack64

TINY = synth.TINY


# ---- quantize_rows ------------------------------------------------------------

def test_quantize_rows_closed_form_power_of_two_scale():
    # amax = 127 * 2^-4 gives the scale 2^-4 exactly, and w = m * 2^-4 the code m
    m = np.arange(-127, 128, dtype=np.float32)
    w = (m * np.float32(2.0 ** -4))[None, :]
    q, s = oracle.quantize_rows(w, 8)
    assert s[0] == np.float32(2.0 ** -4)
    assert np.array_equal(q[0].astype(np.int64), m.astype(np.int64))


def test_quantize_rows_rounds_half_to_even():
    step = np.float32(2.0 ** -3)
    halves = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5], np.float32)
    w = np.concatenate([halves, [127.0]]).astype(np.float32)[None, :] * step
    q, s = oracle.quantize_rows(w, 8)
    assert s[0] == step
    assert q[0].tolist() == [0, 2, 2, 0, -2, -2, 126, 127]


def test_quantize_rows_bits4_equals_section06_packer():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((37, 64)) * rng.uniform(0.01, 2.0, size=(37, 1))).astype(np.float32)
    w[5] = 0.0
    q, s = oracle.quantize_rows(w, 4)
    q4, s4 = oracle.pack_int4(w)
    assert np.array_equal(s, s4)
    assert np.array_equal(q.astype(np.int64), unpack64(q4, 64).astype(np.int64))


def test_quantize_rows_zero_row_and_floor():
    w = np.zeros((2, 16), np.float32)
    w[1, 3] = 5e-7  # amax / 127 is below the 1e-8 floor
    q, s = oracle.quantize_rows(w, 8)
    assert s[0] == np.float32(1e-8) and s[1] == np.float32(1e-8)
    assert not q[0].any()
    assert q[1, 3] == 50 and np.count_nonzero(q[1]) == 1


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_quantize_rows_error_bound_and_range(bits):
    rng = np.random.default_rng(bits)
    w = (rng.standard_normal((64, 200)) * 0.05).astype(np.float32)
    q, s = oracle.quantize_rows(w, bits)
    qmax = (1 << (bits - 1)) - 1
    qi = q.astype(np.int64)
    assert qi.max() <= qmax and qi.min() >= -qmax
    # every row reaches qmax in magnitude at its absmax element
    assert np.array_equal(np.abs(qi).max(axis=1), np.full(64, qmax))
    err = np.abs(qi * s[:, None].astype(np.float64) - w.astype(np.float64))
    assert (err <= s[:, None].astype(np.float64) * (0.5 + 1e-6)).all()
    # a float64 quantizer agrees except at exact rounding ties
    q64 = np.clip(np.rint(w.astype(np.float64) / s[:, None].astype(np.float64)), -qmax - 1, qmax)
    assert (q64 != qi).mean() < 1e-3


def test_quantize_rows_rejects_bad_bits():
    w = np.ones((1, 4), np.float32)
    for bits in (1, 9):
        with pytest.raises(ValueError):
            oracle.quantize_rows(w, bits)


# ---- dot and expert -----------------------------------------------------------

@pytest.mark.parametrize("C", [1, 16, 255, 6144])
def test_dot_i8_equals_int64_and_extreme_bound(C):
    rng = np.random.default_rng(C)
    w = rng.integers(-128, 128, size=C).astype(np.int8)
    x = rng.integers(-127, 128, size=C).astype(np.int8)
    assert oracle.dot_i8_i8(w, x) == int((w.astype(np.int64) * x.astype(np.int64)).sum())
    big_w = np.full(C, -128, np.int8)
    big_x = np.full(C, -127, np.int8)
    assert oracle.dot_i8_i8(big_w, big_x) == 128 * 127 * C


def _int4_as_int8(e4, shape):
    """The int4 expert's codes widened to one int8 per value, same scales."""
    wid = lambda q4, C: np.ascontiguousarray(unpack64(q4, C).astype(np.int8))
    return oracle.HostExpertI8(wid(e4.gate_q4, shape.D), e4.gate_s.copy(), wid(e4.up_q4, shape.D),
                               e4.up_s.copy(), wid(e4.down_q4, shape.I), e4.down_s.copy())


@pytest.mark.parametrize("shape,S", [(TINY, 4), (synth.Shape(D=512, I=96, E=1, K=1), 3)])
def test_int8_expert_with_int4_codes_equals_int4_expert(shape, S):
    # int4 codes are int8 values in [-8, 7]: the int8 path must give the int4
    # path's accumulators, hidden codes and outputs bit for bit
    g, u, d = synth.host_expert_f32(4, shape, 0, 1)
    e4 = oracle.HostExpert.from_f32(g, u, d)
    e8 = _int4_as_int8(e4, shape)
    x = synth.activations(4, S, shape.D)
    xq, sx = oracle.quant_act_i8(x)
    cfg = config_of(shape)
    r4 = oracle.expert_swiglu(cfg, xq, sx, e4)
    r8 = oracle.expert_swiglu_i8(cfg, xq, sx, e8)
    for k in ("acc_gu", "hq", "sh", "acc_d", "y"):
        assert np.array_equal(r4[k], r8[k]), k


def _expert64_q8(xdq, e, requant=True):
    W = lambda q, s: q.astype(np.float64) * s.astype(np.float64)[:, None]
    g = xdq @ W(e.gate_q, e.gate_s).T
    u = xdq @ W(e.up_q, e.up_s).T
    h = g / (1.0 + np.exp(-g)) * u
    if requant:
        q, s = quant_rows64(h)
        h = q * s[:, None]
    return h @ W(e.down_q, e.down_s).T


def test_int8_expert_accumulators_and_float64_reference():
    shape = synth.Shape(D=1024, I=256, E=1, K=1)
    g, u, d = synth.host_expert_f32(5, shape, 0, 2)
    e = oracle.HostExpertI8.from_f32(g, u, d)
    x = synth.activations(5, 3, shape.D)
    xq, sx = oracle.quant_act_i8(x)
    r = oracle.expert_swiglu_i8(config_of(shape), xq, sx, e)
    xi = xq.astype(np.int64)
    assert np.array_equal(r["acc_gu"][:, 0], xi @ e.gate_q.astype(np.int64).T)
    assert np.array_equal(r["acc_gu"][:, 1], xi @ e.up_q.astype(np.int64).T)
    assert np.array_equal(r["acc_d"], r["hq"].astype(np.int64) @ e.down_q.astype(np.int64).T)
    y64 = _expert64_q8(xq.astype(np.float64) * sx[:, None], e)
    assert max_rel_err(r["y"], y64).max() <= 1e-3


def test_int8_expert_is_closer_to_float_than_int4():
    # the article keeps quantization-sensitive weights at int8: the int8
    # expert's error against the unquantized float64 expert is well below the
    # int4 expert's
    shape = synth.Shape(D=512, I=128, E=1, K=1)
    g, u, d = synth.host_expert_f32(6, shape, 0, 3)
    x = synth.activations(6, 4, shape.D)
    xq, sx = oracle.quant_act_i8(x)
    cfg = config_of(shape)
    y8 = oracle.expert_swiglu_i8(cfg, xq, sx, oracle.HostExpertI8.from_f32(g, u, d))["y"]
    y4 = oracle.expert_swiglu(cfg, xq, sx, oracle.HostExpert.from_f32(g, u, d))["y"]
    xf = x.astype(np.float64)
    G, U, Dn = (m.astype(np.float64) for m in (g, u, d))
    gg, uu = xf @ G.T, xf @ U.T
    yf = (gg / (1.0 + np.exp(-gg)) * uu) @ Dn.T
    rms = lambda a: np.sqrt((a ** 2).mean())
    assert rms(y8 - yf) < 0.5 * rms(y4 - yf)


def test_layer_with_int8_shared_on_int4_codes_equals_int4_layer():
    # the shared expert's int4 codes widened to int8 (same scales): the
    # layer with the int8 shared expert gives the int4 layer bit for bit,
    # plain and accumulating
    from oracle.layers import LazyLayer
    shape = TINY
    b = synth.router_b_uniform(2, shape, 0)
    layer = LazyLayer(2, shape, 0, b)
    e4 = layer.shared
    shared8 = _int4_as_int8(e4, shape)
    x = synth.activations(2, 5, shape.D)
    layer.ensure(range(shape.E))
    ref = oracle.layer_forward(layer, x)
    got = oracle.layer_forward_shared_i8(layer, shared8, x)
    assert np.array_equal(ref, got)
    base = synth.activations(3, 5, shape.D)
    ref_acc = oracle.layer_forward(layer, x, out=base.copy(), flags=1)
    got_acc = oracle.layer_forward_shared_i8(layer, shared8, x, out=base.copy(), flags=1)
    assert np.array_equal(ref_acc, got_acc)


def test_layer_with_int8_shared_differs_from_int4_by_the_shared_term():
    # a genuinely int8 shared expert changes only the shared term: the
    # difference to the int4 layer is the difference of the two shared
    # experts' outputs on the token's codes (up to float rounding)
    from oracle.layers import LazyLayer
    shape = TINY
    layer = LazyLayer(4, shape, 0, synth.router_b_uniform(4, shape, 0))
    g, u, d = synth.host_expert_f32(4, shape, 0, synth.SHARED)
    shared8 = oracle.HostExpertI8.from_f32(g, u, d)
    x = synth.activations(4, 3, shape.D)
    layer.ensure(range(shape.E))
    diff = oracle.layer_forward_shared_i8(layer, shared8, x) - oracle.layer_forward(layer, x)
    xq, sx = oracle.quant_act_i8(x)
    cfg = config_of(shape)
    want = oracle.expert_swiglu_i8(cfg, xq, sx, shared8)["y"] - oracle.expert_swiglu(cfg, xq, sx, layer.shared)["y"]
    assert np.abs(diff - want).max() <= 1e-5 * max(1.0, np.abs(want).max())


@pytest.mark.parametrize("shape,S,topp", [(TINY, 5, 0.0), (synth.Shape(D=512, I=256, E=64, K=8), 9, 0.0),
                                          (synth.Shape(D=512, I=256, E=64, K=8), 9, 0.6)])
def test_union_with_int8_shared_equals_per_token_and_int4_codes(shape, S, topp):
    """The union path with the int8 shared expert: equal bit for bit to the
    per-token path with it (plain and accumulating, top-p on or off), and on
    the shared expert's int4 codes widened to int8, to the int4 union."""
    from oracle.layers import LazyLayer
    layer = LazyLayer(6, shape, 0, synth.router_b_uniform(6, shape, 0))
    layer.cfg.expert_topp = topp
    g, u, d = synth.host_expert_f32(6, shape, 0, synth.SHARED)
    shared8 = oracle.HostExpertI8.from_f32(g, u, d)
    x = synth.activations(6, S, shape.D)
    layer.ensure_for(x)
    a = oracle.layer_forward_shared_i8(layer, shared8, x)
    b, uniq = oracle.layer_forward_batch_shared_i8(layer, shared8, x)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    _, _, _, u0 = oracle.layer_forward_batch(layer, x)
    assert uniq.tolist() == u0.tolist()
    base = synth.activations(7, S, shape.D)
    a2 = oracle.layer_forward_shared_i8(layer, shared8, x, out=base.copy(), flags=1)
    b2, _ = oracle.layer_forward_batch_shared_i8(layer, shared8, x, out=base.copy(), flags=1)
    assert np.array_equal(a2.view(np.uint32), b2.view(np.uint32))
    w4 = _int4_as_int8(layer.shared, shape)
    c, _ = oracle.layer_forward_batch_shared_i8(layer, w4, x)
    ref, _, _, _ = oracle.layer_forward_batch(layer, x)
    assert np.array_equal(c.view(np.uint32), ref.view(np.uint32))
