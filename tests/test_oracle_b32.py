"""Pins of the oracle's block-32 activation scales (the summaries' "Q8_0
style" activation format of the reader.mx article "惊呆了！25GB 内存上运行 GLM
5.2 744B 模型"; the block rule is a reading) and the int4 expert on block-32
quantized rows.  CPU only."""
import numpy as np

import oracle
import synth
from oracle.layers import config_of, host_expert
from ref64 import dequant, max_rel_err

TINY = synth.TINY


def test_quant_b32_closed_form_per_block_scales():
    # block b holds m * 2^-(b+3) with max |m| = 127: scale 2^-(b+3), codes m
    rng = np.random.default_rng(1)
    m = rng.integers(-127, 128, size=(1, 128)).astype(np.float32)
    m[0, ::32] = 127
    scale = np.repeat(np.float32(2.0) ** -np.arange(3, 7, dtype=np.float32), 32)[None, :]
    xq, sxb = oracle.quant_act_b32(m * scale)
    assert np.array_equal(sxb[0], np.float32(2.0) ** -np.arange(3, 7, dtype=np.float32))
    assert np.array_equal(xq.astype(np.int64), m.astype(np.int64))


def test_quant_b32_keeps_small_blocks_that_row_scales_crush():
    x = np.zeros((1, 64), np.float32)
    x[0, :32] = 100.0
    x[0, 32:] = np.linspace(-0.1, 0.1, 32, dtype=np.float32)
    xq_row, _ = oracle.quant_act_i8(x)
    xq_b, sxb = oracle.quant_act_b32(x)
    assert not xq_row[0, 32:].any()                 # one row scale: the small block is lost
    assert np.abs(xq_b[0, 32:]).max() == 127         # its own scale keeps it
    assert np.array_equal(xq_b[0, :32], xq_row[0, :32])
    err = np.abs(xq_b.astype(np.float64) * np.repeat(sxb, 32, axis=1) - x)
    assert (err <= np.repeat(sxb, 32, axis=1) * (0.5 + 1e-6)).all()


def test_b32_expert_equals_row_expert_when_blocks_share_the_row_scale():
    # every block of every row has the same absmax, and I = 32 makes the
    # hidden row a single block: block-32 codes and scales are the per-row
    # ones on both projections, so the expert matches the per-row expert up to
    # the order of its float sums
    shape = synth.Shape(D=512, I=32, E=1, K=1)
    e = host_expert(3, shape, 0, 1)
    x = synth.activations(3, 3, shape.D)
    amax = np.abs(x).max(axis=1, keepdims=True)
    x[:, ::32] = amax  # plant the row's absmax in every block
    xq_b, sxb = oracle.quant_act_b32(x)
    xq_r, sxr = oracle.quant_act_i8(x)
    assert np.array_equal(xq_b, xq_r) and np.array_equal(sxb, np.repeat(sxr[:, None], 16, axis=1))
    cfg = config_of(shape)
    rb = oracle.expert_swiglu_b32(cfg, xq_b, sxb, e)
    rr = oracle.expert_swiglu(cfg, xq_r, sxr, e)
    assert np.array_equal(rb["hq"], rr["hq"])
    assert max_rel_err(rb["y"], rr["y"]).max() <= 1e-5


def test_b32_expert_within_1e3_of_float64_reference():
    shape = synth.Shape(D=1024, I=256, E=1, K=1)
    e = host_expert(4, shape, 0, 2)
    x = synth.activations(4, 3, shape.D) * np.repeat(
        np.float32(2.0) ** np.arange(-4, 4, 0.25, dtype=np.float32), 32)[None, :]
    xq, sxb = oracle.quant_act_b32(x)
    r = oracle.expert_swiglu_b32(config_of(shape), xq, sxb, e)
    xd = xq.astype(np.float64) * np.repeat(sxb.astype(np.float64), 32, axis=1)
    g = xd @ dequant(e.gate_q4, e.gate_s, shape.D).T
    u = xd @ dequant(e.up_q4, e.up_s, shape.D).T
    h = g / (1.0 + np.exp(-g)) * u
    hb = h.reshape(3, -1, 32)
    s = np.maximum(np.abs(hb).max(axis=2, keepdims=True) / 127.0, 1e-12)
    hd = (np.clip(np.rint(hb / s), -127, 127) * s).reshape(3, -1)
    y64 = hd @ dequant(e.down_q4, e.down_s, shape.I).T
    assert max_rel_err(r["y"], y64).max() <= 1e-3
    # the requantized hidden codes and block scales match the float64 ones
    assert np.allclose(r["shb"], s[:, :, 0], rtol=1e-5, atol=0)
