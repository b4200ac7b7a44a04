"""Pins of the oracle's per-row int8 activation quantization (section 12 of the
reader.mx article "惊呆了！25GB 内存上运行 GLM 5.2 744B 模型").  CPU only."""
import numpy as np

import oracle
import synth


def test_lossless_special_case():
    # x = m * 2^-j with integer m, max |m| = 127: s = 2^-j exactly and q = m
    rng = np.random.default_rng(5)
    m = rng.integers(-127, 128, size=(7, 333)).astype(np.float32)
    m[:, 17] = 127
    m[1::2, 17] = -127
    for j in (0, 4, 20):
        x = m * np.float32(2.0 ** -j)
        xq, sx = oracle.quant_act_i8(x)
        assert np.all(sx == np.float32(2.0 ** -j))
        assert np.array_equal(xq, m.astype(np.int8))


def test_argmax_maps_to_127_and_error_bound():
    x = synth.activations(0, 16, 6144)
    xq, sx = oracle.quant_act_i8(x)
    am = np.abs(x).argmax(axis=1)
    assert np.all(np.abs(xq[np.arange(16), am].astype(int)) == 127)
    assert np.all(np.sign(xq[np.arange(16), am]) == np.sign(x[np.arange(16), am]))
    err = np.abs(xq.astype(np.float64) - x / sx[:, None].astype(np.float64))
    assert err.max() <= 0.5 + 1e-5
    assert np.abs(xq.astype(int)).max() <= 127


def test_zero_row_and_floor():
    xq, sx = oracle.quant_act_i8(np.zeros((2, 64), np.float32))
    assert np.all(sx == np.float32(1e-12)) and not xq.any()
    tiny = np.full((1, 8), 1e-11, np.float32)  # amax/127 < 1e-12 -> floor applies
    xq, sx = oracle.quant_act_i8(tiny)
    assert sx[0] == np.float32(1e-12)
    assert np.all(xq == 10)


def test_half_way_values_round_to_even():
    x = np.array([[127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5]], np.float32)
    xq, sx = oracle.quant_act_i8(x)
    assert sx[0] == 1.0
    assert xq[0].tolist() == [127, 0, 2, 2, 0, -2, -2, 126]


def test_bf16_input_is_widened_exactly():
    x = synth.activations(1, 8, 512)
    bits = synth.bf16_bits(x)
    xq_b, sx_b = oracle.quant_act_i8_bf16(bits)
    xq_f, sx_f = oracle.quant_act_i8(synth.bf16_to_f32(bits))
    assert np.array_equal(xq_b, xq_f) and np.array_equal(sx_b, sx_f)


def test_row_independence():
    x = synth.activations(2, 9, 256)
    xq, sx = oracle.quant_act_i8(x)
    for s in range(9):
        q1, s1 = oracle.quant_act_i8(x[s:s + 1])
        assert np.array_equal(q1[0], xq[s]) and s1[0] == sx[s]
