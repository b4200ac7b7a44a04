"""Pins of the oracle's packed int2 weight format (the 2-bit path named in
section 12 and the summaries of the reader.mx article "惊呆了！25GB 内存上运行
GLM 5.2 744B 模型"; the byte layout is a reading: the int4 container's rule at
2 bits).  CPU only."""
import numpy as np
import pytest

import oracle
import synth
from oracle.layers import config_of
from ref64 import max_rel_err, quant_rows64


def _unpack_np(q2: np.ndarray, C: int) -> np.ndarray:
    """Independent reader: field k of byte j is column 4j + k, value field - 2."""
    q2 = np.asarray(q2, np.uint8)
    fields = np.stack([(q2 >> (2 * k)) & 3 for k in range(4)], axis=-1)  # [O][rb][4]
    return (fields.reshape(q2.shape[0], -1)[:, :C].astype(np.int64) - 2)


def test_pack_int2_worked_bytes():
    # codes 1 -1 0 1 | 0 0 -1 1 | 1 (pad 0 0 0), stored as code + 2, low bits first
    w = np.array([[1, -1, 0, 1, 0, 0, -1, 1, 1]], np.float32)
    q2, s = oracle.pack_int2(w)
    assert s[0] == 1.0
    assert q2[0].tolist() == [3 | 1 << 2 | 2 << 4 | 3 << 6, 2 | 2 << 2 | 1 << 4 | 3 << 6,
                              3 | 2 << 2 | 2 << 4 | 2 << 6]


@pytest.mark.parametrize("C", [1, 3, 4, 37, 256])
def test_pack_int2_codes_are_the_two_bit_quantizer(C):
    rng = np.random.default_rng(C)
    w = (rng.standard_normal((19, C)) * 0.05).astype(np.float32)
    w[4] = 0.0
    q2, s = oracle.pack_int2(w)
    q, s2 = oracle.quantize_rows(w, 2)
    assert np.array_equal(s, s2)
    assert np.array_equal(_unpack_np(q2, C), q.astype(np.int64))
    assert np.array_equal(oracle.unpack_int2(q2, C).astype(np.int64), q.astype(np.int64))
    # s = amax: every code is -1, 0 or 1 and |w - q s| <= s / 2
    assert set(np.unique(q)).issubset({-1, 0, 1})
    assert np.array_equal(s[np.abs(w).max(axis=1) > 1e-8], np.abs(w).max(axis=1)[np.abs(w).max(axis=1) > 1e-8])
    err = np.abs(q.astype(np.float64) * s[:, None] - w.astype(np.float64))
    assert (err <= s[:, None].astype(np.float64) * (0.5 + 1e-6)).all()


def test_unpack_int2_every_byte():
    b = np.arange(256, dtype=np.uint8)[None, :]
    assert np.array_equal(oracle.unpack_int2(b, 1024).astype(np.int64), _unpack_np(b, 1024))


@pytest.mark.parametrize("shape,S", [(synth.TINY, 4), (synth.Shape(D=512, I=96, E=1, K=1), 3)])
def test_int2_expert_equals_int8_expert_on_widened_codes(shape, S):
    g, u, d = synth.host_expert_f32(7, shape, 0, 2)
    e2 = oracle.HostExpertI2.from_f32(g, u, d)
    wid = lambda q2, C: np.ascontiguousarray(_unpack_np(q2, C).astype(np.int8))
    e8 = oracle.HostExpertI8(wid(e2.gate_q2, shape.D), e2.gate_s, wid(e2.up_q2, shape.D), e2.up_s,
                             wid(e2.down_q2, shape.I), e2.down_s)
    xq, sx = oracle.quant_act_i8(synth.activations(7, S, shape.D))
    cfg = config_of(shape)
    r2 = oracle.expert_swiglu_i2(cfg, xq, sx, e2)
    r8 = oracle.expert_swiglu_i8(cfg, xq, sx, e8)
    for k in ("acc_gu", "hq", "sh", "acc_d", "y"):
        assert np.array_equal(r2[k], r8[k]), k
    xi = xq.astype(np.int64)
    assert np.array_equal(r2["acc_gu"][:, 0], xi @ _unpack_np(e2.gate_q2, shape.D).T)


def test_int2_expert_within_1e3_of_float64_reference():
    shape = synth.Shape(D=1024, I=256, E=1, K=1)
    g, u, d = synth.host_expert_f32(8, shape, 0, 0)
    e = oracle.HostExpertI2.from_f32(g, u, d)
    xq, sx = oracle.quant_act_i8(synth.activations(8, 3, shape.D))
    r = oracle.expert_swiglu_i2(config_of(shape), xq, sx, e)
    W = lambda q2, s, C: _unpack_np(q2, C).astype(np.float64) * s.astype(np.float64)[:, None]
    xd = xq.astype(np.float64) * sx[:, None]
    gg = xd @ W(e.gate_q2, e.gate_s, shape.D).T
    uu = xd @ W(e.up_q2, e.up_s, shape.D).T
    h = gg / (1.0 + np.exp(-gg)) * uu
    q, s = quant_rows64(h)
    y64 = (q * s[:, None]) @ W(e.down_q2, e.down_s, shape.I).T
    assert max_rel_err(r["y"], y64).max() <= 1e-3
