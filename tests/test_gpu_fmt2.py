"""GPU parity of the packed int2 weight format against the CPU oracle: the
packer (2-bit quantizer codes, four per byte) and the SwiGLU expert on the
integer path with int2 weights."""
import numpy as np
import pytest
import torch

import int4_expert_gemv_moe_amd as moe
import oracle
import synth
from gpu_util import assert_close_rows, config_of, say, to_np

pytestmark = pytest.mark.gpu

TINY, GLM = synth.TINY, synth.GLM


@pytest.mark.parametrize("O,C", [(7, 256), (2048, 6144), (6144, 2048), (3, 37), (5, 1), (4, 6)])
def test_pack_int2_bit_exact(O, C):
    say(f"pack_int2 O={O} C={C}")
    w = synth.host_normal(2, synth.stream(synth.K_DOWN, 3, 7), O * C, 0.02).reshape(O, C)
    w[0] = 0.0                  # zero row: the 1e-8 floor
    if O > 2:
        w[1] *= np.float32(1e-9)    # amax below the floor
        w[2, 0] = np.float32(0.5)   # a rounding tie once s = 1
        w[2, -1] = np.float32(1.0) if C > 1 else w[2, -1]
        w[2, 1:-1] = np.clip(w[2, 1:-1], -0.1, 0.1)
    q2, s = moe.moe_pack_int2(torch.from_numpy(w).cuda())
    rq2, rs = oracle.pack_int2(w)
    assert np.array_equal(to_np(q2), rq2)
    assert np.array_equal(to_np(s).view(np.uint32), rs.view(np.uint32))


def _device_i2(he: oracle.HostExpertI2, n: int, e_id: int, shape) -> moe.DeviceExpertsI2:
    dev = moe.DeviceExpertsI2.empty(n, shape.D, shape.I)
    for name in ("gate_q2", "gate_s", "up_q2", "up_s", "down_q2", "down_s"):
        getattr(dev, name)[e_id].copy_(torch.from_numpy(getattr(he, name)))
    return dev


@pytest.mark.parametrize("shape,S", [
    (TINY, 4),
    (synth.Shape(D=256, I=64, E=1, K=1), 1),      # smallest shape
    (synth.Shape(D=1280, I=192, E=3, K=1), 3),    # partial chunks in both projections
    (synth.Shape(D=8192, I=1024, E=1, K=1), 2),   # two chunks per gate/up row
    (synth.Shape(D=256, I=8192, E=1, K=1), 2),    # two chunks per down row
    (synth.Shape(D=256, I=8192, E=1, K=1), 6),    # two passes of 4 tokens' hidden codes
    (GLM, 1), (GLM, 3)])
def test_expert_swiglu_i2_parity(shape, S):
    say(f"swiglu_i2 D={shape.D} I={shape.I} S={S}")
    e_id = shape.E - 1
    he = oracle.HostExpertI2.from_f32(*synth.host_expert_f32(5, shape, 0, e_id))
    cfg = moe.config(shape.D, shape.I, shape.E, shape.K)
    dev = _device_i2(he, shape.E, e_id, shape)
    xq, sx = oracle.quant_act_i8(synth.activations(10, S, shape.D))
    ws = moe.Workspace(cfg, S, moe.WS_SWIGLU8)
    r = moe.moe_expert_swiglu_i2(cfg, torch.from_numpy(xq).cuda(), torch.from_numpy(sx).cuda(), dev,
                                 e_id, ws, probes=True)
    torch.cuda.synchronize()
    ref = oracle.expert_swiglu_i2(config_of(shape), xq, sx, he)
    assert np.array_equal(to_np(r["acc_gu"]), ref["acc_gu"])
    hq = to_np(r["hq"])
    mism = hq != ref["hq"]
    say(f"  hq mismatches: {int(mism.sum())} of {hq.size}")
    assert mism.mean() < 1e-3 and np.abs(hq.astype(int) - ref["hq"]).max() <= 1
    assert np.allclose(to_np(r["sh"]), ref["sh"], rtol=1e-6, atol=0)
    acc_d = to_np(r["acc_d"])
    same = ~mism.any(axis=1)
    assert np.array_equal(acc_d[same], ref["acc_d"][same])
    if (~same).any():
        qd = oracle.unpack_int2(he.down_q2, shape.I).astype(np.int64)
        assert np.array_equal(acc_d[~same], hq[~same].astype(np.int64) @ qd.T)
    assert_close_rows(to_np(r["y"]), ref["y"], what="int2 expert y")


def test_int2_path_equals_int8_path_on_widened_codes():
    """The int2 kernels and the int8 kernels on the same codes (widened to one
    byte each) give the same sums, codes and outputs bit for bit."""
    shape = synth.Shape(D=2048, I=512, E=2, K=1)
    e_id = 1
    he = oracle.HostExpertI2.from_f32(*synth.host_expert_f32(6, shape, 0, e_id))
    cfg = moe.config(shape.D, shape.I, shape.E, shape.K)
    xq, sx = oracle.quant_act_i8(synth.activations(12, 3, shape.D))
    xq_d, sx_d = torch.from_numpy(xq).cuda(), torch.from_numpy(sx).cuda()
    ws = moe.Workspace(cfg, 3, moe.WS_SWIGLU8)
    r2 = moe.moe_expert_swiglu_i2(cfg, xq_d, sx_d, _device_i2(he, shape.E, e_id, shape), e_id, ws,
                                  probes=True)
    d8 = moe.DeviceExpertsI8.empty(shape.E, shape.D, shape.I)
    for q2, s, dq, ds, C in ((he.gate_q2, he.gate_s, d8.gate_q, d8.gate_s, shape.D),
                             (he.up_q2, he.up_s, d8.up_q, d8.up_s, shape.D),
                             (he.down_q2, he.down_s, d8.down_q, d8.down_s, shape.I)):
        dq[e_id].copy_(torch.from_numpy(oracle.unpack_int2(q2, C)))
        ds[e_id].copy_(torch.from_numpy(s))
    r8 = moe.moe_expert_swiglu_i8(cfg, xq_d, sx_d, d8, e_id, ws, probes=True)
    torch.cuda.synchronize()
    for k in ("acc_gu", "hq", "sh", "acc_d", "y"):
        assert torch.equal(r2[k], r8[k]), k
