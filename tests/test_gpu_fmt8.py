"""GPU parity of the int8 weight format against the CPU oracle: the section 05
per-row quantizer and the SwiGLU expert on section 12's integer path with
int8 weights (reader.mx article "惊呆了！25GB 内存上运行 GLM 5.2 744B 模型")."""
import numpy as np
import pytest
import torch

import int4_expert_gemv_moe_amd as moe
import oracle
import synth
from gpu_util import assert_close_rows, config_of, say, to_np
from ref64 import unpack64

pytestmark = pytest.mark.gpu

TINY, GLM = synth.TINY, synth.GLM


@pytest.mark.parametrize("O,C", [(7, 256), (64, 6144), (2048, 6144), (6144, 2048), (3, 37), (5, 1)])
def test_quantize_rows_i8_bit_exact(O, C):
    say(f"quantize_rows_i8 O={O} C={C}")
    w = synth.host_normal(1, synth.stream(synth.K_UP, 3, 7), O * C, 0.02).reshape(O, C)
    w[0] = 0.0                 # zero row: the 1e-8 floor
    if O > 2:
        w[1] *= np.float32(1e-6)   # amax/127 below the floor
        w[2, 0] = np.float32(0.5 * 127 * 2.0 ** -6)  # a rounding tie once s = 2^-6
        w[2, 1:] = np.clip(w[2, 1:], -0.1, 0.1)
        w[2, -1] = np.float32(127 * 2.0 ** -6) if C > 1 else w[2, -1]
    q, s = moe.moe_quantize_rows_i8(torch.from_numpy(w).cuda())
    rq, rs = oracle.quantize_rows(w, 8)
    assert np.array_equal(to_np(q), rq)
    assert np.array_equal(to_np(s).view(np.uint32), rs.view(np.uint32))


def _device_i8(he: oracle.HostExpertI8, n: int, e_id: int, shape) -> moe.DeviceExpertsI8:
    dev = moe.DeviceExpertsI8.empty(n, shape.D, shape.I)
    for name in ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s"):
        getattr(dev, name)[e_id].copy_(torch.from_numpy(getattr(he, name)))
    return dev


def _run(shape, S, he, e_id, seed=9):
    cfg = moe.config(shape.D, shape.I, shape.E, shape.K)
    dev = _device_i8(he, shape.E, e_id, shape)
    x = synth.activations(seed, S, shape.D)
    xq, sx = oracle.quant_act_i8(x)
    ws = moe.Workspace(cfg, S, moe.WS_SWIGLU8)
    r = moe.moe_expert_swiglu_i8(cfg, torch.from_numpy(xq).cuda(), torch.from_numpy(sx).cuda(), dev,
                                 e_id, ws, probes=True)
    torch.cuda.synchronize()
    return r, xq, sx


@pytest.mark.parametrize("shape,S", [
    (TINY, 4),
    (synth.Shape(D=256, I=32, E=1, K=1), 1),      # smallest shape
    (synth.Shape(D=1280, I=96, E=3, K=1), 3),     # ragged chunks in both projections
    (synth.Shape(D=8192, I=1024, E=1, K=1), 2),   # widest rows of gate/up
    (synth.Shape(D=256, I=8192, E=1, K=1), 2),    # widest rows of down
    (synth.Shape(D=256, I=8192, E=1, K=1), 6),    # two passes of 4 tokens' hidden codes
    (GLM, 1), (GLM, 3)])
def test_expert_swiglu_i8_parity(shape, S):
    say(f"swiglu_i8 D={shape.D} I={shape.I} S={S}")
    e_id = shape.E - 1
    he = oracle.HostExpertI8.from_f32(*synth.host_expert_f32(4, shape, 0, e_id))
    r, xq, sx = _run(shape, S, he, e_id)
    ref = oracle.expert_swiglu_i8(config_of(shape), xq, sx, he)
    assert np.array_equal(to_np(r["acc_gu"]), ref["acc_gu"])
    hq = to_np(r["hq"])
    mism = hq != ref["hq"]
    say(f"  hq mismatches: {int(mism.sum())} of {hq.size}")
    # h goes through expf on both sides; a code may sit one step away at a
    # rounding tie of h / sh
    assert mism.mean() < 1e-3 and np.abs(hq.astype(int) - ref["hq"]).max() <= 1
    assert np.allclose(to_np(r["sh"]), ref["sh"], rtol=1e-6, atol=0)
    acc_d = to_np(r["acc_d"])
    same = ~mism.any(axis=1)
    assert np.array_equal(acc_d[same], ref["acc_d"][same])
    if (~same).any():
        assert np.array_equal(acc_d[~same], hq[~same].astype(np.int64) @ he.down_q.astype(np.int64).T)
    assert_close_rows(to_np(r["y"]), ref["y"], what="int8 expert y")


def test_int8_path_on_int4_codes_equals_int4_path():
    """int4 codes widened to int8 (same scales) through the int8 kernels give
    the int4 kernels' integer sums, codes and outputs bit for bit."""
    shape = synth.Shape(D=2048, I=512, E=2, K=1)
    e_id = 1
    g, u, d = synth.host_expert_f32(5, shape, 0, e_id)
    h4 = oracle.HostExpert.from_f32(g, u, d)
    wid = lambda q4, C: np.ascontiguousarray(unpack64(q4, C).astype(np.int8))
    h8 = oracle.HostExpertI8(wid(h4.gate_q4, shape.D), h4.gate_s, wid(h4.up_q4, shape.D), h4.up_s,
                             wid(h4.down_q4, shape.I), h4.down_s)
    r8, xq, sx = _run(shape, 3, h8, e_id, seed=11)
    cfg = moe.config(shape.D, shape.I, shape.E, shape.K)
    dev4 = moe.DeviceExperts.empty(shape.E, shape.D, shape.I)
    for name in ("gate_q4", "gate_s", "up_q4", "up_s", "down_q4", "down_s"):
        getattr(dev4, name)[e_id].copy_(torch.from_numpy(getattr(h4, name)))
    ws = moe.Workspace(cfg, 3, moe.WS_SWIGLU)
    r4 = moe.moe_expert_swiglu_i4(cfg, torch.from_numpy(xq).cuda(), torch.from_numpy(sx).cuda(), dev4,
                                  e_id, ws, probes=True)
    torch.cuda.synchronize()
    for k in ("acc_gu", "hq", "sh", "acc_d", "y"):
        assert torch.equal(r8[k], r4[k]), k


def test_expert_swiglu_i8_repeated_calls_and_smaller_batch():
    """Two calls on one workspace, the second with fewer tokens, each equal to
    a fresh single call (nothing carries over in the workspace)."""
    shape = synth.Shape(D=1024, I=256, E=2, K=1)
    he = oracle.HostExpertI8.from_f32(*synth.host_expert_f32(6, shape, 0, 0))
    cfg = moe.config(shape.D, shape.I, shape.E, shape.K)
    dev = _device_i8(he, shape.E, 0, shape)
    ws = moe.Workspace(cfg, 5, moe.WS_SWIGLU8)
    outs = []
    for S, seed in ((5, 1), (2, 2)):
        xq, sx = oracle.quant_act_i8(synth.activations(seed, S, shape.D))
        r = moe.moe_expert_swiglu_i8(cfg, torch.from_numpy(xq).cuda(), torch.from_numpy(sx).cuda(),
                                     dev, 0, ws)
        torch.cuda.synchronize()
        ref = oracle.expert_swiglu_i8(config_of(shape), xq, sx, he)
        assert_close_rows(to_np(r["y"]), ref["y"], what=f"S={S}")
        outs.append(r["y"])
    assert outs[1].shape == (2, shape.D)
