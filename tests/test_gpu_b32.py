"""GPU parity of the block-32 activation scales against the CPU oracle: the
block quantizer and the int4 SwiGLU expert on block-quantized rows."""
import numpy as np
import pytest
import torch

import int4_expert_gemv_moe_amd as moe
import oracle
import synth
from gpu_util import assert_close_rows, config_of, say, to_np
from oracle.layers import host_expert

pytestmark = pytest.mark.gpu

TINY, GLM = synth.TINY, synth.GLM


def _tokens(seed, S, D):
    """Activations whose 32-blocks span a 2^8 range of magnitudes, one block zero."""
    x = synth.activations(seed, S, D)
    nb = D // 32
    x *= np.repeat(np.float32(2.0) ** ((np.arange(nb) % 32) / 4.0 - 4.0), 32)[None, :].astype(np.float32)
    if nb > 1:
        x[0, 32:64] = 0.0
    return np.ascontiguousarray(x, np.float32)


@pytest.mark.parametrize("S,D", [(3, 6144), (1, 32), (5, 96), (2, 8192)])
def test_quant_act_b32_bit_exact(S, D):
    say(f"quant_b32 S={S} D={D}")
    x = _tokens(1, S, D)
    xq, sxb = moe.moe_quant_act_b32(torch.from_numpy(x).cuda())
    rq, rs = oracle.quant_act_b32(x)
    assert np.array_equal(to_np(xq), rq)
    assert np.array_equal(to_np(sxb).view(np.uint32), rs.view(np.uint32))


@pytest.mark.parametrize("shape,S", [
    (TINY, 4),
    (synth.Shape(D=256, I=32, E=1, K=1), 1),      # smallest shape: one hidden block
    (synth.Shape(D=1280, I=96, E=3, K=1), 3),     # partial chunks, three hidden blocks
    (synth.Shape(D=8192, I=1024, E=1, K=1), 2),   # four chunks per gate/up row
    (synth.Shape(D=256, I=8192, E=1, K=1), 2),    # four chunks per down row
    (GLM, 1), (GLM, 3)])
def test_expert_swiglu_b32_parity(shape, S):
    say(f"swiglu_b32 D={shape.D} I={shape.I} S={S}")
    e_id = shape.E - 1
    he = host_expert(6, shape, 0, e_id)
    dev = moe.DeviceExperts.empty(shape.E, shape.D, shape.I)
    for name in ("gate_q4", "gate_s", "up_q4", "up_s", "down_q4", "down_s"):
        getattr(dev, name)[e_id].copy_(torch.from_numpy(getattr(he, name)))
    cfg = moe.config(shape.D, shape.I, shape.E, shape.K)
    xq, sxb = oracle.quant_act_b32(_tokens(2, S, shape.D))
    ws = moe.Workspace(cfg, S, moe.WS_SWIGLU8)
    r = moe.moe_expert_swiglu_i4_b32(cfg, torch.from_numpy(xq).cuda(), torch.from_numpy(sxb).cuda(),
                                     dev, e_id, ws, probes=True)
    torch.cuda.synchronize()
    ref = oracle.expert_swiglu_b32(config_of(shape), xq, sxb, he)
    hq = to_np(r["hq"])
    mism = hq != ref["hq"]
    say(f"  hq mismatches: {int(mism.sum())} of {hq.size}")
    # the block terms are added in float on the device and in double in the
    # oracle: h agrees to rounding, so a code may move one step at a tie
    assert mism.mean() < 1e-3 and np.abs(hq.astype(int) - ref["hq"]).max() <= 1
    assert np.allclose(to_np(r["shb"]), ref["shb"], rtol=1e-5, atol=0)
    assert_close_rows(to_np(r["y"]), ref["y"], what="block-32 expert y")
