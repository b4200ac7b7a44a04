"""GPU parity of the per-token block with the shared expert in the int8
format against the CPU oracle, plain and accumulating, at the tiny and GLM
shapes."""
import numpy as np
import pytest
import torch

import int4_expert_gemv_moe_amd as moe
import oracle
import synth
from gpu_util import assert_close_rows, bias_for, check_routing, device_layer, oracle_layer, say, to_np

pytestmark = pytest.mark.gpu

TINY, GLM = synth.TINY, synth.GLM


def _shared8(seed, shape):
    g, u, d = synth.host_expert_f32(seed, shape, 0, synth.SHARED)
    h8 = oracle.HostExpertI8.from_f32(g, u, d)
    dev = moe.DeviceExpertsI8.empty(1, shape.D, shape.I)
    for name in ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s"):
        getattr(dev, name)[0].copy_(torch.from_numpy(getattr(h8, name)))
    return h8, dev


@pytest.mark.parametrize("shape,S,acc", [(TINY, 4, False), (TINY, 3, True), (GLM, 2, False),
                                         (GLM, 1, True)])
def test_layer_with_int8_shared_expert(shape, S, acc):
    say(f"shared_i8 D={shape.D} S={S} acc={acc}")
    b = bias_for("uniform", 0, shape)
    dl = device_layer(0, shape, 0, b)
    ol = oracle_layer(0, shape, 0, b)
    h8, d8 = _shared8(7, shape)
    x = synth.activations(13, S, shape.D)
    base = synth.activations(14, S, shape.D)
    ws = moe.Workspace(dl.cfg, S, moe.WS_SHARED8)
    out = torch.from_numpy(base.copy()).cuda() if acc else None
    o = moe.moe_layer_forward_shared_i8(dl, d8, torch.from_numpy(x).cuda(), ws, out=out,
                                        flags=moe.F_ACCUMULATE if acc else 0)
    torch.cuda.synchronize()
    ol.ensure_for(x)
    ref = oracle.layer_forward_shared_i8(ol, h8, x, out=base.copy() if acc else None,
                                         flags=1 if acc else 0)
    idx, _, _, choice = oracle.router_topk(ol.cfg, x, ol.router_w, ol.router_b)
    uniq = check_routing(idx, choice, shape.K)
    assert_close_rows(to_np(o), ref, uniq, what=f"shared int8 S={S}")
