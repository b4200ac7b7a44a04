"""The allocation-free per-token entry point (moe_layer_forward_noalloc):
through the C ABI it returns moe_layer_forward's bits on two calls in a row,
the second with fewer tokens, and refuses a call larger than its scratch."""
import numpy as np
import pytest
import torch

import int4_expert_gemv_moe_amd as moe
import synth
from gpu_util import bias_for, device_layer, say, to_np

pytestmark = pytest.mark.gpu

MID = synth.Shape(D=512, I=256, E=64, K=8)


def _bits(t):
    return to_np(t).view(np.uint32)


@pytest.mark.parametrize("shape,sizes", [(synth.TINY, (4, 1)), (MID, (16, 3)),
                                         (synth.GLM, (2, 1))])
def test_noalloc_equals_workspace_call(shape, sizes):
    say(f"noalloc D={shape.D} E={shape.E} S={sizes}")
    b = bias_for("uniform", 4, shape)
    dl = device_layer(4, shape, 0, b)
    x_all = synth.activations(51, sum(sizes), shape.D)
    lo = 0
    for S in sizes:
        x = torch.from_numpy(x_all[lo:lo + S]).cuda()
        lo += S
        ref = moe.moe_layer_forward(dl, x, moe.Workspace(dl.cfg, S, moe.WS_FORWARD))
        got = moe.moe_layer_forward_noalloc(dl, x)
        base = torch.from_numpy(synth.activations(52, S, shape.D)).cuda()
        ref_acc = moe.moe_layer_forward(dl, x, moe.Workspace(dl.cfg, S, moe.WS_FORWARD),
                                        out=base.clone(), flags=moe.F_ACCUMULATE)
        got_acc = moe.moe_layer_forward_noalloc(dl, x, out=base.clone(), flags=moe.F_ACCUMULATE)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(got), _bits(ref)), f"S={S}"
        assert np.array_equal(_bits(got_acc), _bits(ref_acc)), f"S={S} accumulate"


def test_noalloc_refuses_calls_beyond_its_scratch():
    shape = synth.GLM
    dl = device_layer(4, shape, 0, bias_for("uniform", 4, shape))
    cfg = dl.cfg
    S = 1
    while moe.lib().moe_workspace_bytes(ctypes_ref(cfg), S, moe.WS_FORWARD) <= moe.NOALLOC_WS_BYTES:
        S *= 2
    x = torch.zeros(S, shape.D, dtype=torch.float32, device="cuda")
    with pytest.raises(moe.MoeError, match="workspace"):
        moe.moe_layer_forward_noalloc(dl, x)


def ctypes_ref(cfg):
    import ctypes
    return ctypes.byref(cfg)
