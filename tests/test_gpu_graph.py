"""The layer calls captured in a HIP graph: every replay returns the eager
call's bits.  A call issues kernels and device-to-device copies only (no
memset, no allocation, no host synchronization), so the captured graph is the
same work; the test replays it several times with eager calls on other
buffers and synchronizations in between, as a serving loop would."""
import numpy as np
import pytest
import torch

import int4_expert_gemv_moe_amd as moe
import synth
from gpu_util import bias_for, device_layer, say, to_np

pytestmark = pytest.mark.gpu

MID = synth.Shape(D=512, I=256, E=64, K=8)
GLM = synth.GLM


# path: per-token ("fwd") or union ("batch"); mode: plain, accumulate (out
# reset from a base inside the graph) or prenorm (x normalized and updated in
# place, x reset from x0 inside the graph)
@pytest.mark.parametrize("shape,S,path,mode", [
    (MID, 1, "fwd", "plain"), (MID, 3, "fwd", "plain"), (MID, 37, "batch", "plain"),
    (MID, 100, "batch", "plain"), (MID, 20, "batch", "accumulate"), (MID, 2, "fwd", "prenorm"),
    (MID, 12, "batch", "prenorm"), (GLM, 2, "fwd", "plain"), (GLM, 70, "batch", "plain")])
def test_graph_replays_equal_eager(shape, S, path, mode):
    say(f"graph {path} {mode} D={shape.D} S={S}")
    dl = device_layer(3, shape, 0, bias_for("uniform", 3, shape))
    fn = moe.moe_layer_forward if path == "fwd" else moe.moe_layer_forward_batch
    kind = moe.WS_FORWARD if path == "fwd" else moe.WS_BATCH
    x0 = torch.from_numpy(synth.activations(21, S, shape.D)).cuda()
    base = torch.from_numpy(synth.activations(23, S, shape.D)).cuda()
    gamma = torch.from_numpy(1.0 + 0.1 * synth.activations(24, 1, shape.D)[0]).cuda()
    ws = moe.Workspace(dl.cfg, S, kind)
    x = x0.clone()
    out = torch.empty(S, shape.D, dtype=torch.float32, device="cuda")

    def call(stream=None):
        # the work the graph captures
        if mode == "accumulate":
            out.copy_(base)
            fn(dl, x, ws, out=out, flags=moe.F_ACCUMULATE, stream=stream)
        elif mode == "prenorm":
            x.copy_(x0)
            fn(dl, x, ws, out=x, norm_gamma=gamma, stream=stream)
        else:
            fn(dl, x, ws, out=out, stream=stream)

    def result():
        return to_np(x if mode == "prenorm" else out).copy()

    call()
    torch.cuda.synchronize()
    ref = result()
    # eager work between the replays: the same call on other inputs and buffers
    x2 = torch.from_numpy(synth.activations(22, S, shape.D)).cuda()
    ws2 = moe.Workspace(dl.cfg, S, kind)
    out2 = torch.empty_like(out)
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        call(stream=cap)
    for rep in range(4):
        # poison what the replay must rewrite (the input stays, except in
        # place, where the graph restores it from x0)
        (x if mode == "prenorm" else out).fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = result()
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"replay {rep}"
        fn(dl, x2, ws2, out=out2)
        torch.cuda.synchronize()
    say(f"  4 replays equal the eager call")
