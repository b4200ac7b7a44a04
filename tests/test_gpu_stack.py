"""The layer stack (RMSNorm + MoE block + residual per layer, Zipf-skewed
routing per layer) on the GPU, checked layer by layer against the oracle with
the GPU's own layer inputs (teacher forcing): at each checked layer the
GPU's RMSNorm matches the oracle's, the GPU block on that normalized row
matches the oracle block, and the next layer's input is exactly this
layer's input plus the block's output."""
import gc
import json
import os

import numpy as np
import pytest
import torch

import int4_expert_gemv_moe_amd as moe
import oracle
import synth
from gpu_util import assert_close_rows, device_layer, oracle_block_ref, oracle_layer, say, to_np
from int4_expert_gemv_moe_amd.stack import Stack

pytestmark = pytest.mark.gpu

GLM = synth.GLM
HERE = os.path.dirname(os.path.abspath(__file__))
with open(os.path.join(HERE, "golden", "stack_beta.json")) as _f:
    BETA = json.load(_f)["beta"]
SEED = 0
EPS = 1e-5


def _free():
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _build(n_layers):
    layers = []
    for l in range(n_layers):
        b = synth.zipf_bias(SEED, GLM.E, l, BETA)
        layers.append(device_layer(SEED, GLM, l, b))
    gamma = torch.ones(GLM.D, dtype=torch.float32, device="cuda")
    return Stack(layers, gamma, EPS)


def _check_layers(stack, taps, x_final, check, union):
    """Teacher-forced checks of the listed layers."""
    S = taps[0].shape[0]
    nl = len(stack.layers)
    gamma = np.ones(GLM.D, np.float32)
    ws = moe.Workspace(stack.cfg, S, moe.WS_BATCH if union else moe.WS_FORWARD)
    fn = moe.moe_layer_forward_batch if union else moe.moe_layer_forward
    for l in check:
        x_in = taps[l]
        x_next = taps[l + 1] if l + 1 < nl else x_final
        xn = moe.moe_rmsnorm(x_in, stack.gamma, EPS)
        idx = torch.empty(S, GLM.K, dtype=torch.int32, device="cuda")
        w = torch.empty(S, GLM.K, dtype=torch.float32, device="cuda")
        out = fn(stack.layers[l], xn, ws, topk_idx=idx, topk_w=w)
        torch.cuda.synchronize()
        x_in_h, xn_h, out_h = to_np(x_in), to_np(xn), to_np(out)
        # the stack's update is exactly x + block(rmsnorm(x)) in float32
        assert np.array_equal(to_np(x_next).view(np.uint32), (x_in_h + out_h).view(np.uint32)), \
            f"layer {l}: residual update differs"
        xn_ref = oracle.rmsnorm(x_in_h, gamma, EPS)
        np.testing.assert_allclose(xn_h, xn_ref, rtol=2e-6, atol=1e-6)
        L = oracle_layer(SEED, GLM, l, synth.zipf_bias(SEED, GLM.E, l, BETA))
        ref, _ = oracle_block_ref(L, xn_h, to_np(idx), to_np(w))
        assert_close_rows(out_h, ref, what=f"stack layer {l} ({'union' if union else 'per-token'})")
        del L


def _check_all_layers_gpu(stack, taps, x_final):
    """Every layer, on the GPU alone: the stack's update equals x + block(RMSNorm(x))
    from separate calls, and the per-token and union paths give the same bits."""
    S = taps[0].shape[0]
    nl = len(stack.layers)
    ws_f = moe.Workspace(stack.cfg, S, moe.WS_FORWARD)
    ws_b = moe.Workspace(stack.cfg, S, moe.WS_BATCH)
    for l in range(nl):
        x_in = taps[l]
        x_next = taps[l + 1] if l + 1 < nl else x_final
        xn = moe.moe_rmsnorm(x_in, stack.gamma, EPS)
        out_f = moe.moe_layer_forward(stack.layers[l], xn, ws_f)
        out_b = moe.moe_layer_forward_batch(stack.layers[l], xn, ws_b)
        torch.cuda.synchronize()
        of, ob = to_np(out_f), to_np(out_b)
        assert np.array_equal(of.view(np.uint32), ob.view(np.uint32)), f"layer {l}: union != per-token"
        assert np.array_equal(to_np(x_next).view(np.uint32), (to_np(x_in) + of).view(np.uint32)), \
            f"layer {l}: residual update differs"


@pytest.mark.parametrize("S,union", [(1, False), (4, True)])
def test_stack_3_layers(S, union):
    _free()
    stack = _build(3)
    x = torch.from_numpy(synth.activations(SEED, S, GLM.D, item=50)).cuda()
    ws = moe.Workspace(stack.cfg, S, moe.WS_BATCH if union else moe.WS_FORWARD)
    taps = [torch.empty_like(x) for _ in range(3)]
    stack.forward(x, ws, union=union, taps=taps)
    torch.cuda.synchronize()
    _check_layers(stack, taps, x, range(3), union)
    del stack
    _free()


def test_stack_48_layers_resident():
    """The whole 48-layer stack resident in HBM (about 233 GB of int4
    experts); a decode step of one token and one of four tokens (union path)
    through all layers: every layer checked on the GPU (update = x + block,
    union == per-token bit for bit), layers 0, 23 and 47 against the oracle."""
    _free()
    say("building 48 GLM-shape layers")
    stack = _build(48)
    say(f"  resident: {torch.cuda.memory_allocated() / 2**30:.1f} GiB")
    for S, union in ((1, False), (4, True)):
        x = torch.from_numpy(synth.activations(SEED, S, GLM.D, item=60 + S)).cuda()
        ws = moe.Workspace(stack.cfg, S, moe.WS_BATCH if union else moe.WS_FORWARD)
        taps = [torch.empty_like(x) for _ in range(48)]
        stack.forward(x, ws, union=union, taps=taps)
        torch.cuda.synchronize()
        assert np.isfinite(to_np(x)).all()
        _check_all_layers_gpu(stack, taps, x)
        _check_layers(stack, taps, x, (0, 23, 47), union)
    del stack
    _free()
