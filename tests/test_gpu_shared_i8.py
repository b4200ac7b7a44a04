"""GPU parity of the per-token block with the shared expert in the int8
format against the CPU oracle, plain and accumulating, at the tiny and GLM
shapes."""
import numpy as np
import pytest
import torch

import int4_expert_gemv_moe_amd as moe
import oracle
import synth
from gpu_util import (assert_close_rows, bias_for, device_layer, oracle_block_ref, oracle_layer, say,
                      to_np)

pytestmark = pytest.mark.gpu

TINY, GLM = synth.TINY, synth.GLM


def _shared8(seed, shape):
    g, u, d = synth.host_expert_f32(seed, shape, 0, synth.SHARED)
    h8 = oracle.HostExpertI8.from_f32(g, u, d)
    dev = moe.DeviceExpertsI8.empty(1, shape.D, shape.I)
    for name in ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s"):
        getattr(dev, name)[0].copy_(torch.from_numpy(getattr(h8, name)))
    return h8, dev


MID = synth.Shape(D=512, I=256, E=64, K=8)


# D % 2048 == 0 and I % 1024 == 0: the int8 expert inside the per-token launches
FUSED = synth.Shape(D=2048, I=1024, E=16, K=4)


@pytest.mark.parametrize("shape,S,acc,topp", [(TINY, 4, False, 0.0), (TINY, 3, True, 0.0),
                                              (GLM, 2, False, 0.0), (GLM, 1, True, 0.0),
                                              (MID, 24, False, 0.0), (MID, 9, True, 0.6),
                                              (GLM, 5, False, 0.7), (FUSED, 6, True, 0.0),
                                              (FUSED, 3, False, 0.5)])
def test_layer_with_int8_shared_expert(shape, S, acc, topp):
    say(f"shared_i8 D={shape.D} S={S} acc={acc} topp={topp}")
    b = bias_for("uniform", 0, shape)
    dl = device_layer(0, shape, 0, b)
    ol = oracle_layer(0, shape, 0, b)
    if topp:
        c = dl.cfg
        dl = moe.DeviceLayer(moe.config(c.D, c.I, c.E, c.K, c.n_shared, c.routed_scale, topp),
                             dl.router_w, dl.router_b, dl.routed, dl.shared)
        ol.cfg.expert_topp = topp
    h8, d8 = _shared8(7, shape)
    x = synth.activations(13, S, shape.D)
    base = synth.activations(14, S, shape.D)
    xt = torch.from_numpy(x).cuda()
    ws = moe.Workspace(dl.cfg, S, moe.WS_SHARED8)
    out = torch.from_numpy(base.copy()).cuda() if acc else None
    o = moe.moe_layer_forward_shared_i8(dl, d8, xt, ws, out=out,
                                        flags=moe.F_ACCUMULATE if acc else 0)
    # the GPU's routing: the per-token path selects exactly what the router
    # and top-K kernels select for the same tokens
    idx, w, _ = moe.moe_router_topk(dl.cfg, xt, dl.router_w, dl.router_b,
                                    moe.Workspace(dl.cfg, S, moe.WS_ROUTER))
    torch.cuda.synchronize()
    idx, w = to_np(idx), to_np(w)
    keff = np.array([oracle.expert_keff(w[s], topp) for s in range(S)]) if topp else None
    ref, _ = oracle_block_ref(ol, x, idx, w, keff_gpu=keff, base=base if acc else None,
                              shared8=h8)
    assert_close_rows(to_np(o), ref, what=f"shared int8 S={S}")


# the union's int8 shared expert runs on the int8 matrix cores: up to 511
# tokens in chunks of 64 (100 and 150: two and three chunks, the last ragged),
# from 512 tokens in 128-token tiles through shared memory (520 and 530: a
# ragged last tile); I = 96 leaves a partial contraction step in the down
# projection
I96 = synth.Shape(D=512, I=96, E=16, K=4)


@pytest.mark.parametrize("shape,S,acc", [(TINY, 4, False), (MID, 24, True), (MID, 100, False),
                                         (FUSED, 7, False), (GLM, 4, True), (GLM, 64, False),
                                         (GLM, 100, False), (MID, 150, True), (I96, 70, False),
                                         (GLM, 520, False), (I96, 530, True)])
def test_union_with_int8_shared_expert(shape, S, acc):
    """The union path with the int8 shared expert returns the per-token
    path's bits (whether the per-token path runs the int8 expert inside its
    launches or after them), and matches the oracle on sampled tokens."""
    say(f"union shared_i8 D={shape.D} S={S} acc={acc}")
    b = bias_for("uniform", 2, shape)
    dl = device_layer(2, shape, 0, b)
    h8, d8 = _shared8(9, shape)
    x = synth.activations(15, S, shape.D)
    base = synth.activations(16, S, shape.D)
    xt = torch.from_numpy(x).cuda()
    fl = moe.F_ACCUMULATE if acc else 0
    o_f = moe.moe_layer_forward_shared_i8(
        dl, d8, xt, moe.Workspace(dl.cfg, S, moe.WS_SHARED8),
        out=torch.from_numpy(base.copy()).cuda() if acc else None, flags=fl)
    o_b = moe.moe_layer_forward_shared_i8(
        dl, d8, xt, moe.Workspace(dl.cfg, S, moe.WS_BATCH),
        out=torch.from_numpy(base.copy()).cuda() if acc else None, flags=fl,
        fn_name="moe_layer_forward_batch_shared_i8")
    idx, w, _ = moe.moe_router_topk(dl.cfg, xt, dl.router_w, dl.router_b,
                                    moe.Workspace(dl.cfg, S, moe.WS_ROUTER))
    torch.cuda.synchronize()
    a, c = to_np(o_f), to_np(o_b)
    assert np.array_equal(a.view(np.uint32), c.view(np.uint32))
    rows = np.unique(np.linspace(0, S - 1, min(S, 12)).round().astype(np.int64))
    ol = oracle_layer(2, shape, 0, b)
    ref, _ = oracle_block_ref(ol, x[rows], to_np(idx)[rows], to_np(w)[rows],
                              base=base[rows] if acc else None, shared8=h8)
    assert_close_rows(c[rows], ref, what=f"union shared int8 S={S}")
