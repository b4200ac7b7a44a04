"""GPU parity of the adaptive expert top-p (keff[s] experts per token; the
rule is the oracle's, see its header): the device's keff equals the oracle
rule applied to the device's own weights, outputs match the oracle, and the
union path equals the per-token path bit for bit."""
import numpy as np
import pytest
import torch

import int4_expert_gemv_moe_amd as moe
import oracle
import synth
from gpu_util import (assert_close_rows, bias_for, device_layer, oracle_block_ref, oracle_layer, say,
                      to_np)

pytestmark = pytest.mark.gpu

GLM = synth.GLM
MID = synth.Shape(D=512, I=256, E=64, K=8)


def _with_topp(dl, p):
    c = dl.cfg
    cfg = moe.config(c.D, c.I, c.E, c.K, c.n_shared, c.routed_scale, p)
    return moe.DeviceLayer(cfg, dl.router_w, dl.router_b, dl.routed, dl.shared)


def _run(layer, x_np, path):
    S, K = x_np.shape[0], layer.cfg.K
    ws = moe.Workspace(layer.cfg, S, moe.WS_FORWARD if path == "fwd" else moe.WS_BATCH)
    x = torch.from_numpy(np.ascontiguousarray(x_np)).cuda()
    idx = torch.empty(S, K, dtype=torch.int32, device="cuda")
    w = torch.empty(S, K, dtype=torch.float32, device="cuda")
    keff = torch.empty(S, dtype=torch.int32, device="cuda")
    fn = moe.moe_layer_forward if path == "fwd" else moe.moe_layer_forward_batch
    o = fn(layer, x, ws, topk_idx=idx, topk_w=w, keff=keff)
    torch.cuda.synchronize()
    return to_np(o), to_np(idx), to_np(w), to_np(keff)


K16 = synth.Shape(D=256, I=128, E=64, K=16)   # two routed-down launches per token
E512 = synth.Shape(D=256, I=128, E=512, K=8)  # 16-entry selection lists


@pytest.mark.parametrize("shape,S,p", [(MID, 6, 0.5), (MID, 6, 0.7), (MID, 9, 0.9),
                                       (GLM, 3, 0.7), (K16, 5, 0.4), (K16, 4, 0.8),
                                       (E512, 6, 0.6)])
def test_topp_against_oracle(shape, S, p):
    say(f"top-p {p} D={shape.D} E={shape.E} S={S}")
    b = bias_for("uniform", 8, shape)
    dl = _with_topp(device_layer(8, shape, 0, b), p)
    x = synth.activations(40, S, shape.D)
    for path in ("fwd", "batch"):
        out, idx, w, keff = _run(dl, x, path)
        # keff is the oracle's rule on the device's own weights, exactly
        assert [oracle.expert_keff(w[s], p) for s in range(S)] == keff.tolist()
        ol = oracle_layer(8, shape, 0, b)
        ol.cfg.expert_topp = p
        ref, uniq = oracle_block_ref(ol, x, idx, w, keff_gpu=keff)
        assert uniq.sum() >= S - 1
        assert_close_rows(out, ref, what=f"top-p {p} {path}")
        say(f"  {path}: keff {keff.tolist()}")


# (MID, 800, 0.7): more than 64 tokens, and a pair list long enough that the
# grouping kernel assembles it in shared memory, with dropped pairs
@pytest.mark.parametrize("shape,S,p", [(MID, 5, 0.6), (MID, 37, 0.8), (GLM, 4, 0.7),
                                       (K16, 7, 0.4), (E512, 5, 0.6), (MID, 800, 0.7)])
def test_topp_union_equals_per_token_bit_exact(shape, S, p):
    dl = _with_topp(device_layer(9, shape, 0, bias_for("uniform", 9, shape)), p)
    x = synth.activations(41, S, shape.D)
    a, ia, wa, ka = _run(dl, x, "fwd")
    c, ic, wc, kc = _run(dl, x, "batch")
    assert np.array_equal(ia, ic) and np.array_equal(ka, kc)
    assert np.array_equal(a.view(np.uint32), c.view(np.uint32))
    assert ka.min() < shape.K  # top-p dropped some experts


def test_topp_one_is_the_full_block():
    dl = device_layer(10, MID, 0, bias_for("uniform", 10, MID))
    x = synth.activations(42, 7, MID.D)
    for path in ("fwd", "batch"):
        a, _, _, ka = _run(_with_topp(dl, 1.0), x, path)
        b, _, _, kb = _run(dl, x, path)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
        assert ka.tolist() == kb.tolist() == [MID.K] * 7
