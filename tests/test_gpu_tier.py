"""GPU checks of the given-routing call and of the expert residency tiers
(article section 05 expert cache, section 13 tiers): a layer whose routed
experts live in pinned host memory and a few HBM slots returns the same bits
as the fully resident layer, and its hits and misses are the oracle's."""
import numpy as np
import pytest
import torch

import int4_expert_gemv_moe_amd as moe
import oracle
import synth
from gpu_util import (assert_close_rows, bias_for, device_layer, oracle_block_ref, oracle_layer,
                      say, to_np)

pytestmark = pytest.mark.gpu

TINY, GLM = synth.TINY, synth.GLM
MID = synth.Shape(D=512, I=256, E=64, K=8)


def _resident(dl, x):
    S, K = x.shape[0], dl.cfg.K
    ws = moe.Workspace(dl.cfg, S, moe.WS_FORWARD)
    idx = torch.empty(S, K, dtype=torch.int32, device="cuda")
    w = torch.empty(S, K, dtype=torch.float32, device="cuda")
    o = moe.moe_layer_forward(dl, x, ws, topk_idx=idx, topk_w=w)
    return o, idx, w


def _bits(t):
    return to_np(t).view(np.uint32)


def _vs_oracle(L, x, out, idx, w, rows, what):
    """Rows of a GPU result against the oracle's block on the same tokens
    (tokens near a routing tie on the GPU's routing)."""
    xh = to_np(x)[rows]
    ref, _ = oracle_block_ref(L, xh, to_np(idx)[rows], to_np(w)[rows])
    assert_close_rows(to_np(out)[rows], ref, what=what)


@pytest.mark.parametrize("shape,S", [(TINY, 4), (MID, 5), (GLM, 1), (GLM, 3)])
def test_routed_call_equals_per_token_path(shape, S):
    say(f"routed call D={shape.D} E={shape.E} S={S}")
    dl = device_layer(5, shape, 0, bias_for("uniform", 5, shape))
    x = torch.from_numpy(synth.activations(31, S, shape.D)).cuda()
    ref, idx, w = _resident(dl, x)
    out = moe.moe_layer_forward_routed(dl, x, idx, w, moe.Workspace(dl.cfg, S, moe.WS_FORWARD))
    torch.cuda.synchronize()
    assert np.array_equal(_bits(out), _bits(ref))
    # the oracle's given-routing block on the same routing
    L = oracle_layer(5, shape, 0, bias_for("uniform", 5, shape))
    L.ensure(to_np(idx))
    want = oracle.layer_forward_routed(L, to_np(x), to_np(idx), to_np(w))
    assert_close_rows(to_np(out), want, what=f"routed call S={S}")


def test_routed_call_clamps_indices():
    shape = TINY
    dl = device_layer(6, shape, 0, bias_for("uniform", 6, shape))
    x = torch.from_numpy(synth.activations(32, 3, shape.D)).cuda()
    w = torch.tensor([[0.7, 1.1], [2.0, 0.5], [1.0, 1.0]], dtype=torch.float32, device="cuda")
    bad = torch.tensor([[-5, 3], [shape.E + 3, 1], [2, 2 ** 30]], dtype=torch.int32, device="cuda")
    good = torch.tensor([[0, 3], [shape.E - 1, 1], [2, shape.E - 1]], dtype=torch.int32,
                        device="cuda")
    a = moe.moe_layer_forward_routed(dl, x, bad, w, moe.Workspace(dl.cfg, 3, moe.WS_FORWARD))
    b = moe.moe_layer_forward_routed(dl, x, good, w, moe.Workspace(dl.cfg, 3, moe.WS_FORWARD))
    torch.cuda.synchronize()
    assert np.array_equal(_bits(a), _bits(b))


@pytest.mark.parametrize("shape,n_slots,S,calls", [(MID, 16, 1, 40), (MID, 24, 3, 20),
                                                   (GLM, 24, 1, 12)])
def test_tiered_layer_matches_resident_layer(shape, n_slots, S, calls):
    say(f"tiered D={shape.D} E={shape.E} slots={n_slots} S={S}")
    b = bias_for("zipf", 7, shape, 0, 0.05)
    dl = device_layer(7, shape, 0, b)
    L = oracle_layer(7, shape, 0, b)
    tl = moe.TieredLayer.from_device_layer(dl, n_slots)
    cache = oracle.ExpertCache(1, n_slots)
    wsr = moe.Workspace(dl.cfg, S, moe.WS_ROUTER)
    ws = moe.Workspace(dl.cfg, S, moe.WS_FORWARD)
    x_all = torch.from_numpy(synth.activations(33, S * calls, shape.D)).cuda()
    hits = 0
    for c in range(calls):
        x = x_all[c * S:(c + 1) * S]
        ref, idx, w = _resident(dl, x)
        out, misses = tl.forward(x, wsr, ws)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out), _bits(ref)), f"call {c}"
        if c < 3 or shape is not GLM:
            _vs_oracle(L, x, out, idx, w, np.arange(S), f"tiered call {c}")
        flat = to_np(idx).ravel().tolist()
        eids = [e for i, e in enumerate(flat) if e not in flat[:i]]  # first appearance
        expect = [cache.get(0, e)[1] for e in eids]
        assert misses == sum(expect), f"call {c}"
        hits += len(eids) - misses
    assert tl.tier.stats() == (cache.hits, cache.misses)
    say(f"  hits {cache.hits} misses {cache.misses}")


@pytest.mark.parametrize("shape,S", [(MID, 37), (GLM, 64)])
def test_batch_routed_call_equals_union_path(shape, S):
    dl = device_layer(11, shape, 0, bias_for("uniform", 11, shape))
    x = torch.from_numpy(synth.activations(34, S, shape.D)).cuda()
    ws = moe.Workspace(dl.cfg, S, moe.WS_BATCH)
    idx = torch.empty(S, shape.K, dtype=torch.int32, device="cuda")
    w = torch.empty(S, shape.K, dtype=torch.float32, device="cuda")
    ref = moe.moe_layer_forward_batch(dl, x, ws, topk_idx=idx, topk_w=w)
    out = moe.moe_layer_forward_batch_routed(dl, x, idx, w, moe.Workspace(dl.cfg, S, moe.WS_BATCH))
    torch.cuda.synchronize()
    assert np.array_equal(_bits(out), _bits(ref))


def test_batch_routed_call_clamps_indices():
    shape = MID
    dl = device_layer(12, shape, 0, bias_for("uniform", 12, shape))
    S = 3
    x = torch.from_numpy(synth.activations(35, S, shape.D)).cuda()
    w = torch.rand(S, shape.K, dtype=torch.float32, device="cuda")
    good = torch.randint(0, shape.E, (S, shape.K), dtype=torch.int32, device="cuda")
    bad = good.clone()
    bad[0, 0], bad[1, 3], bad[2, 7] = -7, shape.E + 5, 2 ** 30
    good[0, 0], good[1, 3], good[2, 7] = 0, shape.E - 1, shape.E - 1
    a = moe.moe_layer_forward_batch_routed(dl, x, bad, w, moe.Workspace(dl.cfg, S, moe.WS_BATCH))
    b = moe.moe_layer_forward_batch_routed(dl, x, good, w, moe.Workspace(dl.cfg, S, moe.WS_BATCH))
    torch.cuda.synchronize()
    assert np.array_equal(_bits(a), _bits(b))


@pytest.mark.parametrize("shape,n_slots,S,calls", [(MID, 48, 6, 12), (GLM, 192, 64, 3)])
def test_tiered_union_matches_resident_union(shape, n_slots, S, calls):
    say(f"tiered union D={shape.D} E={shape.E} slots={n_slots} S={S}")
    b = bias_for("zipf", 13, shape, 0, 0.05)
    dl = device_layer(13, shape, 0, b)
    L = oracle_layer(13, shape, 0, b)
    tl = moe.TieredLayer.from_device_layer(dl, n_slots)
    cache = oracle.ExpertCache(1, n_slots)
    wsr = moe.Workspace(dl.cfg, S, moe.WS_ROUTER)
    ws = moe.Workspace(dl.cfg, S, moe.WS_BATCH)
    wsb = moe.Workspace(dl.cfg, S, moe.WS_BATCH)
    x_all = torch.from_numpy(synth.activations(36, S * calls, shape.D)).cuda()
    for c in range(calls):
        x = x_all[c * S:(c + 1) * S]
        idx = torch.empty(S, shape.K, dtype=torch.int32, device="cuda")
        w = torch.empty(S, shape.K, dtype=torch.float32, device="cuda")
        ref = moe.moe_layer_forward_batch(dl, x, wsb, topk_idx=idx, topk_w=w)
        out, misses = tl.forward(x, wsr, ws, union=True)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out), _bits(ref)), f"call {c}"
        if c == 0:
            rows = np.unique(np.linspace(0, S - 1, min(S, 8)).round().astype(np.int64))
            _vs_oracle(L, x, out, idx, w, rows, f"tiered union call {c}")
        flat = to_np(idx).ravel().tolist()
        eids = [e for i, e in enumerate(flat) if e not in flat[:i]]
        assert misses == sum(cache.get(0, e)[1] for e in eids), f"call {c}"
    assert tl.tier.stats() == (cache.hits, cache.misses)
    say(f"  hits {cache.hits} misses {cache.misses}")


@pytest.mark.parametrize("shape,n_slots,n_pinned,calls", [(MID, 12, 8, 60), (GLM, 128, 64, 16)])
def test_tiered_layer_with_pinned_slots_matches_resident(shape, n_slots, n_pinned, calls):
    """Heat-managed pinned slots (section 13 swap rule) in front of the LRU
    slots: the slab copies of a rebalance are ordered after the call that
    decided them, and every call still returns the resident layer's bits."""
    say(f"pinned tier D={shape.D} E={shape.E} lru={n_slots} pinned={n_pinned}")
    b = bias_for("zipf", 14, shape, 0, 0.05)
    dl = device_layer(14, shape, 0, b)
    L = oracle_layer(14, shape, 0, b)
    tl = moe.TieredLayer.from_device_layer(dl, n_slots, n_pinned=n_pinned)
    wsr = moe.Workspace(dl.cfg, 1, moe.WS_ROUTER)
    ws = moe.Workspace(dl.cfg, 1, moe.WS_FORWARD)
    x_all = torch.from_numpy(synth.activations(37, calls, shape.D)).cuda()
    for c in range(calls):
        x = x_all[c:c + 1]
        ref, idx, w = _resident(dl, x)
        out, _ = tl.forward(x, wsr, ws)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out), _bits(ref)), f"call {c}"
        if c % 8 == 7:  # after rebalances have moved experts into pinned slots
            _vs_oracle(L, x, out, idx, w, np.arange(1), f"pinned tier call {c}")
    say(f"  hits/misses {tl.tier.stats()}")
