"""Pins of the oracle's whole block: per-token path, unique-expert union path,
combine, and RMSNorm (sections 04 and 11 of the reader.mx article "惊呆了！25GB
内存上运行 GLM 5.2 744B 模型").  CPU only."""
import numpy as np
import pytest

import oracle
import synth
from oracle.layers import LazyLayer, bias_for, config_of, host_expert
from ref64 import layer64, max_rel_err

TINY = synth.TINY
MID = synth.Shape(D=512, I=256, E=64, K=8)


def _tiny_layer(seed=0):
    L = LazyLayer(seed, TINY, 0, bias_for("uniform", seed, TINY))
    L.ensure(range(TINY.E))
    return L


def test_tiny_layer_within_1e3_of_float64_reference():
    L = _tiny_layer()
    x = synth.activations(0, 4, TINY.D)
    out = oracle.layer_forward(L, x)
    ref, idx64, cs = layer64(x, L.router_w, L.router_b, L.experts, L.shared, TINY.D, TINY.I,
                             TINY.K, TINY.routed_scale)
    idx, _, _, _ = oracle.router_topk(L.cfg, x, L.router_w, L.router_b)
    assert np.all(cs[:, TINY.K - 1] - cs[:, TINY.K] > 1e-5)
    assert np.array_equal(idx, idx64)
    assert max_rel_err(out, ref).max() <= 1e-3


def test_mid_layer_within_1e3_of_float64_reference():
    L = LazyLayer(1, MID, 0, bias_for("uniform", 1, MID))
    x = synth.activations(1, 6, MID.D)
    L.ensure_for(x)
    out = oracle.layer_forward(L, x)
    ref, idx64, cs = layer64(x, L.router_w, L.router_b, L.experts, L.shared, MID.D, MID.I, MID.K,
                             MID.routed_scale)
    ok = cs[:, MID.K - 1] - cs[:, MID.K] > 1e-5
    assert ok.sum() >= 5
    assert max_rel_err(out[ok], ref[ok]).max() <= 1e-3


@pytest.mark.parametrize("S", [1, 4, 37])
def test_batch_union_equals_per_token_bit_exact(S):
    L = LazyLayer(2, MID, 0, bias_for("uniform", 2, MID))
    x = synth.activations(2, S, MID.D)
    if S > 4:
        x[5] = x[1]  # a repeated token routes identically
    L.ensure_for(x)
    a = oracle.layer_forward(L, x)
    b, idx, w, uniq = oracle.layer_forward_batch(L, x)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    # the union is the set of selected experts, in order of first appearance
    first = []
    for e in idx.ravel().tolist():
        if e not in first:
            first.append(e)
    assert uniq.tolist() == first
    assert len(uniq) == len(set(idx.ravel().tolist()))


def test_batch_rows_match_single_token_batches():
    L = _tiny_layer(3)
    x = synth.activations(3, 4, TINY.D)
    b, _, _, _ = oracle.layer_forward_batch(L, x)
    for s in range(4):
        one, _, _, _ = oracle.layer_forward_batch(L, x[s:s + 1])
        assert np.array_equal(one[0].view(np.uint32), b[s].view(np.uint32))


def test_single_expert_closed_form():
    # E = K = 1, b = 0: out = 2.5 * sigmoid(logit) * y + y_shared
    shape = synth.Shape(D=256, I=128, E=1, K=1)
    L = LazyLayer(4, shape, 0, np.zeros(1, np.float32))
    L.ensure([0])
    x = synth.activations(4, 3, shape.D)
    out = oracle.layer_forward(L, x)
    xq, sx = oracle.quant_act_i8(x)
    cfg = config_of(shape)
    y = oracle.expert_swiglu(cfg, xq, sx, L.experts[0])["y"].astype(np.float64)
    ysh = oracle.expert_swiglu(cfg, xq, sx, L.shared)["y"].astype(np.float64)
    logit = x.astype(np.float64) @ L.router_w[0].astype(np.float64)
    want = 2.5 * (1.0 / (1.0 + np.exp(-logit)))[:, None] * y + ysh
    assert max_rel_err(out, want).max() <= 1e-6


def test_no_shared_expert_and_accumulate_flag():
    shape = synth.Shape(D=256, I=128, E=8, K=2, n_shared=0)
    L = LazyLayer(5, shape, 0, bias_for("uniform", 5, shape))
    L.ensure(range(8))
    x = synth.activations(5, 4, shape.D)
    out = oracle.layer_forward(L, x)
    ref, _, _ = layer64(x, L.router_w, L.router_b, L.experts, None, shape.D, shape.I, shape.K, 2.5)
    assert max_rel_err(out, ref).max() <= 1e-3
    base = synth.activations(6, 4, shape.D)
    acc = base.copy()
    oracle.layer_forward(L, x, out=acc, flags=oracle.ACCUMULATE)
    assert np.array_equal(acc, base + out)
    acc2 = base.copy()
    oracle.layer_forward_batch(L, x, out=acc2, flags=oracle.ACCUMULATE)
    assert np.array_equal(acc2, acc)


def test_rmsnorm_closed_forms():
    a = np.float32(3.0)
    y = oracle.rmsnorm(np.full((1, 64), a, np.float32), np.ones(64, np.float32), 1e-5)
    assert np.allclose(y, a / np.sqrt(a * a + 1e-5), rtol=2e-7)
    x = synth.activations(7, 5, 6144) * np.float32(3.0)
    y = oracle.rmsnorm(x, np.ones(6144, np.float32), 1e-5)
    ms = (x.astype(np.float64) ** 2).mean(axis=1)
    assert np.allclose((y.astype(np.float64) ** 2).mean(axis=1), ms / (ms + 1e-5), rtol=1e-5)
    g = np.linspace(0.5, 2.0, 6144, dtype=np.float32)
    yg = oracle.rmsnorm(x, g, 1e-5)
    assert np.allclose(yg, y * g, rtol=2e-7, atol=0)


def test_layer_rejects_missing_shared_and_bad_k():
    shape = synth.Shape(D=256, I=128, E=8, K=2)
    L = LazyLayer(8, shape, 0, np.zeros(8, np.float32))
    L.ensure(range(8))
    L.shared = None
    with pytest.raises(ValueError):
        oracle.layer_forward(L, synth.activations(8, 1, 256))


def test_zipf_recipe_is_skewed():
    # the batched-verify recipe: real router logits follow log p + Gumbel noise
    shape = synth.GLM
    wr = synth.router_w(0, shape)
    x, target, p = synth.zipf_activations(0, shape, 64, wr)
    cfg = config_of(shape)
    idx, _, logits, _ = oracle.router_topk(cfg, x, wr, np.zeros(shape.E, np.float32))
    assert np.abs(logits - target).max() < 1e-3
    counts = np.bincount(idx.ravel(), minlength=shape.E)
    hot = int(np.argmax(p))
    assert counts[hot] >= 40  # the rank-1 expert is in most selections
    assert 100 <= (counts > 0).sum() <= 200  # union size of the batch


# ---- the block on given routing ------------------------------------------

@pytest.mark.parametrize("shape,S,seed", [(TINY, 4, 9), (MID, 11, 10),
                                          (synth.Shape(D=256, I=128, E=8, K=2, n_shared=0), 5, 11)])
def test_routed_on_the_routers_choice_equals_the_block_bit_exact(shape, S, seed):
    """Fed the routing that the router selects, the given-routing calls return
    the routed block's bits (per token and through the union)."""
    L = LazyLayer(seed, shape, 0, bias_for("uniform", seed, shape))
    x = synth.activations(seed, S, shape.D)
    idx = L.ensure_for(x)
    a = oracle.layer_forward(L, x)
    idx2, w2, _, _ = oracle.router_topk(L.cfg, x, L.router_w, L.router_b)
    assert np.array_equal(idx, idx2)
    r = oracle.layer_forward_routed(L, x, idx2, w2)
    b, uniq = oracle.layer_forward_batch_routed(L, x, idx2, w2)
    assert np.array_equal(a.view(np.uint32), r.view(np.uint32))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    _, _, _, u0 = oracle.layer_forward_batch(L, x)
    assert uniq.tolist() == u0.tolist()


def test_routed_closed_form_on_arbitrary_routing():
    """Any routing, duplicates within a token included: out[s] =
    sum_k w[s][k] * y_{idx[s][k]}(x_s) + y_shared(x_s), the sum in k order
    (float32, starting from 0), each y from the single-expert oracle call;
    the union on the same routing returns the same bits."""
    shape = synth.Shape(D=256, I=128, E=8, K=3)
    L = LazyLayer(12, shape, 0, np.zeros(shape.E, np.float32))
    L.ensure(range(shape.E))
    S = 6
    x = synth.activations(12, S, shape.D)
    rng = np.random.default_rng(12)
    idx = rng.integers(0, shape.E, size=(S, shape.K)).astype(np.int32)
    idx[0] = [5, 5, 5]     # one expert three times in one token
    idx[1] = [2, 7, 2]
    w = rng.uniform(-1.5, 2.5, size=(S, shape.K)).astype(np.float32)
    got = oracle.layer_forward_routed(L, x, idx, w)
    xq, sx = oracle.quant_act_i8(x)
    cfg = config_of(shape)
    want = np.zeros((S, shape.D), np.float32)
    for s in range(S):
        acc = np.zeros(shape.D, np.float32)
        for k in range(shape.K):
            y = oracle.expert_swiglu(cfg, xq[s:s + 1], sx[s:s + 1], L.experts[int(idx[s, k])])["y"][0]
            acc = acc + w[s, k] * y
        ysh = oracle.expert_swiglu(cfg, xq[s:s + 1], sx[s:s + 1], L.shared)["y"][0]
        want[s] = acc + ysh
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    b, uniq = oracle.layer_forward_batch_routed(L, x, idx, w)
    assert np.array_equal(b.view(np.uint32), got.view(np.uint32))
    first = []
    for e in idx.ravel().tolist():
        if e not in first:
            first.append(e)
    assert uniq.tolist() == first


def test_routed_within_1e3_of_float64_reference_on_given_routing():
    """The float64 reference fed the same (non-router) routing."""
    from ref64 import expert64
    shape = MID
    L = LazyLayer(13, shape, 0, np.zeros(shape.E, np.float32))
    S = 5
    x = synth.activations(13, S, shape.D)
    rng = np.random.default_rng(13)
    idx = np.stack([rng.permutation(shape.E)[:shape.K] for _ in range(S)]).astype(np.int32)
    w = rng.uniform(0.1, 2.5, size=(S, shape.K)).astype(np.float32)
    L.ensure(idx)
    got = oracle.layer_forward_routed(L, x, idx, w)
    xq, sx = oracle.quant_act_i8(x)
    want = np.zeros((S, shape.D))
    for s in range(S):
        xd = xq[s:s + 1].astype(np.float64) * float(sx[s])
        for k in range(shape.K):
            want[s] += float(w[s, k]) * expert64(xd, L.experts[int(idx[s, k])], shape.D, shape.I)[0]
        want[s] += expert64(xd, L.shared, shape.D, shape.I)[0]
    assert max_rel_err(got, want).max() <= 1e-3


def test_routed_rejects_out_of_range_experts():
    shape = synth.Shape(D=256, I=128, E=8, K=2)
    L = LazyLayer(14, shape, 0, np.zeros(8, np.float32))
    L.ensure(range(8))
    x = synth.activations(14, 2, shape.D)
    w = np.ones((2, 2), np.float32)
    for bad in (8, -1):
        idx = np.array([[0, 1], [bad, 2]], np.int32)
        with pytest.raises(ValueError):
            oracle.layer_forward_routed(L, x, idx, w)
        with pytest.raises(ValueError):
            oracle.layer_forward_batch_routed(L, x, idx, w)
