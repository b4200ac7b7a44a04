"""GPU parity of the whole block, per-token path and unique-expert union path,
against the CPU oracle on the same seeded inputs."""
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


def _run(layer, x_np, path, flags=0, out=None):
    S = x_np.shape[0]
    ws = moe.Workspace(layer.cfg, S, moe.WS_FORWARD if path == "fwd" else moe.WS_BATCH)
    x = torch.from_numpy(np.ascontiguousarray(x_np)).cuda()
    idx = torch.empty(S, layer.cfg.K, dtype=torch.int32, device="cuda")
    w = torch.empty(S, layer.cfg.K, dtype=torch.float32, device="cuda")
    fn = moe.moe_layer_forward if path == "fwd" else moe.moe_layer_forward_batch
    o = fn(layer, x, ws, out=out, flags=flags, topk_idx=idx, topk_w=w)
    torch.cuda.synchronize()
    return to_np(o), to_np(idx), to_np(w)


def _sample_rows(S, n=16):
    """At most n token rows spread evenly over [0, S), first and last included."""
    return np.unique(np.linspace(0, S - 1, min(n, S)).round().astype(np.int64))


def _check_oracle(L, x_np, out, idx, w, rows, what):
    """The GPU block's rows against the oracle (near-tie tokens on the GPU's
    routing, see oracle_block_ref)."""
    ref, _ = oracle_block_ref(L, x_np[rows], idx[rows], w[rows])
    return assert_close_rows(out[rows], ref, what=what)


@pytest.mark.parametrize("path", ["fwd", "batch"])
def test_tiny_block(path):
    b = bias_for("uniform", 0, TINY)
    dl = device_layer(0, TINY, 0, b)
    ol = oracle_layer(0, TINY, 0, b)
    x = synth.activations(0, 4, TINY.D)
    out, idx, w = _run(dl, x, path)
    _check_oracle(ol, x, out, idx, w, np.arange(4), f"tiny {path}")


@pytest.mark.parametrize("shape,S,bias", [(TINY, 4, "uniform"), (TINY, 1, "uniform"),
                                          (MID, 5, "uniform"), (MID, 64, "zero"),
                                          (synth.Shape(D=512, I=256, E=8, K=8), 7, "uniform"),
                                          (synth.Shape(D=256, I=128, E=8, K=2, n_shared=0), 9,
                                           "uniform"),
                                          # K > 8: two routed-down launches per token
                                          (synth.Shape(D=256, I=128, E=64, K=16), 5, "uniform"),
                                          # E > 256: the 16-entry lists of the selection
                                          (synth.Shape(D=256, I=128, E=512, K=8), 6, "uniform"),
                                          # I % 256 != 0: GEMV down, masked row tails
                                          (synth.Shape(D=256, I=384, E=16, K=4), 3, "uniform"),
                                          # the documented limits: E = 1024 and K = 64
                                          # (eight routed-down launches per token)
                                          (synth.Shape(D=256, I=128, E=1024, K=64), 3, "uniform"),
                                          # smallest I (16-byte down rows) and a single
                                          # expert (E = K = 1)
                                          (synth.Shape(D=256, I=32, E=1, K=1), 2, "uniform"),
                                          # widest rows: 4 KB packed gate/up rows
                                          (synth.Shape(D=8192, I=4096, E=8, K=2), 2, "uniform"),
                                          # more than 64 tokens: the 8-wave MFMA kernels
                                          # with 80-pair tiles
                                          (MID, 65, "uniform"), (MID, 100, "zero"),
                                          (MID, 255, "uniform"),
                                          # every group exactly one full 80-pair tile
                                          (synth.Shape(D=512, I=256, E=8, K=8), 80, "uniform"),
                                          # groups of about 127 pairs (a full and a ragged
                                          # tile) and a shared group of four tiles
                                          (synth.Shape(D=512, I=256, E=8, K=4), 255, "uniform"),
                                          # no shared expert, more than 64 tokens
                                          (synth.Shape(D=256, I=128, E=16, K=4, n_shared=0), 130,
                                           "uniform"),
                                          # 4,500 pairs with the shared expert's: the
                                          # grouping kernel assembles the list in shared
                                          # memory; 25,200: more than that holds (24,576),
                                          # so it places them one by one
                                          (MID, 500, "uniform"), (MID, 2800, "uniform"),
                                          # more than 64 tokens with 10 and 26 steps of 128
                                          # columns: the gate/up loop's partial turn of 12
                                          (synth.Shape(D=1280, I=256, E=16, K=4), 100, "uniform"),
                                          (synth.Shape(D=3328, I=256, E=8, K=2), 80, "uniform")])
def test_batch_union_equals_per_token_bit_exact(shape, S, bias):
    b = bias_for(bias, 1, shape)
    dl = device_layer(1, shape, 0, b)
    x = synth.activations(1, S, shape.D)
    a, ia, wa = _run(dl, x, "fwd")
    c, ic, wc = _run(dl, x, "batch")
    assert np.array_equal(ia, ic)
    assert np.array_equal(wa.view(np.uint32), wc.view(np.uint32))
    assert np.array_equal(a.view(np.uint32), c.view(np.uint32))
    ol = oracle_layer(1, shape, 0, b)
    _check_oracle(ol, x, a, ia, wa, _sample_rows(S), f"D={shape.D} E={shape.E} K={shape.K} S={S}")


@pytest.mark.parametrize("S,recipe", [(65, "zipf"), (200, "uniform")])
def test_glm_union_mid_batches(S, recipe):
    """GLM shape, batches between the verify (64) and the prefill (2048)
    sizes through the 8-wave MFMA kernels: union == per-token bit for bit,
    sampled tokens against the oracle."""
    say(f"glm union S={S} {recipe}")
    wr = synth.router_w(2, GLM)
    b = np.zeros(GLM.E, np.float32)
    if recipe == "zipf":
        x, _, _ = synth.zipf_activations(2, GLM, S, wr)
    else:
        x = synth.activations(22, S, GLM.D)
    dl = device_layer(2, GLM, 0, b, router_w=wr)
    out_b, idx_b, w_b = _run(dl, x, "batch")
    out_f, idx_f, w_f = _run(dl, x, "fwd")
    assert np.array_equal(idx_b, idx_f)
    assert np.array_equal(out_b.view(np.uint32), out_f.view(np.uint32))
    counts = np.bincount(idx_b.ravel(), minlength=GLM.E)
    say(f"  union size {int((counts > 0).sum())}, largest group {int(counts.max())} pairs")
    ol = oracle_layer(2, GLM, 0, b, router_w=wr)
    _check_oracle(ol, x, out_b, idx_b, w_b, _sample_rows(S), f"glm union S={S}")


@pytest.mark.parametrize("shape,S", [(MID, 33), (MID, 64), (MID, 100), (TINY, 48)])
def test_batch_routed_repeated_and_clamped_experts(shape, S):
    """Given routing may repeat an expert within a token and name experts
    outside [0, E), which the library clamps into the stack: one expert then
    holds more pairs than a batch of S tokens would give it, up to several
    tiles.  The union equals the per-token routed call bit for bit, and the
    oracle on the clamped routing."""
    say(f"batch routed repeats D={shape.D} E={shape.E} K={shape.K} S={S}")
    b = bias_for("uniform", 3, shape)
    dl = device_layer(3, shape, 0, b)
    K, E = shape.K, shape.E
    rng = np.random.default_rng(S)
    idx = np.stack([rng.permutation(E)[:K] for _ in range(S)]).astype(np.int32)
    idx[:, 0] = 3                      # expert 3 in every token ...
    idx[::2, K - 1] = 3                # ... and twice in every other token
    idx[1::3, 1 % K] = E + 7           # clamps to E - 1
    idx[2::5, K // 2] = -4             # clamps to 0
    w = rng.uniform(0.05, 2.5, size=(S, K)).astype(np.float32)
    x = synth.activations(23, S, shape.D)
    xt = torch.from_numpy(x).cuda()
    it, wt = torch.from_numpy(idx).cuda(), torch.from_numpy(w).cuda()
    o_f = moe.moe_layer_forward_routed(dl, xt, it, wt, moe.Workspace(dl.cfg, S, moe.WS_FORWARD))
    o_b = moe.moe_layer_forward_routed(dl, xt, it, wt, moe.Workspace(dl.cfg, S, moe.WS_BATCH),
                                       fn_name="moe_layer_forward_batch_routed")
    torch.cuda.synchronize()
    a, c = to_np(o_f), to_np(o_b)
    assert np.array_equal(a.view(np.uint32), c.view(np.uint32))
    ol = oracle_layer(3, shape, 0, b)
    clamped = np.clip(idx, 0, E - 1)
    ol.ensure(clamped)
    rows = _sample_rows(S, 12)
    ref = oracle.layer_forward_routed(ol, x[rows], clamped[rows], w[rows])
    assert_close_rows(a[rows], ref, what=f"batch routed S={S}")


def test_accumulate_flag_and_residual():
    b = bias_for("uniform", 2, MID)
    dl = device_layer(2, MID, 0, b)
    x = synth.activations(2, 6, MID.D)
    base = synth.activations(3, 6, MID.D)
    plain, _, _ = _run(dl, x, "fwd")
    for path in ("fwd", "batch"):
        acc = torch.from_numpy(base.copy()).cuda()
        got, _, _ = _run(dl, x, path, flags=moe.F_ACCUMULATE, out=acc)
        assert np.array_equal(got, base + plain)


@pytest.mark.parametrize("shape,S,path", [(MID, 3, "fwd"), (MID, 6, "batch"), (MID, 20, "batch"),
                                          (GLM, 1, "fwd"), (GLM, 4, "batch")])
def test_prenorm_in_place_matches_separate_rmsnorm(shape, S, path):
    """MOE_F_PRENORM with out == x (one in-place decoder-layer update) gives
    the same bits as moe_rmsnorm into a scratch block followed by the plain
    call with MOE_F_ACCUMULATE; without accumulation, the same bits as the
    plain call on the normalized rows."""
    say(f"prenorm {path} D={shape.D} S={S}")
    b = bias_for("uniform", 4, shape)
    dl = device_layer(4, shape, 0, b)
    x0 = torch.from_numpy(synth.activations(12, S, shape.D)).cuda()
    gamma = torch.from_numpy((1.0 + 0.1 * synth.activations(13, 1, shape.D)[0]).astype(np.float32)).cuda()
    ws = moe.Workspace(dl.cfg, S, moe.WS_FORWARD if path == "fwd" else moe.WS_BATCH)
    fn = moe.moe_layer_forward if path == "fwd" else moe.moe_layer_forward_batch
    xn = moe.moe_rmsnorm(x0, gamma, 1e-5)
    ref = x0.clone()
    fn(dl, xn, ws, out=ref, flags=moe.F_ACCUMULATE)
    y = x0.clone()
    fn(dl, y, ws, out=y, flags=moe.F_ACCUMULATE, norm_gamma=gamma, norm_eps=1e-5)
    plain = fn(dl, xn, ws)
    fused = fn(dl, x0, ws, norm_gamma=gamma, norm_eps=1e-5)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(y).view(np.uint32), to_np(ref).view(np.uint32))
    assert np.array_equal(to_np(fused).view(np.uint32), to_np(plain).view(np.uint32))


def test_glm_decode_tokens():
    """GLM shape, one token per call (the decode step), several tokens."""
    b = bias_for("uniform", 0, GLM)
    dl = device_layer(0, GLM, 0, b)
    ol = oracle_layer(0, GLM, 0, b)
    x = synth.activations(11, 4, GLM.D)
    outs, idxs, ws = [], [], []
    for s in range(4):
        say(f"glm decode token {s}")
        o, i, w = _run(dl, x[s:s + 1], "fwd")
        outs.append(o[0])
        idxs.append(i[0])
        ws.append(w[0])
    _check_oracle(ol, x, np.stack(outs), np.stack(idxs), np.stack(ws), np.arange(4), "glm decode")


def test_glm_batched_verify_zipf():
    """GLM shape, 64 tokens with Zipf(1.1)-skewed routing through the union
    path; 16 sampled tokens against the oracle; batch == per-token on the GPU."""
    wr = synth.router_w(0, GLM)
    b = np.zeros(GLM.E, np.float32)
    x, _, _ = synth.zipf_activations(0, GLM, 64, wr)
    dl = device_layer(0, GLM, 0, b, router_w=wr)
    out_b, idx_b, w_b = _run(dl, x, "batch")
    out_f, idx_f, _ = _run(dl, x, "fwd")
    assert np.array_equal(idx_b, idx_f)
    assert np.array_equal(out_b.view(np.uint32), out_f.view(np.uint32))
    counts = np.bincount(idx_b.ravel(), minlength=GLM.E)
    say(f"  union size {int((counts > 0).sum())}, hottest expert {int(counts.max())} tokens")
    ol = oracle_layer(0, GLM, 0, b, router_w=wr)
    _check_oracle(ol, x, out_b, idx_b, w_b, _sample_rows(64), "glm zipf verify")


@pytest.mark.slow
def test_glm_prefill_2048_bf16():
    """GLM shape, 2048 tokens whose activations are bf16 values, uniform
    routing (b = 0), through the union path: two calls give the same bits,
    the union equals the per-token path bit for bit on every token, and 64
    tokens spread over the batch match the oracle."""
    b = np.zeros(GLM.E, np.float32)
    x = synth.bf16_to_f32(synth.bf16_bits(synth.activations(12, 2048, GLM.D)))
    dl = device_layer(1, GLM, 0, b)
    say("prefill: union path twice")
    out_b, idx_b, w_b = _run(dl, x, "batch")
    out_b2, idx_b2, _ = _run(dl, x, "batch")
    assert np.array_equal(idx_b, idx_b2)
    assert np.array_equal(out_b.view(np.uint32), out_b2.view(np.uint32))
    say("prefill: union path on the bf16 rows themselves")
    out_h, idx_h = _run_bf16(dl, x)
    assert np.array_equal(idx_b, idx_h)
    assert np.array_equal(out_b.view(np.uint32), out_h.view(np.uint32))
    say("prefill: per-token path")
    out_f, idx_f, w_f = _run(dl, x, "fwd")
    assert np.array_equal(idx_b, idx_f)
    assert np.array_equal(w_b.view(np.uint32), w_f.view(np.uint32))
    assert np.array_equal(out_b.view(np.uint32), out_f.view(np.uint32))
    counts = np.bincount(idx_b.ravel(), minlength=GLM.E)
    say(f"  tokens per expert: min {counts.min()} max {counts.max()}")
    ol = oracle_layer(1, GLM, 0, b)
    say("prefill: 64 tokens through the oracle")
    _check_oracle(ol, x, out_b, idx_b, w_b, _sample_rows(2048, 64), "glm prefill")


def _run_bf16(layer, x_np, idx=None, w=None):
    """The union path on bf16 rows (x_np must hold bf16 values); with idx/w
    the given-routing union instead."""
    S = x_np.shape[0]
    bits = synth.bf16_bits(x_np)
    assert np.array_equal(synth.bf16_to_f32(bits).view(np.uint32), x_np.view(np.uint32))
    xh = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    ws = moe.Workspace(layer.cfg, S, moe.WS_BATCH)
    if idx is not None:
        o = moe.moe_layer_forward_batch_routed(layer, xh, idx, w, ws)
        torch.cuda.synchronize()
        return to_np(o), None
    ti = torch.empty(S, layer.cfg.K, dtype=torch.int32, device="cuda")
    o = moe.moe_layer_forward_batch(layer, xh, ws, topk_idx=ti)
    torch.cuda.synchronize()
    return to_np(o), to_np(ti)


# the router's three launch shapes: up to 8 tokens, up to 255, and more
@pytest.mark.parametrize("shape,S", [(MID, 5), (MID, 100), (MID, 300), (TINY, 1)])
def test_bf16_tokens_equal_their_float32_widening(shape, S):
    """bf16 token rows through the union path (router and quantization widen
    them as they load) return the bits of the float32 rows they widen to,
    with the router's selection and with given routing; the per-token path
    refuses the flag."""
    b = bias_for("uniform", 7, shape)
    dl = device_layer(7, shape, 0, b)
    x = synth.bf16_to_f32(synth.bf16_bits(synth.activations(30 + S, S, shape.D)))
    say(f"bf16 tokens {shape} S={S}")
    out_f, idx_f, w_f = _run(dl, x, "batch")
    out_h, idx_h = _run_bf16(dl, x)
    assert np.array_equal(idx_f, idx_h)
    assert np.array_equal(out_f.view(np.uint32), out_h.view(np.uint32))
    ti = torch.from_numpy(idx_f).cuda()
    tw = torch.from_numpy(w_f).cuda()
    out_r, _ = _run_bf16(dl, x, ti, tw)
    assert np.array_equal(out_f.view(np.uint32), out_r.view(np.uint32))
    xf = torch.from_numpy(x).cuda()
    with pytest.raises(moe.MoeError):
        moe.moe_layer_forward(dl, xf, moe.Workspace(dl.cfg, S, moe.WS_FORWARD),
                              flags=moe.F_X_BF16)


def test_error_codes():
    cfg = moe.config(256, 128, 8, 2)
    b = bias_for("uniform", 0, TINY)
    dl = device_layer(0, TINY, 0, b)
    x = torch.from_numpy(synth.activations(0, 4, 256)).cuda()
    small = moe.Workspace(cfg, 1, moe.WS_FORWARD)
    with pytest.raises(moe.MoeError, match="workspace"):
        moe.moe_layer_forward(dl, x, small)
    ws = moe.Workspace(cfg, 4, moe.WS_FORWARD)
    xbig = torch.zeros(4 * 256 + 1, dtype=torch.float32, device="cuda")
    with pytest.raises(moe.MoeError, match="misaligned"):
        moe.moe_layer_forward(dl, xbig[1:].view(4, 256), ws)
    bad = moe.config(250, 128, 8, 2)
    with pytest.raises(moe.MoeError):
        moe.Workspace(bad, 1, moe.WS_FORWARD)


@pytest.mark.parametrize("S", [1, 4])
def test_per_token_selection_repeated_calls(S):
    """The per-token path selects inside its gate/up launch (every routed
    gate/up workgroup runs the token's selection rounds; the first one
    publishes them).  Many consecutive calls on one workspace must select
    exactly what the separate router and top-K kernels select for the same
    tokens (same logit bits, same rule), with the same weights."""
    shape = GLM
    b = bias_for("uniform", 3, shape)
    dl = device_layer(3, shape, 0, b)
    cfg = dl.cfg
    n_calls = 48
    x = torch.from_numpy(synth.activations(21, n_calls * S, shape.D)).cuda()
    ws = moe.Workspace(cfg, S, moe.WS_FORWARD)
    idx = torch.empty(n_calls, S, cfg.K, dtype=torch.int32, device="cuda")
    w = torch.empty(n_calls, S, cfg.K, dtype=torch.float32, device="cuda")
    for c in range(n_calls):
        moe.moe_layer_forward(dl, x[c * S:(c + 1) * S], ws, topk_idx=idx[c], topk_w=w[c])
    wsr = moe.Workspace(cfg, n_calls * S, moe.WS_ROUTER)
    ridx, rw, _ = moe.moe_router_topk(cfg, x, dl.router_w, dl.router_b, wsr)
    torch.cuda.synchronize()
    assert torch.equal(idx.view(-1, cfg.K), ridx)
    assert torch.equal(w.view(-1, cfg.K).view(torch.int32), rw.view(torch.int32))


@pytest.mark.parametrize("path,shape,S", [("fwd", MID, 5), ("batch", MID, 70), ("fwd", GLM, 1),
                                          ("batch", GLM, 4)])
def test_workspace_contents_do_not_matter(path, shape, S):
    """No kernel reads workspace memory it has not written in the same call:
    a workspace filled with 0xFF bytes (NaN floats, -1 integers) gives the
    bits of a zero-filled one."""
    b = bias_for("uniform", 5, shape)
    dl = device_layer(5, shape, 0, b)
    x = torch.from_numpy(synth.activations(24, S, shape.D)).cuda()
    which = moe.WS_FORWARD if path == "fwd" else moe.WS_BATCH
    fn = moe.moe_layer_forward if path == "fwd" else moe.moe_layer_forward_batch
    clean = moe.Workspace(dl.cfg, S, which)
    dirty = moe.Workspace(dl.cfg, S, which)
    dirty.view.fill_(0xFF)
    a = fn(dl, x, clean)
    c = fn(dl, x, dirty)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(a).view(np.uint32), to_np(c).view(np.uint32))
