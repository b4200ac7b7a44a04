"""GPU parity of the library's building blocks against the CPU oracle:
int4 packer, activation quantization, router/top-K, and one SwiGLU expert."""
import numpy as np
import pytest
import torch

import int4_expert_gemv_moe_amd as moe
import oracle
import synth
from gpu_util import (assert_close_rows, check_routing, config_of, say, to_np)
from oracle.layers import host_expert
from ref64 import unpack64

pytestmark = pytest.mark.gpu

TINY, GLM = synth.TINY, synth.GLM


def _dev_normal(seed, strm, n, sigma):
    t = torch.empty(n, dtype=torch.float32, device="cuda")
    synth.dev_fill_normal(t.data_ptr(), seed, strm, n, sigma, torch.cuda.current_stream().cuda_stream)
    return t


def test_device_generator_matches_host():
    strm = synth.stream(synth.K_GATE, 2, 5)
    d = to_np(_dev_normal(3, strm, 1 << 20, 0.02))
    h = synth.host_normal(3, strm, 1 << 20, 0.02)
    assert np.array_equal(d.view(np.uint32), h.view(np.uint32))


@pytest.mark.parametrize("O,C", [(7, 256), (64, 6144), (2048, 6144), (6144, 2048), (3, 34)])
def test_pack_bit_exact(O, C):
    say(f"pack O={O} C={C}")
    strm = synth.stream(synth.K_UP, 1, 9)
    w = _dev_normal(0, strm, O * C, 0.02).view(O, C)
    q4, s = moe.moe_pack_int4(w)
    rq4, rs = oracle.pack_int4(synth.host_normal(0, strm, O * C, 0.02).reshape(O, C))
    assert np.array_equal(to_np(q4), rq4)
    assert np.array_equal(to_np(s).view(np.uint32), rs.view(np.uint32))


def test_pack_edge_rows():
    w = np.zeros((4, 64), np.float32)
    w[1, 3] = 7.0
    w[1, 4] = 3.5  # a tie: rounds to even
    w[2] = np.linspace(-1, 1, 64, dtype=np.float32)
    w[3, :] = 1e-9  # scale floor
    q4, s = moe.moe_pack_int4(torch.from_numpy(w).cuda())
    rq4, rs = oracle.pack_int4(w)
    assert np.array_equal(to_np(q4), rq4) and np.array_equal(to_np(s), rs)


@pytest.mark.parametrize("S,D", [(1, 6144), (4, 256), (64, 6144), (33, 1024)])
def test_quant_bit_exact(S, D):
    x = synth.activations(5, S, D)
    x[0, 3] = 0.0
    xq, sx = moe.moe_quant_act_i8(torch.from_numpy(x).cuda())
    rxq, rsx = oracle.quant_act_i8(x)
    assert np.array_equal(to_np(xq), rxq)
    assert np.array_equal(to_np(sx).view(np.uint32), rsx.view(np.uint32))


def test_quant_bf16_and_degenerate_rows():
    x = synth.activations(6, 16, 512)
    x[1] = 0.0
    x[2] = 1e-11
    x[3, ::2] = 127.5  # half-way codes after scaling
    bits = synth.bf16_bits(x)
    xb = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    xq, sx = moe.moe_quant_act_i8(xb)
    rxq, rsx = oracle.quant_act_i8_bf16(bits)
    assert np.array_equal(to_np(xq), rxq) and np.array_equal(to_np(sx), rsx)
    xq2, sx2 = moe.moe_quant_act_i8(torch.from_numpy(x).cuda())
    rxq2, rsx2 = oracle.quant_act_i8(x)
    assert np.array_equal(to_np(xq2), rxq2) and np.array_equal(to_np(sx2), rsx2)


# the router's launch shapes: up to 8 tokens, 9 to 255 (8 x 8 tiles through
# shared memory; 37 experts and 29 tokens leave both tile edges ragged), and
# 256 and more (16 x 16 tiles through shared memory; 37 experts and 301
# tokens leave both edges ragged, and 512 columns are fewer steps than the
# ring has stages)
@pytest.mark.parametrize("shape,S,bias", [(TINY, 4, "uniform"), (GLM, 1, "uniform"),
                                          (GLM, 64, "uniform"), (GLM, 200, "zero"),
                                          (synth.Shape(D=512, I=64, E=37, K=4), 29, "uniform"),
                                          (GLM, 300, "uniform"),
                                          (synth.Shape(D=512, I=64, E=37, K=4), 301, "uniform")])
def test_router_topk(shape, S, bias):
    say(f"router D={shape.D} E={shape.E} S={S}")
    cfg_o = config_of(shape)
    cfg = moe.config(shape.D, shape.I, shape.E, shape.K, shape.n_shared, shape.routed_scale)
    wr = synth.router_w(1, shape)
    b = synth.router_b_uniform(1, shape) if bias == "uniform" else np.zeros(shape.E, np.float32)
    x = synth.activations(7, S, shape.D)
    ws = moe.Workspace(cfg, S, moe.WS_ROUTER)
    idx, w, logits = moe.moe_router_topk(cfg, torch.from_numpy(x).cuda(), torch.from_numpy(wr).cuda(),
                                         torch.from_numpy(b).cuda(), ws, want_logits=True)
    ridx, rw, rlogits, rchoice = oracle.router_topk(cfg_o, x, wr, b)
    lg = to_np(logits)
    assert np.abs(lg - rlogits).max() <= 2e-6 * max(1.0, np.abs(rlogits).max())
    uniq = check_routing(to_np(idx), rchoice, shape.K)
    wg = to_np(w)
    assert np.allclose(wg[uniq], rw[uniq], rtol=1e-5, atol=0)
    say(f"  unique routing for {uniq.sum()}/{S} tokens")


@pytest.mark.parametrize("S", [37, 301, 2048])
def test_router_batch_invariance(S):
    # a token's routing does not depend on the batch it is in (37 tokens: the
    # 8 x 8 tiles through shared memory with a ragged last tile; 301: the
    # 16 x 16 tiles with a ragged last tile; 2048: the prefill batch)
    shape = GLM
    cfg = moe.config(shape.D, shape.I, shape.E, shape.K)
    wr = torch.from_numpy(synth.router_w(2, shape)).cuda()
    b = torch.from_numpy(synth.router_b_uniform(2, shape)).cuda()
    x = torch.from_numpy(synth.activations(8, S, shape.D)).cuda()
    ws = moe.Workspace(cfg, S, moe.WS_ROUTER)
    _, _, lg_all = moe.moe_router_topk(cfg, x, wr, b, ws, want_logits=True)
    for s in (0, 5, 36, S - 1):
        _, _, lg1 = moe.moe_router_topk(cfg, x[s:s + 1].contiguous(), wr, b, ws, want_logits=True)
        assert torch.equal(lg1[0], lg_all[s])


# off: byte offset of the code rows; 16-byte aligned rows are read as they
# are, others go through the layout copy first (same results)
@pytest.mark.parametrize("shape,S,off", [(TINY, 4, 0), (TINY, 4, 8), (GLM, 1, 0), (GLM, 1, 8),
                                         (GLM, 3, 0)])
def test_expert_swiglu_parity(shape, S, off):
    say(f"swiglu D={shape.D} I={shape.I} S={S} offset {off}")
    cfg = moe.config(shape.D, shape.I, shape.E, shape.K)
    e_id = 3
    he = host_expert(4, shape, 0, e_id)
    dev = moe.DeviceExperts.empty(shape.E, shape.D, shape.I)
    for name in ("gate_q4", "gate_s", "up_q4", "up_s", "down_q4", "down_s"):
        getattr(dev, name)[e_id].copy_(torch.from_numpy(getattr(he, name)))
    x = synth.activations(9, S, shape.D)
    xq, sx = oracle.quant_act_i8(x)
    ws = moe.Workspace(cfg, S, moe.WS_SWIGLU)
    buf = torch.zeros(xq.size + 16, dtype=torch.int8, device="cuda")
    xq_d = buf[off:off + xq.size].view(S, shape.D)
    xq_d.copy_(torch.from_numpy(xq))
    r = moe.moe_expert_swiglu_i4(cfg, xq_d, torch.from_numpy(sx).cuda(), dev, e_id, ws, probes=True)
    ref = oracle.expert_swiglu(config_of(shape), xq, sx, he)
    assert np.array_equal(to_np(r["acc_gu"]), ref["acc_gu"])
    hq = to_np(r["hq"])
    mism = (hq != ref["hq"])
    say(f"  hq mismatches: {int(mism.sum())} of {hq.size}")
    assert mism.mean() < 1e-3 and np.abs(hq.astype(int) - ref["hq"]).max() <= 1
    assert np.allclose(to_np(r["sh"]), ref["sh"], rtol=1e-6, atol=0)
    acc_d = to_np(r["acc_d"])
    same = ~mism.any(axis=1)
    assert np.array_equal(acc_d[same], ref["acc_d"][same])
    # rows whose codes moved by one step: the GPU's down accumulators are the
    # exact integer products of its own codes
    if (~same).any():
        qd = unpack64(he.down_q4, shape.I).astype(np.int64)
        assert np.array_equal(acc_d[~same], hq[~same].astype(np.int64) @ qd.T)
    assert_close_rows(to_np(r["y"]), ref["y"], what="expert y")


@pytest.mark.parametrize("S,D,offset", [(1, 6144, 0), (4, 6144, 0), (3, 1000, 0), (2, 256, 1),
                                        (1, 9000, 0)])
def test_rmsnorm_matches_oracle(S, D, offset):
    """Section 04 RMSNorm against the oracle's (mean of squares in double),
    on the vector path (aligned rows) and the plain one (offset rows, odd D,
    D > 8192), with a non-unit gain."""
    x = synth.activations(30, S, D) * 3.0
    g = (1.0 + 0.5 * synth.activations(31, 1, D)[0]).astype(np.float32)
    ref = oracle.rmsnorm(x, g, 1e-5)
    xb = torch.zeros(S * D + offset, dtype=torch.float32, device="cuda")
    xb[offset:] = torch.from_numpy(x.ravel()).cuda()
    xt = xb[offset:].view(S, D)
    yb = torch.zeros(S * D + offset, dtype=torch.float32, device="cuda")
    yt = yb[offset:].view(S, D)
    gt = torch.from_numpy(g).cuda()
    moe.moe_rmsnorm(xt, gt, 1e-5, out=yt)
    torch.cuda.synchronize()
    np.testing.assert_allclose(to_np(yt), ref, rtol=2e-6, atol=1e-6)


def test_stream_read_reference():
    """The measurement reference reads the buffer (deterministic sink words,
    sensitive to the data) and rejects misaligned or ragged buffers."""
    buf = torch.arange(1 << 22, dtype=torch.int32, device="cuda")  # 16 MiB
    s1 = moe.moe_stream_read(buf)
    s2 = moe.moe_stream_read(buf)
    buf[12345] += 1
    s3 = moe.moe_stream_read(buf)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2) and not torch.equal(s1, s3)
    with pytest.raises(moe.MoeError, match="misaligned"):
        moe.moe_stream_read(buf[1:5])
    with pytest.raises(moe.MoeError, match="shape"):
        moe.moe_stream_read(buf[:3])
