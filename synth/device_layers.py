"""GPU-side construction of synthetic MoE layers.

Float weights are drawn on the device by the seeded generator (the same bits
the host generator gives), one matrix at a time into a float32 staging
buffer, and packed to the int4 container by the library's own packer
(moe_pack_int4).  A full GLM-shape layer (257 experts, about 4.86 GB) is built
in well under a second without the host ever holding it.
"""
from __future__ import annotations

import numpy as np
import torch

import int4_expert_gemv_moe_amd as moe
import synth


def build_device_layer(seed: int, shape: synth.Shape, layer: int, router_b: np.ndarray,
                       router_w: np.ndarray | None = None, device: str = "cuda") -> moe.DeviceLayer:
    D, I, E = shape.D, shape.I, shape.E
    st = torch.cuda.current_stream().cuda_stream
    cfg = moe.config(D, I, E, shape.K, shape.n_shared, shape.routed_scale)
    if router_w is None:
        wr = torch.empty(E, D, dtype=torch.float32, device=device)
        synth.dev_fill_normal(wr.data_ptr(), seed, synth.stream(synth.K_ROUTER_W, layer), E * D,
                              synth.WEIGHT_SIGMA, st)
    else:
        wr = torch.from_numpy(np.ascontiguousarray(router_w, np.float32)).to(device)
    rb = torch.from_numpy(np.ascontiguousarray(router_b, np.float32)).to(device)
    routed = moe.DeviceExperts.empty(E, D, I, device)
    shared = moe.DeviceExperts.empty(1, D, I, device) if shape.n_shared else None
    tmp = torch.empty(max(I * D, D * I), dtype=torch.float32, device=device)

    def fill(dst: moe.DeviceExperts, slot: int, item: int):
        sg, su, sd = synth.expert_streams(layer, item)
        for strm, q4, sc, O, C in ((sg, dst.gate_q4, dst.gate_s, I, D), (su, dst.up_q4, dst.up_s, I, D),
                                   (sd, dst.down_q4, dst.down_s, D, I)):
            synth.dev_fill_normal(tmp.data_ptr(), seed, strm, O * C, synth.WEIGHT_SIGMA, st)
            moe.moe_pack_int4(tmp[: O * C].view(O, C), q4[slot], sc[slot])

    for e in range(E):
        fill(routed, e, e)
    if shared is not None:
        fill(shared, 0, synth.SHARED)
    del tmp
    return moe.DeviceLayer(cfg, wr, rb, routed, shared)


def build_device_experts_i8(seed: int, shape: synth.Shape, layer: int, n: int,
                            device: str = "cuda") -> moe.DeviceExpertsI8:
    """n experts of the shape in the int8 weight format, drawn from the same
    streams as experts 0..n-1 of the layer and quantized by the library's
    section 05 quantizer (moe_quantize_rows_i8)."""
    D, I = shape.D, shape.I
    st = torch.cuda.current_stream().cuda_stream
    out = moe.DeviceExpertsI8.empty(n, D, I, device)
    tmp = torch.empty(I * D, dtype=torch.float32, device=device)
    for e in range(n):
        sg, su, sd = synth.expert_streams(layer, e)
        for strm, q, sc, O, C in ((sg, out.gate_q, out.gate_s, I, D), (su, out.up_q, out.up_s, I, D),
                                  (sd, out.down_q, out.down_s, D, I)):
            synth.dev_fill_normal(tmp.data_ptr(), seed, strm, O * C, synth.WEIGHT_SIGMA, st)
            moe.moe_quantize_rows_i8(tmp[: O * C].view(O, C), q[e], sc[e])
    del tmp
    return out


def build_device_experts_i2(seed: int, shape: synth.Shape, layer: int, n: int,
                            device: str = "cuda") -> moe.DeviceExpertsI2:
    """n experts of the shape in the packed int2 format (moe_pack_int2), drawn
    from the same streams as experts 0..n-1 of the layer."""
    D, I = shape.D, shape.I
    st = torch.cuda.current_stream().cuda_stream
    out = moe.DeviceExpertsI2.empty(n, D, I, device)
    tmp = torch.empty(I * D, dtype=torch.float32, device=device)
    for e in range(n):
        sg, su, sd = synth.expert_streams(layer, e)
        for strm, q, sc, O, C in ((sg, out.gate_q2, out.gate_s, I, D),
                                  (su, out.up_q2, out.up_s, I, D),
                                  (sd, out.down_q2, out.down_s, D, I)):
            synth.dev_fill_normal(tmp.data_ptr(), seed, strm, O * C, synth.WEIGHT_SIGMA, st)
            moe.moe_pack_int2(tmp[: O * C].view(O, C), q[e], sc[e])
    del tmp
    return out
