"""A stack of MoE layers on one residual stream, in the layer order of
section 04 of the reader.mx article "惊呆了！25GB 内存上运行 GLM 5.2 744B 模型":
for every layer, x <- x + block(rmsnorm(x)).

Each layer is one library call on the caller's stream: moe_layer_forward (or
moe_layer_forward_batch, the unique-expert union) with MOE_F_PRENORM and
MOE_F_ACCUMULATE on x in place; the per-token path normalizes inside its
first launch.  With fused=False the normalization is a moe_rmsnorm call
into a scratch row block first (the same bits).  The calls take prebuilt
argument structs, so a step is cheap to issue and can be captured in a HIP
graph as it is.
"""
from __future__ import annotations

import ctypes

import torch

from . import F_ACCUMULATE, F_PRENORM, DeviceLayer, MoeError, Probe, Workspace, _check, _dev, lib


class Stack:
    def __init__(self, layers: list[DeviceLayer], gamma: torch.Tensor, eps: float = 1e-5):
        if not layers:
            raise MoeError("empty stack")
        cfg = layers[0].cfg
        for l in layers:
            if (l.cfg.D, l.cfg.I, l.cfg.E, l.cfg.K) != (cfg.D, cfg.I, cfg.E, cfg.K):
                raise MoeError("stack layers must share one shape")
        _dev(gamma, torch.float32, "gamma")
        if gamma.numel() != cfg.D:
            raise MoeError("gamma must hold D values")
        self.layers = layers
        self.cfg = cfg
        self.gamma = gamma
        self.eps = float(eps)
        self._lc = [l.cstruct(gamma, self.eps) for l in layers]  # kept alive for the calls

    def forward(self, x: torch.Tensor, ws: Workspace, xn: torch.Tensor | None = None,
                union: bool = False, stream=None, taps: list | None = None,
                topk_idx: list | None = None, fused: bool = True) -> torch.Tensor:
        """Runs every layer on x [S][D] (float32, updated in place).

        union: use the unique-expert union path.  fused: normalize inside the
        layer call (else a separate moe_rmsnorm into xn, allocated if
        omitted).  taps[l] (optional tensors of x's shape) receive x before
        layer l, topk_idx[l] (int32 [S][K]) its selection; both are written
        on the given stream."""
        _dev(x, torch.float32, "x")
        S, D = x.shape
        if D != self.cfg.D:
            raise MoeError("x has the wrong width")
        if not fused:
            xn = torch.empty_like(x) if xn is None else xn
        L = lib()
        fn = L.moe_layer_forward_batch if union else L.moe_layer_forward
        s = torch.cuda.current_stream() if stream is None else stream
        st = ctypes.c_void_p(s.cuda_stream)
        xp, gp = ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(self.gamma.data_ptr())
        xnp = None if fused else ctypes.c_void_p(xn.data_ptr())
        cref = ctypes.byref(self.cfg)
        for i, lc in enumerate(self._lc):
            if taps is not None:
                with torch.cuda.stream(s):
                    taps[i].copy_(x)
            probe = None
            if topk_idx is not None:
                p = Probe()
                p.topk_idx = topk_idx[i].data_ptr()
                probe = ctypes.byref(p)
            if fused:
                _check(fn(cref, ctypes.byref(lc), xp, S, xp, F_ACCUMULATE | F_PRENORM, probe, ws.ptr,
                          ws.nbytes, st), "moe_layer_forward")
            else:
                _check(L.moe_rmsnorm(xp, gp, S, D, self.eps, xnp, st), "moe_rmsnorm")
                _check(fn(cref, ctypes.byref(lc), xnp, S, xp, F_ACCUMULATE, probe, ws.ptr, ws.nbytes,
                          st), "moe_layer_forward")
        return x
