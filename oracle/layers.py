"""Host-side (oracle) construction of synthetic MoE layers.

TEST INFRASTRUCTURE ONLY.  Weights come from the seeded generator (synth) and
are packed by the oracle's own int4 packer, so nothing here depends on the GPU
library.  Experts are materialized lazily: a full GLM-shape layer holds 257
experts of about 19 MB each, and a check usually needs only the few that the
routing selects.
"""
from __future__ import annotations

import numpy as np

import synth
from . import Config, HostExpert, HostLayer, make_config, router_topk


def config_of(shape: synth.Shape) -> Config:
    return make_config(shape.D, shape.I, shape.E, shape.K, shape.n_shared, shape.routed_scale)


def host_expert(seed: int, shape: synth.Shape, layer: int, expert: int) -> HostExpert:
    g, u, d = synth.host_expert_f32(seed, shape, layer, expert)
    return HostExpert.from_f32(g, u, d)


class LazyLayer(HostLayer):
    """A HostLayer whose routed experts are generated and packed on demand."""

    def __init__(self, seed: int, shape: synth.Shape, layer: int, router_b: np.ndarray,
                 router_w: np.ndarray | None = None):
        cfg = config_of(shape)
        wr = synth.router_w(seed, shape, layer) if router_w is None else router_w
        shared = host_expert(seed, shape, layer, synth.SHARED) if shape.n_shared else None
        super().__init__(cfg, wr, router_b, {}, shared)
        self.seed, self.shape, self.layer = seed, shape, layer

    def ensure(self, ids, workers: int = 1) -> None:
        """Materialize the listed experts; with workers > 1 they are generated
        and packed by that many threads (the generator and the packer are C
        calls that run outside the interpreter lock)."""
        todo = [e for e in sorted(set(int(i) for i in np.asarray(ids).ravel()))
                if e not in self.experts]
        if workers <= 1 or len(todo) < 2:
            for e in todo:
                self.experts[e] = host_expert(self.seed, self.shape, self.layer, e)
            return
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=workers) as ex:
            made = ex.map(lambda e: (e, host_expert(self.seed, self.shape, self.layer, e)), todo)
            for e, h in made:
                self.experts[e] = h

    def ensure_for(self, x: np.ndarray) -> np.ndarray:
        """Route x with the oracle router and materialize the selected experts."""
        idx, _, _, _ = router_topk(self.cfg, x, self.router_w, self.router_b)
        self.ensure(idx)
        return idx

    def drop_routed(self) -> None:
        self.experts.clear()


def bias_for(recipe: str, seed: int, shape: synth.Shape, layer: int = 0, beta: float = 0.0):
    if recipe == "uniform":
        return synth.router_b_uniform(seed, shape, layer)
    if recipe == "zero":
        return np.zeros(shape.E, np.float32)
    if recipe == "zipf":
        return synth.zipf_bias(seed, shape.E, layer, beta)
    raise ValueError(recipe)
