"""The library's expert-tier bookkeeping (host code, no GPU) makes the same
decisions as the oracle's section 05 expert cache and section 13 swap rule
and score on the same inputs; host checks reject what they must."""
import numpy as np
import pytest

import int4_expert_gemv_moe_amd as moe
import oracle


@pytest.mark.parametrize("n_layers,E,n_slots,calls,per_call,seed",
                         [(1, 8, 3, 60, 2, 0), (2, 64, 16, 200, 8, 1), (3, 256, 64, 300, 9, 2),
                          (1, 256, 9, 100, 9, 3)])
def test_tier_map_matches_oracle_expert_cache(n_layers, E, n_slots, calls, per_call, seed):
    rng = np.random.default_rng(seed)
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    p /= p.sum()
    t = moe.Tier(n_layers, E, n_slots)
    c = oracle.ExpertCache(n_layers, n_slots)
    for _ in range(calls):
        layer = int(rng.integers(0, n_layers))
        eids = rng.choice(E, size=per_call, replace=False, p=p).astype(np.int32)
        slots, loads, misses = t.map(layer, eids)
        ref = [c.get(layer, int(e)) for e in eids]
        assert slots.tolist() == [r[0] for r in ref]
        assert loads.tolist() == [r[1] for r in ref]
        assert misses == sum(r[1] for r in ref)
        # the experts of one call sit in distinct slots
        assert len(set(slots.tolist())) == per_call
    assert t.stats() == (c.hits, c.misses)


def test_tier_map_rejections_leave_state_unchanged():
    t = moe.Tier(2, 16, 4)
    t.map(0, [1, 2])
    with pytest.raises(moe.MoeError):
        t.map(0, [1, 2, 3, 4, 5])          # more experts than slots
    with pytest.raises(moe.MoeError):
        t.map(0, [3, 16])                  # expert outside the layer
    with pytest.raises(moe.MoeError):
        t.map(2, [0])                      # no such layer
    assert t.stats() == (0, 2)
    slots, loads, _ = t.map(0, [2, 1])
    assert loads.tolist() == [0, 0] and sorted(slots.tolist()) == [0, 1]


@pytest.mark.parametrize("seed", range(8))
def test_pick_swap_matches_oracle(seed):
    rng = np.random.default_rng(100 + seed)
    E = int(rng.integers(2, 300))
    heat = rng.integers(0, int(rng.choice([6, 50, 5000])), size=E).astype(np.uint32)
    npin = int(rng.integers(1, E))
    pinned = rng.permutation(E)[:npin].astype(np.int32)
    assert moe.tier_pick_swap(heat, pinned) == oracle.tier_pick_swap(heat, pinned)


def test_lfru_score_matches_oracle():
    rng = np.random.default_rng(7)
    for _ in range(500):
        h, last, clock = (int(v) for v in rng.integers(0, 2 ** 32, size=3, dtype=np.uint64))
        if rng.random() < 0.5:
            clock = (last + int(rng.integers(0, 400))) % 2 ** 32
        assert moe.tier_lfru_score(h, last, clock) == oracle.tier_lfru_score(h, last, clock)


def test_slab_layout_closed_form():
    for D, I in ((6144, 2048), (256, 128), (256, 32)):
        lay = moe.slab_layout(moe.config(D, I, 8, 2))
        gu, dn = I * D // 2, D * I // 2
        assert (lay.gate_q4, lay.up_q4, lay.down_q4) == (0, gu, 2 * gu)
        assert (lay.gate_s, lay.up_s, lay.down_s) == (2 * gu + dn, 2 * gu + dn + 4 * I,
                                                     2 * gu + dn + 8 * I)
        assert lay.bytes == 3 * I * D // 2 + 4 * (2 * I + D)
        assert all(v % 16 == 0 for v in (lay.up_q4, lay.down_q4, lay.gate_s, lay.up_s, lay.down_s,
                                         lay.bytes))
    assert moe.slab_layout(moe.config(6144, 2048, 256, 8)).bytes == 18_915_328


class PinnedRef:
    """The pinned tier composed from the oracle's parts: heat = lookups so far,
    pinned slots checked first, the section 05 expert cache behind them
    (slots numbered after the pinned ones), and per rebalance either the
    hottest unpinned expert into an empty pinned slot or the section 13 swap."""

    def __init__(self, E, n_lru, n_pin):
        self.E, self.np = E, n_pin
        self.pinned = [-1] * n_pin
        self.heat = np.zeros(E, np.uint32)
        self.cache = oracle.ExpertCache(1, n_lru)
        self.pin_hits = 0

    def map(self, eids):
        slots, loads = [], []
        for e in eids:
            self.heat[e] += 1
            if e in self.pinned:
                slots.append(self.pinned.index(e))
                loads.append(0)
                self.pin_hits += 1
            else:
                s, l = self.cache.get(0, int(e))
                slots.append(self.np + s)
                loads.append(l)
        return slots, loads

    def rebalance(self):
        if -1 in self.pinned:
            z = self.pinned.index(-1)
            free = [e for e in range(self.E) if e not in self.pinned and self.heat[e] > 0]
            if not free:
                return False, -1, -1, -1
            hot = min(free, key=lambda e: (-int(self.heat[e]), e))
            self.pinned[z] = hot
            return True, z, hot, -1
        ok, z, e, _ = oracle.tier_pick_swap(self.heat, self.pinned)
        if not ok:
            return False, -1, -1, -1
        old = self.pinned[z]
        self.pinned[z] = e
        return True, z, e, old


@pytest.mark.parametrize("E,n_lru,n_pin,calls,per_call,seed", [(16, 4, 2, 80, 2, 0),
                                                                (256, 128, 64, 400, 8, 1),
                                                                (64, 12, 8, 300, 8, 2)])
def test_pinned_tier_matches_composed_oracle(E, n_lru, n_pin, calls, per_call, seed):
    rng = np.random.default_rng(seed)
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    p /= p.sum()
    t = moe.Tier(1, E, n_lru, n_pin)
    ref = PinnedRef(E, n_lru, n_pin)
    swaps = 0
    for _ in range(calls):
        eids = rng.choice(E, size=per_call, replace=False, p=p).astype(np.int32)
        slots, loads, misses = t.map(0, eids)
        rs, rl = ref.map(eids.tolist())
        assert slots.tolist() == rs and loads.tolist() == rl and misses == sum(rl)
        got = t.rebalance(0)
        assert got == ref.rebalance()
        swaps += got[0] and got[3] >= 0
    assert t.stats() == (ref.cache.hits + ref.pin_hits, ref.cache.misses)
    assert all(e >= 0 for e in ref.pinned) and len(set(ref.pinned)) == n_pin
