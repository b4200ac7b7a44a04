"""Pins of the oracle's expert-cache and tier-policy functions (article
section 05 expert cache; section 13 swap margin and frequency-first score)
against independent formulations: a textbook LRU list, brute-force argmax
and argmin, and closed forms."""
import numpy as np
import pytest

import oracle


def lru_list_model(seq, cap):
    """Textbook LRU over slot numbers: residents kept in recency order (oldest
    first); a miss fills the next never-used slot while there is one, else
    the oldest resident's slot."""
    order = []      # expert ids, least recent first
    slot_of = {}
    out = []
    for e in seq:
        if e in slot_of:
            order.remove(e)
            order.append(e)
            out.append((slot_of[e], 0))
            continue
        if len(slot_of) < cap:
            s = len(slot_of)
        else:
            victim = order.pop(0)
            s = slot_of.pop(victim)
        slot_of[e] = s
        order.append(e)
        out.append((s, 1))
    return out


@pytest.mark.parametrize("cap,n,E,seed", [(1, 50, 4, 0), (3, 200, 8, 1), (8, 500, 40, 2),
                                         (16, 2000, 256, 3)])
def test_expert_get_matches_lru_list(cap, n, E, seed):
    rng = np.random.default_rng(seed)
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    seq = rng.choice(E, size=n, p=p / p.sum())
    c = oracle.ExpertCache(1, cap)
    got = [c.get(0, int(e)) for e in seq]
    assert got == lru_list_model(seq.tolist(), cap)
    assert c.hits + c.misses == n
    assert c.misses == sum(l for _, l in got)


def test_expert_get_layers_are_separate_and_share_the_counters():
    c = oracle.ExpertCache(2, 2)
    assert c.get(0, 5) == (0, 1)
    assert c.get(1, 5) == (0, 1)   # another layer's cache: a miss of its own
    assert c.get(0, 5) == (0, 0)
    assert c.get(0, 7) == (1, 1)
    assert c.get(0, 9) == (0, 1)   # evicts expert 5 (used before 7)
    assert (c.hits, c.misses) == (1, 4)
    assert int(c.counters[0]) == 5  # one clock tick per lookup


def test_expert_get_warm_cache_only_misses_on_first_use():
    rng = np.random.default_rng(4)
    seq = rng.integers(0, 12, size=300)
    c = oracle.ExpertCache(1, 12)
    for e in seq:
        c.get(0, int(e))
    assert c.misses == len(set(seq.tolist()))


def brute_swap(heat, pinned):
    heat = [int(h) for h in heat]
    cold = min(range(len(pinned)), key=lambda z: (heat[pinned[z]], z))
    outside = [e for e in range(len(heat)) if e not in set(pinned) and heat[e] > 0]
    if not outside:
        return False, -1, -1, 0
    hot = min(outside, key=lambda e: (-heat[e], e))
    fc = heat[pinned[cold]]
    if 4 * heat[hot] <= 5 * fc + 16 - (fc % 4):   # heat > fc + floor(fc/4) + 4
        return False, -1, -1, 0
    return True, cold, hot, heat[hot] - fc


def test_pick_swap_margin_boundaries():
    # fc = 0: the newcomer needs heat 5 or more
    assert oracle.tier_pick_swap([0, 4, 0], [0])[0] is False
    assert oracle.tier_pick_swap([0, 5, 0], [0]) == (True, 0, 1, 5)
    # fc = 100: bound 100 + 25 + 4 = 129
    assert oracle.tier_pick_swap([100, 129], [0])[0] is False
    assert oracle.tier_pick_swap([100, 130], [0]) == (True, 0, 1, 30)
    # fc = 7: floor(7/4) = 1, bound 12
    assert oracle.tier_pick_swap([7, 12], [0])[0] is False
    assert oracle.tier_pick_swap([7, 13], [0])[0] is True
    # nothing outside the pinned set, or nothing hot outside it
    assert oracle.tier_pick_swap([3, 9], [0, 1])[0] is False
    assert oracle.tier_pick_swap([3, 0, 0], [0])[0] is False


@pytest.mark.parametrize("seed", range(6))
def test_pick_swap_brute_force(seed):
    rng = np.random.default_rng(10 + seed)
    E = int(rng.integers(2, 60))
    heat = rng.integers(0, 40, size=E).astype(np.uint32)
    npin = int(rng.integers(1, E))
    pinned = rng.permutation(E)[:npin].astype(np.int32)
    assert oracle.tier_pick_swap(heat, pinned) == brute_swap(heat, pinned.tolist())


def test_lfru_score_closed_forms():
    s = oracle.tier_lfru_score
    assert s(0, 10, 10) == 255
    assert s(3, 10, 10) == 3 * 256 + 255
    assert s(3, 10, 264) == 3 * 256 + 1      # age 254
    assert s(3, 10, 265) == 3 * 256          # age 255: no recency left
    assert s(3, 10, 10 ** 6) == 3 * 256
    assert s(1, 2 ** 32 - 3, 2) == 256 + 250  # the clock wrapped: age 5
    # heat dominates recency
    assert s(5, 0, 10 ** 6) > s(4, 7, 7)
