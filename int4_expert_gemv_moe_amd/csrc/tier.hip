// tier.hip -- expert residency between pinned host memory and HBM slots
// (reader.mx article "惊呆了！25GB 内存上运行 GLM 5.2 744B 模型": section 05,
// the per-layer expert cache and its get rule; section 13, the five residency
// tiers, the 25 % + 4 swap margin, the frequency-first score and the one-read
// expert slab).
//
// On one MI355X the tiers are: HBM slots (a fixed number per layer, each one
// expert slab) and pinned host memory holding every expert's slab.  The
// routing of a call is known on the host before its experts are needed (the
// router call runs first), so the host maps the call's experts to slots, the
// missing slabs are copied in with one DMA each, and the per-token block then
// runs on the slot stack with the given routing.  Everything here is host
// code: bookkeeping plus the copies it enqueues.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <new>
#include <vector>

#include "../../include/moe_i4.h"

struct moe_tier {
  int n_layers, n_experts, n_slots;  // n_slots: the LRU slots of a layer
  int n_pinned = 0;                  // heat-managed slots of a layer, numbered first
  // per layer and LRU slot: the expert it holds (-1: empty) and the clock
  // value of its last use
  std::vector<int32_t> slot_eid;
  std::vector<uint64_t> slot_used;
  // per layer and expert: the LRU slot holding it (-1: none), so a lookup
  // does not scan the slots
  std::vector<int32_t> where;
  // per layer: the expert of each pinned slot (-1: empty) and every expert's
  // heat (lookups so far)
  std::vector<int32_t> pinned;
  std::vector<uint32_t> heat;
  uint64_t clock = 0, hits = 0, misses = 0;
};

namespace {

// The LRU slot a missing expert takes: the lowest empty slot while there is
// one (slots fill in order 0, 1, ...), else the least recently used slot,
// the lowest among equals.
int lru_victim(const int32_t *eid, const uint64_t *used, int n) {
  int v = -1;
  for (int z = 0; z < n; z++) {
    if (eid[z] < 0) return z;
    if (v < 0 || used[z] < used[v]) v = z;
  }
  return v;
}

}  // namespace

extern "C" {

int moe_slab_layout_of(const moe_config *cfg, moe_slab_layout *out) {
  if (!cfg || !out) return MOE_EINVAL;
  if (cfg->D < 2 || cfg->I < 2 || (cfg->D & 31) || (cfg->I & 31)) return MOE_ESHAPE;
  const int64_t gu = (int64_t)cfg->I * (cfg->D / 2), dn = (int64_t)cfg->D * (cfg->I / 2);
  // the three packed matrices, then the three scale vectors; every piece
  // starts on a 16-byte boundary (D and I are multiples of 32)
  out->gate_q4 = 0;
  out->up_q4 = gu;
  out->down_q4 = 2 * gu;
  out->gate_s = 2 * gu + dn;
  out->up_s = out->gate_s + 4 * (int64_t)cfg->I;
  out->down_s = out->up_s + 4 * (int64_t)cfg->I;
  out->bytes = out->down_s + 4 * (int64_t)cfg->D;
  return MOE_OK;
}

moe_tier *moe_tier_create(int n_layers, int n_experts, int n_slots) {
  if (n_layers < 1 || n_experts < 1 || n_slots < 1) return nullptr;
  moe_tier *t = new (std::nothrow) moe_tier;
  if (!t) return nullptr;
  t->n_layers = n_layers;
  t->n_experts = n_experts;
  t->n_slots = n_slots;
  try {
    t->slot_eid.assign((size_t)n_layers * n_slots, -1);
    t->slot_used.assign((size_t)n_layers * n_slots, 0);
    t->where.assign((size_t)n_layers * n_experts, -1);
  } catch (...) {
    delete t;
    return nullptr;
  }
  return t;
}

moe_tier *moe_tier_create_pinned(int n_layers, int n_experts, int n_lru, int n_pinned) {
  if (n_pinned < 0 || n_pinned >= n_experts) return nullptr;
  moe_tier *t = moe_tier_create(n_layers, n_experts, n_lru);
  if (!t) return nullptr;
  t->n_pinned = n_pinned;
  try {
    t->pinned.assign((size_t)n_layers * n_pinned, -1);
    t->heat.assign((size_t)n_layers * n_experts, 0u);
  } catch (...) {
    delete t;
    return nullptr;
  }
  return t;
}

void moe_tier_destroy(moe_tier *t) { delete t; }

int moe_tier_map(moe_tier *t, int layer, const int32_t *eids, int n, int32_t *slots,
                 int32_t *loads) {
  if (!t || !eids || !slots || !loads) return MOE_EINVAL;
  if (layer < 0 || layer >= t->n_layers || n < 0) return MOE_EINVAL;
  // every expert of the call must stay resident until the call has run: a
  // slot taken or refreshed in this call carries a newer clock than any other
  // slot, so with n <= n_slots no eviction hits one of them
  if (n > t->n_slots) return MOE_ESHAPE;
  for (int i = 0; i < n; i++)
    if (eids[i] < 0 || eids[i] >= t->n_experts) return MOE_EINVAL;
  int32_t *eid = t->slot_eid.data() + (size_t)layer * t->n_slots;
  uint64_t *used = t->slot_used.data() + (size_t)layer * t->n_slots;
  int32_t *where = t->where.data() + (size_t)layer * t->n_experts;
  const int np = t->n_pinned;
  const int32_t *pin = np ? t->pinned.data() + (size_t)layer * np : nullptr;
  uint32_t *heat = np ? t->heat.data() + (size_t)layer * t->n_experts : nullptr;
  int misses = 0;
  for (int i = 0; i < n; i++) {
    const int32_t e = eids[i];
    if (heat) heat[e]++;
    // a pinned expert is a hit in its pinned slot (slots 0 .. n_pinned-1)
    int z = 0;
    while (z < np && pin[z] != e) z++;
    loads[i] = 0;
    if (z < np) {
      t->hits++;
      slots[i] = z;
      continue;
    }
    z = where[e];
    if (z >= 0) {
      t->hits++;
    } else {
      t->misses++;
      misses++;
      z = lru_victim(eid, used, t->n_slots);
      if (eid[z] >= 0) where[eid[z]] = -1;  // evicted
      eid[z] = e;
      where[e] = z;
      loads[i] = 1;
    }
    used[z] = ++t->clock;
    slots[i] = np + z;
  }
  return misses;
}

int moe_tier_rebalance(moe_tier *t, int layer, int32_t *slot, int32_t *eid, int32_t *old_eid) {
  if (!t || !slot || !eid || !old_eid || layer < 0 || layer >= t->n_layers) return MOE_EINVAL;
  const int np = t->n_pinned;
  if (np == 0) return 0;
  int32_t *pin = t->pinned.data() + (size_t)layer * np;
  const uint32_t *heat = t->heat.data() + (size_t)layer * t->n_experts;
  // an empty pinned slot takes the hottest expert not pinned (heat > 0,
  // first of equals)
  for (int z = 0; z < np; z++) {
    if (pin[z] >= 0) continue;
    int hot = -1;
    uint32_t hh = 0;
    for (int e = 0; e < t->n_experts; e++) {
      bool held = false;
      for (int y = 0; y < np; y++) held = held || pin[y] == e;
      if (!held && heat[e] > hh) {
        hh = heat[e];
        hot = e;
      }
    }
    if (hot < 0) return 0;
    *slot = z;
    *eid = hot;
    *old_eid = -1;
    pin[z] = hot;
    return 1;
  }
  // all filled: the section 13 swap rule
  int32_t z, e;
  int64_t gain;
  if (!moe_tier_pick_swap(heat, t->n_experts, pin, np, &z, &e, &gain)) return 0;
  *slot = z;
  *eid = e;
  *old_eid = pin[z];
  pin[z] = e;
  return 1;
}

int moe_tier_stats(const moe_tier *t, uint64_t *hits, uint64_t *misses) {
  if (!t) return MOE_EINVAL;
  if (hits) *hits = t->hits;
  if (misses) *misses = t->misses;
  return MOE_OK;
}

int moe_tier_fetch(const void *host_slabs, void *hbm_slots, size_t slab_bytes,
                   const int32_t *eids, const int32_t *slots, const int32_t *loads, int n,
                   hipStream_t stream) {
  if (!host_slabs || !hbm_slots || !eids || !slots || !loads || n < 0) return MOE_EINVAL;
  if (slab_bytes == 0 || (slab_bytes & 15u)) return MOE_EALIGN;
  for (int i = 0; i < n; i++) {
    if (!loads[i]) continue;
    if (eids[i] < 0 || slots[i] < 0) return MOE_EINVAL;
    const char *src = static_cast<const char *>(host_slabs) + (size_t)eids[i] * slab_bytes;
    char *dst = static_cast<char *>(hbm_slots) + (size_t)slots[i] * slab_bytes;
    if (hipMemcpyAsync(dst, src, slab_bytes, hipMemcpyHostToDevice, stream) != hipSuccess)
      return MOE_EHIP;
  }
  return MOE_OK;
}

int moe_tier_pick_swap(const uint32_t *heat, int n_experts, const int32_t *pinned, int n_pinned,
                       int32_t *slot, int32_t *eid, int64_t *gain) {
  if (!heat || !pinned || !slot || !eid || !gain || n_pinned < 1 || n_experts < 1) return 0;
  for (int z = 0; z < n_pinned; z++)
    if (pinned[z] < 0 || pinned[z] >= n_experts) return 0;
  // coldest pinned expert (first of equals)
  int cold = 0;
  for (int z = 1; z < n_pinned; z++)
    if (heat[pinned[z]] < heat[pinned[cold]]) cold = z;
  // hottest expert not pinned (first of equals)
  std::vector<char> is_pinned((size_t)n_experts, 0);
  for (int z = 0; z < n_pinned; z++) is_pinned[pinned[z]] = 1;
  int hot = -1;
  uint32_t hot_heat = 0;
  for (int e = 0; e < n_experts; e++)
    if (!is_pinned[e] && heat[e] > hot_heat) {
      hot_heat = heat[e];
      hot = e;
    }
  if (hot < 0) return 0;
  // the newcomer must beat the coldest by a quarter of its heat plus 4
  const uint64_t cold_heat = heat[pinned[cold]];
  if ((uint64_t)hot_heat <= cold_heat + (cold_heat >> 2) + 4) return 0;
  *slot = cold;
  *eid = hot;
  *gain = (int64_t)hot_heat - (int64_t)cold_heat;
  return 1;
}

uint64_t moe_tier_lfru_score(uint32_t heat, uint32_t last, uint32_t clock) {
  // frequency first; recency (255 steps, newest highest) only orders equal heat
  const uint32_t age = clock - last;
  const uint32_t recent = age < 255u ? 255u - age : 0u;
  return ((uint64_t)heat << 8) | recent;
}

}  // extern "C"

namespace moe {

void tier_sizes(const moe_tier *t, int *n_experts, int *n_slot_total) {
  *n_experts = t->n_experts;
  *n_slot_total = t->n_pinned + t->n_slots;
}

// Undo the loads of one moe_tier_map call whose copies were not enqueued: the
// LRU slots it filled become empty again (they are taken first by the next
// miss), so no later lookup finds an expert whose slab never arrived.
void tier_unmap_loads(moe_tier *t, int layer, const int32_t *eids, const int32_t *slots,
                      const int32_t *loads, int n) {
  int32_t *eid = t->slot_eid.data() + (size_t)layer * t->n_slots;
  uint64_t *used = t->slot_used.data() + (size_t)layer * t->n_slots;
  int32_t *where = t->where.data() + (size_t)layer * t->n_experts;
  for (int i = 0; i < n; i++) {
    if (!loads[i]) continue;
    const int z = slots[i] - t->n_pinned;
    if (z < 0 || z >= t->n_slots || eid[z] != eids[i]) continue;
    where[eids[i]] = -1;
    eid[z] = -1;
    used[z] = 0;
  }
}

}  // namespace moe
