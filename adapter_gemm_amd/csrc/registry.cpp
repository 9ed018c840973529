// Adapter residency: which adapter occupies which pool slot ("LLM-stack
// book" 7.14.4, the adapter registry: name -> slot, reference counts of
// in-flight use, eviction of a resident adapter that no batch uses, LRU by
// default or LFU by per-adapter hit count; 7.14.3, loading a slot with an
// asynchronous copy on a side stream).  Host-side bookkeeping only; the copy
// into a slot is lora_pool_install.
#include <cstdint>
#include <unordered_map>
#include <vector>

#include "lora.h"

struct lora_registry {
  int32_t n_slots = 0;
  int32_t policy = LORA_EVICT_LRU;
  uint64_t clock = 0;
  std::unordered_map<int64_t, int32_t> slot_of;   // resident adapter -> slot
  std::unordered_map<int64_t, uint64_t> hits;     // uses per adapter, kept across evictions (LFU)
  std::vector<int64_t> key_of;                    // slot -> adapter, or -1
  std::vector<int32_t> ref;                       // in-flight uses per slot
  std::vector<uint64_t> last_use;                 // clock of the last acquire per slot
  int64_t n_hits = 0, n_misses = 0, n_evictions = 0;
};

namespace {

// The slot a miss takes: the lowest free slot, else the victim the policy
// picks among slots no batch uses (LRU: oldest last use; LFU: fewest hits,
// then oldest), else -1.
int32_t pick_slot(const lora_registry& r) {
  int32_t best = -1;
  for (int32_t s = 0; s < r.n_slots; ++s) {
    if (r.key_of[s] < 0) return s;
    if (r.ref[s] > 0) continue;
    if (best < 0) {
      best = s;
      continue;
    }
    if (r.policy == LORA_EVICT_LFU) {
      const uint64_t hs = r.hits.at(r.key_of[s]), hb = r.hits.at(r.key_of[best]);
      if (hs < hb || (hs == hb && r.last_use[s] < r.last_use[best])) best = s;
    } else if (r.last_use[s] < r.last_use[best]) {
      best = s;
    }
  }
  return best;
}

}  // namespace

extern "C" {

int lora_registry_create(int32_t n_slots, int32_t policy, lora_registry_t** out) {
  if (!out) return LORA_E_ARG;
  *out = nullptr;
  if (n_slots <= 0 || (policy != LORA_EVICT_LRU && policy != LORA_EVICT_LFU)) return LORA_E_ARG;
  lora_registry* r = new lora_registry;
  r->n_slots = n_slots;
  r->policy = policy;
  r->key_of.assign(n_slots, -1);
  r->ref.assign(n_slots, 0);
  r->last_use.assign(n_slots, 0);
  *out = r;
  return LORA_OK;
}

void lora_registry_destroy(lora_registry_t* r) { delete r; }

int lora_registry_acquire(lora_registry_t* r, int64_t key, int32_t* slot, int32_t* needs_install) {
  if (!r || !slot || !needs_install || key < 0) return LORA_E_ARG;
  *slot = -1;
  *needs_install = 0;
  ++r->clock;
  auto it = r->slot_of.find(key);
  if (it != r->slot_of.end()) {                 // resident
    const int32_t s = it->second;
    ++r->ref[s];
    r->last_use[s] = r->clock;
    ++r->hits[key];
    ++r->n_hits;
    *slot = s;
    return LORA_OK;
  }
  const int32_t s = pick_slot(*r);
  if (s < 0) return LORA_E_SIZE;               // every slot holds an adapter in use
  if (r->key_of[s] >= 0) {
    r->slot_of.erase(r->key_of[s]);
    ++r->n_evictions;
  }
  r->key_of[s] = key;
  r->slot_of[key] = s;
  r->ref[s] = 1;
  r->last_use[s] = r->clock;
  ++r->hits[key];
  ++r->n_misses;
  *slot = s;
  *needs_install = 1;
  return LORA_OK;
}

int lora_registry_release(lora_registry_t* r, int64_t key) {
  if (!r) return LORA_E_ARG;
  auto it = r->slot_of.find(key);
  if (it == r->slot_of.end() || r->ref[it->second] == 0) return LORA_E_ARG;
  --r->ref[it->second];
  return LORA_OK;
}

int lora_registry_lookup(const lora_registry_t* r, int64_t key, int32_t* slot) {
  if (!r || !slot) return LORA_E_ARG;
  auto it = r->slot_of.find(key);
  *slot = it == r->slot_of.end() ? -1 : it->second;
  return LORA_OK;
}

int lora_registry_stats(const lora_registry_t* r, int64_t* out4) {
  if (!r || !out4) return LORA_E_ARG;
  out4[0] = r->n_hits;
  out4[1] = r->n_misses;
  out4[2] = r->n_evictions;
  out4[3] = (int64_t)r->slot_of.size();
  return LORA_OK;
}

}  // extern "C"
