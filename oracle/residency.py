"""Adapter residency rules of a slot registry (integer bookkeeping).

Test infrastructure only.  From "LLM-stack book 7.14 Multi-Tenant LoRA &
Adapter Serving at Scale":

* 7.14.4 The Adapter Registry, Eviction & Fairness: the registry maps an
  adapter to the GPU slot that holds it and counts the uses in flight; when a
  new adapter needs a slot and none is free, it evicts a resident adapter
  whose use count is zero, never one in use.  LRU (oldest use) is the default
  policy; the LFU variant (its exercise 6) counts every use of an adapter over
  its life and evicts the resident, unused adapter with the fewest; if every
  resident adapter is in use, the request is refused.
* 7.14.3 Hot-swapping and the prefetch pipeline: a miss means the adapter's
  weights must be copied into its slot before the LoRA kernels read them.

Readings where the pages leave a choice open: a miss takes the lowest free
slot first (the pages pop from a free list in no stated order); LFU ties go to
the adapter used least recently (the pages' sketch breaks them by name); a use
is counted per acquire, hit or miss.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Tuple


class Residency:
    """n_slots slots, all free; policy "lru" or "lfu"."""

    def __init__(self, n_slots: int, policy: str = "lru"):
        assert n_slots > 0 and policy in ("lru", "lfu")
        self.policy = policy
        self.holder: List[Optional[int]] = [None] * n_slots   # adapter in each slot
        self.in_use: List[int] = [0] * n_slots                  # uses in flight
        self.last_use: List[int] = [0] * n_slots                # time of the holder's last acquire
        self.uses: Dict[int, int] = {}                          # acquires of each adapter, ever
        self.time = 0
        self.hits = self.misses = self.evictions = 0

    def lookup(self, key: int) -> int:
        return self.holder.index(key) if key in self.holder else -1

    def acquire(self, key: int) -> Optional[Tuple[int, bool]]:
        """(slot, needs_install), or None when every slot holds an adapter in use."""
        self.time += 1
        slot = self.lookup(key)
        if slot >= 0:
            self.hits += 1
            needs_install = False
        else:
            free = [s for s, h in enumerate(self.holder) if h is None]
            if free:
                slot = free[0]
            else:
                idle = [s for s in range(len(self.holder)) if self.in_use[s] == 0]
                if not idle:
                    return None          # refused: nothing changes, no use is counted
                slot = self.victim(idle)
                self.evictions += 1
            self.misses += 1
            self.holder[slot] = key
            needs_install = True
        self.in_use[slot] += 1
        self.last_use[slot] = self.time
        self.uses[key] = self.uses.get(key, 0) + 1
        return slot, needs_install

    def victim(self, idle: List[int]) -> int:
        """The slot evicted among the idle ones: oldest last use (LRU), or
        fewest lifetime uses, then oldest last use (LFU)."""
        if self.policy == "lru":
            return min(idle, key=lambda s: self.last_use[s])
        return min(idle, key=lambda s: (self.uses[self.holder[s]], self.last_use[s]))

    def release(self, key: int) -> bool:
        """End one use; False if the adapter is not resident or has no use to end."""
        slot = self.lookup(key)
        if slot < 0 or self.in_use[slot] == 0:
            return False
        self.in_use[slot] -= 1
        return True

    def resident(self) -> int:
        return sum(h is not None for h in self.holder)
