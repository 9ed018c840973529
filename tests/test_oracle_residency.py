"""Pins of the oracle's adapter residency rules ("LLM-stack book" 7.14.4: the
registry evicts only an adapter no batch uses, LRU by default, LFU counting
every use over an adapter's life, and refuses when every resident adapter is
in use).  The expected slots below were worked out by hand from those rules;
each planted mistake at the end must fail at least one pin."""
import pytest

from oracle import Residency

A, B, C = 5, 2, 9            # adapter names (LFU ties must not fall back to the name order)


def _use(r, key):
    got = r.acquire(key)
    assert got is not None
    assert r.release(key)
    return got


def pin_lru_and_lfu_pick_different_victims(cls):
    """Two slots: A used twice, then B once; C must evict A under LRU (older
    last use) and B under LFU (fewer uses)."""
    out = {}
    for policy in ("lru", "lfu"):
        r = cls(2, policy)
        assert _use(r, A) == (0, True)
        assert _use(r, A) == (0, False)
        assert _use(r, B) == (1, True)
        out[policy] = r.acquire(C)
    return out == {"lru": (0, True), "lfu": (1, True)}


def pin_in_use_is_never_evicted(cls):
    """A (older) stays held, B is released: C must take B's slot although A is
    the least recently used; with both held, D is refused and nothing
    changes."""
    r = cls(2, "lru")
    r.acquire(A)
    _use(r, B)
    if r.acquire(C) != (1, True):
        return False
    if r.acquire(7) is not None:                     # A and C both in use
        return False
    return (r.lookup(A), r.lookup(C), r.lookup(B), r.evictions, r.misses) == (0, 1, -1, 1, 3)


def pin_lfu_counts_survive_eviction(cls):
    """Two slots, LFU.  Uses: A x3 (slot 0); B, C, B, C, B alternate in slot
    1, each evicting the other (A always has more uses).  Then A and B both
    have 3 lifetime uses, and the tie goes to the least recent, A: C takes
    slot 0.  Counting uses only since the last install would give B 1 use and
    evict B instead."""
    r = cls(2, "lfu")
    for _ in range(3):
        _use(r, A)
    seq = [(B, (1, True)), (C, (1, True)), (B, (1, True)), (C, (1, True)), (B, (1, True))]
    for key, want in seq:
        if _use(r, key) != want:
            return False
    return r.acquire(C) == (0, True)


def pin_lfu_tie_goes_to_least_recent(cls):
    """Two slots, LFU, A then B used once each: C evicts A (older), not B
    (smaller name)."""
    r = cls(2, "lfu")
    _use(r, A)
    _use(r, B)
    return r.acquire(C) == (0, True)


def pin_counts_and_releases(cls):
    """Slots for every adapter: each first acquire is a miss into the lowest
    free slot, every later one a hit, no eviction; releases beyond the uses
    in flight, or of an unknown adapter, are refused."""
    r = cls(4, "lru")
    keys = [3, 1, 3, 3, 8, 1, 0]
    got = [r.acquire(k) for k in keys]
    ok = got == [(0, True), (1, True), (0, False), (0, False), (2, True), (1, False), (3, True)]
    ok &= (r.hits, r.misses, r.evictions, r.resident()) == (3, 4, 0, 4)
    for k in keys:
        ok &= r.release(k)
    ok &= not r.release(3) and not r.release(42)
    return ok


PINS = [pin_lru_and_lfu_pick_different_victims, pin_in_use_is_never_evicted, pin_lfu_counts_survive_eviction,
        pin_lfu_tie_goes_to_least_recent, pin_counts_and_releases]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_residency_pins(pin):
    assert pin(Residency)


# ---- planted mistakes: each must fail at least one pin ------------------------------

class _EvictsInUse(Residency):
    def acquire(self, key):
        held = self.in_use[:]
        self.in_use = [0] * len(self.in_use)        # the victim search ignores uses in flight
        try:
            got = super().acquire(key)
        finally:
            for s, n in enumerate(held):
                self.in_use[s] = n + (1 if got is not None and s == got[0] else 0)
        return got


class _MostRecent(Residency):
    def victim(self, idle):
        return max(idle, key=lambda s: self.last_use[s]) if self.policy == "lru" else super().victim(idle)


class _LfuSinceInstall(Residency):
    def acquire(self, key):
        got = super().acquire(key)
        if got is not None and got[1]:
            self.uses[key] = 1                      # forgets the uses before the last eviction
        return got


class _LfuTieByName(Residency):
    def victim(self, idle):
        if self.policy == "lru":
            return super().victim(idle)
        return min(idle, key=lambda s: (self.uses[self.holder[s]], self.holder[s]))


@pytest.mark.parametrize("plant", [_EvictsInUse, _MostRecent, _LfuSinceInstall, _LfuTieByName],
                         ids=lambda c: c.__name__)
def test_planted_residency_mistakes_are_caught(plant):
    assert not all(pin(plant) for pin in PINS)
