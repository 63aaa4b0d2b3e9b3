"""Plain model of the adapter slot cache's policy (no device, no copies).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: the tests compare
the library's cache (run in its host-only mode) with this model call by
call.  It shares no code with the library.

What it follows:
  * "Multi-LoRA batching and adapter paging", section "Adapter paging":
    GPU adapter slots are an LRU cache; an adapter already on the GPU is
    scheduled at once; a missing one evicts a cold adapter and is copied
    in; the number of loads at once is capped; pinned adapters are never
    evicted.
  * "Serving many LoRA adapters" (blog.ecitis.org), section "Paging
    adapters": a miss must not block the step: it starts a prefetch and
    defers that request; eviction is plain LRU over adapter ids (with a
    pin for committed adapters); an adapter with queued requests is not
    evicted.

Readings where the pages leave a choice open (the library makes the same
ones; they are stated here as the definition under test):
  * a miss that cannot start a load (cap reached, or no evictable slot) is
    deferred without queueing a load; the caller asks again later;
  * empty slots are filled first, lowest slot number first; among
    evictable slots the least recently used goes, ties to the lowest slot;
  * "used" means asked for (hit or still loading), loaded, or bound to a
    batch; a slot bound to a batch that has not been released is not
    evictable, nor is one whose load is still in flight;
  * a load completes only when the caller polls (the model has no clock).

Parity pins: ``tests/golden/paging_walk.json`` is a call sequence worked
out by hand from the two passages above; ``tests/test_cache_policy.py``
checks this model against it before comparing the library with it.
"""
from __future__ import annotations

from dataclasses import dataclass, field

RESIDENT, LOADING, DEFERRED = 0, 1, 2
NOT_RESIDENT = "not_resident"


@dataclass
class _Slot:
    adapter: int = -1
    state: str = "empty"        # "empty" | "loading" | "ready"
    bound: bool = False
    last_use: int = 0


@dataclass
class PagingModel:
    n_adapters: int
    n_slots: int
    max_loads: int
    slots: list = field(default_factory=list)
    where: dict = field(default_factory=dict)      # adapter -> slot
    registered: set = field(default_factory=set)
    pinned: set = field(default_factory=set)
    holds: dict = field(default_factory=dict)
    clock: int = 0
    counts: dict = field(default_factory=dict)

    def __post_init__(self):
        self.slots = [_Slot() for _ in range(self.n_slots)]
        self.counts = dict(requests=0, hits=0, pending=0, loads_started=0, deferred_load_cap=0,
                           deferred_no_slot=0, loads_completed=0, evictions=0)

    def _tick(self):
        self.clock += 1
        return self.clock

    def register(self, a):
        assert a not in self.where
        self.registered.add(a)

    def pin(self, a, on=True):
        (self.pinned.add if on else self.pinned.discard)(a)

    def hold(self, a, delta):
        n = self.holds.get(a, 0) + delta
        assert n >= 0
        self.holds[a] = n

    def _loading(self):
        return [i for i, s in enumerate(self.slots) if s.state == "loading"]

    def poll(self):
        done = 0
        for s in self.slots:
            if s.state == "loading":
                s.state = "ready"
                done += 1
        self.counts["loads_completed"] += done
        return done

    def _victim(self):
        for i, s in enumerate(self.slots):
            if s.state == "empty":
                return i
        cands = [i for i, s in enumerate(self.slots)
                 if s.state == "ready" and not s.bound and s.adapter not in self.pinned
                 and self.holds.get(s.adapter, 0) == 0]
        if not cands:
            return -1
        return min(cands, key=lambda i: (self.slots[i].last_use, i))

    def request(self, a):
        self.counts["requests"] += 1
        if a in self.where:
            s = self.slots[self.where[a]]
            s.last_use = self._tick()
            if s.state == "ready":
                self.counts["hits"] += 1
                return RESIDENT
            self.counts["pending"] += 1
            return LOADING
        if len(self._loading()) >= self.max_loads:
            self.counts["deferred_load_cap"] += 1
            return DEFERRED
        v = self._victim()
        if v < 0:
            self.counts["deferred_no_slot"] += 1
            return DEFERRED
        s = self.slots[v]
        if s.adapter >= 0:
            del self.where[s.adapter]
            self.counts["evictions"] += 1
        s.adapter, s.state, s.last_use = a, "loading", self._tick()
        self.where[a] = v
        self.counts["loads_started"] += 1
        return LOADING

    def map(self, ids):
        for a in ids:
            if a == -1:
                continue
            if a not in self.where or self.slots[self.where[a]].state != "ready":
                return NOT_RESIDENT
        out = []
        for a in ids:
            if a == -1:
                out.append(-1)
                continue
            v = self.where[a]
            s = self.slots[v]
            s.last_use = self._tick()
            s.bound = True
            out.append(v)
        return out

    def release(self):
        for s in self.slots:
            s.bound = False

    def slot_of(self, a):
        return self.where.get(a, -1)

    def snapshot(self):
        """Integer state comparable with the library: (slot of each adapter,
        counters, resident/loading/bound slot counts)."""
        return dict(
            slot_of=[self.slot_of(a) for a in range(self.n_adapters)],
            slots_resident=sum(s.state == "ready" for s in self.slots),
            slots_loading=sum(s.state == "loading" for s in self.slots),
            slots_bound=sum(s.bound for s in self.slots),
            **self.counts,
        )
