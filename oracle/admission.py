"""Plain model of adapter-aware admission (which queued requests form a
step's batch).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: the tests compare
the library's scheduler with this model step by step.  It shares no code
with the library.

What it follows:
  * "Serving many LoRA adapters" (blog.ecitis.org), section "Adapter-aware
    scheduling": a queued request's priority is a fairness part linear in
    its wait (weight w_fair) plus a locality bonus, when its adapter is
    already active, proportional to the work it brings (weight w_local per
    row); since the fairness part keeps growing, no request waits forever.
  * "Serving multiple LoRAs: segmented matrix multiplies and adapter
    scheduling", section "Scheduling the adapters": a cap on the adapters a
    batch may hold (requests beyond it wait for a later batch); exercise 2:
    batch by rank group.
  * "Serving many LoRA adapters", section "Paging adapters": a request whose
    adapter is not resident is deferred while its adapter loads.

Readings where the pages leave a choice open (the library makes the same;
here they are the definition under test):
  * "active" adapters are those of the previous step's batch and those
    already admitted to the batch being formed;
  * the batch fills greedily: the best-scoring pending request is decided
    next (ties: earlier arrival, then earlier submission); a request that
    does not fit (rows, adapter cap, rank class, not resident) is skipped
    for this step only;
  * the checks run in the order: residency (asking the cache starts the
    load), rows, adapter cap, rank class; base-only requests (adapter -1)
    never count toward the cap and have no locality;
  * rank classes are 1, 2, 3-4, 5-8, 9-16, 17-32, 33-64;
  * the score is evaluated as (w_fair * wait) + (w_local * locality) * rows
    in double precision, without fused multiply-adds.

Parity pins: ``tests/golden/admission_walk.json`` holds steps worked out by
hand; ``tests/test_admission.py`` also checks that with w_local = 0 the
model is first-come-first-served and that an unpopular request waits at
most the bound the linear wait term implies.
"""
from __future__ import annotations

from dataclasses import dataclass, field


def rank_class(r: int) -> int:
    c = 0
    while (1 << c) < r:
        c += 1
    return c


@dataclass
class AdmissionModel:
    n_adapters: int
    w_fair: float = 1.0
    w_local: float = 0.35
    max_adapters: int = 32
    max_rows: int = 256
    rank_groups: bool = False
    ranks: list = None
    resident: object = None          # callable adapter -> bool (asks the cache), or None
    queue: list = field(default_factory=list)
    seq: int = 0
    prev_active: set = field(default_factory=set)

    def submit(self, request, adapter, rows, arrival):
        assert -1 <= adapter < self.n_adapters and rows >= 1
        self.queue.append((request, adapter, rows, arrival, self.seq))
        self.seq += 1

    def _priority(self, wait, adapter_active, rows):
        # fairness grows linearly with the wait; a request whose adapter is
        # already active gets a locality bonus in proportion to its rows
        fairness = self.w_fair * wait
        locality_bonus = self.w_local * rows if adapter_active else 0.0
        return fairness + locality_bonus

    def step(self, now, capacity):
        batch, in_batch, taken = [], [], []
        rows = 0
        cls = None
        decided = set()
        known = {}
        info = dict(skipped_rows=0, skipped_cap=0, skipped_rank_group=0, deferred_not_resident=0)
        while len(batch) < capacity and rows < self.max_rows:
            best = None
            for i, (rid, a, rw, arr, sq) in enumerate(self.queue):
                if i in decided:
                    continue
                local = a >= 0 and (a in self.prev_active or a in in_batch)
                key = (self._priority(now - arr, local, rw), -arr, -sq)
                if best is None or key > best[0]:
                    best = (key, i)
            if best is None:
                break
            i = best[1]
            decided.add(i)
            rid, a, rw, arr, sq = self.queue[i]
            if a >= 0 and self.resident is not None:
                if a not in known:
                    known[a] = bool(self.resident(a))
                if not known[a]:
                    info["deferred_not_resident"] += 1
                    continue
            if rows + rw > self.max_rows:
                info["skipped_rows"] += 1
                continue
            if a >= 0 and a not in in_batch and len(in_batch) >= self.max_adapters:
                info["skipped_cap"] += 1
                continue
            if a >= 0 and self.rank_groups:
                k = rank_class(self.ranks[a])
                if cls is not None and k != cls:
                    info["skipped_rank_group"] += 1
                    continue
                cls = k
            if a >= 0 and a not in in_batch:
                in_batch.append(a)
            batch.append((rid, a, rw, now - arr))
            taken.append(i)
            rows += rw
        self.queue = [q for i, q in enumerate(self.queue) if i not in set(taken)]
        self.prev_active = set(in_batch)
        info.update(admitted=len(batch), rows=rows, distinct_adapters=len(in_batch), queued=len(self.queue))
        return batch, info
