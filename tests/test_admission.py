"""CPU checks of adapter-aware admission (no device).

The plain model in ``oracle/admission.py`` is pinned to scenarios worked
out by hand from the pages ("Serving many LoRA adapters" (blog.ecitis.org),
section "Adapter-aware scheduling"; "Serving multiple LoRAs...", section
"Scheduling the adapters"), to two properties the pages state (with no
locality weight the order is first come, first served; the linear wait
term bounds starvation), and plausible mistakes in it must break those
pins.  The library's scheduler must then match the model step for step
over seeded random runs, alone and gating admission on a host-only slot
cache that follows the paging model.  All compared results are integers or
the same double expression: compared exactly."""
from __future__ import annotations

import json
import os

import numpy as np
import pytest

from oracle import admission as am
from oracle import paging as pm

HERE = os.path.dirname(os.path.abspath(__file__))
WALK = json.load(open(os.path.join(HERE, "golden", "admission_walk.json")))


def _model(sc, cls=am.AdmissionModel, **kw):
    return cls(sc["n_adapters"], sc["w_fair"], sc["w_local"], sc["max_adapters"], sc["max_rows"],
               bool(sc.get("rank_groups", 0)), sc.get("ranks"), **kw)


class _Lib:
    """The library scheduler behind the model's interface."""

    def __init__(self, sc, cache=None):
        from lora_bgmv_shrink_amd import binding as b
        self.s = b.Scheduler(sc["n_adapters"], sc["w_fair"], sc["w_local"], sc["max_adapters"], sc["max_rows"],
                             bool(sc.get("rank_groups", 0)), sc.get("ranks"), cache=cache)

    def submit(self, *a):
        self.s.submit(*a)

    def step(self, now, capacity):
        (req, ad, rw, wt), info = self.s.step(now, capacity)
        return [(int(r), int(a), int(n), float(w)) for r, a, n, w in zip(req, ad, rw, wt)], info


def _run_scenario(drv, sc):
    for k, st in enumerate(sc["steps"]):
        for r in st["submit"]:
            drv.submit(*r)
        batch, info = drv.step(st["now"], st["capacity"])
        assert [b[0] for b in batch] == st["batch"], (sc["name"], k, batch)
        for key, v in st["info"].items():
            assert info[key] == v, (sc["name"], k, key, info[key], v)


@pytest.mark.parametrize("sc", WALK["scenarios"], ids=[s["name"] for s in WALK["scenarios"]])
def test_model_matches_hand_scenarios(sc):
    _run_scenario(_model(sc), sc)


@pytest.mark.parametrize("sc", WALK["scenarios"], ids=[s["name"] for s in WALK["scenarios"]])
def test_library_matches_hand_scenarios(sc):
    _run_scenario(_Lib(sc), sc)


# Plausible mistakes in the model; each must break at least one scenario.
class _NoLocality(am.AdmissionModel):
    def _priority(self, wait, adapter_active, rows):
        return self.w_fair * wait


class _NoCarryOver(am.AdmissionModel):
    def step(self, now, capacity):
        self.prev_active = set()
        return super().step(now, capacity)


class _BaseCountsToCap(am.AdmissionModel):
    def submit(self, request, adapter, rows, arrival):
        super().submit(request, adapter if adapter >= 0 else self.n_adapters - 1, rows, arrival)


class _NoCap(am.AdmissionModel):
    def __init__(self, *a, **k):
        super().__init__(*a, **k)
        self.max_adapters = 10 ** 9


class _LaterSubmissionWins(am.AdmissionModel):
    def submit(self, request, adapter, rows, arrival):
        self.queue.append((request, adapter, rows, arrival, -self.seq))
        self.seq += 1


class _NoRankGroups(am.AdmissionModel):
    def __init__(self, *a, **k):
        super().__init__(*a, **k)
        self.rank_groups = False


class _LocalityNotScaledByRows(am.AdmissionModel):
    def _priority(self, wait, adapter_active, rows):
        return self.w_fair * wait + (self.w_local if adapter_active else 0.0)


@pytest.mark.parametrize("cls", [_NoLocality, _NoCarryOver, _BaseCountsToCap, _NoCap, _LaterSubmissionWins,
                                 _NoRankGroups, _LocalityNotScaledByRows])
def test_model_mutations_break_a_scenario(cls):
    broke = False
    for sc in WALK["scenarios"]:
        try:
            _run_scenario(_model(sc, cls), sc)
        except AssertionError:
            broke = True
    assert broke, cls.__name__


def _random_run(drv_list, seed, n_adapters, steps, cap_lo=1, cap_hi=64, check=None):
    rng = np.random.default_rng(seed)
    p = 1.0 / np.arange(1, n_adapters + 1) ** 1.1
    p /= p.sum()
    t, rid = 0.0, 0
    outs = [[] for _ in drv_list]
    for step in range(steps):
        for _ in range(int(rng.poisson(6))):
            t += float(rng.exponential(0.05))
            a = -1 if rng.random() < 0.05 else int(rng.choice(n_adapters, p=p))
            rows = int(rng.integers(1, 9))
            for d in drv_list:
                d.submit(rid, a, rows, t)
            rid += 1
        t += 0.1
        cap = int(rng.integers(cap_lo, cap_hi + 1))
        res = [d.step(t, cap) for d in drv_list]
        for o, r in zip(outs, res):
            o.append(r)
        if check:
            check(step, res)
    return outs


def test_fifo_when_locality_weight_is_zero():
    """w_local = 0 and no caps: the batch is the oldest requests, in arrival
    order (ties by submission), as many as fit."""
    sc = dict(n_adapters=50, w_fair=1.0, w_local=0.0, max_adapters=10 ** 6, max_rows=10 ** 6)
    m = _model(sc)
    pending = []

    class Rec:
        def submit(self, *r):
            pending.append(r)
            m.submit(*r)

        def step(self, now, cap):
            batch, info = m.step(now, cap)
            order = sorted(pending, key=lambda r: (r[3], r[0]))[:cap]
            assert [b[0] for b in batch] == [r[0] for r in order]
            for r in order:
                pending.remove(r)
            return batch, info

    _random_run([Rec()], 0, 50, 200)


def test_linear_wait_bounds_starvation():
    """A request whose wait exceeds every other queued request's by more
    than w_local * max_rows / w_fair outscores them all, so it is decided
    first; with a rows budget it fits in, it is admitted first."""
    sc = dict(n_adapters=200, w_fair=1.0, w_local=2.0, max_adapters=4, max_rows=16)
    m = _model(sc)
    hits = [0]

    class Rec:
        def submit(self, *r):
            m.submit(*r)

        def step(self, now, cap):
            q = list(m.queue)
            batch, info = m.step(now, cap)
            if len(q) >= 2:
                w = sorted(((now - r[3]), r[0]) for r in q)
                if w[-1][0] - w[-2][0] > sc["w_local"] * sc["max_rows"] / sc["w_fair"]:
                    hits[0] += 1
                    assert batch and batch[0][0] == w[-1][1]
            return batch, info

    # sparse arrivals so that gaps in waiting time occur
    rng = np.random.default_rng(5)
    t = 0.0
    for i in range(3000):
        t += float(rng.exponential(8.0))
        a = int(rng.integers(0, 200))
        Rec().submit(i, a, int(rng.integers(1, 9)), t)
        if i % 3 == 0:
            Rec().step(t + 0.01, int(rng.integers(1, 4)))
    assert hits[0] > 20


@pytest.mark.parametrize("seed,rank_groups", [(0, 0), (1, 0), (2, 1), (3, 1)])
def test_library_matches_model_random(seed, rank_groups):
    n = 120
    ranks = list(np.random.default_rng(100 + seed).choice([8, 16, 32, 64], size=n, p=[.4, .3, .2, .1]))
    sc = dict(n_adapters=n, w_fair=1.0, w_local=0.35, max_adapters=int(4 + seed * 3), max_rows=64,
              rank_groups=rank_groups, ranks=[int(r) for r in ranks])

    def check(step, res):
        (b1, i1), (b2, i2) = res
        assert b1 == b2, step
        assert {k: i1[k] for k in i1} == {k: i2[k] for k in i1}, step

    _random_run([_model(sc), _Lib(sc)], seed, n, 400, check=check)


class _ModelWithCache(am.AdmissionModel):
    """The admission model gating on the paging model, with the holds the
    library keeps: one per queued request, kept one step past admission."""

    def __init__(self, sc, paging):
        super().__init__(sc["n_adapters"], sc["w_fair"], sc["w_local"], sc["max_adapters"], sc["max_rows"],
                         resident=lambda a: paging.request(a) == pm.RESIDENT)
        self.paging = paging
        self.held = []

    def submit(self, request, adapter, rows, arrival):
        if adapter >= 0:
            self.paging.hold(adapter, 1)
        super().submit(request, adapter, rows, arrival)

    def step(self, now, capacity):
        for a in self.held:
            self.paging.hold(a, -1)
        batch, info = super().step(now, capacity)
        self.held = [b[1] for b in batch if b[1] >= 0]
        return batch, info


@pytest.mark.parametrize("seed,n_slots,max_loads", [(0, 8, 2), (1, 24, 4), (2, 3, 1)])
def test_library_with_cache_matches_models(seed, n_slots, max_loads):
    import torch
    from lora_bgmv_shrink_amd import binding as b
    n = 60
    sc = dict(n_adapters=n, w_fair=1.0, w_local=0.35, max_adapters=6, max_rows=48)
    paging = pm.PagingModel(n, n_slots, max_loads)
    cache = b.Cache(torch.bfloat16, [(64, 32)], 16, n, n_slots, max_loads, host_only=True)
    for a in range(n):
        paging.register(a)
        cache.register(a, 16, 1.0)
    m = _ModelWithCache(sc, paging)
    lib = _Lib(sc, cache=cache)
    rng = np.random.default_rng(seed + 50)
    keys = ("requests", "hits", "pending", "loads_started", "deferred_load_cap", "deferred_no_slot",
            "loads_completed", "evictions", "slots_resident", "slots_loading")

    def check(step, res):
        (b1, i1), (b2, i2) = res
        assert b1 == b2, step
        assert {k: i1[k] for k in i1} == {k: i2[k] for k in i1}, step
        if rng.random() < 0.5:           # loads complete between some steps
            assert paging.poll() == cache.poll()
        s1, s2 = paging.snapshot(), cache.stats()
        assert {k: s1[k] for k in keys} == {k: s2[k] for k in keys}, step
        assert s1["slot_of"] == [cache.slot_of(a) for a in range(n)], step

    outs = _random_run([m, lib], seed, n, 300, check=check)
    deferred = sum(i["deferred_not_resident"] for _, i in outs[0])
    assert deferred > 0
    lib.s.destroy()
    cache.destroy()


def test_scheduler_argument_checks():
    from lora_bgmv_shrink_amd import binding as b
    with pytest.raises(b.LoraError):
        b.Scheduler(0)
    with pytest.raises(b.LoraError):
        b.Scheduler(4, max_adapters=0)
    with pytest.raises(b.LoraError):
        b.Scheduler(4, rank_groups=True)          # needs ranks
    with pytest.raises(b.LoraError):
        b.Scheduler(4, w_local=-1.0)
    s = b.Scheduler(4)
    for args in ((0, 4, 1, 0.0), (0, -2, 1, 0.0), (0, 1, 0, 0.0), (0, 1, 1, float("nan"))):
        with pytest.raises(b.LoraError):
            s.submit(*args)
    s.submit(0, 1, 1, 0.0)
    (req, ad, rw, wt), info = s.step(1.0, 0)      # capacity 0: nothing admitted
    assert info["admitted"] == 0 and info["queued"] == 1 and s.queued() == 1
    (req, ad, rw, wt), info = s.step(2.0, 4)
    assert list(req) == [0] and list(ad) == [1] and list(wt) == [2.0] and s.queued() == 0
