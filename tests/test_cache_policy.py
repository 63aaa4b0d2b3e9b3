"""CPU checks of the adapter slot cache's policy (no device).

The plain model in ``oracle/paging.py`` is first pinned to a call sequence
worked out by hand from the pages ("Multi-LoRA batching and adapter
paging", section "Adapter paging"; "Serving many LoRA adapters"
(blog.ecitis.org), section "Paging adapters"), and plausible mistakes in
it (MRU instead of LRU, pins, holds or the running batch ignored, no load
cap) are shown to break that pin.  The library's cache, in its host-only
mode (the same policy code with no copies), must then match the walk and
agree with the model state for state over long seeded random call
sequences.  Integer results: compared exactly."""
from __future__ import annotations

import json
import os

import numpy as np
import pytest

from oracle import paging as pm

HERE = os.path.dirname(os.path.abspath(__file__))
WALK = json.load(open(os.path.join(HERE, "golden", "paging_walk.json")))
NAMES = {"RESIDENT": pm.RESIDENT, "LOADING": pm.LOADING, "DEFERRED": pm.DEFERRED}


def _lib_cache(n_adapters, n_slots, max_loads):
    import torch
    from lora_bgmv_shrink_amd import binding as b
    c = b.Cache(torch.bfloat16, [(64, 32), (32, 96)], 16, n_adapters, n_slots, max_loads, host_only=True)
    for a in range(n_adapters):
        c.register(a, 16, 2.0)
    return c


class _LibDriver:
    """The library cache behind the model's method names."""

    def __init__(self, n_adapters, n_slots, max_loads):
        from lora_bgmv_shrink_amd import binding as b
        self.b = b
        self.n_adapters = n_adapters
        self.c = _lib_cache(n_adapters, n_slots, max_loads)

    def request(self, a):
        return self.c.request(a)

    def poll(self):
        return self.c.poll()

    def pin(self, a, on=True):
        self.c.pin(a, on)

    def hold(self, a, delta):
        self.c.hold(a, delta)

    def map(self, ids):
        try:
            return [int(v) for v in self.c.map(ids)]
        except self.b.LoraError as e:
            assert e.status == self.b.LORA_E_NOT_RESIDENT
            return pm.NOT_RESIDENT

    def release(self):
        self.c.release()

    def snapshot(self):
        s = self.c.stats()
        keys = ("requests", "hits", "pending", "loads_started", "deferred_load_cap", "deferred_no_slot",
                "loads_completed", "evictions", "slots_resident", "slots_loading", "slots_bound")
        out = {k: s[k] for k in keys}
        out["slot_of"] = [self.c.slot_of(a) for a in range(self.n_adapters)]
        return out


def _new_model(n_adapters, n_slots, max_loads, cls=pm.PagingModel):
    m = cls(n_adapters, n_slots, max_loads)
    for a in range(n_adapters):
        m.register(a)
    return m


def _run_walk(drv):
    for i, st in enumerate(WALK["steps"]):
        op = st["op"]
        if op == "request":
            got = drv.request(st["a"])
            assert got == NAMES[st["expect"]], (i, st, got)
        elif op == "poll":
            assert drv.poll() == st["expect"], (i, st)
        elif op == "map":
            got = drv.map(st["ids"])
            want = pm.NOT_RESIDENT if st["expect"] == "NOT_RESIDENT" else st["expect"]
            assert got == want, (i, st, got)
        elif op == "release":
            drv.release()
        elif op == "pin":
            drv.pin(st["a"], bool(st["on"]))
        elif op == "hold":
            drv.hold(st["a"], st["delta"])
        else:
            raise AssertionError(op)
    snap = drv.snapshot()
    for k, v in WALK["final"].items():
        assert snap[k] == v, (k, snap[k], v)


def _walk_args():
    return WALK["n_adapters"], WALK["n_slots"], WALK["max_loads"]


def test_model_matches_hand_walk():
    _run_walk(_new_model(*_walk_args()))


# Plausible mistakes in the model; each must break the hand-worked walk.
class _MRU(pm.PagingModel):
    def _victim(self):
        for i, s in enumerate(self.slots):
            if s.state == "empty":
                return i
        c = [i for i, s in enumerate(self.slots) if s.state == "ready" and not s.bound
             and s.adapter not in self.pinned and self.holds.get(s.adapter, 0) == 0]
        return max(c, key=lambda i: (self.slots[i].last_use, -i)) if c else -1


class _NoPin(pm.PagingModel):
    def pin(self, a, on=True):
        pass


class _NoHold(pm.PagingModel):
    def hold(self, a, delta):
        pass


class _NoBound(pm.PagingModel):
    def map(self, ids):
        out = super().map(ids)
        for s in self.slots:
            s.bound = False
        return out


class _NoCap(pm.PagingModel):
    def _loading(self):
        return []


class _HitNotTouched(pm.PagingModel):
    def request(self, a):
        if a in self.where and self.slots[self.where[a]].state == "ready":
            self.counts["requests"] += 1
            self.counts["hits"] += 1
            return pm.RESIDENT
        return super().request(a)


class _BlockingMap(pm.PagingModel):
    """Waits for (completes) in-flight loads instead of deferring."""
    def map(self, ids):
        self.poll()
        return super().map(ids)


@pytest.mark.parametrize("cls", [_MRU, _NoPin, _NoHold, _NoBound, _NoCap, _HitNotTouched, _BlockingMap])
def test_model_mutations_break_the_walk(cls):
    with pytest.raises(AssertionError):
        _run_walk(_new_model(*_walk_args(), cls=cls))


def test_library_matches_hand_walk():
    _run_walk(_LibDriver(*_walk_args()))


@pytest.mark.parametrize("seed,n_adapters,n_slots,max_loads", [
    (0, 6, 2, 1), (1, 12, 4, 2), (2, 40, 8, 3), (3, 200, 16, 4), (4, 9, 9, 9), (5, 30, 1, 1)])
def test_library_matches_model_random(seed, n_adapters, n_slots, max_loads):
    rng = np.random.default_rng(seed)
    m = _new_model(n_adapters, n_slots, max_loads)
    d = _LibDriver(n_adapters, n_slots, max_loads)
    # Zipf-like popularity so that hits, evictions and deferrals all occur
    p = 1.0 / np.arange(1, n_adapters + 1) ** 1.1
    p /= p.sum()
    holds = np.zeros(n_adapters, np.int64)
    for step in range(3000):
        r = rng.random()
        if r < 0.55:
            a = int(rng.choice(n_adapters, p=p))
            assert m.request(a) == d.request(a), step
        elif r < 0.70:
            assert m.poll() == d.poll(), step
        elif r < 0.82:
            ids = [int(v) if rng.random() > 0.1 else -1 for v in rng.choice(n_adapters, size=rng.integers(1, 6), p=p)]
            assert m.map(ids) == d.map(ids), step
        elif r < 0.90:
            m.release()
            d.release()
        elif r < 0.95:
            a, on = int(rng.integers(n_adapters)), bool(rng.random() < 0.3)
            m.pin(a, on)
            d.pin(a, on)
        else:
            a = int(rng.integers(n_adapters))
            delta = 1 if (holds[a] == 0 or rng.random() < 0.5) else -1
            holds[a] += delta
            m.hold(a, delta)
            d.hold(a, delta)
        if step % 50 == 0:
            assert m.snapshot() == d.snapshot(), step
    assert m.snapshot() == d.snapshot()
    s = m.snapshot()
    assert s["hits"] > 0 and s["loads_started"] > 0
    if n_slots < n_adapters:
        assert s["evictions"] > 0


def test_cache_argument_checks():
    import torch
    from lora_bgmv_shrink_amd import binding as b
    c = _lib_cache(4, 2, 1)
    for call in (lambda: c.request(4), lambda: c.request(-1), lambda: c.pin(9), lambda: c.hold(0, -1),
                 lambda: c.map([7])):
        with pytest.raises(b.LoraError) as e:
            call()
        assert e.value.status == b.LORA_E_INVALID
    assert c.request(0) == pm.LOADING
    with pytest.raises(b.LoraError) as e:       # re-register while loading
        c.register(0, 16, 1.0)
    assert e.value.status == b.LORA_E_INVALID
    with pytest.raises(b.LoraError) as e:       # rank above r_max
        c.register(1, 32, 1.0)
    assert e.value.status == b.LORA_E_UNSUPPORTED
    with pytest.raises(b.LoraError) as e:       # bf16 streaming ranks are multiples of 8
        c.register(1, 12, 1.0)
    assert e.value.status == b.LORA_E_UNSUPPORTED
    with pytest.raises(b.LoraError):            # no pools without a device
        c.pool(0)
    # unregistered adapter
    c2 = b.Cache(torch.bfloat16, [(64, 32)], 16, 4, 2, 1, host_only=True)
    with pytest.raises(b.LoraError):
        c2.request(0)
    c3 = b.Cache(torch.bfloat16, [(64, 32)], 16, 4, 2, 1, host_only=True, any_rank=True)
    c3.register(1, 12, 1.0)
    # bad create arguments
    for args in ((torch.bfloat16, [], 16, 4, 2, 1), (torch.bfloat16, [(64, 32)], 65, 4, 2, 1),
                 (torch.bfloat16, [(64, 32)], 16, 4, 0, 1), (torch.bfloat16, [(64, 32)], 16, 4, 2, 0)):
        with pytest.raises(b.LoraError):
            b.Cache(*args, host_only=True)


def test_blob_layout():
    """Part blocks in order A_0, B_0, A_1, B_1 ..., each rounded up to 128
    elements (256 bytes in bf16)."""
    c = _lib_cache(2, 1, 1)
    a_off, b_off, total = c.blob_layout(16)
    r128 = lambda v: -(-v // 128) * 128
    assert list(a_off) == [0, r128(64 * 16) + r128(16 * 32)]
    assert list(b_off) == [r128(64 * 16), a_off[1] + r128(32 * 16)]
    assert total == b_off[1] + r128(16 * 96)
