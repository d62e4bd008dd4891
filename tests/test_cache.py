"""The delta cache's policy, on the host (policy mode: no HIP calls).

What "BitDelta : servir 14 modèles Zen depuis un seul cluster GPU"
(hanzo-blog, 2026-02-28), "Infrastructure details", fixes: a variant that is
not cached is loaded on its first request and then stays until evicted (cold
start); requests for a variant whose delta is loading wait for that one load
(routing); eviction is LRU, with the variants of highest request rate pinned
(the top 6 in the post's deployment of 14).  The rate weighting is read as an
exponentially decayed request count; a small reference model of that reading,
written here independently of the library, replays random request streams
and must agree with every decision."""

import math
import random

import pytest

from tenant_serving_amd import bitdelta
from tenant_serving_amd.cache import bd_cache


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import os
    if not os.path.exists(bitdelta.LIBRARY):
        from tenant_serving_amd import build
        build.build()


def make(nv=14, slots=10, pinned=6, half_life=60.0, slot_bytes=1 << 20):
    return bd_cache(nv, slots, pinned, half_life, slot_bytes)


def test_cold_start_then_resident():
    c = make()
    assert c.bd_cache_request(3, 0.0) == ("load", 0, -1)
    c.bd_cache_complete(3)
    c.bd_cache_release(3)
    assert c.bd_cache_request(3, 1.0) == ("hit", 0, -1)
    c.bd_cache_release(3)
    assert c.bd_cache_query(3) == (0, 1, 0)
    assert c.bd_cache_query(4) == (-1, -1, 0)
    st = c.bd_cache_get_stats()
    assert (st["requests"], st["loads"], st["hits"], st["bytes_loaded"]) == (2, 1, 1, 1 << 20)


def test_requests_during_a_load_join_it():
    c = make()
    assert c.bd_cache_request(5, 0.0)[0] == "load"
    for i in range(7):
        assert c.bd_cache_request(5, 0.1 * i)[0] == "join"
    assert c.bd_cache_query(5) == (0, 0, 8)
    c.bd_cache_complete(5)
    assert c.bd_cache_request(5, 1.0)[0] == "hit"
    st = c.bd_cache_get_stats()
    assert st["loads"] == 1 and st["joins"] == 7


def _fill(c, variants, t0=0.0):
    for i, v in enumerate(variants):
        a, s, e = c.bd_cache_request(v, t0 + i)
        assert a == "load"
        c.bd_cache_complete(v)
        c.bd_cache_release(v)


def test_lru_eviction_without_pins():
    c = make(nv=6, slots=3, pinned=0)
    _fill(c, [0, 1, 2])
    a, s, e = c.bd_cache_request(0, 10.0)     # touch 0: now 1 is least recent
    assert a == "hit"
    c.bd_cache_release(0)
    a, s, e = c.bd_cache_request(3, 11.0)
    assert a == "load" and e == 1
    assert c.bd_cache_query(1)[0] == -1
    c.bd_cache_complete(3)
    c.bd_cache_release(3)
    a, s, e = c.bd_cache_request(4, 12.0)
    assert e == 2


def test_busiest_variants_are_pinned():
    # variant 0 is requested often but long ago; LRU alone would evict it
    c = make(nv=6, slots=3, pinned=1, half_life=1000.0)
    for i in range(20):
        c.bd_cache_request(0, float(i))
        if i == 0:
            c.bd_cache_complete(0)
        c.bd_cache_release(0)
    _fill(c, [1, 2], 30.0)
    a, s, e = c.bd_cache_request(3, 40.0)
    assert a == "load" and e == 1             # 0 is pinned, 1 is the LRU of the rest
    assert c.bd_cache_query(0)[2] == 0 and c.bd_cache_query(0)[1] == 1


def test_pins_follow_the_decayed_rate():
    # 0 was busy long ago; with a short half-life 1 is now the busier
    c = make(nv=6, slots=2, pinned=1, half_life=1.0)
    for i in range(10):
        c.bd_cache_request(0, 0.01 * i)
        if i == 0:
            c.bd_cache_complete(0)
        c.bd_cache_release(0)
    for i in range(3):
        c.bd_cache_request(1, 50.0 + i)
        if i == 0:
            c.bd_cache_complete(1)
        c.bd_cache_release(1)
    a, s, e = c.bd_cache_request(2, 60.0)
    assert a == "load" and e == 0             # 0 decayed to ~10·2^-60, 1 is pinned


def test_in_use_variants_are_not_evicted_and_busy_changes_nothing():
    c = make(nv=4, slots=2, pinned=1)
    assert c.bd_cache_request(0, 0.0)[0] == "load"
    assert c.bd_cache_request(1, 1.0)[0] == "load"
    # both held (references): nothing can be evicted
    assert c.bd_cache_request(2, 2.0) == ("busy", -1, -1)
    assert c.bd_cache_query(0) == (0, 0, 1) and c.bd_cache_query(1) == (1, 0, 1)
    c.bd_cache_complete(0)
    c.bd_cache_release(0)
    c.bd_cache_complete(1)
    c.bd_cache_release(1)
    st = c.bd_cache_get_stats()
    assert st["busy"] == 1 and st["loads"] == 2
    # once released both can go; the one pinned slot of rate goes to the
    # requester itself (its rate counts this request, the others have decayed),
    # so the least recently requested resident variant, 0, is evicted
    a, s, e = c.bd_cache_request(3, 3.0)
    assert a == "load" and e == 0


def test_argument_errors():
    lib = bitdelta.library()
    c = make(nv=4, slots=2, pinned=1)
    with pytest.raises(bitdelta.BitDeltaError):
        c.bd_cache_release(0)                # not resident
    c.bd_cache_request(0, 0.0)
    c.bd_cache_release(0)
    with pytest.raises(bitdelta.BitDeltaError):
        c.bd_cache_release(0)                # no reference left
    with pytest.raises(bitdelta.BitDeltaError):
        c.bd_cache_request(4, 1.0)           # out of range
    with pytest.raises(bitdelta.BitDeltaError):
        c.bd_cache_complete(3)               # not resident
    for t in (-1.0, math.nan, math.inf):     # time going back, or not finite
        with pytest.raises(bitdelta.BitDeltaError) as ei:
            c.bd_cache_request(1, t)
        assert ei.value.status == 2
    assert c.bd_cache_query(1)[0] == -1 and c.bd_cache_get_stats()["requests"] == 1
    c.bd_cache_request(1, 0.0)               # the same time again is fine
    for bad in ((0, 1, 0, 1.0, 8), (4, 5, 0, 1.0, 8), (4, 2, 2, 1.0, 8), (4, 2, 1, 0.0, 8),
                (4, 2, 1, math.inf, 8), (4, 2, 1, 1.0, 0), (4, 0, 0, 1.0, 8), (2000, 2, 1, 1.0, 8)):
        with pytest.raises(bitdelta.BitDeltaError) as ei:
            bd_cache(*bad)
        assert ei.value.status == 2
    del lib


class Model:
    """The policy as the header states it, written plainly."""

    def __init__(self, nv, slots, pinned, half_life):
        self.nv, self.nslots, self.pinned, self.h = nv, slots, pinned, half_life
        self.rate = [0.0] * nv
        self.t = [0.0] * nv
        self.seen = [False] * nv
        self.last = [0] * nv
        self.tick = 0
        self.slot_of = [-1] * nv
        self.slot_var = [-1] * slots
        self.ready = [False] * slots
        self.refs = [0] * slots

    def dec(self, v, now):
        return self.rate[v] * 2.0 ** (-(now - self.t[v]) / self.h) if self.seen[v] else 0.0

    def request(self, v, now):
        self.rate[v] = self.dec(v, now) + 1.0
        self.t[v] = now
        self.seen[v] = True
        self.tick += 1
        self.last[v] = self.tick
        if self.slot_of[v] >= 0:
            s = self.slot_of[v]
            self.refs[s] += 1
            return ("hit" if self.ready[s] else "join", s, -1)
        free = [i for i in range(self.nslots) if self.slot_var[i] < 0]
        if free:
            s = free[0]
        else:
            ranked = sorted((i for i in range(self.nv) if self.seen[i]),
                            key=lambda i: (-self.dec(i, now), i))
            pin = set(ranked[:self.pinned])
            cand = [i for i in range(self.nslots)
                    if self.refs[i] == 0 and self.slot_var[i] not in pin]
            if not cand:
                return ("busy", -1, -1)
            s = min(cand, key=lambda i: self.last[self.slot_var[i]])
        ev = self.slot_var[s]
        if ev >= 0:
            self.slot_of[ev] = -1
        self.slot_var[s] = v
        self.slot_of[v] = s
        self.ready[s] = False
        self.refs[s] = 1
        return ("load", s, ev)

    def load_failed(self, v):
        s = self.slot_of[v]
        self.slot_var[s] = -1
        self.slot_of[v] = -1
        self.ready[s] = False
        self.refs[s] = 0


@pytest.mark.parametrize("seed", range(6))
def test_matches_the_reference_model_on_random_traffic(seed):
    # 14 variants, top 6 pinned, 10 slots (so 8 share 4), skewed traffic,
    # loads completing after a random delay, requests released in batches
    rng = random.Random(seed)
    nv, slots, pinned, h = 14, 10 - (seed % 3), 6 - (seed % 2) * 3, [5.0, 50.0, 500.0][seed % 3]
    c = bd_cache(nv, slots, pinned, h, 4096)
    m = Model(nv, slots, pinned, h)
    weights = [1.0 / (i + 1) ** 1.1 for i in range(nv)]
    now = 0.0
    held = []
    loading = []
    failed = 0
    for step in range(3000):
        now += rng.expovariate(4.0)
        v = rng.choices(range(nv), weights)[0]
        got = c.bd_cache_request(v, now)
        want = m.request(v, now)
        assert got == want, (step, v, got, want)
        if got[0] != "busy":
            held.append(v)
        if got[0] == "load":
            loading.append(v)
        if loading and rng.random() < 0.5:
            u = loading.pop(0)
            if c.bd_cache_query(u)[0] >= 0:
                if rng.random() < 0.15:
                    # the load failed: every request waiting on it is dropped
                    c.bd_cache_load_failed(u)
                    m.load_failed(u)
                    failed += 1
                    held = [h for h in held if h != u]
                else:
                    c.bd_cache_complete(u)
                    m.ready[m.slot_of[u]] = True
        if len(held) > rng.randint(0, 12):
            rng.shuffle(held)
            while held:
                u = held.pop()
                c.bd_cache_release(u)
                m.refs[m.slot_of[u]] -= 1
        for u in range(nv):
            s, st, r = c.bd_cache_query(u)
            ms = m.slot_of[u]
            assert s == ms and r == (m.refs[ms] if ms >= 0 else 0)
    st = c.bd_cache_get_stats()
    assert st["requests"] == 3000
    assert failed > 0
    assert st["hits"] + st["joins"] + st["loads"] + st["busy"] + failed == 3000


def test_a_failed_load_frees_its_slot():
    c = make(nv=6, slots=3, pinned=0)
    _fill(c, [0, 1, 2])
    a, s, e = c.bd_cache_request(3, 10.0)          # evicts 0, the least recent
    assert (a, e) == ("load", 0)
    assert c.bd_cache_request(3, 10.5)[0] == "join"
    c.bd_cache_load_failed(3)
    assert c.bd_cache_query(3) == (-1, -1, 0)       # not resident, no reference left
    assert c.bd_cache_query(0)[0] == -1             # the evicted variant stays evicted
    st = c.bd_cache_get_stats()
    assert st["loads"] == 3 and st["bytes_loaded"] == 3 << 20 and st["evictions"] == 1
    with pytest.raises(bitdelta.BitDeltaError) as ei:
        c.bd_cache_release(3)                       # the failed requests hold nothing
    assert ei.value.status == 2
    with pytest.raises(bitdelta.BitDeltaError):
        c.bd_cache_load_failed(3)                   # nothing is loading any more
    with pytest.raises(bitdelta.BitDeltaError):
        c.bd_cache_load_failed(1)                   # resident, not loading
    # the freed slot is taken without another eviction
    a, s2, e = c.bd_cache_request(4, 11.0)
    assert (a, s2, e) == ("load", s, -1)
    c.bd_cache_complete(4)
    c.bd_cache_release(4)
    assert c.bd_cache_request(3, 12.0)[0] == "load"  # and 3 can be asked for again


def test_top_six_of_fourteen_stay_resident():
    # the post's deployment: 14 variants, the 6 busiest always resident, the
    # other 8 sharing the remaining slots under LRU
    rng = random.Random(7)
    nv, slots = 14, 10
    c = bd_cache(nv, slots, 6, 30.0, 4096)
    heavy = list(range(6))
    now = 0.0
    evicted = []
    for step in range(4000):
        now += 0.05
        v = rng.choice(heavy) if rng.random() < 0.8 else rng.randrange(6, 14)
        a, s, e = c.bd_cache_request(v, now)
        if a == "load":
            c.bd_cache_complete(v)
        if a != "busy":
            c.bd_cache_release(v)
        if e >= 0 and step > 500:
            evicted.append(e)
    assert evicted and all(e >= 6 for e in evicted)
    for v in heavy:
        assert c.bd_cache_query(v)[1] == 1


def test_c_abi_checks_before_any_hip_call():
    # argument checks of the device-mode entry points run on the host first,
    # so they answer on a machine without a GPU
    import ctypes
    from tenant_serving_amd.cache import CacheConfig, CacheGrant, declare
    lib = declare(bitdelta.library())
    cfg = CacheConfig(4, 2, 1, 10.0, 4096)
    h = ctypes.c_void_p(0)
    assert lib.bd_cache_create(ctypes.byref(cfg), ctypes.c_void_p((1 << 20) + 8), None, ctypes.byref(h)) == 3
    assert lib.bd_cache_create(None, None, None, ctypes.byref(h)) == 1
    assert lib.bd_cache_create(ctypes.byref(cfg), None, None, None) == 1
    assert lib.bd_cache_create(ctypes.byref(cfg), None, None, ctypes.byref(h)) == 0
    g = CacheGrant()
    ptr = ctypes.c_void_p(0)
    # device-mode calls on a policy-mode cache are refused
    assert lib.bd_cache_acquire(h, 0, 0.0, None, ctypes.byref(ptr), ctypes.byref(g)) == 2
    assert lib.bd_cache_set_source(h, 0, ctypes.c_void_p(1 << 20)) == 2
    n = ctypes.c_int32(0)
    busy = ctypes.c_int32(0)
    assert lib.bd_cache_acquire_batch(h, None, 0, 0.0, None, None, None, None, ctypes.byref(n),
                                      ctypes.byref(busy)) == 2
    # and policy-mode calls answer
    assert lib.bd_cache_request(h, 5, 0.0, ctypes.byref(g)) == 2     # out of range
    assert lib.bd_cache_request(h, 1, 0.0, ctypes.byref(g)) == 0 and g.action == 2
    assert lib.bd_cache_release_batch(h, None, -1, None) == 2
    assert lib.bd_cache_destroy(h) == 0
    assert lib.bd_cache_destroy(None) == 0
