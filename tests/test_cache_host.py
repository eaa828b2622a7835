"""Host logic of the user-keyed sketch cache (sa_cache_lookup, no GPU).

The library's lookup is checked, request by request, against a separate
plain-Python model of the policy include/sa.h states (freshness while
now - t_computed < ttl; a miss takes the lowest free slot, else the expired
entry used least recently, else the least recently used entry that the
current batch does not hold; repeated users within a batch share one miss;
stale entries are recomputed in place), on seeded synthetic request traces:
skewed user popularity, batches of requests with increasing timestamps, TTL
crossings and evictions."""
import ctypes

import numpy as np
import pytest

import prototype_attention_compression_amd as sa
from prototype_attention_compression_amd import _lib

FAKE_SLAB = 0x100000   # never dereferenced by the host-only calls


class Model:
    def __init__(self, cap, ttl):
        self.cap, self.ttl = cap, ttl
        self.entries = {}            # user -> [slot, t_computed, t_used, batch]
        self.slot_user = [None] * cap
        self.batch = 0

    def lookup(self, users, now):
        self.batch += 1
        b = self.batch
        slots, misses = [], []
        st = dict(hits=0, misses=0, evictions=0, expired=0)
        for u in users:
            e = self.entries.get(u)
            if e is not None:
                if now - e[1] < self.ttl or e[3] == b:
                    e[2], e[3] = now, b
                    slots.append(e[0])
                    st["hits"] += 1
                    continue
                e[1], e[2], e[3] = now, now, b
                slots.append(e[0])
                misses.append((u, e[0]))
                st["misses"] += 1
                st["expired"] += 1
                continue
            free = [s for s in range(self.cap) if self.slot_user[s] is None]
            if free:
                slot = free[0]
            else:
                cands = [s for s in range(self.cap) if self.entries[self.slot_user[s]][3] != b]
                if not cands:
                    raise RuntimeError("capacity")
                # expired first, then least recently used, then lowest slot
                def key(s):
                    e2 = self.entries[self.slot_user[s]]
                    return (0 if now - e2[1] >= self.ttl else 1, e2[2], s)
                slot = min(cands, key=key)
                del self.entries[self.slot_user[slot]]
                st["evictions"] += 1
            self.slot_user[slot] = u
            self.entries[u] = [slot, now, now, b]
            slots.append(slot)
            misses.append((u, slot))
            st["misses"] += 1
        return slots, misses, st


@pytest.mark.parametrize("seed,cap,ttl", [(0, 8, 10.0), (1, 3, 2.5), (2, 32, 100.0), (3, 5, 1.0)])
def test_lookup_matches_policy_model(seed, cap, ttl):
    g = np.random.default_rng(seed)
    cache = sa.SketchCache(cap, 64, 64, ttl, FAKE_SLAB)
    model = Model(cap, ttl)
    now = 0.0
    tot = dict(hits=0, misses=0)
    for _ in range(60):
        now += float(g.exponential(ttl / 4))
        n = int(g.integers(0, 2 * cap))
        # skewed popularity: a few users recur often
        users = (g.zipf(1.6, size=n) % (4 * cap)).astype(np.int64)
        # never more distinct users in a batch than slots
        keep, seen = [], set()
        for u in users:
            if u in seen or len(seen) < cap:
                keep.append(u)
                seen.add(u)
        users = np.array(keep, dtype=np.int64)
        slots, mu, ms, st = cache.lookup(users, now)
        rslots, rmiss, rst = model.lookup(users.tolist(), now)
        assert slots.tolist() == rslots
        assert list(zip(mu.tolist(), ms.tolist())) == rmiss
        assert st == rst
        tot["hits"] += st["hits"]
        tot["misses"] += st["misses"]
        # every request's slot holds its user
        for u, s in zip(users.tolist(), slots.tolist()):
            assert model.slot_user[s] == u
    assert tot["hits"] > 0 and tot["misses"] > 0
    cache.close()


def test_ttl_and_batch_sharing():
    cache = sa.SketchCache(2, 64, 64, 10.0, FAKE_SLAB)
    slots, mu, ms, st = cache.lookup([7, 7, 9, 7], 0.0)
    assert st == dict(hits=2, misses=2, evictions=0, expired=0)
    assert slots.tolist() == [0, 0, 1, 0] and mu.tolist() == [7, 9]
    _, mu, _, st = cache.lookup([9, 7], 9.9)          # both fresh
    assert st["hits"] == 2 and mu.size == 0
    _, mu, ms, st = cache.lookup([7], 10.0)            # age 10 = ttl: stale, recomputed in place
    assert st == dict(hits=0, misses=1, evictions=0, expired=1) and ms.tolist() == [0]
    _, mu, ms, st = cache.lookup([11], 10.5)           # full: evict 9 (expired) not 7 (fresh)
    assert mu.tolist() == [11] and ms.tolist() == [1] and st["evictions"] == 1
    _, mu, _, st = cache.lookup([7, 9], 11.0)          # 9 was evicted: a miss again (evicting 11)
    assert mu.tolist() == [9] and st["hits"] == 1
    with pytest.raises(sa.SaError):
        cache.lookup([1, 2, 3], 12.0)                  # three distinct users, two slots
    cache.close()


def test_hit_rate_of_repeated_instances():
    """Training-style trace: every user recurs about twice within the TTL, so
    about half of the instances hit (the pages quote 0.5 for training)."""
    g = np.random.default_rng(5)
    users = np.repeat(np.arange(4000), 2)
    g.shuffle(users)
    cache = sa.SketchCache(8000, 64, 64, 3 * 3600.0, FAKE_SLAB)
    hits = misses = 0
    for i in range(0, users.size, 40):                 # R = 40 instances per batch
        _, _, _, st = cache.lookup(users[i:i + 40], i / 40.0)
        hits += st["hits"]
        misses += st["misses"]
    assert misses == 4000 and hits == 4000
    cache.close()


def test_argument_errors():
    lib = _lib.load()
    h = ctypes.c_void_p()
    assert lib.sa_cache_create(0, 64, 64, 1.0, FAKE_SLAB, None, ctypes.byref(h)) == sa.SA_E_INVALID
    assert lib.sa_cache_create(4, 64, 64, 0.0, FAKE_SLAB, None, ctypes.byref(h)) == sa.SA_E_INVALID
    assert lib.sa_cache_create(4, 64, 64, 1.0, None, None, ctypes.byref(h)) == sa.SA_E_INVALID
    assert lib.sa_cache_create(4, 64, 64, 1.0, FAKE_SLAB + 4, None, ctypes.byref(h)) == sa.SA_E_INVALID
    assert lib.sa_cache_create(4, 64, 64, 1.0, FAKE_SLAB, None, None) == sa.SA_E_INVALID
    pb = _lib.problem(3, 100, 128, 256, 0)
    out = ctypes.c_size_t(0)
    assert lib.sa_cache_fill_workspace_size(ctypes.byref(pb), 3, 100, ctypes.byref(out)) == sa.SA_OK
    assert out.value >= sa.workspace_size(3, 100, 128, 256)
    assert lib.sa_cache_fill_workspace_size(ctypes.byref(pb), -1, 100, ctypes.byref(out)) == sa.SA_E_INVALID


def test_refused_batch_leaves_the_cache_unchanged():
    """A batch with more distinct users than slots is refused before any
    state changes: the lookups that follow give exactly what they give on a
    cache that never saw the refused batch (slots, misses, statistics)."""
    g = np.random.default_rng(9)
    cap, ttl = 6, 5.0
    a = sa.SketchCache(cap, 64, 64, ttl, FAKE_SLAB)
    b = sa.SketchCache(cap, 64, 64, ttl, FAKE_SLAB)
    now = 0.0
    for step in range(40):
        now += float(g.exponential(1.0))
        users = g.integers(0, 12, size=int(g.integers(1, 9))).astype(np.int64)
        if len(set(users.tolist())) > cap:
            users = users[:cap]
        if step % 5 == 2:
            # some users already cached, then more distinct users than slots
            refused = np.concatenate([users, np.arange(100, 100 + cap + 1)]).astype(np.int64)
            with pytest.raises(sa.SaError):
                a.lookup(refused, now)
        ra, rb = a.lookup(users, now), b.lookup(users, now)
        assert ra[0].tolist() == rb[0].tolist()
        assert ra[1].tolist() == rb[1].tolist() and ra[2].tolist() == rb[2].tolist()
        assert ra[3] == rb[3]
    a.close()
    b.close()
