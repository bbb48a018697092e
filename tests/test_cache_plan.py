"""The bounded expert cache's host logic (rl_cache_* in planning mode: no device memory), CPU only.

Its policy, as include/rl_moe.h states it: a prepare makes every requested expert resident at
once; each missing expert takes a free slot (lowest index first), else the slot whose expert was
requested least recently among those not in the current request (ties: lowest slot index).
Checked against an independent Python model of that policy on seeded request streams (slot of
every expert after every prepare, and the hit / miss / eviction counts), and by invariants that
any correct LRU union-prepare keeps: every requested expert is resident afterwards, at most
n_slots experts are, each evicted expert was requested no later than every resident expert outside
the request, and a request larger than the cache is refused without any change."""
import numpy as np
import pytest

import routed_experts_bit_amd as rl
from workload import make_experts


class Model:
    def __init__(self, E, n):
        self.slot = [-1] * n       # expert in each slot
        self.used = [-1] * n       # tick of the last request of each slot
        self.where = {}            # expert -> slot
        self.tick = 0
        self.hits = self.misses = self.evictions = 0

    def prepare(self, ids):
        req = list(dict.fromkeys(int(i) for i in ids))
        if len(req) > len(self.slot):
            return False
        self.tick += 1
        t = self.tick
        for e in req:
            if e in self.where:
                self.used[self.where[e]] = t
                self.hits += 1
        for e in req:
            if e in self.where:
                continue
            self.misses += 1
            free = [s for s in range(len(self.slot)) if self.slot[s] < 0]
            if free:
                v = free[0]
            else:
                cand = [s for s in range(len(self.slot)) if self.used[s] != t]
                v = min(cand, key=lambda s: (self.used[s], s))
                del self.where[self.slot[v]]
                self.evictions += 1
            self.slot[v], self.used[v], self.where[e] = e, t, v
        return True


@pytest.fixture(scope="module")
def experts():
    return make_experts(64, 256, 64, [1, 2] * 32, seed=91)


def _cache(experts, n):
    return rl.ExpertCache(experts.arena, experts.desc, experts.E, experts.H, experts.I, n, plan_only=True)


@pytest.mark.parametrize("n_slots,seed", [(16, 0), (1, 1), (10, 2), (64, 3), (33, 4)])
def test_matches_policy_model(experts, n_slots, seed):
    rng = np.random.default_rng(seed)
    c = _cache(experts, n_slots)
    m = Model(experts.E, n_slots)
    last = {}  # expert -> tick of its last request (for the LRU invariant)
    for step in range(300):
        size = int(rng.integers(1, min(n_slots, 12) + 1))
        # skewed requests (hot experts repeat) with duplicates inside a request
        ids = rng.choice(experts.E, size=size + int(rng.integers(0, 3)), p=None if step % 3 else
                         (lambda q: q / q.sum())(1.0 / np.arange(1, experts.E + 1) ** 1.2))
        ids = np.concatenate([ids, ids[:1]])
        if len(set(ids.tolist())) > n_slots:
            ids = np.array(list(dict.fromkeys(ids.tolist()))[:n_slots])
        before = {e: c.slot_of(e) for e in range(experts.E)}
        c.prepare(ids)
        assert m.prepare(ids)
        after = {e: c.slot_of(e) for e in range(experts.E)}
        assert after == {e: m.where.get(e, -1) for e in range(experts.E)}
        st = c.stats()
        assert (st["hits"], st["misses"], st["evictions"]) == (m.hits, m.misses, m.evictions)
        # invariants
        req = set(int(i) for i in ids)
        assert all(after[e] >= 0 for e in req)
        assert sum(v >= 0 for v in after.values()) <= n_slots
        evicted = [e for e in range(experts.E) if before[e] >= 0 and after[e] < 0]
        kept_outside = [e for e in range(experts.E) if after[e] >= 0 and e not in req]
        for e in evicted:
            assert all(last[e] <= last[o] for o in kept_outside)
        for e in req:
            last[e] = step


def test_refuses_oversized_request(experts):
    c = _cache(experts, 4)
    c.prepare([1, 2, 3])
    snap = [c.slot_of(e) for e in range(experts.E)], c.stats()
    with pytest.raises(rl.RlError, match="cache slots"):
        c.prepare([5, 6, 7, 8, 9])
    assert ([c.slot_of(e) for e in range(experts.E)], c.stats()) == snap
    c.prepare([9, 9, 9, 9, 9, 8, 7, 6])  # four distinct experts fit
    assert all(c.slot_of(e) >= 0 for e in (6, 7, 8, 9))


def test_rejects_bad_arguments(experts):
    c = _cache(experts, 8)
    with pytest.raises(rl.RlError):
        c.prepare([experts.E])
    with pytest.raises(rl.RlError):
        c.prepare([-1])
    with pytest.raises(rl.RlError):
        rl.ExpertCache(experts.arena, experts.desc, experts.E, experts.H, experts.I, experts.E + 1, plan_only=True)
    bad = experts.desc.copy()
    bad["down_off"][3] = experts.arena.size
    with pytest.raises(rl.RlError):
        rl.ExpertCache(experts.arena, bad, experts.E, experts.H, experts.I, 8, plan_only=True)
    assert rl.lib().rl_cache_slot_bytes(256, 64) == 3 * ((256 * 64 // 256 * 74 + 255) // 256 * 256)
    assert rl.lib().rl_cache_slot_bytes(200, 64) == 0
