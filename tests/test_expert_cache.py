"""Host logic of the tiered expert store: the slot cache and pass planner
(colibri_cache_* in include/colibri.h, expert_cache.cpp), run without a GPU.

Two kinds of checks:
  * a plain-Python model of the documented policy (distinct experts in order
    of first appearance; hits in pass 0; misses over a ring of free slots in
    LRU order followed by unpinned hit slots; chunks of max(1, R/2) misses
    with miss i in ring slot i mod R when the misses do not fit) must give
    the same codes, loads, pass sizes and slot map after every plan;
  * semantic invariants that hold for any correct planner, checked by
    replaying the plan: every pass finds each of its pairs' experts in the
    slot its code names, no load overwrites a slot that a pass at or after
    the load's wait point still reads, pinned slots are never overwritten,
    loads of one pass go to distinct slots, and every routed expert that
    was not resident is loaded exactly once.
"""

import random

import pytest

import quantized_routed_expert_sigmoid_amd as q

pytestmark = pytest.mark.skipif(not __import__("os").path.exists(q.LIB_PATH),
                                reason="libcolibri.so not built")

B = q.PLAN_SLOT_BITS


class ModelCache:
    """The documented policy, written out plainly."""

    def __init__(self, E, n):
        self.E, self.n = E, n
        self.expert_in = [-1] * n
        self.last = [0] * n
        self.pinned = [False] * n
        self.inflight = [False] * n
        self.tick = 0

    def slot_of(self, e):
        return self.expert_in.index(e) if e in self.expert_in else -1

    def victims(self, excluded):
        cand = [s for s in range(self.n) if not self.pinned[s] and s not in excluded]
        return sorted(cand, key=lambda s: (self.expert_in[s] >= 0,
                                           self.last[s] if self.expert_in[s] >= 0 else 0, s))

    def place(self, e, s):
        self.expert_in[s] = e
        self.last[s] = self.tick

    def pin(self, experts):
        self.tick += 1
        loads = []
        for e in experts:
            s = self.slot_of(e)
            if s < 0:
                s = self.victims(set())[0]
                self.place(e, s)
                loads.append((e, s))
            self.pinned[s] = True
            self.last[s] = self.tick
        return loads

    def plan(self, ids):
        self.tick += 1
        order = list(dict.fromkeys(e for e in ids if e >= 0))
        hits = {}
        for e in order:
            s = self.slot_of(e)
            if s >= 0:
                hits[e] = s
                self.last[s] = self.tick
        misses = [e for e in order if e not in hits]
        free = self.victims(set(hits.values()))
        # when the misses fit the free slots, a hit on a slot a prefetch
        # filled (late) runs in pass 1 and stays out of the ring
        late = {e for e, s in hits.items() if self.inflight[s]} if len(misses) <= len(free) else set()
        ring = free + sorted(s for e, s in hits.items() if not self.pinned[s] and e not in late)
        ready = [-1] * len(free) + [0] * (len(ring) - len(free))
        R, m = len(ring), len(misses)
        where = {e: (1 if e in late else 0, s) for e, s in hits.items()}
        loads = []
        n_pass = 1
        if m:
            c = m if m <= R else max(1, R // 2)
            for i, e in enumerate(misses):
                p, r = 1 + i // c, i % R
                loads.append((e, ring[r], p, ready[r]))
                ready[r] = p
                self.place(e, ring[r])
                where[e] = (p, ring[r])
            n_pass = 1 + (m + c - 1) // c
        if late:
            n_pass = max(n_pass, 2)
        self.inflight = [False] * self.n
        codes = [-1 if e < 0 else (where[e][0] << B) | where[e][1] for e in ids]
        pp = [0] * n_pass
        for e in ids:
            if e >= 0:
                pp[where[e][0]] += 1
        return codes, loads, pp

    def prefetch(self, ids):
        self.tick += 1
        order = list(dict.fromkeys(e for e in ids if e >= 0))
        hits = {}
        for e in order:
            s = self.slot_of(e)
            if s >= 0:
                hits[e] = s
                self.last[s] = self.tick
        free = self.victims(set(hits.values()))
        misses = [e for e in order if e not in hits]
        loads = []
        for e, s in zip(misses, free):
            self.place(e, s)
            self.inflight[s] = True
            loads.append((e, s, 1, -1))
        return loads

    def slot_map(self):
        m = [-1] * self.E
        for s, e in enumerate(self.expert_in):
            if e >= 0:
                m[e] = s
        return m


def check_invariants(before_slot_of, pinned_slots, ids, res, n_slots):
    """Replays a plan against the slot contents before it."""
    contents = [-1] * n_slots
    for e, s in enumerate(before_slot_of):
        if s >= 0:
            contents[s] = e
    n_pass = res["n_pass"]
    loads = res["loads"]
    # passes reading each slot's current content, per slot
    readers = {s: set() for s in range(n_slots)}
    by_pass = {}
    for e, s, p, after in loads:
        by_pass.setdefault(p, []).append((e, s, after))
    pair_pass = {}
    for p_idx, (e, code) in enumerate(zip(ids, res["codes"])):
        if e < 0:
            assert code == -1
            continue
        assert code >= 0
        pair_pass.setdefault(code >> B, []).append((e, code & ((1 << B) - 1)))
    resident_before = {e for e, s in enumerate(before_slot_of) if s >= 0}
    routed = {e for e in ids if e >= 0}
    loaded = [e for e, _, _, _ in loads]
    assert sorted(loaded) == sorted(routed - resident_before), "each miss loaded exactly once"
    assert res["n_hit"] == len(routed & resident_before)
    assert res["n_miss"] == len(loaded)
    assert sum(res["pass_pairs"]) == sum(1 for e in ids if e >= 0)
    for p in range(n_pass):
        # loads needed by pass p
        slots_p = [s for _, s, _ in by_pass.get(p, [])]
        assert len(slots_p) == len(set(slots_p)), "one pass loads distinct slots"
        for e, s, after in by_pass.get(p, []):
            assert 0 <= after < p or after == -1
            assert s not in pinned_slots, "pinned slot overwritten"
            # every pass that read the old content must be <= after
            assert all(r <= after for r in readers[s]), (s, readers[s], after)
            contents[s] = e
            readers[s] = set()
        pairs = pair_pass.get(p, [])
        assert len(pairs) == res["pass_pairs"][p]
        for e, s in pairs:
            assert contents[s] == e, f"pass {p} reads slot {s} holding {contents[s]}, wants {e}"
            readers[s].add(p)
    assert set(pair_pass) <= set(range(n_pass))
    return contents


def run_sequence(E, n_slots, batches, pins=()):
    c = q.ExpertCache(E, n_slots)
    m = ModelCache(E, n_slots)
    if pins:
        assert c.pin(pins) == m.pin(pins)
    pinned_slots = {s for s in range(n_slots) if m.pinned[s]}
    for ids in batches:
        before, _ = c.state()
        res = c.plan(ids)
        codes, loads, pp = m.plan(ids)
        assert res["codes"] == codes
        assert res["loads"] == loads
        assert res["pass_pairs"] == pp
        contents = check_invariants(before, pinned_slots, ids, res, n_slots)
        slot_of, _ = c.state()
        assert slot_of == m.slot_map()
        for s, e in enumerate(contents):
            assert e < 0 or slot_of[e] == s
    return c, m


def random_batches(rng, E, n_batches, max_pairs, p_drop=0.1, hot=None):
    out = []
    for _ in range(n_batches):
        P = rng.randint(1, max_pairs)
        ids = []
        for _ in range(P):
            if rng.random() < p_drop:
                ids.append(-1)
            elif hot and rng.random() < 0.6:
                ids.append(rng.choice(hot))
            else:
                ids.append(rng.randrange(E))
        out.append(ids)
    return out


@pytest.mark.parametrize("seed", range(12))
def test_plans_match_model_and_invariants(seed):
    rng = random.Random(seed)
    E = rng.choice([4, 8, 16, 33, 64, 256])
    n_slots = rng.randint(1, E)
    hot = rng.sample(range(E), max(1, E // 8))
    batches = random_batches(rng, E, 30, rng.choice([2, 8, 24, 80]), hot=hot)
    run_sequence(E, n_slots, batches)


@pytest.mark.parametrize("seed", range(6))
def test_plans_with_pins(seed):
    rng = random.Random(100 + seed)
    E = rng.choice([8, 16, 64])
    n_slots = rng.randint(2, E)
    pins = rng.sample(range(E), rng.randint(1, n_slots - 1))
    batches = random_batches(rng, E, 25, 40)
    c, _ = run_sequence(E, n_slots, batches, pins)
    st = c.stats()
    assert st["pinned"] == len(pins)
    slot_of, _ = c.state()
    assert all(slot_of[e] >= 0 for e in pins), "pinned experts stay resident"


def test_single_slot_runs_one_miss_per_pass():
    c = q.ExpertCache(6, 1)
    r = c.plan([0, 1, 2, 1, 0])
    assert r["n_pass"] == 4 and r["pass_pairs"] == [0, 2, 2, 1]
    assert [l[3] for l in r["loads"]] == [-1, 1, 2]  # each load waits for the previous pass


@pytest.mark.parametrize("n_slots,n_pass", [(8, 11), (3, 41), (5, 21), (2, 41)])
def test_double_buffered_chunks_overlap(n_slots, n_pass):
    """With R >= 2 ring slots, a chunk's loads never wait for the pass right
    before it (they overlap its compute), and every slot is used."""
    c = q.ExpertCache(64, n_slots)
    r = c.plan(list(range(40)))
    assert r["n_pass"] == n_pass  # c = max(1, R // 2)
    for e, s, p, after in r["loads"]:
        assert after <= p - 2
    assert sorted({s for _, s, _, _ in r["loads"]}) == list(range(n_slots))


def test_hits_run_in_pass_zero_and_lru_victim():
    c = q.ExpertCache(8, 4)
    c.plan([0, 1, 2, 3])          # slots 0..3 = experts 0..3
    c.plan([2, 3])                # 0 and 1 become the oldest
    r = c.plan([4, 2])            # 2 hits, 4 misses -> victim: slot of expert 0
    assert r["n_hit"] == 1 and r["codes"][1] == (0 << B) | 2
    assert r["loads"] == [(4, 0, 1, -1)]
    slot_of, usage = c.state()
    assert slot_of[0] == -1 and slot_of[4] == 0
    assert usage[2] == 3 and usage[4] == 1


def test_full_residency_never_misses():
    E = 16
    c = q.ExpertCache(E, E)
    loads = c.pin(list(range(E)))
    assert sorted(s for _, s in loads) == list(range(E))
    rng = random.Random(5)
    for ids in random_batches(rng, E, 10, 64):
        r = c.plan(ids)
        assert r["n_miss"] == 0 and r["n_pass"] == 1


def test_pin_limits_and_validation():
    c = q.ExpertCache(8, 4)
    with pytest.raises(q.ColibriError) as ei:
        c.pin([0, 1, 2, 3])       # would leave no slot for misses
    assert ei.value.status == q.COLI_E_UNSUPPORTED
    assert c.stats()["pinned"] == 0 and c.stats()["resident"] == 0
    with pytest.raises(q.ColibriError):
        c.pin([1, 1])             # repeated
    with pytest.raises(q.ColibriError):
        c.pin([8])                # out of range
    assert c.pin([5, 6, 7]) == [(5, 0), (6, 1), (7, 2)]
    assert c.pin([5]) == []       # already pinned: no load, no new pin
    with pytest.raises(q.ColibriError):
        c.pin([0])                # the fourth pin would fill every slot
    c.unpin()
    assert c.stats()["pinned"] == 0 and c.stats()["resident"] == 3


def test_plan_validation_changes_nothing():
    c = q.ExpertCache(8, 2)
    c.plan([1, 2])
    before = c.state(), c.stats()
    with pytest.raises(q.ColibriError):
        c.plan([0, 8])
    assert (c.state(), c.stats()) == before
    r = c.plan([])
    assert r["n_pass"] == 1 and r["codes"] == [] and r["pass_pairs"] == [0]
    r = c.plan([-1, -1])
    assert r["codes"] == [-1, -1] and r["n_hit"] == 0 and r["n_miss"] == 0
    for bad in [(0, 1), (4, 0), (4, 5), (2000, 2)]:
        with pytest.raises(q.ColibriError):
            q.ExpertCache(*bad)


def test_stats_accumulate():
    c = q.ExpertCache(16, 4)
    rng = random.Random(9)
    batches = random_batches(rng, 16, 20, 12)
    hits = misses = passes = pairs = 0
    for ids in batches:
        r = c.plan(ids)
        hits += r["n_hit"]
        misses += r["n_miss"]
        passes += r["n_pass"]
        pairs += sum(1 for e in ids if e >= 0)
    st = c.stats()
    assert (st["plans"], st["hits"], st["misses"], st["passes"], st["pairs"]) == \
        (len(batches), hits, misses, passes, pairs)
    _, usage = c.state()
    assert sum(usage) == pairs


@pytest.mark.parametrize("seed", range(8))
def test_prefetch_matches_model(seed):
    """Look-ahead prefetches interleaved with plans: same loads and slot map
    as the model; a prefetch never gives up the slot of a predicted expert or
    a pinned one, never counts usage, and a plan of the predicted batch right
    after it finds every prefetched expert resident."""
    rng = random.Random(500 + seed)
    E = rng.choice([8, 16, 64, 256])
    n_slots = rng.randint(2, E)
    c = q.ExpertCache(E, n_slots)
    m = ModelCache(E, n_slots)
    if seed % 2:
        pins = rng.sample(range(E), rng.randint(1, n_slots - 1))
        assert c.pin(pins) == m.pin(pins)
    pinned_slots = {s for s in range(n_slots) if m.pinned[s]}
    for ids in random_batches(rng, E, 30, 24, hot=rng.sample(range(E), max(1, E // 8))):
        if rng.random() < 0.5:
            before, usage_before = c.state()
            st_before = c.stats()
            r = c.prefetch(ids)
            loads = m.prefetch(ids)
            assert r["loads"] == loads
            assert all(s not in pinned_slots for _, s, _, _ in loads)
            predicted = {e for e in ids if e >= 0}
            for e, s in enumerate(before):
                if e in predicted and s >= 0:
                    assert c.state()[0][e] == s, "a predicted resident expert kept its slot"
            assert c.state()[1] == usage_before
            st = c.stats()
            assert st["prefetches"] == st_before["prefetches"] + 1
            assert st["prefetch_loads"] == st_before["prefetch_loads"] + len(loads)
            assert st["plans"] == st_before["plans"]
            if len(predicted) <= n_slots - len(pinned_slots):
                # a plan of the predicted batch right after the prefetch: no
                # misses, the prefetched experts as late hits in pass 1
                r2 = c.plan(ids)
                codes, _, pp = m.plan(ids)
                assert r2["n_miss"] == 0 and r2["codes"] == codes and r2["pass_pairs"] == pp
                assert r2["n_pass"] == (2 if loads else 1)
        else:
            res = c.plan(ids)
            codes, loads, pp = m.plan(ids)
            assert (res["codes"], res["loads"], res["pass_pairs"]) == (codes, loads, pp)
        assert c.state()[0] == m.slot_map()
