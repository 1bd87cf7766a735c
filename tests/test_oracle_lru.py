"""Pins for oracle/lru.py: hand-worked traces, an independent list LRU, LRU properties."""

import os

import numpy as np
from hypothesis import given, settings, strategies as st

from oracle.lru import HIT, MISS_CPU, MISS_STREAM, LRUPool, hybrid_cpu_count, split_waves

GOLD = os.path.join(os.path.dirname(__file__), "golden")
FL = {"H": HIT, "S": MISS_STREAM, "C": MISS_CPU}


def _run_call(pool, layer, sel, share):
    flags, slots, ev = [], [], 0
    for t0, t1 in split_waves(sel, pool.C):
        r = pool.resolve_wave(layer, sel[t0:t1], share)
        flags += list(r["flag"])
        slots += list(r["slot"])
        ev += r["evictions"]
    return flags, slots, ev


def test_golden_traces():
    pool, share, n = None, 0.0, 0
    for line in open(os.path.join(GOLD, "lru_traces.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        tok = line.split()
        if tok[0] == "pool":
            pool, share = LRUPool(int(tok[1])), float(tok[3])
            continue
        lhs, rhs = line.split("->")
        lt = lhs.split()
        layer, k = int(lt[1]), int(lt[2].split("=")[1])
        sel = np.array([int(v) for v in lt[3:]]).reshape(-1, k)
        ef, es, ev = [s.split() for s in rhs.split(";")]
        flags, slots, evn = _run_call(pool, layer, sel, share)
        assert flags == [FL[f] for f in ef], line
        assert slots == [int(s) for s in es], line
        assert evn == int(ev[0]), line
        n += 1
    assert n == 17


class ListLRU:
    """Independent brute force: an explicit recency list plus a slot map.

    Per wave: victims are taken from the free slots (ascending) and then from
    the recency list (oldest first) skipping this wave's hits; afterwards the
    touched keys move to the recent end in order of their last pair.
    """

    def __init__(self, C):
        self.C = C
        self.order = []  # keys, least recent first
        self.slot = {}
        self.free = list(range(C))

    def wave(self, layer, pairs, share):
        D = []
        last = {}
        for p, e in enumerate(pairs):
            if e not in last:
                D.append(e)
            last[e] = p
        hits = [e for e in D if (layer, e) in self.slot]
        miss = [e for e in D if (layer, e) not in self.slot]
        ncpu = int(np.floor(len(miss) * share + 0.5))
        stream = miss[:len(miss) - ncpu]
        cpu = miss[len(miss) - ncpu:]
        hitkeys = {(layer, e) for e in hits}
        cand = list(self.free) + [k for k in self.order if k not in hitkeys]
        ev = 0
        for e in stream:
            c = cand.pop(0)
            if isinstance(c, int):
                self.free.remove(c)
                s = c
            else:
                s = self.slot.pop(c)
                self.order.remove(c)
                ev += 1
            self.slot[(layer, e)] = s
        touched = sorted(hits + stream, key=lambda e: last[e])
        for e in touched:
            if (layer, e) in self.order:
                self.order.remove((layer, e))
            self.order.append((layer, e))
        out = []
        for e in pairs:
            if e in hits:
                out.append((HIT, self.slot[(layer, e)]))
            elif e in cpu:
                out.append((MISS_CPU, -1))
            else:
                out.append((MISS_STREAM, self.slot[(layer, e)]))
        return out, ev


def _random_calls(rng, L, E, k, ncalls, maxT):
    calls = []
    for _ in range(ncalls):
        T = int(rng.integers(1, maxT + 1))
        layer = int(rng.integers(0, L))
        pop = rng.zipf(1.3, size=(T, 4 * k)) % E
        sel = np.zeros((T, k), np.int64)
        for t in range(T):
            seen = []
            for v in list(pop[t]) + list(rng.permutation(E)):
                if v not in seen:
                    seen.append(int(v))
                if len(seen) == k:
                    break
            sel[t] = seen
        calls.append((layer, sel))
    return calls


@settings(max_examples=60, deadline=None)
@given(seed=st.integers(0, 10_000), C=st.integers(2, 12), share=st.sampled_from([0.0, 0.0, 0.3, 0.5, 1.0]))
def test_matches_independent_list_lru(seed, C, share):
    rng = np.random.default_rng(seed)
    k = int(rng.integers(1, min(C, 3) + 1))
    calls = _random_calls(rng, L=3, E=9, k=k, ncalls=25, maxT=4)
    pool, ref = LRUPool(C), ListLRU(C)
    for layer, sel in calls:
        for t0, t1 in split_waves(sel, C):
            r = pool.resolve_wave(layer, sel[t0:t1], share)
            exp, ev = ref.wave(layer, [int(v) for v in sel[t0:t1].reshape(-1)], share)
            assert list(zip(r["flag"], r["slot"])) == exp
            assert r["evictions"] == ev
            assert r["pair_hits"] + (len(exp) - r["pair_hits"]) == sel[t0:t1].size


@settings(max_examples=40, deadline=None)
@given(seed=st.integers(0, 10_000))
def test_capacity_at_least_all_keys_gives_only_compulsory_misses(seed):
    rng = np.random.default_rng(seed)
    L, E, k = 3, 8, 2
    pool = LRUPool(L * E)
    seen = set()
    for layer, sel in _random_calls(rng, L, E, k, 40, 5):
        for t0, t1 in split_waves(sel, pool.C):
            r = pool.resolve_wave(layer, sel[t0:t1])
            new = {(layer, int(e)) for e in sel[t0:t1].reshape(-1)} - seen
            assert r["expert_misses"] == len(new)
            assert r["evictions"] == 0
            seen |= new


@settings(max_examples=30, deadline=None)
@given(seed=st.integers(0, 10_000))
def test_inclusion_hits_nondecreasing_in_capacity(seed):
    # With no wave splits the step-set pool is a stack algorithm: the residents
    # are the C most recently used keys, so a larger pool never hits less.
    rng = np.random.default_rng(seed)
    k = 2
    calls = _random_calls(rng, 2, 10, k, 40, 2)  # <= 4 distinct per call
    prev = -1
    for C in range(4, 21):
        pool = LRUPool(C)
        hits = 0
        for layer, sel in calls:
            waves = split_waves(sel, C)
            assert len(waves) == 1
            hits += pool.resolve_wave(layer, sel)["pair_hits"]
        assert hits >= prev
        prev = hits


def test_cyclic_trace_larger_than_pool_never_hits():
    for C in (1, 3, 8):
        pool = LRUPool(C)
        for rep in range(5):
            for e in range(C + 1):
                r = pool.resolve_wave(0, np.array([[e]]))
                assert r["pair_hits"] == 0


def test_hits_plus_misses_equal_pairs_and_slots_unique():
    rng = np.random.default_rng(11)
    pool = LRUPool(6)
    for layer, sel in _random_calls(rng, 2, 12, 3, 50, 6):
        for t0, t1 in split_waves(sel, pool.C):
            r = pool.resolve_wave(layer, sel[t0:t1])
            P = sel[t0:t1].size
            assert r["pair_hits"] + int((r["flag"] != HIT).sum()) == P
            keys = [k for k in pool.key_of if k is not None]
            assert len(keys) == len(set(keys)) == len(pool.slot_of)
            for key, s in pool.slot_of.items():
                assert pool.key_of[s] == key


def test_hybrid_share_zero_is_pure_offload_and_share_one_moves_nothing():
    rng = np.random.default_rng(12)
    calls = _random_calls(rng, 2, 10, 2, 40, 4)
    a, b = LRUPool(5), LRUPool(5)
    for layer, sel in calls:
        for t0, t1 in split_waves(sel, 5):
            ra = a.resolve_wave(layer, sel[t0:t1], 0.0)
            rb = b.resolve_wave(layer, sel[t0:t1])
            assert np.array_equal(ra["flag"], rb["flag"]) and np.array_equal(ra["slot"], rb["slot"])
    c = LRUPool(5)
    for layer, sel in calls:
        before = list(c.key_of)
        for t0, t1 in split_waves(sel, 5):
            r = c.resolve_wave(layer, sel[t0:t1], 1.0)
            assert r["evictions"] == 0 and not r["stream"]
        assert c.key_of == before


def test_hybrid_count_rounding():
    assert hybrid_cpu_count(3, 0.5) == 2
    assert hybrid_cpu_count(1, 0.5) == 1
    assert hybrid_cpu_count(64, 0.03) == 2
    assert hybrid_cpu_count(0, 0.7) == 0


def test_prefill_staging_slots_and_evictions():
    pool = LRUPool(10)
    for e in range(6):
        pool.resolve_wave(1, np.array([[e]]))  # keys (1,0..5) -> slots 0..5
    sel = np.array([[3, 1], [0, 3]])
    r = pool.stage_layer(0, 4, sel, num_layers=2)
    assert list(r["slot"]) == [3, 1, 0, 3] and (r["flag"] == MISS_STREAM).all()
    # both halves [0,4) and [4,8) are emptied: slots 0..5 held residents
    assert r["evictions"] == 6 and not pool.resident(1, 2)
    r = pool.stage_layer(1, 4, sel, num_layers=2)
    assert list(r["slot"]) == [7, 5, 4, 7] and r["evictions"] == 0
    # a decode access afterwards takes the lowest free slot
    assert pool.resolve_wave(1, np.array([[9]]))["stream"] == [(9, 0)]
