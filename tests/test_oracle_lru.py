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


    def resize(self, new_C):
        # the new_C most recent keys survive; a surviving slot index below
        # new_C stays, the others move (ascending old slot) to the lowest free
        # indices below new_C
        n_ev = max(0, len(self.order) - new_C)
        for key in self.order[:n_ev]:
            del self.slot[key]
        self.order = self.order[n_ev:]
        stay = {key: s for key, s in self.slot.items() if s < new_C}
        movers = sorted((s, key) for key, s in self.slot.items() if s >= new_C)
        taken = set(stay.values())
        holes = [s for s in range(new_C) if s not in taken]
        for (s, key), t in zip(movers, holes):
            stay[key] = t
        self.slot = stay
        used = set(stay.values())
        self.free = [s for s in range(new_C) if s not in used]
        self.C = new_C


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


def test_prefill_hit_d2d_hand_worked():
    # C = 12, E = 4: the staging region is [0, 8)
    pool = LRUPool(12)
    pool.resolve_wave(0, np.array([[0]]))          # (0,0) -> slot 0 (inside staging)
    pool.resolve_wave(0, np.array([[1]]))          # (0,1) -> slot 1 (inside staging)
    for e in range(6):
        pool.resolve_wave(2, np.array([[e]]))      # (2,0..5) -> slots 2..7
    pool.resolve_wave(0, np.array([[2]]))          # (0,2) -> slot 8 (beyond staging)
    sel = np.array([[2, 0], [3, 2]])
    r = pool.stage_layer(0, 4, sel, num_layers=2, hit_d2d=True)
    # residents inside the staging region are evicted before residency is taken
    assert r["evictions"] == 8
    assert list(r["slot"]) == [8, 0, 3, 8]
    assert list(r["flag"]) == [HIT, MISS_STREAM, MISS_STREAM, HIT]
    assert r["stream"] == [(0, 0), (1, 1), (3, 3)]
    assert (r["pair_hits"], r["expert_hits"], r["expert_misses"]) == (2, 1, 3)
    # the copied experts 0, 1, 3 are residents of slots 0, 1, 3.  Clock 9 before
    # the call: the unselected copied expert 1 takes tick 9; then the pairs
    # [2, 0, 3, 2] (last positions 2->3, 0->1, 3->2) take 9 + 1 + position
    key, last, clock = pool.snapshot()
    assert key[:4] == [(0, 0), (0, 1), None, (0, 3)] and key[8] == (0, 2)
    assert (last[0], last[1], last[3], last[8], clock) == (11, 9, 12, 13, 14)
    assert all(k is None for k in key[4:8] + key[9:])


def test_prefill_hit_d2d_uses_resident_slots():
    # E = 4, C = 12: staging [0, 8); keys (1,2) and (1,0) resident at slots 8 and 9
    pool = LRUPool(12)
    for e in range(8):
        pool.resolve_wave(0, np.array([[e]]))      # keys (0,0..7) fill slots 0..7
    pool.resolve_wave(1, np.array([[2]]))          # -> slot 8
    pool.resolve_wave(1, np.array([[0]]))          # -> slot 9
    table_before = pool.snapshot()
    plain = LRUPool(12)
    plain.key_of, plain.last_use, plain.clock = list(table_before[0]), list(table_before[1]), table_before[2]
    plain.slot_of = {k: s for s, k in enumerate(table_before[0]) if k is not None}
    sel = np.array([[0, 3], [2, 0], [1, 2]])
    r0 = pool.stage_layer(0, 4, sel, num_layers=2, hit_d2d=True)
    assert r0["evictions"] == 8 and r0["expert_hits"] == 0
    p0 = plain.stage_layer(0, 4, sel, num_layers=2)
    r1 = pool.stage_layer(1, 4, sel, num_layers=2, hit_d2d=True)
    # layer 1 half is [4, 8): experts 0 and 2 are used from slots 9 and 8
    assert list(r1["slot"]) == [9, 7, 8, 9, 5, 8]
    assert list(r1["flag"]) == [HIT, MISS_STREAM, HIT, HIT, MISS_STREAM, HIT]
    assert r1["stream"] == [(1, 5), (3, 7)]
    assert r1["pair_hits"] == 4 and r1["expert_hits"] == 2 and r1["expert_misses"] == 2
    # evictions are those of plain staging (the clears); the table differs by
    # the registered copies and the clock
    p1 = plain.stage_layer(1, 4, sel, num_layers=2)
    assert (r0["evictions"], r1["evictions"]) == (p0["evictions"], p1["evictions"]) == (8, 0)
    key, last, clock = pool.snapshot()
    pkey, plast, pclock = plain.snapshot()
    # layer 0 (clock 10 -> 16, pairs [0,3,2,0,1,2]) and layer 1 (16 -> 22,
    # experts 1 and 3 copied into slots 5 and 7, 0 and 2 read from 9 and 8)
    assert key[:8] == [(0, 0), (0, 1), (0, 2), (0, 3), None, (1, 1), None, (1, 3)]
    assert pkey[:8] == [None] * 8 and key[8:] == pkey[8:]
    assert (clock, pclock) == (22, 10)
    assert (last[0], last[1], last[2], last[3]) == (13, 14, 15, 11)
    assert (last[5], last[7], last[8], last[9]) == (20, 17, 21, 19)


@given(seed=st.integers(0, 10_000))
@settings(max_examples=60, deadline=None)
def test_prefill_hit_d2d_without_residents_is_plain_staging(seed):
    rng = np.random.default_rng(seed)
    E, L = 6, 3
    a, b = LRUPool(2 * E + 3), LRUPool(2 * E + 3)
    for l in range(L):
        sel = np.stack([rng.choice(E, 2, replace=False) for _ in range(5)])
        ra = a.stage_layer(l, E, sel, L, hit_d2d=True)
        rb = b.stage_layer(l, E, sel, L)
        for key in ("slot", "flag"):
            assert np.array_equal(ra[key], rb[key])
        assert ra["stream"] == rb["stream"] and ra["expert_misses"] == E
    # the last two staged layers stay resident in their halves under hit-D2D
    ka, kb = a.snapshot()[0], b.snapshot()[0]
    assert all(k is None for k in kb[:2 * E])
    assert sorted(k for k in ka[:2 * E]) == sorted((l, e) for l in (L - 2, L - 1) for e in range(E))
    assert all(ka[(l % 2) * E + e] == (l, e) for l in (L - 2, L - 1) for e in range(E))


def test_prefill_hit_d2d_registers_staged_experts_hand_worked():
    """L = 3 layers of E = 2 experts, k = 1, C = 6: staging [0, 4), slots 4, 5
    beyond it.  Six one-token decode calls fill the pool: (0,0)..(2,1) in
    slots 0..5 with last uses 0..5, clock 6.  A hit-D2D chunk of 2 tokens:
      layer 0, sel [1, 1]: clears [0,2) and [2,4) (4 evictions); copies 0, 1
        into slots 0, 1; unselected copy 0 -> tick 6; expert 1's last pair is
        position 1 -> 6 + 1 + 1 = 8; clock 9.
      layer 1, sel [0, 1]: clears [2,4) and [0,2) (2 evictions: layer 0's
        copies); copies into slots 2, 3; last uses 9 + 0 and 9 + 1; clock 11.
      layer 2, sel [1, 1]: clears [0,2) only (no layer 3); (2,0) and (2,1)
        are resident in slots 4, 5 and read in place; expert 1's last pair is
        position 1 -> 12; expert 0 keeps 4; clock 13.
    Afterwards a decode call of layer 1 hits the staged copy in slot 2, and a
    miss takes the lowest free slot, 0."""
    pool = LRUPool(6)
    for key in range(6):
        pool.resolve_wave(key // 2, np.array([[key % 2]]))
    assert pool.clock == 6
    r0 = pool.stage_layer(0, 2, np.array([[1], [1]]), 3, hit_d2d=True)
    r1 = pool.stage_layer(1, 2, np.array([[0], [1]]), 3, hit_d2d=True)
    r2 = pool.stage_layer(2, 2, np.array([[1], [1]]), 3, hit_d2d=True)
    assert [r["evictions"] for r in (r0, r1, r2)] == [4, 2, 0]
    assert [r["expert_hits"] for r in (r0, r1, r2)] == [0, 0, 2]
    assert [len(r["stream"]) for r in (r0, r1, r2)] == [2, 2, 0]
    assert list(r2["flag"]) == [HIT, HIT] and list(r2["slot"]) == [5, 5]
    key, last, clock = pool.snapshot()
    assert key == [None, None, (1, 0), (1, 1), (2, 0), (2, 1)]
    assert last[2:] == [9, 10, 4, 12] and clock == 13
    d = pool.resolve_wave(1, np.array([[0]]))
    assert list(d["flag"]) == [HIT] and list(d["slot"]) == [2]
    m = pool.resolve_wave(0, np.array([[0]]))
    assert m["stream"] == [(0, 0)] and m["evictions"] == 0


@settings(max_examples=60, deadline=None)
@given(seed=st.integers(0, 10_000), C=st.integers(3, 12), share=st.sampled_from([0.0, 0.3]))
def test_resize_matches_independent_list_lru(seed, C, share):
    """Random traces interleaved with random grows and shrinks: decisions,
    slots and evictions equal the list model's, and after every resize the
    residents are the most recently used keys that fit."""
    rng = np.random.default_rng(seed)
    k = int(rng.integers(1, 3))
    calls = _random_calls(rng, L=3, E=9, k=k, ncalls=30, maxT=3)
    pool, ref = LRUPool(C), ListLRU(C)
    for i, (layer, sel) in enumerate(calls):
        if i % 5 == 4:
            newC = int(rng.integers(max(k, 2), 14))
            recent = list(ref.order)[-newC:]
            r = pool.resize(newC)
            ref.resize(newC)
            assert sorted(pool.slot_of.items()) == sorted(ref.slot.items())
            assert set(pool.slot_of) == set(recent)
            assert all(s < newC for s in pool.slot_of.values())
            assert all(key not in pool.slot_of for key in r["evicted"])
        for t0, t1 in split_waves(sel, pool.C):
            got = pool.resolve_wave(layer, sel[t0:t1], share)
            exp, ev = ref.wave(layer, [int(v) for v in sel[t0:t1].reshape(-1)], share)
            assert list(zip(got["flag"], got["slot"])) == exp
            assert got["evictions"] == ev


def test_resize_is_textbook_lru_with_a_changing_capacity():
    """T = k = 1 calls make the pool textbook LRU; a capacity change keeps the
    most recently used keys (an OrderedDict-based recency list, no slots)."""
    from collections import OrderedDict

    rng = np.random.default_rng(7)
    pool = LRUPool(4)
    lru, cap = OrderedDict(), 4
    for i in range(400):
        if i % 37 == 36:
            cap = int(rng.integers(1, 8))
            pool.resize(cap)
            while len(lru) > cap:
                lru.popitem(last=False)
        e = int(rng.zipf(1.4) % 10)
        r = pool.resolve_wave(0, np.array([[e]]))
        hit = e in lru
        assert (r["flag"][0] == HIT) == hit, i
        if hit:
            lru.move_to_end(e)
        else:
            if len(lru) >= cap:
                lru.popitem(last=False)
            lru[e] = True
        assert set(k[1] for k in pool.slot_of) == set(lru), i


def test_resize_hand_worked():
    """Five residents with last uses 10..14 in slots 0..4 of 6 slots:
    shrinking to 3 keeps the keys used at 12, 13, 14; the one in slot 2 stays,
    the ones in slots 3 and 4 move to slots 0 and 1; growing to 8 moves nothing."""
    pool = LRUPool(6)
    for s, (e, last) in enumerate([(5, 10), (6, 11), (7, 12), (8, 13), (9, 14)]):
        pool.key_of[s], pool.last_use[s] = (0, e), last
        pool.slot_of[(0, e)] = s
    r = pool.resize(3)
    assert r["evicted"] == [(0, 5), (0, 6)]
    assert r["moves"] == [(3, 0), (4, 1)]
    assert pool.key_of == [(0, 8), (0, 9), (0, 7)] and pool.last_use == [13, 14, 12]
    r = pool.resize(8)
    assert r == dict(evicted=[], moves=[]) and pool.key_of[3:] == [None] * 5


def test_layer_stack_share_per_format():
    """A share given per weight format applies to the layers of that format
    only: with 0 for MXFP4 and 1 for FP8, MXFP4 layers stream every miss and
    FP8 layers compute every miss on the host (and leave the pool alone)."""
    import moe_synth as ms
    from oracle.layer import OracleLayerStack

    MX, F8 = ms.FMT_MXFP4, ms.FMT_FP8_B128
    w = ms.Workload(135, "small-135", 2, 256, 128, 8, 2, (MX, F8), 8, (4,), 4, "decode", None, None,
                    False, False, None)
    o = OracleLayerStack(w, share={MX: 0.0, F8: 1.0})
    for step in range(2):
        for l in range(2):
            r = o.forward(l, ms.activations(w, l, step, 3), None, outputs=False)
            stream = [m for wv in r["waves"] for m in wv["stream"]]
            cpu = [e for wv in r["waves"] for e in wv["cpu"]]
            if l == 0:
                assert cpu == [] and (step > 0 or len(stream) > 0)
            else:
                assert stream == [] and len(cpu) == len(set(r["sel"].reshape(-1).tolist()))
    key, _, _ = o.pool.snapshot()
    assert all(k is None or k[0] == 0 for k in key)
    assert o.share_of(0) == 0.0 and o.share_of(1) == 1.0
    assert OracleLayerStack(w, share=0.25).share_of(1) == 0.25
