"""The global LRU pool of GPU expert slots, simulated with dicts and lists.

TEST INFRASTRUCTURE (oracle).  What the pages fix: the GPU keeps a
least-recently-used cache of expert slots; an expert already cached runs in
place and a miss is streamed over PCIe (devpik article, "Why a Huge MoE Model
Fits on One Consumer GPU"); one LRU pool is shared by all layers (same
section); the hybrid strategy splits each step's misses between host compute
and streaming (same section; byteiota article, "The Bandwidth-Adaptive
Runtime").  Finer points are readings of the pages:

* Keys are (layer, expert).  A call's tokens are walked in order; a *wave* is
  the longest run of consecutive tokens whose union of selected experts has
  at most C members.  Each wave is resolved as a set: an expert needed later
  in the same wave is never evicted by an earlier miss.
* Pairs P = (token, rank) in token-major order; D = distinct experts in order
  of first appearance; hits Hs = members of D resident at the wave's start;
  misses M = D minus Hs, in D order.
* Hybrid: m_cpu = floor(|M| * share + 1/2) (IEEE double); the last m_cpu
  misses go to host compute and are not inserted into the pool; the rest
  stream.
* Victims: free slots by ascending index, then resident slots not holding a
  hit of this wave, by ascending last use.  The i-th streamed miss takes the
  i-th victim.
* Clock: one tick per pair of the wave; a touched slot's last use is the
  clock at the wave start plus the position of its expert's last pair.
* Prefill staging: the call streams all E experts of the layer into slots
  (layer mod 2) * E + e; every pair is a streamed miss; since the call also
  starts the copy of layer l+1 into the other half, residents of both halves
  are evicted (the second only if l+1 < L); the LRU order of other slots is
  untouched and the clock does not move (devpik article, "Long Prompts Are
  the Bottleneck").  With the hit-D2D option, resident experts are read in
  place and the copied ones become residents of their staging slots (see
  stage_layer).

Pins (tests/test_oracle_lru.py): an independent brute-force list LRU,
hand-worked traces, the compulsory-miss, inclusion and cyclic-thrash
properties of LRU, hits + misses = T*k; for resize, the list LRU's own resize
and a textbook recency-list LRU whose capacity changes (T = k = 1).
"""

from __future__ import annotations

import math
from typing import List, Sequence

import numpy as np

HIT, MISS_STREAM, MISS_CPU = 0, 1, 2


def split_waves(sel: np.ndarray, capacity: int):
    """Token ranges [(t0, t1)] of the waves of one call."""
    T = sel.shape[0]
    waves = []
    t0 = 0
    cur = set()
    for t in range(T):
        new = cur | set(int(e) for e in sel[t])
        if len(new) > capacity:
            waves.append((t0, t))
            t0 = t
            cur = set(int(e) for e in sel[t])
        else:
            cur = new
    if T > 0:
        waves.append((t0, T))
    return waves


def hybrid_cpu_count(m: int, share: float) -> int:
    return int(math.floor(float(m) * float(share) + 0.5))


class LRUPool:
    def __init__(self, capacity: int):
        self.C = int(capacity)
        self.slot_of = {}  # (layer, expert) -> slot
        self.key_of: List = [None] * self.C
        self.last_use: List = [None] * self.C
        self.clock = 0

    def resident(self, layer: int, e: int) -> bool:
        return (layer, e) in self.slot_of

    def resolve_wave(self, layer: int, sel_wave: np.ndarray, share: float = 0.0):
        """Resolve one wave.  sel_wave: [Tw, k] expert ids.

        Returns dict with per-pair flag/slot, the streamed-miss list
        [(expert, slot)] in D order, the CPU-miss list, D, and counters.
        """
        pairs = [int(e) for e in np.asarray(sel_wave).reshape(-1)]
        P = len(pairs)
        D = []
        last_pos = {}
        for p, e in enumerate(pairs):
            if e not in last_pos:
                D.append(e)
            last_pos[e] = p
        assert len(D) <= self.C
        hits = [e for e in D if self.resident(layer, e)]
        misses = [e for e in D if not self.resident(layer, e)]
        m_cpu = hybrid_cpu_count(len(misses), share)
        m_str = len(misses) - m_cpu
        stream = misses[:m_str]
        cpu = misses[m_str:]

        protected = {self.slot_of[(layer, e)] for e in hits}
        free = [s for s in range(self.C) if self.key_of[s] is None]
        used = [s for s in range(self.C) if self.key_of[s] is not None and s not in protected]
        used.sort(key=lambda s: self.last_use[s])
        victims = free + used
        evictions = 0
        stream_list = []
        for i, e in enumerate(stream):
            s = victims[i]
            old = self.key_of[s]
            if old is not None:
                del self.slot_of[old]
                evictions += 1
            self.key_of[s] = (layer, e)
            self.slot_of[(layer, e)] = s
            stream_list.append((e, s))
        for e in hits + stream:
            self.last_use[self.slot_of[(layer, e)]] = self.clock + last_pos[e]
        self.clock += P

        hit_set, cpu_set = set(hits), set(cpu)
        flag = np.empty(P, np.uint8)
        slot = np.empty(P, np.int32)
        for p, e in enumerate(pairs):
            if e in hit_set:
                flag[p] = HIT
                slot[p] = self.slot_of[(layer, e)]
            elif e in cpu_set:
                flag[p] = MISS_CPU
                slot[p] = -1
            else:
                flag[p] = MISS_STREAM
                slot[p] = self.slot_of[(layer, e)]
        return dict(flag=flag, slot=slot, stream=stream_list, cpu=list(cpu), D=D,
                    pair_hits=int((flag == HIT).sum()), expert_hits=len(hits),
                    expert_misses=len(misses), cpu_misses=len(cpu), evictions=evictions)

    def stage_layer(self, layer: int, num_experts: int, sel: np.ndarray, num_layers: int,
                    hit_d2d: bool = False):
        """Prefill staging of one layer into half (layer mod 2) of slots [0, 2E).

        The call for layer l also starts the copy of layer l+1 into the other
        half (layer N+1 copies while layer N computes), so both halves lose
        their LRU residents here (the second one only if l+1 < L).

        hit_d2d: experts of the layer already resident in the pool are not
        copied again; only the others cross PCIe (devpik article, "Long
        Prompts Are the Bottleneck": the prefill option that skips experts
        already in the GPU cache).  Readings: a resident expert is used from
        its pool slot (its pairs are HIT with that slot), and residency is
        taken after the staging halves are cleared (so it lies outside them).
        The copied experts become LRU residents of their staging slots (until
        a later call clears that half), and the call updates the LRU order
        like one decode wave over its pairs: the copied experts that no token
        selects take the first clock ticks, in expert order; then every expert
        the tokens select -- read in place or copied -- takes the clock at its
        last pair; the clock advances by both counts.  Without hit_d2d the
        LRU order, the clock and the staging slots' residency are untouched.
        """
        E = num_experts
        assert self.C >= 2 * E
        base = (layer % 2) * E
        halves = [layer % 2] + ([(layer + 1) % 2] if layer + 1 < num_layers else [])
        evictions = 0
        for h in halves:
            for s in range(h * E, h * E + E):
                old = self.key_of[s]
                if old is not None:
                    del self.slot_of[old]
                    self.key_of[s] = None
                    self.last_use[s] = None
                    evictions += 1
        resident = {}
        if hit_d2d:
            for e in range(E):
                if (layer, e) in self.slot_of:
                    resident[e] = self.slot_of[(layer, e)]
        pairs = np.asarray(sel).reshape(-1)
        flag = np.array([HIT if int(e) in resident else MISS_STREAM for e in pairs], np.uint8)
        slot = np.array([resident.get(int(e), base + int(e)) for e in pairs], np.int32)
        D = []
        last_pos = {}
        for p, e in enumerate(pairs):
            if int(e) not in last_pos:
                D.append(int(e))
            last_pos[int(e)] = p
        if hit_d2d:
            copied = [e for e in range(E) if e not in resident]
            for e in copied:
                self.key_of[base + e] = (layer, e)
                self.slot_of[(layer, e)] = base + e
            unselected = [e for e in copied if e not in last_pos]
            for i, e in enumerate(unselected):
                self.last_use[base + e] = self.clock + i
            for e in D:
                self.last_use[self.slot_of[(layer, e)]] = self.clock + len(unselected) + last_pos[e]
            self.clock += len(unselected) + len(pairs)
        return dict(flag=flag, slot=slot, stream=[(e, base + e) for e in range(E) if e not in resident], cpu=[],
                    D=D, pair_hits=int((flag == HIT).sum()), expert_hits=len(resident),
                    expert_misses=E - len(resident), cpu_misses=0, evictions=evictions)

    def resize(self, new_capacity: int):
        """Elastic resize of the pool at runtime (the pages: VRAM is
        re-allocated between the expert cache and other memory while the
        engine runs -- dev.to article "FreeToken uses bandwidth-adaptive CPU-GPU
        co-execution on your desktop", section "Memory that moves while the
        engine runs").  Readings: the new_capacity most recently used residents
        survive (a shrink evicts the LRU tail); a survivor keeps its slot when
        that slot still exists, the others -- in ascending old slot -- take the
        lowest free slots below new_capacity; last-use values and the clock are
        unchanged.  Returns the evicted keys and the (old slot, new slot) moves.
        """
        new_C = int(new_capacity)
        assert new_C >= 1
        res = [s for s in range(self.C) if self.key_of[s] is not None]
        res.sort(key=lambda s: self.last_use[s])
        n_ev = max(0, len(res) - new_C)
        evicted, survivors = res[:n_ev], res[n_ev:]
        keep = sorted(s for s in survivors if s < new_C)
        move = sorted(s for s in survivors if s >= new_C)
        kept = set(keep)
        free_low = [s for s in range(new_C) if s not in kept]
        key_of, last_use = [None] * new_C, [None] * new_C
        moves = []
        for s in keep:
            key_of[s], last_use[s] = self.key_of[s], self.last_use[s]
        for s, t in zip(move, free_low):
            key_of[t], last_use[t] = self.key_of[s], self.last_use[s]
            moves.append((s, t))
        evicted_keys = [self.key_of[s] for s in evicted]
        self.C, self.key_of, self.last_use = new_C, key_of, last_use
        self.slot_of = {key: s for s, key in enumerate(key_of) if key is not None}
        return dict(evicted=evicted_keys, moves=moves)

    def snapshot(self):
        """(key_of, last_use) copies, for comparisons with the device table."""
        return list(self.key_of), list(self.last_use), self.clock
