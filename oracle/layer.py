"""One offloaded MoE layer call, and a run over a workload's steps and layers.

TEST INFRASTRUCTURE (oracle).  A decode call: router -> waves -> per wave the
LRU resolve -> expert FFN per pair -> combine.  A prefill call stages the
whole layer instead of resolving against the LRU pool (devpik article, "Long
Prompts Are the Bottleneck").  The output of a pair depends only on its token,
its expert's weights and its routing weight, so the oracle evaluates the FFN
per distinct expert over that expert's rows, with no permutation, no slots and
no blocking; the cache decisions and the numbers are computed independently.

Every input comes from `moe_synth`; nothing here reads anything produced by
the GPU library.
"""

from __future__ import annotations

from typing import Callable, Dict, Optional

import numpy as np

import moe_synth as ms

from . import ffn, formats, router
from .lru import HIT, MISS_CPU, MISS_STREAM, LRUPool, split_waves


class DequantCache:
    """Memoises dequantised experts (fp64 matrices) by blob identity."""

    def __init__(self, max_items: int = 64):
        self.max_items = max_items
        self._d: Dict = {}

    def get(self, key, fmt, blob_fn, hidden, inter):
        if key in self._d:
            v = self._d.pop(key)
            self._d[key] = v
            return v
        v = formats.dequant_expert(fmt, blob_fn(), hidden, inter)
        self._d[key] = v
        while len(self._d) > self.max_items:
            self._d.pop(next(iter(self._d)))
        return v


class OracleLayerStack:
    """Oracle state for one workload: the global pool plus per-layer weights."""

    def __init__(self, w: ms.Workload, pool_slots: Optional[int] = None, share=0.0,
                 act_mode: int = ffn.ACT_BF16, blob_fn: Optional[Callable] = None,
                 dequant_items: int = 64, threads: int = 1):
        self.w = w
        self.C = w.pool_slots if pool_slots is None else pool_slots
        self.pool = LRUPool(self.C)
        # the hybrid share: one number for every layer, or a mapping from weight
        # format to the share of that format's layers (the split rule is the
        # same; only the share it is given differs by format)
        self.share = share
        self.act_mode = act_mode
        self._router = {}
        self._blob_fn = blob_fn or (lambda l, e: ms.expert_blob(w, l, e))
        self.deq = DequantCache(dequant_items)
        # threads > 1: the distinct experts of a call are dequantised
        # concurrently, `threads` at a time (independent work; the arithmetic
        # and the order of every sum are unchanged)
        self.threads = max(1, int(threads))
        self.stats = dict(pair_hits=0, pair_misses=0, expert_hits=0, expert_misses=0,
                          cpu_misses=0, evictions=0, bytes_h2d=0, calls=0)

    def share_of(self, layer: int) -> float:
        if isinstance(self.share, dict):
            return float(self.share.get(self.w.fmt(layer), 0.0))
        return float(self.share)

    def router_w(self, layer):
        if layer not in self._router:
            self._router[layer] = ms.router_weight(self.w, layer)
        return self._router[layer]

    def expert_mats(self, layer, e):
        w = self.w
        f = w.fmt(layer)
        key = ("x", f, w.blob_id(layer, e))
        return self.deq.get(key, f, lambda: self._blob_fn(layer, e), w.hidden, w.inter)

    def shared_mats(self, layer):
        w = self.w
        f = w.fmt(layer)
        return self.deq.get(("s", layer), f, lambda: ms.shared_blob(w, layer), w.hidden, w.inter)

    def forward(self, layer: int, x_bits: np.ndarray, bias: Optional[np.ndarray],
                prefill: bool = False, outputs: bool = True, out_tokens=None, hit_d2d: bool = False):
        """Run one layer call; x_bits uint16 [T,H] bf16 bit patterns.

        out_tokens: compute the output only for these token indices (each
        token's output depends only on its own row and routing)."""
        w = self.w
        T, k, E = x_bits.shape[0], w.top_k, w.num_experts
        x = formats.bf16_from_bits(x_bits)
        z, sel, wts = router.route(x, self.router_w(layer), bias, k)
        gap = router.min_topk_gap(z, k)
        eb = ms.expert_bytes(w.fmt(layer), w.hidden, w.inter)

        flag = np.empty(T * k, np.uint8)
        slot = np.empty(T * k, np.int32)
        waves = []
        if prefill:
            r = self.pool.stage_layer(layer, E, sel, w.num_layers, hit_d2d=hit_d2d)
            flag[:], slot[:] = r["flag"], r["slot"]
            waves.append(dict(t0=0, t1=T, **r))
            st = dict(pair_hits=r["pair_hits"], expert_hits=r["expert_hits"], expert_misses=r["expert_misses"],
                      cpu_misses=0, evictions=r["evictions"], bytes_h2d=len(r["stream"]) * eb)
        else:
            st = dict(pair_hits=0, expert_hits=0, expert_misses=0, cpu_misses=0, evictions=0, bytes_h2d=0)
            for (t0, t1) in split_waves(sel, self.pool.C):
                r = self.pool.resolve_wave(layer, sel[t0:t1], self.share_of(layer))
                flag[t0 * k:t1 * k] = r["flag"]
                slot[t0 * k:t1 * k] = r["slot"]
                waves.append(dict(t0=t0, t1=t1, **r))
                for c in ("pair_hits", "expert_hits", "expert_misses", "cpu_misses", "evictions"):
                    st[c] += r[c]
                cpu_rows = int((r["flag"] == MISS_CPU).sum())
                st["bytes_h2d"] += len(r["stream"]) * eb + cpu_rows * w.hidden * 2
        st["pair_misses"] = T * k - st["pair_hits"]
        for c, v in st.items():
            self.stats[c] += v
        self.stats["calls"] += 1

        res = dict(sel=sel, w=wts, flag=flag, slot=slot, waves=waves, gap=gap, stats=st, z=z)
        if outputs:
            if out_tokens is None:
                res["out"] = self.outputs(layer, x, sel, wts)
            else:
                tk = np.asarray(out_tokens)
                res["out"] = self.outputs(layer, x[tk], sel[tk], wts[tk])
                res["out_tokens"] = tk
        return res

    def _mats_of(self, layer, experts):
        """Dequantised matrices of several experts of one layer."""
        if self.threads == 1 or len(experts) == 1:
            return [self.expert_mats(layer, int(e)) for e in experts]
        from concurrent.futures import ThreadPoolExecutor

        with ThreadPoolExecutor(self.threads) as ex:
            return list(ex.map(lambda e: self.expert_mats_uncached(layer, int(e)), experts))

    def expert_mats_uncached(self, layer, e):
        w = self.w
        return formats.dequant_expert(w.fmt(layer), self._blob_fn(layer, e), w.hidden, w.inter)

    def outputs(self, layer, x, sel, wts):
        w = self.w
        T, k = sel.shape
        p = np.zeros((T, k, w.hidden), np.float64)
        experts = np.unique(sel)
        for c0 in range(0, len(experts), self.threads):
            chunk = experts[c0:c0 + self.threads]
            for e, (wg, wu, wd) in zip(chunk, self._mats_of(layer, chunk)):
                rows = np.argwhere(sel == e)  # (t, j) pairs
                y = ffn.expert_forward(x[rows[:, 0]], wg, wu, wd, self.act_mode)
                p[rows[:, 0], rows[:, 1]] = ffn.weighted_rows(y, wts[rows[:, 0], rows[:, 1]])
        shared = None
        if w.shared_expert:
            sg, su, sd = self.shared_mats(layer)
            shared = ffn.expert_forward(x, sg, su, sd, self.act_mode)
        return ffn.combine(p, shared)
