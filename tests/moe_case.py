"""Test helpers: build a GPU pool and an oracle stack for the same workload,
run calls on both, and compare them.  Used by the GPU parity tests."""

from __future__ import annotations

import numpy as np

import moe_synth as ms
import lru_expert_cache_amd as ft
from oracle import formats as OF
from oracle.layer import OracleLayerStack


class GpuLayerStack:
    """A GPU pool for a workload, created from the seeded generators."""

    def __init__(self, w: ms.Workload, pool_slots=None, share=0.0, store=None, device=0):
        import torch

        self.torch = torch
        self.w = w
        self.C = w.pool_slots if pool_slots is None else pool_slots
        self.store = store or ms.BlobStore(w)
        L, E = w.num_layers, w.num_experts
        blobs = [self.store.expert(l, e) for l in range(L) for e in range(E)]
        router = np.stack([ms.router_weight(w, l) for l in range(L)])
        shared = [self.store.shared(l) for l in range(L)] if w.shared_expert else None
        per_fmt = isinstance(share, dict)
        cfg = ft.make_config(L, w.hidden, w.inter, E, w.top_k, w.layer_fmt, pool_slots=self.C, shared=w.shared_expert,
                             hybrid_cpu_share=0.0 if per_fmt else share, device=device)
        self.pool, self.init_rc = ft.ft_moe_init_pool(cfg, blobs, router, shared)
        if per_fmt and self.pool:
            for f, v in share.items():
                ft.ft_moe_set_hybrid_share_format(self.pool, f, v)
        self.dev = torch.device("cuda", device)

    def close(self):
        if self.pool:
            ft.ft_moe_destroy_pool(self.pool)
            self.pool = None

    def bias(self, layer, step):
        b = ms.popularity_bias(self.w, layer, self.w.phase(step))
        return None if b is None else self.torch.from_numpy(b).to(self.dev)

    def forward(self, layer, x_bits, bias_t, prefill=False, act=0, hit_d2d=False):
        torch = self.torch
        T, k = x_bits.shape[0], self.w.top_k
        x = torch.from_numpy(x_bits.view(np.int16)).to(self.dev)
        out = torch.empty_like(x)
        tr = dict(sel=torch.empty(T * k, dtype=torch.int32, device=self.dev),
                  w=torch.empty(T * k, dtype=torch.float32, device=self.dev),
                  slot=torch.empty(T * k, dtype=torch.int32, device=self.dev),
                  flag=torch.empty(T * k, dtype=torch.uint8, device=self.dev),
                  row=torch.empty(T * k, dtype=torch.int32, device=self.dev))
        flags = (ft.FT_FWD_PREFILL_STAGED if prefill else ft.FT_FWD_DECODE) | act
        if hit_d2d:
            flags |= ft.FT_FWD_PREFILL_HIT_D2D
        ft.ft_moe_layer_forward(self.pool, layer, T, x, bias_t, out, flags, None, tr)
        torch.cuda.synchronize()
        res = {n: t.cpu().numpy() for n, t in tr.items()}
        res["sel"] = res["sel"].reshape(T, k)
        res["w"] = res["w"].reshape(T, k)
        res["out_bits"] = out.cpu().numpy().view(np.uint16)
        res["stream"], res["cpu"] = ft.ft_moe_last_misses(self.pool)
        return res


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def compare_call(g, o, k, check_out=True, tol=2e-3):
    """Exact decisions, rel-L2 on the output; returns the output rel-L2."""
    assert np.array_equal(g["sel"], o["sel"]), "selected experts differ"
    assert np.abs(g["w"] - o["w"]).max() <= 1e-6, "routing weights differ"
    assert np.array_equal(g["flag"], o["flag"]), "hit/miss flags differ"
    assert np.array_equal(g["slot"], o["slot"]), "slot assignment differs"
    ostream = [tuple(m) for wv in o["waves"] for m in wv["stream"]]
    ocpu = [e for wv in o["waves"] for e in wv["cpu"]]
    assert [tuple(m) for m in g["stream"]] == ostream, "streamed-miss list differs"
    assert list(g["cpu"]) == ocpu, "host-miss list differs"
    check_rows(g, o, k)
    if check_out:
        go = OF.bf16_from_bits(g["out_bits"])
        if "out_tokens" in o:
            go = go[o["out_tokens"]]
        assert np.isfinite(go).all() and np.linalg.norm(o["out"]) > 0
        r = rel_l2(go, o["out"])
        assert r <= tol, f"output rel-L2 {r}"
        return r
    return None


def check_rows(g, o, k):
    """Rows group each wave's pairs by expert in first-appearance order, in pair order."""
    row = g["row"]
    for wv in o["waves"]:
        t0, t1 = wv["t0"], wv["t1"]
        sel = o["sel"][t0:t1].reshape(-1)
        r = row[t0 * k:t1 * k]
        expect = np.empty_like(r)
        base = 0
        for e in wv["D"]:
            idx = np.nonzero(sel == e)[0]
            expect[idx] = base + np.arange(idx.size)
            base += idx.size
        assert np.array_equal(r, expect), "permuted row order differs"


def compare_table(gstack: GpuLayerStack, ostack: OracleLayerStack):
    key, last, clock = ft.ft_moe_pool_table(gstack.pool, gstack.C)
    okey, olast, oclock = ostack.pool.snapshot()
    E = gstack.w.num_experts
    exp_key = np.array([-1 if kk is None else kk[0] * E + kk[1] for kk in okey], np.int64)
    assert np.array_equal(key.astype(np.int64), exp_key), "slot table keys differ"
    used = exp_key >= 0
    exp_last = np.array([0 if v is None else v for v in olast], np.uint64)
    assert np.array_equal(last[used], exp_last[used]), "slot last-use clocks differ"
    assert clock == oclock
