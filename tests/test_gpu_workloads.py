"""GPU parity at the full sizes of the layer shapes, in the launch configuration
the benchmark uses (whole layer stacks, the pool sizes of each workload).

Decisions (experts, weights, hit/miss flags, slots, miss lists, grouped row
order) are compared exactly on every call; outputs (rel-L2 <= 2e-3, bf16) on
sampled calls the oracle computes one by one.
"""

import numpy as np
import pytest

import moe_synth as ms
from oracle.layer import OracleLayerStack

pytestmark = pytest.mark.gpu

_STORES = {}


def _decode_run(w, T, steps, sample, share=0.0, store=None, layers_out=None):
    from tests.moe_case import GpuLayerStack, compare_call, compare_table

    g = GpuLayerStack(w, share=share, store=store)
    o = OracleLayerStack(w, pool_slots=g.C, share=share, blob_fn=lambda l, e: g.store.expert(l, e), dequant_items=16)
    rels = []
    try:
        for s in range(steps):
            for l in range(w.num_layers):
                x = ms.activations(w, l, s, T)
                b = ms.popularity_bias(w, l, w.phase(s))
                want = (s, l) in sample
                gr = g.forward(l, x, g.bias(l, s))
                orr = o.forward(l, x, b, outputs=want)
                r = compare_call(gr, orr, w.top_k, check_out=want)
                if r is not None:
                    rels.append(r)
            print(f"{w.name} T={T} step {s} ok", flush=True)
        compare_table(g, o)
        import lru_expert_cache_amd as ft

        st = ft.ft_moe_pool_stats(g.pool)
        for key in ("pair_hits", "pair_misses", "expert_hits", "expert_misses", "cpu_misses", "evictions",
                    "bytes_h2d", "calls"):
            assert st[key] == o.stats[key], (key, st[key], o.stats[key])
        assert st["min_topk_gap"] > 1e-9
        return rels, st
    finally:
        g.close()


@pytest.fixture(scope="module")
def qwen_store():
    return ms.BlobStore(ms.workload("qwen-a3b-decode"))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T", [16, 1, 4])
def test_qwen_a3b_decode(qwen_store, T):
    w = ms.workload("qwen-a3b-decode")
    steps = 3
    sample = {(0, 0), (1, 23), (steps - 1, 47), (steps - 1, 5)}
    rels, st = _decode_run(w, T, steps, sample, store=qwen_store)
    print("rel-L2", rels, "hits", st["pair_hits"], "misses", st["pair_misses"], "evictions", st["evictions"])
    assert max(rels) <= 2e-3


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("T,steps", [(1, 2), (8, 2), (64, 1)])
def test_deepseek_decode_nvfp4_shared(T, steps):
    w = ms.workload("deepseek-v4-flash-decode")
    from tests.moe_case import GpuLayerStack, compare_call, compare_table
    import lru_expert_cache_amd as ft

    if w.name not in _STORES:
        _STORES[w.name] = ms.BlobStore(w)
    store = _STORES[w.name]
    g = GpuLayerStack(w, store=store)
    o = OracleLayerStack(w, pool_slots=g.C, blob_fn=lambda l, e: store.expert(l, e), dequant_items=24)
    try:
        rels = []
        for s in range(steps):
            for l in range(w.num_layers):
                x = ms.activations(w, l, s, T)
                b = ms.popularity_bias(w, l, 0)
                want = (s, l) in {(0, 0), (steps - 1, 60)}
                gr = g.forward(l, x, g.bias(l, s))
                orr = o.forward(l, x, b, outputs=want, out_tokens=[0, T - 1] if want else None)
                r = compare_call(gr, orr, w.top_k, check_out=want)
                if r is not None:
                    rels.append(r)
            print(f"deepseek T={T} step {s} ok", flush=True)
        compare_table(g, o)
        st = ft.ft_moe_pool_stats(g.pool)
        for key in ("pair_hits", "pair_misses", "expert_misses", "evictions", "bytes_h2d", "calls"):
            assert st[key] == o.stats[key], key
        print("rel-L2", rels, st)
    finally:
        g.close()



@pytest.mark.timeout(1200)
def test_glm_mixed_formats_hybrid():
    w = ms.workload("glm-5.2-mixed-decode")
    from tests.moe_case import GpuLayerStack, compare_call, compare_table
    import lru_expert_cache_amd as ft

    store = ms.BlobStore(w)
    share = 0.02
    g = GpuLayerStack(w, store=store, share=share)
    o = OracleLayerStack(w, pool_slots=g.C, share=share, blob_fn=lambda l, e: store.expert(l, e), dequant_items=24)
    T = 32
    try:
        rels = []
        for s in (0, 33):  # two popularity phases
            for l in range(w.num_layers):
                x = ms.activations(w, l, s, T)
                b = ms.popularity_bias(w, l, w.phase(s))
                want = (s, l) in {(0, 0), (0, 1), (33, 90), (33, 91)}
                gr = g.forward(l, x, g.bias(l, s))
                orr = o.forward(l, x, b, outputs=want, out_tokens=[3, 17] if want else None)
                r = compare_call(gr, orr, w.top_k, check_out=want)
                if r is not None:
                    rels.append(r)
            print(f"glm step {s} ok", flush=True)
        compare_table(g, o)
        st = ft.ft_moe_pool_stats(g.pool)
        for key in ("pair_hits", "pair_misses", "expert_misses", "cpu_misses", "evictions", "bytes_h2d", "calls"):
            assert st[key] == o.stats[key], key
        assert st["cpu_misses"] > 0
        print("rel-L2", rels, st)
    finally:
        g.close()


@pytest.mark.timeout(1200)
def test_qwen_a3b_prefill_4096(qwen_store):
    w = ms.workload("qwen-a3b-prefill-4096")
    from tests.moe_case import GpuLayerStack, compare_call, compare_table
    import lru_expert_cache_amd as ft

    g = GpuLayerStack(w, store=qwen_store)
    o = OracleLayerStack(w, pool_slots=g.C, blob_fn=lambda l, e: qwen_store.expert(l, e), dequant_items=130)
    T = 4096
    rng = np.random.default_rng(0)
    try:
        rels = []
        for l in range(w.num_layers):
            x = ms.activations(w, l, 0, T)
            b = ms.popularity_bias(w, l, 0)
            want = l in (0, 1, 24, 47)
            toks = np.sort(rng.choice(T, 24, replace=False)) if want else None
            gr = g.forward(l, x, g.bias(l, 0), prefill=True)
            orr = o.forward(l, x, b, prefill=True, outputs=want, out_tokens=toks)
            r = compare_call(gr, orr, w.top_k, check_out=want)
            if r is not None:
                rels.append(r)
        compare_table(g, o)
        st = ft.ft_moe_pool_stats(g.pool)
        assert st["bytes_h2d"] == o.stats["bytes_h2d"] == w.num_layers * w.num_experts * ms.expert_bytes(
            ms.FMT_MXFP4, w.hidden, w.inter)
        assert st["pair_hits"] == 0 and st["pair_misses"] == w.num_layers * T * w.top_k
        print("rel-L2", rels)
    finally:
        g.close()


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("act", ["mxfp8", "mxfp4"])
def test_qwen_a3b_prefill_4096_mx_activations(qwen_store, act):
    """Full 4096-token chunk through all 48 staged layers with x and h
    MX-quantised: decisions exact on every layer, outputs on sampled tokens."""
    w = ms.workload("qwen-a3b-prefill-4096")
    from tests.moe_case import GpuLayerStack, compare_call
    from oracle import ffn as OFFN
    import lru_expert_cache_amd as ft

    mode = OFFN.ACT_MXFP4 if act == "mxfp4" else OFFN.ACT_MXFP8
    flag = ft.FT_ACT_MXFP4 if act == "mxfp4" else ft.FT_ACT_MXFP8
    g = GpuLayerStack(w, store=qwen_store)
    o = OracleLayerStack(w, pool_slots=g.C, blob_fn=lambda l, e: qwen_store.expert(l, e), dequant_items=130,
                         act_mode=mode)
    T = 4096
    rng = np.random.default_rng(1)
    try:
        rels = []
        for l in range(w.num_layers):
            x = ms.activations(w, l, 0, T)
            b = ms.popularity_bias(w, l, 0)
            want = l in (0, 47)
            toks = np.sort(rng.choice(T, 16, replace=False)) if want else None
            gr = g.forward(l, x, g.bias(l, 0), prefill=True, act=flag)
            orr = o.forward(l, x, b, prefill=True, outputs=want, out_tokens=toks)
            r = compare_call(gr, orr, w.top_k, check_out=want, tol=2e-3 if act == "mxfp8" else 6e-3)
            if r is not None:
                rels.append(r)
        print(act, "rel-L2", rels)
        assert len(rels) == 2
    finally:
        g.close()
