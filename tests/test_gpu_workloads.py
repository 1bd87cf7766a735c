"""GPU parity at the full sizes of the layer shapes, in the launch configuration
the benchmark uses (whole layer stacks, the pool sizes of each workload).

Decisions (experts, weights, hit/miss flags, slots, miss lists, grouped row
order) are compared exactly on every call; outputs (rel-L2 <= 2e-3, bf16) on
every row of sampled calls the oracle computes one by one (the prefill chunk:
on sampled rows).
"""

import os

import numpy as np
import pytest

import moe_synth as ms
from oracle.layer import OracleLayerStack

pytestmark = pytest.mark.gpu

_STORES = {}
# the oracle dequantises the distinct experts of a sampled call this many at a time
THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


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
        # copy time: the streamed bytes over it is a plausible host-to-device rate
        if st["bytes_h2d"] > 0:
            rate = st["bytes_h2d"] / (st["copy_ms"] * 1e-3)
            print(f"copy {st['copy_ms']:.1f} ms, {rate / 1e9:.1f} GB/s")
            assert 1e9 < rate < 200e9, rate
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
def test_qwen_a3b_decode_all_256_steps(qwen_store):
    """The whole Qwen-A3B-shaped decode run at batch 16: 256 steps x 48 layers,
    every call's decisions exact (experts, weights, flags, slots, miss lists,
    rows) and the table and counters after it; outputs on steps {0, 127, 255}
    x layers {0, 23, 47}."""
    w = ms.workload("qwen-a3b-decode")
    sample = {(s, l) for s in (0, 127, 255) for l in (0, 23, 47)}
    rels, st = _decode_run(w, 16, 256, sample, store=qwen_store)
    print("rel-L2", rels, "hits", st["pair_hits"], "misses", st["pair_misses"], "evictions", st["evictions"])
    assert len(rels) == len(sample) and max(rels) <= 2e-3


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("T,steps", [(1, 128), (8, 2), (32, 1), (64, 1)])
def test_deepseek_decode_nvfp4_shared(T, steps):
    w = ms.workload("deepseek-v4-flash-decode")
    from tests.moe_case import GpuLayerStack, compare_call, compare_table
    import lru_expert_cache_amd as ft

    if w.name not in _STORES:
        _STORES[w.name] = ms.BlobStore(w)
    store = _STORES[w.name]
    g = GpuLayerStack(w, store=store)
    o = OracleLayerStack(w, pool_slots=g.C, blob_fn=lambda l, e: store.expert(l, e), dequant_items=24,
                         threads=THREADS)
    try:
        rels = []
        for s in range(steps):
            for l in range(w.num_layers):
                x = ms.activations(w, l, s, T)
                b = ms.popularity_bias(w, l, 0)
                want = (s, l) in {(0, 0), (steps - 1, 60)}
                gr = g.forward(l, x, g.bias(l, s))
                orr = o.forward(l, x, b, outputs=want)
                r = compare_call(gr, orr, w.top_k, check_out=want)
                if r is not None:
                    rels.append(r)
            print(f"deepseek T={T} step {s} ok", flush=True)
        compare_table(g, o)
        st = ft.ft_moe_pool_stats(g.pool)
        for key in ("pair_hits", "pair_misses", "expert_misses", "evictions", "bytes_h2d", "calls"):
            assert st[key] == o.stats[key], key
        assert len(rels) == 2
        print("rel-L2", rels, st)
    finally:
        g.close()


@pytest.mark.timeout(1200)
def test_glm_mixed_formats_hybrid():
    """The GLM-shaped stack at the hybrid share the library measures on this
    machine (ft_moe_measure_mode's balanced share: streamed and host-computed
    misses finish together)."""
    w = ms.workload("glm-5.2-mixed-decode")
    from tests.moe_case import GpuLayerStack, compare_call, compare_table
    import lru_expert_cache_amd as ft

    store = ms.BlobStore(w)
    T = 32
    g = GpuLayerStack(w, store=store)
    rep = ft.ft_moe_measure_mode(g.pool, max(1, T * w.top_k // 64))
    share = rep["balanced_share"]
    print("measured mode", ["offload", "hybrid", "fused"][rep["mode"]], "balanced share", share)
    assert 0.0 < share < 1.0
    ft.ft_moe_set_hybrid_share(g.pool, share)
    o = OracleLayerStack(w, pool_slots=g.C, share=share, blob_fn=lambda l, e: store.expert(l, e), dequant_items=24,
                         threads=THREADS)
    try:
        rels = []
        for s in (0, 33, 65, 97, 127):  # every popularity phase (a shift every 32 steps) and the last step
            for l in range(w.num_layers):
                x = ms.activations(w, l, s, T)
                b = ms.popularity_bias(w, l, w.phase(s))
                want = (s, l) in {(0, 0), (0, 1), (33, 90), (33, 91), (127, 90), (127, 91)}
                gr = g.forward(l, x, g.bias(l, s))
                orr = o.forward(l, x, b, outputs=want)
                r = compare_call(gr, orr, w.top_k, check_out=want)
                if r is not None:
                    rels.append(r)
            print(f"glm step {s} ok", flush=True)
        compare_table(g, o)
        st = ft.ft_moe_pool_stats(g.pool)
        for key in ("pair_hits", "pair_misses", "expert_misses", "cpu_misses", "evictions", "bytes_h2d", "calls"):
            assert st[key] == o.stats[key], key
        assert st["cpu_misses"] > 0 and len(rels) == 6
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
            r = compare_call(gr, orr, w.top_k, check_out=want)
            if r is not None:
                rels.append(r)
        print(act, "rel-L2", rels)
        assert len(rels) == 2
    finally:
        g.close()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T", [8192, 1])
def test_qwen_a3b_prefill_other_chunk_sizes(T):
    """The staged path at the pages' default chunk of 8,192 tokens (devpik,
    "Long Prompts Are the Bottleneck": 65,536 pairs, ~640 row tiles per layer)
    and at a one-token chunk, on the first four Qwen-A3B-shaped layers with
    MXFP4 activations: decisions exact on every layer and the pool table after
    the chunk; outputs on sampled rows of the first and the last layer."""
    from tests.moe_case import GpuLayerStack, compare_call, compare_table
    from oracle import ffn as OFFN
    import lru_expert_cache_amd as ft

    w0 = ms.workload("qwen-a3b-prefill-4096")
    w = w0.with_(num_layers=4, layer_fmt=w0.layer_fmt[:4], batches=(T,))
    store = ms.BlobStore(w)
    g = GpuLayerStack(w, store=store)
    o = OracleLayerStack(w, pool_slots=g.C, blob_fn=lambda l, e: store.expert(l, e), dequant_items=130,
                         act_mode=OFFN.ACT_MXFP4)
    rng = np.random.default_rng(2)
    try:
        rels = []
        for l in range(w.num_layers):
            x = ms.activations(w, l, 0, T)
            b = ms.popularity_bias(w, l, 0)
            want = l in (0, w.num_layers - 1)
            toks = np.sort(rng.choice(T, min(T, 24), replace=False)) if want else None
            gr = g.forward(l, x, g.bias(l, 0), prefill=True, act=ft.FT_ACT_MXFP4)
            orr = o.forward(l, x, b, prefill=True, outputs=want, out_tokens=toks)
            r = compare_call(gr, orr, w.top_k, check_out=want)
            if r is not None:
                rels.append(r)
        compare_table(g, o)
        st = ft.ft_moe_pool_stats(g.pool)
        assert st["bytes_h2d"] == o.stats["bytes_h2d"] == w.num_layers * w.num_experts * ms.expert_bytes(
            ms.FMT_MXFP4, w.hidden, w.inter)
        assert st["pair_misses"] == w.num_layers * T * w.top_k
        print(f"T={T} rel-L2", rels)
        assert len(rels) == 2
    finally:
        g.close()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["deepseek-v4-flash-decode", "glm-5.2-mixed-decode"])
def test_split_k_ffn_at_full_shapes(name):
    """The split-K expert FFN (k_ffn: NVFP4 and FP8 prefill, and decode calls of
    more than 64 tokens) at the DeepSeek- and GLM-shaped layer sizes, on their
    first two layers: a 128-token decode call per layer (with DeepSeek's 968
    slots its 1,024 pairs run in two waves), a 256-token staged prefill chunk,
    then decode again.  Decisions, tables and counters exact; outputs on four
    sampled rows of every call."""
    from tests.moe_case import GpuLayerStack, compare_call, compare_table
    import lru_expert_cache_amd as ft

    w0 = ms.workload(name)
    w = w0.with_(num_layers=2, layer_fmt=w0.layer_fmt[:2])
    store = ms.BlobStore(w)
    g = GpuLayerStack(w, store=store)
    o = OracleLayerStack(w, pool_slots=g.C, blob_fn=lambda l, e: store.expert(l, e), dequant_items=24,
                         threads=THREADS)
    rng = np.random.default_rng(3)
    try:
        rels = []
        for step, (prefill, T) in enumerate(((False, 128), (True, 256), (False, 128))):
            for l in range(w.num_layers):
                x = ms.activations(w, l, 5 + step, T)
                b = ms.popularity_bias(w, l, 0)
                toks = np.sort(rng.choice(T, 4, replace=False))
                gr = g.forward(l, x, g.bias(l, 0), prefill=prefill)
                orr = o.forward(l, x, b, prefill=prefill, outputs=True, out_tokens=toks)
                rels.append(compare_call(gr, orr, w.top_k))
            # the last call ran layer 1 (NVFP4, or FP8): the split-K kernel
            kern = ft.ft_moe_ffn_kernel_name("ffn_gateup")
            print(f"{name} {'prefill' if prefill else 'decode'} T={T} ok, {kern}", flush=True)
            assert kern.startswith("k_ffn<"), kern
        compare_table(g, o)
        st = ft.ft_moe_pool_stats(g.pool)
        for key in ("pair_hits", "pair_misses", "expert_hits", "expert_misses", "evictions", "bytes_h2d", "calls"):
            assert st[key] == o.stats[key], (key, st[key], o.stats[key])
        print("rel-L2", rels)
    finally:
        g.close()
