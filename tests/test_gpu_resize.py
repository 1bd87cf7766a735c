"""Elastic resize of the pool between decode calls: shrinking keeps the most
recently used residents, growing keeps everything, and the calls after a
resize make the same decisions, tables and counters as the oracle's pool
resized the same way (dev.to "FreeToken uses bandwidth-adaptive CPU-GPU
co-execution on your desktop", section "Memory that moves while the engine
runs").  Outputs after the resize check that the moved expert bytes landed in
their new slots."""

import numpy as np
import pytest

import moe_synth as ms
from oracle.layer import OracleLayerStack

pytestmark = pytest.mark.gpu

MX, NV, F8 = ms.FMT_MXFP4, ms.FMT_NVFP4, ms.FMT_FP8_B128


def _w():
    return ms.Workload(131, "small-131", 3, 256, 256, 16, 4, (MX, F8, NV), 30, (4,), 4, "decode", None, None,
                       True, False, None)


def test_resize_between_decode_calls_matches_oracle():
    from tests.moe_case import GpuLayerStack, compare_call, compare_table
    import lru_expert_cache_amd as ft

    w = _w()
    T, L = 4, w.num_layers
    g = GpuLayerStack(w)
    o = OracleLayerStack(w, pool_slots=g.C)
    step = 0

    def run(n):
        nonlocal step
        for _ in range(n):
            for l in range(L):
                x = ms.activations(w, l, step, T)
                compare_call(g.forward(l, x, None), o.forward(l, x, None), w.top_k)
            step += 1

    try:
        run(3)
        compare_table(g, o)
        # the slot counts: shrink below the residents, shrink to the minimum
        # (top-k), grow back past the original size
        for new_c in (11, w.top_k, 40, 18):
            resident = sum(k is not None for k in o.pool.snapshot()[0])
            rc = ft.ft_moe_resize_pool(g.pool, new_c)
            assert rc == (ft.FT_WARN_STAGING_SMALL if new_c < 2 * w.num_experts else ft.FT_OK)
            info = o.pool.resize(new_c)
            g.C = new_c
            assert len(info["evicted"]) == max(0, resident - new_c)
            compare_table(g, o)
            run(2)
            compare_table(g, o)
        s = ft.ft_moe_pool_stats(g.pool)
        for key in ("pair_hits", "pair_misses", "expert_hits", "expert_misses", "evictions", "bytes_h2d", "calls"):
            assert s[key] == o.stats[key], (key, s[key], o.stats[key])
        assert s["slots_total"] == 18
    finally:
        g.close()


def test_resize_rejects_bad_sizes():
    from tests.moe_case import GpuLayerStack
    import lru_expert_cache_amd as ft

    g = GpuLayerStack(_w())
    try:
        for bad in (g.w.top_k - 1, 0, 65537):
            with pytest.raises(ft.FtError):
                ft.ft_moe_resize_pool(g.pool, bad)
        assert ft.ft_moe_pool_stats(g.pool)["slots_total"] == g.C
    finally:
        g.close()
