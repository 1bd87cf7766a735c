"""One-time strategy choice measured on the device (ft_moe_measure_mode):
the rates are real, the decision equals the oracle's rule on the same rates,
measuring leaves the slot table and counters alone, and the applied share is
the one later calls split their misses by (mindstudio "FreeToken Explained:
Run 290B+ MoE Models on One Gaming GPU", section "How does the benchmark decide
between hybrid and offload mode?")."""

import math

import numpy as np
import pytest

import moe_synth as ms
from oracle.layer import OracleLayerStack
from oracle.mode import FUSED, choose_mode

pytestmark = pytest.mark.gpu

MX, NV, F8 = ms.FMT_MXFP4, ms.FMT_NVFP4, ms.FMT_FP8_B128


def _w(C):
    return ms.Workload(132, "small-132", 3, 256, 256, 16, 4, (MX, F8, NV), C, (4,), 4, "decode", None, None,
                       True, False, None)


def _oracle_decision(rep, w):
    fmts = list(w.layer_fmt)
    f = lambda key: {g: rep[key][g] for g in set(fmts)}
    return choose_mode(fmts, f("expert_bytes"), f("h2d_bytes_per_s"), f("gpu_bytes_per_s"), f("cpu_bytes_per_s"),
                       rep["pool_slots"], w.num_experts)


@pytest.mark.parametrize("tokens", [1, 16])
def test_measured_mode_matches_rule_and_leaves_the_pool_alone(tokens):
    from tests.moe_case import GpuLayerStack, compare_call, compare_table
    import lru_expert_cache_amd as ft

    w = _w(24)
    g = GpuLayerStack(w)
    o = OracleLayerStack(w, pool_slots=g.C)
    try:
        for step in range(2):
            for l in range(w.num_layers):
                x = ms.activations(w, l, step, 4)
                compare_call(g.forward(l, x, None), o.forward(l, x, None), w.top_k)
        st0 = ft.ft_moe_pool_stats(g.pool)
        rep = ft.ft_moe_measure_mode(g.pool, tokens, apply=True)
        assert rep["tokens"] == tokens and rep["pool_slots"] == 24 and rep["all_experts"] == 48
        for f in (MX, NV, F8):
            assert rep["layers"][f] == 1
            assert rep["expert_bytes"][f] == ms.expert_bytes(f, w.hidden, w.inter)
            for key in ("h2d_bytes_per_s", "gpu_bytes_per_s", "cpu_bytes_per_s"):
                assert math.isfinite(rep[key][f]) and rep[key][f] > 0, (key, f)
            # plausible magnitudes for a PCIe link and HBM-fed kernels
            assert 1e8 < rep["h2d_bytes_per_s"][f] < 2e11
        want = _oracle_decision(rep, w)
        assert rep["mode"] == want["mode"]
        assert math.isclose(rep["share"], want["share"], rel_tol=1e-12, abs_tol=0.0)
        assert math.isclose(rep["t_stream"], want["t_stream"], rel_tol=1e-12)
        # measuring moved nothing
        compare_table(g, o)
        assert ft.ft_moe_pool_stats(g.pool) == st0
        # later calls split their misses by the applied share
        o.share = rep["share"]
        for step in range(2, 4):
            for l in range(w.num_layers):
                x = ms.activations(w, l, step, 4)
                compare_call(g.forward(l, x, None), o.forward(l, x, None), w.top_k)
        compare_table(g, o)
    finally:
        g.close()


def test_pool_with_a_slot_for_every_expert_is_fused():
    from tests.moe_case import GpuLayerStack
    import lru_expert_cache_amd as ft

    w = _w(48)
    g = GpuLayerStack(w)
    try:
        rep = ft.ft_moe_measure_mode(g.pool, 4, apply=True)
        assert rep["mode"] == FUSED and rep["share"] == 0.0
        assert rep["mode"] == _oracle_decision(rep, w)["mode"]
        with pytest.raises(ft.FtError):
            ft.ft_moe_measure_mode(g.pool, 65)
    finally:
        g.close()


def test_share_per_format_splits_each_layer_by_its_format():
    """Each layer's misses split by the share of its weight format, exactly
    as the oracle's split rule with that share."""
    from tests.moe_case import GpuLayerStack, compare_call, compare_table
    import lru_expert_cache_amd as ft

    w = ms.Workload(133, "small-133", 3, 256, 256, 16, 4, (MX, F8, NV), 24, (4,), 4, "decode", None, None,
                    True, False, None)
    shares = {MX: 0.25, F8: 0.75, NV: 0.5}
    g = GpuLayerStack(w, share=shares)
    o = OracleLayerStack(w, pool_slots=g.C, share=shares)
    try:
        for f, v in shares.items():
            assert ft.ft_moe_get_hybrid_share(g.pool, f) == v
        for step in range(3):
            for l in range(w.num_layers):
                x = ms.activations(w, l, step, 5)
                compare_call(g.forward(l, x, None), o.forward(l, x, None), w.top_k)
        compare_table(g, o)
        st = ft.ft_moe_pool_stats(g.pool)
        assert st["cpu_misses"] == o.stats["cpu_misses"] > 0
        with pytest.raises(ft.FtError):
            ft.ft_moe_set_hybrid_share_format(g.pool, 4, 0.5)
        with pytest.raises(ft.FtError):
            ft.ft_moe_set_hybrid_share_format(g.pool, MX, 1.5)
    finally:
        g.close()


def test_rebalance_from_in_situ_rates():
    """ft_moe_rebalance: the bytes it observed are exactly the host-computed and
    streamed expert bytes of the calls since the last share change (by
    format, from the oracle's miss lists); the refined share of each format is
    the balanced split of its observed costs per byte; later calls split by
    the new shares exactly as the oracle does with them; the observations
    start again from zero."""
    from tests.moe_case import GpuLayerStack, compare_call, compare_table
    import lru_expert_cache_amd as ft

    w = ms.Workload(134, "small-134", 4, 256, 256, 16, 4, (MX, F8, MX, F8), 24, (4,), 4, "decode", None, None,
                    False, False, None)
    g = GpuLayerStack(w, share=0.5)
    o = OracleLayerStack(w, pool_slots=g.C, share=0.5)
    eb = {f: ms.expert_bytes(f, w.hidden, w.inter) for f in (MX, F8)}
    host_b = {MX: 0, F8: 0}
    copy_b = {MX: 0, F8: 0}
    try:
        rep0 = ft.ft_moe_measure_mode(g.pool, 4, apply=False)  # keeps the device FFN rates
        for step in range(3):
            for l in range(w.num_layers):
                x = ms.activations(w, l, step, 6)
                ro = o.forward(l, x, None)
                compare_call(g.forward(l, x, None), ro, w.top_k)
                f = w.fmt(l)
                host_b[f] += eb[f] * sum(len(wv["cpu"]) for wv in ro["waves"])
                copy_b[f] += eb[f] * sum(len(wv["stream"]) for wv in ro["waves"])
        rep = ft.ft_moe_rebalance(g.pool, apply=True)
        for f in (MX, F8):
            assert host_b[f] > 0 and copy_b[f] > 0
            assert rep["host_bytes"][f] == host_b[f] and rep["copy_bytes"][f] == copy_b[f]
            assert rep["host_seconds"][f] > 0 and rep["copy_seconds"][f] > 0
            assert rep["gpu_bytes_per_s"][f] == rep0["gpu_bytes_per_s"][f] > 0
            ts = rep["copy_seconds"][f] / copy_b[f] + 1.0 / rep["gpu_bytes_per_s"][f]
            tc = rep["host_seconds"][f] / host_b[f]
            assert rep["changed"][f] == 1 and 0.0 < rep["share"][f] < 1.0
            assert math.isclose(rep["share"][f], ts / (ts + tc), rel_tol=1e-12)
            assert ft.ft_moe_get_hybrid_share(g.pool, f) == rep["share"][f]
        assert rep["changed"][NV] == 0 and rep["host_bytes"][NV] == 0
        again = ft.ft_moe_rebalance(g.pool, apply=True)
        assert again["changed"] == [0, 0, 0, 0] and sum(again["host_bytes"]) == 0
        o.share = {f: rep["share"][f] for f in (MX, F8)}
        for step in range(3, 5):
            for l in range(w.num_layers):
                x = ms.activations(w, l, step, 6)
                compare_call(g.forward(l, x, None), o.forward(l, x, None), w.top_k)
        compare_table(g, o)
    finally:
        g.close()
