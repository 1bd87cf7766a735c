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
