"""Prefill staging that skips experts already resident in the pool
(FT_FWD_PREFILL_HIT_D2D; devpik "FreeToken: Run Frontier MoE Models on Your
Own GPU, and the RAM It Takes", section "Long Prompts Are the Bottleneck"):
decisions, outputs, tables and counters against the oracle's staging with the
same option, chunks interleaved with decode calls, an MX activation chunk, a
chunk whose pool has no residents beyond the staging region, and the
same-option rule inside a chunk.  With the option the copied experts become
residents of their staging slots, so later decode calls can hit them."""

import numpy as np
import pytest

import moe_synth as ms
from oracle.layer import OracleLayerStack

pytestmark = pytest.mark.gpu

MX, NV, F8 = ms.FMT_MXFP4, ms.FMT_NVFP4, ms.FMT_FP8_B128


def _small(cfg_id, L, H, I, E, k, fmts, C, shared=False, alpha=None):
    # uniform routing by default: decode calls touch every key, so residents
    # also sit beyond the staging region
    return ms.Workload(cfg_id, f"small-{cfg_id}", L, H, I, E, k, tuple(fmts), C, (8,), 4, "decode", alpha, None,
                       shared, False, None)


@pytest.mark.parametrize("shared", [False, True])
def test_hit_d2d_chunks_between_decode_calls(shared):
    from tests.moe_case import GpuLayerStack, compare_call, compare_table
    import lru_expert_cache_amd as ft

    # 3 layers of 8 experts, top-2; staging takes slots [0, 16), 14 slots beyond
    w = _small(140 + int(shared), 3, 256, 128, 8, 2, [MX, F8, NV], 30, shared=shared)
    g = GpuLayerStack(w)
    o = OracleLayerStack(w, pool_slots=g.C)
    hits = 0
    staged_hits = 0  # decode pairs served by a previous chunk's staged copies
    try:
        for rnd in range(3):
            for s in range(3):
                for l in range(3):
                    x = ms.activations(w, l, 10 * rnd + s, 8)
                    orr = o.forward(l, x, ms.popularity_bias(w, l, 0))
                    compare_call(g.forward(l, x, g.bias(l, 0)), orr, 2)
                    staged_hits += int(((orr["flag"] == ft.FT_PAIR_HIT) & (orr["slot"] < 2 * w.num_experts)).sum())
            for l in range(3):
                x = ms.activations(w, l, 200 + rnd, 45)
                gr = g.forward(l, x, g.bias(l, 0), prefill=True, hit_d2d=True)
                orr = o.forward(l, x, ms.popularity_bias(w, l, 0), prefill=True, hit_d2d=True)
                compare_call(gr, orr, 2)
                hits += int((orr["flag"] == ft.FT_PAIR_HIT).sum())
            compare_table(g, o)
        st = ft.ft_moe_pool_stats(g.pool)
        for key in ("pair_hits", "pair_misses", "expert_hits", "expert_misses", "evictions", "bytes_h2d", "calls"):
            assert st[key] == o.stats[key], (key, st[key], o.stats[key])
        assert hits > 0, "no resident expert was reused: the case does not exercise the option"
        assert staged_hits > 0, "no decode call hit a staged copy"
    finally:
        g.close()


def test_hit_d2d_with_mx_activations():
    from tests.moe_case import GpuLayerStack, compare_call, rel_l2
    from oracle import ffn as OFFN, formats as OF
    import lru_expert_cache_amd as ft

    w = _small(142, 3, 256, 256, 8, 2, [MX, MX, MX], 28)
    g = GpuLayerStack(w)
    od = OracleLayerStack(w, pool_slots=g.C)
    om = OracleLayerStack(w, pool_slots=g.C, act_mode=OFFN.ACT_MXFP4)
    try:
        for s in range(3):
            for l in range(3):
                x = ms.activations(w, l, s, 8)
                g.forward(l, x, g.bias(l, 0))
                od.forward(l, x, ms.popularity_bias(w, l, 0), outputs=False)
                om.forward(l, x, ms.popularity_bias(w, l, 0), outputs=False)
        n_hit = 0
        for l in range(3):
            x = ms.activations(w, l, 300, 300)
            gr = g.forward(l, x, g.bias(l, 0), prefill=True, act=ft.FT_ACT_MXFP4, hit_d2d=True)
            orr = om.forward(l, x, ms.popularity_bias(w, l, 0), prefill=True, hit_d2d=True)
            compare_call(gr, orr, 2, check_out=False)
            assert rel_l2(OF.bf16_from_bits(gr["out_bits"]), orr["out"]) <= 2e-3
            n_hit += int((orr["flag"] == ft.FT_PAIR_HIT).sum())
        assert n_hit > 0
    finally:
        g.close()


def test_hit_d2d_without_residents_streams_everything_and_option_is_per_chunk():
    import torch
    from tests.moe_case import GpuLayerStack, compare_call
    import lru_expert_cache_amd as ft

    # pool of exactly two staging layers: nothing can be resident beyond them
    w = _small(143, 3, 256, 128, 8, 2, [NV, MX, F8], 16, alpha=1.0)
    g = GpuLayerStack(w)
    o = OracleLayerStack(w, pool_slots=g.C)
    try:
        for l in range(3):
            x = ms.activations(w, l, 0, 6)
            compare_call(g.forward(l, x, g.bias(l, 0)), o.forward(l, x, ms.popularity_bias(w, l, 0)), 2)
        for l in range(3):
            x = ms.activations(w, l, 1, 40)
            gr = g.forward(l, x, g.bias(l, 0), prefill=True, hit_d2d=True)
            orr = o.forward(l, x, ms.popularity_bias(w, l, 0), prefill=True, hit_d2d=True)
            compare_call(gr, orr, 2)
            assert len(gr["stream"]) == 8 and (orr["flag"] != ft.FT_PAIR_HIT).all()
        x = torch.zeros((4, 256), dtype=torch.int16, device="cuda")
        out = torch.empty_like(x)
        ft.ft_moe_layer_forward(g.pool, 0, 4, x, None, out, ft.FT_FWD_PREFILL_STAGED | ft.FT_FWD_PREFILL_HIT_D2D)
        with pytest.raises(ft.FtError) as ei:
            ft.ft_moe_layer_forward(g.pool, 1, 4, x, None, out, ft.FT_FWD_PREFILL_STAGED)
        assert ei.value.code == ft.FT_E_STATE
        with pytest.raises(ft.FtError) as ei:
            ft.ft_moe_layer_forward(g.pool, 0, 4, x, None, out, ft.FT_FWD_DECODE | ft.FT_FWD_PREFILL_HIT_D2D)
        assert ei.value.code == ft.FT_E_INVALID
    finally:
        g.close()


@pytest.mark.parametrize("hit_d2d", [False, True])
def test_staged_resolve_many_experts_several_chunks(hit_d2d):
    """Staged calls resolve over many workgroups (chunks of 1024 pairs): 512
    experts, the most a layer may have (two threads per expert in the
    per-expert totals), and 700 tokens x top-4 = 2800 pairs (three chunks, the
    last one partial), with and without hit-D2D, between decode calls: the
    same decisions, tables and counters as the oracle's staging."""
    from tests.moe_case import GpuLayerStack, compare_call, compare_table
    import lru_expert_cache_amd as ft

    w = _small(145 + int(hit_d2d), 2, 128, 128, 512, 4, [MX, NV], 2 * 512 + 200)
    g = GpuLayerStack(w)
    o = OracleLayerStack(w, pool_slots=g.C)
    try:
        for rnd in range(2):
            for l in range(2):
                x = ms.activations(w, l, 10 * rnd, 8)
                compare_call(g.forward(l, x, g.bias(l, 0)), o.forward(l, x, ms.popularity_bias(w, l, 0)), 4)
            for l in range(2):
                x = ms.activations(w, l, 300 + rnd, 700)
                gr = g.forward(l, x, g.bias(l, 0), prefill=True, hit_d2d=hit_d2d)
                compare_call(gr, o.forward(l, x, ms.popularity_bias(w, l, 0), prefill=True, hit_d2d=hit_d2d), 4)
            compare_table(g, o)
        st = ft.ft_moe_pool_stats(g.pool)
        for key in ("pair_hits", "pair_misses", "expert_hits", "expert_misses", "evictions", "bytes_h2d", "calls"):
            assert st[key] == o.stats[key], (key, st[key], o.stats[key])
    finally:
        g.close()
