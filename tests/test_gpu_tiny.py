"""GPU parity on the tiny layer (H 256, I 128, 16 experts, top-2, MXFP4, 8 slots)
and on small synthetic layers covering the edge cases."""

import numpy as np
import pytest

import moe_synth as ms
from oracle.layer import OracleLayerStack

pytestmark = pytest.mark.gpu


def _stacks(w, **kw):
    from tests.moe_case import GpuLayerStack

    share = kw.pop("share", 0.0)
    g = GpuLayerStack(w, share=share, **kw)
    o = OracleLayerStack(w, pool_slots=g.C, share=share)
    return g, o


def _run(g, o, layer, step, T, prefill=False, check_out=True):
    from tests.moe_case import compare_call

    x = ms.activations(g.w, layer, step, T)
    b = ms.popularity_bias(g.w, layer, g.w.phase(step))
    gr = g.forward(layer, x, g.bias(layer, step), prefill=prefill)
    orr = o.forward(layer, x, b, prefill=prefill, outputs=check_out)
    return compare_call(gr, orr, g.w.top_k, check_out=check_out)


def test_tiny_one_call_of_64_tokens_in_waves():
    from tests.moe_case import compare_table

    w = ms.workload(0)
    g, o = _stacks(w)
    try:
        print("tiny T=64", flush=True)
        r = _run(g, o, 0, 0, 64)
        compare_table(g, o)
        assert len(o.pool.snapshot()[0]) == 8
        print("rel-L2", r)
    finally:
        g.close()


def test_tiny_64_calls_of_one_token():
    from tests.moe_case import compare_table
    import lru_expert_cache_amd as ft

    w = ms.workload(0)
    g, o = _stacks(w)
    try:
        for s in range(64):
            _run(g, o, 0, s, 1)
        compare_table(g, o)
        st = ft.ft_moe_pool_stats(g.pool)
        for key in ("pair_hits", "pair_misses", "expert_hits", "expert_misses", "evictions", "calls"):
            assert st[key] == o.stats[key], key
        assert st["bytes_h2d"] == o.stats["bytes_h2d"]
        assert st["slots_used"] == 8 and st["slots_total"] == 8
    finally:
        g.close()


@pytest.mark.parametrize("kind,sheet_tflops", [(0, 10100.0), (1, 5000.0), (2, 2500.0), (3, 2500.0), (4, 78.6)])
def test_mfma_rate_is_below_the_data_sheet_peak(kind, sheet_tflops):
    # register-only MFMA loops: a positive rate that no instruction mix can push
    # past the data-sheet dense peak of its operand type
    import lru_expert_cache_amd as ft

    tf = ft.ft_moe_mfma_rate(kind, iters=500) / 1e12
    print("kind", kind, "TFLOP/s", tf)
    assert 0.05 * sheet_tflops < tf <= 1.02 * sheet_tflops
