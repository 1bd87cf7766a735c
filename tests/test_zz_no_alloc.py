"""ft_moe_layer_forward_noalloc (per-call work buffers in the library's static
per-GPU scratch, no allocation) against ft_moe_layer_forward: two pools of
the same workload driven call for call, the regular one also checked against
the oracle; decisions, outputs, tables and counters must be identical, on
consecutive calls whose second one is smaller, and no device memory may be
allocated by the no-alloc calls."""

import numpy as np
import pytest

import moe_synth as ms
from oracle.layer import OracleLayerStack

pytestmark = pytest.mark.gpu

MX, NV, F8 = ms.FMT_MXFP4, ms.FMT_NVFP4, ms.FMT_FP8_B128


def _small(cfg_id, L, H, I, E, k, fmts, C, shared=False, alpha=1.0):
    return ms.Workload(cfg_id, f"small-{cfg_id}", L, H, I, E, k, tuple(fmts), C, (8,), 4, "decode", alpha, None,
                       shared, False, None)


def _noalloc_call(ft, torch, g, layer, x_bits, bias):
    T, k = x_bits.shape[0], g.w.top_k
    x = torch.from_numpy(x_bits.view(np.int16)).to(g.dev)
    out = torch.empty_like(x)
    tr = dict(sel=torch.empty(T * k, dtype=torch.int32, device=g.dev),
              w=torch.empty(T * k, dtype=torch.float32, device=g.dev),
              slot=torch.empty(T * k, dtype=torch.int32, device=g.dev),
              flag=torch.empty(T * k, dtype=torch.uint8, device=g.dev),
              row=torch.empty(T * k, dtype=torch.int32, device=g.dev))
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info(g.dev)[0]
    ft.ft_moe_layer_forward_noalloc(g.pool, layer, T, x, bias, out, ft.FT_FWD_DECODE, None, tr)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info(g.dev)[0]
    res = {n: t.cpu().numpy() for n, t in tr.items()}
    res["out_bits"] = out.cpu().numpy().view(np.uint16)
    return res, free0 - free1


# (workload, calls): mixed formats and a shared expert, uniform routing over
# pools that hold fewer keys than the calls touch (so calls evict), every call one wave (T * k <=
# slots, the device-driven path); calls of <= 16 tokens take the wide FFN
# kernel, larger ones the streaming kernel
CASES = {
    "16-experts": (_small(160, 3, 512, 256, 16, 2, [MX, F8, NV], 40, shared=True, alpha=None),
                   [(20, 0), (5, 1), (16, 2), (1, 3)]),
    "64-experts": (_small(163, 4, 256, 256, 64, 2, [NV, MX, F8, MX], 200, shared=True, alpha=None), [(64, 0), (3, 1)]),
}


def _deepseek_four_layers():
    """The DeepSeek-shaped layers (H 7168, I 2048, 256 NVFP4 experts, top-8,
    shared expert), four of them over 520 slots: 64-token calls (512 pairs, one
    wave) take about two thirds of the scratch array, and the layers' distinct
    experts outnumber the slots, so calls evict."""
    w0 = ms.workload("deepseek-v4-flash-decode")
    return w0.with_(num_layers=4, layer_fmt=w0.layer_fmt[:4], pool_slots=520)


# full-size case: decisions against the oracle, outputs against the regular
# entry point bit for bit (the regular path's outputs at this shape are checked
# against the oracle by the workload tests)
FULL_CASES = {"deepseek-shape": (_deepseek_four_layers, [(64, 0), (16, 1)])}


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", list(CASES) + list(FULL_CASES))
def test_noalloc_matches_forward_on_consecutive_calls(name):
    import torch
    from tests.moe_case import GpuLayerStack, compare_call, compare_table
    import lru_expert_cache_amd as ft

    full = name in FULL_CASES
    if full:
        make, calls = FULL_CASES[name]
        w = make()
        store = ms.BlobStore(w)
        o = OracleLayerStack(w, pool_slots=w.pool_slots, blob_fn=lambda l, e: store.expert(l, e))
    else:
        w, calls = CASES[name]
        store = None
        o = OracleLayerStack(w, pool_slots=w.pool_slots)
    ga = GpuLayerStack(w, store=store)
    gn = GpuLayerStack(w, store=store)
    try:
        for T, s in calls:
            for l in range(w.num_layers):
                x_bits = ms.activations(w, l, s, T)
                ra = ga.forward(l, x_bits, ga.bias(l, s))
                compare_call(ra, o.forward(l, x_bits, ms.popularity_bias(w, l, 0), outputs=not full), w.top_k,
                             check_out=not full)
                rn, grew = _noalloc_call(ft, torch, gn, l, x_bits, gn.bias(l, s))
                assert grew == 0, f"device memory fell by {grew} bytes during a no-alloc call"
                assert np.array_equal(rn["out_bits"], ra["out_bits"]), (T, l)
                for key in ("w", "slot", "flag", "row"):
                    assert np.array_equal(rn[key], ra[key].reshape(-1)), (key, T, l)
                assert np.array_equal(rn["sel"].reshape(T, w.top_k), ra["sel"]), (T, l)
        compare_table(ga, o)
        compare_table(gn, o)
        sa, sn = ft.ft_moe_pool_stats(ga.pool), ft.ft_moe_pool_stats(gn.pool)
        assert sa.pop("copy_ms") > 0 and sn.pop("copy_ms") > 0  # measured, not computed
        assert sa == sn, (sa, sn)
        assert sn["evictions"] > 0 and sn["pair_hits"] > 0
    finally:
        ga.close()
        gn.close()


def test_noalloc_rejects_calls_it_cannot_run():
    import torch
    from tests.moe_case import GpuLayerStack
    import lru_expert_cache_amd as ft

    w = _small(161, 2, 256, 128, 8, 2, [MX, MX], 16)
    g = GpuLayerStack(w)
    try:
        x = torch.zeros((4, 256), dtype=torch.int16, device=g.dev)
        out = torch.empty_like(x)
        # prefill calls, host-driven hybrid calls: not the device-driven decode path
        with pytest.raises(ft.FtError) as ei:
            ft.ft_moe_layer_forward_noalloc(g.pool, 0, 4, x, None, out, ft.FT_FWD_PREFILL_STAGED)
        assert ei.value.code == ft.FT_E_INVALID and "device-driven decode" in str(ei.value)
        ft.ft_moe_set_hybrid_share(g.pool, 0.5)
        with pytest.raises(ft.FtError) as ei:
            ft.ft_moe_layer_forward_noalloc(g.pool, 0, 4, x, None, out, ft.FT_FWD_DECODE)
        assert ei.value.code == ft.FT_E_INVALID
        ft.ft_moe_set_hybrid_share(g.pool, 0.0)
        ft.ft_moe_layer_forward_noalloc(g.pool, 0, 4, x, None, out, ft.FT_FWD_DECODE)
        torch.cuda.synchronize()
    finally:
        g.close()
    # a call whose buffers exceed the 16 MiB array: 2048 tokens x 16 experts of
    # H = I = 128 need 16.8 MiB (h and p rows alone are 16 MiB); rejected before
    # any device work
    big = _small(162, 1, 128, 128, 16, 16, [MX], 2048 * 16, alpha=None)
    g = GpuLayerStack(big)
    try:
        x = torch.zeros((2048, 128), dtype=torch.int16, device=g.dev)
        with pytest.raises(ft.FtError) as ei:
            ft.ft_moe_layer_forward_noalloc(g.pool, 0, 2048, x, None, torch.empty_like(x), ft.FT_FWD_DECODE)
        assert ei.value.code == ft.FT_E_INVALID and "scratch" in str(ei.value)
        # 1024 tokens fit
        ft.ft_moe_layer_forward_noalloc(g.pool, 0, 1024, x, None, torch.empty_like(x), ft.FT_FWD_DECODE)
        torch.cuda.synchronize()
    finally:
        g.close()
