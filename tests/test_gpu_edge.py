"""GPU parity on small synthetic layers that cover the edge cases: every
format, ragged token counts, odd expert counts, k = 1, the largest expert
count and top-k, waves, the all-resident ("fused") pool, the shared expert,
hybrid shares 0 < s < 1 and s = 1, calls with no tokens, prefill staging
followed by decode, and the error paths forced from the host."""

import os

import numpy as np
import pytest

import moe_synth as ms
from oracle.layer import OracleLayerStack

pytestmark = pytest.mark.gpu

MX, NV, F8 = ms.FMT_MXFP4, ms.FMT_NVFP4, ms.FMT_FP8_B128


def _small(cfg_id, L, H, I, E, k, fmts, C, shared=False, alpha=1.0, n_blobs=None):
    return ms.Workload(cfg_id, f"small-{cfg_id}", L, H, I, E, k, tuple(fmts), C, (8,), 4, "decode", alpha, None,
                       shared, False, n_blobs)


CASES = {
    "nvfp4-plain": (_small(107, 1, 256, 128, 8, 2, [NV], 16), [(4, 0)], 0.0),
    "mxfp4-shared": (_small(108, 1, 256, 128, 8, 2, [MX], 16, shared=True), [(4, 0)], 0.0),
    "fp8-waves": (_small(100, 2, 256, 128, 8, 2, [F8, F8], 6), [(8, 0), (3, 1), (8, 2)], 0.0),
    "nvfp4-shared-fused": (_small(101, 2, 384, 256, 12, 3, [NV, NV], 40, shared=True), [(5, 0), (7, 1), (1, 2)], 0.0),
    "mixed-hybrid": (_small(102, 3, 256, 384, 10, 2, [MX, F8, NV], 12), [(5, 0), (9, 1), (2, 2)], 0.5),
    "all-host": (_small(103, 2, 256, 128, 9, 2, [MX, F8], 9), [(4, 0), (4, 1)], 1.0),
    "k1-odd-E": (_small(104, 2, 128, 128, 5, 1, [MX, MX], 3, alpha=None), [(17, 0), (1, 1), (33, 2)], 0.0),
    "wide-k": (_small(105, 1, 512, 256, 40, 16, [MX], 48), [(3, 0), (11, 1)], 0.0),
    "aliased-blobs": (_small(106, 4, 256, 128, 8, 2, [MX, NV, MX, F8], 10, n_blobs=5), [(6, 0), (6, 1)], 0.0),
    # the largest expert count and top-k the library takes (512, 16); the second call's 640 pairs
    # exceed the 600 slots, so it runs in waves
    "max-experts-top16": (_small(110, 1, 128, 128, 512, 16, [MX], 600), [(12, 0), (40, 1)], 0.0),
}


@pytest.mark.parametrize("name", list(CASES))
def test_small_case(name):
    from tests.moe_case import GpuLayerStack, compare_call, compare_table
    import lru_expert_cache_amd as ft

    w, calls, share = CASES[name]
    g = GpuLayerStack(w, share=share)
    o = OracleLayerStack(w, pool_slots=g.C, share=share)
    try:
        for T, s in calls:
            for l in range(w.num_layers):
                x = ms.activations(w, l, s, T)
                b = ms.popularity_bias(w, l, 0)
                gr = g.forward(l, x, g.bias(l, s))
                orr = o.forward(l, x, b)
                compare_call(gr, orr, w.top_k)
        compare_table(g, o)
        st = ft.ft_moe_pool_stats(g.pool)
        for key in ("pair_hits", "pair_misses", "expert_hits", "expert_misses", "cpu_misses", "evictions",
                    "bytes_h2d", "calls"):
            assert st[key] == o.stats[key], (key, st[key], o.stats[key])
        if name == "nvfp4-shared-fused":
            assert st["evictions"] == 0
        if name == "all-host":
            assert st["pair_hits"] == 0 and st["slots_used"] == 0
    finally:
        g.close()


def test_prefill_then_decode_small():
    from tests.moe_case import GpuLayerStack, compare_call, compare_table

    w = _small(110, 3, 256, 128, 8, 2, [MX, F8, NV], 20)
    g = GpuLayerStack(w)
    o = OracleLayerStack(w, pool_slots=g.C)
    try:
        for s in range(2):  # decode, then a prefill chunk, then decode again
            for l in range(3):
                x = ms.activations(w, l, s, 6)
                compare_call(g.forward(l, x, g.bias(l, s)), o.forward(l, x, ms.popularity_bias(w, l, 0)), 2)
            for l in range(3):
                x = ms.activations(w, l, 100 + s, 45)
                compare_call(g.forward(l, x, g.bias(l, 0), prefill=True),
                             o.forward(l, x, ms.popularity_bias(w, l, 0), prefill=True), 2)
        compare_table(g, o)
    finally:
        g.close()


def test_state_errors_and_staging_warning():
    import torch
    from tests.moe_case import GpuLayerStack
    import lru_expert_cache_amd as ft

    w = _small(111, 3, 256, 128, 8, 2, [MX, MX, MX], 20)
    g = GpuLayerStack(w)
    try:
        x = torch.zeros((4, 256), dtype=torch.int16, device="cuda")
        out = torch.empty_like(x)
        with pytest.raises(ft.FtError) as ei:
            ft.ft_moe_layer_forward(g.pool, 1, 4, x, None, out, ft.FT_FWD_PREFILL_STAGED)
        assert ei.value.code == ft.FT_E_STATE
        ft.ft_moe_layer_forward(g.pool, 0, 4, x, None, out, ft.FT_FWD_PREFILL_STAGED)
        with pytest.raises(ft.FtError) as ei:
            ft.ft_moe_layer_forward(g.pool, 0, 4, x, None, out, ft.FT_FWD_DECODE)
        assert ei.value.code == ft.FT_E_STATE
        ft.ft_moe_layer_forward(g.pool, 1, 4, x, None, out, ft.FT_FWD_PREFILL_STAGED)
        ft.ft_moe_layer_forward(g.pool, 2, 4, x, None, out, ft.FT_FWD_PREFILL_STAGED)
        ft.ft_moe_layer_forward(g.pool, 0, 4, x, None, out, ft.FT_FWD_DECODE)
        with pytest.raises(ft.FtError) as ei:
            ft.ft_moe_layer_forward(g.pool, 0, 4, x, None, out, ft.FT_FWD_DECODE | ft.FT_ACT_MXFP4)
        assert ei.value.code == ft.FT_E_INVALID
        torch.cuda.synchronize()
    finally:
        g.close()
    small = _small(112, 2, 256, 128, 8, 2, [MX, MX], 10)
    g = GpuLayerStack(small)
    try:
        assert g.init_rc == ft.FT_WARN_STAGING_SMALL
        x = torch.zeros((4, 256), dtype=torch.int16, device="cuda")
        with pytest.raises(ft.FtError) as ei:
            ft.ft_moe_layer_forward(g.pool, 0, 4, x, None, torch.empty_like(x), ft.FT_FWD_PREFILL_STAGED)
        assert ei.value.code == ft.FT_E_INVALID
    finally:
        g.close()


def test_failed_copy_leaves_key_non_resident(monkeypatch):
    import torch
    from tests.moe_case import GpuLayerStack
    import lru_expert_cache_amd as ft

    w = _small(113, 2, 256, 128, 8, 2, [MX, MX], 16)
    monkeypatch.setenv("FT_MOE_FAULT", "copy:3")
    g = GpuLayerStack(w)
    monkeypatch.delenv("FT_MOE_FAULT")
    try:
        x = torch.from_numpy(ms.activations(w, 0, 0, 4).view(np.int16)).cuda()
        out = torch.empty_like(x)
        with pytest.raises(ft.FtError) as ei:
            ft.ft_moe_layer_forward(g.pool, 0, 4, x, None, out, ft.FT_FWD_DECODE)
        assert ei.value.code == ft.FT_E_HIP and "injected" in str(ei.value)
        stream, _ = ft.ft_moe_last_misses(g.pool)
        assert len(stream) >= 3
        key, _, _ = ft.ft_moe_pool_table(g.pool, 16)
        ok = {e for e, s in stream[:2]}
        failed = {e for e, s in stream[2:]}
        resident = {int(k) for k in key if k >= 0}
        assert ok <= resident and not (failed & resident)
        assert (key >= 0).sum() == 2
        # the pool keeps working: the failed experts miss again and are fetched
        ft.ft_moe_layer_forward(g.pool, 0, 4, x, None, out, ft.FT_FWD_DECODE)
        torch.cuda.synchronize()
        key, _, _ = ft.ft_moe_pool_table(g.pool, 16)
        assert failed <= {int(k) for k in key if k >= 0}
        assert torch.isfinite(out.view(torch.bfloat16).float()).all()
    finally:
        g.close()


def _act_case(shared, act_mode, H=256, T=300, cfg_id=120):
    from tests.moe_case import GpuLayerStack, rel_l2
    from oracle import ffn as OFFN, formats as OF
    import lru_expert_cache_amd as ft

    w = _small(cfg_id + int(shared), 3, H, 256, 8, 2, [MX, MX, MX], 16, shared=shared)
    g = GpuLayerStack(w)
    o = OracleLayerStack(w, pool_slots=g.C, act_mode=act_mode)
    flag = {OFFN.ACT_MXFP4: ft.FT_ACT_MXFP4, OFFN.ACT_MXFP8: ft.FT_ACT_MXFP8, OFFN.ACT_BF16: ft.FT_ACT_BF16}[act_mode]
    rels = []
    try:
        for l in range(3):
            x = ms.activations(w, l, 7, T)  # T=300: ~75 rows per expert, one ragged 128-row tile
            gr = g.forward(l, x, g.bias(l, 0), prefill=True, act=flag)
            orr = o.forward(l, x, ms.popularity_bias(w, l, 0), prefill=True)
            from tests.moe_case import compare_call
            compare_call(gr, orr, w.top_k, check_out=False)
            got = OF.bf16_from_bits(gr["out_bits"])
            rels.append(rel_l2(got, orr["out"]))
        return rels
    finally:
        g.close()


@pytest.mark.parametrize("shared", [False, True])
@pytest.mark.parametrize("act", ["mxfp8", "mxfp4"])
def test_prefill_mx_activation_modes_small(shared, act):
    from oracle import ffn as OFFN

    mode = OFFN.ACT_MXFP4 if act == "mxfp4" else OFFN.ACT_MXFP8
    rels = _act_case(shared, mode)
    print(act, "shared" if shared else "", "rel-L2", rels)
    assert max(rels) <= 2e-3


@pytest.mark.parametrize("act", ["mxfp8", "mxfp4"])
def test_prefill_mx_narrow_workgroup_tiles(act):
    # hidden 384: the down GEMM's 384 output features take the 2-wave-column
    # workgroup tile (128 features), the gate/up's 256 the wider ones; 600
    # tokens give ~150 rows per expert, two 128-row tiles with a ragged tail
    from oracle import ffn as OFFN

    mode = OFFN.ACT_MXFP4 if act == "mxfp4" else OFFN.ACT_MXFP8
    rels = _act_case(True, mode, H=384, T=600, cfg_id=124)
    print(act, "rel-L2", rels)
    assert max(rels) <= 2e-3


def test_prefill_bf16_wide_wave_tiles():
    # hidden 512, intermediate 256: with bf16 activations both GEMMs take the
    # 64-row x 128-column wave tiles (feature blocks of 256 and 512), two
    # workgroup stages; 600 tokens give two row tiles per expert with a ragged
    # tail
    from oracle import ffn as OFFN

    rels = _act_case(True, OFFN.ACT_BF16, H=512, T=600, cfg_id=126)
    print("bf16 rel-L2", rels)
    assert max(rels) <= 2e-3


def test_device_driven_and_host_driven_decode_agree():
    """Decode calls that fit one wave run device-driven (the GPU copies its own
    misses and the host never waits); FT_MOE_DECODE_PATH=host forces the
    host-driven path.  Both must give the oracle's decisions and bit-identical
    outputs, tables and counters.  The device-driven pool is driven
    asynchronously across three streams with no host wait between calls."""
    import torch

    from tests.moe_case import GpuLayerStack, compare_call, compare_table
    import lru_expert_cache_amd as ft

    w = _small(111, 3, 256, 256, 12, 3, [MX, F8, NV], 20, shared=True, alpha=None)  # uniform: evicts
    os.environ["FT_MOE_DECODE_PATH"] = "host"
    try:
        gh = GpuLayerStack(w)
    finally:
        del os.environ["FT_MOE_DECODE_PATH"]
    gd = GpuLayerStack(w)
    o = OracleLayerStack(w, pool_slots=gh.C)
    dev = gd.dev
    streams = [None, torch.cuda.Stream(dev), torch.cuda.Stream(dev)]
    try:
        calls = [(6, 0), (1, 1), (5, 2), (2, 3), (6, 4), (3, 5)]
        pending = []
        for i, (T, s) in enumerate(calls):
            for l in range(w.num_layers):
                x_bits = ms.activations(w, l, s, T)
                hr = gh.forward(l, x_bits, gh.bias(l, s))
                compare_call(hr, o.forward(l, x_bits, ms.popularity_bias(w, l, 0)), w.top_k)
                x = torch.from_numpy(x_bits.view(np.int16)).to(dev)
                out = torch.empty_like(x)
                sel = torch.empty(T * w.top_k, dtype=torch.int32, device=dev)
                slot = torch.empty_like(sel)
                st = streams[(i * w.num_layers + l) % 3]
                bias = gd.bias(l, s)
                ft.ft_moe_layer_forward(gd.pool, l, T, x, bias, out, ft.FT_FWD_DECODE, st,
                                        {"sel": sel, "slot": slot})
                pending.append((hr, out, sel, slot, (x, bias)))  # inputs stay alive until the sync
        torch.cuda.synchronize()
        for hr, out, sel, slot, _ in pending:
            assert np.array_equal(out.cpu().numpy().view(np.uint16), hr["out_bits"])
            assert np.array_equal(sel.cpu().numpy().reshape(hr["sel"].shape), hr["sel"])
            assert np.array_equal(slot.cpu().numpy(), hr["slot"])
        assert ft.ft_moe_last_misses(gd.pool) == ft.ft_moe_last_misses(gh.pool)
        compare_table(gd, o)
        sh, sd = ft.ft_moe_pool_stats(gh.pool), ft.ft_moe_pool_stats(gd.pool)
        # copy time is measured, not computed: both paths report some
        assert sh.pop("copy_ms") > 0 and sd.pop("copy_ms") > 0
        assert sh == sd, (sh, sd)
        assert sd["evictions"] > 0 and sd["pair_hits"] > 0
    finally:
        gh.close()
        gd.close()


def test_failed_work_buffer_allocation_recovers(monkeypatch):
    """A device allocation of the per-call buffers fails (injected): the call
    returns FT_E_OOM_DEVICE before any work is enqueued, and the next call
    allocates the buffers again and matches the oracle."""
    import torch
    from tests.moe_case import GpuLayerStack, compare_call, compare_table
    import lru_expert_cache_amd as ft

    w = _small(114, 2, 256, 128, 8, 2, [MX, NV], 16)
    monkeypatch.setenv("FT_MOE_FAULT", "work_alloc:5")
    g = GpuLayerStack(w)
    monkeypatch.delenv("FT_MOE_FAULT")
    o = OracleLayerStack(w, pool_slots=g.C)
    try:
        x_bits = ms.activations(w, 0, 0, 100)  # more than the 64 tokens buffers start with
        x = torch.from_numpy(x_bits.view(np.int16)).cuda()
        with pytest.raises(ft.FtError) as ei:
            ft.ft_moe_layer_forward(g.pool, 0, 100, x, None, torch.empty_like(x), ft.FT_FWD_DECODE)
        assert ei.value.code == ft.FT_E_OOM_DEVICE and "injected" in str(ei.value)
        for l in range(2):
            xb = ms.activations(w, l, 0, 100)
            compare_call(g.forward(l, xb, g.bias(l, 0)), o.forward(l, xb, ms.popularity_bias(w, l, 0)), 2)
        compare_table(g, o)
        st = ft.ft_moe_pool_stats(g.pool)
        assert st["calls"] == o.stats["calls"] and st["bytes_h2d"] == o.stats["bytes_h2d"]
    finally:
        g.close()


@pytest.mark.parametrize("which", [1, 3, 4])
def test_failed_mx_tile_allocation_recovers(monkeypatch, which):
    """One of the four MX activation-tile buffers fails to allocate
    (injected): the prefill call returns FT_E_OOM_DEVICE with none of them
    left allocated, and the retried chunk allocates all four and matches the
    oracle."""
    import torch
    from tests.moe_case import GpuLayerStack, compare_call, rel_l2
    from oracle import ffn as OFFN, formats as OF
    import lru_expert_cache_amd as ft

    w = _small(115, 2, 256, 256, 8, 2, [MX, MX], 16)
    monkeypatch.setenv("FT_MOE_FAULT", f"mx_alloc:{which}")
    g = GpuLayerStack(w)
    monkeypatch.delenv("FT_MOE_FAULT")
    o = OracleLayerStack(w, pool_slots=g.C, act_mode=OFFN.ACT_MXFP4)
    try:
        x_bits = ms.activations(w, 0, 3, 200)
        x = torch.from_numpy(x_bits.view(np.int16)).cuda()
        with pytest.raises(ft.FtError) as ei:
            ft.ft_moe_layer_forward(g.pool, 0, 200, x, None, torch.empty_like(x),
                                    ft.FT_FWD_PREFILL_STAGED | ft.FT_ACT_MXFP4)
        assert ei.value.code == ft.FT_E_OOM_DEVICE and "injected" in str(ei.value)
        torch.cuda.synchronize()
        for l in range(2):
            xb = ms.activations(w, l, 3, 200)
            gr = g.forward(l, xb, g.bias(l, 0), prefill=True, act=ft.FT_ACT_MXFP4)
            orr = o.forward(l, xb, ms.popularity_bias(w, l, 0), prefill=True)
            compare_call(gr, orr, 2, check_out=False)
            assert rel_l2(OF.bf16_from_bits(gr["out_bits"]), orr["out"]) <= 2e-3
    finally:
        g.close()


def test_zero_token_calls_change_nothing():
    """Calls with no tokens (decode, a staged prefill layer, the no-alloc entry
    point) return FT_OK and change nothing: the output buffer, the counters and
    the slot table stay as they were, a staged prefill does not start, and the
    next calls still match the oracle, which never saw the empty calls."""
    import torch

    import lru_expert_cache_amd as ft
    from tests.moe_case import GpuLayerStack, compare_call, compare_table

    w = _small(109, 2, 256, 128, 8, 2, [MX, F8], 6)
    g = GpuLayerStack(w)
    o = OracleLayerStack(w, pool_slots=g.C)
    try:
        def calls(step):
            for l in range(w.num_layers):
                x = ms.activations(w, l, step, 5)
                compare_call(g.forward(l, x, g.bias(l, step)), o.forward(l, x, ms.popularity_bias(w, l, 0)),
                             w.top_k)

        calls(0)
        st0 = ft.ft_moe_pool_stats(g.pool)
        x = torch.zeros((1, w.hidden), dtype=torch.int16, device=g.dev)
        out = torch.full((1, w.hidden), 0x1234, dtype=torch.int16, device=g.dev)
        for l in range(w.num_layers):
            assert ft.ft_moe_layer_forward(g.pool, l, 0, x, None, out, ft.FT_FWD_DECODE) == ft.FT_OK
            assert ft.ft_moe_layer_forward(g.pool, l, 0, x, None, out, ft.FT_FWD_PREFILL_STAGED) == ft.FT_OK
            assert ft.ft_moe_layer_forward_noalloc(g.pool, l, 0, x, None, out, ft.FT_FWD_DECODE) == ft.FT_OK
        torch.cuda.synchronize()
        assert bool((out == 0x1234).all())
        assert ft.ft_moe_pool_stats(g.pool) == st0
        compare_table(g, o)
        calls(1)  # decode still allowed: no prefill chunk was started
        compare_table(g, o)
    finally:
        g.close()
