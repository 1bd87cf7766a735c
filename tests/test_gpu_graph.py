"""Graph-compatible decode: a decode step captured into a HIP graph and
replayed must give, replay after replay, the outputs, slot table and counters
of the same calls made eagerly, with eager work (input copies, an eager decode
call) between the replays.  The pages list graph-compatible execution among
the runtime's mechanisms (dev.to "FreeToken uses bandwidth-adaptive CPU-GPU
co-execution on your desktop", section "What the project says it does")."""

import numpy as np
import pytest

import moe_synth as ms
from oracle.layer import OracleLayerStack

pytestmark = pytest.mark.gpu

MX, NV, F8 = ms.FMT_MXFP4, ms.FMT_NVFP4, ms.FMT_FP8_B128


def _w():
    # 3 layers of 16 experts, top-4, 24 slots: a 4-token call (16 pairs) is one wave
    return ms.Workload(130, "small-130", 3, 256, 256, 16, 4, (MX, F8, NV), 24, (4,), 4, "decode", None, None,
                       True, False, None)


def _qwen_four_layers():
    # the Qwen-A3B-shaped layers (H 2048, I 768, 128 MXFP4 experts, top-8), four of
    # them over 154 slots (30% of their keys): a 16-token call (128 pairs) is one wave
    w0 = ms.workload("qwen-a3b-decode")
    return w0.with_(num_layers=4, layer_fmt=w0.layer_fmt[:4], pool_slots=154)


def test_captured_decode_step_replays_like_eager_calls():
    _replay_case(_w(), 4, 6, big_tokens=7)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("T", [16, 1])
def test_captured_qwen_a3b_step_replays_like_eager_calls(T):
    """The same at the Qwen-A3B layer size, in the launch shapes of the
    benchmark's graph replays (batch 16 and 1)."""
    # enough steps that the calls' distinct experts outnumber the slots (evictions)
    _replay_case(_qwen_four_layers(), T, 4 if T > 1 else 8, big_tokens=0)


def _replay_case(w, T, steps, big_tokens):
    import torch

    from tests.moe_case import GpuLayerStack, compare_table
    import lru_expert_cache_amd as ft

    L, H = w.num_layers, w.hidden
    store = ms.BlobStore(w)
    ga, ge = GpuLayerStack(w, store=store), GpuLayerStack(w, store=store)  # graph-driven, eager
    o = OracleLayerStack(w, pool_slots=ga.C, blob_fn=lambda l, e: store.expert(l, e))
    dev = ga.dev
    s = torch.cuda.Stream(dev)
    try:
        ft.ft_moe_reserve(ga.pool, T)
        xin = torch.zeros((L, T, H), dtype=torch.int16, device=dev)
        outs = torch.zeros((L, T, H), dtype=torch.int16, device=dev)
        big = torch.zeros((max(big_tokens, 1), H), dtype=torch.int16, device=dev)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for l in range(L):
                ft.ft_moe_layer_forward(ga.pool, l, T, xin[l], None, outs[l], ft.FT_FWD_DECODE, s, None)
            if big_tokens:
                # 7 tokens x top-4 > 24 slots: a call the host splits into waves cannot be
                # captured; it is rejected and nothing is captured for it
                with pytest.raises(ft.FtError):
                    ft.ft_moe_layer_forward(ga.pool, 0, big_tokens, big, None, big, ft.FT_FWD_DECODE, s, None)
        torch.cuda.synchronize()
        assert int(outs.abs().sum().item()) == 0, "capturing ran the calls"

        for step in range(steps):
            xs = [ms.activations(w, l, step, T) for l in range(L)]
            xin.copy_(torch.from_numpy(np.stack(xs).view(np.int16)))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for l in range(L):
                want = ge.forward(l, xs[l], None)
                assert np.array_equal(outs[l].cpu().numpy().view(np.uint16), want["out_bits"]), (step, l)
                o.forward(l, xs[l], None, outputs=False)
            if step % 2 == 1:
                # an eager call on both pools between replays
                xe = ms.activations(w, 1, 100 + step, T)
                ga.forward(1, xe, None)
                ge.forward(1, xe, None)
                o.forward(1, xe, None, outputs=False)
        torch.cuda.synchronize()
        ka, la, ca = ft.ft_moe_pool_table(ga.pool, ga.C)
        ke, le, ce = ft.ft_moe_pool_table(ge.pool, ge.C)
        assert np.array_equal(ka, ke) and np.array_equal(la, le) and ca == ce
        compare_table(ga, o)
        sa, se = ft.ft_moe_pool_stats(ga.pool), ft.ft_moe_pool_stats(ge.pool)
        # copy time is measured (also inside replays, on the device clock), not computed
        assert sa.pop("copy_ms") > 0 and se.pop("copy_ms") > 0
        assert sa == se, (sa, se)
        for key in ("pair_hits", "pair_misses", "expert_hits", "expert_misses", "evictions", "bytes_h2d", "calls"):
            assert sa[key] == o.stats[key], (key, sa[key], o.stats[key])
        assert sa["evictions"] > 0
    finally:
        ga.close()
        ge.close()
