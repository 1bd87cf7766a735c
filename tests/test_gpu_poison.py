"""Debug modes against races and damaged slots.

Poison-on-evict (FT_MOE_POISON at pool creation): every slot is filled with
0xFF bytes -- NaN block scales in every format -- just before a copy into it.
A read of a slot that races its copy (an FFN of this call running before the
copy, or of the previous call after it) would then produce NaN instead of
plausible stale weights.  With poison on, device-driven decode, host-driven
decode, the hybrid split and hit-D2D prefill must stay bit-identical to poison
off (and to the oracle's decisions).

Slot checksums (FT_MOE_DEBUG_CHECKSUM): before an FFN reads a slot, a kernel
recomputes its checksum against the key's blob; the same paths run clean, and a
copy damaged on purpose (FT_MOE_FAULT=corrupt:<n>, forced from the host) is
reported with its key.  FT_MOE_LOG=<n> prints a counters line every n calls."""

import os

import numpy as np
import pytest

import moe_synth as ms
from oracle.layer import OracleLayerStack

pytestmark = pytest.mark.gpu

MX, NV, F8 = ms.FMT_MXFP4, ms.FMT_NVFP4, ms.FMT_FP8_B128


def _small(cfg_id, L, H, I, E, k, fmts, C, shared=False, alpha=None):
    return ms.Workload(cfg_id, f"small-{cfg_id}", L, H, I, E, k, tuple(fmts), C, (8,), 4, "decode", alpha, None,
                       shared, False, None)


ENV_KEYS = ("FT_MOE_POISON", "FT_MOE_DECODE_PATH", "FT_MOE_DEBUG_CHECKSUM", "FT_MOE_FAULT", "FT_MOE_LOG")


def _pool(w, poison, share=0.0, host_path=False, env=None):
    """A pool created with the given debug environment (read at creation)."""
    from tests.moe_case import GpuLayerStack

    saved = {k: os.environ.get(k) for k in ENV_KEYS}
    try:
        for k in ENV_KEYS:
            os.environ.pop(k, None)
        if poison:
            os.environ["FT_MOE_POISON"] = "1"
        if host_path:
            os.environ["FT_MOE_DECODE_PATH"] = "host"
        os.environ.update(env or {})
        return GpuLayerStack(w, share=share)
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


@pytest.mark.parametrize("mode", ["poison", "checksum"])
@pytest.mark.parametrize("path", ["device", "host", "hybrid", "prefill-hit-d2d"])
def test_debug_mode_changes_nothing(path, mode):
    from tests.moe_case import compare_call, compare_table
    import lru_expert_cache_amd as ft

    w = _small(150, 3, 256, 256, 12, 2, [MX, F8, NV], 30, shared=True)  # uniform routing: evicts
    share = 0.4 if path == "hybrid" else 0.0
    host = path in ("host", "hybrid")
    plain = _pool(w, False, share, host)
    pois = _pool(w, mode == "poison", share, host, env={"FT_MOE_DEBUG_CHECKSUM": "1"} if mode == "checksum" else None)
    o = OracleLayerStack(w, pool_slots=plain.C, share=share)
    try:
        for rnd in range(3):
            for s, T in ((0, 7), (1, 12), (2, 3)):
                for l in range(w.num_layers):
                    x = ms.activations(w, l, 10 * rnd + s, T)
                    a = plain.forward(l, x, plain.bias(l, 0))
                    b = pois.forward(l, x, pois.bias(l, 0))
                    compare_call(a, o.forward(l, x, ms.popularity_bias(w, l, 0)), w.top_k)
                    assert np.array_equal(a["out_bits"], b["out_bits"]), (path, rnd, s, l)
                    for key in ("sel", "w", "slot", "flag", "row"):
                        assert np.array_equal(a[key], b[key]), key
            if path == "prefill-hit-d2d":
                for l in range(w.num_layers):
                    x = ms.activations(w, l, 100 + rnd, 40)
                    a = plain.forward(l, x, plain.bias(l, 0), prefill=True, hit_d2d=True)
                    b = pois.forward(l, x, pois.bias(l, 0), prefill=True, hit_d2d=True)
                    compare_call(a, o.forward(l, x, ms.popularity_bias(w, l, 0), prefill=True, hit_d2d=True),
                                 w.top_k)
                    assert np.array_equal(a["out_bits"], b["out_bits"]), (path, rnd, "chunk", l)
        compare_table(plain, o)
        compare_table(pois, o)
        sa, sb = ft.ft_moe_pool_stats(plain.pool), ft.ft_moe_pool_stats(pois.pool)
        sa.pop("copy_ms")
        sb.pop("copy_ms")
        assert sa == sb
        assert sb["evictions"] > 0 and (sb["cpu_misses"] > 0) == (path == "hybrid")
    finally:
        plain.close()
        pois.close()


def test_poison_on_evict_with_calls_on_three_streams_and_no_host_wait():
    """The device-driven pool with poison on, its calls spread over three
    streams with no host synchronisation between them (the library orders
    calls on different streams itself): outputs equal those of synchronous
    calls on a pool without poison."""
    import torch
    import lru_expert_cache_amd as ft

    w = _small(151, 3, 256, 256, 12, 3, [MX, F8, NV], 20, shared=True)
    plain = _pool(w, False)
    pois = _pool(w, True)
    dev = pois.dev
    streams = [None, torch.cuda.Stream(dev), torch.cuda.Stream(dev)]
    calls = [(6, 0), (1, 1), (5, 2), (2, 3), (6, 4), (3, 5), (4, 6)]
    try:
        # reference outputs first (these calls synchronise the device)
        wants = [plain.forward(l, ms.activations(w, l, s, T), plain.bias(l, 0))["out_bits"]
                 for T, s in calls for l in range(w.num_layers)]
        inputs = [(T, l, torch.from_numpy(ms.activations(w, l, s, T).view(np.int16)).to(dev), pois.bias(l, 0))
                  for T, s in calls for l in range(w.num_layers)]
        torch.cuda.synchronize()
        pending = []
        for i, (T, l, x, bias) in enumerate(inputs):
            out = torch.empty_like(x)
            ft.ft_moe_layer_forward(pois.pool, l, T, x, bias, out, ft.FT_FWD_DECODE, streams[i % 3], None)
            pending.append((wants[i], out))
        torch.cuda.synchronize()
        for want, out in pending:
            assert np.array_equal(out.cpu().numpy().view(np.uint16), want)
        sa, sb = ft.ft_moe_pool_stats(plain.pool), ft.ft_moe_pool_stats(pois.pool)
        sa.pop("copy_ms")
        sb.pop("copy_ms")
        assert sa == sb and sb["evictions"] > 0
    finally:
        plain.close()
        pois.close()


def test_checksum_reports_a_damaged_copy():
    """The third miss copy of the pool lands damaged (256 bytes overwritten,
    forced from the host): the call whose FFN would read it fails with the
    key and slot named, before any output is used."""
    import torch
    import lru_expert_cache_amd as ft

    w = _small(152, 2, 256, 256, 12, 2, [MX, NV], 20)
    g = _pool(w, False, env={"FT_MOE_DEBUG_CHECKSUM": "1", "FT_MOE_FAULT": "corrupt:3"})
    try:
        x = torch.from_numpy(ms.activations(w, 0, 0, 6).view(np.int16)).to(g.dev)
        with pytest.raises(ft.FtError) as ei:
            ft.ft_moe_layer_forward(g.pool, 0, 6, x, None, torch.empty_like(x), ft.FT_FWD_DECODE)
        assert ei.value.code == ft.FT_E_HIP and "checksum mismatch" in str(ei.value)
        stream, _ = ft.ft_moe_last_misses(g.pool)
        e3, s3 = stream[2]
        assert f"expert {e3}) in slot {s3}" in str(ei.value)
    finally:
        g.close()


def test_log_line_every_n_calls(capfd):
    import torch
    import lru_expert_cache_amd as ft

    w = _small(153, 2, 256, 128, 8, 2, [MX, MX], 16)
    g = _pool(w, False, env={"FT_MOE_LOG": "3"})
    try:
        for i in range(7):
            x = torch.from_numpy(ms.activations(w, i % 2, i, 4).view(np.int16)).to(g.dev)
            ft.ft_moe_layer_forward(g.pool, i % 2, 4, x, None, torch.empty_like(x), ft.FT_FWD_DECODE)
        torch.cuda.synchronize()
    finally:
        g.close()
    lines = [l for l in capfd.readouterr().err.splitlines() if l.startswith("ftmoe:")]
    assert len(lines) == 2 and lines[0].startswith("ftmoe: 3 calls") and lines[1].startswith("ftmoe: 6 calls")
