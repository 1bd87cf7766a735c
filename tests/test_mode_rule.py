"""The library's strategy decision (ft_moe_decide_mode, host code in the
C-ABI library, no device work) against the oracle's rule on the same rates:
mindstudio "FreeToken Explained: Run 290B+ MoE Models on One Gaming GPU",
section "How does the benchmark decide between hybrid and offload mode?"."""

import math

import numpy as np
import pytest

from oracle.mode import choose_mode


def _lib():
    import lru_expert_cache_amd as ft

    try:
        ft.lib()
    except Exception as e:  # pragma: no cover - the build step makes it
        pytest.skip(f"library not built: {e}")
    return ft


def _report(rng, fmts, E, C):
    rep = dict(tokens=16, layers=[0, 0, 0, 0], expert_bytes=[0.0] * 4, h2d_bytes_per_s=[0.0] * 4,
               gpu_bytes_per_s=[0.0] * 4, cpu_bytes_per_s=[0.0] * 4, pool_slots=C, all_experts=len(fmts) * E)
    for f in set(fmts):
        rep["layers"][f] = fmts.count(f)
        rep["expert_bytes"][f] = float(rng.integers(50_000, 40_000_000))
        rep["h2d_bytes_per_s"][f] = float(10 ** rng.uniform(9, 11))
        rep["gpu_bytes_per_s"][f] = float(10 ** rng.uniform(11, 13))
        rep["cpu_bytes_per_s"][f] = float(10 ** rng.uniform(8.5, 11.5))
    return rep


def test_library_rule_matches_oracle():
    ft = _lib()
    rng = np.random.default_rng(5)
    seen = set()
    for case in range(400):
        L = int(rng.integers(1, 10))
        fmts = [int(rng.integers(1, 4)) for _ in range(L)]
        E = int(rng.integers(2, 300))
        C = int(rng.integers(1, L * E + 3))
        rep = _report(rng, fmts, E, C)
        got = ft.ft_moe_decide_mode(rep)
        f = lambda key: {g: rep[key][g] for g in set(fmts)}
        want = choose_mode(fmts, f("expert_bytes"), f("h2d_bytes_per_s"), f("gpu_bytes_per_s"), f("cpu_bytes_per_s"),
                           C, E)
        assert math.isclose(got["t_stream"], want["t_stream"], rel_tol=1e-12)
        assert math.isclose(got["t_cpu"], want["t_cpu"], rel_tol=1e-12)
        assert math.isclose(got["balanced_share"], want["balanced_share"], rel_tol=1e-12)
        # the decision is taken on the same totals unless they tie within rounding
        if abs(want["t_cpu"] - want["t_stream"]) > 1e-9 * want["t_stream"]:
            assert got["mode"] == want["mode"], case
            assert math.isclose(got["share"], want["share"], rel_tol=1e-12, abs_tol=0.0)
        seen.add(got["mode"])
    assert seen == {0, 1, 2}


def test_library_rule_rejects_missing_rates():
    ft = _lib()
    rep = _report(np.random.default_rng(1), [1, 1], 8, 4)
    rep["cpu_bytes_per_s"][1] = 0.0
    with pytest.raises(ft.FtError):
        ft.ft_moe_decide_mode(rep)
