"""CPU-side checks of the C ABI: the library loads, exports every function the
header declares, and rejects invalid configurations before touching a GPU."""

import ctypes
import os
import re

import numpy as np
import pytest

import lru_expert_cache_amd as ft

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    src = open(os.path.join(ROOT, "include", "ftmoe.h")).read()
    return sorted(set(re.findall(r"\b(ft_moe_[a-z_]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert _header_functions() == sorted(ft.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = ft.lib()
    for name in _header_functions():
        assert hasattr(L, name), name


def _c_layout(structs):
    """Sizes and field offsets of header structs, as gcc lays them out."""
    import shutil
    import subprocess
    import tempfile

    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "ftmoe.h"', "int main(void) {"]
    for st, fields in structs.items():
        lines.append(f'  printf("{st} size %zu\\n", sizeof({st}));')
        for f in fields:
            lines.append(f'  printf("{st} {f} %zu\\n", offsetof({st}, {f}));')
    lines += ["  return 0;", "}"]
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "l.c"), os.path.join(d, "l")
        open(src, "w").write("\n".join(lines) + "\n")
        subprocess.run([cc, "-I", os.path.join(ROOT, "include"), src, "-o", exe], check=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    return {tuple(l.split()[:2]): int(l.split()[2]) for l in out.splitlines()}


def test_struct_layouts_match_header():
    # every struct the binding declares, field by field, against the C compiler
    structs = {"ft_moe_config": ft.ft_moe_config, "ft_moe_weights": ft.ft_moe_weights,
               "ft_moe_trace": ft.ft_moe_trace, "ft_moe_stats": ft.ft_moe_stats,
               "ft_moe_mode_report": ft.ft_moe_mode_report, "ft_moe_profile": ft.ft_moe_profile,
               "ft_moe_rebalance_report": ft.ft_moe_rebalance_report}
    c = _c_layout({n: [f for f, _ in t._fields_] for n, t in structs.items()})
    for n, t in structs.items():
        assert c[(n, "size")] == ctypes.sizeof(t), n
        for f, _ in t._fields_:
            assert c[(n, f)] == getattr(t, f).offset, (n, f)


def test_profile_stages_match_header():
    # the binding's stage names follow the header's FT_STAGE_* order up to FT_STAGE_COUNT
    src = open(os.path.join(ROOT, "include", "ftmoe.h")).read()
    body = re.search(r"enum\s*\{\s*(FT_STAGE_ROUTER[^}]*)\}", src).group(1)
    names = [n.strip().split("=")[0].strip() for n in re.sub(r"/\*.*?\*/", "", body, flags=re.S).split(",")]
    names = [n for n in names if n]
    assert names[-1] == "FT_STAGE_COUNT"
    assert [n[len("FT_STAGE_"):].lower() for n in names[:-1]] == ft.FT_STAGES
    assert ctypes.sizeof(ft.ft_moe_profile) == 4 * 8 * (len(names) - 1)


def _cfg(**kw):
    d = dict(num_layers=1, hidden=256, inter=128, num_experts=16, top_k=2, layer_fmt=[1], pool_slots=8)
    d.update(kw)
    return ft.make_config(**d)


@pytest.mark.parametrize("kw", [dict(hidden=200), dict(inter=100), dict(num_experts=600), dict(top_k=17),
                                dict(top_k=20, num_experts=16), dict(pool_slots=1), dict(layer_fmt=[7]),
                                dict(hidden=16384), dict(hybrid_cpu_share=1.5)])
def test_invalid_config_rejected_before_gpu(kw):
    cfg = _cfg(**kw)
    blobs = [np.zeros(16, np.uint8)] * (cfg.num_layers * cfg.num_experts)
    rw = np.zeros((cfg.num_layers, cfg.num_experts, cfg.hidden), np.float32)
    with pytest.raises(ft.FtError) as ei:
        ft.ft_moe_init_pool(cfg, blobs, rw)
    assert ei.value.code == ft.FT_E_INVALID
    assert ft.ft_moe_last_error()


def test_null_arguments_rejected():
    L = ft.lib()
    assert L.ft_moe_init_pool(None, None, None) == ft.FT_E_INVALID
    assert L.ft_moe_layer_forward(None, 0, 1, None, None, None, 0, None, None) == ft.FT_E_INVALID
    st = ft.ft_moe_stats()
    assert L.ft_moe_pool_stats(None, -1, ctypes.byref(st), 0) == ft.FT_E_INVALID
    assert L.ft_moe_set_hybrid_share(None, 0.5) == ft.FT_E_INVALID
    L.ft_moe_destroy_pool(None)


def test_mfma_rate_rejects_bad_arguments_before_gpu():
    L = ft.lib()
    r = ctypes.c_double(0.0)
    assert L.ft_moe_mfma_rate(5, 10, None, ctypes.byref(r)) == ft.FT_E_INVALID
    assert L.ft_moe_mfma_rate(-1, 10, None, ctypes.byref(r)) == ft.FT_E_INVALID
    assert L.ft_moe_mfma_rate(0, 0, None, ctypes.byref(r)) == ft.FT_E_INVALID
    assert L.ft_moe_mfma_rate(0, 10, None, None) == ft.FT_E_INVALID
    with pytest.raises(ft.FtError):
        ft.ft_moe_mfma_rate(6)


def test_pinned_allocation_failure_is_reported(monkeypatch):
    monkeypatch.setenv("FT_MOE_FAULT", "pinned_alloc")
    cfg = _cfg()
    blobs = [np.zeros(52_224, np.uint8)] * 16
    rw = np.zeros((1, 16, 256), np.float32)
    with pytest.raises(ft.FtError) as ei:
        ft.ft_moe_init_pool(cfg, blobs, rw)
    assert ei.value.code == ft.FT_E_OOM_PINNED
