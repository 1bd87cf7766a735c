"""Pins for oracle/mode.py: hand-worked decisions in exact fractions, the
balance that defines the hybrid share, the fused bound, and the case of a host
far slower than the PCIe link."""

from fractions import Fraction as Fr

import numpy as np
from hypothesis import given, settings, strategies as st

from oracle.mode import FUSED, HYBRID, OFFLOAD, choose_mode

MX, NV, F8 = 1, 2, 3
INF = float("inf")


def test_cpu_twice_as_fast_as_pcie_takes_two_thirds():
    # b = 2.5 MB; PCIe 50 GB/s -> 50 us; device FFN negligible; host 100 GB/s -> 25 us
    r = choose_mode([MX], {MX: 2.5e6}, {MX: 50e9}, {MX: INF}, {MX: 100e9}, pool_slots=10, num_experts=128)
    assert r["mode"] == HYBRID
    assert abs(r["share"] - 2 / 3) < 1e-15
    assert abs(r["t_stream"] - 50e-6) < 1e-18 and abs(r["t_cpu"] - 25e-6) < 1e-18


def test_slow_host_gives_offload():
    # the machine measured here: host expert path 0.58 GB/s against 55.4 GB/s over PCIe
    r = choose_mode([MX] * 48, {MX: 2506752.0}, {MX: 55.4e9}, {MX: 4.0e12}, {MX: 0.58e9}, 1843, 128)
    assert r["mode"] == OFFLOAD and r["share"] == 0.0


def test_equal_cost_is_not_hybrid():
    # the host must be strictly faster
    r = choose_mode([MX], {MX: 1e6}, {MX: 2e9}, {MX: 2e9}, {MX: 1e9}, 4, 16)
    assert r["t_cpu"] == r["t_stream"] == 1e-3
    assert r["mode"] == OFFLOAD


def test_device_ffn_time_counts_on_the_streaming_side():
    # PCIe alone (1 ms) beats the host (1.25 ms); with the device FFN (0.5 ms) it does not
    base = dict(expert_bytes={MX: 1e6}, h2d={MX: 1e9}, cpu={MX: 0.8e9}, pool_slots=4, num_experts=16)
    r_fast = choose_mode([MX], gpu={MX: INF}, **base)
    r_slow = choose_mode([MX], gpu={MX: 2e9}, **base)
    assert r_fast["mode"] == OFFLOAD
    assert r_slow["mode"] == HYBRID
    # 1.5 ms streamed vs 1.25 ms on the host: share = 1.5 / 2.75 = 6/11
    assert abs(r_slow["share"] - 6 / 11) < 1e-15


def test_mixed_formats_sum_over_layers():
    # layer 0 MXFP4 (2 MB), layer 1 FP8 (4 MB)
    eb = {MX: 2e6, F8: 4e6}
    h2d = {MX: 1e9, F8: 2e9}      # 2 ms + 2 ms
    gpu = {MX: 4e9, F8: 4e9}      # 0.5 ms + 1 ms
    cpu = {MX: 0.5e9, F8: 8e9}    # 4 ms + 0.5 ms
    r = choose_mode([MX, F8], eb, h2d, gpu, cpu, pool_slots=3, num_experts=8)
    assert abs(r["t_stream"] - 5.5e-3) < 1e-15 and abs(r["t_cpu"] - 4.5e-3) < 1e-15
    assert r["mode"] == HYBRID and abs(r["share"] - 5.5 / 10) < 1e-15
    # per layer the host is faster only on the FP8 layer; the model-wide sum decides
    r1 = choose_mode([MX, MX, F8], eb, h2d, gpu, cpu, pool_slots=3, num_experts=8)
    assert r1["mode"] == OFFLOAD


def test_fused_when_every_expert_has_a_slot():
    for C in (48 * 128, 48 * 128 + 7):
        r = choose_mode([MX] * 48, {MX: 2.5e6}, {MX: 50e9}, {MX: INF}, {MX: 500e9}, C, 128)
        assert r["mode"] == FUSED and r["share"] == 0.0
    r = choose_mode([MX] * 48, {MX: 2.5e6}, {MX: 50e9}, {MX: INF}, {MX: 500e9}, 48 * 128 - 1, 128)
    assert r["mode"] == HYBRID


@settings(max_examples=200, deadline=None)
@given(h=st.floats(1e8, 1e11), g=st.floats(1e9, 1e13), c=st.floats(1e7, 1e12), b=st.floats(1e4, 1e8))
def test_hybrid_share_balances_the_two_paths(h, g, c, b):
    r = choose_mode([NV], {NV: b}, {NV: h}, {NV: g}, {NV: c}, pool_slots=1, num_experts=2)
    ts, tc = Fr(b) / Fr(h) + Fr(b) / Fr(g), Fr(b) / Fr(c)
    if tc < ts:
        assert r["mode"] == HYBRID
        assert 0.5 < r["share"] < 1.0
        # both paths finish together on a step of m misses
        m = 1000
        cpu_time = m * r["share"] * float(tc)
        pcie_time = m * (1 - r["share"]) * float(ts)
        assert abs(cpu_time - pcie_time) <= 1e-9 * max(cpu_time, pcie_time)
        # and the overlapped step beats either path alone
        assert cpu_time < m * float(min(tc, ts))
    else:
        assert r["mode"] == OFFLOAD and r["share"] == 0.0


def test_balanced_share_is_reported_for_every_mode():
    # one layer, b = 1 byte: streamed 1/3 + 1/6 = 1/2 s, host 1 s -> offload,
    # and the split at which both paths finish together is (1/2) / (3/2) = 1/3
    r = choose_mode([MX], {MX: 1.0}, {MX: 3.0}, {MX: 6.0}, {MX: 1.0}, 1, 2)
    assert r["mode"] == OFFLOAD and r["share"] == 0.0
    assert abs(r["balanced_share"] - 1 / 3) < 1e-15
    # m misses split at that share: m/3 on the host take m/3 s, 2m/3 streamed take m/3 s
    m = 9.0
    assert abs(m * r["balanced_share"] * r["t_cpu"] - m * (1 - r["balanced_share"]) * r["t_stream"]) < 1e-12
    # a hybrid decision reports the same split as its share
    r2 = choose_mode([MX], {MX: 1.0}, {MX: 3.0}, {MX: 6.0}, {MX: 4.0}, 1, 2)
    assert r2["mode"] == HYBRID and r2["share"] == r2["balanced_share"] == 0.5 / 0.75
