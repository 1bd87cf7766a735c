"""The one-time choice between the fused, offload and hybrid strategies.

TEST INFRASTRUCTURE (oracle).  What the pages fix: before serving, the engine
runs a benchmark on the machine at hand -- real GPU kernels for each
quantisation format in the model, the host's compute speed and the PCIe
transfer speed -- and picks hybrid when the host computes an expert's output
sooner than its weights could be streamed over PCIe, offload otherwise; the
choice is made once per model and machine (mindstudio article "FreeToken
Explained: Run 290B+ MoE Models on One Gaming GPU", section "How does the
benchmark decide between hybrid and offload mode?").  When every expert fits
in VRAM the fused strategy keeps them all resident (devpik article "FreeToken:
Run Frontier MoE Models on Your Own GPU, and the RAM It Takes", section "Why a
Huge MoE Model Fits on One Consumer GPU").  Hybrid splits each step's misses
between the two paths, overlapped, from the measured bandwidths (same section).

Readings where the pages stop short:

* Rates are expert-weight bytes per second, one per format f present:
  h2d[f] (pinned host to device), gpu[f] (the device's grouped expert FFN at
  the measured rows per expert) and cpu[f] (the host expert path at the same
  rows).
* Cost of one miss in every layer: streamed, the copy then the device FFN,
  t_stream = sum over layers of b/h2d[f] + b/gpu[f]; on host cores,
  t_cpu = sum over layers of b/cpu[f] (b = the layer's expert bytes).  The
  activation rows a host expert exchanges with the device are left out (at
  most a few percent of an expert's bytes at decode batch sizes).
* fused when the pool has a slot for every (layer, expert) key; otherwise
  hybrid when t_cpu < t_stream strictly, else offload.
* Hybrid share: the fraction of a step's misses sent to the host such that
  both paths finish together, m*share*t_cpu = m*(1 - share)*t_stream, i.e.
  share = t_stream / (t_stream + t_cpu).  offload and fused use share 0.  The
  pages' "cpu" strategy is share 1, chosen by the user, never by this rule.
  The same split (balanced_share) is reported for every mode, for a caller
  that picks the hybrid strategy itself (a workload whose configuration names
  a host/PCIe split uses it).

Pins: tests/test_oracle_mode.py (hand-worked cases in exact fractions, the
balance property, the fused bound, the measured-machine case).
"""

from __future__ import annotations

from typing import Dict, Sequence

OFFLOAD, HYBRID, FUSED = 0, 1, 2


def choose_mode(layer_fmt: Sequence[int], expert_bytes: Dict[int, float], h2d: Dict[int, float],
                gpu: Dict[int, float], cpu: Dict[int, float], pool_slots: int, num_experts: int) -> dict:
    """layer_fmt: the format of each layer; the dicts map a format to its
    expert bytes and measured rates (bytes per second)."""
    t_stream = 0.0
    t_cpu = 0.0
    for f in layer_fmt:
        b = expert_bytes[f]
        t_stream += b / h2d[f] + b / gpu[f]
        t_cpu += b / cpu[f]
    balanced = t_stream / (t_stream + t_cpu)
    if pool_slots >= len(layer_fmt) * num_experts:
        mode, share = FUSED, 0.0
    elif t_cpu < t_stream:
        mode, share = HYBRID, t_stream / (t_stream + t_cpu)
    else:
        mode, share = OFFLOAD, 0.0
    return dict(mode=mode, share=share, t_stream=t_stream, t_cpu=t_cpu, balanced_share=balanced)
