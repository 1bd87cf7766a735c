"""Sizing arithmetic of the offloaded MoE layer: weight bytes and prefill
copy time.

TEST INFRASTRUCTURE (oracle).  The pages estimate the host RAM an offloaded
model needs from its parameter count and bits per weight, with NVFP4 at 4
bits plus an 8-bit scale per 16 weights (devpik article "FreeToken: Run
Frontier MoE Models on Your Own GPU, and the RAM It Takes", section "The Real
Requirement Is System RAM").  For prefill they state that each MoE layer
copies all of its experts per chunk, so the copy time of a chunk is about the
expert bytes divided by the host-to-device bandwidth, and derive a token rate
and a time to first token from it (same article, section "Long Prompts Are the
Bottleneck").  These functions restate that arithmetic; the benchmark uses the
same formula to predict the staged-prefill rate of a layer stack from its
measured copy bandwidth.

Pins (tests/test_oracle_sizing.py, tests/golden/pages_sizing.txt): every
figure the two sections print, within the rounding their wording implies, and
the per-expert bytes of the generated layouts.
"""

from __future__ import annotations

import math


def block_scaled_bits(elem_bits: float, scale_bits: float, block: int) -> float:
    """Bits per weight of a block-scaled format: element bits plus one shared
    scale per `block` elements (NVFP4: 4 + 8/16 = 4.5; MXFP4: 4 + 8/32)."""
    return float(elem_bits) + float(scale_bits) / float(block)


def weight_bytes(params: float, bits_per_weight: float) -> float:
    """Bytes of `params` weights stored at `bits_per_weight`."""
    return float(params) * float(bits_per_weight) / 8.0


def prefill_copy_seconds(expert_bytes: float, h2d_bytes_per_s: float) -> float:
    """Copy time of one prefill chunk: every expert of every MoE layer crosses
    the link once, so time = expert bytes / bandwidth."""
    return float(expert_bytes) / float(h2d_bytes_per_s)


def prefill_tokens_per_s(chunk_tokens: int, copy_seconds: float) -> float:
    """Token rate of prefill while the copy is the bottleneck."""
    return float(chunk_tokens) / float(copy_seconds)


def prefill_chunks(context_tokens: int, chunk_tokens: int) -> int:
    """Chunks needed to read a context (the last chunk may be partial)."""
    return int(math.ceil(int(context_tokens) / int(chunk_tokens)))


def prefill_seconds(context_tokens: int, chunk_tokens: int, expert_bytes: float, h2d_bytes_per_s: float) -> float:
    """Copy-bound time to read a whole context: chunks x copy time per chunk."""
    return prefill_chunks(context_tokens, chunk_tokens) * prefill_copy_seconds(expert_bytes, h2d_bytes_per_s)
