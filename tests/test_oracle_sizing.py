"""Pins for oracle/sizing.py: the figures the pages print for their own sizing
arithmetic (tests/golden/pages_sizing.txt), and the bits per weight of the
generated blob layouts."""

import os

import pytest

import moe_synth as ms
from oracle import sizing as S

NVFP4_BITS = S.block_scaled_bits(4, 8, 16)


def _cases():
    path = os.path.join(os.path.dirname(__file__), "golden", "pages_sizing.txt")
    rows = [l.strip() for l in open(path) if l.strip() and not l.startswith("#")]
    return [[t.strip() for t in r.split(";")] for r in rows]


def _computed():
    copy_s = S.prefill_copy_seconds(150e9, 55.6e9)
    return {
        "ram_284b_4bit": S.weight_bytes(284e9, 4),
        "ram_284b_nvfp4": S.weight_bytes(284e9, NVFP4_BITS),
        "ram_753b_nvfp4": S.weight_bytes(753e9, NVFP4_BITS),
        "ram_35b_4p5bit": S.weight_bytes(35e9, 4.5),
        "copy_s_per_chunk": copy_s,
        "prefill_tok_s": S.prefill_tokens_per_s(8192, copy_s),
        "chunks_100k": S.prefill_chunks(100000, 8192),
        "ttft_100k": S.prefill_seconds(100000, 8192, 150e9, 55.6e9),
        "ttft_100k_pcie4": S.prefill_seconds(100000, 8192, 150e9, 27.8e9),
    }


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c[0])
def test_pages_printed_figures(case):
    name, _, printed, how = case
    got = _computed()[name]
    want = float(printed)
    if how == "exact":
        assert got == want
    elif how == "above":
        assert got > want
    else:
        kind, tol = how.split()
        err = abs(got - want) / want if kind == "rel" else abs(got - want)
        assert err <= float(tol), (name, got, want)


def test_every_fixture_row_is_computed():
    assert sorted(c[0] for c in _cases()) == sorted(_computed())


def test_bits_per_weight_of_the_layouts():
    # NVFP4 is 4.5 bits per weight (plus 12 bytes of per-matrix fp32 scales),
    # MXFP4 4.25 and FP8 with a fp32 scale per 128 weights 8.25
    H, I = 7168, 2048
    n = 3 * H * I
    assert (ms.expert_bytes(ms.FMT_NVFP4, H, I) - 12) * 8 / n == NVFP4_BITS == 4.5
    assert ms.expert_bytes(ms.FMT_MXFP4, H, I) * 8 / n == S.block_scaled_bits(4, 8, 32)
    assert ms.expert_bytes(ms.FMT_FP8_B128, H, I) * 8 / n == S.block_scaled_bits(8, 32, 128)


def test_prefill_rate_of_the_qwen_shape():
    # the formula applied to the Qwen-35B-A3B-shaped stack: 48 layers x 128
    # experts x 2,506,752 bytes = 15.40 GB per chunk; at 55.6 GB/s a 4,096-token
    # chunk takes 0.277 s, i.e. about 14.8k tokens/s while the copy is the bottleneck
    eb = 48 * 128 * ms.expert_bytes(ms.FMT_MXFP4, 2048, 768)
    assert eb == 15_401_484_288
    t = S.prefill_copy_seconds(eb, 55.6e9)
    assert abs(t - 0.2770) < 1e-3
    assert abs(S.prefill_tokens_per_s(4096, t) - 14787) < 10
