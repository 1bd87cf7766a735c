"""Pins for oracle/formats.py: code tables, rounding, MX quantiser, blob decode."""

import math
import os

import numpy as np
import pytest
import torch

import moe_synth as ms
from oracle import formats as F

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_e2m1_matches_ocp_table():
    rows = [l.split() for l in open(os.path.join(GOLD, "e2m1_ocp_table.txt")) if l.strip() and not l.startswith("#")]
    assert len(rows) == 16
    for code, val in rows:
        got = F.e2m1_value(int(code))
        assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val))
    assert F.E2M1_TABLE.max() == 6.0


def test_e4m3_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.E4M3_TABLE
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert nan.sum() == 2  # S.1111.111 only
    assert np.array_equal(ref[~nan], got[~nan])
    assert got[0x7E] == 448.0 and got[0x38] == 1.0 and got[0x01] == 2.0 ** -9


def test_e8m0_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = F.E8M0_TABLE
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(ref[:255], got[:255])
    assert got[127] == 1.0


def test_round_bf16_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    # ties, subnormals, the overflow edge and signed zeros
    extra = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -130, 2 ** -133, 3 * 2 ** -134,
                      3.3895313892515355e38, 3.4e38, 0.0, -0.0, 1e-45], np.float32)
    x = np.concatenate([x, extra])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = F.round_bf16(x.astype(np.float64))
    assert np.array_equal(np.isinf(ref), np.isinf(got))
    fin = np.isfinite(ref)
    assert np.array_equal(ref[fin], got[fin])


def test_round_bf16_rounds_once_from_fp64():
    # 1 + 2^-8 is a tie at bf16 precision; the extra 2^-30 puts the fp64 value
    # above it, so one rounding gives 1 + 2^-7.  Rounding through fp32 first
    # would lose the 2^-30 and give 1.0.
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert F.round_bf16(np.array([x]))[0] == 1.0 + 2.0 ** -7
    assert F.round_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0


def _nearest_grid_brute(v, grid_mags, mant_even):
    """Brute force: the nearest grid magnitude, ties to the code with even mantissa."""
    a = abs(v)
    best = None
    for mag, even in zip(grid_mags, mant_even):
        d = abs(a - mag)
        if best is None or d < best[0] - 1e-300 or (d == best[0] and even and not best[2]):
            best = (d, mag, even)
    return math.copysign(best[1], v) if best[1] != 0 else 0.0


def test_round_to_e2m1_brute_force():
    mags = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    even = [True, False, True, False, True, False, True, False]
    vals = np.concatenate([np.arange(-7, 7.0001, 0.125), np.random.default_rng(2).uniform(-6, 6, 2000)])
    got = F.round_to_element(vals, "e2m1")
    for v, g in zip(vals, got):
        exp = _nearest_grid_brute(v, mags, even) if abs(v) <= 6 else math.copysign(6, v)
        assert g == exp, (v, g, exp)


def test_round_to_e4m3_matches_torch_in_range():
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 0.01,
                        np.ldexp(rng.uniform(-1, 1, 5000), rng.integers(-12, 9, 5000))])
    v = v[np.abs(v) <= 448]
    v32 = v.astype(np.float32).astype(np.float64)  # torch casts from fp32
    ref = torch.from_numpy(v32).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.round_to_element(v32, "e4m3")
    assert np.array_equal(ref, got)


def test_mx_quantize_golden_blocks():
    n = 0
    for line in open(os.path.join(GOLD, "mx_quant_blocks.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        elem, vin, sexp, vout = [s.strip() for s in line.split(";")]
        vin = np.array([float(t) for t in vin.split()])
        vout = np.array([float(t) for t in vout.split()])
        deq, _, sbyte = F.mx_quantize(vin[None, :], elem)
        assert int(sbyte[0, 0]) - 127 == int(sexp)
        assert np.array_equal(deq[0], vout), (deq[0], vout)
        n += 1
    assert n == 4


@pytest.mark.parametrize("elem,vmax", [("e2m1", 6.0), ("e4m3", 448.0)])
def test_mx_quantize_properties(elem, vmax):
    rng = np.random.default_rng(7)
    v = rng.standard_normal((64, 256)) * np.exp(rng.uniform(-5, 5, (64, 1)))
    deq, el, sb = F.mx_quantize(v, elem)
    # idempotent
    deq2, _, _ = F.mx_quantize(deq, elem)
    assert np.array_equal(deq, deq2)
    # every element within the grid range, and the block max maps into the top binade
    assert np.abs(el).max() <= vmax
    blk = np.abs(el.reshape(64, 8, 32)).max(axis=-1)
    emax = F.ELEM[elem][3]
    assert (blk >= 2.0 ** emax).all()
    # relative error bounded by half an element ulp of the block max
    rel = np.abs(deq - v).reshape(64, 8, 32).max(-1) / np.abs(v).reshape(64, 8, 32).max(-1)
    mb = F.ELEM[elem][0]
    assert rel.max() <= 2.0 ** -mb


def _per_element_decode(fmt, blob, H, I):
    """Element-by-element decode following the written blob layout, for small shapes."""
    cod, sca, ts, _ = F.blob_offsets(fmt, H, I)
    shapes = [(I, H), (I, H), (H, I)]
    g = [1.0] * 3
    if ts is not None:
        g = list(np.frombuffer(bytes(blob[ts:ts + 12]), "<f4").astype(float))
    out = []
    for m, (R, K) in enumerate(shapes):
        W = np.zeros((R, K))
        co, so = cod[m][0], sca[m][0]
        for r in range(R):
            for c in range(K):
                i = r * K + c
                if fmt == F.FMT_FP8_B128:
                    code = int(blob[co + i])
                    el = F.e4m3fn_value(code)
                    s = float(np.frombuffer(bytes(blob[so + 4 * (i // 128): so + 4 * (i // 128) + 4]), "<f4")[0])
                else:
                    byte = int(blob[co + i // 2])
                    code = (byte & 0xF) if i % 2 == 0 else (byte >> 4)
                    el = F.e2m1_value(code)
                    blk = 32 if fmt == F.FMT_MXFP4 else 16
                    sb = int(blob[so + i // blk])
                    s = F.e8m0_value(sb) if fmt == F.FMT_MXFP4 else F.e4m3fn_value(sb)
                W[r, c] = el * s * g[m]
        out.append(W)
    return out


@pytest.mark.parametrize("fmt", [ms.FMT_MXFP4, ms.FMT_NVFP4, ms.FMT_FP8_B128])
def test_dequant_expert_matches_per_element_decode(fmt):
    H, I = 128, 128
    blob = ms.gen_blob(99, ms.KIND_EXPERT, fmt, H, I, 3)
    vec = F.dequant_expert(fmt, blob, H, I)
    ref = _per_element_decode(fmt, blob, H, I)
    for a, b in zip(vec, ref):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("fmt", [ms.FMT_MXFP4, ms.FMT_NVFP4, ms.FMT_FP8_B128])
def test_blob_layout_agrees_with_generator(fmt):
    for H, I in [(256, 128), (2048, 768), (7168, 2048), (6144, 2048)]:
        cod, sca, ts, total = F.blob_offsets(fmt, H, I)
        lay = ms.blob_layout(fmt, H, I)
        assert total == lay.nbytes
        assert tuple(cod) == lay.codes and tuple(sca) == lay.scales


def test_expert_bytes_of_the_workloads():
    # per-expert sizes of the five layer shapes (3 matrices each)
    assert ms.expert_bytes(ms.FMT_MXFP4, 256, 128) == 52_224
    assert ms.expert_bytes(ms.FMT_MXFP4, 2048, 768) == 2_506_752
    assert ms.expert_bytes(ms.FMT_NVFP4, 7168, 2048) == 24_772_620
    assert ms.expert_bytes(ms.FMT_MXFP4, 6144, 2048) == 20_054_016
    assert ms.expert_bytes(ms.FMT_FP8_B128, 6144, 2048) == 38_928_384
    # NVFP4 stores 4.5 bits per weight (an 8-bit scale per 16 weights)
    n = 3 * 7168 * 2048
    assert (ms.expert_bytes(ms.FMT_NVFP4, 7168, 2048) - 12) * 8 / n == 4.5
