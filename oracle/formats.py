"""Number formats: exact decoding, bf16 rounding, MX activation quantiser.

TEST INFRASTRUCTURE (oracle).  Closed forms from the public specifications:

* E2M1 (OCP MX v1.0, FP4 element): sign bit, 2 exponent bits (bias 1), 1
  mantissa bit; exponent field 0 is subnormal (value m/2); no inf/NaN.
* E8M0 (OCP MX v1.0, shared scale): value 2^(b-127); 0xFF is NaN.
* E4M3 "FN" (OCP OFP8): bias 7; exponent field 0 is subnormal
  (2^-6 * m/8); S.1111.111 is NaN; max 448; no infinities.
* MXFP4 = E2M1 element x E8M0 scale per 32 elements along K.
* NVFP4 = E2M1 element x E4M3 scale per 16 elements x fp32 per-tensor scale
  (the pages: "an 8-bit scale for every 16 weights", devpik article, "The Real
  Requirement Is System RAM").
* FP8-b128 = E4M3 element x fp32 scale per 128 elements along K.

The canonical blob layout is re-derived here from its written description
(it is not imported from the generator): [gate codes][up codes][down codes]
[gate scales][up scales][down scales][3 fp32 tensor scales, NVFP4 only];
matrices row-major [out, in]; FP4 low nibble = even index.

Pins (tests/test_oracle_formats.py): OCP code tables, torch's float8 decoders,
torch's bf16 cast on fp32 inputs, the fp64 double-rounding trap, hand-worked
MX quantisation blocks, idempotence and saturation of the quantiser.
"""

from __future__ import annotations

import math

import numpy as np

FMT_MXFP4, FMT_NVFP4, FMT_FP8_B128 = 1, 2, 3


def e2m1_value(code: int) -> float:
    sign = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        mag = 0.5 * m
    else:
        mag = 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return sign * mag


def e8m0_value(b: int) -> float:
    if b == 0xFF:
        return math.nan
    return 2.0 ** (b - 127)


def e4m3fn_value(b: int) -> float:
    sign = -1.0 if b & 0x80 else 1.0
    e = (b >> 3) & 0xF
    m = b & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        mag = 2.0 ** -6 * (m / 8.0)
    else:
        mag = 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return sign * mag


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], np.float64)
E8M0_TABLE = np.array([e8m0_value(b) for b in range(256)], np.float64)
E4M3_TABLE = np.array([e4m3fn_value(b) for b in range(256)], np.float64)


def unpack_fp4(codes: np.ndarray, n: int) -> np.ndarray:
    """Bytes -> n E2M1 codes; element 2i is the low nibble of byte i."""
    b = np.asarray(codes, np.uint8)
    out = np.empty(2 * b.size, np.uint8)
    out[0::2] = b & 0xF
    out[1::2] = b >> 4
    return out[:n]


# ---------------------------------------------------------------- blob layout
def _block(fmt):
    return {FMT_MXFP4: 32, FMT_NVFP4: 16, FMT_FP8_B128: 128}[fmt]


def blob_offsets(fmt: int, hidden: int, inter: int):
    """Return ([(code_off, code_len)]*3, [(scale_off, scale_len)]*3, tensor_scale_off|None, total)."""
    shapes = [(inter, hidden), (inter, hidden), (hidden, inter)]
    off = 0
    cod = []
    for r, c in shapes:
        n = r * c if fmt == FMT_FP8_B128 else r * c // 2
        cod.append((off, n))
        off += n
    sca = []
    for r, c in shapes:
        nb = r * c // _block(fmt)
        n = 4 * nb if fmt == FMT_FP8_B128 else nb
        sca.append((off, n))
        off += n
    ts = None
    if fmt == FMT_NVFP4:
        ts = off
        off += 12
    return cod, sca, ts, off


def dequant_matrix(fmt: int, codes: np.ndarray, scales: np.ndarray, rows: int, cols: int,
                   tensor_scale: float = 1.0) -> np.ndarray:
    """Exact fp64 values of one [rows, cols] matrix."""
    if fmt == FMT_MXFP4:
        v = E2M1_TABLE[unpack_fp4(codes, rows * cols)].reshape(rows, cols // 32, 32)
        s = E8M0_TABLE[np.asarray(scales, np.uint8)].reshape(rows, cols // 32, 1)
        return (v * s).reshape(rows, cols)
    if fmt == FMT_NVFP4:
        v = E2M1_TABLE[unpack_fp4(codes, rows * cols)].reshape(rows, cols // 16, 16)
        s = E4M3_TABLE[np.asarray(scales, np.uint8)].reshape(rows, cols // 16, 1)
        return (v * s).reshape(rows, cols) * float(tensor_scale)
    if fmt == FMT_FP8_B128:
        v = E4M3_TABLE[np.asarray(codes, np.uint8)].reshape(rows, cols // 128, 128)
        s = np.asarray(scales, np.uint8).view("<f4").astype(np.float64).reshape(rows, cols // 128, 1)
        return (v * s).reshape(rows, cols)
    raise ValueError(fmt)


def dequant_expert(fmt: int, blob: np.ndarray, hidden: int, inter: int):
    """Canonical blob -> (W_gate [I,H], W_up [I,H], W_down [H,I]) exact fp64."""
    blob = np.asarray(blob, np.uint8)
    cod, sca, ts, total = blob_offsets(fmt, hidden, inter)
    assert blob.size == total, (blob.size, total)
    g = [1.0, 1.0, 1.0]
    if ts is not None:
        g = [float(x) for x in blob[ts:ts + 12].view("<f4")]
    shapes = [(inter, hidden), (inter, hidden), (hidden, inter)]
    mats = []
    for m, (r, c) in enumerate(shapes):
        co, cn = cod[m]
        so, sn = sca[m]
        mats.append(dequant_matrix(fmt, blob[co:co + cn], blob[so:so + sn], r, c, g[m]))
    return tuple(mats)


# ------------------------------------------------------------------ rounding
BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_bf16(x) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value, ties to even, in one step.

    bf16 keeps 8 significant bits; normal exponents reach down to 2^-126 and
    subnormals have quantum 2^-133.  Returns fp64 holding bf16 values.
    """
    x = np.asarray(x, np.float64)
    _, e = np.frexp(x)  # x = m 2^e with 0.5 <= |m| < 1, so the leading bit is 2^(e-1)
    e = np.maximum(e, -125)
    q = np.ldexp(1.0, e - 8)
    r = np.rint(x / q) * q
    r = np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, x), r)
    return np.where(np.isfinite(x), r, x)


def bf16_bits(v) -> np.ndarray:
    """bf16 values (fp64 holding exact bf16 values) -> uint16 bit patterns."""
    f = np.asarray(v, np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def bf16_from_bits(b) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ----------------------------------------------------- MX activation quantiser
ELEM = {
    # name: (mantissa bits, min normal exponent, max magnitude, emax)
    "e2m1": (1, 0, 6.0, 2),
    "e4m3": (3, -6, 448.0, 8),
}


def round_to_element(v: np.ndarray, elem: str) -> np.ndarray:
    """Round (already scaled) values onto the element grid, ties to even,
    saturating at +-max."""
    mbits, emin, vmax, _ = ELEM[elem]
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    _, e = np.frexp(a)
    e = np.maximum(e - 1, emin)  # exponent of the leading bit, clamped to the normal range
    q = np.ldexp(1.0, e - mbits)
    r = np.rint(a / q) * q
    r = np.minimum(r, vmax)
    return np.copysign(r, v) * (a > 0)


def mx_quantize(v: np.ndarray, elem: str):
    """OCP MX v1.0 conversion along the last axis in blocks of 32.

    For each block: amax = max |v|; shared exponent X = 2^(floor(log2 amax) - emax)
    (X = 2^-127 when amax = 0); elements = round_to_element(v / X).  Returns
    (dequantised fp64 values, element values, scale bytes).
    """
    v = np.asarray(v, np.float64)
    shp = v.shape
    assert shp[-1] % 32 == 0
    blk = v.reshape(shp[:-1] + (shp[-1] // 32, 32))
    amax = np.abs(blk).max(axis=-1, keepdims=True)
    _, e = np.frexp(amax)
    emax = ELEM[elem][3]
    sexp = np.where(amax > 0, (e - 1) - emax, -127)
    sexp = np.clip(sexp, -127, 127)
    X = np.ldexp(1.0, sexp)
    el = round_to_element(blk / X, elem)
    deq = (el * X).reshape(shp)
    return deq, el.reshape(shp), (sexp + 127).astype(np.uint8)[..., 0]
