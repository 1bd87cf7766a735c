"""Seeded synthetic workloads for the offloaded MoE layer.

This module is the only code shared by the CPU oracle and the GPU path.  It
draws random inputs (expert weight blobs, router weights, popularity biases,
activations) and knows the byte layout of a *canonical expert blob*, which is
the input format of the library.  It performs none of the layer's arithmetic:
no decoding of the number formats, no routing, no cache decisions, no FFN.

Workload shapes follow the five layer shapes that the FreeToken pages discuss
(a tiny test layer; a Qwen-35B-A3B-shaped layer in decode and prefill; a
DeepSeek-V4-Flash-shaped layer; a GLM-5.2-shaped layer).  The pages describe
experts kept in host RAM in MXFP4, NVFP4 or FP8 (devpik article, "The Real
Requirement Is System RAM"; byteiota article, "Setup Is Four Commands").

Seeding: every tensor is drawn from
``np.random.Generator(PCG64(SeedSequence([master, cfg_id, kind, a, b, ...])))``
so any single tensor can be regenerated on its own, in any order.
"""

from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

# Number-format identifiers (match the C header's FT_FMT_* values).
FMT_MXFP4 = 1
FMT_NVFP4 = 2
FMT_FP8_B128 = 3
FMT_NAMES = {FMT_MXFP4: "mxfp4", FMT_NVFP4: "nvfp4", FMT_FP8_B128: "fp8_b128"}

# Tensor kinds used in the seed sequence.
KIND_EXPERT = 1
KIND_ROUTER = 2
KIND_POPULARITY = 3
KIND_ACT = 4
KIND_SHARED = 5

MASTER_SEED = 0


# --------------------------------------------------------------------------
# Canonical expert blob layout
# --------------------------------------------------------------------------
# One routed expert = three matrices W_gate [I,H], W_up [I,H], W_down [H,I],
# each stored row-major as [out, in] with the block scales running along `in`.
# Byte order of a blob:
#   [gate codes][up codes][down codes][gate scales][up scales][down scales]
#   [3 x fp32 per-matrix scale]   (NVFP4 only)
# FP4 codes: two per byte, the element with the even index in the low nibble.
# MXFP4 scales: one E8M0 byte per 32 elements.  NVFP4 scales: one E4M3 byte
# per 16 elements.  FP8 codes: one E4M3 byte each; scales: one little-endian
# fp32 per 128 elements.

BLOCK = {FMT_MXFP4: 32, FMT_NVFP4: 16, FMT_FP8_B128: 128}


def code_bytes(fmt: int, rows: int, cols: int) -> int:
    n = rows * cols
    return n if fmt == FMT_FP8_B128 else n // 2


def scale_bytes(fmt: int, rows: int, cols: int) -> int:
    nblk = rows * cols // BLOCK[fmt]
    return nblk * 4 if fmt == FMT_FP8_B128 else nblk


@dataclasses.dataclass(frozen=True)
class BlobLayout:
    """Byte offsets of the pieces of one canonical expert blob."""

    fmt: int
    hidden: int
    inter: int
    codes: tuple  # (offset, nbytes) for gate, up, down
    scales: tuple  # (offset, nbytes) for gate, up, down
    tensor_scales: Optional[tuple]  # (offset, 12) for NVFP4
    nbytes: int


def blob_layout(fmt: int, hidden: int, inter: int) -> BlobLayout:
    shapes = [(inter, hidden), (inter, hidden), (hidden, inter)]
    off = 0
    codes = []
    for r, c in shapes:
        n = code_bytes(fmt, r, c)
        codes.append((off, n))
        off += n
    scales = []
    for r, c in shapes:
        n = scale_bytes(fmt, r, c)
        scales.append((off, n))
        off += n
    ts = None
    if fmt == FMT_NVFP4:
        ts = (off, 12)
        off += 12
    return BlobLayout(fmt, hidden, inter, tuple(codes), tuple(scales), ts, off)


def expert_bytes(fmt: int, hidden: int, inter: int) -> int:
    return blob_layout(fmt, hidden, inter).nbytes


# --------------------------------------------------------------------------
# Workload definitions
# --------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class Workload:
    cfg_id: int
    name: str
    num_layers: int
    hidden: int
    inter: int
    num_experts: int
    top_k: int
    layer_fmt: tuple  # per layer FMT_*
    pool_slots: int
    batches: tuple  # tokens per call
    steps: int
    mode: str  # "decode" or "prefill"
    zipf_alpha: Optional[float]  # None: no popularity bias
    phase_steps: Optional[int]  # popularity permutation redrawn every this many steps
    shared_expert: bool
    hybrid: bool
    n_blobs: Optional[int]  # host-blob aliasing: key (l,e) -> blob (l*E+e) mod n_blobs
    router_std: float = 0.02

    @property
    def max_expert_bytes(self) -> int:
        return max(expert_bytes(f, self.hidden, self.inter) for f in set(self.layer_fmt))

    def fmt(self, layer: int) -> int:
        return self.layer_fmt[layer]

    def blob_id(self, layer: int, expert: int) -> int:
        key = layer * self.num_experts + expert
        return key if self.n_blobs is None else key % self.n_blobs

    def phase(self, step: int) -> int:
        return 0 if self.phase_steps is None else step // self.phase_steps

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _pool_from_budget(budget_bytes: float, slot_bytes: int) -> int:
    return int(budget_bytes // slot_bytes)


def _mk_workloads() -> List[Workload]:
    ws = []
    # Tiny parity layer: 1 layer, H 256, I 128, 16 experts, top-2, MXFP4, 64 tokens, 8 slots.
    ws.append(Workload(0, "tiny-h256-e16", 1, 256, 128, 16, 2, (FMT_MXFP4,), 8, (64, 1), 64,
                       "decode", None, None, False, False, None))
    # Qwen-35B-A3B-shaped decode: 48 layers, H 2048, I 768, 128 experts, top-8, MXFP4,
    # pool = 30% of the 6144 experts.
    ws.append(Workload(1, "qwen-a3b-decode", 48, 2048, 768, 128, 8, (FMT_MXFP4,) * 48,
                       int(math.floor(0.3 * 48 * 128)), (1, 4, 16), 256, "decode", 1.0, None,
                       False, False, None))
    # Same layer, one 4096-token prefill chunk, pool = two staging layers.
    ws.append(Workload(2, "qwen-a3b-prefill-4096", 48, 2048, 768, 128, 8, (FMT_MXFP4,) * 48,
                       2 * 128, (4096,), 1, "prefill", 1.0, None, False, False, None))
    # DeepSeek-V4-Flash-shaped decode: 61 layers, H 7168, I 2048, 256 experts + 1 shared,
    # top-8, NVFP4, pool sized to 24 GB; host blobs aliased to fit a test box.
    ds_bytes = expert_bytes(FMT_NVFP4, 7168, 2048)
    ws.append(Workload(3, "deepseek-v4-flash-decode", 61, 7168, 2048, 256, 8, (FMT_NVFP4,) * 61,
                       _pool_from_budget(24e9, ds_bytes), (1, 8, 32, 64), 128, "decode", 0.8, None,
                       True, False, 512))
    # GLM-5.2-shaped decode: 92 layers, H 6144, I 2048, 160 experts, top-8, even layers
    # MXFP4 / odd layers FP8-b128, pool sized to 40 GB of uniform max-size slots,
    # popularity redrawn every 32 steps, hybrid host/PCIe miss split.
    glm_fmt = tuple(FMT_MXFP4 if l % 2 == 0 else FMT_FP8_B128 for l in range(92))
    glm_bytes = expert_bytes(FMT_FP8_B128, 6144, 2048)
    ws.append(Workload(4, "glm-5.2-mixed-decode", 92, 6144, 2048, 160, 8, glm_fmt,
                       _pool_from_budget(40e9, glm_bytes), (32,), 128, "decode", 1.2, 32,
                       False, True, 256))
    return ws


WORKLOADS = _mk_workloads()
BY_NAME = {w.name: w for w in WORKLOADS}


def workload(key) -> Workload:
    if isinstance(key, int):
        return WORKLOADS[key]
    return BY_NAME[key]


# --------------------------------------------------------------------------
# Random streams
# --------------------------------------------------------------------------


def rng_for(cfg_id: int, kind: int, *ids: int) -> np.random.Generator:
    ss = np.random.SeedSequence([MASTER_SEED, cfg_id, kind] + [int(i) for i in ids])
    return np.random.Generator(np.random.PCG64(ss))


def _random_bytes(rng: np.random.Generator, n: int) -> np.ndarray:
    """n uniformly random bytes (each nibble is then uniform over 0..15)."""
    words = (n + 7) // 8
    return rng.bit_generator.random_raw(words).view(np.uint8)[:n].copy()


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 samples to the nearest bf16 (ties to even); returns uint16 bits.

    Used only to produce bf16 inputs from fp32 random draws.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return r


def gen_matrix_parts(rng: np.random.Generator, fmt: int, rows: int, cols: int):
    """Draw (codes, scales) bytes for one [rows, cols] matrix in `fmt`.

    MXFP4: E2M1 codes uniform over 0..15, E8M0 scale bytes uniform in 123..127
    (scales 2^-4 .. 2^0).  NVFP4: codes uniform, E4M3 block scales uniform over
    the positive normal codes 0x18..0x38 (2^-4 .. 1.0).  FP8: E4M3 codes
    uniform over the 254 finite codes, fp32 block scales 2^u with u uniform in
    -8..-4.
    """
    nblk = rows * cols // BLOCK[fmt]
    if fmt == FMT_MXFP4:
        codes = _random_bytes(rng, rows * cols // 2)
        scales = rng.integers(123, 128, size=nblk, dtype=np.uint8)
    elif fmt == FMT_NVFP4:
        codes = _random_bytes(rng, rows * cols // 2)
        scales = rng.integers(0x18, 0x39, size=nblk, dtype=np.uint8)
    elif fmt == FMT_FP8_B128:
        c = rng.integers(0, 254, size=rows * cols, dtype=np.uint8)
        # 254 finite codes: skip 0x7F and 0xFF (the two NaN encodings)
        c = c + (c >= 0x7F).astype(np.uint8)
        codes = c
        u = rng.integers(-8, -3, size=nblk)
        scales = np.ldexp(np.ones(nblk, np.float32), u).astype(np.float32).view(np.uint8)
    else:
        raise ValueError(fmt)
    return codes, scales


def gen_blob(cfg_id: int, kind: int, fmt: int, hidden: int, inter: int, blob_id: int) -> np.ndarray:
    """One canonical expert blob (uint8 array), regenerated from its id alone."""
    lay = blob_layout(fmt, hidden, inter)
    rng = rng_for(cfg_id, kind, fmt, blob_id)
    out = np.empty(lay.nbytes, np.uint8)
    shapes = [(inter, hidden), (inter, hidden), (hidden, inter)]
    for m, (r, c) in enumerate(shapes):
        codes, scales = gen_matrix_parts(rng, fmt, r, c)
        co, cn = lay.codes[m]
        so, sn = lay.scales[m]
        out[co:co + cn] = codes
        out[so:so + sn] = scales
    if fmt == FMT_NVFP4:
        g = rng.uniform(0.5, 1.0, size=3).astype(np.float32)
        to, tn = lay.tensor_scales
        out[to:to + tn] = g.view(np.uint8)
    return out


def expert_blob(w: Workload, layer: int, expert: int) -> np.ndarray:
    return gen_blob(w.cfg_id, KIND_EXPERT, w.fmt(layer), w.hidden, w.inter, w.blob_id(layer, expert))


def shared_blob(w: Workload, layer: int) -> np.ndarray:
    assert w.shared_expert
    return gen_blob(w.cfg_id, KIND_SHARED, w.fmt(layer), w.hidden, w.inter, layer)


def router_weight(w: Workload, layer: int) -> np.ndarray:
    """fp32 [E, H], N(0, router_std^2)."""
    rng = rng_for(w.cfg_id, KIND_ROUTER, layer)
    return (rng.standard_normal((w.num_experts, w.hidden), dtype=np.float32) * np.float32(w.router_std)).astype(np.float32)


def popularity_bias(w: Workload, layer: int, phase: int) -> Optional[np.ndarray]:
    """fp32 [E] logit bias encoding a Zipf(alpha) expert popularity.

    A seeded permutation gives each expert a rank r in 1..E; its bias is
    fp32(ln p_r) with p_r = r^-alpha / sum_{r'<=E} r'^-alpha.
    """
    if w.zipf_alpha is None:
        return None
    rng = rng_for(w.cfg_id, KIND_POPULARITY, layer, phase)
    perm = rng.permutation(w.num_experts)
    ranks = np.arange(1, w.num_experts + 1, dtype=np.float64)
    p = ranks ** (-w.zipf_alpha)
    p /= p.sum()
    bias = np.empty(w.num_experts, np.float32)
    bias[perm] = np.log(p).astype(np.float32)
    return bias


def activations(w: Workload, layer: int, step: int, tokens: int) -> np.ndarray:
    """bf16 bits (uint16) [tokens, H]: N(0,1) draws rounded to bf16."""
    rng = rng_for(w.cfg_id, KIND_ACT, layer, step, tokens)
    x = rng.standard_normal((tokens, w.hidden), dtype=np.float32)
    return f32_to_bf16_bits(x).reshape(tokens, w.hidden)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32 values."""
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def distinct_blob_ids(w: Workload, layers: Optional[Sequence[int]] = None):
    """Sorted (fmt, blob_id) pairs referenced by the given layers."""
    layers = range(w.num_layers) if layers is None else layers
    seen = set()
    for l in layers:
        for e in range(w.num_experts):
            seen.add((w.fmt(l), w.blob_id(l, e)))
    return sorted(seen)


class BlobStore:
    """Generates each distinct blob once and hands out the per-key views."""

    def __init__(self, w: Workload, layers: Optional[Sequence[int]] = None):
        self.w = w
        self.layers = list(range(w.num_layers)) if layers is None else list(layers)
        self._blobs = {}
        for l in self.layers:
            f = w.fmt(l)
            for e in range(w.num_experts):
                bid = w.blob_id(l, e)
                if (f, bid) not in self._blobs:
                    self._blobs[(f, bid)] = gen_blob(w.cfg_id, KIND_EXPERT, f, w.hidden, w.inter, bid)
        self._shared = {}
        if w.shared_expert:
            for l in self.layers:
                self._shared[l] = shared_blob(w, l)

    def expert(self, layer: int, e: int) -> np.ndarray:
        return self._blobs[(self.w.fmt(layer), self.w.blob_id(layer, e))]

    def shared(self, layer: int) -> np.ndarray:
        return self._shared[layer]

    @property
    def nbytes(self) -> int:
        return sum(b.nbytes for b in self._blobs.values())
