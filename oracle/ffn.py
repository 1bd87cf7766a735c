"""SwiGLU expert FFN and the weighted combine.

TEST INFRASTRUCTURE (oracle).  The pages say only that a routed token runs
through the few experts its router picks (devpik article, "Why a Huge MoE
Model Fits on One Consumer GPU") and that experts are stored in MXFP4, NVFP4,
FP8 or BF16 (devpik article, "The Real Requirement Is System RAM").  The
expert is the usual SwiGLU MLP; the pages fix no rounding points, so these are a reading:

  g = W_g x', u = W_u x'            (fp64 here)
  h = bf16(silu(g) * u),  silu(g) = g / (1 + exp(-g))
  y = W_d h'
  p_j = bf16(w_j * y)               one row per (token, rank) pair
  p_s = bf16(y_shared)              shared expert, weight 1
  out = bf16(((p_0 + p_1) + ...) + p_{k-1} (+ p_s))   summed in fp32, in order

x' = x and h' = h in the default bf16-activation mode; in the MX activation
modes x' and h' are the OCP MX quantisation of x and h (blocks of 32 along
K) with E4M3 (mxfp8) or E2M1 (mxfp4) elements.

Pins (tests/test_oracle_ffn.py): a dense per-token fp64 reference without
rounding points; a one-hot case whose output is a closed-form expression of
three known weights; the same kind of closed form in all three activation
modes (tests/golden/mx_act_closed_form.txt: where Q applies to x and h, and
its saturation); the combine with a shared expert worked by hand
(tests/golden/combine_shared.txt: order and rounding point).
"""

from __future__ import annotations

import numpy as np

from .formats import mx_quantize, round_bf16

ACT_BF16, ACT_MXFP8, ACT_MXFP4 = 0, 1, 2
_ELEM = {ACT_MXFP8: "e4m3", ACT_MXFP4: "e2m1"}


def silu(g: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):  # exp(-g) = inf for g << 0 gives silu = -0
        return g / (1.0 + np.exp(-g))


def act_quant(v: np.ndarray, act_mode: int) -> np.ndarray:
    if act_mode == ACT_BF16:
        return v
    return mx_quantize(v, _ELEM[act_mode])[0]


def expert_forward(x: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray,
                   act_mode: int = ACT_BF16) -> np.ndarray:
    """x: [M,H] (bf16 values, fp64) -> y [M,H] fp64 (before the routing weight)."""
    xi = act_quant(np.asarray(x, np.float64), act_mode)
    g = xi @ wg.T
    u = xi @ wu.T
    h = round_bf16(silu(g) * u)
    hi = act_quant(h, act_mode)
    return hi @ wd.T


def weighted_rows(y: np.ndarray, w: np.ndarray) -> np.ndarray:
    """p = bf16(w * y) per row; w fp32 [M]."""
    return round_bf16(np.asarray(w, np.float32).astype(np.float64)[:, None] * y)


def combine(p: np.ndarray, shared_y=None) -> np.ndarray:
    """p: [T,k,H] bf16 values; shared_y: [T,H] output of the shared expert
    (before any rounding) or None -> out [T,H] bf16 values.

    Sequential fp32 accumulation in rank order; the shared expert (weight 1)
    is rounded to bf16 on its own and added last.
    """
    p32 = np.asarray(p, np.float64).astype(np.float32)
    acc = p32[:, 0, :].copy()
    for j in range(1, p32.shape[1]):
        acc = (acc + p32[:, j, :]).astype(np.float32)
    if shared_y is not None:
        ps = round_bf16(np.asarray(shared_y, np.float64))
        acc = (acc + ps.astype(np.float32)).astype(np.float32)
    return round_bf16(acc.astype(np.float64))
