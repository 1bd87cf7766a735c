"""Router: logits, top-k selection, renormalised softmax weights.

TEST INFRASTRUCTURE (oracle).  The pages say a router sends each token to a
few of a layer's experts (devpik article, "Why a Huge MoE Model Fits on One
Consumer GPU"; mindstudio article, "How does FreeToken let you run models
bigger than your VRAM?").  They fix nothing finer, so this follows the plain
reading:

* logits z[t,e] = sum_h x[t,h] * Wr[e,h] + bias[e], with x bf16 and Wr fp32.
  Each product is exact in fp64 (8 x 24 significant bits); the sum is fp64.
* selection: the k largest z per token, ordered by z descending and, on equal
  z, by the lower expert index.
* weights: softmax over the selected logits after rounding them to fp32, i.e.
  w_j = exp(zeta_j - zeta_0) / sum_i exp(zeta_i - zeta_0), evaluated in fp64
  and rounded to fp32.  This equals the full softmax renormalised over the
  top-k.

Pins (tests/test_oracle_router.py): exact math.fsum logits on small cases,
brute-force sort, k = E equals scipy's softmax, k = 1 is argmax with w = 1,
sum of weights = 1.
"""

from __future__ import annotations

import numpy as np


def logits(x: np.ndarray, wr: np.ndarray, bias=None) -> np.ndarray:
    """x: [T,H] values of bf16 inputs; wr: [E,H] fp32; bias: [E] fp32 or None."""
    z = np.asarray(x, np.float64) @ np.asarray(wr, np.float32).astype(np.float64).T
    if bias is not None:
        z = z + np.asarray(bias, np.float32).astype(np.float64)[None, :]
    return z


def select_topk(z: np.ndarray, k: int) -> np.ndarray:
    """[T,E] -> int32 [T,k], rank order (z descending, expert index ascending)."""
    T, E = z.shape
    sel = np.empty((T, k), np.int32)
    idx = np.arange(E)
    for t in range(T):
        order = np.lexsort((idx, -z[t]))  # primary key -z, secondary key index
        sel[t] = order[:k]
    return sel


def topk_weights(z: np.ndarray, sel: np.ndarray) -> np.ndarray:
    zs = np.take_along_axis(z, sel.astype(np.int64), axis=1)
    zeta = zs.astype(np.float32).astype(np.float64)
    ex = np.exp(zeta - zeta[:, :1])
    return (ex / ex.sum(axis=1, keepdims=True)).astype(np.float32)


def min_topk_gap(z: np.ndarray, k: int) -> float:
    """Smallest z_(k) - z_(k+1) over the tokens (inf when k = E)."""
    T, E = z.shape
    if k >= E:
        return float("inf")
    s = -np.sort(-z, axis=1)
    return float((s[:, k - 1] - s[:, k]).min())


def route(x, wr, bias, k):
    z = logits(x, wr, bias)
    sel = select_topk(z, k)
    return z, sel, topk_weights(z, sel)
