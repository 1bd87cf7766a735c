"""Pins for oracle/router.py."""

import math

import numpy as np
import scipy.special

from oracle import router as R


def _bf16_values(rng, shape):
    x = rng.standard_normal(shape).astype(np.float32)
    b = (x.view(np.uint32) + 0x8000) & 0xFFFF0000  # any bf16 values will do
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def test_logits_equal_exact_sums():
    rng = np.random.default_rng(0)
    T, H, E = 4, 48, 6
    x = _bf16_values(rng, (T, H))
    wr = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    bias = rng.standard_normal(E).astype(np.float32)
    z = R.logits(x, wr, bias)
    for t in range(T):
        for e in range(E):
            exact = math.fsum([float(x[t, h]) * float(wr[e, h]) for h in range(H)] + [float(bias[e])])
            assert abs(z[t, e] - exact) <= 4 * abs(exact) * 2.0 ** -52 + 1e-300


def test_select_topk_brute_force_with_ties():
    rng = np.random.default_rng(1)
    for _ in range(200):
        E = int(rng.integers(2, 20))
        k = int(rng.integers(1, E + 1))
        z = rng.integers(-3, 4, size=(3, E)).astype(np.float64)  # many ties
        sel = R.select_topk(z, k)
        for t in range(3):
            ref = sorted(range(E), key=lambda e: (-z[t, e], e))[:k]
            assert list(sel[t]) == ref


def test_k_equals_e_is_full_softmax():
    rng = np.random.default_rng(2)
    z = rng.standard_normal((5, 16)) * 3
    sel = R.select_topk(z, 16)
    w = R.topk_weights(z, sel)
    ref = scipy.special.softmax(z.astype(np.float32).astype(np.float64), axis=1)
    ref_sel = np.take_along_axis(ref, sel.astype(np.int64), axis=1)
    assert np.allclose(w, ref_sel, rtol=2e-7, atol=1e-9)


def test_k1_is_argmax_with_unit_weight():
    rng = np.random.default_rng(3)
    z = rng.standard_normal((50, 32))
    sel = R.select_topk(z, 1)
    assert np.array_equal(sel[:, 0], z.argmax(axis=1))
    assert np.all(R.topk_weights(z, sel) == 1.0)


def test_weights_sum_to_one_and_are_descending():
    rng = np.random.default_rng(4)
    z = rng.standard_normal((200, 128)) + np.log(rng.dirichlet(np.ones(128)))[None, :]
    sel = R.select_topk(z, 8)
    w = R.topk_weights(z, sel)
    assert np.abs(w.astype(np.float64).sum(1) - 1).max() <= 1e-6
    assert (np.diff(w, axis=1) <= 0).all()


def test_min_gap():
    z = np.array([[3.0, 1.0, 2.0, 2.5]])
    assert R.min_topk_gap(z, 2) == 0.5
    assert R.min_topk_gap(z, 4) == float("inf")
