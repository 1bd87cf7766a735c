"""Pins for oracle/ffn.py and oracle/layer.py."""

import math

import numpy as np
import pytest

import moe_synth as ms
from oracle import ffn, formats as F, router
from oracle.layer import OracleLayerStack


def _dense_reference(x, experts, sel, w):
    """Per token, loop over its k experts; fp64 throughout, no rounding points."""
    T = x.shape[0]
    out = np.zeros_like(x)
    for t in range(T):
        for j in range(sel.shape[1]):
            wg, wu, wd = experts[int(sel[t, j])]
            g = wg @ x[t]
            u = wu @ x[t]
            h = g / (1 + np.exp(-g)) * u
            out[t] += float(w[t, j]) * (wd @ h)
    return out


def test_layer_output_close_to_dense_fp64_reference():
    w = ms.workload(0)
    stack = OracleLayerStack(w)
    x_bits = ms.activations(w, 0, 0, 16)
    res = stack.forward(0, x_bits, None)
    x = F.bf16_from_bits(x_bits)
    experts = {e: F.dequant_expert(w.fmt(0), ms.expert_blob(w, 0, e), w.hidden, w.inter) for e in range(w.num_experts)}
    ref = _dense_reference(x, experts, res["sel"], res["w"])
    rel = np.linalg.norm(res["out"] - ref) / np.linalg.norm(ref)
    # only the bf16 rounding points separate the two
    assert 1e-4 < rel < 3e-3, rel


def _blob_with(fmt, H, I, entries):
    """A blob with all codes zero except the given (matrix, row, col, code);
    all scales = 1 except where noted."""
    lay = ms.blob_layout(fmt, H, I)
    blob = np.zeros(lay.nbytes, np.uint8)
    assert fmt == ms.FMT_MXFP4
    for m in range(3):
        so, sn = lay.scales[m]
        blob[so:so + sn] = 127
    shapes = [(I, H), (I, H), (H, I)]
    for (m, r, c, code, sbyte) in entries:
        R, K = shapes[m]
        co, _ = lay.codes[m]
        i = r * K + c
        b = co + i // 2
        if i % 2 == 0:
            blob[b] = (blob[b] & 0xF0) | code
        else:
            blob[b] = (blob[b] & 0x0F) | (code << 4)
        so, _ = lay.scales[m]
        blob[so + i // 32] = sbyte
    return blob


def test_one_hot_closed_form():
    """x = e_h0, k = 1 (w = 1), one non-zero weight per row in W_down.

    Then out[o] = bf16( c_o * s_o * bf16( silu(a_i) * b_i ) ) with i = the
    column of row o's single W_down weight, a_i = W_g[i,h0], b_i = W_u[i,h0].
    Catches transposed operands, nibble order and scale indexing.
    """
    H, I = 64, 32
    h0 = 37  # odd: high nibble
    entries = []
    a = {3: (5, 126), 10: (3, 128), 17: (13, 125)}  # row i of W_g: (code, scale byte) at column h0
    b = {3: (6, 127), 10: (10, 126), 17: (7, 129)}
    for i, (c, s) in a.items():
        entries.append((0, i, h0, c, s))
    for i, (c, s) in b.items():
        entries.append((1, i, h0, c, s))
    down = {0: (3, 7, 127), 5: (10, 2, 128), 63: (17, 5, 126), 40: (3, 12, 127)}  # row o: (col i, code, scale)
    for o, (i, c, s) in down.items():
        entries.append((2, o, i, c, s))
    blob = _blob_with(ms.FMT_MXFP4, H, I, entries)
    wg, wu, wd = F.dequant_expert(ms.FMT_MXFP4, blob, H, I)
    x = np.zeros((1, H))
    x[0, h0] = 1.0
    y = ffn.expert_forward(x, wg, wu, wd)
    p = ffn.weighted_rows(y, np.array([1.0], np.float32))
    out = ffn.combine(p[:, None, :])
    def v(code, sb):
        return F.E2M1_TABLE[code] * 2.0 ** (sb - 127)
    expect = np.zeros(H)
    for o, (i, c, s) in down.items():
        ga, gb = v(*a[i]), v(*b[i])
        hv = F.round_bf16(np.array([ga / (1 + math.exp(-ga)) * gb]))[0]
        expect[o] = F.round_bf16(np.array([v(c, s) * hv]))[0]
    assert np.array_equal(out[0], expect)
    assert np.count_nonzero(expect) == 4


def test_combine_is_sequential_fp32():
    p = np.array([[[1.0], [2.0 ** -24], [2.0 ** -24]]])
    # (1 + 2^-24) rounds to 1 in fp32 (tie to even), twice -> 1.0
    assert ffn.combine(p)[0, 0] == 1.0
    p2 = np.array([[[2.0 ** -24], [2.0 ** -24], [1.0]]])
    assert ffn.combine(p2)[0, 0] == F.round_bf16(np.array([1.0 + 2.0 ** -23]))[0]


def _golden(name):
    import os

    path = os.path.join(os.path.dirname(__file__), "golden", name)
    return [l.strip() for l in open(path) if l.strip() and not l.startswith("#")]


def _num(tok):
    if "2^" in tok:
        return sum(2.0 ** float(t.split("^")[1]) for t in tok.split("+"))
    return float(tok)


@pytest.mark.parametrize("mode", ["bf16", "mxfp4", "mxfp8"])
def test_act_modes_closed_form(mode):
    """tests/golden/mx_act_closed_form.txt: x and h quantised (OCP MX v1.0) in
    blocks of 32 along K, h after its bf16 rounding; worked by hand."""
    H, I = 64, 32
    entries = [
        (0, 3, 5, 3, 127), (1, 3, 5, 3, 127),      # a = b = 1.5
        (0, 10, 37, 5, 127), (1, 10, 37, 3, 123),  # a = 3.0, b = 0.09375
        (0, 17, 5, 1, 126), (1, 17, 5, 5, 127),    # a = 0.25, b = 3.0
        (0, 20, 40, 4, 127), (1, 20, 40, 2, 127),  # a = 2.0, b = 1.0
        (2, 0, 3, 2, 127), (2, 1, 10, 1, 128), (2, 2, 17, 10, 127), (2, 3, 20, 5, 127),
    ]
    blob = _blob_with(ms.FMT_MXFP4, H, I, entries)
    wg, wu, wd = F.dequant_expert(ms.FMT_MXFP4, blob, H, I)
    x = np.zeros((1, H))
    x[0, 5], x[0, 37], x[0, 40] = 1.0, 1.5, F.round_bf16(np.array([0.3]))[0]
    assert x[0, 40] == 0.30078125
    act = {"bf16": ffn.ACT_BF16, "mxfp4": ffn.ACT_MXFP4, "mxfp8": ffn.ACT_MXFP8}[mode]
    y = ffn.expert_forward(x, wg, wu, wd, act)
    out = ffn.combine(ffn.weighted_rows(y, np.array([1.0], np.float32))[:, None, :])
    rows = {l.split(";")[0].strip(): [float(v) for v in l.split(";")[1].split()] for l in _golden("mx_act_closed_form.txt")}
    expect = np.zeros(H)
    expect[:4] = rows[mode]
    assert np.array_equal(out[0], expect), (out[0, :4], expect[:4])


def test_combine_shared_by_hand():
    """tests/golden/combine_shared.txt: the shared expert is rounded to bf16 on
    its own and added after the routed rows, in the same fp32 accumulator."""
    lines = [[_num(t.strip()) for t in l.split(";")] for l in _golden("combine_shared.txt")]
    p = np.array([[[l[0] for l in lines], [l[1] for l in lines]]]).transpose(0, 1, 2)  # [T=1, k=2, H]
    ys = np.array([[l[2] for l in lines]])
    out = ffn.combine(p, ys)
    assert np.array_equal(out[0], np.array([l[3] for l in lines])), out


def test_shared_expert_added_last():
    w = ms.workload(3).with_(num_layers=1, hidden=256, inter=128, num_experts=8, layer_fmt=(ms.FMT_NVFP4,),
                             pool_slots=16, n_blobs=None)
    st = OracleLayerStack(w)
    x_bits = ms.activations(w, 0, 0, 3)
    res = st.forward(0, x_bits, ms.popularity_bias(w, 0, 0))
    x = F.bf16_from_bits(x_bits)
    sg, su, sd = F.dequant_expert(ms.FMT_NVFP4, ms.shared_blob(w, 0), 256, 128)
    ys = F.round_bf16(ffn.expert_forward(x, sg, su, sd))
    assert np.count_nonzero(ys) > 0
    w_no = w.with_(shared_expert=False)
    st2 = OracleLayerStack(w_no)
    res2 = st2.forward(0, x_bits, ms.popularity_bias(w, 0, 0))
    assert np.array_equal(res["sel"], res2["sel"])
    # out = bf16(routed_fp32_sum + shared): recompute from the no-shared routed part is
    # impossible after rounding, so check closeness and that the shared term matters
    diff = res["out"] - res2["out"]
    assert np.linalg.norm(diff - ys) / np.linalg.norm(ys) < 2e-2
