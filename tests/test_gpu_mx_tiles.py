"""The h tiles of the MX activation modes, read back from the device: in a
prefill call with MXFP4 or MXFP8 activations the gate/up GEMM quantises h
(OCP MX v1.0, blocks of 32 along the intermediate axis) straight into the down
GEMM's activation tiles, at the tile slot the resolve kernel gives each row.
For every (token, expert) row, the codes and E8M0 scales found at its slot
must be the oracle's quantisation of its h = bf16(silu(g) * u).  The GPU sums
g and u in fp32 and the oracle in fp64, so h can differ in its last bf16 bit
and a block's scale or an element's rounding can land on the neighbouring
value; a row, K-step or slot taken from the wrong place would not agree at
all."""

import numpy as np
import pytest

import moe_synth as ms
from oracle import ffn as OFFN, formats as F

pytestmark = pytest.mark.gpu

MX = ms.FMT_MXFP4


def _decode_row(codes, scales, slot, I, fp4):
    """Element values and scale bytes of one row from the tile layout."""
    nk = I // 128
    tl, i = divmod(int(slot), 128)
    sub = i // 16
    n = i % 16
    code_blk = 8192 if fp4 else 16384
    el = np.empty(I, np.float64)
    sb = np.empty(I // 32, np.uint8)
    for ks in range(nk):
        blk = tl * nk + ks
        for q in range(4):
            sb[ks * 4 + q] = scales[blk * 512 + i * 4 + q]
            base = blk * code_blk + sub * (1024 if fp4 else 2048)
            if fp4:
                b = codes[base + (16 * q + n) * 16: base + (16 * q + n) * 16 + 16]
                nib = np.empty(32, np.uint8)
                nib[0::2] = b & 15
                nib[1::2] = b >> 4
                vals = F.E2M1_TABLE[nib]
            else:
                h, qq = q // 2, 2 * q - 4 * (q // 2)
                lo = codes[base + h * 1024 + (16 * qq + n) * 16: base + h * 1024 + (16 * qq + n) * 16 + 16]
                hi = codes[base + h * 1024 + (16 * (qq + 1) + n) * 16: base + h * 1024 + (16 * (qq + 1) + n) * 16 + 16]
                vals = F.E4M3_TABLE[np.concatenate([lo, hi])]
            el[ks * 128 + 32 * q: ks * 128 + 32 * q + 32] = vals
    return el, sb


@pytest.mark.parametrize("act", ["mxfp4", "mxfp8"])
def test_h_tiles_hold_the_oracles_quantised_h(act):
    from tests.moe_case import GpuLayerStack
    import lru_expert_cache_amd as ft

    mode = OFFN.ACT_MXFP4 if act == "mxfp4" else OFFN.ACT_MXFP8
    flag = ft.FT_ACT_MXFP4 if act == "mxfp4" else ft.FT_ACT_MXFP8
    fp4 = act == "mxfp4"
    H, I, E, k, T = 256, 384, 8, 2, 150
    w = ms.Workload(170 + int(fp4), f"small-{170 + int(fp4)}", 1, H, I, E, k, (MX,), 2 * E + 4, (8,), 4, "decode",
                    None, None, False, False, None)
    g = GpuLayerStack(w)
    try:
        x_bits = ms.activations(w, 0, 3, T)
        r = g.forward(0, x_bits, None, prefill=True, act=flag)
        rows = T * k
        slot_of = np.frombuffer(ft.ft_moe_debug_read(g.pool, ft.FT_DBG_ROW_SLOT, rows * 4), np.int32)
        nslot = int(slot_of[:rows].max()) + 1
        nblk = (nslot + 127) // 128 * (I // 128)
        codes = np.frombuffer(ft.ft_moe_debug_read(g.pool, ft.FT_DBG_H_CODES, nblk * (8192 if fp4 else 16384)),
                              np.uint8)
        scales = np.frombuffer(ft.ft_moe_debug_read(g.pool, ft.FT_DBG_H_SCALES, nblk * 512), np.uint8)
        x = F.bf16_from_bits(x_bits)
        mats = {e: F.dequant_expert(MX, ms.expert_blob(w, 0, e), H, I) for e in range(E)}
        elem = "e2m1" if fp4 else "e4m3"
        same_el = same_sb = total_el = total_sb = 0
        for t in range(T):
            for j in range(k):
                e = int(r["sel"][t, j])
                row = int(r["row"][t * k + j])
                wg, wu, _ = mats[e]
                xq = OFFN.act_quant(x[t:t + 1], mode)
                h = F.round_bf16(OFFN.silu(xq @ wg.T) * (xq @ wu.T))
                _, el, sb = F.mx_quantize(h, elem)
                gel, gsb = _decode_row(codes, scales, slot_of[row], I, fp4)
                el, sb = el.reshape(-1), sb.reshape(-1)
                same = np.repeat(gsb == sb, 32)
                same_el += int(((gel == el) & same).sum())
                same_sb += int((gsb == sb).sum())
                total_el += I
                total_sb += I // 32
                # the values the codes stand for differ by at most one step of
                # the element grid (E2M1: 2, E4M3: 32 in units of the larger
                # of the two block scales)
                Xg = np.repeat(np.ldexp(1.0, gsb.astype(np.int64) - 127), 32)
                Xo = np.repeat(np.ldexp(1.0, sb.astype(np.int64) - 127), 32)
                d = np.abs(gel * Xg - el * Xo)
                assert (d <= (2.0 if fp4 else 32.0) * np.maximum(Xg, Xo)).all(), (t, j, e, d.max())
        assert same_sb >= 0.99 * total_sb, (same_sb, total_sb)
        assert same_el >= 0.98 * total_el, (same_el, total_el)
        print(act, "equal scales", same_sb / total_sb, "equal elements", same_el / total_el)
    finally:
        g.close()
