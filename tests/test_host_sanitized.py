"""The host runtime pieces that need no GPU -- repacking canonical blobs into
the device layout (layout.cpp) and the host expert path of the hybrid split
(host_ffn.cpp, with its worker threads) -- built with g++ under the address
and undefined-behaviour sanitizers (and the thread sanitizer) and run on
seeded blobs of every format, in the AVX2 and the portable build.  The decoded
matrices must equal the oracle's exactly; the host expert's rows must match the
oracle's expert FFN (same rounding points, fp32 sums) within the parity bar; no
sanitizer may report."""

import os
import shutil
import subprocess

import numpy as np
import pytest

import moe_synth as ms
from oracle import ffn, formats as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "lru_expert_cache_amd", "csrc")


def _build(tmp_path_factory, name, sanitize):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no g++")
    exe = str(tmp_path_factory.mktemp(name) / "host_check")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", sanitize, "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(ROOT, "tests", "native", "host_check.cpp"),
           os.path.join(CSRC, "layout.cpp"), os.path.join(CSRC, "host_ffn.cpp"), "-lpthread", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


@pytest.fixture(scope="module")
def host_check(tmp_path_factory):
    return _build(tmp_path_factory, "asan", "-fsanitize=address,undefined")


@pytest.fixture(scope="module")
def host_check_tsan(tmp_path_factory):
    return _build(tmp_path_factory, "tsan", "-fsanitize=thread")


# rows 1-4 of MXFP4 and FP8 take the few-rows loop of the AVX-512 build (all
# four K quarters in registers up to 2 rows, two at a time for 3 and 4), other
# counts the general one
CASES = [(ms.FMT_MXFP4, 256, 128, 1), (ms.FMT_MXFP4, 384, 256, 5), (ms.FMT_NVFP4, 256, 384, 3),
         (ms.FMT_FP8_B128, 384, 256, 4), (ms.FMT_FP8_B128, 256, 128, 1), (ms.FMT_MXFP4, 384, 256, 2),
         (ms.FMT_MXFP4, 256, 384, 3), (ms.FMT_FP8_B128, 384, 128, 2), (ms.FMT_FP8_B128, 256, 384, 3)]


ISAS = ["native", "avx2", "portable"]  # the widest build the CPU runs, then capped ones


def _plant_e8m0_edges_small(blob, H, I):
    """E8M0 scales 0 and 1 (2^-127 and 2^-126: subnormal weights) in one block
    of W_gate and of W_down; their weights are tiny, so the expert's output
    stays comparable with the oracle's."""
    _, sca, _, _ = F.blob_offsets(ms.FMT_MXFP4, H, I)
    blob[sca[0][0] + 6] = 0
    blob[sca[2][0] + 3] = 1


def _plant_e8m0_edges(blob, H, I):
    """E8M0 block scales at the small and large ends of the range (0, 1, 2:
    2^-127 .. 2^-125, subnormal weights among them; 251, 252: up to
    6 * 2^125) in W_gate and W_down; every weight stays finite in fp32, so
    each must decode exactly."""
    _, sca, _, _ = F.blob_offsets(ms.FMT_MXFP4, H, I)
    for m, blocks in ((0, (0, 1, 2, 3, 4, 37)), (2, (5, 9))):
        so, _ = sca[m]
        for b, v in zip(blocks, (0, 1, 2, 251, 252, 0)):
            blob[so + b] = v


@pytest.mark.parametrize("isa", ISAS)
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{ms.FMT_NAMES[c[0]]}-H{c[1]}-I{c[2]}-rows{c[3]}")
def test_repack_and_host_expert_under_sanitizers(host_check, tmp_path, case, isa):
    fmt, H, I, rows = case
    blob = ms.gen_blob(91, ms.KIND_EXPERT, fmt, H, I, H + I + rows)
    if fmt == ms.FMT_MXFP4:
        _plant_e8m0_edges_small(blob, H, I)
    x_bits = ms.f32_to_bf16_bits(np.random.default_rng(H + rows).standard_normal((rows, H)).astype(np.float32))
    w = np.random.default_rng(I).uniform(0.05, 1.0, rows).astype(np.float32)
    blob.tofile(tmp_path / "blob.bin")
    x_bits.astype(np.uint16).tofile(tmp_path / "x.bin")
    w.tofile(tmp_path / "w.bin")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    if isa != "native":
        env["FT_MOE_HOST_ISA"] = isa
    r = subprocess.run([host_check, str(fmt), str(H), str(I), str(rows), "3", str(tmp_path)], capture_output=True,
                       text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    wg, wu, wd = F.dequant_expert(fmt, blob, H, I)
    mats = np.fromfile(tmp_path / "mats.bin", np.float64)
    got = np.split(mats, [I * H, 2 * I * H])
    # the device layout decodes to exactly the canonical blob's values
    for a, b in zip(got, (wg, wu, wd)):
        assert np.array_equal(a, b.reshape(-1))
    p = F.bf16_from_bits(np.fromfile(tmp_path / "p.bin", np.uint16).reshape(rows, H))
    want = ffn.weighted_rows(ffn.expert_forward(F.bf16_from_bits(x_bits), wg, wu, wd), w)
    rel = np.linalg.norm(p - want) / np.linalg.norm(want)
    assert rel <= 2e-3, rel


@pytest.mark.parametrize("case", CASES[:3], ids=lambda c: f"{ms.FMT_NAMES[c[0]]}-H{c[1]}-I{c[2]}-rows{c[3]}")
def test_host_worker_pool_under_thread_sanitizer(host_check_tsan, tmp_path, case):
    """The host worker pool (persistent threads taking work items) runs the
    expert without a data race that ThreadSanitizer can see."""
    fmt, H, I, rows = case
    blob = ms.gen_blob(92, ms.KIND_EXPERT, fmt, H, I, 7)
    x_bits = ms.f32_to_bf16_bits(np.random.default_rng(3).standard_normal((rows, H)).astype(np.float32))
    blob.tofile(tmp_path / "blob.bin")
    x_bits.astype(np.uint16).tofile(tmp_path / "x.bin")
    np.full(rows, 0.5, np.float32).tofile(tmp_path / "w.bin")
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([host_check_tsan, str(fmt), str(H), str(I), str(rows), "4", str(tmp_path)],
                       capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0 and "ThreadSanitizer" not in r.stderr, r.stderr[-4000:]


@pytest.mark.parametrize("isa", ISAS)
@pytest.mark.parametrize("fmt", [ms.FMT_FP8_B128, ms.FMT_MXFP4, ms.FMT_NVFP4], ids=lambda f: ms.FMT_NAMES[f])
def test_host_lane_decode_is_exact(host_check, tmp_path, fmt, isa):
    """Every weight the host FFN decodes, lane by lane from the device layout,
    equals the oracle's exact value rounded once to fp32 (NVFP4: the E4M3 block
    scale times the per-matrix scale is rounded first, so two roundings).  The
    FP8 blob gets NaN codes planted in two lanes (S.1111.111, both signs):
    they must decode as NaN, the rest of their lanes as usual."""
    H, I = 256, 384
    blob = ms.gen_blob(93, ms.KIND_EXPERT, fmt, H, I, 11)
    if fmt == ms.FMT_FP8_B128:
        cod, _, _, _ = F.blob_offsets(fmt, H, I)
        co, _ = cod[0]
        blob[co + 3] = 0x7F
        blob[co + 5 * H + 200] = 0xFF
    if fmt == ms.FMT_MXFP4:
        _plant_e8m0_edges(blob, H, I)
    blob.tofile(tmp_path / "blob.bin")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    if isa != "native":
        env["FT_MOE_HOST_ISA"] = isa
    r = subprocess.run([host_check, "decode", str(fmt), str(H), str(I), str(tmp_path)], capture_output=True,
                       text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    got = np.split(np.fromfile(tmp_path / "dec.bin", np.float32), [I * H, 2 * I * H])
    for a, b in zip(got, F.dequant_expert(fmt, blob, H, I)):
        b = b.reshape(-1)
        if fmt == ms.FMT_NVFP4:
            assert np.allclose(a, b, rtol=2.0 ** -22, atol=0.0)
        else:
            assert np.array_equal(a, b.astype(np.float32), equal_nan=True)
    if fmt == ms.FMT_FP8_B128:
        assert np.isnan(got[0][3]) and np.isnan(got[0][5 * H + 200]) and np.isnan(got[0]).sum() == 2


@pytest.mark.parametrize("isa", ISAS)
@pytest.mark.parametrize("rows", [2, 6])
def test_host_expert_fp8_nan_code_reaches_its_output_only(host_check, tmp_path, rows, isa):
    """An FP8 NaN code (S.1111.111) planted in W_down at (output 5, input 17)
    makes output feature 5 NaN for every row and leaves every other output
    finite and equal to the oracle's within the parity bar: the host decodes
    NaN lanes by table in both the few-rows loop (2 rows) and the general one
    (6 rows), as the oracle's E4M3 decode does."""
    fmt, H, I = ms.FMT_FP8_B128, 256, 384
    blob = ms.gen_blob(95, ms.KIND_EXPERT, fmt, H, I, rows)
    cod, _, _, _ = F.blob_offsets(fmt, H, I)
    co, _ = cod[2]
    blob[co + 5 * I + 17] = 0x7F
    x_bits = ms.f32_to_bf16_bits(np.random.default_rng(rows).standard_normal((rows, H)).astype(np.float32))
    w = np.random.default_rng(I + rows).uniform(0.05, 1.0, rows).astype(np.float32)
    blob.tofile(tmp_path / "blob.bin")
    x_bits.astype(np.uint16).tofile(tmp_path / "x.bin")
    w.tofile(tmp_path / "w.bin")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    if isa != "native":
        env["FT_MOE_HOST_ISA"] = isa
    r = subprocess.run([host_check, str(fmt), str(H), str(I), str(rows), "2", str(tmp_path)], capture_output=True,
                       text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    p = F.bf16_from_bits(np.fromfile(tmp_path / "p.bin", np.uint16).reshape(rows, H))
    wg, wu, wd = F.dequant_expert(fmt, blob, H, I)
    want = ffn.weighted_rows(ffn.expert_forward(F.bf16_from_bits(x_bits), wg, wu, wd), w)
    assert np.isnan(want[:, 5]).all() and np.isnan(p[:, 5]).all()
    keep = np.arange(H) != 5
    assert np.isfinite(p[:, keep]).all()
    rel = np.linalg.norm(p[:, keep] - want[:, keep]) / np.linalg.norm(want[:, keep])
    assert rel <= 2e-3, rel
