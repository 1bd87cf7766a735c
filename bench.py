#!/usr/bin/env python3
"""Throughput of the offloaded MoE layer stack on one MI355X.

Workload (default): the Qwen-35B-A3B-shaped decode layer stack -- 48 layers,
hidden 2048, expert intermediate 768, 128 MXFP4 experts per layer, top-8,
Zipf(1.0) popularity, one global LRU pool of 1843 slots (30% of the 6144
experts), batch 16.  A step is one decode step through all 48 MoE layers:
router, resolve against the pool, miss streaming from pinned host RAM,
grouped expert FFN, combine.  Inputs are seeded and synthetic and are resident
in HBM before the timed region starts.

Prints one JSON line (see `result` below) with
  * value = tokens per second through the whole 48-layer stack,
  * roofline of the dominant kernel (the gate/up expert FFN), from HIP events
    recorded by the library on the stream the kernel runs on,
  * cpu_baseline = the CPU oracle timed on the host cores on a bounded sample.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measure_h2d(torch, dev, sizes=(52_224, 2_506_752, 20_054_016, 320_864_256), reps=6):
    """Pinned host -> device copy bandwidth (GB/s) per size."""
    out = {}
    big = max(sizes)
    host = torch.empty(big, dtype=torch.uint8, pin_memory=True)
    host.fill_(1)
    dst = torch.empty(big, dtype=torch.uint8, device=dev)
    s = torch.cuda.current_stream()
    for n in sizes:
        dst[:n].copy_(host[:n], non_blocking=True)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(reps):
            dst[:n].copy_(host[:n], non_blocking=True)
        e1.record(s)
        torch.cuda.synchronize()
        out[n] = n * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    return out


def measure_hbm_copy(torch, dev, nbytes=2 << 30, reps=5):
    a = torch.empty(nbytes // 2, dtype=torch.int16, device=dev)
    b = torch.empty_like(a)
    a.fill_(3)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    return 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9


def measured_traffic():
    """HBM bytes per launch of the gate/up FFN kernel from the committed rocprofv3
    counter summary, or None when ffn.hip has changed since it was taken."""
    import hashlib

    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", "ffn_gateup_qwen_a3b_decode_b16_hbm_traffic.md")
    src = os.path.join(root, "lru_expert_cache_amd", "csrc", "ffn.hip")
    try:
        kv = dict(l.strip().split("=", 1) for l in open(path) if "=" in l and not l.startswith(" "))
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
        if kv.get("ffn_source_sha256") != sha:
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(w, batch, ncalls, one_thread_calls=2):
    """The oracle as it stands, on the first `ncalls` (step 0, layer l) calls,
    with every host thread; then on `one_thread_calls` of them with one BLAS
    thread (returned separately)."""
    import moe_synth as ms
    from oracle.layer import OracleLayerStack

    threads = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info

        info = [i.get("num_threads", 1) for i in threadpool_info()]
        threads = max(info) if info else threads
    except Exception:
        pass
    st = OracleLayerStack(w)
    xs = [ms.activations(w, l, 0, batch) for l in range(ncalls)]
    bs = [ms.popularity_bias(w, l, 0) for l in range(ncalls)]
    t0 = time.perf_counter()
    for l in range(ncalls):
        st.forward(l, xs[l], bs[l], outputs=True)
    sec = (time.perf_counter() - t0) / ncalls
    full = {"value": batch / (sec * w.num_layers), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{ncalls} layer calls (step 0, layers 0..{ncalls - 1}) at batch {batch}, routing + LRU + "
                      f"fp64 expert FFN + combine; {sec:.2f} s per layer call, scaled to the {w.num_layers}-layer "
                      f"stack"}
    one = None
    n1 = min(one_thread_calls, ncalls)
    if n1 > 0:
        try:
            from threadpoolctl import threadpool_limits
        except ImportError:
            threadpool_limits = None
        if threadpool_limits is not None:
            st1 = OracleLayerStack(w)
            with threadpool_limits(limits=1):
                t0 = time.perf_counter()
                for l in range(n1):
                    st1.forward(l, xs[l], bs[l], outputs=True)
                sec1 = (time.perf_counter() - t0) / n1
            one = {"value": batch / (sec1 * w.num_layers), "unit": "tokens/s", "cores": 1, "kind": "oracle",
                   "sample": f"{n1} layer calls (step 0, layers 0..{n1 - 1}) at batch {batch} with one BLAS "
                             f"thread; {sec1:.2f} s per layer call"}
    return full, one


def measure_prefill(ft, torch, ms, pool, dev):
    """One 4096-token chunk through the 48 staged layers (Qwen-A3B prefill
    shape), with bf16 expert inputs and with x and h MX-quantised (MXFP8,
    MXFP4).  The MX GEMM rate is priced against the MFMA peak of its narrower
    operand rate: FP8 (5.0 PFLOP/s) when either operand is FP8, FP4 (10.1)."""
    w = ms.workload("qwen-a3b-prefill-4096")
    T, L = w.batches[0], w.num_layers
    xs = torch.from_numpy(np.stack([ms.activations(w, l, 0, T) for l in range(L)]).view(np.int16)).to(dev)
    bias = torch.from_numpy(np.stack([ms.popularity_bias(w, l, 0) for l in range(L)])).to(dev)
    out = torch.empty((T, w.hidden), dtype=torch.int16, device=dev)
    res = {"chunk_tokens": T, "layers": L}
    for name, act, peak in (("bf16", ft.FT_ACT_BF16, None), ("mxfp8", ft.FT_ACT_MXFP8, 5.0e15),
                            ("mxfp4", ft.FT_ACT_MXFP4, 10.1e15)):
        flags = ft.FT_FWD_PREFILL_STAGED | act
        for l in range(L):  # warm
            ft.ft_moe_layer_forward(pool, l, T, xs[l], bias[l], out, flags, None, None)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for l in range(L):
            ft.ft_moe_layer_forward(pool, l, T, xs[l], bias[l], out, flags, None, None)
        torch.cuda.synchronize()
        sec = time.perf_counter() - t0
        ft.ft_moe_set_profiling(pool, None)
        ft.ft_moe_profile_read(pool, reset=True)
        for l in range(L):
            ft.ft_moe_layer_forward(pool, l, T, xs[l], bias[l], out, flags, None, None)
        ft.ft_moe_set_profiling(pool, [])
        pr = ft.ft_moe_profile_read(pool, reset=True)
        gemm_ms = pr["ffn_gateup"]["ms"] + pr["ffn_down"]["ms"]
        flops = pr["ffn_gateup"]["flops"] + pr["ffn_down"]["flops"]
        tf = flops / (gemm_ms * 1e-3) if gemm_ms else None
        r = {"chunk_s": sec, "tokens_per_s": T / sec,
             "copy_GBps": pr["copy"]["bytes"] / (pr["copy"]["ms"] * 1e-3) / 1e9 if pr["copy"]["ms"] else None,
             "ffn_ms_per_layer": gemm_ms / L, "ffn_TFLOPs": tf / 1e12 if tf else None,
             "stage_ms_per_layer": {k: v["ms"] / L for k, v in pr.items()}}
        if peak and tf:
            r["ffn_peak_TFLOPs"] = peak / 1e12
            r["ffn_frac_of_peak"] = tf / peak
        res[name] = r
        log(f"[bench] prefill {name}: {T / sec:.0f} tokens/s, FFN {gemm_ms / L:.3f} ms/layer"
            + (f" at {tf / 1e12:.0f} TFLOP/s" if tf else ""))
    return res


def measure_prefill_hits(ft, torch, ms, w, pool, bias_of, dev):
    """A 4096-token prefill chunk on the decode pool after its decode steps,
    with FT_FWD_PREFILL_HIT_D2D (experts resident in the pool are read in
    place, only the others are copied) and without it, on the same residents
    (a chunk leaves the pool beyond the staging region unchanged)."""
    T, L = 4096, w.num_layers
    xs = torch.from_numpy(np.stack([ms.activations(w, l, 5000, T) for l in range(L)]).view(np.int16)).to(dev)
    out = torch.empty((T, w.hidden), dtype=torch.int16, device=dev)
    res = {"chunk_tokens": T}

    def chunk(flags):
        st0 = ft.ft_moe_pool_stats(pool)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for l in range(L):
            ft.ft_moe_layer_forward(pool, l, T, xs[l], bias_of(0, l), out, flags, None, None)
        torch.cuda.synchronize()
        sec = time.perf_counter() - t0
        st1 = ft.ft_moe_pool_stats(pool)
        d = {k: st1[k] - st0[k] for k in ("pair_hits", "pair_misses", "expert_hits", "expert_misses", "bytes_h2d")}
        return sec, d

    plain = ft.FT_FWD_PREFILL_STAGED
    hit = plain | ft.FT_FWD_PREFILL_HIT_D2D
    chunk(hit)
    chunk(plain)
    for name, flags in (("hit_d2d", hit), ("plain", plain)):
        sec, d = chunk(flags)
        res[name] = {"tokens_per_s": T / sec, "chunk_s": sec, "h2d_GB": d["bytes_h2d"] / 1e9,
                     "pair_hit_rate": d["pair_hits"] / max(d["pair_hits"] + d["pair_misses"], 1),
                     "experts_copied": d["expert_misses"], "experts_resident": d["expert_hits"]}
        log(f"[bench] prefill on the decode pool, {name}: {T / sec:.0f} tokens/s, {d['bytes_h2d'] / 1e9:.2f} GB copied")
    return res


def measure_graph(ft, torch, pool, x_all, bias_of, L, B, first, nrep, dev):
    """Tokens/s of a whole decode step (L layer calls) captured once into a
    HIP graph and replayed; each replay's inputs are copied into the captured
    input buffers first (that copy is inside the timing)."""
    H = x_all.shape[-1]
    ft.ft_moe_reserve(pool, B)
    xin = torch.empty((L, B, H), dtype=torch.int16, device=dev)
    outs = torch.empty((L, B, H), dtype=torch.int16, device=dev)
    side = torch.cuda.Stream(dev)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for l in range(L):
            ft.ft_moe_layer_forward(pool, l, B, xin[l], bias_of(first, l), outs[l], ft.FT_FWD_DECODE, side, None)
    ns = x_all.shape[0]
    for s in range(first, first + 2):  # warm replays
        xin.copy_(x_all[s % ns])
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(first + 2, first + 2 + nrep):
        xin.copy_(x_all[s % ns])
        g.replay()
    torch.cuda.synchronize()
    return B * nrep / (time.perf_counter() - t0)


def run_steps(ft, torch, pool, x_all, bias_of, out, first, nsteps, L, B, sample_gateup=False):
    """Decode steps (x_all[s] is step s's input).  bias_of(s, l): the router
    bias of layer l at step s (popularity phases), or None.  sample_gateup:
    time the gate/up launch of one layer per step (rotating over the layers)
    with HIP events; an event between two kernels costs a few microseconds of
    queue time, so timing every launch would slow the step it measures."""
    for s in range(first, first + nsteps):
        lp = (s * 7) % L if sample_gateup else -1
        for l in range(L):
            if l == lp:
                ft.ft_moe_set_profiling(pool, ["ffn_gateup"])
            ft.ft_moe_layer_forward(pool, l, B, x_all[s, l], bias_of(s, l), out, ft.FT_FWD_DECODE, None, None)
            if l == lp:
                ft.ft_moe_set_profiling(pool, [])


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload", default="qwen-a3b-decode",
                    help="decode workload: qwen-a3b-decode (default), deepseek-v4-flash-decode, glm-5.2-mixed-decode")
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default 240; 8 for the other workloads)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (default 16; 2 for the other workloads)")
    ap.add_argument("--batch", type=int, default=None, help="tokens per call (default: the workload's largest)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-calls", type=int, default=24)
    ap.add_argument("--no-extras", action="store_true", help="skip the batch 1/4 and link measurements")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this build has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import lru_expert_cache_amd as ft
    import moe_synth as ms

    ft.lib()
    dev = torch.device("cuda", 0)
    w = ms.workload(args.workload)
    if w.mode != "decode":
        print(f"bench.py times decode workloads; {w.name} is a {w.mode} workload (its chunk is timed as an extra)",
              file=sys.stderr)
        sys.exit(2)
    headline = w.name == "qwen-a3b-decode"
    if args.steps is None:
        args.steps = 240 if headline else 8
    if args.warmup is None:
        args.warmup = 16 if headline else 2
    if not headline:
        args.no_extras = True  # the batch sweep, link and prefill extras belong to the default workload
    L, E, H, B = w.num_layers, w.num_experts, w.hidden, args.batch or w.batches[-1]
    nsteps = args.warmup + args.steps

    t = time.perf_counter()
    store = ms.BlobStore(w)
    log(f"[bench] generated {store.nbytes / 1e9:.2f} GB of expert blobs in {time.perf_counter() - t:.1f} s")
    t = time.perf_counter()
    blobs = [store.expert(l, e) for l in range(L) for e in range(E)]
    router = np.stack([ms.router_weight(w, l) for l in range(L)])
    shared = [store.shared(l) for l in range(L)] if w.shared_expert else None
    cfg = ft.make_config(L, H, w.inter, E, w.top_k, w.layer_fmt, pool_slots=w.pool_slots, shared=w.shared_expert)
    pool, _ = ft.ft_moe_init_pool(cfg, blobs, router, shared)
    prefill_pool = None
    if not args.no_extras:
        wp = ms.workload("qwen-a3b-prefill-4096")
        cfgp = ft.make_config(L, H, w.inter, E, w.top_k, wp.layer_fmt, pool_slots=wp.pool_slots)
        prefill_pool, _ = ft.ft_moe_init_pool(cfgp, blobs, router)
    del blobs, store, shared
    log(f"[bench] pool of {w.pool_slots} slots ready in {time.perf_counter() - t:.1f} s")
    share = 0.0
    if w.hybrid:
        # the one-time measurement behind the split: host expert rate vs pinned H2D rate
        eb = ms.expert_bytes(w.layer_fmt[0], H, w.inter)
        cpu_bps = ft.ft_moe_host_expert_rate(pool, 0, max(1, B * w.top_k // 64), 1)
        link = measure_h2d(torch, dev, sizes=(eb,), reps=4)[eb] * 1e9
        share = cpu_bps / (cpu_bps + link)
        ft.ft_moe_set_hybrid_share(pool, share)
        log(f"[bench] hybrid share {share:.4f} (host {cpu_bps / 1e9:.2f} GB/s, link {link / 1e9:.1f} GB/s)")

    t = time.perf_counter()
    x_host = np.empty((nsteps, L, B, H), np.uint16)
    for s in range(nsteps):
        for l in range(L):
            x_host[s, l] = ms.activations(w, l, s, B)
    x_all = torch.from_numpy(x_host.view(np.int16)).to(dev)
    phases = sorted({w.phase(s) for s in range(nsteps)})
    biases = {}
    if w.zipf_alpha is not None:
        for ph in phases:
            biases[ph] = torch.from_numpy(np.stack([ms.popularity_bias(w, l, ph) for l in range(L)])).to(dev)

    def bias_of(s, l):
        return biases[w.phase(s)][l] if biases else None

    out = torch.empty((B, H), dtype=torch.int16, device=dev)
    del x_host
    log(f"[bench] {nsteps} steps of activations resident on the GPU ({time.perf_counter() - t:.1f} s)")

    run_steps(ft, torch, pool, x_all, bias_of, out, 0, args.warmup, L, B)
    torch.cuda.synchronize()
    ft.ft_moe_pool_stats(pool, reset=True)
    # timed region: events bracket the dominant kernel (gate/up FFN) and the
    ft.ft_moe_set_profiling(pool, [])
    ft.ft_moe_profile_read(pool, reset=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(ft, torch, pool, x_all, bias_of, out, args.warmup, args.steps, L, B, sample_gateup=True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gu_kernel = ft.ft_moe_ffn_kernel_name("ffn_gateup")  # the kernel behind the timed launches
    ft.ft_moe_set_profiling(pool, [])
    prof = ft.ft_moe_profile_read(pool, reset=True)
    st = ft.ft_moe_pool_stats(pool)
    log(f"[bench] timed {args.steps} steps in {elapsed:.3f} s")
    # a short extra pass with every stage timed, for the per-stage breakdown
    nb = min(8, args.steps)
    ft.ft_moe_set_profiling(pool, None)
    run_steps(ft, torch, pool, x_all, bias_of, out, args.warmup, nb, L, B)
    ft.ft_moe_set_profiling(pool, [])
    stages = ft.ft_moe_profile_read(pool, reset=True)

    gu = prof["ffn_gateup"]
    gu_avg_ms = gu["ms"] / max(gu["launches"], 1)
    gu_gbs = gu["bytes"] / (gu["ms"] * 1e-3) / 1e9 if gu["ms"] > 0 else 0.0
    dn = stages["ffn_down"]
    cp = stages["copy"]
    h2d_stream = cp["bytes"] / (cp["ms"] * 1e-3) / 1e9 if cp["ms"] > 0 else 0.0
    pairs = st["pair_hits"] + st["pair_misses"]
    extras = {
        "hit_rate_pairs": st["pair_hits"] / max(pairs, 1),
        "hit_rate_experts": st["expert_hits"] / max(st["expert_hits"] + st["expert_misses"], 1),
        "streamed_gb_per_step": st["bytes_h2d"] / 1e9 / args.steps,
        "min_topk_gap": st["min_topk_gap"],
        "stage_avg_us": {k: v["ms"] / max(v["launches"], 1) * 1e3 for k, v in stages.items()},
        "stage_ms_per_step": {k: v["ms"] / nb for k, v in stages.items()},
        "ffn_gateup": {"launches": gu["launches"], "avg_us": gu_avg_ms * 1e3, "GBps": gu_gbs},
        "ffn_down": {"launches": dn["launches"], "avg_us": dn["ms"] / max(dn["launches"], 1) * 1e3,
                     "GBps": dn["bytes"] / (dn["ms"] * 1e-3) / 1e9 if dn["ms"] > 0 else 0.0},
        "miss_stream_GBps": h2d_stream,
    }
    if not args.no_extras:
        link = measure_h2d(torch, dev)
        peak_h2d = max(link.values())
        extras["h2d_sweep_GBps"] = {str(k): round(v, 2) for k, v in link.items()}
        extras["miss_stream_frac_of_measured_h2d"] = h2d_stream / peak_h2d if peak_h2d else None
        extras["hbm_copy_GBps"] = measure_hbm_copy(torch, dev)
        for b in (1, 4):
            xb = torch.from_numpy(np.stack([[ms.activations(w, l, 1000 + s, b) for l in range(L)]
                                            for s in range(24)]).view(np.int16)).to(dev)
            ob = torch.empty((b, H), dtype=torch.int16, device=dev)
            run_steps(ft, torch, pool, xb, bias_of, ob, 0, 8, L, b)
            torch.cuda.synchronize()
            ta = time.perf_counter()
            run_steps(ft, torch, pool, xb, bias_of, ob, 8, 16, L, b)
            torch.cuda.synchronize()
            extras[f"tokens_per_s_batch{b}"] = b * 16 / (time.perf_counter() - ta)
            if b == 1:
                extras["graph_tokens_per_s_batch1"] = measure_graph(ft, torch, pool, xb, bias_of, L, 1, 0, 16, dev)
        extras["graph_tokens_per_s_batch16"] = measure_graph(ft, torch, pool, x_all, bias_of, L, B, 0, 16, dev)
        # the one-time strategy choice at this batch (measured, not applied)
        rep = ft.ft_moe_measure_mode(pool, B, apply=False)
        fm = sorted({f for f in w.layer_fmt})
        extras["mode_choice"] = {
            "mode": ["offload", "hybrid", "fused"][rep["mode"]], "share": rep["share"],
            "t_stream_ms": rep["t_stream"] * 1e3, "t_cpu_ms": rep["t_cpu"] * 1e3, "tokens": rep["tokens"],
            **{f"{k}_GBps_fmt{f}": rep[f"{k}_bytes_per_s"][f] / 1e9 for k in ("h2d", "gpu", "cpu") for f in fm}}
        log(f"mode choice: {extras['mode_choice']}")
        if w.pool_slots >= 2 * w.num_experts:
            extras["prefill_on_decode_pool"] = measure_prefill_hits(ft, torch, ms, w, pool, bias_of, dev)
    ft.ft_moe_destroy_pool(pool)
    if prefill_pool is not None:
        extras["prefill"] = measure_prefill(ft, torch, ms, prefill_pool, dev)
        ft.ft_moe_destroy_pool(prefill_pool)
        # measured matrix-core rates (register-only MFMA loops), beside the data-sheet peaks
        rates = {name: ft.ft_moe_mfma_rate(kind) / 1e12
                 for name, kind in (("fp4_32x32x64", ft.FT_MFMA_FP4_32X32X64),
                                    ("fp8_16x16x128", ft.FT_MFMA_FP8_16X16X128),
                                    ("bf16_16x16x32", ft.FT_MFMA_BF16_16X16X32),
                                    ("bf16_32x32x16", ft.FT_MFMA_BF16_32X32X16))}
        extras["mfma_measured_TFLOPs"] = rates
        log(f"[bench] measured MFMA rates (TFLOP/s): {rates}")
        for mode, key in (("bf16", "bf16_16x16x32"), ("mxfp8", "fp8_16x16x128"), ("mxfp4", "fp4_32x32x64")):
            r = extras["prefill"].get(mode)
            if r and r.get("ffn_TFLOPs"):
                r["ffn_frac_of_measured_mfma"] = r["ffn_TFLOPs"] / rates[key]
    if args.calibrate_copy:
        a = torch.empty(128 << 20, dtype=torch.int16, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        extras["calibration_copy_bytes"] = a.numel() * 2

    cpu = None
    if not args.no_cpu_baseline and headline:
        t = time.perf_counter()
        cpu, cpu1 = cpu_baseline(w, B, args.cpu_calls)
        if cpu1 is not None:
            extras["cpu_baseline_one_thread"] = cpu1
        log(f"[bench] cpu baseline {time.perf_counter() - t:.1f} s")

    value = B * args.steps / elapsed
    result = {
        "metric": "MoE-layer tokens/s (decode & prefill); % HBM BW / FP4 MFMA peak; hit rate",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "|".join(sorted({ {1: "mxfp4", 2: "nvfp4", 3: "fp8"}[f] for f in w.layer_fmt})) + "-weights/bf16-act/fp32-acc",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": L, "hidden": H, "expert_inter": w.inter, "experts": E,
                   "top_k": w.top_k, "batch": B, "pool_slots": w.pool_slots,
                   "format": "|".join(sorted({ {1: "mxfp4", 2: "nvfp4", 3: "fp8-b128"}[f] for f in w.layer_fmt})),
                   "zipf_alpha": w.zipf_alpha, "shared_expert": w.shared_expert, "hybrid_share": share,
                   "host_blob_aliasing": w.n_blobs},
        "roofline": {"kernel": gu_kernel, "bound": "hbm", "achieved": gu_gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": gu_gbs / HBM_PEAK_GBS, "traffic": measured_traffic() if headline else None,
                     "algorithmic_bytes_per_launch": gu["bytes"] / max(gu["launches"], 1),
                     "avg_launch_us": gu_avg_ms * 1e3},
        "cpu_baseline": cpu,
        "extras": extras,
    }
    print(json.dumps(result))


if __name__ == "__main__":
    main()
