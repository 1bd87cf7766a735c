#!/usr/bin/env python3
"""Throughput of the offloaded MoE layer stack on one MI355X.

Headline workload (default): the GLM-5.2-shaped decode stack -- 92 layers,
hidden 6144, expert intermediate 2048, 160 experts per layer, top-8, even
layers MXFP4 and odd layers FP8 with a fp32 scale per 128 weights, Zipf(1.2)
popularity redrawn every 32 steps, one global LRU pool of 1027 slots (40 GB
of the largest expert size), batch 32, with the hybrid strategy: each step's
misses are split between host-core compute and PCIe streaming at the share
the library measures on this machine (ft_moe_measure_mode's balanced share),
refined per weight format after each warm-up step from the copy and host
rates the library observed in it (ft_moe_rebalance).
The store uses host-blob aliasing (key (l, e) reads blob (l*E + e) mod 256
per format) so that it fits the host; keys, cache decisions and the bytes
moved are those of the full model.

A step is one decode step through all 92 MoE layers: router, resolve against
the pool, miss streaming from pinned host RAM and host-computed misses,
grouped expert FFN, combine.  Inputs are seeded and synthetic and resident in
HBM before the timed region starts.

Prints one JSON line with
  * value = tokens per second through the whole layer stack,
  * roofline of the dominant kernel, the gate/up expert FFN of the FP8
    layers (the larger experts), from HIP events the library records on the
    stream the kernel runs on,
  * cpu_baseline = the CPU oracle timed on the host cores on a bounded sample,
  * extras: the other measurements (Qwen-A3B decode and prefill, link and
    HBM rates, measured MFMA rates).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
FMT_NAME = {1: "mxfp4", 2: "nvfp4", 3: "fp8"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def host_threads():
    return max(1, min(16, len(os.sched_getaffinity(0))))


# Host worker threads of the hybrid split (--host-threads; default every core)
HYBRID_THREADS = None


def hybrid_threads():
    return HYBRID_THREADS or host_threads()


def measure_h2d(torch, dev, sizes=(52_224, 2_506_752, 20_054_016, 38_928_384, 320_864_256), reps=6):
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


def measured_traffic(profile_name, algorithmic_bytes):
    """HBM bytes per launch of a kernel from a committed rocprofv3 counter
    summary, or None when the kernel's source has changed since it was taken
    or when this run's launches are not the workload the counters saw (their
    algorithmic bytes per launch differ by more than 5%: the hybrid split,
    measured per run, moves them by a few percent)."""
    path = os.path.join(ROOT, "profiles", profile_name)
    src = os.path.join(ROOT, "lru_expert_cache_amd", "csrc", "ffn.hip")
    try:
        kv = dict(l.strip().split("=", 1) for l in open(path) if "=" in l and not l.startswith(" "))
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
        if kv.get("ffn_source_sha256") != sha:
            return None
        ref = float(kv["algorithmic_bytes_per_launch"])
        if not abs(algorithmic_bytes - ref) <= 0.05 * ref:
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def oracle_rate(w, batch, calls, share, blob_fn, threads):
    """The oracle as it stands on layer calls (step 0, layers 0..calls-1):
    routing, LRU, expert FFN in fp64 and combine.  Returns seconds per call."""
    import moe_synth as ms
    from oracle.layer import OracleLayerStack

    st = OracleLayerStack(w, share=share, blob_fn=blob_fn, threads=threads, dequant_items=16)
    xs = [ms.activations(w, l, 0, batch) for l in range(calls)]
    bs = [ms.popularity_bias(w, l, 0) for l in range(calls)]
    t0 = time.perf_counter()
    for l in range(calls):
        st.forward(l, xs[l], bs[l], outputs=True)
    return (time.perf_counter() - t0) / calls


def cpu_baseline(w, batch, calls, share, blob_fn):
    threads = host_threads()
    sec = oracle_rate(w, batch, calls, share, blob_fn, threads)
    return {"value": batch / (sec * w.num_layers), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{calls} layer calls (step 0, layers 0..{calls - 1}) of {w.name} at batch {batch}: routing, "
                      f"LRU, fp64 expert FFN (distinct experts dequantised {threads} at a time) and combine; "
                      f"{sec:.2f} s per layer call, scaled to the {w.num_layers}-layer stack"}


class DecodeRun:
    """A pool for one decode workload, its resident inputs and timed steps."""

    def __init__(self, ft, torch, ms, w, batch, nsteps, dev, first_step=0):
        self.ft, self.torch, self.w, self.B, self.dev = ft, torch, w, batch, dev
        L, E, H = w.num_layers, w.num_experts, w.hidden
        t = time.perf_counter()
        self.store = ms.BlobStore(w)
        log(f"[bench] {w.name}: {self.store.nbytes / 1e9:.2f} GB of expert blobs in {time.perf_counter() - t:.1f} s")
        t = time.perf_counter()
        blobs = [self.store.expert(l, e) for l in range(L) for e in range(E)]
        router = np.stack([ms.router_weight(w, l) for l in range(L)])
        shared = [self.store.shared(l) for l in range(L)] if w.shared_expert else None
        cfg = ft.make_config(L, H, w.inter, E, w.top_k, w.layer_fmt, pool_slots=w.pool_slots, shared=w.shared_expert,
                             cpu_threads=hybrid_threads())
        self.pool, _ = ft.ft_moe_init_pool(cfg, blobs, router, shared)
        del blobs
        log(f"[bench] {w.name}: pool of {w.pool_slots} slots ready in {time.perf_counter() - t:.1f} s")
        self.share, self.mode_report = 0.0, None
        if w.hybrid:
            # the one-time measurement behind the split (pinned H2D, device FFN
            # and host expert rates per format), taken by the library
            rep = ft.ft_moe_measure_mode(self.pool, max(1, batch * w.top_k // 64))
            self.share = rep["balanced_share"]
            self.mode_report = rep
            ft.ft_moe_set_hybrid_share(self.pool, self.share)
            log(f"[bench] hybrid share {self.share:.4f} (the rule's own choice: "
                f"{['offload', 'hybrid', 'fused'][rep['mode']]})")
        t = time.perf_counter()
        x_host = np.empty((nsteps, L, batch, H), np.uint16)
        for s in range(nsteps):
            for l in range(L):
                x_host[s, l] = ms.activations(w, l, first_step + s, batch)
        self.x_all = torch.from_numpy(x_host.view(np.int16)).to(dev)
        del x_host
        self.biases = {}
        if w.zipf_alpha is not None:
            for ph in sorted({w.phase(first_step + s) for s in range(nsteps)}):
                self.biases[ph] = torch.from_numpy(np.stack([ms.popularity_bias(w, l, ph) for l in range(L)])).to(dev)
        self.first_step = first_step
        self.out = torch.empty((batch, H), dtype=torch.int16, device=dev)
        log(f"[bench] {w.name}: {nsteps} steps of activations resident ({time.perf_counter() - t:.1f} s)")

    def bias_of(self, s, l):
        return self.biases[self.w.phase(self.first_step + s)][l] if self.biases else None

    def steps(self, first, n, timed_layers=None, x_all=None, out=None, batch=None):
        """Decode steps first..first+n-1.  timed_layers(s) -> layers whose
        gate/up launch is bracketed by HIP events in step s."""
        ft, w = self.ft, self.w
        x_all = self.x_all if x_all is None else x_all
        out = self.out if out is None else out
        B = self.B if batch is None else batch
        ns = x_all.shape[0]
        for s in range(first, first + n):
            tl = timed_layers(s) if timed_layers else ()
            for l in range(w.num_layers):
                if l in tl:
                    ft.ft_moe_set_profiling(self.pool, ["ffn_gateup"])
                ft.ft_moe_layer_forward(self.pool, l, B, x_all[s % ns, l], self.bias_of(s, l), out, ft.FT_FWD_DECODE,
                                        None, None)
                if l in tl:
                    ft.ft_moe_set_profiling(self.pool, [])

    def timed(self, warmup, steps, timed_layers):
        ft, torch = self.ft, self.torch
        self.rebalances = []
        for s in range(warmup):
            self.steps(s, 1)
            if self.w.hybrid:
                # bandwidth-adaptive refinement: each format's share from the
                # copy and host rates the library observed in this step
                rep = ft.ft_moe_rebalance(self.pool, apply=True)
                self.rebalances.append(rep)
                log("[bench] warm-up step %d: shares %s" % (s, {FMT_NAME[f]: round(rep["share"][f], 4)
                                                                for f in range(1, 4) if rep["changed"][f]}))
        torch.cuda.synchronize()
        ft.ft_moe_pool_stats(self.pool, reset=True)
        ft.ft_moe_set_profiling(self.pool, [])
        ft.ft_moe_profile_read(self.pool, reset=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        self.steps(warmup, steps, timed_layers)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        kernel = ft.ft_moe_ffn_kernel_name("ffn_gateup")  # the kernel behind the timed launches
        ft.ft_moe_set_profiling(self.pool, [])
        prof = ft.ft_moe_profile_read(self.pool, reset=True)
        st = ft.ft_moe_pool_stats(self.pool)
        return elapsed, kernel, prof, st

    def breakdown(self, first, n):
        """Every stage timed with events over n more steps."""
        ft = self.ft
        ft.ft_moe_set_profiling(self.pool, None)
        self.steps(first, n)
        ft.ft_moe_set_profiling(self.pool, [])
        return ft.ft_moe_profile_read(self.pool, reset=True)

    def close(self):
        if self.pool:
            self.ft.ft_moe_destroy_pool(self.pool)
            self.pool = None


def summarize(run, elapsed, steps, prof, st, stages, nb):
    w, B = run.w, run.B
    pairs = st["pair_hits"] + st["pair_misses"]
    cp = stages["copy"]
    gu = prof["ffn_gateup"]
    return {
        "tokens_per_s": B * steps / elapsed,
        "ms_per_step": elapsed / steps * 1e3,
        "hit_rate_pairs": st["pair_hits"] / max(pairs, 1),
        "hit_rate_experts": st["expert_hits"] / max(st["expert_hits"] + st["expert_misses"], 1),
        "streamed_gb_per_step": st["bytes_h2d"] / 1e9 / steps,
        "host_computed_experts_per_step": st["cpu_misses"] / steps,
        "copy_ms_per_step": st["copy_ms"] / steps,
        "miss_stream_GBps": cp["bytes"] / (cp["ms"] * 1e-3) / 1e9 if cp["ms"] > 0 else None,
        "min_topk_gap": st["min_topk_gap"],
        "stage_avg_us": {k: v["ms"] / max(v["launches"], 1) * 1e3 for k, v in stages.items()},
        "stage_ms_per_step": {k: v["ms"] / nb for k, v in stages.items()},
        "ffn_gateup_timed": {"launches": gu["launches"], "avg_us": gu["ms"] / max(gu["launches"], 1) * 1e3,
                             "GBps": gu["bytes"] / (gu["ms"] * 1e-3) / 1e9 if gu["ms"] > 0 else None},
        "ffn_down": {"avg_us": stages["ffn_down"]["ms"] / max(stages["ffn_down"]["launches"], 1) * 1e3,
                     "GBps": stages["ffn_down"]["bytes"] / (stages["ffn_down"]["ms"] * 1e-3) / 1e9
                     if stages["ffn_down"]["ms"] > 0 else None},
    }


def measure_prefill(ft, torch, ms, blobs, router, dev):
    """One 4096-token chunk through the 48 staged Qwen-A3B-shaped layers, with
    bf16 expert inputs and with x and h MX-quantised (MXFP8, MXFP4).  The MX
    GEMM rate is priced against the MFMA peak of its narrower operand: FP8
    (5.0 PFLOP/s) when either operand is FP8, FP4 (10.1)."""
    w = ms.workload("qwen-a3b-prefill-4096")
    T, L = w.batches[0], w.num_layers
    cfgp = ft.make_config(L, w.hidden, w.inter, w.num_experts, w.top_k, w.layer_fmt, pool_slots=w.pool_slots)
    pool, _ = ft.ft_moe_init_pool(cfgp, blobs, router)
    xs = torch.from_numpy(np.stack([ms.activations(w, l, 0, T) for l in range(L)]).view(np.int16)).to(dev)
    bias = torch.from_numpy(np.stack([ms.popularity_bias(w, l, 0) for l in range(L)])).to(dev)
    out = torch.empty((T, w.hidden), dtype=torch.int16, device=dev)
    res = {"chunk_tokens": T, "layers": L}
    try:
        for name, act, peak in (("bf16", ft.FT_ACT_BF16, None), ("mxfp8", ft.FT_ACT_MXFP8, 5.0e15),
                                ("mxfp4", ft.FT_ACT_MXFP4, 10.1e15)):
            flags = ft.FT_FWD_PREFILL_STAGED | act
            for l in range(L):  # warm
                ft.ft_moe_layer_forward(pool, l, T, xs[l], bias[l], out, flags, None, None)
            torch.cuda.synchronize()
            st0 = ft.ft_moe_pool_stats(pool)
            t0 = time.perf_counter()
            for l in range(L):
                ft.ft_moe_layer_forward(pool, l, T, xs[l], bias[l], out, flags, None, None)
            torch.cuda.synchronize()
            sec = time.perf_counter() - t0
            st1 = ft.ft_moe_pool_stats(pool)
            ft.ft_moe_set_profiling(pool, None)
            ft.ft_moe_profile_read(pool, reset=True)
            for l in range(L):
                ft.ft_moe_layer_forward(pool, l, T, xs[l], bias[l], out, flags, None, None)
            ft.ft_moe_set_profiling(pool, [])
            pr = ft.ft_moe_profile_read(pool, reset=True)
            gemm_ms = pr["ffn_gateup"]["ms"] + pr["ffn_down"]["ms"]
            flops = pr["ffn_gateup"]["flops"] + pr["ffn_down"]["flops"]
            tf = flops / (gemm_ms * 1e-3) if gemm_ms else None
            copied = st1["bytes_h2d"] - st0["bytes_h2d"]
            copy_ms = st1["copy_ms"] - st0["copy_ms"]
            r = {"chunk_s": sec, "tokens_per_s": T / sec,
                 "copy_GBps": copied / (copy_ms * 1e-3) / 1e9 if copy_ms > 0 else None,
                 "ffn_ms_per_layer": gemm_ms / L, "ffn_TFLOPs": tf / 1e12 if tf else None,
                 "gateup_us": pr["ffn_gateup"]["ms"] / max(pr["ffn_gateup"]["launches"], 1) * 1e3,
                 "down_us": pr["ffn_down"]["ms"] / max(pr["ffn_down"]["launches"], 1) * 1e3,
                 "stage_ms_per_layer": {k: v["ms"] / L for k, v in pr.items()}}
            # the pages' copy-bound formula with this run's own copy rate
            if r["copy_GBps"]:
                from oracle import sizing

                r["copy_bound_tokens_per_s"] = sizing.prefill_tokens_per_s(
                    T, sizing.prefill_copy_seconds(copied, r["copy_GBps"] * 1e9))
            if peak and tf:
                r["ffn_peak_TFLOPs"] = peak / 1e12
                r["ffn_frac_of_peak"] = tf / peak
            res[name] = r
            log(f"[bench] prefill {name}: {T / sec:.0f} tokens/s, FFN {gemm_ms / L:.3f} ms/layer"
                + (f" at {tf / 1e12:.0f} TFLOP/s" if tf else ""))
    finally:
        ft.ft_moe_destroy_pool(pool)
    return res


def measure_prefill_hits(ft, torch, ms, run):
    """A 4096-token prefill chunk on the decode pool after its decode steps,
    with FT_FWD_PREFILL_HIT_D2D (experts resident in the pool are read in
    place, only the others are copied) and without it."""
    w, pool, dev = run.w, run.pool, run.dev
    T, L = 4096, w.num_layers
    xs = torch.from_numpy(np.stack([ms.activations(w, l, 5000, T) for l in range(L)]).view(np.int16)).to(dev)
    out = torch.empty((T, w.hidden), dtype=torch.int16, device=dev)
    res = {"chunk_tokens": T}

    def chunk(flags):
        st0 = ft.ft_moe_pool_stats(pool)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for l in range(L):
            ft.ft_moe_layer_forward(pool, l, T, xs[l], run.bias_of(0, l), out, flags, None, None)
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


def measure_graph(ft, torch, run, x_all, B, nrep):
    """Tokens/s of a whole decode step captured once into a HIP graph and
    replayed; each replay's inputs are copied into the captured input buffers
    first (that copy is inside the timing)."""
    pool, dev, L, H = run.pool, run.dev, run.w.num_layers, x_all.shape[-1]
    ft.ft_moe_reserve(pool, B)
    xin = torch.empty((L, B, H), dtype=torch.int16, device=dev)
    outs = torch.empty((L, B, H), dtype=torch.int16, device=dev)
    side = torch.cuda.Stream(dev)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for l in range(L):
            ft.ft_moe_layer_forward(pool, l, B, xin[l], run.bias_of(0, l), outs[l], ft.FT_FWD_DECODE, side, None)
    ns = x_all.shape[0]
    for s in range(2):  # warm replays
        xin.copy_(x_all[s % ns])
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(2, 2 + nrep):
        xin.copy_(x_all[s % ns])
        g.replay()
    torch.cuda.synchronize()
    return B * nrep / (time.perf_counter() - t0)


def qwen_extras(ft, torch, ms, dev, steps, warmup, cpu):
    """Qwen-A3B-shaped decode (batch 16, and 1 / 4), graph replay, the
    one-time mode choice, prefill on the decode pool, and the staged prefill
    chunk in three activation modes."""
    w = ms.workload("qwen-a3b-decode")
    B, L = 16, w.num_layers
    run = DecodeRun(ft, torch, ms, w, B, warmup + steps, dev)
    res = {}
    try:
        # the gate/up launch of one layer per step (rotating over the layers)
        # is timed: an event between two kernels costs a few microseconds of
        # queue time, a percent of a layer here
        elapsed, kernel, prof, st = run.timed(warmup, steps, lambda s: ((s * 7) % L,))
        stages = run.breakdown(warmup, min(8, steps))
        res["decode_b16"] = summarize(run, elapsed, steps, prof, st, stages, min(8, steps))
        gu = prof["ffn_gateup"]
        gbs = gu["bytes"] / (gu["ms"] * 1e-3) / 1e9 if gu["ms"] > 0 else 0.0
        res["decode_b16"]["roofline_gateup"] = {
            "kernel": kernel, "bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": gu["bytes"] / max(gu["launches"], 1),
            "traffic": measured_traffic("ffn_gateup_qwen_a3b_decode_b16_hbm_traffic.md",
                                        gu["bytes"] / max(gu["launches"], 1))}
        log(f"[bench] qwen-a3b decode b16: {res['decode_b16']['tokens_per_s']:.0f} tokens/s, gate/up {gbs:.0f} GB/s")
        for b in (1, 4):
            xb = torch.from_numpy(np.stack([[ms.activations(w, l, 1000 + s, b) for l in range(L)]
                                            for s in range(24)]).view(np.int16)).to(dev)
            ob = torch.empty((b, w.hidden), dtype=torch.int16, device=dev)
            run.steps(0, 8, x_all=xb, out=ob, batch=b)
            torch.cuda.synchronize()
            ta = time.perf_counter()
            run.steps(8, 16, x_all=xb, out=ob, batch=b)
            torch.cuda.synchronize()
            res[f"decode_b{b}_tokens_per_s"] = b * 16 / (time.perf_counter() - ta)
            if b == 1:
                res["graph_b1_tokens_per_s"] = measure_graph(ft, torch, run, xb, 1, 16)
        res["graph_b16_tokens_per_s"] = measure_graph(ft, torch, run, run.x_all, B, 16)
        rep = ft.ft_moe_measure_mode(run.pool, B, apply=False)
        res["mode_choice_b16"] = {
            "mode": ["offload", "hybrid", "fused"][rep["mode"]], "share": rep["share"],
            "balanced_share": rep["balanced_share"], "t_stream_ms": rep["t_stream"] * 1e3,
            "t_cpu_ms": rep["t_cpu"] * 1e3,
            **{f"{k}_GBps": rep[f"{k}_bytes_per_s"][1] / 1e9 for k in ("h2d", "gpu", "cpu")}}
        res["prefill_on_decode_pool"] = measure_prefill_hits(ft, torch, ms, run)
        if cpu:
            sec1 = None
            try:
                from threadpoolctl import threadpool_limits

                with threadpool_limits(limits=1):
                    sec1 = oracle_rate(w, B, 2, 0.0, run.store.expert, 1)
            except ImportError:
                pass
            secn = oracle_rate(w, B, 24, 0.0, run.store.expert, host_threads())
            res["cpu_baseline_b16"] = {"value": B / (secn * L), "cores": host_threads(), "sec_per_call": secn,
                                       "calls": 24}
            if sec1 is not None:
                res["cpu_baseline_b16_one_thread"] = {"value": B / (sec1 * L), "cores": 1, "sec_per_call": sec1,
                                                      "calls": 2}
        run.close()
        blobs = [run.store.expert(l, e) for l in range(L) for e in range(w.num_experts)]
        router = np.stack([ms.router_weight(w, l) for l in range(L)])
        res["prefill"] = measure_prefill(ft, torch, ms, blobs, router, dev)
    finally:
        run.close()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload", default="glm-5.2-mixed-decode",
                    help="decode workload: glm-5.2-mixed-decode (default), deepseek-v4-flash-decode, qwen-a3b-decode")
    ap.add_argument("--steps", type=int, default=20, help="timed decode steps")
    ap.add_argument("--warmup", type=int, default=3, help="untimed decode steps")
    ap.add_argument("--batch", type=int, default=None, help="tokens per call (default: the workload's largest)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-calls", type=int, default=4, help="oracle layer calls in the CPU baseline sample")
    ap.add_argument("--no-extras", action="store_true", help="skip the Qwen-A3B, link, HBM and MFMA measurements")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (reference for HBM byte counters)")
    ap.add_argument("--host-threads", type=int, default=None,
                    help="host worker threads of the hybrid split (default: every core)")
    ap.add_argument("--only", choices=["prefill"], default=None,
                    help="prefill: time only the staged Qwen-A3B prefill chunk (one JSON line of its figures; for "
                         "profiling the prefill kernels)")
    args = ap.parse_args()
    global HYBRID_THREADS
    HYBRID_THREADS = args.host_threads
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the library has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import lru_expert_cache_amd as ft
    import moe_synth as ms

    ft.lib()
    dev = torch.device("cuda", 0)
    if args.only == "prefill":
        wq = ms.workload("qwen-a3b-prefill-4096")
        store = ms.BlobStore(wq)
        blobs = [store.expert(l, e) for l in range(wq.num_layers) for e in range(wq.num_experts)]
        router = np.stack([ms.router_weight(wq, l) for l in range(wq.num_layers)])
        print(json.dumps({"prefill": measure_prefill(ft, torch, ms, blobs, router, dev)}))
        return
    w = ms.workload(args.workload)
    if w.mode != "decode":
        print(f"bench.py times decode workloads; {w.name} is a {w.mode} workload (its chunk is timed as an extra)",
              file=sys.stderr)
        sys.exit(2)
    L, B = w.num_layers, args.batch or w.batches[-1]
    run = DecodeRun(ft, torch, ms, w, B, args.warmup + args.steps, dev)
    try:
        # the dominant kernel: the gate/up FFN of the layers with the largest
        # experts (every such launch is timed; a layer here takes milliseconds,
        # so the events cost nothing measurable)
        big = max(set(w.layer_fmt), key=lambda f: ms.expert_bytes(f, w.hidden, w.inter))
        big_layers = tuple(l for l in range(L) if w.fmt(l) == big)
        elapsed, kernel, prof, st = run.timed(args.warmup, args.steps, lambda s: big_layers)
        shares = {f: ft.ft_moe_get_hybrid_share(run.pool, f) for f in sorted(set(w.layer_fmt))}
        share_used = {FMT_NAME[f]: v for f, v in shares.items()} if w.hybrid else 0.0
        log(f"[bench] timed {args.steps} steps in {elapsed:.3f} s")
        nb = min(2, args.steps)
        stages = run.breakdown(args.warmup, nb)
        head = summarize(run, elapsed, args.steps, prof, st, stages, nb)
        gu = prof["ffn_gateup"]
        gu_gbs = gu["bytes"] / (gu["ms"] * 1e-3) / 1e9 if gu["ms"] > 0 else 0.0
        extras = {"headline": head}
        if run.mode_report is not None:
            rep = run.mode_report
            fm = sorted(set(w.layer_fmt))
            extras["hybrid_measurement"] = {
                "rule_mode": ["offload", "hybrid", "fused"][rep["mode"]], "rule_share": rep["share"],
                "balanced_share_used": rep["balanced_share"], "t_stream_ms": rep["t_stream"] * 1e3,
                "t_cpu_ms": rep["t_cpu"] * 1e3, "rows_per_expert": rep["tokens"],
                **{f"{k}_GBps_{FMT_NAME[f]}": rep[f"{k}_bytes_per_s"][f] / 1e9 for k in ("h2d", "gpu", "cpu")
                   for f in fm}}
            # the in-situ refinement after each warm-up step (ft_moe_rebalance)
            extras["hybrid_measurement"]["rebalance"] = [
                {FMT_NAME[f]: {"share": r["share"][f],
                               "host_GBps": r["host_bytes"][f] / r["host_seconds"][f] / 1e9
                               if r["host_seconds"][f] > 0 else None,
                               "copy_GBps": r["copy_bytes"][f] / r["copy_seconds"][f] / 1e9
                               if r["copy_seconds"][f] > 0 else None} for f in fm}
                for r in run.rebalances]
        cpu = None
        if not args.no_cpu_baseline:
            t = time.perf_counter()
            cpu = cpu_baseline(w, B, args.cpu_calls, shares if w.hybrid else 0.0, run.store.expert)
            log(f"[bench] cpu baseline {time.perf_counter() - t:.1f} s")
    finally:
        run.close()
    del run
    # a plain device copy (2 GiB read + 2 GiB written), the practical HBM rate beside the data sheet's
    extras["hbm_copy_GBps"] = measure_hbm_copy(torch, dev)
    if not args.no_extras:
        link = measure_h2d(torch, dev)
        peak_h2d = max(link.values())
        extras["h2d_sweep_GBps"] = {str(k): round(v, 2) for k, v in link.items()}
        if head["miss_stream_GBps"]:
            extras["miss_stream_frac_of_measured_h2d"] = head["miss_stream_GBps"] / peak_h2d
        extras["qwen_a3b"] = qwen_extras(ft, torch, ms, dev, 20, 5, not args.no_cpu_baseline)
        rq = extras["qwen_a3b"]["decode_b16"]["roofline_gateup"]
        rq["frac_of_measured_copy"] = rq["achieved"] / extras["hbm_copy_GBps"]
        rates = {name: ft.ft_moe_mfma_rate(kind) / 1e12
                 for name, kind in (("fp4_32x32x64", ft.FT_MFMA_FP4_32X32X64),
                                    ("fp8_16x16x128", ft.FT_MFMA_FP8_16X16X128),
                                    ("bf16_16x16x32", ft.FT_MFMA_BF16_16X16X32),
                                    ("bf16_32x32x16", ft.FT_MFMA_BF16_32X32X16),
                                    ("f64_16x16x4", ft.FT_MFMA_F64_16X16X4))}
        extras["mfma_measured_TFLOPs"] = rates
        for mode, key in (("bf16", "bf16_16x16x32"), ("mxfp8", "fp8_16x16x128"), ("mxfp4", "fp4_32x32x64")):
            r = extras["qwen_a3b"]["prefill"].get(mode)
            if r and r.get("ffn_TFLOPs"):
                r["ffn_frac_of_measured_mfma"] = r["ffn_TFLOPs"] / rates[key]
        # the prefill router (fp64 logits on the matrix cores), 2 T E H flop per layer
        pf, wq = extras["qwen_a3b"]["prefill"], ms.workload("qwen-a3b-prefill-4096")
        rt = pf.get("mxfp4", {}).get("stage_ms_per_layer", {}).get("router")
        if rt:
            tf = 2.0 * pf["chunk_tokens"] * wq.num_experts * wq.hidden / (rt * 1e-3) / 1e12
            pf["router"] = {"us_per_layer": rt * 1e3, "TFLOPs": tf, "frac_of_sheet_fp64": tf / 78.6,
                            "frac_of_measured_fp64": tf / rates["f64_16x16x4"]}
    if args.calibrate_copy:
        a = torch.empty(128 << 20, dtype=torch.int16, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        extras["calibration_copy_bytes"] = a.numel() * 2

    fmts = sorted(set(w.layer_fmt))
    traffic_profile = f"ffn_gateup_{FMT_NAME[big]}_{w.name}_b{B}_hbm_traffic.md"
    result = {
        "metric": "MoE-layer tokens/s (decode & prefill); % HBM BW / FP4 MFMA peak; hit rate",
        "value": B * args.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "|".join(FMT_NAME[f] for f in fmts) + "-weights/bf16-act/fp32-acc",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": L, "hidden": w.hidden, "expert_inter": w.inter,
                   "experts": w.num_experts, "top_k": w.top_k, "batch": B, "pool_slots": w.pool_slots,
                   "format": "|".join({1: "mxfp4", 2: "nvfp4", 3: "fp8-b128"}[f] for f in fmts),
                   "zipf_alpha": w.zipf_alpha, "popularity_shift_steps": w.phase_steps,
                   "shared_expert": w.shared_expert, "hybrid_share": share_used,
                   "host_threads": hybrid_threads() if w.hybrid else 0,
                   "host_blob_aliasing": w.n_blobs},
        "roofline": {"kernel": kernel, "bound": "hbm", "achieved": gu_gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": gu_gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic(traffic_profile, gu["bytes"] / max(gu["launches"], 1)),
                     "algorithmic_bytes_per_launch": gu["bytes"] / max(gu["launches"], 1),
                     "avg_launch_us": gu["ms"] / max(gu["launches"], 1) * 1e3, "launches": gu["launches"],
                     "frac_of_measured_copy": gu_gbs / extras["hbm_copy_GBps"],
                     "layers_timed": f"every {FMT_NAME[big]} layer"},
        "cpu_baseline": cpu,
        "extras": extras,
    }
    print(json.dumps(result))


if __name__ == "__main__":
    main()
