"""Benchmark of the IO-aware exact attention hot path on one MI355X.

Default run (no flags): N=1 GPU, the long-sequence bf16 workload
B=1 H=16 N=16384 d=128 (non-causal), Q/K/V ~ N(0,1) from seed 0. One step =
one forward pass (fa_fwd) plus one backward pass (fa_bwd) over that batch,
inputs already resident in HBM. Prints ONE JSON line.

FLOP convention: forward 4*B*H*N^2*d (halved when causal); backward 2.5x
the forward. value = (fwd + bwd FLOP) / step time, in TFLOP/s.

Roofline: every fa_fwd and fa_bwd call in the timed region is bracketed by
HIP events on the stream it runs on. fa_fwd is one kernel. fa_bwd (16-bit
types) is three kernels back to back on that stream: the row term D
(memory-bound, well under 1% of the call), the key-outer dK/dV kernel and
the query-outer dQ kernel, which together hold all the matrix work; the
committed rocprofv3 trace gives their split. `roofline` describes the
direction that takes longer; `roofline_fwd` / `roofline_bwd` give both.
achieved = algorithmic FLOP per call / mean call duration, against the
MI355X dense bf16/fp16 MFMA peak (2.5 PFLOP/s; fp32 MFMA: 157.3 TFLOP/s).
`traffic` (measured HBM bytes per call: FETCH_SIZE and WRITE_SIZE scaled by
what the same counters read for a plain copy of known size) is read from the
committed rocprofv3 counter summary only when that summary was taken from
the current kernel sources (their hash is recorded in it), else null.

cpu_baseline: the CPU oracle (float64 numpy) on a bounded sample of the same
workload -- whole heads, forward and backward, until ~10 s have elapsed --
reported in the same unit.

Other modes (used to collect the rocprofv3 summaries under profiles/):
  --only fwd|bwd        time only that direction (no CPU baseline)
  --sweep               forward over N in {1k,2k,4k,8k,16k}, B=1 H=16 d=128
  --sweep-bwd           the same for the backward (after one forward per N)
  --variants            split-KV, grouped K/V heads, a local window and the
                        8-bit float forward against the plain calls (one JSON
                        line per case)
  --fp8                 the E4M3 forward alone, B=1 H=16 N=16384 d=128
  --small               small grids: the causal B=2 H=8 N=1024 d=64 workload
                        through fa_fwd, each forward kernel and split-KV, the
                        fixed cost of a launch and the host time of one call
  --copy-bytes BYTES    a plain device copy of BYTES bytes (counter scaling)
  --summarize DIR       turn rocprofv3 output under DIR into a text table
  --summarize-by-grid DIR   kernel-trace durations per (kernel, grid size)
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd/bwd TFLOP/s (bf16, N=4k-16k, d=128) and % of MFMA peak"
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}  # MI355X dense MFMA
PEAK_FP8_TFLOPS = 5033.2  # MI355X dense FP8 (E4M3) MFMA
KERNEL_SOURCES = {
    "fwd": ["exact_attention_120_amd/csrc/fa_fwd.hip", "exact_attention_120_amd/csrc/fa_device.hpp"],
    "bwd": ["exact_attention_120_amd/csrc/fa_bwd.hip", "exact_attention_120_amd/csrc/fa_device.hpp"],
}
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "fa_bf16_n16k_d128_hbm_traffic.md")


def kernel_source_hash(direction: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[direction]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(direction: str, workload: str):
    """Per-call HBM bytes from the committed counter summary, if current."""
    if workload != "bf16_n16k_d128" or not os.path.exists(TRAFFIC_SUMMARY):
        return None
    text = open(TRAFFIC_SUMMARY).read()
    m_hash = re.search(direction + r"-kernel-source-hash:\s*([0-9a-f]+)", text)
    m_bytes = re.search(direction + r"-hbm-bytes-per-call:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash(direction):
        return None
    return float(m_bytes.group(1))


def cpu_baseline(w, inputs, budget_s=10.0, max_s=30.0):
    """Time the float64 oracle (fwd + bwd) over whole heads of the workload."""
    import numpy as np
    import threadpoolctl

    from fa_inputs import to_f64
    from oracle import attention_backward, attention_forward

    q, k, v, do = (to_f64(inputs[n]) for n in ("q", "k", "v", "do"))
    q, k, v, do = (x.reshape(-1, w.N, w.d) for x in (q, k, v, do))
    heads, flop, t0 = 0, 0.0, time.perf_counter()
    per_head = (w.fwd_flops() + w.bwd_flops()) / (w.B * w.H)
    while heads < q.shape[0]:
        o, _ = attention_forward(q[heads], k[heads], v[heads], w.scale, w.causal)
        attention_backward(q[heads], k[heads], v[heads], do[heads], w.scale, w.causal)
        np.asarray(o)
        heads += 1
        flop += per_head
        el = time.perf_counter() - t0
        if el >= budget_s or el + el / heads > max_s:
            break
    el = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] or [1])
    cores = len(os.sched_getaffinity(0))
    return {"value": flop / el / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "blas_threads": threads,
            "sample": f"float64 numpy oracle, forward + backward of {heads} of {w.B * w.H} "
                      f"heads (all {w.N} rows each) of this workload, {el:.1f} s; "
                      f"{cores} host cores available, BLAS threads {threads}"}


def per_call_ms(fn, min_s=0.25, max_calls=4096):
    """Mean duration of fn() (one library call on the current stream), from
    HIP events around back-to-back calls: doubles the call count until the
    timed batch lasts at least min_s."""
    import torch

    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    n = 1
    while True:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        if ms * 1e-3 >= min_s or n >= max_calls:
            return ms / n
        n *= 2


def config_rates(peak):
    """Forward (and where the workload has one, backward) rates of every named
    workload other than the headline one, and a TFLOP/s-versus-N sweep, each
    timed with HIP events on the stream the calls run on. Returns a dict for
    the JSON line."""
    import torch

    import exact_attention_120_amd as fa
    from fa_inputs import WORKLOADS, make_inputs, workload_inputs

    dev = torch.device("cuda:0")

    def rates(q, k, v, do, scale, causal, fwd_flop, with_bwd, pk):
        B, H, N, d = q.shape
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        f_ms = per_call_ms(lambda: fa.fa_fwd(q, k, v, o, lse, scale, causal))
        r = {"fwd_ms": f_ms, "fwd_tflops": fwd_flop / (f_ms * 1e-3) / 1e12}
        r["fwd_frac_of_peak"] = r["fwd_tflops"] / pk
        if with_bwd:
            dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
            ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d), dtype=torch.uint8, device=dev)
            b_ms = per_call_ms(lambda: fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, scale, causal,
                                                 ws))
            r.update(bwd_ms=b_ms, bwd_tflops=2.5 * fwd_flop / (b_ms * 1e-3) / 1e12)
            r["bwd_frac_of_peak"] = r["bwd_tflops"] / pk
        return r

    out = {}
    for name, with_bwd in (("tiny_f32", False), ("causal_bf16_n1k", False),
                           ("bf16_n4k_d128", True), ("bf16_n16k_d128_causal", True),
                           ("f16_n2k_fwdbwd_causal", True)):
        w = WORKLOADS[name]
        inp = workload_inputs(type(w)(**{**w.__dict__, "backward": True}))
        q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
        pk = PEAK_TFLOPS[w.dtype]
        r = rates(q, k, v, do, w.scale, w.causal, w.fwd_flops(), with_bwd, pk)
        out[name] = dict({"B": w.B, "H": w.H, "N": w.N, "d": w.d, "dtype": w.dtype,
                          "causal": w.causal}, **r)
        del q, k, v, do, inp
    # Sequence-length sweep, bf16 d=128, 16384 tokens per call (B = 16384/N,
    # H = 16), both causal settings; inputs N(0,1) drawn on the device from a
    # seeded generator (timing only).
    sweep = []
    g = torch.Generator(device=dev)
    for N in (512, 1024, 2048, 4096, 8192, 16384):
        B, H, d = 16384 // N, 16, 128
        g.manual_seed(N)
        q, k, v, do = (torch.randn((B, H, N, d), generator=g, device=dev).to(torch.bfloat16)
                       for _ in range(4))
        for causal in (False, True):
            fl = 4.0 * B * H * N * N * d / (2 if causal else 1)
            r = rates(q, k, v, do, 128 ** -0.5, causal, fl, True, PEAK_TFLOPS["bf16"])
            sweep.append(dict({"B": B, "H": H, "N": N, "d": d, "causal": causal}, **r))
        del q, k, v, do
    return out, sweep


def time_calls(fn, steps, warmup, events_per_call, warmup_s=0.0):
    """Run fn() warmup+steps times; returns (total_ms, [per-call event ms lists]).

    The untimed warm-up runs at least `warmup` steps and at least `warmup_s`
    seconds: the GPU's clock ramps up over the first second of sustained
    load, and a short warm-up would time the ramp instead of the kernels.
    """
    import torch

    t0 = time.perf_counter()
    done = 0
    while done < warmup or time.perf_counter() - t0 < warmup_s:
        fn(None)
        done += 1
        if done % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(events_per_call + 1)]
          for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        fn(ev[i])
    end.record()
    torch.cuda.synchronize()
    total = start.elapsed_time(end)
    per = [[e[j].elapsed_time(e[j + 1]) for e in ev] for j in range(events_per_call)]
    return total, per


def run_main(args):
    import torch

    import exact_attention_120_amd as fa
    from fa_inputs import WORKLOADS, workload_inputs

    w = WORKLOADS[args.workload]
    if w.dtype != "bf16" and args.workload == "bf16_n16k_d128":
        raise SystemExit("unexpected workload table")
    inp = workload_inputs(type(w)(**{**w.__dict__, "backward": True}))
    dev = torch.device("cuda:0")
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d), dtype=torch.uint8, device=dev)
    do_fwd, do_bwd = args.only in (None, "fwd"), args.only in (None, "bwd")
    if do_bwd:  # the backward needs a forward output
        fa.fa_fwd(q, k, v, o, lse, w.scale, w.causal)
        torch.cuda.synchronize()

    def step(ev):
        j = 0
        if ev is not None:
            ev[j].record()
        if do_fwd:
            fa.fa_fwd(q, k, v, o, lse, w.scale, w.causal)
            if ev is not None:
                j += 1
                ev[j].record()
        if do_bwd:
            fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, w.scale, w.causal, ws)
            if ev is not None:
                j += 1
                ev[j].record()

    n_ev = int(do_fwd) + int(do_bwd)
    total_ms, per = time_calls(step, args.steps, args.warmup, n_ev, args.warmup_seconds)
    ms_step = total_ms / args.steps
    fwd_flop, bwd_flop = w.fwd_flops(), w.bwd_flops()
    flop = fwd_flop * do_fwd + bwd_flop * do_bwd
    peak = PEAK_TFLOPS[w.dtype]
    out = {
        "metric": METRIC, "value": flop / (ms_step * 1e-3) / 1e12, "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "N": N, "d": d, "causal": w.causal,
                   "step": "+".join(x for x, on in (("fwd", do_fwd), ("bwd", do_bwd)) if on),
                   "inputs": "Q,K,V,dO ~ N(0,1) float32 from seed 0, rounded to bf16"},
        "frac_of_peak": flop / (ms_step * 1e-3) / 1e12 / peak,
    }
    j, roofs = 0, {}
    for name, on, fl, kern in (
            ("fwd", do_fwd, fwd_flop, "fwd_pp_kernel (the one kernel of fa_fwd)"),
            ("bwd", do_bwd, bwd_flop, "fa_bwd call: bwd_pre_kernel (D, <1%) + bwd_kv16_kernel"
                                      " (dK, dV) + bwd_dq16_kernel (dQ)")):
        if not on:
            continue
        ms = sum(per[j]) / len(per[j])
        tf = fl / (ms * 1e-3) / 1e12
        out[name] = {"ms": ms, "tflops": tf, "frac_of_peak": tf / peak}
        roofs[name] = {"bound": "mfma", "achieved": tf, "peak": peak, "unit": "TFLOP/s",
                       "frac": tf / peak, "traffic": read_traffic(name, w.name),
                       "kernel": kern, "flop_per_call": fl, "ms_per_call": ms}
        j += 1
    dominant = max(roofs, key=lambda n: roofs[n]["ms_per_call"])
    out["roofline"] = dict(roofs[dominant], direction=dominant)
    for name, r in roofs.items():
        out["roofline_" + name] = r
    if args.only is None and not args.no_configs:
        out["configs"], out["sweep_bf16_d128"] = config_rates(peak)
    if args.only is None and not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inp)
    print(json.dumps(out), flush=True)


def run_sweep(args):
    import torch

    import exact_attention_120_amd as fa
    from fa_inputs import make_inputs

    for n in (1024, 2048, 4096, 8192, 16384):
        for causal in (False, True):
            inp = make_inputs(1, 16, n, 128, "bf16", seed=0)
            q, k, v = (inp[x].to("cuda:0") for x in ("q", "k", "v"))
            o, lse = torch.empty_like(q), torch.empty((1, 16, n), device="cuda:0")
            for _ in range(3):
                fa.fa_fwd(q, k, v, o, lse, 128 ** -0.5, causal)
            torch.cuda.synchronize()
            print(json.dumps({"sweep_N": n, "causal": causal}), flush=True)


def run_sweep_bwd(args):
    """Backward over N in {1k, 2k, 4k, 8k, 16k}, B=1 H=16 d=128, both causal
    settings: one forward for O and LSE, then three fa_bwd calls (for the
    HBM-bytes-versus-N counters)."""
    import torch

    import exact_attention_120_amd as fa
    from fa_inputs import make_inputs

    for n in (1024, 2048, 4096, 8192, 16384):
        for causal in (False, True):
            inp = make_inputs(1, 16, n, 128, "bf16", seed=0, backward=True)
            q, k, v, do = (inp[x].to("cuda:0") for x in ("q", "k", "v", "do"))
            o, lse = torch.empty_like(q), torch.empty((1, 16, n), device="cuda:0")
            dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
            ws = torch.empty(fa.fa_bwd_workspace_size(1, 16, n, 128), dtype=torch.uint8, device="cuda:0")
            fa.fa_fwd(q, k, v, o, lse, 128 ** -0.5, causal)
            for _ in range(3):
                fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, 128 ** -0.5, causal, ws)
            torch.cuda.synchronize()
            print(json.dumps({"sweep_bwd_N": n, "causal": causal}), flush=True)


def run_variants(args):
    """Time the variant rows against the plain calls (HIP events on the
    current stream, back-to-back calls with preallocated buffers): split-KV
    on short/few-head shapes, grouped K/V heads and a local window at
    N = 16384, block-sparse masks at N = 16384, and the E4M3 forward against
    the bf16 one. One JSON line per case."""
    import torch

    import exact_attention_120_amd as fa
    from fa_inputs import make_inputs

    dev = torch.device("cuda:0")

    def per_call_ms(fn):
        return globals()["per_call_ms"](fn, min_s=0.4)

    # Split-KV: the library's slice count and fixed counts against fa_fwd.
    for (B, H, N, d, causal) in ((2, 8, 1024, 64, True), (1, 8, 2048, 128, False),
                                 (1, 4, 4096, 128, True)):
        inp = make_inputs(B, H, N, d, "bf16", seed=0)
        q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
        o, lse = torch.empty_like(q), torch.empty((B, H, N), device=dev)
        sc = d ** -0.5
        flop = 4.0 * B * H * N * N * d / (2 if causal else 1)
        res = {"case": "splitkv", "B": B, "H": H, "N": N, "d": d, "causal": causal,
               "auto_splits": fa.fa_fwd_num_splits(B, H, N, d, q.dtype)}
        res["plain_us"] = per_call_ms(lambda: fa.fa_fwd(q, k, v, o, lse, sc, causal)) * 1e3
        for ns in sorted({2, 4, 8, res["auto_splits"]}):
            nb = fa.fa_fwd_splitkv_workspace_size(B, H, N, d, q.dtype, ns)
            ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
            res[f"split{ns}_us"] = per_call_ms(
                lambda: fa.fa_fwd_splitkv(q, k, v, o, lse, sc, causal, ns, ws)) * 1e3
        best = min(v for kk, v in res.items() if kk.startswith("split"))
        res["plain_tflops"] = flop / (res["plain_us"] * 1e-6) / 1e12
        res["best_split_tflops"] = flop / (best * 1e-6) / 1e12
        print(json.dumps(res), flush=True)

    # Grouped K/V heads and a local window, forward and backward, bf16
    # B=1 H=16 N=16384 d=128. FLOP counts only the visible (query, key) pairs.
    B, H, N, d = 1, 16, 16384, 128
    sc = d ** -0.5
    for (hkv, causal, window) in ((16, False, None), (4, False, None), (1, False, None),
                                  (16, True, None), (4, True, (1024, 0))):
        inp = make_inputs(B, H, N, d, "bf16", seed=0, backward=True, kv_heads=hkv)
        q, k, v, do = (inp[x].to(dev) for x in ("q", "k", "v", "do"))
        o, lse = torch.empty_like(q), torch.empty((B, H, N), device=dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d), dtype=torch.uint8, device=dev)
        if window is None:
            pairs = N * N / 2 if causal else N * N
        else:
            i = torch.arange(N, dtype=torch.float64)
            pairs = float((torch.clamp(i, max=window[0]) + 1).sum())
        fl = 4.0 * B * H * pairs * d
        f_ms = per_call_ms(lambda: fa.fa_fwd_ex(q, k, v, o, lse, sc, causal, window))
        b_ms = per_call_ms(lambda: fa.fa_bwd_ex(q, k, v, o, do, lse, dq, dk, dv, sc, causal, ws,
                                                window))
        print(json.dumps({"case": "heads_window", "B": B, "H": H, "Hkv": hkv, "N": N, "d": d,
                          "causal": causal, "window": window, "fwd_ms": f_ms, "bwd_ms": b_ms,
                          "fwd_tflops": fl / (f_ms * 1e-3) / 1e12,
                          "bwd_tflops": 2.5 * fl / (b_ms * 1e-3) / 1e12}), flush=True)

    # Block-sparse masks (64 x 64 blocks) at B=1 H=16 N=16384 d=128, forward
    # and backward, against the dense calls. FLOP counts the visible
    # (query, key) pairs only; "dense" is the all-ones mask (the sparse
    # kernels' overhead over the plain ones).
    from fa_inputs import make_block_mask
    inp = make_inputs(B, H, N, d, "bf16", seed=0, backward=True)
    q, k, v, do = (inp[x].to(dev) for x in ("q", "k", "v", "do"))
    o, lse = torch.empty_like(q), torch.empty((B, H, N), device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d), dtype=torch.uint8, device=dev)
    for causal in (False, True):
        f_dense = per_call_ms(lambda: fa.fa_fwd(q, k, v, o, lse, sc, causal))
        b_dense = per_call_ms(lambda: fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, sc, causal, ws))
        for kind, dens in (("dense", 1.0), ("random", 0.5), ("random", 0.25),
                           ("band_global", 0.05)):
            m = make_block_mask(N, kind, seed=0, density=dens)
            ib, jb = torch.meshgrid(torch.arange(m.shape[0]), torch.arange(m.shape[0]),
                                    indexing="ij")
            per_block = (torch.where(jb < ib, 4096.0, torch.where(jb == ib, 2080.0, 0.0))
                         if causal else torch.full(m.shape, 4096.0))
            pairs = float((per_block * (m != 0)).sum())
            fl = 4.0 * B * H * pairs * d
            md = m.to(dev)
            f_ms = per_call_ms(lambda: fa.fa_fwd_sparse(q, k, v, o, lse, sc, causal, md))
            b_ms = per_call_ms(lambda: fa.fa_bwd_sparse(q, k, v, o, do, lse, dq, dk, dv, sc,
                                                        causal, md, ws))
            print(json.dumps({"case": "block_sparse", "B": B, "H": H, "N": N, "d": d,
                              "causal": causal, "mask": kind, "density": dens,
                              "kept_blocks": float((m != 0).float().mean()),
                              "fwd_ms": f_ms, "bwd_ms": b_ms,
                              "dense_fwd_ms": f_dense, "dense_bwd_ms": b_dense,
                              "fwd_tflops": fl / (f_ms * 1e-3) / 1e12,
                              "bwd_tflops": 2.5 * fl / (b_ms * 1e-3) / 1e12,
                              "fwd_speedup_vs_dense": f_dense / f_ms,
                              "bwd_speedup_vs_dense": b_dense / b_ms}), flush=True)

    # 8-bit float forward (E4M3 Q, K, V, bf16 O) against the bf16 forward on
    # the same shape. Peak: MI355X dense FP8 MFMA, 5.0 PFLOP/s.
    from fa_inputs import make_fp8_inputs
    for (B, H, N, d, causal) in ((1, 16, 16384, 128, False), (1, 16, 16384, 128, True),
                                 (4, 16, 4096, 128, False), (2, 16, 4096, 64, False)):
        x = make_fp8_inputs(B, H, N, d, seed=0)
        q8, k8, v8 = (x[n].to(dev) for n in ("q8", "k8", "v8"))
        inp = make_inputs(B, H, N, d, "bf16", seed=0)
        q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
        o, lse = torch.empty_like(q), torch.empty((B, H, N), device=dev)
        sc = d ** -0.5
        fl = 4.0 * B * H * N * N * d / (2 if causal else 1)
        f8_ms = per_call_ms(lambda: fa.fa_fwd_fp8(q8, k8, v8, o, lse, sc, causal, *x["descale"]))
        b16_ms = per_call_ms(lambda: fa.fa_fwd(q, k, v, o, lse, sc, causal))
        print(json.dumps({"case": "fp8_fwd", "B": B, "H": H, "N": N, "d": d, "causal": causal,
                          "fp8_ms": f8_ms, "bf16_ms": b16_ms,
                          "fp8_tflops": fl / (f8_ms * 1e-3) / 1e12,
                          "fp8_frac_of_peak": fl / (f8_ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS,
                          "bf16_tflops": fl / (b16_ms * 1e-3) / 1e12,
                          "speedup_vs_bf16": b16_ms / f8_ms}), flush=True)


def run_small(args):
    """Small grids: the causal bf16 B=2 H=8 N=1024 d=64 workload (64
    workgroups of 256 rows) through fa_fwd (which picks the key-split kernel
    here), through each forward kernel alone and with 2, 4, 8 key slices; the
    fixed cost of a launch -- bf16 B=16 H=16 non-causal at N = 64 .. 1024 (one
    workgroup per CU up to N = 256) for d = 64 and 128 -- beside a one-element
    torch kernel timed the same way (the floor of back-to-back launches); and
    the host time of one call through the binding and through the C ABI.
    HIP events on the current stream; one JSON line per case."""
    import torch

    import exact_attention_120_amd as fa
    from fa_inputs import make_inputs

    dev = torch.device("cuda:0")
    B, H, N, d = 2, 8, 1024, 64
    inp = make_inputs(B, H, N, d, "bf16", seed=0)
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    o, lse = torch.empty_like(q), torch.empty((B, H, N), device=dev)
    sc = d ** -0.5
    res = {"case": "small_causal", "B": B, "H": H, "N": N, "d": d,
           "fa_fwd_us": per_call_ms(lambda: fa.fa_fwd(q, k, v, o, lse, sc, True)) * 1e3,
           "key_split_us": per_call_ms(lambda: fa.fa_fwd_keysplit(q, k, v, o, lse, sc, True)) * 1e3,
           "row_tiles_us": per_call_ms(
               lambda: fa.fa_fwd_splitkv(q, k, v, o, lse, sc, True, 1, None)) * 1e3}
    for ns in (2, 4, 8):
        ws = torch.empty(fa.fa_fwd_splitkv_workspace_size(B, H, N, d, q.dtype, ns),
                         dtype=torch.uint8, device=dev)
        res[f"split{ns}_us"] = per_call_ms(
            lambda: fa.fa_fwd_splitkv(q, k, v, o, lse, sc, True, ns, ws)) * 1e3
    print(json.dumps(res), flush=True)
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    for dd in (64, 128):
        for n in (64, 128, 256, 512, 1024):
            q, k, v = (torch.randn((16, 16, n, dd), generator=g, device=dev).to(torch.bfloat16)
                       for _ in range(3))
            o, lse = torch.empty_like(q), torch.empty((16, 16, n), device=dev)
            us = per_call_ms(lambda: fa.fa_fwd(q, k, v, o, lse, dd ** -0.5, False)) * 1e3
            print(json.dumps({"case": "fixed_cost", "B": 16, "H": 16, "N": n, "d": dd,
                              "workgroups": 256 * ((n + 255) // 256),
                              "key_tiles_per_workgroup": (n + 63) // 64, "us": us}), flush=True)
    x = torch.zeros(1, device=dev)
    print(json.dumps({"case": "launch_floor", "kernel": "torch add_ on one element",
                      "us": per_call_ms(lambda: x.add_(1.0)) * 1e3}), flush=True)
    # Host time of one call: through the Python binding, and straight through
    # the C ABI with the arguments prepared once (B=16 H=16 N=64 d=64, one
    # key tile per workgroup; the GPU keeps up, so these are host-bound).
    from exact_attention_120_amd import _lib
    q, k, v = (torch.randn((16, 16, 64, 64), generator=g, device=dev).to(torch.bfloat16)
               for _ in range(3))
    o, lse = torch.empty_like(q), torch.empty((16, 16, 64), device=dev)
    lib = _lib.load()
    raw = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), 16, 16, 64, 64,
           0.125, 0, fa.DTYPES[q.dtype], torch.cuda.current_stream().cuda_stream)

    def host_us(fn, n=4000):
        for _ in range(100):
            fn()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(n):
            fn()
        us = (time.perf_counter() - t) / n * 1e6
        torch.cuda.synchronize()
        return us
    print(json.dumps({"case": "host_call", "B": 16, "H": 16, "N": 64, "d": 64,
                      "binding_us": host_us(lambda: fa.fa_fwd(q, k, v, o, lse, 0.125, False)),
                      "c_abi_us": host_us(lambda: lib.fa_fwd(*raw)),
                      "torch_add_us": host_us(lambda: x.add_(1.0))}), flush=True)


def run_fp8(args):
    """The E4M3 forward alone at B=1 H=16 N=16384 d=128 (non-causal), timed
    like the main line; one JSON line (used for its rocprofv3 summaries)."""
    import torch

    import exact_attention_120_amd as fa
    from fa_inputs import make_fp8_inputs

    B, H, N, d = 1, 16, 16384, 128
    dev = torch.device("cuda:0")
    x = make_fp8_inputs(B, H, N, d, seed=0)
    q8, k8, v8 = (x[n].to(dev) for n in ("q8", "k8", "v8"))
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    sc = float(torch.tensor(d ** -0.5, dtype=torch.float32))

    def step(ev):
        if ev is not None:
            ev[0].record()
        fa.fa_fwd_fp8(q8, k8, v8, o, lse, sc, False, *x["descale"])
        if ev is not None:
            ev[1].record()

    total_ms, per = time_calls(step, args.steps, args.warmup, 1, args.warmup_seconds)
    ms = sum(per[0]) / len(per[0])
    tf = 4.0 * B * H * N * N * d / (ms * 1e-3) / 1e12
    print(json.dumps({"case": "fp8_fwd", "B": B, "H": H, "N": N, "d": d, "causal": False,
                      "steps": args.steps, "ms_per_call": ms, "tflops": tf,
                      "frac_of_fp8_peak": tf / PEAK_FP8_TFLOPS}), flush=True)


def run_copy(args):
    import torch

    n = args.copy_bytes // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n * 4}), flush=True)


def _short(name: str) -> str:
    """Readable kernel name from a (possibly mangled) symbol."""
    m = re.search(r"(fwd_pp_kernel|fwd_ks_kernel|fwd_fp8_kernel|fwd_kernel|fwd_merge_kernel|"
                  r"bwd_kv16_kernel|bwd_fused16_kernel|bwd_kvsum_kernel|"
                  r"bwd_main_kernel|"
                  r"bwd_pre_kernel|bwd_dq16_kernel|bwd_dq_kernel)I(.*?)EEv", name)
    if m and m.group(1) == "fwd_fp8_kernel":  # <D, CAUSAL, output type>
        a = m.group(2)
        d = re.search(r"Li(\d+)E", a)
        return (f"fwd_fp8_kernel<d={d.group(1) if d else '?'},"
                f"{'causal' if 'Lb1' in a else 'noncausal'},out="
                f"{'bf16' if 'DF16b' in a else 'f16'}>")
    if m:
        a = m.group(2)
        ty = "bf16" if a.startswith("DF16b") else "f16" if a.startswith("DF16_") else \
            "f32" if a.startswith("f") else ""
        d = re.search(r"Li(\d+)E", a)
        flags = re.findall(r"Lb([01])E", a)
        parts = [ty] + ([f"d={d.group(1)}"] if d else [])
        if flags:
            parts.append("causal" if flags[0] == "1" else "noncausal")
        if len(flags) > 1 and flags[1] == "1":
            parts.append("sparse")
        return m.group(1) + "<" + ",".join(p for p in parts if p) + ">"
    return name[:70]


def summarize_by_grid(path):
    """Median and minimum duration per (kernel, grid size) from the rocprofv3
    kernel traces found under path (one row per distinct launch shape)."""
    rows = {}
    for f in sorted(glob.glob(os.path.join(path, "**", "*kernel_trace.csv"), recursive=True)):
        for r in csv.DictReader(open(f)):
            grid = r.get("Grid_Size") or r.get("Grid_Size_X") or ""
            d = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            rows.setdefault((_short(r["Kernel_Name"]), grid), []).append(d)
    print("| kernel | grid (threads) | dispatches | median ns | min ns |")
    print("|---|---|---|---|---|")
    for (k, g), v in sorted(rows.items(), key=lambda x: (x[0][0], int(x[0][1] or 0))):
        v.sort()
        print(f"| {k} | {g} | {len(v)} | {v[len(v) // 2]} | {v[0]} |")


def summarize(path):
    """Print per-kernel tables from rocprofv3 CSV output found under path."""
    for f in sorted(glob.glob(os.path.join(path, "**", "*kernel_stats.csv"), recursive=True)):
        print("| kernel | calls | average ns | min ns | max ns | % time |")
        print("|---|---|---|---|---|---|")
        for r in csv.DictReader(open(f)):
            print(f"| {_short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                  f"{r['MinNs']} | {r['MaxNs']} | {float(r['Percentage']):.2f} |")
    rows = []
    for f in glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    if rows:
        agg = {}
        for r in rows:
            key = (_short(r.get("Kernel_Name", "?")), r.get("Grid_Size", ""),
                   r.get("Counter_Name", ""))
            agg.setdefault(key, []).append(float(r.get("Counter_Value", 0)))
        print("| kernel | grid | counter | dispatches | mean value per dispatch |")
        print("|---|---|---|---|---|")
        for (kname, grid, cname), vals in sorted(agg.items()):
            print(f"| {kname} | {grid} | {cname} | {len(vals)} | {sum(vals) / len(vals):.6g} |")
    for d in ("fwd", "bwd"):
        print(f"{d}-kernel-source-hash (current tree): {kernel_source_hash(d)}")


def main():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--warmup-seconds", type=float, default=1.5,
                   help="minimum untimed warm-up time (clock ramp-up), in seconds")
    p.add_argument("--workload", default="bf16_n16k_d128")
    p.add_argument("--only", choices=["fwd", "bwd"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-configs", action="store_true",
                   help="skip the other workloads' rates and the N sweep")
    p.add_argument("--sweep", action="store_true")
    p.add_argument("--sweep-bwd", action="store_true")
    p.add_argument("--variants", action="store_true")
    p.add_argument("--fp8", action="store_true")
    p.add_argument("--small", action="store_true")
    p.add_argument("--copy-bytes", type=int)
    p.add_argument("--summarize")
    p.add_argument("--summarize-by-grid")
    args = p.parse_args()
    if args.summarize:
        return summarize(args.summarize)
    if args.summarize_by_grid:
        return summarize_by_grid(args.summarize_by_grid)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(heads shard across GPUs with no communication; see the design notes)",
              file=sys.stderr)
        raise SystemExit(2)
    if args.copy_bytes:
        return run_copy(args)
    if args.sweep:
        return run_sweep(args)
    if args.sweep_bwd:
        return run_sweep_bwd(args)
    if args.variants:
        return run_variants(args)
    if args.fp8:
        return run_fp8(args)
    if args.small:
        return run_small(args)
    return run_main(args)


if __name__ == "__main__":
    main()
