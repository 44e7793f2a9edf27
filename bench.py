#!/usr/bin/env python3
"""Throughput of exact attention (forward + backward) on one MI355X.

One step is the whole hot path on one batch of seeded synthetic input:
fa_fwd, then the backward as the two launches fa_bwd enqueues (fa_bwd_dq,
which also forms D_i = rowsum(dO * O), then fa_bwd_dkdv), all on one stream. The workload is the
GPT-2-shaped forward+backward case: B=8, H=12, N=1024, d=64, bf16, causal,
Q, K, V, dO ~ N(0, 1) from seed 0 (the only listed workload with a
backward; the other shapes are parity-test cases and appear here only under
"extra"). Inputs are resident in HBM before the timed region starts.

Algorithmic work (what the method must do, not what the kernels happen to
do): forward 4*B*H*N^2*d, backward 2.5x that (five N^2 d products: S
recompute, dP, dV, dK, dQ), both halved for causal.

The timed region is K whole steps with nothing else on the stream. Each
kernel's average duration (for the roofline object) is then taken with two
HIP events around K back-to-back launches of that kernel alone.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd/bwd TFLOP/s and % of bf16 MFMA peak on 1x MI355X"
# MI355X dense peaks: bf16/fp16 MFMA 256 CU x 4096 FLOP/clk x 2.4 GHz, HBM3E 8 TB/s.
PEAK_BF16_FLOPS = 256 * 4096 * 2.4e9
PEAK_HBM_BYTES = 8.0e12
PEAK_FP8_FLOPS = 256 * 8192 * 2.4e9  # dense FP8 matrix-core rate, twice bf16
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")

# roofline bound of each kernel of the step
BOUND = {"fwd": "mfma", "dq": "mfma", "dkdv": "mfma"}
WARM_SECONDS = 1.5


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def fwd_flops(w) -> float:
    return 4.0 * w.B * w.H * w.N * w.N * w.d * (0.5 if w.causal else 1.0)


def compulsory_bytes(w, backward: bool) -> float:
    """Bytes the pass must move to or from HBM at least: forward reads Q, K, V
    and writes O and LSE; backward reads Q, K, V, O, dO, LSE (and D) and
    writes dQ, dK, dV (and D). K, V, dK, dV have the workload's K/V heads."""
    e = 4 if w.dtype == "fp32" else 2
    q_row = (4 * w.d * e + 8) if backward else (2 * w.d * e + 4)   # per query row
    kv_row = (4 * w.d * e) if backward else (2 * w.d * e)          # per key row of a K/V head
    return float(w.B * w.N * (w.H * q_row + w.kv_heads * kv_row))


def device_info(torch) -> dict:
    """Name, CU count and the runtime's peak clock of device 0."""
    import ctypes
    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "arch": p.gcnArchName, "cus": p.multi_processor_count,
            "l2_bytes": p.L2_cache_size}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        khz = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(khz), 5, 0) == 0:  # hipDeviceAttributeClockRate
            info["peak_clock_mhz"] = khz.value / 1000.0
    except OSError:
        pass
    return info


def kernel_work(name: str, w) -> float:
    """Algorithmic FLOPs (mfma kernels) or bytes (hbm kernels) per launch."""
    half = 0.5 if w.causal else 1.0
    pairs = w.B * w.H * w.N * w.N * half          # visible (query, key) pairs
    if name == "fwd":
        return 4.0 * w.d * pairs                   # S = QK^T and PV: 2d each
    if name == "dkdv":
        return 8.0 * w.d * pairs                   # S recompute, dP, dV, dK
    if name == "dq":
        return 2.0 * w.d * pairs                   # dQ (its S/dP recompute is overhead)
    raise KeyError(name)


def traffic_for(name: str, workload: str):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none for this kernel and workload or the kernel changed since."""
    from exact_io_aware_07_amd.profiling import traffic_record
    rec = traffic_record(TRAFFIC_FILE, workload, name)
    return None if rec is None else rec[0] + rec[1]


def kernel_rooflines(torch, w, iters: int = 10) -> dict:
    """Each kernel of workload ``w``'s pass (the forward, and dQ and dK/dV
    when it has a backward) launched back to back with two HIP events around
    ``iters`` launches, on the launch stream, in batches until at least 50
    launches and 100 ms; per kernel the median launch time, its algorithmic
    work (kernel_work) over that time against the bf16 peak, and the HBM
    traffic per launch from the committed counters (None when stale)."""
    from exact_io_aware_07_amd import fa_bwd_dkdv, fa_bwd_dq, fa_fwd
    inp = {n: (t.cuda() if t is not None else None) for n, t in W_make(w).items()}
    q, k, v, do, kv = inp["q"], inp["k"], inp["v"], inp["do"], inp["kv_len"]
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    dsum = torch.empty_like(lse)
    stream = torch.cuda.current_stream()
    fns = {"fwd": lambda: fa_fwd(q, k, v, o, lse, w.scale, w.causal, kv, stream)}
    if w.backward:
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
        fns["dq"] = lambda: fa_bwd_dq(q, k, v, o, do, lse, dsum, dq, w.scale, w.causal, kv, stream)
        fns["dkdv"] = lambda: fa_bwd_dkdv(q, k, v, do, lse, dsum, dk, dv, w.scale, w.causal, kv,
                                          stream)
    out = {}
    for name, fn in fns.items():
        t_w = time.perf_counter()
        while time.perf_counter() - t_w < 0.3:
            fn()
            torch.cuda.synchronize()
        batches, total = [], 0.0
        while len(batches) * iters < 50 or total < 100.0:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(iters):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            batches.append(e0.elapsed_time(e1) / iters)
            total += batches[-1] * iters
        ms = statistics.median(batches)
        work = kernel_work(name, w)
        achieved = work / (ms * 1e-3)
        out[name] = {"bound": BOUND[name], "avg_us": ms * 1e3, "achieved": achieved / 1e12,
                     "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_FLOPS, "work_per_launch": work,
                     "traffic": traffic_for(name, w.name)}
    return out


def W_make(w):
    from exact_io_aware_07_amd import workloads as W
    return W.make_inputs(w, seed=0)


def run_gpu(args):
    import torch
    from exact_io_aware_07_amd import fa_bwd_dkdv, fa_bwd_dq, fa_fwd, lib
    from exact_io_aware_07_amd import workloads as W

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU (no device visible)")
    lib()  # fail loudly if libfa.so is missing
    w = W.GPT2
    inp = W.make_inputs(w, seed=0)
    q, k, v, do = (inp[n].cuda() for n in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    dsum = torch.empty_like(lse)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    stream = torch.cuda.current_stream()

    kernels_fn = {
        "fwd": lambda: fa_fwd(q, k, v, o, lse, w.scale, w.causal, None, stream),
        "dq": lambda: fa_bwd_dq(q, k, v, o, do, lse, dsum, dq, w.scale, w.causal, None, stream),
        "dkdv": lambda: fa_bwd_dkdv(q, k, v, do, lse, dsum, dk, dv, w.scale, w.causal, None,
                                    stream),
    }
    names = ["fwd", "dq", "dkdv"]

    def step():
        for n in names:
            kernels_fn[n]()

    # Warm-up: the requested W steps, continued until at least WARM_SECONDS of
    # GPU work have run, because the clocks take about a second of load to
    # reach their steady state (a cold first second reads ~15% slow).
    log(f"[bench] warmup: {args.warmup} steps of {w.name}, at least {WARM_SECONDS} s")
    t_w = time.perf_counter()
    n_w = 0
    while n_w < args.warmup or time.perf_counter() - t_w < WARM_SECONDS:
        step()
        n_w += 1
        if n_w % 50 == 0:
            torch.cuda.synchronize()
    # Timed region: K whole steps, nothing else on the stream.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    # Per-kernel duration: two HIP events on the launch stream around K
    # back-to-back launches of that kernel alone (an event between two
    # kernels of a step would add its own few microseconds to each).
    avg_ms = {}
    for n in names:
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(args.steps):
            kernels_fn[n]()
        ev1.record(stream)
        torch.cuda.synchronize()
        avg_ms[n] = ev0.elapsed_time(ev1) / args.steps
    log(f"[bench] {args.steps} steps: {ms_step:.4f} ms/step; kernels (ms) {avg_ms}")
    # Cold caches: before each of up to 50 steps, write a 512 MiB scratch
    # buffer (more than L2 and the 256 MB MALL together), then time the step
    # alone with two events; the median step is reported.
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    cold = []
    for i in range(min(args.steps, 50)):
        flush.fill_(i & 0xFF)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        cold.append((e0, e1))
    torch.cuda.synchronize()
    cold_ms = statistics.median(a.elapsed_time(b) for a, b in cold)
    del flush

    f_fwd = fwd_flops(w)
    f_bwd = 2.5 * f_fwd
    value = (f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12
    dom = max(names, key=lambda n: avg_ms[n])
    bound = BOUND[dom]
    work = kernel_work(dom, w)
    achieved = work / (avg_ms[dom] * 1e-3)
    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": achieved / 1e12, "peak": PEAK_BF16_FLOPS / 1e12,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_FLOPS}
    else:
        roof = {"bound": "hbm", "achieved": achieved / 1e9, "peak": PEAK_HBM_BYTES / 1e9,
                "unit": "GB/s", "frac": achieved / PEAK_HBM_BYTES}
    roof["kernel"] = dom
    roof["traffic"] = traffic_for(dom, w.name)
    kernels = {}
    for n in names:
        kw = kernel_work(n, w)
        rate = kw / (avg_ms[n] * 1e-3)
        if BOUND[n] == "mfma":
            kernels[n] = {"avg_us": avg_ms[n] * 1e3, "tflops": rate / 1e12,
                          "frac_bf16_peak": rate / PEAK_BF16_FLOPS}
        else:
            kernels[n] = {"avg_us": avg_ms[n] * 1e3, "gbps": rate / 1e9,
                          "frac_hbm_peak": rate / PEAK_HBM_BYTES}
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "seed": 0,
                   "flops_per_step": f_fwd + f_bwd,
                   "flop_convention": "fwd 4BHN^2d, bwd 2.5x fwd, x0.5 causal"},
        "pct_of_bf16_peak": 100.0 * value * 1e12 / PEAK_BF16_FLOPS,
        "fwd_tflops": f_fwd / (avg_ms["fwd"] * 1e-3) / 1e12,
        "bwd_tflops": f_bwd / ((avg_ms["dq"] + avg_ms["dkdv"]) * 1e-3) / 1e12,
        "kernels": kernels,
        "kernel_sum_us": sum(avg_ms.values()) * 1e3,
        "cold_cache": {"ms_per_step": cold_ms, "tflops": (f_fwd + f_bwd) / (cold_ms * 1e-3) / 1e12,
                       "steps": len(cold), "flush_bytes": 512 << 20},
        "device": device_info(torch),
        "roofline": roof,
    }
    if not args.no_extra:
        out["extra"] = extra_configs(torch, W)
        out["extra"][W.FEW_HEADS.name] = split_config(torch, W)
        out["extra"][W.GQA.name] = gqa_config(torch, W)
        for sw in (W.SPARSE, W.SPARSE_GLOBAL):
            out["extra"][sw.name] = sparse_config(torch, W, sw)
        out["extra"][W.FP8.name] = fp8_config(torch, W)
    return out


def fp8_config(torch, W):
    """The FP8 forward with incoherent processing on the outlier-channel
    workload: the quantisation launches (HBM-bound) and the attention kernel
    timed apart and together, against the bf16 forward on the same inputs.
    FLOPs are the forward's 4 d N^2 per head (x 1/2 causal)."""
    from exact_io_aware_07_amd import (fa_fp8_quantize, fa_fwd, fa_fwd_fp8, fa_fwd_fp8_incoherent,
                                       fa_fwd_fp8_workspace_bytes, fp8_buffers)
    w = W.FP8
    inp = W.make_inputs(w)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    signs = W.random_signs(w.d, seed=0).cuda()
    bufs = fp8_buffers(w.B, w.H, w.N, w.d)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    ws = torch.empty(fa_fwd_fp8_workspace_bytes(w.B, w.H, w.N, w.d), dtype=torch.uint8, device="cuda")
    fa_fp8_quantize(q, k, v, signs, bufs)
    flops = fwd_flops(w)
    runs = {
        "quantize": lambda: fa_fp8_quantize(q, k, v, signs, bufs),
        "attention_fp8": lambda: fa_fwd_fp8(bufs, True, o, lse, w.scale, w.causal),
        "fp8_total": lambda: fa_fwd_fp8_incoherent(q, k, v, signs, o, lse, w.scale, w.causal, None, ws),
        "bf16_fwd": lambda: fa_fwd(q, k, v, o, lse, w.scale, w.causal),
    }
    entry = {}
    for name, fn in runs.items():
        entry[f"{name}_ms"] = median_ms(torch, fn)
    # compulsory bytes of the quantisation: Q, K, V read once (2 bytes each),
    # the three code arrays written (1 byte each); V is in fact read twice
    qbytes = 9 * w.B * w.H * w.N * w.d
    entry["quantize_gbps_compulsory"] = qbytes / (entry["quantize_ms"] * 1e-3) / 1e9
    for name in ("attention_fp8", "fp8_total", "bf16_fwd"):
        rate = flops / (entry[f"{name}_ms"] * 1e-3)
        entry[f"{name}_tflops"] = rate / 1e12
    entry["attention_fp8_pct_of_fp8_peak"] = 100 * entry["attention_fp8_tflops"] * 1e12 / PEAK_FP8_FLOPS
    entry["speedup_total_vs_bf16"] = entry["bf16_fwd_ms"] / entry["fp8_total_ms"]
    log(f"[bench] extra {w.name}: {entry}")
    return entry


def median_ms(torch, fn, iters: int = 10) -> float:
    """Median per-call time of ``fn`` in batches of ``iters`` calls between two
    events, after 0.3 s of warm-up, over at least 50 calls and 100 ms."""
    t_w = time.perf_counter()
    while time.perf_counter() - t_w < 0.3:
        fn()
        torch.cuda.synchronize()
    batches = []
    while len(batches) * iters < 50 or sum(batches) * iters < 100.0:
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(iters):
            fn()
        e.record()
        torch.cuda.synchronize()
        batches.append(s.elapsed_time(e) / iters)
    return statistics.median(batches)


def sparse_config(torch, W, w):
    """Block-sparse attention on one of its masks: forward and backward
    through fa_fwd_sparse / fa_bwd_sparse and through the planned entry
    points (long mask lines cut into pieces), TFLOP/s counted on the kept
    (query, key) pairs only, and the dense entry points on the same inputs
    for the speed-up (ideal: 1 / kept fraction)."""
    from exact_io_aware_07_amd import (fa_bwd, fa_bwd_sparse, fa_bwd_sparse_planned,
                                       fa_bwd_sparse_planned_workspace_bytes, fa_fwd, fa_fwd_sparse,
                                       fa_fwd_sparse_planned, fa_fwd_sparse_planned_workspace_bytes,
                                       fa_sparse_plan)
    inp = W.make_inputs(w)
    q, k, v, do = (inp[n].cuda() for n in ("q", "k", "v", "do"))
    mask = W.block_mask(w).cuda()
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(w.B * w.H * w.N * 4, dtype=torch.uint8, device="cuda")
    # kept pairs: every kept 128 x 128 block is whole (N is a multiple of 128)
    kept = float(mask.sum().item()) * W.MASK_BLOCK * W.MASK_BLOCK * w.B * w.H
    fwd_kept = 4.0 * w.d * kept
    fa_fwd_sparse(q, k, v, o, lse, mask, w.scale, w.causal)
    plan = fa_sparse_plan(W.block_mask(w), w.B, w.H, w.N, w.causal)
    plan = {"plan": plan["plan"].cuda(), "counts": plan["counts"]}
    ws_f = torch.empty(max(fa_fwd_sparse_planned_workspace_bytes(w.B, w.H, w.N, w.d, plan["counts"]), 16),
                       dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(fa_bwd_sparse_planned_workspace_bytes(w.B, w.H, w.N, w.d, plan["counts"]),
                       dtype=torch.uint8, device="cuda")
    o_p, lse_p = torch.empty_like(o), torch.empty_like(lse)
    runs = {
        "fwd_sparse": (lambda: fa_fwd_sparse(q, k, v, o, lse, mask, w.scale, w.causal), 1.0),
        "fwd_sparse_planned": (lambda: fa_fwd_sparse_planned(q, k, v, o_p, lse_p, mask, plan, w.scale,
                                                             w.causal, None, ws_f), 1.0),
        "bwd_sparse": (lambda: fa_bwd_sparse(q, k, v, o, do, lse, dq, dk, dv, mask, w.scale,
                                             w.causal, None, ws), 2.5),
        "bwd_sparse_planned": (lambda: fa_bwd_sparse_planned(q, k, v, o, do, lse, dq, dk, dv, mask, plan,
                                                             w.scale, w.causal, None, ws_b), 2.5),
    }
    c = plan["counts"].tolist()
    entry = {"kept_fraction": kept / (w.B * w.H * w.N * w.N), "mask": w.block_pattern,
             "plan_pieces": {"col_slots": c[2], "row_slots": c[5]}}
    for name, (fn, mult) in runs.items():
        ms = median_ms(torch, fn)
        rate = mult * fwd_kept / (ms * 1e-3)
        entry[f"{name}_ms"] = ms
        entry[f"{name}_tflops_on_kept_pairs"] = rate / 1e12
        entry[f"{name}_pct_of_bf16_peak"] = 100 * rate / PEAK_BF16_FLOPS
    o2, lse2 = torch.empty_like(q), torch.empty_like(lse)
    fa_fwd(q, k, v, o2, lse2, w.scale, w.causal)
    dense = {"fwd_dense_ms": lambda: fa_fwd(q, k, v, o2, lse2, w.scale, w.causal),
             "bwd_dense_ms": lambda: fa_bwd(q, k, v, o2, do, lse2, dq, dk, dv, w.scale, w.causal,
                                            None, ws)}
    for name, fn in dense.items():
        entry[name] = median_ms(torch, fn)
    for p in ("fwd", "bwd"):
        for v_ in ("sparse", "sparse_planned"):
            entry[f"{p}_{v_}_speedup_vs_dense"] = entry[f"{p}_dense_ms"] / entry[f"{p}_{v_}_ms"]
    log(f"[bench] extra {w.name}: {entry}")
    return entry


def gqa_config(torch, W):
    """Grouped-query attention (32 query heads on 8 K/V heads): forward and
    backward through fa_fwd_gqa / fa_bwd_gqa, and for comparison the plain
    entry points on K/V repeated over each group (the same FLOPs, four times
    the K/V bytes)."""
    from exact_io_aware_07_amd import fa_bwd, fa_bwd_gqa, fa_bwd_gqa_workspace_bytes, fa_fwd, fa_fwd_gqa
    w = W.GQA
    inp = W.make_inputs(w)
    q, k, v, do = (inp[n].cuda() for n in ("q", "k", "v", "do"))
    G = w.H // w.kv_heads
    kr, vr = (t.repeat_interleave(G, dim=1).contiguous() for t in (k, v))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    dq = torch.empty_like(q)
    dk, dv, dkr, dvr = (torch.empty_like(t) for t in (k, v, kr, vr))
    ws_bytes = max(fa_bwd_gqa_workspace_bytes(w.B, w.H, w.kv_heads, w.N, w.d), w.B * w.H * w.N * 4)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    fa_fwd_gqa(q, k, v, o, lse, w.scale, w.causal)
    runs = {
        "fwd_gqa": (lambda: fa_fwd_gqa(q, k, v, o, lse, w.scale, w.causal), 1.0),
        "bwd_gqa": (lambda: fa_bwd_gqa(q, k, v, o, do, lse, dq, dk, dv, w.scale, w.causal,
                                       None, ws), 2.5),
        "fwd_repeated_kv": (lambda: fa_fwd(q, kr, vr, o, lse, w.scale, w.causal), 1.0),
        "bwd_repeated_kv": (lambda: fa_bwd(q, kr, vr, o, do, lse, dq, dkr, dvr, w.scale, w.causal,
                                           None, ws), 2.5),
    }
    entry = {"H": w.H, "Hkv": w.kv_heads, "B": w.B, "N": w.N, "d": w.d,
             "gqa_workspace_bytes": fa_bwd_gqa_workspace_bytes(w.B, w.H, w.kv_heads, w.N, w.d)}
    for name, (fn, mult) in runs.items():
        ms = median_ms(torch, fn)
        rate = mult * fwd_flops(w) / (ms * 1e-3)
        entry[f"{name}_ms"] = ms
        entry[f"{name}_tflops"] = rate / 1e12
        entry[f"{name}_pct_of_bf16_peak"] = 100 * rate / PEAK_BF16_FLOPS
    log(f"[bench] extra {w.name}: {entry}")
    return entry


def extra_configs(torch, W, iters: int = 10):
    """Forward (and backward, at N >= 4096) TFLOP/s of the other workloads."""
    from exact_io_aware_07_amd import attention_backward, attention_forward
    res = {}
    for w in (W.BERT, W.LONG, W.TRADE, W.LONG_BWD, W.TRADE_BWD):
        inp = {n: (t.cuda() if t is not None else None) for n, t in W.make_inputs(w).items()}
        fwd = lambda: attention_forward(inp["q"], inp["k"], inp["v"], w.causal, inp["kv_len"], w.scale)
        o, lse = fwd()
        if w.backward:
            fn = lambda: attention_backward(inp["q"], inp["k"], inp["v"], o, inp["do"], lse,
                                            w.causal, inp["kv_len"], w.scale)
            flops = 2.5 * fwd_flops(w)
        else:
            fn = fwd
            flops = fwd_flops(w)
        t_w = time.perf_counter()
        while time.perf_counter() - t_w < 0.3:
            fn()
            torch.cuda.synchronize()
        # batches of `iters` calls between two events, until at least 50
        # calls and 100 ms; the median batch gives the time per call
        batches, total_ms = [], 0.0
        while len(batches) * iters < 50 or total_ms < 100.0:
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for _ in range(iters):
                fn()
            e.record()
            torch.cuda.synchronize()
            batches.append(s.elapsed_time(e) / iters)
            total_ms += batches[-1] * iters
        ms = statistics.median(batches)
        rate = flops / (ms * 1e-3)
        gbps = compulsory_bytes(w, w.backward) / (ms * 1e-3) / 1e9
        entry = {"ms": ms, "tflops": rate / 1e12, "pct_of_bf16_peak": 100 * rate / PEAK_BF16_FLOPS,
                 "calls": len(batches) * iters, "compulsory_gbps": gbps,
                 "pct_of_hbm_peak": 100 * gbps * 1e9 / PEAK_HBM_BYTES}
        if w.kv_len_range is not None:
            eff = 4.0 * w.H * w.N * w.d * float(inp["kv_len"].sum().item())
            entry["tflops_effective_kv_len"] = eff / (ms * 1e-3) / 1e12
        del inp, o, lse
        if w.N >= 4096:
            entry["kernels"] = kernel_rooflines(torch, w)
        res[w.name] = entry
        log(f"[bench] extra {w.name}: {entry}")
    return res


def split_config(torch, W, num_splits: int = 2):
    """The few-heads causal shape with the plain forward and with the
    key-split forward (num_splits parts, one launch, then one merge launch)."""
    from exact_io_aware_07_amd import fa_fwd, fa_fwd_split, fa_fwd_split_workspace_bytes
    w = W.FEW_HEADS
    inp = W.make_inputs(w)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(fa_fwd_split_workspace_bytes(w.B, w.H, w.N, w.d, num_splits), 16),
                     dtype=torch.uint8, device="cuda")
    runs = {"fwd": lambda: fa_fwd(q, k, v, o, lse, w.scale, w.causal),
            "split": lambda: fa_fwd_split(q, k, v, o, lse, w.scale, w.causal, None, num_splits, ws)}
    flops = fwd_flops(w)
    entry = {"num_splits": num_splits, "workspace_bytes": ws.numel()}
    for name, fn in runs.items():
        t_w = time.perf_counter()
        while time.perf_counter() - t_w < 0.3:
            fn()
            torch.cuda.synchronize()
        batches = []
        while len(batches) < 5 or sum(batches) * 10 < 100.0:
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for _ in range(10):
                fn()
            e.record()
            torch.cuda.synchronize()
            batches.append(s.elapsed_time(e) / 10)
        ms = statistics.median(batches)
        entry[f"{name}_ms"] = ms
        entry[f"{name}_tflops"] = flops / (ms * 1e-3) / 1e12
        entry[f"{name}_pct_of_bf16_peak"] = 100 * flops / (ms * 1e-3) / PEAK_BF16_FLOPS
    entry["split_speedup"] = entry["fwd_ms"] / entry["split_ms"]
    log(f"[bench] extra {w.name}: {entry}")
    return entry


def cpu_baseline(target_s: float = 12.0):
    """The fp64 oracle on the host cores, on a bounded sample of the same
    workload: forward and backward of as many (b, h) heads as fit in about
    ``target_s`` seconds, repeated (at least 3 times) while the total stays
    near ``target_s``; the median pass is reported, in the GPU value's unit."""
    import numpy as np  # noqa: F401
    from exact_io_aware_07_amd import workloads as W
    from oracle import attn_bwd64, attn_fwd64
    w = W.GPT2
    inp = W.make_inputs(w, seed=0)
    q, k, v, do = (inp[n] for n in ("q", "k", "v", "do"))
    heads_all = [(b, h) for b in range(w.B) for h in range(w.H)]

    def run(heads):
        t = time.perf_counter()
        attn_fwd64(q, k, v, w.scale, w.causal, heads=heads)
        attn_bwd64(q, k, v, do, w.scale, w.causal, heads=heads)
        return time.perf_counter() - t

    t1 = run(heads_all[:1])
    n = max(1, min(len(heads_all), int(target_s / max(t1, 1e-3))))
    times = [run(heads_all[:n])]
    while len(times) < 3 or sum(times) < target_s * 0.8:
        times.append(run(heads_all[:n]))
        if sum(times) > 2 * target_s:
            break
    elapsed = statistics.median(times)
    flops = 3.5 * fwd_flops(w) * n / len(heads_all)
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads") or 0) for p in threadpool_info()) or None
    except Exception:
        threads = None
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), None)
    except OSError:
        pass
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s",
            "cores": threads or os.cpu_count(), "kind": "oracle", "cpu_model": cpu_model,
            "sample": f"{w.name}: forward+backward of {n} of {len(heads_all)} heads "
                      f"(fp64, materialised S), median of {len(times)} passes, {elapsed:.2f} s each",
            "seconds": elapsed}


def copy_calibration(nbytes: int) -> None:
    """A plain device-to-device copy of ``nbytes`` (5 times), so that HBM
    counters read under a profiler can be scaled to bytes: each copy kernel
    reads and writes exactly ``nbytes``."""
    import torch
    src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "copies": 5}), flush=True)


def profile_workload(name: str, iters: int) -> None:
    """Run one workload's forward (and backward, if it has one) ``iters`` times,
    for use under a profiler; prints one JSON line with the mean times."""
    import torch
    from exact_io_aware_07_amd import attention_backward, attention_forward, lib
    from exact_io_aware_07_amd import workloads as W
    lib()
    from exact_io_aware_07_amd import (fa_bwd_sparse_planned, fa_fwd_fp8_incoherent,
                                       fa_fwd_sparse_planned, fa_sparse_plan)
    w = W.ALL[name]
    inp = {n: (t.cuda() if t is not None else None) for n, t in W.make_inputs(w).items()}
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    fwd_ms, bwd_ms = [], []
    mask = W.block_mask(w)
    if mask is not None:          # block-sparse: the planned entry points
        plan = fa_sparse_plan(mask, w.B, w.H, w.N, w.causal)
        mask = mask.cuda()
    signs = W.random_signs(w.d, seed=0).cuda() if w.ch_outliers else None
    for _ in range(iters):
        ev[0].record()
        if mask is not None:      # block-sparse
            o = torch.empty_like(inp["q"])
            lse = torch.empty(inp["q"].shape[:3], dtype=torch.float32, device="cuda")
            fa_fwd_sparse_planned(inp["q"], inp["k"], inp["v"], o, lse, mask, plan, w.scale, w.causal)
        elif signs is not None:   # FP8 with the rotation
            o = torch.empty_like(inp["q"])
            lse = torch.empty(inp["q"].shape[:3], dtype=torch.float32, device="cuda")
            fa_fwd_fp8_incoherent(inp["q"], inp["k"], inp["v"], signs, o, lse, w.scale, w.causal)
        else:
            o, lse = attention_forward(inp["q"], inp["k"], inp["v"], w.causal, inp["kv_len"], w.scale)
        ev[1].record()
        if w.backward and mask is not None:
            g = [torch.empty_like(inp["q"]) for _ in range(3)]
            fa_bwd_sparse_planned(inp["q"], inp["k"], inp["v"], o, inp["do"], lse, *g, mask, plan, w.scale,
                                  w.causal)
        elif w.backward:
            attention_backward(inp["q"], inp["k"], inp["v"], o, inp["do"], lse, w.causal,
                               inp["kv_len"], w.scale)
        ev[2].record()
        torch.cuda.synchronize()
        fwd_ms.append(ev[0].elapsed_time(ev[1]))
        bwd_ms.append(ev[1].elapsed_time(ev[2]))
    print(json.dumps({"workload": name, "iters": iters, "fwd_ms": statistics.fmean(fwd_ms),
                      "bwd_ms": statistics.fmean(bwd_ms) if w.backward else None}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip timing the oracle")
    ap.add_argument("--copy-calibration", type=int, metavar="BYTES", default=0,
                    help="only run a plain copy of BYTES (for scaling HBM counters) and exit")
    ap.add_argument("--profile-workload", metavar="NAME", default="",
                    help="only run NAME's forward (+backward) --iters times and exit")
    ap.add_argument("--iters", type=int, default=10)
    args = ap.parse_args()
    if args.profile_workload:
        profile_workload(args.profile_workload, args.iters)
        return
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only (asked for --gpus {args.gpus}); "
              "the per-head work is independent and would shard by (batch, head) with no "
              "exchange, but only the single-GPU path exists", file=sys.stderr)
        raise SystemExit(2)
    out = run_gpu(args)
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on the host")
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
