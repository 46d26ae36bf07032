#!/usr/bin/env python3
"""Throughput of exact attention (forward + backward) on one MI355X.

One step = one forward pass and one backward pass of the whole path
(fused online-softmax forward writing O and LSE; D pre-pass, dK/dV pass and
dQ pass of the backward) over one batch of seeded synthetic inputs already
resident in HBM.  The default workload is the long-context causal shape
B=4, H=40, N=8192, d=128 in bf16 (Q, K, V, dO iid N(0,1) x 0.5).

FLOPs follow the convention of the FlashAttention-2 notes ("Reproducibility
notes"): forward 4 B H N^2 d, backward 2.5x forward, halved for causal,
scaled by the realized block density for block-sparse masks.

Prints ONE JSON line on stdout (rank 0); anything else goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}   # MI355X dense MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "fwd/bwd attention TFLOP/s + % of bf16 MFMA peak, N=1k–16k, d=64/128"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class ClockSampler:
    """Samples the shader clock amdsmi reports (current_gfxclks, MHz, mean
    over the XCDs) while the timed region runs; median() is None when it
    cannot be read.  This is the clock the firmware reports; the effective
    rate under the attention kernels (GRBM_GUI_ACTIVE cycles over kernel
    time, in the counter summaries) can be lower."""

    def __init__(self, period_s=0.005):
        import threading
        self.period = period_s
        self.samples = []
        self._stop = threading.Event()
        self._thread = None
        self._read = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handle = amdsmi.amdsmi_get_processor_handles()[0]

            def read():
                m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
                clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float)) and 0 < c < 10000]
                if not clks and isinstance(m.get("current_gfxclk"), (int, float)):
                    clks = [m["current_gfxclk"]]
                return sum(clks) / len(clks) if clks else None
            read()
            self._read = read
        except Exception:  # pragma: no cover - no amdsmi or no permission
            self._read = None

    def _loop(self):
        while not self._stop.is_set():
            try:
                v = self._read()
                if v:
                    self.samples.append(v)
            except Exception:
                pass
            self._stop.wait(self.period)

    def __enter__(self):
        import threading
        if self._read:
            self._thread = threading.Thread(target=self._loop, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread:
            self._thread.join()

    def median(self):
        if not self.samples:
            return None
        v = sorted(self.samples)
        return float(v[len(v) // 2])


def flop_counts(w, mask):
    """(forward, backward) FLOPs of one step by the pages' convention."""
    f = 4.0 * w["B"] * w["H"] * w["N"] ** 2 * w["d"]
    if w["causal"]:
        f *= 0.5
    if mask is not None:
        f *= float(mask.float().mean())
    return f, (2.5 * f if w["backward"] else 0.0)


def kernel_flops(w, mask):
    """Algorithmic FLOPs per launch of each compute kernel: the products the
    convention counts that this kernel performs (recomputed S and dP inside
    the dQ pass are not counted)."""
    unit = 2.0 * w["B"] * w["H"] * w["N"] ** 2 * w["d"]   # one N x N x d product
    if w["causal"]:
        unit *= 0.5
    if mask is not None:
        unit *= float(mask.float().mean())
    return {"fwd": 2 * unit, "fwd_f32": 2 * unit, "bwd_dkdv": 4 * unit, "bwd_dq": 1 * unit}


def kernel_bytes(w):
    """Compulsory HBM bytes per launch: what each kernel must read and write
    at least once (tensor T = B H N d elements, a per-row array = B H N
    float32).  Forward: Q, K, V read, O written (4T) plus LSE.  Pre-pass: O,
    dO, LSE read; D and the base-2 LSE written.  dK/dV pass: Q, K, V, dO
    and the two per-row arrays read, dK and dV written (6T + 2 rows).  dQ
    pass: Q, K, V, dO, LSE, D read, dQ written (5T + 2 rows).  Only the
    pre-pass is memory bound; for the others the figure gives the achieved
    HBM rate the compulsory traffic implies."""
    el = {"bf16": 2, "f16": 2, "f32": 4}[w["dtype"]]
    rows = w["B"] * w["H"] * w["N"]
    t = rows * w["d"] * el
    fwd = 4 * t + 4 * rows
    return {"fwd": fwd, "fwd_f32": fwd, "bwd_pre": rows * (2 * w["d"] * el + 12),
            "bwd_dkdv": 6 * t + 8 * rows, "bwd_dq": 5 * t + 8 * rows}


# HBM bytes per launch measured with rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE
# (each scaled by what the counter reads for a plain device copy of known
# size, see profiles/), keyed by kernel and workload, valid only while the
# kernel's sources hash to the recorded value.
KERNEL_SOURCES = {
    "fwd": ["fa_fwd2.hip", "fa_device.hpp", "fa_kernels.hpp"],
    "bwd_pre": ["fa_bwd.hip", "fa_device.hpp", "fa_kernels.hpp"],
    "bwd_dkdv": ["fa_bwd.hip", "fa_device.hpp", "fa_kernels.hpp"],
    "bwd_dq": ["fa_bwd.hip", "fa_device.hpp", "fa_kernels.hpp"],
}
MEASURED_TRAFFIC = {
    # (kernel, workload): (sources sha256 prefix, bytes per launch)
    ("fwd", 4): ("3a587413d31acff7", 1979772928),
    ("bwd_pre", 4): ("ca9d5a6c178398a1", 692115456),
    ("bwd_dkdv", 4): ("ca9d5a6c178398a1", 2118136832),
    ("bwd_dq", 4): ("ca9d5a6c178398a1", 2377652224),
}


def sources_sha(kernel):
    import hashlib
    d = os.path.join(os.path.dirname(os.path.abspath(__file__)), "io_aware_exact_flash_amd", "csrc")
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kernel, []):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, num):
    rec = MEASURED_TRAFFIC.get((kernel, num))
    if rec is None or rec[0] != sources_sha(kernel):
        return None          # not measured, or the kernel changed since
    return rec[1]


def cpu_baseline(num, heads):
    """The float64 oracle, as it stands, on a bounded sample of the workload."""
    import numpy as np
    from oracle import attention as A
    from io_aware_exact_flash_amd import workloads
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    w = workloads.WORKLOADS[num]
    q, k, v, do, mask = workloads.workload_inputs(num)
    s = float(np.float32(1.0 / math.sqrt(w["d"])))
    m = None if mask is None else mask.numpy()
    pairs = workloads.head_subset(w["B"], w["H"], heads, seed=num + 2000)
    t0 = time.perf_counter()
    for (b, h) in pairs:
        qq, kk, vv = (t[b, h].double().numpy() for t in (q, k, v))
        A.forward_head(qq, kk, vv, s, w["causal"], m)
        if w["backward"]:
            A.backward_head(qq, kk, vv, do[b, h].double().numpy(), s, w["causal"], m)
    dt = time.perf_counter() - t0
    one = dict(w, B=1, H=1)
    fl = flop_counts(one, mask)
    per_head = fl[0] + fl[1]
    return {"value": per_head * len(pairs) / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{len(pairs)} of {w['B'] * w['H']} (batch, head) pairs of the same workload, "
                      f"forward{'+backward' if w['backward'] else ''} in float64 (NumPy), {dt:.1f} s"}


def step_bytes(w):
    """Compulsory HBM bytes of one step: the forward reads Q, K, V and writes
    O and LSE; the backward reads Q, K, V, O, dO and LSE and writes dQ, dK,
    dV (tensor T = B H N d elements, per-row arrays B H N float32)."""
    el = {"bf16": 2, "f16": 2, "f32": 4}[w["dtype"]]
    rows = w["B"] * w["H"] * w["N"]
    t = rows * w["d"] * el
    return 4 * t + 4 * rows + ((8 * t + 4 * rows) if w["backward"] else 0)


def _time_steps(step, steps, warmup, e_mid_holder, sampler=None):
    """Run `steps` timed steps after `warmup` untimed ones; HIP events on
    torch's current stream (the library's launch stream) around each step
    and at the forward/backward boundary."""
    import contextlib
    import torch
    from io_aware_exact_flash_amd import flash
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    flash.timing_collect()          # drop anything recorded before the timed region
    flash.timing_enable(True)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    mids = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    with (sampler if sampler is not None else contextlib.nullcontext()):
        t0 = time.perf_counter()
        for i in range(steps):
            starts[i].record()
            e_mid_holder[0] = mids[i]
            step()
            ends[i].record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    flash.timing_enable(False)
    kt = flash.timing_collect()
    per_step = sorted(starts[i].elapsed_time(ends[i]) for i in range(steps))
    fwd_ms = sum(starts[i].elapsed_time(mids[i]) for i in range(steps)) / steps
    bwd_ms = sum(mids[i].elapsed_time(ends[i]) for i in range(steps)) / steps
    return (t1 - t0) * 1e3 / steps, per_step, fwd_ms, bwd_ms, kt


def run_workload(num, steps, warmup, quiet=False, sample_clock=False):
    import torch
    from io_aware_exact_flash_amd import flash, workloads

    w = workloads.WORKLOADS[num]
    q, k, v, do, mask = workloads.workload_inputs(num)
    dev = torch.device("cuda", 0)
    q, k, v, do = (t.to(dev) for t in (q, k, v, do))
    gm = None if mask is None else mask.to(dev)
    s = float(1.0 / math.sqrt(w["d"]))
    causal = w["causal"]
    ws = torch.empty(max(1, flash.bwd_workspace_size(w["B"], w["H"], w["N"], w["d"], q.dtype)),
                     dtype=torch.uint8, device=dev)
    e_mid = [None]

    def make_step(sparse):
        def step():
            if sparse:
                o, lse = flash.blocksparse_fwd(q, k, v, gm, scale=s, causal=causal)
            else:
                o, lse = flash.fwd(q, k, v, scale=s, causal=causal)
            if e_mid[0] is not None:
                e_mid[0].record()
            if w["backward"]:
                if sparse:
                    flash.blocksparse_bwd(q, k, v, o, do, lse, gm, scale=s, causal=causal, workspace=ws)
                else:
                    flash.bwd(q, k, v, o, do, lse, scale=s, causal=causal, workspace=ws)
            return o
        return step

    sampler = ClockSampler() if sample_clock else None
    ms_step, per_step, fwd_ms, bwd_ms, kt = _time_steps(make_step(gm is not None), steps, warmup, e_mid, sampler)
    ff, fb = flop_counts(w, mask)
    peak = PEAK_TFLOPS[w["dtype"]]
    kf = kernel_flops(w, mask)
    kb = kernel_bytes(w)
    kernels = {}
    for name, (tot, cnt) in kt.items():
        if cnt:
            avg = tot / cnt
            entry = {"avg_ms": round(avg, 4), "launches": cnt}
            if name in kf:
                entry["tflops"] = round(kf[name] / (avg * 1e-3) / 1e12, 2)
            if name in kb:
                entry["gbs"] = round(kb[name] / (avg * 1e-3) / 1e9, 1)
            kernels[name] = entry
    dom = max(kernels, key=lambda n: kt[n][0]) if kernels else None
    if dom in kf:
        ach = kf[dom] / (kernels[dom]["avg_ms"] * 1e-3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(ach / peak, 4), "traffic": measured_traffic(dom, num)}
    elif dom in kb:
        ach = kb[dom] / (kernels[dom]["avg_ms"] * 1e-3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": measured_traffic(dom, num)}
    else:
        roof = None
    res = {
        "value": (ff + fb) / (ms_step * 1e-3) / 1e12,
        "ms_per_step": ms_step,
        "fwd_ms": fwd_ms, "bwd_ms": bwd_ms,
        "fwd_tflops": ff / (fwd_ms * 1e-3) / 1e12,
        "bwd_tflops": (fb / (bwd_ms * 1e-3) / 1e12) if fb else None,
        "peak": peak, "kernels": kernels, "roofline": roof,
        "step_ms_median": per_step[len(per_step) // 2], "step_ms_min": per_step[0],
        "density": None if mask is None else float(mask.float().mean()),
        # compulsory HBM bytes of the step over its time (the small shapes'
        # memory-side figure; the MFMA-bound shapes sit far below 8 TB/s)
        "hbm_gbs": step_bytes(w) / (per_step[len(per_step) // 2] * 1e-3) / 1e9,
        "sclk_mhz": None if sampler is None else sampler.median(),
    }
    res["fwd_frac_of_peak"] = res["fwd_tflops"] / peak
    res["bwd_frac_of_peak"] = res["bwd_tflops"] / peak if fb else None
    if mask is not None:
        # every kernel visits exactly the kept tiles of its mask row or column
        # (one 128-row mask row per forward/dQ workgroup at d = 64), so the
        # visited fraction is the realized density; the skip efficiency is
        # the sparse kernels' throughput on the work they do over the dense
        # kernels' throughput at the same shape
        e_mid[0] = None
        d_ms, d_per, d_fwd, d_bwd, _ = _time_steps(make_step(False), max(3, steps // 2), 2, e_mid)
        dense_f, dense_b = flop_counts(w, None)
        dense_tf = (dense_f + dense_b) / (d_per[len(d_per) // 2] * 1e-3) / 1e12
        sparse_tf = (ff + fb) / (per_step[len(per_step) // 2] * 1e-3) / 1e12
        res["tiles_visited_frac"] = res["density"]
        res["dense_same_shape"] = {"ms_per_step": round(d_per[len(d_per) // 2], 4), "tflops": round(dense_tf, 2)}
        res["skip_efficiency"] = sparse_tf / dense_tf
    if not quiet:
        log(f"workload {num} ({w['name']}): {ms_step:.3f} ms/step, fwd {res['fwd_tflops']:.1f} TF/s "
            f"({100 * res['fwd_frac_of_peak']:.1f}%), bwd "
            + (f"{res['bwd_tflops']:.1f} TF/s ({100 * res['bwd_frac_of_peak']:.1f}%)" if fb else "-")
            + f", {res['hbm_gbs']:.0f} GB/s compulsory, kernels {kernels}"
            + (f", skip efficiency {res['skip_efficiency']:.2f}" if mask is not None else ""))
    del q, k, v, do, ws
    torch.cuda.empty_cache()
    return w, res


def workload_summary(num, w, r):
    """Per-workload entry of the JSON line."""
    out = {"workload": f"{w['name']}: B={w['B']} H={w['H']} N={w['N']} d={w['d']} {w['dtype']}, "
                       f"{'causal' if w['causal'] else 'non-causal'}"
                       + (", block-sparse" if w["density"] else "")
                       + (", forward+backward" if w["backward"] else ", forward"),
           "ms_per_step": round(r["step_ms_median"], 4),
           "fwd_ms": round(r["fwd_ms"], 4),
           "bwd_ms": None if not w["backward"] else round(r["bwd_ms"], 4),
           "fwd_tflops": round(r["fwd_tflops"], 2),
           "bwd_tflops": None if r["bwd_tflops"] is None else round(r["bwd_tflops"], 2),
           "fwd_frac_of_peak": round(r["fwd_frac_of_peak"], 4),
           "bwd_frac_of_peak": None if r["bwd_frac_of_peak"] is None else round(r["bwd_frac_of_peak"], 4),
           "peak_tflops": r["peak"],
           "hbm_gbs": round(r["hbm_gbs"], 1),
           "kernels": r["kernels"]}
    if r["density"] is not None:
        out.update(density=round(r["density"], 4), tiles_visited_frac=round(r["tiles_visited_frac"], 4),
                   dense_same_shape=r["dense_same_shape"], skip_efficiency=round(r["skip_efficiency"], 3))
    return out


# Shapes for the variants that widen the path (timed with --variants; stderr
# lines plus a "variants" object in the JSON line).  FLOPs as for the main
# workloads (causal halved).
VARIANTS = {
    "splitkv": dict(name="split-KV forward, few heads", B=1, H=8, N=8192, d=128, dtype="bf16", causal=True,
                    splits=(2, 4), seed=11),
    "gqa": dict(name="grouped K/V heads (4 query heads per K/V head)", B=4, H=32, Hkv=8, N=4096, d=128,
                dtype="bf16", causal=True, seed=12),
    "mqa": dict(name="multi-query (one K/V head)", B=4, H=32, Hkv=1, N=4096, d=128,
                dtype="bf16", causal=True, seed=13),
    "dropout": dict(name="dropout p=0.1", B=4, H=32, N=2048, d=128, dtype="bf16", causal=True, p=0.1, seed=15),
    "varlen": dict(name="packed variable-length batch", B=8, H=16, Hkv=16, max_len=4096, d=128,
                   dtype="bf16", causal=True, seed=14),
    # one new query per head against a key/value cache (decoding), grouped
    # heads; HBM bound: every cached byte is read once
    "decode": [dict(name="decode, 32k-token cache", B=8, H=64, Hkv=8, Nq=1, Nk=32768, d=128, dtype="bf16",
                    causal=True, seed=16),
               dict(name="decode, 8k-token cache", B=32, H=32, Hkv=8, Nq=1, Nk=8192, d=128, dtype="bf16",
                    causal=True, seed=17)],
}


def time_ms(fn, steps, warmup):
    """Average milliseconds of fn() over `steps` calls, bracketed by events on
    torch's current stream (the stream the library launches on)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def run_variants(steps, warmup):
    import torch
    from io_aware_exact_flash_amd import flash, workloads

    out = {}
    v = VARIANTS["splitkv"]
    q, k, vv, _ = (t.cuda() for t in workloads.qkvdo(v["B"], v["H"], v["N"], v["d"], v["dtype"], seed=v["seed"]))
    f = 4.0 * v["B"] * v["H"] * v["N"] ** 2 * v["d"] * (0.5 if v["causal"] else 1.0)
    res = {"plain": time_ms(lambda: flash.fwd(q, k, vv, causal=v["causal"]), steps, warmup)}
    for sp in v["splits"]:
        nb = flash.fwd_splitkv_workspace_size(v["B"], v["H"], v["N"], v["d"], sp, q.dtype)
        ws = torch.empty(nb, dtype=torch.uint8, device=q.device)
        res[f"splits_{sp}"] = time_ms(lambda: flash.fwd_splitkv(q, k, vv, sp, causal=v["causal"], workspace=ws),
                                      steps, warmup)
    out["splitkv"] = {"workload": f"{v['name']}: B={v['B']} H={v['H']} N={v['N']} d={v['d']} {v['dtype']} causal",
                      "fwd_ms": {n: round(t, 4) for n, t in res.items()},
                      "fwd_tflops": {n: round(f / (t * 1e-3) / 1e12, 1) for n, t in res.items()}}
    log(f"variant splitkv: {out['splitkv']}")
    del q, k, vv

    for key in ("gqa", "mqa"):
        v = VARIANTS[key]
        q, k, vv, do = (t.cuda() for t in workloads.qkvdo_grouped(v["B"], v["H"], v["Hkv"], v["N"], v["d"],
                                                                   v["dtype"], seed=v["seed"]))
        krep = k.repeat_interleave(v["H"] // v["Hkv"], dim=1).contiguous()
        vrep = vv.repeat_interleave(v["H"] // v["Hkv"], dim=1).contiguous()
        ws = torch.empty(flash.bwd_workspace_size(v["B"], v["H"], v["N"], v["d"], q.dtype), dtype=torch.uint8,
                         device=q.device)
        wsg = torch.empty(flash.bwd_gqa_workspace_size(v["B"], v["H"], v["Hkv"], v["N"], v["d"], q.dtype),
                          dtype=torch.uint8, device=q.device)
        f = 4.0 * v["B"] * v["H"] * v["N"] ** 2 * v["d"] * (0.5 if v["causal"] else 1.0)
        o, lse = flash.fwd_gqa(q, k, vv, causal=v["causal"])
        c = v["causal"]
        res = {
            "broadcast_fwd": (time_ms(lambda: flash.fwd(q, krep, vrep, causal=c), steps, warmup), f),
            "grouped_fwd": (time_ms(lambda: flash.fwd_gqa(q, k, vv, causal=c), steps, warmup), f),
            "broadcast_bwd": (time_ms(lambda: flash.bwd(q, krep, vrep, o, do, lse, causal=c, workspace=ws),
                                      steps, warmup), 2.5 * f),
            "grouped_bwd": (time_ms(lambda: flash.bwd_gqa(q, k, vv, o, do, lse, causal=c, workspace=wsg),
                                    steps, warmup), 2.5 * f),
        }
        out[key] = {"workload": f"{v['name']}: B={v['B']} H={v['H']} Hkv={v['Hkv']} N={v['N']} d={v['d']} "
                                f"{v['dtype']} causal; broadcast_* = the plain calls on K/V copied to every head",
                    "ms": {n: round(t, 4) for n, (t, _) in res.items()},
                    "tflops": {n: round(fl / (t * 1e-3) / 1e12, 1) for n, (t, fl) in res.items()}}
        log(f"variant {key}: {out[key]}")
        del q, k, vv, do, krep, vrep, ws, wsg, o, lse

    v = VARIANTS["varlen"]
    lens = workloads.seq_lengths(v["B"], v["max_len"], v["seed"])
    q, k, vv, do, cu = workloads.packed_qkvdo(lens, v["H"], v["Hkv"], v["d"], v["dtype"], seed=v["seed"])
    q, k, vv, do, cu = (t.cuda() for t in (q, k, vv, do, cu))
    T, mx, c = sum(lens), max(lens), v["causal"]
    f = sum(4.0 * v["H"] * n * n * v["d"] * (0.5 if c else 1.0) for n in lens)
    wsv = torch.empty(flash.varlen_bwd_workspace_size(v["B"], v["H"], v["Hkv"], T, mx, v["d"], q.dtype),
                      dtype=torch.uint8, device=q.device)
    o, lse = flash.varlen_fwd(q, k, vv, cu, mx, causal=c)
    # the same sequences padded to the longest one, through the dense calls
    qp, kp, vp, dop = (torch.zeros((v["B"], v["H"], mx, v["d"]), dtype=q.dtype, device=q.device)
                       for _ in range(4))
    ws = torch.empty(flash.bwd_workspace_size(v["B"], v["H"], mx, v["d"], q.dtype), dtype=torch.uint8,
                     device=q.device)
    op, lsep = flash.fwd(qp, kp, vp, causal=c)
    res = {
        "packed_fwd": time_ms(lambda: flash.varlen_fwd(q, k, vv, cu, mx, causal=c), steps, warmup),
        "packed_bwd": time_ms(lambda: flash.varlen_bwd(q, k, vv, o, do, lse, cu, mx, causal=c, workspace=wsv),
                              steps, warmup),
        "padded_fwd": time_ms(lambda: flash.fwd(qp, kp, vp, causal=c), steps, warmup),
        "padded_bwd": time_ms(lambda: flash.bwd(qp, kp, vp, op, dop, lsep, causal=c, workspace=ws), steps, warmup),
    }
    out["varlen"] = {"workload": f"{v['name']}: lengths {lens} (total {T}), H={v['H']} d={v['d']} {v['dtype']} "
                                 f"causal; padded_* = the dense calls on the batch padded to {mx}",
                     "ms": {n: round(t, 4) for n, t in res.items()},
                     "tflops_useful": {n: round((2.5 * f if n.endswith("bwd") else f) / (t * 1e-3) / 1e12, 1)
                                       for n, t in res.items()}}
    log(f"variant varlen: {out['varlen']}")
    del q, k, vv, do, cu, o, lse, qp, kp, vp, dop, op, lsep, ws, wsv

    out["decode"] = []
    for v in VARIANTS["decode"]:
        q, k, vv = (t.cuda() for t in workloads.kvcache_qkv(v["B"], v["H"], v["Hkv"], v["Nq"], v["Nk"], v["d"],
                                                             v["dtype"], seed=v["seed"]))
        sp = flash.fwd_kvcache_num_splits(v["B"], v["H"], v["Hkv"], v["Nq"], v["Nk"], v["d"])
        ws = torch.empty(max(1, flash.fwd_kvcache_workspace_size(v["B"], v["H"], v["Hkv"], v["Nq"], v["Nk"], v["d"],
                                                                  sp, q.dtype)), dtype=torch.uint8, device=q.device)
        t = time_ms(lambda: flash.fwd_kvcache(q, k, vv, num_splits=sp, causal=v["causal"], workspace=ws),
                    max(steps, 20), warmup)
        el = 2
        byts = (2 * v["B"] * v["Hkv"] * v["Nk"] * v["d"] + 2 * v["B"] * v["H"] * v["Nq"] * v["d"]) * el \
            + 4 * v["B"] * v["H"] * v["Nq"]
        flops = 4.0 * v["B"] * v["H"] * v["Nq"] * v["Nk"] * v["d"]
        e = {"workload": f"{v['name']}: B={v['B']} H={v['H']} Hkv={v['Hkv']} Nq={v['Nq']} Nk={v['Nk']} "
                         f"d={v['d']} {v['dtype']}, {sp} key splits",
             "ms": round(t, 4), "gbs": round(byts / (t * 1e-3) / 1e9, 1),
             "frac_of_hbm_peak": round(byts / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
             "tflops": round(flops / (t * 1e-3) / 1e12, 2), "bytes": byts}
        out["decode"].append(e)
        log(f"variant decode: {e}")
        del q, k, vv, ws

    v = VARIANTS["dropout"]
    q, k, vv, do = (t.cuda() for t in workloads.qkvdo(v["B"], v["H"], v["N"], v["d"], v["dtype"], seed=v["seed"]))
    c, pd = v["causal"], v["p"]
    f = 4.0 * v["B"] * v["H"] * v["N"] ** 2 * v["d"] * (0.5 if c else 1.0)
    ws = torch.empty(flash.bwd_workspace_size(v["B"], v["H"], v["N"], v["d"], q.dtype), dtype=torch.uint8,
                     device=q.device)
    o, lse = flash.fwd(q, k, vv, causal=c)
    od, lsed = flash.fwd_dropout(q, k, vv, pd, 1, 0, causal=c)
    res = {
        "plain_fwd": (time_ms(lambda: flash.fwd(q, k, vv, causal=c), steps, warmup), f),
        "dropout_fwd": (time_ms(lambda: flash.fwd_dropout(q, k, vv, pd, 1, 0, causal=c), steps, warmup), f),
        "plain_bwd": (time_ms(lambda: flash.bwd(q, k, vv, o, do, lse, causal=c, workspace=ws), steps, warmup),
                      2.5 * f),
        "dropout_bwd": (time_ms(lambda: flash.bwd_dropout(q, k, vv, od, do, lsed, pd, 1, 0, causal=c, workspace=ws),
                                steps, warmup), 2.5 * f),
    }
    out["dropout"] = {"workload": f"{v['name']}: B={v['B']} H={v['H']} N={v['N']} d={v['d']} {v['dtype']} causal",
                      "ms": {n: round(t, 4) for n, (t, _) in res.items()},
                      "tflops": {n: round(fl / (t * 1e-3) / 1e12, 1) for n, (t, fl) in res.items()}}
    log(f"variant dropout: {out['dropout']}")
    del q, k, vv, do, ws, o, lse, od, lsed
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=4, choices=[1, 2, 3, 4, 5],
                    help="workload timed for the JSON line (default 4: 4x40x8192x128 causal bf16)")
    ap.add_argument("--only", action="store_true",
                    help="time only the headline workload (default: all five, the others under 'workloads')")
    ap.add_argument("--all", action="store_true", help=argparse.SUPPRESS)  # the default now
    ap.add_argument("--cpu-heads", type=int, default=10, help="(batch, head) pairs the oracle baseline runs (about 1 s each at N=8192)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--variants", action="store_true",
                    help="also time the split-KV forward, grouped K/V heads, a packed variable-length "
                         "batch and dropout (adds a 'variants' object)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after the run, copy a device buffer of this many bytes 3 times "
                         "(calibrates the HBM byte counters of a profiling run)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(heads shard across GPUs with no exchange; run one process per GPU instead).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a HIP device (MI355X); none is visible.", file=sys.stderr)
        sys.exit(3)
    torch.cuda.set_device(0)

    # the other workloads first (their entries go to "workloads"), then the
    # headline workload, whose timed region the top-level fields describe
    others = {}
    if not args.only:
        for num in (1, 2, 3, 5, 4):
            if num != args.workload:
                ow, r = run_workload(num, args.steps, args.warmup)
                others[num] = workload_summary(num, ow, r)
    w, r = run_workload(args.workload, args.steps, args.warmup, sample_clock=True)

    if args.copy_bytes > 0:
        src = torch.empty(args.copy_bytes, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {args.copy_bytes} bytes 3 times")
        del src, dst

    variants = run_variants(args.steps, args.warmup) if args.variants else None
    cpu = None if args.no_cpu_baseline else cpu_baseline(args.workload, args.cpu_heads)
    line = {
        "metric": METRIC,
        "value": round(r["value"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "step_ms_median": round(r["step_ms_median"], 4),   # HIP events around each step
        "step_ms_min": round(r["step_ms_min"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w["dtype"],
        "data": "synthetic",
        "config": {"workload": f"{w['name']} attention, B={w['B']} H={w['H']} N={w['N']} d={w['d']} "
                               f"{w['dtype']}, {'causal' if w['causal'] else 'non-causal'}"
                               + (", block-sparse" if w["density"] else "")
                               + (", forward+backward" if w["backward"] else ", forward"),
                   "B": w["B"], "H": w["H"], "N": w["N"], "d": w["d"], "causal": w["causal"],
                   "parallelism": "single-gpu"},
        "fwd_tflops": round(r["fwd_tflops"], 2),
        "bwd_tflops": None if r["bwd_tflops"] is None else round(r["bwd_tflops"], 2),
        "fwd_frac_of_peak": round(r["fwd_frac_of_peak"], 4),
        "bwd_frac_of_peak": None if r["bwd_frac_of_peak"] is None else round(r["bwd_frac_of_peak"], 4),
        "kernels": r["kernels"],
        "roofline": r["roofline"],
        "cpu_baseline": cpu,
        # shader clock sampled (amdsmi) during the headline timed region: the
        # fixed 2516.6 TF/s peak assumes 2.4 GHz
        "sclk_mhz": None if r["sclk_mhz"] is None else round(r["sclk_mhz"], 1),
        "hbm_gbs": round(r["hbm_gbs"], 1),
        "workloads": {str(n): e for n, e in sorted({**others, args.workload: workload_summary(
            args.workload, w, r)}.items())},
    }
    if variants is not None:
        line["variants"] = variants
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
